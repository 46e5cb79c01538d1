"""GPU parity at the large tiles' edges, over two-round grids, across shard counts, and for
the b2/T form of the block tail.

* Every 256-class tile with a ragged row or column edge, and grids of two rounds of
  workgroups, forward and backward, element by element against the fp64 oracle
  (tests/tile_cases.py; each case first asks the library which tile each product takes).
* T in {1, 2, 4, 8} on the GPT-2-medium and Llama-3-70B FFN shapes: all T shards of one full
  weight, summed with b2 once, on sampled token rows [Z 11].
* b2 split over the ranks [Z 05]: bit-exact on integer data for T a power of two, within
  rounding otherwise, and on the bf16 shapes.
* The split-contraction forward (mlp_tp_shard_fwd_ws) on shapes with too few tiles to fill the
  GPU [Z 04], element by element, deterministic, and unsplit when the workspace is short.

Bars as in test_parity_gpu.py: bit-exact on integer-valued fp32 data, else
max|gpu - ref| / max|ref| <= 1e-2 per output tensor.

Pages cited:
  [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from tensor_mlp_block_amd import binding as mt
from tensor_mlp_block_amd import synth, workloads
from tensor_mlp_block_amd.workloads import Workload
from tile_cases import EDGE_CASES

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU; deselect them with -m 'not gpu'"
    mt.load()
    yield
    torch.cuda.synchronize()


def _dt(w):
    return mt.BF16 if w.dtype == "bf16" else mt.F32


def _tdt(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def rel_err(gpu, ref):
    g = gpu.detach().to("cpu", torch.float64).numpy()
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    denom = np.max(np.abs(ref))
    return float(np.max(np.abs(g))) if denom == 0.0 else float(np.max(np.abs(g - ref)) / denom)


def assert_close(name, gpu, ref, tol=TOL):
    e = rel_err(gpu, ref)
    _say(f"    {name}: rel err {e:.3e}")
    assert e <= tol, f"{name}: rel err {e:.3e} > {tol}"


def assert_exact(name, gpu, ref):
    g = gpu.detach().to("cpu", torch.float64).numpy()
    assert not np.any(np.isnan(g)), name
    assert np.array_equal(g, np.asarray(ref, dtype=np.float64)), f"{name}: not bit-exact"


def _sample(n, extra, seed):
    rng = np.random.default_rng(seed)
    base = [0, 1, 127, 128, 255, 256, n // 2 - 1, n // 2, n - 257, n - 256, n - 2, n - 1]
    base += list(rng.integers(0, n, size=extra))
    return np.array(sorted({int(i) for i in base if 0 <= i < n}))


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


# --------------------------------------------------------------------------------------------
# Ragged edges of the 256-class tiles and two-round grids, element by element
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("w,expect", EDGE_CASES, ids=lambda x: getattr(x, "name", ""))
def test_large_tile_edges_forward_and_backward(w, expect):
    _say(f"  workload {w.name} tiles {expect}")
    cus = _cus()
    for prod, tile in expect.items():
        got = mt.mlp_tp_shard_tile(prod, w.N, w.D, w.F, w.T, cus)
        if cus == 256:
            assert got == (*tile, 0), (prod, got)
        _say(f"    {prod} on {got[0]}x{got[1]} ({cus} CUs)")
    Xc, dYc = synth.gen_X(w), synth.gen_dY(w)
    W1c, b1c, W2c = synth.gen_W1(w), synth.gen_b1(w), synth.gen_W2(w)
    dev = "cuda"
    X, dY, W1, b1, W2 = (t.to(dev) for t in (Xc, dYc, W1c, b1c, W2c))
    Fs = w.Fs
    H = torch.empty((w.N, Fs), dtype=_tdt(w), device=dev)
    Z = torch.empty_like(H)
    P = torch.empty((w.N, w.D), device=dev)
    mt.mlp_tp_shard_fwd(X, W1, b1, W2, H, Z, P, w.N, w.D, w.F, w.T, _dt(w), w.act)
    dZ = torch.empty_like(H)
    dW1 = torch.empty((w.D, Fs), device=dev)
    dW2 = torch.empty((Fs, w.D), device=dev)
    db1 = torch.empty((Fs,), device=dev)
    dX = torch.empty((w.N, w.D), device=dev)
    nb = mt.mlp_tp_shard_bwd_workspace_bytes(w.N, w.D, w.F, w.T)
    ws = torch.empty((max(nb, 16),), dtype=torch.uint8, device=dev)
    mt.mlp_tp_shard_bwd(X, W1, W2, Z, H, dY, dZ, dW1, db1, dW2, dX, ws, ws.numel(), w.N, w.D,
                        w.F, w.T, _dt(w), w.act)
    torch.cuda.synchronize()
    Zr, Hr, Pr = oracle.shard_fwd(Xc, W1c, b1c, W2c, 1, 0, act=w.act)
    assert_close("Z", Z, Zr)
    assert_close("H", H, Hr)
    assert_close("P", P, Pr)
    g = oracle.shard_bwd(Xc, W1c, b1c, W2c, dYc, 1, 0, act=w.act)
    for name, t in (("dZ", dZ), ("dW1", dW1), ("db1", db1), ("dW2", dW2), ("dX", dX)):
        assert_close(name, t, g[name])


# --------------------------------------------------------------------------------------------
# Shard-count sweep on the pages' model shapes [Z 11]
# --------------------------------------------------------------------------------------------

class _Full:
    """One fixed full weight set; every shard of every T is a slice of it [Z 09]."""

    def __init__(self, w):
        self.w = w
        self.Xc = synth.gen_X(w)
        self.W1, self.b1 = synth.gen_W1(w), synth.gen_b1(w)
        self.W2, self.b2 = synth.gen_W2(w), synth.gen_b2(w)
        self.X = self.Xc.cuda()
        self.b2d = self.b2.cuda()


def _run_shards(full, T):
    """All T shards on the GPU: per rank the partial, and the partial with its b2/T share."""
    w = full.w.with_(T=T)
    Fs = w.Fs
    parts, shares = [], []
    H = torch.empty((w.N, Fs), dtype=torch.bfloat16, device="cuda")
    for r in range(T):
        c0, c1 = r * Fs, (r + 1) * Fs
        W1r = full.W1[:, c0:c1].contiguous().cuda()
        W2r = full.W2[c0:c1, :].contiguous().cuda()
        b1r = full.b1[c0:c1].contiguous().cuda()
        P = torch.empty((w.N, w.D), device="cuda")
        mt.mlp_tp_shard_fwd(full.X, W1r, b1r, W2r, H, None, P, w.N, w.D, w.F, T, mt.BF16, w.act)
        Ps = torch.empty((w.N, w.D), device="cuda")
        mt.mlp_tp_down_proj_bias_share(H, W2r, full.b2d, mt.BF16, Ps, w.N, w.D, w.F, T, mt.BF16)
        parts.append(P)
        shares.append(Ps)
        del W1r, W2r, b1r
    Y = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_partial_reduce(parts, T, full.b2d, mt.BF16, Y, w.N, w.D)
    Yshare = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_partial_reduce(shares, T, None, mt.BF16, Yshare, w.N, w.D)
    torch.cuda.synchronize()
    return parts, Y, Yshare


@pytest.mark.parametrize("base", [workloads.GPT2_MEDIUM_T2, workloads.LLAMA70B_SHARD_T8],
                         ids=lambda w: w.name)
def test_shard_count_sweep_sampled_rows(base):
    """T = 1, 2, 4, 8 shards of one full weight (GPT-2-medium: D 1024, F 4096; Llama-3-70B FFN:
    D 8192, F 28672; 4096 tokens): Y with b2 once, and with b2/T per rank, on sampled token rows
    against the oracle's sharded computation at the same T [Z 11], [Z 05]."""
    _say(f"  workload {base.name}")
    full = _Full(base)
    rows = _sample(base.N, 4, 11)
    Xrows = full.Xc[rows]
    for T in (1, 2, 4, 8):
        parts, Y, Yshare = _run_shards(full, T)
        Fs = base.F // T
        refs = []
        for r in range(T):
            c0, c1 = r * Fs, (r + 1) * Fs
            refs.append(oracle.shard_fwd(Xrows, full.W1[:, c0:c1], full.b1[c0:c1],
                                         full.W2[c0:c1, :], 1, 0, act=base.act)[2])
        assert_close(f"T={T} P[0] rows", parts[0][rows], refs[0])
        assert_close(f"T={T} Y rows", Y[rows], oracle.partial_sum(refs, full.b2))
        assert_close(f"T={T} Y (b2/T per rank) rows", Yshare[rows],
                     oracle.partial_sum_bias_share(refs, full.b2, T))
        _say(f"    T={T} done")
        del parts, Y, Yshare


# --------------------------------------------------------------------------------------------
# b2 split over the ranks on integer data [Z 05]
# --------------------------------------------------------------------------------------------

def _int_shards(w):
    Xc = synth.gen_X(w)
    X = Xc.cuda()
    b2 = synth.gen_b2(w)
    out = []
    for r in range(w.T):
        c0, c1 = r * w.Fs, (r + 1) * w.Fs
        W1, b1, W2 = synth.gen_W1(w, c0, c1), synth.gen_b1(w, c0, c1), synth.gen_W2(w, c0, c1)
        H = torch.empty((w.N, w.Fs), device="cuda")
        P = torch.empty((w.N, w.D), device="cuda")
        W2d = W2.cuda()
        mt.mlp_tp_up_proj(X, W1.cuda(), b1.cuda(), None, H, w.N, w.D, w.F, w.T, mt.F32, w.act)
        mt.mlp_tp_down_proj_bias_share(H, W2d, b2.cuda(), mt.F32, P, w.N, w.D, w.F, w.T, mt.F32)
        ref = oracle.shard_fwd(Xc, W1, b1, W2, 1, 0, act=w.act)[2]
        out.append((P, ref))
    torch.cuda.synchronize()
    return Xc, b2, out


@pytest.mark.parametrize("T", (1, 2, 4, 8))
def test_bias_share_bit_exact_on_integer_data(T):
    """Each rank's partial carries b2/T; the plain sum of the partials equals the b2-once
    block bit for bit (T a power of two: b2/T is exact)."""
    w = workloads.INT_EXACT.with_(T=T)
    Xc, b2, shards = _int_shards(w)
    for r, (P, ref) in enumerate(shards):
        assert_exact(f"P[{r}] + b2/T", P, oracle.partial_sum_bias_share([ref], b2, T))
    Y = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_partial_reduce([P for P, _ in shards], T, None, mt.F32, Y, w.N, w.D)
    torch.cuda.synchronize()
    once = oracle.block_fwd(Xc, synth.gen_W1(w), synth.gen_b1(w), synth.gen_W2(w), b2, T,
                            act=w.act)
    assert_exact("Y", Y, once)


def test_bias_share_at_three_ranks():
    """T = 3: b2/3 is rounded (to fp32 on the GPU, fp64 in the oracle); the result is within
    fp32 rounding of the oracle's b2/T tail and of the b2-once block."""
    w = workloads.INT_EXACT.with_(F=192, T=3)
    Xc, b2, shards = _int_shards(w)
    Y = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_partial_reduce([P for P, _ in shards], 3, None, mt.F32, Y, w.N, w.D)
    torch.cuda.synchronize()
    assert_close("Y (b2/3 per rank)", Y, oracle.partial_sum_bias_share([r for _, r in shards],
                                                                       b2, 3), 1e-6)
    once = oracle.block_fwd(Xc, synth.gen_W1(w), synth.gen_b1(w), synth.gen_W2(w), b2, 3,
                            act=w.act)
    assert_close("Y against b2 once", Y, once, 1e-6)


# --------------------------------------------------------------------------------------------
# Split contractions for products with too few tiles to fill the GPU [Z 04]
# --------------------------------------------------------------------------------------------

SPLIT_CASES = [
    # the pages' example shape (d_model 4096, d_ff 11008, 2 x 128 tokens) for each T
    workloads.PAGE_EXAMPLE_MLP.with_(T=1),
    workloads.PAGE_EXAMPLE_MLP.with_(T=8),
    # ragged everywhere: 200 tokens, D = 1000, Fs = 3000 (splits of the 3000- and 1000-deep
    # contractions end mid-stage)
    Workload("split_ragged_n200_d1000_f6000_t2", 200, 1000, 6000, 2, "gelu_erf", "bf16", 7301,
             "normal"),
]


@pytest.mark.parametrize("w", SPLIT_CASES, ids=lambda w: w.name)
def test_split_contraction_forward_matches_oracle(w):
    """mlp_tp_shard_fwd_ws with the workspace its query asks for: Z, H and P element by element
    against the oracle; the unsplit call agrees within the same bar; two calls agree bit for bit
    (the partials are summed in a fixed order); a workspace one byte short leaves the products
    unsplit, bit for bit mlp_tp_shard_fwd."""
    _say(f"  workload {w.name}")
    nb = mt.mlp_tp_shard_fwd_workspace_bytes(w.N, w.D, w.F, w.T)
    _say(f"    workspace {nb} bytes")
    assert nb > 0, "these shapes are meant to split on a 256-CU GPU"
    Xc = synth.gen_X(w)
    W1c, b1c, W2c = (synth.gen_W1(w, 0, w.Fs), synth.gen_b1(w, 0, w.Fs),
                     synth.gen_W2(w, 0, w.Fs))
    X, W1, b1, W2 = (t.cuda() for t in (Xc, W1c, b1c, W2c))
    ws = torch.empty((nb,), dtype=torch.uint8, device="cuda")

    def run(wsp, wsb):
        H = torch.empty((w.N, w.Fs), dtype=torch.bfloat16, device="cuda")
        Z = torch.empty_like(H)
        P = torch.empty((w.N, w.D), device="cuda")
        if wsp is None:
            mt.mlp_tp_shard_fwd(X, W1, b1, W2, H, Z, P, w.N, w.D, w.F, w.T, mt.BF16, w.act)
        else:
            mt.mlp_tp_shard_fwd_ws(X, W1, b1, W2, H, Z, P, wsp, wsb, w.N, w.D, w.F, w.T, mt.BF16,
                                   w.act)
        torch.cuda.synchronize()
        return Z, H, P

    Zs, Hs, Ps = run(ws, nb)
    Zr, Hr, Pr = oracle.shard_fwd(Xc, W1c, b1c, W2c, 1, 0, act=w.act)
    assert_close("Z (split)", Zs, Zr)
    assert_close("H (split)", Hs, Hr)
    assert_close("P (split)", Ps, Pr)
    Zu, Hu, Pu = run(None, 0)
    assert_close("P (unsplit)", Pu, Pr)
    again = run(ws, nb)
    assert all(torch.equal(a, b) for a, b in zip(again, (Zs, Hs, Ps))), "split not deterministic"
    short = run(ws, nb - 1)
    assert all(torch.equal(a, b) for a, b in zip(short, (Zu, Hu, Pu))), "short workspace split"
