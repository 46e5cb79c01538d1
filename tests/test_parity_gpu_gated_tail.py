"""GPU parity of the gated (SwiGLU) shard and of the two other forms of the block tail: the
token-sliced (reduce-scatter) reduction and the down-projection that accumulates into one
running fp32 sum. HIP library through the C ABI against the fp64 CPU oracle.

Bars as for the plain shard: bit-exact (==, no NaN) on integer-valued fp32 data; otherwise,
per output tensor, max|gpu - ref| / max|ref| <= 1e-2 (bf16 inputs, fp32 accumulation, bf16
stores of G, U and H).

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


def _np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(gpu, ref):
    g = _np(gpu)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    denom = np.max(np.abs(ref)) if ref.size else 0.0
    if denom == 0.0:
        return float(np.max(np.abs(g))) if g.size else 0.0
    return float(np.max(np.abs(g - ref)) / denom)


def assert_close(name, gpu, ref, tol=TOL):
    e = rel_err(gpu, ref)
    _say(f"    {name}: rel err {e:.3e}")
    assert e <= tol, f"{name}: rel err {e:.3e} > {tol}"


def assert_exact(name, gpu, ref):
    g = _np(gpu)
    assert not np.any(np.isnan(g)), name
    assert np.array_equal(g, np.asarray(ref, dtype=np.float64)), f"{name}: not bit-exact"


def _sample(n, extra, seed):
    rng = np.random.default_rng(seed)
    base = [0, 1, 63, 64, 127, 128, n // 2 - 1, n // 2, n - 129, n - 128, n - 2, n - 1]
    base += list(rng.integers(0, n, size=extra))
    return np.array(sorted({int(i) for i in base if 0 <= i < n}))


# --------------------------------------------------------------------------------------------
# Gated (SwiGLU) shard [Z 08]
# --------------------------------------------------------------------------------------------

GATED = [
    # bf16, D and Fs multiples of 8: the fused gate+up GEMM, ragged token and column tails
    Workload("gated_n300_d520_f1552_t2", 300, 520, 1552, 2, "swiglu", "bf16", 8001, "normal",
             bias=False),
    # exact tile multiples, four shards
    Workload("gated_n256_d256_f1024_t4", 256, 256, 1024, 4, "swiglu", "bf16", 8002, "normal",
             bias=False),
    # leading dimensions that are not multiples of 8: two GEMMs, gate staged in memory
    Workload("gated_n77_d200_f300_t3", 77, 200, 300, 3, "swiglu", "bf16", 8003, "normal",
             bias=False),
    # fp32 storage (not exact data): the two-GEMM form in fp32, fp32 tolerance
    Workload("gated_f32_n70_d48_f96_t2", 70, 48, 96, 2, "swiglu", "f32", 8004, "normal",
             bias=False),
]


class GatedShard:
    def __init__(self, w, X, r, keep_gu=True):
        c0, c1 = r * w.Fs, (r + 1) * w.Fs
        self.r = r
        self.Wg, self.Wu = synth.gen_Wg(w, c0, c1), synth.gen_Wu(w, c0, c1)
        self.W2 = synth.gen_W2(w, c0, c1)
        self.dWg, self.dWu, self.dW2 = self.Wg.cuda(), self.Wu.cuda(), self.W2.cuda()
        mk = lambda: torch.empty((w.N, w.Fs), dtype=_tdt(w), device="cuda")  # noqa: E731
        self.G = mk() if keep_gu else None
        self.U = mk() if keep_gu else None
        self.H = mk()
        self.P = torch.empty((w.N, w.D), dtype=torch.float32, device="cuda")
        mt.mlp_tp_swiglu_shard_fwd(X, self.dWg, self.dWu, self.dW2, self.G, self.U, self.H,
                                   self.P, w.N, w.D, w.F, w.T, _dt(w))


@pytest.mark.parametrize("w", GATED, ids=lambda w: w.name)
def test_gated_shards_and_block_elementwise(w):
    """Every rank's G, U, H and P against the oracle, then the sum of the T partials against
    the unsharded gated MLP: the gate and up shards cut at the same columns line up channel for
    channel [Z 08], [Z 10]."""
    _say(f"  workload {w.name}")
    Xc = synth.gen_X(w)
    X = Xc.cuda()
    tol = 1e-5 if w.dtype == "f32" else TOL
    shards = [GatedShard(w, X, r) for r in range(w.T)]
    Y = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_partial_reduce([s.P for s in shards], w.T, None, mt.F32, Y, w.N, w.D)
    torch.cuda.synchronize()
    for s in shards:
        G, U, H, P = oracle.swiglu_shard_fwd(Xc, s.Wg, s.Wu, s.W2, 1, 0)
        assert_close(f"G[{s.r}]", s.G, G, tol)
        assert_close(f"U[{s.r}]", s.U, U, tol)
        assert_close(f"H[{s.r}]", s.H, H, tol)
        assert_close(f"P[{s.r}]", s.P, P, tol)
    Yref = oracle.swiglu_dense_fwd(Xc, synth.gen_Wg(w), synth.gen_Wu(w), synth.gen_W2(w))
    assert_close("Y", Y, Yref, tol)


@pytest.mark.parametrize("w", GATED, ids=lambda w: w.name)
def test_gated_up_projection_without_kept_projections(w):
    """G and U are optional outputs: leaving them out must not change H."""
    Xc = synth.gen_X(w)
    X = Xc.cuda()
    kept = GatedShard(w, X, w.T - 1, keep_gu=True)
    H = torch.empty_like(kept.H)
    mt.mlp_tp_swiglu_up_proj(X, kept.dWg, kept.dWu, None, None, H, w.N, w.D, w.F, w.T, _dt(w))
    torch.cuda.synchronize()
    assert torch.equal(H, kept.H)


def test_gated_zero_tokens_is_a_no_op():
    Wg = torch.randn((64, 64), device="cuda").bfloat16()
    Wu = torch.randn((64, 64), device="cuda").bfloat16()
    W2 = torch.randn((64, 64), device="cuda").bfloat16()
    d = [torch.full((16,), 3.0, device="cuda",
                    dtype=torch.float32 if i == 4 else torch.bfloat16) for i in range(5)]
    mt.mlp_tp_swiglu_shard_fwd(d[0], Wg, Wu, W2, d[1], d[2], d[3], d[4], 0, 64, 128, 2, mt.BF16)
    torch.cuda.synchronize()
    for t in d:
        assert torch.all(t == 3.0)


def test_llama70b_gated_shard_full_size():
    """The gated form of the Llama-3-70B FFN shard (N=4096, D=8192, F/T=3584), on sampled
    token rows."""
    w = workloads.LLAMA70B_SWIGLU_SHARD_T8
    _say(f"  workload {w.name}")
    Xc = synth.gen_X(w)
    X = Xc.cuda()
    s = GatedShard(w, X, 0, keep_gu=False)
    torch.cuda.synchronize()
    rows = _sample(w.N, 6, 6)
    _, _, H, P = oracle.swiglu_shard_fwd(Xc[rows], s.Wg, s.Wu, s.W2, 1, 0)
    assert_close("H rows", s.H[rows], H)
    assert_close("P rows", s.P[rows], P)


def _run_gated_bwd(w, X, s, dY):
    dev = "cuda"
    out = {
        "dG": torch.empty((w.N, w.Fs), dtype=_tdt(w), device=dev),
        "dU": torch.empty((w.N, w.Fs), dtype=_tdt(w), device=dev),
        "dWg": torch.empty((w.D, w.Fs), dtype=torch.float32, device=dev),
        "dWu": torch.empty((w.D, w.Fs), dtype=torch.float32, device=dev),
        "dW2": torch.empty((w.Fs, w.D), dtype=torch.float32, device=dev),
        "dX": torch.empty((w.N, w.D), dtype=torch.float32, device=dev),
    }
    mt.mlp_tp_swiglu_shard_bwd(X, s.dWg, s.dWu, s.dW2, s.G, s.U, s.H, dY, out["dG"], out["dU"],
                               out["dWg"], out["dWu"], out["dW2"], out["dX"], w.N, w.D, w.F,
                               w.T, _dt(w))
    return out


GATED_GRADS = ("dG", "dU", "dWg", "dWu", "dW2", "dX")


@pytest.mark.parametrize("w", GATED, ids=lambda w: w.name)
def test_gated_backward_shards_and_summed_dx(w):
    """Every rank's gated gradients against the oracle (product rule through SiLU(G) * U
    [Z 08]); the dX partials summed over the ranks against the unsharded gated MLP's dX."""
    _say(f"  workload {w.name}")
    Xc, dYc = synth.gen_X(w), synth.gen_dY(w)
    X, dY = Xc.cuda(), dYc.cuda()
    tol = 1e-5 if w.dtype == "f32" else TOL
    parts = []
    for r in range(w.T):
        s = GatedShard(w, X, r)
        g = _run_gated_bwd(w, X, s, dY)
        torch.cuda.synchronize()
        ref = oracle.swiglu_shard_bwd(Xc, s.Wg, s.Wu, s.W2, dYc, 1, 0)
        for k in GATED_GRADS:
            assert_close(f"{k}[{r}]", g[k], ref[k], tol)
        parts.append(g["dX"])
    dX = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_partial_reduce(parts, w.T, None, mt.F32, dX, w.N, w.D)
    torch.cuda.synchronize()
    dense = oracle.swiglu_shard_bwd(Xc, synth.gen_Wg(w), synth.gen_Wu(w), synth.gen_W2(w), dYc,
                                    1, 0)
    assert_close("sum dX", dX, dense["dX"], tol)


def test_gated_backward_zero_tokens_zeroes_weight_gradients():
    """N = 0: dG, dU and dX are empty; the weight gradients are empty sums, written as 0."""
    D, F, T = 64, 128, 2
    Fs = F // T
    Wg = torch.randn((D, Fs), device="cuda").bfloat16()
    Wu = torch.randn((D, Fs), device="cuda").bfloat16()
    W2 = torch.randn((Fs, D), device="cuda").bfloat16()
    d = [torch.full((16,), 3.0, device="cuda",
                    dtype=torch.float32 if i == 7 else torch.bfloat16) for i in range(8)]
    dWg = torch.full((D, Fs), 5.0, device="cuda")
    dWu = torch.full((D, Fs), 5.0, device="cuda")
    dW2 = torch.full((Fs, D), 5.0, device="cuda")
    mt.mlp_tp_swiglu_shard_bwd(d[0], Wg, Wu, W2, d[1], d[2], d[3], d[4], d[5], d[6], dWg, dWu,
                               dW2, d[7], 0, D, F, T, mt.BF16)
    torch.cuda.synchronize()
    for t in (dWg, dWu, dW2):
        assert torch.all(t == 0.0)
    for t in d:
        assert torch.all(t == 3.0)


def test_llama70b_gated_backward_full_size():
    """Gated backward of the Llama-3-70B FFN shard (N=4096, D=8192, F/T=3584), dY ~ N(0,1):
    dG, dU and dX^(0) on sampled token rows; dWg, dWu and dW2 on sampled hidden columns."""
    w = workloads.LLAMA70B_SWIGLU_SHARD_T8
    _say(f"  workload {w.name}")
    Xc, dYc = synth.gen_X(w), synth.gen_dY(w)
    X, dY = Xc.cuda(), dYc.cuda()
    s = GatedShard(w, X, 0)
    g = _run_gated_bwd(w, X, s, dY)
    torch.cuda.synchronize()
    rows = _sample(w.N, 4, 14)
    cols = _sample(w.Fs, 4, 15)
    ref_rows = oracle.swiglu_shard_bwd(Xc[rows], s.Wg, s.Wu, s.W2, dYc[rows], 1, 0)
    for k in ("dG", "dU", "dX"):
        assert_close(f"{k} rows", g[k][rows], ref_rows[k])
    ref_cols = oracle.swiglu_shard_bwd(Xc, s.Wg[:, cols], s.Wu[:, cols], s.W2[cols, :], dYc, 1,
                                       0)
    assert_close("dG cols", g["dG"][:, cols], ref_cols["dG"])
    for k in ("dWg", "dWu"):
        assert_close(f"{k} cols", g[k][:, cols], ref_cols[k])
    assert_close("dW2 cols", g["dW2"][cols, :], ref_cols["dW2"])


# --------------------------------------------------------------------------------------------
# Block tail, reduce-scatter layout [Z 04]
# --------------------------------------------------------------------------------------------

def _int_parts(T, N, D, seed):
    return [synth.blocked_slice(seed + r, 1, (N, D), 0, 0, N, "int", 1.0) for r in range(T)]


@pytest.mark.parametrize("T,N,D,bias", [(2, 64, 1024, "bf16"), (4, 10, 8, None),
                                        (8, 3, 12, "f32"), (3, 17, 7, "f32"),
                                        (8, 2048, 12288, "f32")])
def test_reduce_scatter_slices_match_oracle(T, N, D, bias):
    """Every token slice r against the oracle, exact on integer data; b2 only in the slice's
    own rows; the slices put together equal the full block tail; the in-place form over a
    partial's own slice rows."""
    _say(f"  T={T} N={N} D={D} bias={bias}")
    parts_c = _int_parts(T, N, D, 950 + T)
    parts = [p.cuda() for p in parts_c]
    b2c = b2d = None
    if bias:
        w = Workload("scatter", N=N, D=D, F=T, T=T, act="identity", dtype="f32", seed=960 + T,
                     dist="int")
        b2c = synth.gen_b2(w)
        b2d = b2c.to(torch.bfloat16).cuda() if bias == "bf16" else b2c.cuda()
    bdt = mt.BF16 if bias == "bf16" else mt.F32
    Yfull = torch.empty((N, D), device="cuda")
    mt.mlp_tp_partial_reduce(parts, T, b2d, bdt, Yfull, N, D)
    slices = []
    for r in range(T):
        row0, rows = mt.mlp_tp_token_slice(N, T, r)
        assert (row0, rows) == oracle.token_slice(N, T, r)
        Yr = torch.full((max(rows, 1), D), 7.0, device="cuda")[:rows]
        mt.mlp_tp_partial_reduce_scatter(parts, T, r, b2d, bdt, Yr, N, D)
        torch.cuda.synchronize()
        if rows and N * D <= 1 << 20:
            assert_exact(f"Y slice {r}", Yr, oracle.partial_reduce_scatter(parts_c, r, b2c))
        elif rows:
            # large case: the oracle on the slice's rows only (every row is its own sum)
            sub = [p[row0:row0 + rows] for p in parts_c]
            assert_exact(f"Y slice {r}", Yr, oracle.partial_sum(sub, b2c))
        slices.append(Yr)
    assert torch.equal(torch.cat(slices), Yfull)
    # in place over partial s's own slice rows, for each r
    for r in range(T):
        row0, rows = mt.mlp_tp_token_slice(N, T, r)
        s = r % T
        view = parts[s][row0:row0 + rows]
        if rows == 0 or (row0 * D) % 4:
            continue  # nothing to write, or the slice's rows are not 16-byte aligned
        before = [p[row0:row0 + rows].clone() for p in parts]
        mt.mlp_tp_partial_reduce_scatter(parts, T, r, b2d, bdt, view, N, D)
        torch.cuda.synchronize()
        assert torch.equal(view, slices[r]), f"in-place slice {r}"
        parts[s][row0:row0 + rows] = before[s]


# --------------------------------------------------------------------------------------------
# Down-projection accumulating into one fp32 buffer [Z 02]
# --------------------------------------------------------------------------------------------

def _up(w, X, r):
    c0, c1 = r * w.Fs, (r + 1) * w.Fs
    W1, W2 = synth.gen_W1(w, c0, c1), synth.gen_W2(w, c0, c1)
    b1 = synth.gen_b1(w, c0, c1) if w.bias else None
    H = torch.empty((w.N, w.Fs), dtype=_tdt(w), device="cuda")
    mt.mlp_tp_up_proj(X, W1.cuda(), b1.cuda() if b1 is not None else None, None, H, w.N, w.D,
                      w.F, w.T, _dt(w), w.act)
    return W1, b1, W2, H


ACCUM = [
    workloads.INT_EXACT,
    Workload("accum_n300_d520_f1552_t2", 300, 520, 1552, 2, "gelu_tanh", "bf16", 8101,
             "normal"),
    Workload("accum_n77_d200_f300_t3", 77, 200, 300, 3, "gelu_tanh", "bf16", 8102, "normal"),
    Workload("accum_n130_d264_f896_t4", 130, 264, 896, 4, "relu", "bf16", 8103, "normal"),
]


@pytest.mark.parametrize("w", ACCUM, ids=lambda w: w.name)
def test_accumulating_down_projection(w):
    """T shards added in turn into one buffer seeded with b2: the block tail Y in one buffer.
    Exact on the integer workload; within the bf16 bar otherwise; and bit-identical to T
    separate partials reduced in rank order (the same fp32 adds in the same order)."""
    _say(f"  workload {w.name}")
    Xc = synth.gen_X(w)
    X = Xc.cuda()
    b2 = synth.gen_b2(w)
    Yacc = torch.zeros((w.N, w.D), device="cuda")
    parts, refs = [], []
    for r in range(w.T):
        W1, b1, W2, H = _up(w, X, r)
        dW2 = W2.cuda()
        mt.mlp_tp_down_proj_accumulate(H, dW2, Yacc, w.N, w.D, w.F, w.T, _dt(w))
        P = torch.empty((w.N, w.D), device="cuda")
        mt.mlp_tp_down_proj(H, dW2, P, w.N, w.D, w.F, w.T, _dt(w))
        parts.append(P)
        refs.append(oracle.shard_fwd(Xc, W1, b1, W2, 1, 0, act=w.act)[2])
    Ysep = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_partial_reduce(parts, w.T, None, mt.F32, Ysep, w.N, w.D)
    torch.cuda.synchronize()
    assert torch.equal(Yacc, Ysep)
    ref = oracle.partial_sum(refs)
    if w.dist == "int":
        assert_exact("sum P (accumulated)", Yacc, ref)
    else:
        assert_close("sum P (accumulated)", Yacc, ref)
    # a buffer seeded with b2 rows: Y = b2 + sum_r P^(r), b2 still counted once
    Yb = b2.to(torch.float32).cuda().expand(w.N, w.D).contiguous()
    for r in range(w.T):
        _, _, W2, H = _up(w, X, r)
        mt.mlp_tp_down_proj_accumulate(H, W2.cuda(), Yb, w.N, w.D, w.F, w.T, _dt(w))
    torch.cuda.synchronize()
    if w.dist == "int":
        assert_exact("b2 + sum P", Yb, ref + b2.double().numpy())
    else:
        assert_close("b2 + sum P", Yb, ref + b2.double().numpy())
