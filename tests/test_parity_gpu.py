"""GPU parity: the HIP library (through the C ABI) against the fp64 CPU oracle.

Bars: bit-exact (==, no NaN) on integer-valued fp32 data; otherwise, per output tensor,
max|gpu - ref| / max|ref| <= 1e-2 (fp32 accumulation, bf16 inputs, H/Z/dZ stored as bf16).
Small and medium shapes are compared element by element; the full-size workloads are
compared on sampled token rows (and sampled hidden columns for the weight gradients), which
the oracle computes exactly because every row of P, Y, H, dZ, dX depends only on its own
token row and every column of dW1, dW2, db1 only on its own hidden column.

Pages cited:
  [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
  [C] charliedreemur.github.io, "TP:Column / Row Parallel Linear 怎么切? MLP 和 attention 怎么切?"
"""
import json
import os
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
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


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
    g = gpu.detach().to("cpu", torch.float64).numpy() if isinstance(gpu, torch.Tensor) else gpu
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    denom = np.max(np.abs(ref))
    if denom == 0.0:
        return float(np.max(np.abs(g)))
    return float(np.max(np.abs(g - ref)) / denom)


def assert_close(name, gpu, ref, tol=TOL):
    e = rel_err(gpu, ref)
    _say(f"    {name}: rel err {e:.3e}")
    assert e <= tol, f"{name}: rel err {e:.3e} > {tol}"


def assert_exact(name, gpu, ref):
    g = gpu.detach().to("cpu", torch.float64).numpy()
    assert not np.any(np.isnan(g)), name
    assert np.array_equal(g, np.asarray(ref, dtype=np.float64)), f"{name}: not bit-exact"


def _cols(w, r):
    return r * w.Fs, (r + 1) * w.Fs


def _sample(n, extra, seed):
    rng = np.random.default_rng(seed)
    base = [0, 1, 63, 64, 127, 128, n // 2 - 1, n // 2, n - 129, n - 128, n - 2, n - 1]
    base += list(rng.integers(0, n, size=extra))
    return np.array(sorted({int(i) for i in base if 0 <= i < n}))


class Shard:
    """Device buffers of one rank's forward shard, filled through the C ABI."""

    def __init__(self, w, X, r, want_z=True):
        self.w, self.r = w, r
        c0, c1 = _cols(w, r)
        self.W1 = synth.gen_W1(w, c0, c1)
        self.b1 = synth.gen_b1(w, c0, c1) if w.bias else None
        self.W2 = synth.gen_W2(w, c0, c1)
        dev = "cuda"
        self.dW1, self.dW2 = self.W1.to(dev), self.W2.to(dev)
        self.db1 = self.b1.to(dev) if self.b1 is not None else None
        self.H = torch.empty((w.N, w.Fs), dtype=_tdt(w), device=dev)
        self.Z = torch.empty((w.N, w.Fs), dtype=_tdt(w), device=dev) if want_z else None
        self.P = torch.empty((w.N, w.D), dtype=torch.float32, device=dev)
        mt.mlp_tp_shard_fwd(X, self.dW1, self.db1, self.dW2, self.H, self.Z, self.P, w.N, w.D,
                            w.F, w.T, _dt(w), w.act)


def _oracle_shard(w, X_cpu, shard, rows=None):
    Xr = X_cpu if rows is None else X_cpu[rows]
    return oracle.shard_fwd(Xr, shard.W1, shard.b1, shard.W2, 1, 0, act=w.act)


# --------------------------------------------------------------------------------------------
# The pages' worked example and the exact integer workload
# --------------------------------------------------------------------------------------------

def test_worked_example_bit_exact():
    """[Z 03]: x=[1,2] through the 2x4 W1 and 4x2 W2 under ReLU on two shards gives partials
    [1,2] and [3,3] and Y = [4,5]; with b2 = [1,-1] added once, [5,4]."""
    with open(os.path.join(GOLDEN, "worked_example_fwd.json")) as f:
        g = json.load(f)
    x = torch.tensor(g["x"], dtype=torch.float32, device="cuda")
    W1 = torch.tensor(g["W1"], dtype=torch.float32)
    W2 = torch.tensor(g["W2"], dtype=torch.float32)
    T = g["T"]
    parts = []
    for r in range(T):
        W1r = W1[:, 2 * r:2 * r + 2].contiguous().cuda()
        W2r = W2[2 * r:2 * r + 2, :].contiguous().cuda()
        H = torch.empty((1, 2), device="cuda")
        Z = torch.empty((1, 2), device="cuda")
        P = torch.empty((1, 2), device="cuda")
        mt.mlp_tp_shard_fwd(x, W1r, None, W2r, H, Z, P, 1, 2, 4, T, mt.F32, "relu")
        torch.cuda.synchronize()
        assert_exact("Z", Z, g["pre_activation_per_rank"][r])
        assert_exact("H", H, g["h_per_rank"][r])
        assert_exact("P", P, g["partial_per_rank"][r])
        parts.append(P)
    Y = torch.empty((1, 2), device="cuda")
    mt.mlp_tp_partial_reduce(parts, T, None, mt.F32, Y, 1, 2)
    torch.cuda.synchronize()
    assert_exact("Y", Y, g["Y_sharded"])
    b2 = torch.tensor([1.0, -1.0], device="cuda")
    mt.mlp_tp_partial_reduce(parts, T, b2, mt.F32, Y, 1, 2)
    torch.cuda.synchronize()
    assert_exact("Y+b2", Y, [[5.0, 4.0]])


@pytest.mark.parametrize("T", (1, 2, 4))
def test_integer_workload_bit_exact_for_every_T(T):
    """Uniform integers in [-2, 2], fp32, ReLU: every value is an exact integer, so every
    shard output and the block result must equal the oracle bit for bit, for any T [Z 11]."""
    w = workloads.INT_EXACT.with_(T=T)
    _say(f"  workload {w.name} T={T}")
    Xc = synth.gen_X(w)
    X = Xc.cuda()
    shards = [Shard(w, X, r) for r in range(T)]
    Y = torch.empty((w.N, w.D), device="cuda")
    b2 = synth.gen_b2(w)
    mt.mlp_tp_partial_reduce([s.P for s in shards], T, b2.cuda(), mt.F32, Y, w.N, w.D)
    torch.cuda.synchronize()
    for s in shards:
        Z, H, P = _oracle_shard(w, Xc, s)
        assert_exact(f"Z[{s.r}]", s.Z, Z)
        assert_exact(f"H[{s.r}]", s.H, H)
        assert_exact(f"P[{s.r}]", s.P, P)
    W1 = synth.gen_W1(w)
    Yref = oracle.block_fwd(Xc, W1, synth.gen_b1(w), synth.gen_W2(w), b2, T, act=w.act)
    assert_exact("Y", Y, Yref)
    # b2 exactly once [Z 05]: Y - sum_r P^(r) == b2
    raw = sum(s.P.double() for s in shards)
    assert torch.equal((Y.double() - raw).cpu(), b2.double().expand(w.N, w.D))


def test_integer_backward_bit_exact():
    """Backward on integer data (fp32, ReLU): dZ, dW1, db1, dW2 and dX exact; the dX partials
    summed over the shards equal the unsharded dX [Z 06]."""
    w = workloads.INT_EXACT
    Xc = synth.gen_X(w)
    dYc = synth.gen_dY(w)
    X, dY = Xc.cuda(), dYc.cuda()
    parts = []
    for r in range(w.T):
        s = Shard(w, X, r)
        g = _run_bwd(w, X, s, dY)
        torch.cuda.synchronize()
        ref = oracle.shard_bwd(Xc, s.W1, s.b1, s.W2, dYc, 1, 0, act=w.act)
        for k in ("dZ", "dW1", "db1", "dW2", "dX"):
            assert_exact(f"{k}[{r}]", g[k], ref[k])
        parts.append(g["dX"])
    dX = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_partial_reduce(parts, w.T, None, mt.F32, dX, w.N, w.D)
    torch.cuda.synchronize()
    dense = oracle.dense_bwd(Xc, synth.gen_W1(w), synth.gen_b1(w), synth.gen_W2(w), dYc,
                             act=w.act)
    assert_exact("sum dX", dX, dense["dX"])


def _run_bwd(w, X, s, dY, want_db1=True):
    dev = "cuda"
    out = {
        "dZ": torch.empty((w.N, w.Fs), dtype=_tdt(w), device=dev),
        "dW1": torch.empty((w.D, w.Fs), dtype=torch.float32, device=dev),
        "db1": torch.empty((w.Fs,), dtype=torch.float32, device=dev) if want_db1 else None,
        "dW2": torch.empty((w.Fs, w.D), dtype=torch.float32, device=dev),
        "dX": torch.empty((w.N, w.D), dtype=torch.float32, device=dev),
    }
    nbytes = mt.mlp_tp_shard_bwd_workspace_bytes(w.N, w.D, w.F, w.T)
    ws = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=dev)
    mt.mlp_tp_shard_bwd(X, s.dW1, s.dW2, s.Z, s.H, dY, out["dZ"], out["dW1"], out["db1"],
                        out["dW2"], out["dX"], ws, ws.numel(), w.N, w.D, w.F, w.T, _dt(w), w.act)
    return out


# --------------------------------------------------------------------------------------------
# Element-by-element parity on shapes that span several tiles with ragged tails
# --------------------------------------------------------------------------------------------

RAGGED = [
    # several 128-tiles with ragged M, N and K; every leading dimension a multiple of 8
    Workload("ragged_n300_d520_f1552_t2", 300, 520, 1552, 2, "gelu_tanh", "bf16", 7001, "normal"),
    # leading dimensions that are not multiples of 8: element loads
    Workload("odd_n77_d200_f300_t3", 77, 200, 300, 3, "relu", "bf16", 7002, "normal"),
    # output rows not a multiple of 4: element stores
    Workload("tiny_n33_d36_f36_t2", 33, 36, 36, 2, "gelu_erf", "bf16", 7003, "normal"),
    # exact tile multiples
    Workload("even_n256_d256_f512_t2", 256, 256, 512, 2, "gelu_sigmoid", "bf16", 7004, "normal"),
    Workload("identity_n130_d264_f272_t4", 130, 264, 272, 4, "identity", "bf16", 7005, "normal"),
    # fp32 storage on normal data (not exact): fp32 tolerance
    Workload("f32_n70_d48_f96_t2", 70, 48, 96, 2, "gelu_tanh", "f32", 7006, "normal"),
    # no biases
    Workload("nobias_n128_d128_f256_t2", 128, 128, 256, 2, "gelu_tanh", "bf16", 7007, "normal",
             bias=False),
    # Shapes that fill the GPU with the large tiles (small ones take the 128 x 128 tile); a short
    # contraction keeps the oracle cheap, and D = 72 is one full and one partial k stage.
    # up-projection and dH on 256 x 224 (Fs = 16 x 224, 256 tiles)
    Workload("tile224_n4096_d72_f3584_t1", 4096, 72, 3584, 1, "gelu_tanh", "bf16", 7008, "normal"),
    # up-projection on 256 x 192 (Fs = 32 x 192, 256 tiles)
    Workload("tile192_n2048_d72_f6144_t1", 2048, 72, 6144, 1, "gelu_tanh", "bf16", 7009, "normal"),
    # down-projection and dX on 256 x 256 (256 tiles)
    Workload("tile256_n4096_d4096_f64_t1", 4096, 4096, 64, 1, "gelu_tanh", "bf16", 7012,
             "normal"),
    # down-projection on 224 x 256 (N = 16 x 224 tokens, 256 tiles)
    Workload("tile224m_n3584_d4096_f64_t1", 3584, 4096, 64, 1, "gelu_tanh", "bf16", 7013,
             "normal"),
    # contraction shorter than one 64-deep stage (K = 40 up, 48 down): one partial stage
    Workload("kshort_n130_d40_f96_t2", 130, 40, 96, 2, "gelu_tanh", "bf16", 7010, "normal"),
    # contraction of exactly one stage (K = 64 both ways)
    Workload("kone_n64_d64_f128_t2", 64, 64, 128, 2, "gelu_tanh", "bf16", 7011, "normal"),
]


@pytest.mark.parametrize("w", RAGGED, ids=lambda w: w.name)
def test_forward_block_elementwise(w):
    _say(f"  workload {w.name}")
    Xc = synth.gen_X(w)
    X = Xc.cuda()
    shards = [Shard(w, X, r) for r in range(w.T)]
    b2 = synth.gen_b2(w) if w.bias else None
    Y = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_partial_reduce([s.P for s in shards], w.T, b2.cuda() if b2 is not None else None,
                             _dt(w), Y, w.N, w.D)
    torch.cuda.synchronize()
    tol = 1e-5 if w.dtype == "f32" else TOL
    for s in shards:
        Z, H, P = _oracle_shard(w, Xc, s)
        assert_close(f"Z[{s.r}]", s.Z, Z, tol)
        assert_close(f"H[{s.r}]", s.H, H, tol)
        assert_close(f"P[{s.r}]", s.P, P, tol)
    Yref = oracle.block_fwd(Xc, synth.gen_W1(w), synth.gen_b1(w) if w.bias else None,
                            synth.gen_W2(w), b2, w.T, act=w.act)
    assert_close("Y", Y, Yref, tol)


def test_huge_leading_dimension_takes_register_staged_kernel():
    """D = 4194368: one 256-row tile of X spans more than 2^31 bytes, past what the direct-to-LDS
    kernel's 32-bit tile offsets cover, so the up-projection runs on the register-staged kernel
    (the down-projection's W2 tile spans 64 rows and stays on the direct kernel). Z, H and P
    against the oracle."""
    w = Workload("hugeld_n8_d4194368_f16_t1", 8, 4194368, 16, 1, "gelu_tanh", "bf16", 7100,
                 "normal")
    _say(f"  workload {w.name}")
    Xc = synth.gen_X(w)
    X = Xc.cuda()
    s = Shard(w, X, 0)
    torch.cuda.synchronize()
    Z, H, P = _oracle_shard(w, Xc, s)
    assert_close("Z", s.Z, Z)
    assert_close("H", s.H, H)
    assert_close("P", s.P, P)


@pytest.mark.parametrize("act", ["identity", "relu", "gelu_tanh", "gelu_erf", "gelu_sigmoid"])
@pytest.mark.parametrize("dtype,N,F,T,bias", [("bf16", 77, 200, 2, True), ("bf16", 33, 60, 2, True),
                                              ("f32", 64, 96, 1, True), ("bf16", 50, 128, 4, False),
                                              ("f32", 9, 30, 3, False)])
def test_bias_act_matches_oracle(act, dtype, N, F, T, bias):
    """The epilogue on its own [Z 02], [Z 05]: phi(Z + b1) against the oracle's phi in fp64 on the
    same values. Fs = 100, 128 and 96 take the vector path, 30 and 10 the element path."""
    Fs = F // T
    g = torch.Generator().manual_seed(4000 + N + F)
    Zc = torch.randn((N, Fs), generator=g) * 2.0
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    bc = (torch.randn((Fs,), generator=g) * 0.5).to(tdt) if bias else None
    H = torch.empty((N, Fs), dtype=tdt, device="cuda")
    mt.mlp_tp_bias_act(Zc.cuda(), bc.cuda() if bias else None, H, N, F, T,
                       mt.BF16 if dtype == "bf16" else mt.F32, act)
    torch.cuda.synchronize()
    pre = Zc.double().numpy() + (bc.double().numpy() if bias else 0.0)
    ref = oracle.act(act, pre)
    assert_close(f"H ({act})", H, ref, TOL if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("act", ["identity", "relu", "gelu_tanh", "gelu_erf", "gelu_sigmoid"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_activations_far_from_zero_and_at_zero(act, dtype):
    """phi at pre-activations from -1e4 to 1e4, at +-0 and at tiny values, element by element
    with a relative bound (the max-normalised error of the other tests would hide the small
    outputs): the saturating GELU forms must give z far right and 0 far left, not inf or NaN,
    and the erf form must not lose the small outputs of negative z to cancellation.
    The bound is rtol |ref| + 1e-15: rtol is 1e-2 for bf16 storage and 1e-4 for fp32 (an
    exponential of an argument near 70 carries about 70 fp32 epsilons of relative error), and
    1e-15 covers the fp64 oracle's own absolute error where its 1 + erf or 1 + tanh cancels."""
    mags = [0.0, 1e-30, 1e-8, 1e-3, 0.1, 0.5, 1.0, 2.0, 3.0, 5.0, 8.0, 12.0, 20.0, 50.0, 100.0,
            1e3, 1e4]
    vals = sorted({s * m for m in mags for s in (1.0, -1.0)} | {-0.0})
    Fs = 8 * ((len(vals) + 7) // 8)
    Zc = torch.zeros((4, Fs), dtype=torch.float32)
    Zc[0, :len(vals)] = torch.tensor(vals, dtype=torch.float32)
    Zc[1, :len(vals)] = torch.tensor(vals[::-1], dtype=torch.float32)
    Zc[2] = Zc[0] * 0.75
    Zc[3] = -Zc[1] * 1.5
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    H = torch.empty((4, Fs), dtype=tdt, device="cuda")
    mt.mlp_tp_bias_act(Zc.cuda(), None, H, 4, Fs, 1, mt.BF16 if dtype == "bf16" else mt.F32, act)
    torch.cuda.synchronize()
    h = H.double().cpu().numpy()
    ref = oracle.act(act, Zc.double().numpy())
    assert np.all(np.isfinite(h)), f"{act}: non-finite outputs {h[~np.isfinite(h)]}"
    rtol = 1e-2 if dtype == "bf16" else 1e-4
    bad = np.abs(h - ref) > rtol * np.abs(ref) + 1e-15
    assert not bad.any(), (f"{act} ({dtype}): z={Zc.double().numpy()[bad][:6]} "
                           f"gpu={h[bad][:6]} ref={ref[bad][:6]}")


@pytest.mark.parametrize("act", ["identity", "relu", "gelu_tanh", "gelu_erf", "gelu_sigmoid"])
def test_activation_derivative_far_from_zero_and_at_zero(act):
    """phi' through the backward's dH GEMM epilogue [Z 06], element by element: with W2^(r) the
    identity and dY all ones, dH = 1 and the stored dZ is phi'(Z) rounded to bf16. Z spans -1e4
    to 1e4 with +-0 and tiny values; all outputs finite, ReLU'(0) = 0, and each element within
    1e-2 |ref| + atol(z). The fp64 oracle evaluates 1 + tanh(u), 1 - tanh(u)^2 and 1 - sigmoid
    as written, which keep only an absolute ~1e-16 once they approach 0 (z near -7 for the tanh
    form), and phi' multiplies that by z du; atol(z) = 4e-16 (1 + |z| max(du, 1.702)) + 1e-15
    with du = sqrt(2/pi) (1 + 3 (0.044715) z^2) covers exactly that and nothing more."""
    mags = [0.0, 1e-30, 1e-8, 1e-3, 0.1, 0.5, 1.0, 2.0, 3.0, 5.0, 8.0, 12.0, 20.0, 50.0, 100.0,
            1e3, 1e4]
    vals = sorted({s * m for m in mags for s in (1.0, -1.0)} | {-0.0})
    N, Fs = 64, 64
    D, F, T = Fs, Fs, 1
    Zc = torch.zeros((N, Fs), dtype=torch.float32)
    for r in range(N):
        Zc[r, :len(vals)] = torch.tensor(vals, dtype=torch.float32) * (1.0 + 0.01 * r)
    Zb = Zc.to(torch.bfloat16)
    dev = "cuda"
    Z = Zb.to(dev)
    W2 = torch.eye(Fs, D, dtype=torch.bfloat16, device=dev)
    dY = torch.ones((N, D), dtype=torch.bfloat16, device=dev)
    X = torch.zeros((N, D), dtype=torch.bfloat16, device=dev)
    W1 = torch.zeros((D, Fs), dtype=torch.bfloat16, device=dev)
    H = torch.zeros((N, Fs), dtype=torch.bfloat16, device=dev)
    dZ = torch.empty((N, Fs), dtype=torch.bfloat16, device=dev)
    dW1 = torch.empty((D, Fs), device=dev)
    dW2 = torch.empty((Fs, D), device=dev)
    db1 = torch.empty((Fs,), device=dev)
    dX = torch.empty((N, D), device=dev)
    nb = mt.mlp_tp_shard_bwd_workspace_bytes(N, D, F, T)
    ws = torch.empty((max(nb, 16),), dtype=torch.uint8, device=dev)
    mt.mlp_tp_shard_bwd(X, W1, W2, Z, H, dY, dZ, dW1, db1, dW2, dX, ws, ws.numel(), N, D, F, T,
                        mt.BF16, act)
    torch.cuda.synchronize()
    g = dZ.double().cpu().numpy()
    z = Zb.double().numpy()
    ref = oracle.act_deriv(act, z)
    assert np.all(np.isfinite(g)), f"{act}: non-finite phi'"
    du = np.sqrt(2.0 / np.pi) * (1.0 + 3.0 * 0.044715 * z * z)
    atol = 4e-16 * (1.0 + np.abs(z) * np.maximum(du, 1.702)) + 1e-15
    bad = np.abs(g - ref) > 1e-2 * np.abs(ref) + atol
    assert not bad.any(), (f"{act}: z={Zb.double().numpy()[bad][:6]} gpu={g[bad][:6]} "
                           f"ref={ref[bad][:6]}")
    if act == "relu":
        assert np.all(g[Zb.double().numpy() == 0.0] == 0.0)


def test_unfused_epilogue_equals_fused_up_projection():
    """The same GEMM writing its fp32 result (the down-projection entry point on X and W1^(r)),
    then the standalone epilogue, gives the fused up-projection's H bit for bit: the same fp32
    sums, the same bias add, phi and rounding."""
    w = Workload("unfused_n300_d520_f1552_t2", 300, 520, 1552, 2, "gelu_tanh", "bf16", 7020,
                 "normal")
    Xc = synth.gen_X(w)
    X = Xc.cuda()
    s = Shard(w, X, 0)
    Z32 = torch.empty((w.N, w.Fs), device="cuda")
    # P[N, D'] = H'[N, F'/T'] W2'[F'/T', D'] with H' = X, W2' = W1^(r): D' = Fs, F' = D, T' = 1.
    mt.mlp_tp_down_proj(X, s.dW1, Z32, w.N, w.Fs, w.D, 1, mt.BF16)
    H = torch.empty_like(s.H)
    mt.mlp_tp_bias_act(Z32, s.db1, H, w.N, w.F, w.T, mt.BF16, w.act)
    torch.cuda.synchronize()
    assert torch.equal(H, s.H)


@pytest.mark.parametrize("w", [x for x in RAGGED if x.act != "relu"], ids=lambda w: w.name)
def test_backward_shard_elementwise(w):
    """ReLU backward on real-valued data is left to the exact integer test: there the sign of
    Z, which decides phi', is exact on both sides."""
    _say(f"  workload {w.name}")
    Xc, dYc = synth.gen_X(w), synth.gen_dY(w)
    X, dY = Xc.cuda(), dYc.cuda()
    tol = 1e-5 if w.dtype == "f32" else TOL
    parts = []
    for r in range(w.T):
        s = Shard(w, X, r)
        g = _run_bwd(w, X, s, dY)
        torch.cuda.synchronize()
        ref = oracle.shard_bwd(Xc, s.W1, s.b1, s.W2, dYc, 1, 0, act=w.act)
        for k in ("dZ", "dW1", "db1", "dW2", "dX"):
            assert_close(f"{k}[{r}]", g[k], ref[k], tol)
        parts.append(g["dX"])
    dX = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_partial_reduce(parts, w.T, None, mt.F32, dX, w.N, w.D)
    torch.cuda.synchronize()
    dense = oracle.dense_bwd(Xc, synth.gen_W1(w), synth.gen_b1(w) if w.bias else None,
                             synth.gen_W2(w), dYc, act=w.act)
    assert_close("sum dX", dX, dense["dX"], tol)


# --------------------------------------------------------------------------------------------
# Block-tail reduction on its own
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,N,D,bias", [(1, 5, 8, "f32"), (2, 64, 1024, "bf16"),
                                        (8, 33, 12, "f32"), (3, 17, 7, "f32"),
                                        (64, 9, 16, "bf16"), (5, 40, 100, None)])
def test_partial_reduce_matches_oracle(T, N, D, bias):
    w = Workload("reduce", N=N, D=D, F=T, T=T, act="identity", dtype="f32", seed=900 + T,
                 dist="int")
    parts_c = [synth.blocked_slice(901 + r, 1, (N, D), 0, 0, N, "int", 1.0) for r in range(T)]
    parts = [p.cuda() for p in parts_c]
    b2c = None
    if bias:
        b2c = synth.gen_b2(w)
        b2d = b2c.to(torch.bfloat16).cuda() if bias == "bf16" else b2c.cuda()
    Y = torch.empty((N, D), device="cuda")
    mt.mlp_tp_partial_reduce(parts, T, b2d if bias else None,
                             mt.BF16 if bias == "bf16" else mt.F32, Y, N, D)
    torch.cuda.synchronize()
    assert_exact("Y", Y, oracle.partial_sum(parts_c, b2c))
    # in place: Y aliases the first partial
    mt.mlp_tp_partial_reduce(parts, T, b2d if bias else None,
                             mt.BF16 if bias == "bf16" else mt.F32, parts[0], N, D)
    torch.cuda.synchronize()
    assert_exact("Y in place", parts[0], oracle.partial_sum(parts_c, b2c))


def test_zero_tokens_leave_outputs_untouched_and_zero_weight_grads():
    """N = 0 tokens: the forward is a no-op and the weight gradients are empty sums (zeros)."""
    W1 = torch.randn((64, 64), device="cuda").bfloat16()
    W2 = torch.randn((64, 64), device="cuda").bfloat16()
    # Zero-row activations still need valid aligned pointers: small placeholders of each
    # argument's element type (P and dXr are float, the rest bf16).
    d = [torch.full((16,), 3.0, device="cuda",
                    dtype=torch.float32 if i in (3, 6) else torch.bfloat16) for i in range(8)]
    mt.mlp_tp_shard_fwd(d[0], W1, None, W2, d[1], d[2], d[3], 0, 64, 128, 2, mt.BF16,
                        "gelu_tanh")
    dW1 = torch.full((64, 64), 7.0, device="cuda")
    dW2 = torch.full((64, 64), 7.0, device="cuda")
    db1 = torch.full((64,), 7.0, device="cuda")
    mt.mlp_tp_shard_bwd(d[0], W1, W2, d[1], d[2], d[4], d[5], dW1, db1, dW2, d[6], None, 0,
                        0, 64, 128, 2, mt.BF16, "gelu_tanh")
    torch.cuda.synchronize()
    for t in d:
        assert torch.all(t == 3.0)
    assert torch.count_nonzero(dW1) == 0 and torch.count_nonzero(dW2) == 0
    assert torch.count_nonzero(db1) == 0


def test_results_are_deterministic():
    w = RAGGED[0]
    X = synth.gen_X(w).cuda()
    dY = synth.gen_dY(w).cuda()
    a = Shard(w, X, 1)
    b = Shard(w, X, 1)
    torch.cuda.synchronize()
    assert torch.equal(a.P, b.P) and torch.equal(a.H, b.H) and torch.equal(a.Z, b.Z)
    ga, gb = _run_bwd(w, X, a, dY), _run_bwd(w, X, b, dY)
    torch.cuda.synchronize()
    for k in ga:
        assert torch.equal(ga[k], gb[k]), k


# --------------------------------------------------------------------------------------------
# Full-size workloads: sampled outputs
# --------------------------------------------------------------------------------------------

def test_gpt2_medium_two_shards_full_size():
    """Both shards and the reduce at N=4096, D=1024, F=4096, T=2 (bf16, GELU-tanh)."""
    w = workloads.GPT2_MEDIUM_T2
    _say(f"  workload {w.name}")
    Xc = synth.gen_X(w)
    X = Xc.cuda()
    shards = [Shard(w, X, r, want_z=False) for r in range(w.T)]
    b2 = synth.gen_b2(w)
    Y = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_partial_reduce([s.P for s in shards], w.T, b2.cuda(), mt.BF16, Y, w.N, w.D)
    torch.cuda.synchronize()
    rows = _sample(w.N, 8, 1)
    refs = []
    for s in shards:
        _, H, P = _oracle_shard(w, Xc, s, rows)
        assert_close(f"H[{s.r}] rows", s.H[rows], H)
        assert_close(f"P[{s.r}] rows", s.P[rows], P)
        refs.append(P)
    assert_close("Y rows", Y[rows], oracle.partial_sum(refs, b2))


def test_llama70b_shard_full_size():
    """One rank's shard at N=4096, D=8192, F/T=3584 (shard 0 of F=28672), the headline
    forward, exactly as the benchmark launches it (up-projection then down-projection)."""
    w = workloads.LLAMA70B_SHARD_T8
    _say(f"  workload {w.name}")
    Xc = synth.gen_X(w)
    X = Xc.cuda()
    c0, c1 = _cols(w, 0)

    class S:
        pass

    s = S()
    s.W1, s.b1, s.W2 = synth.gen_W1(w, c0, c1), synth.gen_b1(w, c0, c1), synth.gen_W2(w, c0, c1)
    H = torch.empty((w.N, w.Fs), dtype=torch.bfloat16, device="cuda")
    P = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_up_proj(X, s.W1.cuda(), s.b1.cuda(), None, H, w.N, w.D, w.F, w.T, mt.BF16, w.act)
    mt.mlp_tp_down_proj(H, s.W2.cuda(), P, w.N, w.D, w.F, w.T, mt.BF16)
    torch.cuda.synchronize()
    rows = _sample(w.N, 6, 2)
    _, Hr, Pr = oracle.shard_fwd(Xc[rows], s.W1, s.b1, s.W2, 1, 0, act=w.act)
    assert_close("H rows", H[rows], Hr)
    assert_close("P rows", P[rows], Pr)


def test_gpt3_175b_eight_shards_and_reduce_full_size():
    """8 shards of F/T=6144 in sequence on one GPU (N=2048, D=12288), then the block tail
    with b2 added once; checked on sampled rows of Y and of P^(0)."""
    w = workloads.GPT3_175B_T8
    _say(f"  workload {w.name}")
    Xc = synth.gen_X(w)
    X = Xc.cuda()
    rows = _sample(w.N, 4, 3)
    parts, refs = [], []
    H = torch.empty((w.N, w.Fs), dtype=torch.bfloat16, device="cuda")
    for r in range(w.T):
        c0, c1 = _cols(w, r)
        W1, b1, W2 = synth.gen_W1(w, c0, c1), synth.gen_b1(w, c0, c1), synth.gen_W2(w, c0, c1)
        P = torch.empty((w.N, w.D), device="cuda")
        mt.mlp_tp_shard_fwd(X, W1.cuda(), b1.cuda(), W2.cuda(), H, None, P, w.N, w.D, w.F, w.T,
                            mt.BF16, w.act)
        parts.append(P)
        refs.append(oracle.shard_fwd(Xc[rows], W1, b1, W2, 1, 0, act=w.act)[2])
        _say(f"    shard {r} done")
    b2 = synth.gen_b2(w)
    Y = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_partial_reduce(parts, w.T, b2.cuda(), mt.BF16, Y, w.N, w.D)
    torch.cuda.synchronize()
    assert_close("P[0] rows", parts[0][rows], refs[0])
    assert_close("Y rows", Y[rows], oracle.partial_sum(refs, b2))


def test_llama70b_backward_full_size():
    """Backward of the shard at N=4096, D=8192, F/T=3584 with dY ~ N(0,1): dZ and dX^(0) on
    sampled token rows, dW1, dW2 and db1 on sampled hidden columns; then the dX partials of
    all 8 shards summed on one GPU, on sampled rows."""
    w = workloads.LLAMA70B_SHARD_T8_BWD
    _say(f"  workload {w.name}")
    Xc, dYc = synth.gen_X(w), synth.gen_dY(w)
    X, dY = Xc.cuda(), dYc.cuda()
    rows = _sample(w.N, 4, 4)
    cols = _sample(w.Fs, 4, 5)
    dx_parts, dx_refs = [], []
    for r in range(w.T):
        s = Shard(w, X, r)
        g = _run_bwd(w, X, s, dY)
        torch.cuda.synchronize()
        ref_rows = oracle.shard_bwd(Xc[rows], s.W1, s.b1, s.W2, dYc[rows], 1, 0, act=w.act,
                                    want=("dZ", "dX"))
        if r == 0:
            assert_close("dZ rows", g["dZ"][rows], ref_rows["dZ"])
            assert_close("dX[0] rows", g["dX"][rows], ref_rows["dX"])
            ref_cols = oracle.shard_bwd(Xc, s.W1[:, cols], s.b1[cols], s.W2[cols, :], dYc, 1, 0,
                                        act=w.act, want=("dZ", "dW1", "db1", "dW2"))
            assert_close("dW1 cols", g["dW1"][:, cols], ref_cols["dW1"])
            assert_close("dW2 cols", g["dW2"][cols, :], ref_cols["dW2"])
            assert_close("db1 cols", g["db1"][cols], ref_cols["db1"])
        dx_parts.append(g["dX"])
        dx_refs.append(ref_rows["dX"])
        del s, g
        _say(f"    shard {r} done")
    dX = torch.empty((w.N, w.D), device="cuda")
    mt.mlp_tp_partial_reduce(dx_parts, w.T, None, mt.F32, dX, w.N, w.D)
    torch.cuda.synchronize()
    assert_close("sum dX rows", dX[rows], oracle.partial_sum(dx_refs))
