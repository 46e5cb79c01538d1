"""GPU parity of the block tail overlapped with the last shard's down-projection, and of the
shard-count sweep on the pages' example MLP shape. HIP library through the C ABI against the
fp64 CPU oracle.

Pages cited:
  [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
  [U] unpurerationalist.github.io, "LLM Systems 16: Model Parallel Training"
  [C] charliedreemur.github.io, "TP:Column / Row Parallel Linear 怎么切? MLP 和 attention 怎么切?"
  [F] 5688vip.com, "4、张量并行原理：张量切分方式（行并行、列并行）…"
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


def rel_err(gpu, ref):
    g = gpu.detach().to("cpu", torch.float64).numpy()
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    denom = np.max(np.abs(ref))
    return float(np.max(np.abs(g - ref)) / denom) if denom else float(np.max(np.abs(g)))


def assert_close(name, gpu, ref, tol=TOL):
    e = rel_err(gpu, ref)
    _say(f"    {name}: rel err {e:.3e}")
    assert e <= tol, f"{name}: rel err {e:.3e} > {tol}"


def _sample(n, extra, seed):
    rng = np.random.default_rng(seed)
    base = [0, 1, 63, 64, 127, 128, n // 2 - 1, n // 2, n - 129, n - 128, n - 2, n - 1]
    base += list(rng.integers(0, n, size=extra))
    return np.array(sorted({int(i) for i in base if 0 <= i < n}))


def _shard(w, X, r):
    c0, c1 = r * w.Fs, (r + 1) * w.Fs
    W1, W2 = synth.gen_W1(w, c0, c1), synth.gen_W2(w, c0, c1)
    b1 = synth.gen_b1(w, c0, c1) if w.bias else None
    H = torch.empty((w.N, w.Fs), dtype=_tdt(w), device="cuda")
    mt.mlp_tp_up_proj(X, W1.cuda(), b1.cuda() if b1 is not None else None, None, H, w.N, w.D,
                      w.F, w.T, _dt(w), w.act)
    return W1, b1, W2, H


OVERLAP = [
    # exact integer data: the overlapped tail must equal the oracle bit for bit
    (workloads.INT_EXACT, 16),
    # bf16, ragged token count: the last chunk is short; these small products run on the
    # 128 x 128 tile with ragged edges (the 256-class tiles' edges are covered by
    # test_parity_gpu_tiles.py)
    (Workload("overlap_n300_d520_f1552_t2", 300, 520, 1552, 2, "gelu_tanh", "bf16", 8201,
              "normal"), 128),
    (Workload("overlap_n515_d264_f1024_t4", 515, 264, 1024, 4, "relu", "bf16", 8202, "normal"),
     100),
    # one chunk covering everything
    (Workload("overlap_n64_d136_f272_t2", 64, 136, 272, 2, "gelu_tanh", "bf16", 8203, "normal"),
     4096),
]


@pytest.mark.parametrize("w,chunk", OVERLAP, ids=lambda x: getattr(x, "name", str(x)))
@pytest.mark.parametrize("two_streams", [True, False])
def test_overlapped_tail_matches_oracle_and_plain_tail(w, chunk, two_streams):
    """Shards 0 .. T-2 computed as usual; the last shard's down-projection runs in token chunks
    with the block tail of each finished chunk on a second stream [F 4.4.2]. Y must equal the
    plain path (the same kernels on the same rows, bit for bit) and the oracle [Z 05]."""
    _say(f"  workload {w.name} chunk {chunk} two_streams {two_streams}")
    Xc = synth.gen_X(w)
    X = Xc.cuda()
    b2 = synth.gen_b2(w) if w.bias else None
    b2d = b2.cuda() if b2 is not None else None
    parts, refs = [], []
    last = None
    for r in range(w.T):
        W1, b1, W2, H = _shard(w, X, r)
        P = torch.full((w.N, w.D), float("nan"), device="cuda")
        if r < w.T - 1:
            mt.mlp_tp_down_proj(H, W2.cuda(), P, w.N, w.D, w.F, w.T, _dt(w))
        else:
            last = (H, W2.cuda())
        parts.append(P)
        refs.append(oracle.shard_fwd(Xc, W1, b1, W2, 1, 0, act=w.act)[2])
    Y = torch.empty((w.N, w.D), device="cuda")
    side = torch.cuda.Stream() if two_streams else None
    mt.mlp_tp_down_proj_overlap_tail(last[0], last[1], parts, w.T, w.T - 1, b2d, _dt(w), Y, w.N,
                                     w.D, w.F, _dt(w), chunk, tail_stream=side)
    # Y is complete for work on the current stream; compare with the plain tail there.
    Yplain = torch.empty_like(Y)
    mt.mlp_tp_partial_reduce(parts, w.T, b2d, _dt(w), Yplain, w.N, w.D)
    torch.cuda.synchronize()
    assert torch.equal(Y, Yplain)
    ref = oracle.partial_sum(refs, b2)
    if w.dist == "int":
        g = Y.double().cpu().numpy()
        assert np.array_equal(g, ref), "not bit-exact"
    else:
        assert_close("Y", Y, ref)
    # in place over the last partial itself
    mt.mlp_tp_down_proj_overlap_tail(last[0], last[1], parts, w.T, w.T - 1, b2d, _dt(w),
                                     parts[-1], w.N, w.D, w.F, _dt(w), chunk, tail_stream=side)
    torch.cuda.synchronize()
    assert torch.equal(parts[-1], Yplain)


# --------------------------------------------------------------------------------------------
# Shard-count sweep on the pages' example MLP (d_model 4096, d_ff 11008, x [2, 128, 4096])
# --------------------------------------------------------------------------------------------

def test_shard_count_sweep_page_example():
    """T = 1, 2, 4, 8 column/row shards of the same weights [Z 11], [C 代码]: every T gives the
    same block output as the unsharded MLP (the oracle's dense result on sampled rows), and the
    T results agree with each other up to fp32 summation order."""
    base = workloads.PAGE_EXAMPLE_MLP
    Xc = synth.gen_X(base)
    X = Xc.cuda()
    rows = _sample(base.N, 6, 7)
    W1f, b1f, W2f = synth.gen_W1(base), synth.gen_b1(base), synth.gen_W2(base)
    b2 = synth.gen_b2(base)
    dense = oracle.dense_fwd(Xc[rows], W1f, b1f, W2f, b2, act=base.act)
    outs = {}
    for T in (1, 2, 4, 8):
        w = base.with_(T=T)
        parts = []
        for r in range(T):
            W1, b1, W2, H = _shard(w, X, r)
            P = torch.empty((w.N, w.D), device="cuda")
            mt.mlp_tp_down_proj(H, W2.cuda(), P, w.N, w.D, w.F, w.T, mt.BF16)
            parts.append(P)
        Y = torch.empty((w.N, w.D), device="cuda")
        mt.mlp_tp_partial_reduce(parts, T, b2.cuda(), mt.BF16, Y, w.N, w.D)
        torch.cuda.synchronize()
        assert_close(f"Y (T={T}) rows vs unsharded oracle", Y[rows], dense)
        outs[T] = Y
        del parts
    for T in (2, 4, 8):
        # H is the same element for element for every T (one output column per shard column);
        # only the grouping of the fp32 sum over the hidden units changes.
        assert_close(f"Y (T={T}) vs Y (T=1)", outs[T], outs[1].double().cpu().numpy(), 1e-5)
