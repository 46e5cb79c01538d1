"""The allocation-free backward (mlp_tp_shard_bwd_noalloc) against mlp_tp_shard_bwd.

It runs the same kernels with the library's own per-GPU device buffer as the column sum's
workspace, so its outputs must equal those of the workspace-argument entry point bit for bit.
Two calls in a row, the second on a smaller input, check that the buffer's previous contents
do not leak into a later result.
"""
import sys

import pytest
import torch

from tensor_mlp_block_amd import binding as mt
from tensor_mlp_block_amd import synth
from tensor_mlp_block_amd.workloads import Workload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(w):
    dev = "cuda"
    X, dY = synth.gen_X(w).to(dev), synth.gen_dY(w).to(dev)
    W1, b1, W2 = synth.gen_W1(w).to(dev), synth.gen_b1(w).to(dev), synth.gen_W2(w).to(dev)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dt = mt.BF16 if w.dtype == "bf16" else mt.F32
    H = torch.empty((w.N, w.Fs), dtype=tdt, device=dev)
    Z = torch.empty_like(H)
    P = torch.empty((w.N, w.D), device=dev)
    mt.mlp_tp_shard_fwd(X, W1, b1, W2, H, Z, P, w.N, w.D, w.F, w.T, dt, w.act)
    return X, dY, W1, W2, H, Z, dt, tdt


def _outputs(w, tdt):
    dev = "cuda"
    # filled with a value no result has, so an element left unwritten shows
    return {"dZ": torch.full((w.N, w.Fs), 7.0, dtype=tdt, device=dev),
            "dW1": torch.full((w.D, w.Fs), 7.0, device=dev),
            "db1": torch.full((w.Fs,), 7.0, device=dev),
            "dW2": torch.full((w.Fs, w.D), 7.0, device=dev),
            "dX": torch.full((w.N, w.D), 7.0, device=dev)}


CASES = [
    # a larger call, then a smaller one: the buffer still holds the first call's slab sums
    Workload("noalloc_a_n1000_d264_f1552_t2", 1000, 264, 1552, 2, "gelu_tanh", "bf16", 9301,
             "normal"),
    Workload("noalloc_b_n130_d136_f272_t2", 130, 136, 272, 2, "gelu_erf", "bf16", 9302,
             "normal"),
]


def test_noalloc_backward_equals_workspace_backward():
    for w in CASES:
        _say(f"  workload {w.name}")
        X, dY, W1, W2, H, Z, dt, tdt = _inputs(w)
        ref = _outputs(w, tdt)
        nb = mt.mlp_tp_shard_bwd_workspace_bytes(w.N, w.D, w.F, w.T)
        assert 0 < nb <= mt.NOALLOC_SCRATCH_BYTES
        ws = torch.empty((nb,), dtype=torch.uint8, device="cuda")
        mt.mlp_tp_shard_bwd(X, W1, W2, Z, H, dY, ref["dZ"], ref["dW1"], ref["db1"], ref["dW2"],
                            ref["dX"], ws, nb, w.N, w.D, w.F, w.T, dt, w.act)
        got = _outputs(w, tdt)
        mt.mlp_tp_shard_bwd_noalloc(X, W1, W2, Z, H, dY, got["dZ"], got["dW1"], got["db1"],
                                    got["dW2"], got["dX"], w.N, w.D, w.F, w.T, dt, w.act)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"{w.name}: {k} differs"
        _say(f"    equal: {sorted(ref)}")


def test_noalloc_backward_rejects_sizes_beyond_its_buffer():
    # ceil(N / 64) * Fs * 4 bytes of column-sum workspace: 32776 tokens of Fs = 4096 need 8.4 MB
    N, D, F, T = 32776, 64, 4096, 1
    assert mt.mlp_tp_shard_bwd_workspace_bytes(N, D, F, T) > mt.NOALLOC_SCRATCH_BYTES
    dev = "cuda"
    bf = torch.bfloat16
    X, dY = torch.zeros((N, D), dtype=bf, device=dev), torch.zeros((N, D), dtype=bf, device=dev)
    W1, W2 = torch.zeros((D, F), dtype=bf, device=dev), torch.zeros((F, D), dtype=bf, device=dev)
    H, Z, dZ = (torch.zeros((N, F), dtype=bf, device=dev) for _ in range(3))
    dW1, dW2 = torch.zeros((D, F), device=dev), torch.zeros((F, D), device=dev)
    db1, dX = torch.zeros((F,), device=dev), torch.zeros((N, D), device=dev)
    with pytest.raises(mt.MlpTpError) as e:
        mt.mlp_tp_shard_bwd_noalloc(X, W1, W2, Z, H, dY, dZ, dW1, db1, dW2, dX, N, D, F, T,
                                    mt.BF16, "gelu_tanh")
    assert e.value.code == mt.E_WORKSPACE
    # without db1 no workspace is needed, so the same sizes are accepted
    mt.mlp_tp_shard_bwd_noalloc(X, W1, W2, Z, H, dY, dZ, dW1, None, dW2, dX, N, D, F, T,
                                mt.BF16, "gelu_tanh")
    torch.cuda.synchronize()
    assert torch.count_nonzero(dW1) == 0 and torch.count_nonzero(dX) == 0
