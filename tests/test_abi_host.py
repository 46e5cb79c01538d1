"""Host-side tests of the C ABI (no GPU needed).

The library must load and export every function include/mlp_tp.h declares, and every
argument check must return its code before any HIP call. These calls pass fake, never
dereferenced device addresses and are all rejected (or are N = 0 no-ops) on the host, so no
kernel is launched.

Pages cited:
  [U] unpurerationalist.github.io, "LLM Systems 16: Model Parallel Training"
  [C] charliedreemur.github.io, "TP:Column / Row Parallel Linear 怎么切? MLP 和 attention 怎么切?"
  [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
"""
import os
import subprocess

import pytest

from tensor_mlp_block_amd import binding as mt

A = 0x10000  # fake 16-byte-aligned addresses, far apart
B = 0x20000000
C = 0x40000000
Dp = 0x60000000
E = 0x80000000
G = 0xA0000000
S = 0  # null stream


@pytest.fixture(scope="module")
def lib():
    return mt.load()


def test_library_exports_every_declared_function(lib):
    declared = mt.declared_functions()
    assert set(declared) >= {"mlp_tp_shard_fwd", "mlp_tp_partial_reduce", "mlp_tp_shard_bwd",
                             "mlp_tp_up_proj", "mlp_tp_down_proj", "mlp_tp_strerror",
                             "mlp_tp_shard_bwd_workspace_bytes"}
    out = subprocess.run(["nm", "-D", "--defined-only", mt.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared:
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_library_is_built_for_gfx950():
    # The embedded code object's target triple names the architecture it was built for.
    with open(mt.LIB_PATH, "rb") as f:
        assert b"amdgcn-amd-amdhsa--gfx950" in f.read()


def test_strerror_covers_every_code(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert mt.strerror(code) and mt.strerror(code) != "unknown error code"
    assert mt.strerror(-123) == "unknown error code"


def _fwd(lib, **kw):
    a = dict(X=A, W1r=B, b1r=None, W2r=C, H=Dp, Z=None, P=E, N=4, D=8, F=16, T=2,
             dtype=mt.BF16, act=mt.ACT["gelu_tanh"])
    a.update(kw)
    return lib.mlp_tp_shard_fwd(a["X"], a["W1r"], a["b1r"], a["W2r"], a["H"], a["Z"], a["P"],
                                a["N"], a["D"], a["F"], a["T"], a["dtype"], a["act"], S)


def test_shard_fwd_argument_checks(lib):
    assert _fwd(lib, X=None) == mt.E_NULL
    assert _fwd(lib, W2r=None) == mt.E_NULL
    assert _fwd(lib, P=None) == mt.E_NULL
    assert _fwd(lib, D=0) == mt.E_SHAPE
    assert _fwd(lib, F=0) == mt.E_SHAPE
    assert _fwd(lib, N=-1) == mt.E_SHAPE
    assert _fwd(lib, T=0) == mt.E_SHAPE
    assert _fwd(lib, F=18, T=4) == mt.E_INDIVISIBLE   # the shard count must divide F [U 3.8]
    assert _fwd(lib, dtype=2) == mt.E_DTYPE
    assert _fwd(lib, act=7) == mt.E_ACT
    assert _fwd(lib, X=A + 8) == mt.E_ALIGN
    assert _fwd(lib, b1r=G + 4) == mt.E_ALIGN
    assert _fwd(lib, H=A) == mt.E_ALIAS                # H over X
    assert _fwd(lib, P=C) == mt.E_ALIAS                # P over W2r
    assert _fwd(lib, Z=Dp) == mt.E_ALIAS               # Z over H
    assert _fwd(lib, P=A + 16) == mt.E_ALIAS           # P over part of X
    assert _fwd(lib, N=1 << 40) == mt.E_SHAPE          # too large to index safely


def test_zero_tokens_is_a_host_noop(lib):
    # N = 0 is valid and returns before any HIP call (this container has no GPU).
    assert _fwd(lib, N=0) == mt.OK
    assert lib.mlp_tp_up_proj(A, B, None, None, Dp, 0, 8, 16, 2, mt.BF16, 1, S) == mt.OK
    assert lib.mlp_tp_down_proj(A, B, E, 0, 8, 16, 2, mt.F32, S) == mt.OK


def test_up_and_down_proj_checks(lib):
    assert lib.mlp_tp_up_proj(A, B, None, None, None, 4, 8, 16, 2, mt.BF16, 1, S) == mt.E_NULL
    assert lib.mlp_tp_up_proj(A, B, None, Dp, Dp, 4, 8, 16, 2, mt.BF16, 1, S) == mt.E_ALIAS
    assert lib.mlp_tp_up_proj(A, B, None, None, Dp, 4, 8, 16, 3, mt.BF16, 1, S) == mt.E_INDIVISIBLE
    assert lib.mlp_tp_down_proj(A, B, A, 4, 8, 16, 2, mt.BF16, S) == mt.E_ALIAS
    assert lib.mlp_tp_down_proj(A, B, E + 4, 4, 8, 16, 2, mt.BF16, S) == mt.E_ALIGN


def _reduce(lib, ptrs, T=None, b2=None, b2_dtype=mt.F32, Y=G, N=4, D=8):
    import ctypes
    T = len(ptrs) if T is None else T
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    return lib.mlp_tp_partial_reduce(ctypes.cast(arr, ctypes.c_void_p), T, b2, b2_dtype, Y, N,
                                     D, S)


def test_partial_reduce_checks(lib):
    assert lib.mlp_tp_partial_reduce(None, 2, None, 0, G, 4, 8, S) == mt.E_NULL
    assert _reduce(lib, [A, None]) == mt.E_NULL
    assert _reduce(lib, [A, B], T=0) == mt.E_SHAPE
    assert _reduce(lib, [A] * 65) == mt.E_SHAPE                    # above MLP_TP_MAX_REDUCE_T
    assert _reduce(lib, [A, B], D=0) == mt.E_SHAPE
    assert _reduce(lib, [A, B], b2=C, b2_dtype=5) == mt.E_DTYPE
    assert _reduce(lib, [A, B + 4]) == mt.E_ALIGN
    assert _reduce(lib, [A, B], Y=A + 16) == mt.E_ALIAS            # partial overlap with P[0]
    assert _reduce(lib, [A, B], b2=G) == mt.E_ALIAS                # Y over b2
    assert _reduce(lib, [A, B], N=0) == mt.OK                      # no tokens: no-op
    assert _reduce(lib, [A, B], Y=A, N=0) == mt.OK                 # exact in-place is allowed


def _scatter(lib, ptrs, r, T=None, b2=None, b2_dtype=mt.F32, Y=G, N=10, D=8):
    import ctypes
    T = len(ptrs) if T is None else T
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    return lib.mlp_tp_partial_reduce_scatter(ctypes.cast(arr, ctypes.c_void_p), T, r, b2,
                                             b2_dtype, Y, N, D, S)


def test_token_slices_match_the_oracle():
    # [Z 04] reduce-scatter layout: the library's slice bounds are the oracle's.
    import oracle
    for N, T in [(10, 4), (4096, 8), (3, 8), (0, 2), (7, 1)]:
        for r in range(T):
            assert mt.mlp_tp_token_slice(N, T, r) == oracle.token_slice(N, T, r)
    with pytest.raises(mt.MlpTpError):
        mt.mlp_tp_token_slice(4, 2, 2)
    assert mt.load().mlp_tp_token_slice(4, 2, 0, None, None) == mt.E_NULL


def test_partial_reduce_scatter_checks(lib):
    assert _scatter(lib, [A, B], r=2) == mt.E_SHAPE                  # r outside [0, T)
    assert _scatter(lib, [A, B], r=-1) == mt.E_SHAPE
    assert _scatter(lib, [A, None], r=0) == mt.E_NULL
    assert _scatter(lib, [A, B + 4], r=0) == mt.E_ALIGN
    assert _scatter(lib, [A, B], r=0, Y=A + 16) == mt.E_ALIAS        # not the slice's own rows
    assert _scatter(lib, [A, B], r=1, Y=A) == mt.E_ALIAS             # P[0] rows 0.., slice 1 at row 5
    assert _scatter(lib, [A, B], r=0, b2=G) == mt.E_ALIAS            # Yr over b2
    assert _scatter(lib, [A, B], r=1, N=1) == mt.OK                  # empty slice: no-op
    assert _scatter(lib, [A, B], r=0, N=0) == mt.OK


def test_accumulate_and_gated_checks(lib):
    acc = lib.mlp_tp_down_proj_accumulate
    assert acc(A, B, None, 4, 8, 16, 2, mt.BF16, S) == mt.E_NULL
    assert acc(A, B, A, 4, 8, 16, 2, mt.BF16, S) == mt.E_ALIAS
    assert acc(A, B, E, 4, 8, 16, 3, mt.BF16, S) == mt.E_INDIVISIBLE
    assert acc(A, B, E, 0, 8, 16, 2, mt.BF16, S) == mt.OK
    up = lib.mlp_tp_swiglu_up_proj
    assert up(A, B, None, None, None, Dp, 4, 8, 16, 2, mt.BF16, S) == mt.E_NULL   # Wur
    assert up(A, B, C, None, None, None, 4, 8, 16, 2, mt.BF16, S) == mt.E_NULL    # H
    assert up(A, B, C, Dp, None, Dp, 4, 8, 16, 2, mt.BF16, S) == mt.E_ALIAS       # G over H
    assert up(A, B, C, None, B, Dp, 4, 8, 16, 2, mt.BF16, S) == mt.E_ALIAS        # U over Wgr
    assert up(A, B, C, None, None, Dp, 4, 8, 18, 4, mt.BF16, S) == mt.E_INDIVISIBLE
    assert up(A, B, C, None, None, Dp + 2, 4, 8, 16, 2, mt.BF16, S) == mt.E_ALIGN
    assert up(A, B, C, None, None, Dp, 4, 8, 16, 2, 7, S) == mt.E_DTYPE
    assert up(A, B, C, None, None, Dp, 0, 8, 16, 2, mt.BF16, S) == mt.OK
    fwd = lib.mlp_tp_swiglu_shard_fwd
    assert fwd(A, B, C, None, None, None, Dp, E, 4, 8, 16, 2, mt.BF16, S) == mt.E_NULL  # W2r
    assert fwd(A, B, C, G, None, None, Dp, C, 4, 8, 16, 2, mt.BF16, S) == mt.E_ALIAS   # P over Wur
    assert fwd(A, B, C, G, None, None, G, E, 4, 8, 16, 2, mt.BF16, S) == mt.E_ALIAS    # H over W2r
    assert fwd(A, B, C, G, None, None, Dp, E, 0, 8, 16, 2, mt.BF16, S) == mt.OK


def test_workspace_query_uses_global_sizes(lib):
    """[C 先弄清楚]: a [8192, 32768] weight split 8 ways gives [8192, 4096] per card; the
    library derives Fs = F / T from the global F itself. The db1 workspace holds one fp32 row
    of Fs per 64 tokens."""
    assert lib.mlp_tp_shard_bwd_workspace_bytes(128, 8192, 32768, 8) == 2 * 4096 * 4
    assert lib.mlp_tp_shard_bwd_workspace_bytes(4096, 8192, 28672, 8) == 64 * 3584 * 4
    assert lib.mlp_tp_shard_bwd_workspace_bytes(300, 8, 16, 2) == 5 * 8 * 4
    assert lib.mlp_tp_shard_bwd_workspace_bytes(0, 8, 16, 2) == 0
    assert lib.mlp_tp_shard_bwd_workspace_bytes(4, 8, 18, 4) == mt.E_INDIVISIBLE
    assert lib.mlp_tp_shard_bwd_workspace_bytes(4, 0, 16, 2) == mt.E_SHAPE


def _bwd(lib, **kw):
    a = dict(X=A, W1r=A + 0x1000, W2r=A + 0x2000, Z=A + 0x3000, H=A + 0x4000, dY=A + 0x5000,
             dZ=B, dW1r=C, db1r=Dp, dW2r=E, dXr=G, ws=G + 0x100000, wsb=1 << 20, N=4, D=8, F=16,
             T=2, dtype=mt.BF16, act=mt.ACT["gelu_tanh"])
    a.update(kw)
    return lib.mlp_tp_shard_bwd(a["X"], a["W1r"], a["W2r"], a["Z"], a["H"], a["dY"], a["dZ"],
                                a["dW1r"], a["db1r"], a["dW2r"], a["dXr"], a["ws"], a["wsb"],
                                a["N"], a["D"], a["F"], a["T"], a["dtype"], a["act"], S)


def test_shard_bwd_argument_checks(lib):
    assert _bwd(lib, dY=None) == mt.E_NULL
    assert _bwd(lib, dXr=None) == mt.E_NULL
    assert _bwd(lib, T=3) == mt.E_INDIVISIBLE
    assert _bwd(lib, act=-1) == mt.E_ACT
    assert _bwd(lib, dtype=9) == mt.E_DTYPE
    assert _bwd(lib, dW2r=E + 8) == mt.E_ALIGN
    assert _bwd(lib, ws=None) == mt.E_WORKSPACE
    assert _bwd(lib, wsb=15) == mt.E_WORKSPACE
    assert _bwd(lib, dZ=A + 0x3000) == mt.E_ALIAS     # dZ over Z
    assert _bwd(lib, dW1r=B) == mt.E_ALIAS            # two outputs on one buffer
    assert _bwd(lib, ws=G) == mt.E_ALIAS              # workspace over dXr


def _gbwd(lib, **kw):
    a = dict(X=A, Wg=A + 0x1000, Wu=A + 0x2000, W2r=A + 0x3000, G=A + 0x4000, U=A + 0x5000,
             H=A + 0x6000, dY=A + 0x7000, dG=B, dU=B + 0x1000, dWg=C, dWu=C + 0x1000, dW2r=E,
             dXr=G, N=4, D=8, F=16, T=2, dtype=mt.BF16)
    a.update(kw)
    return lib.mlp_tp_swiglu_shard_bwd(a["X"], a["Wg"], a["Wu"], a["W2r"], a["G"], a["U"],
                                       a["H"], a["dY"], a["dG"], a["dU"], a["dWg"], a["dWu"],
                                       a["dW2r"], a["dXr"], a["N"], a["D"], a["F"], a["T"],
                                       a["dtype"], S)


def test_swiglu_shard_bwd_argument_checks(lib):
    # Gated backward [Z 08]: every pointer is required, and no output may overlap anything.
    for k in ("X", "Wg", "Wu", "W2r", "G", "U", "H", "dY", "dG", "dU", "dWg", "dWu", "dW2r",
              "dXr"):
        assert _gbwd(lib, **{k: None}) == mt.E_NULL, k
    assert _gbwd(lib, T=3) == mt.E_INDIVISIBLE
    assert _gbwd(lib, T=0) == mt.E_SHAPE
    assert _gbwd(lib, N=-1) == mt.E_SHAPE
    assert _gbwd(lib, dtype=9) == mt.E_DTYPE
    assert _gbwd(lib, dU=B + 0x1008) == mt.E_ALIGN
    assert _gbwd(lib, dG=A + 0x4000) == mt.E_ALIAS    # dG over G
    assert _gbwd(lib, dU=B + 0x10) == mt.E_ALIAS      # dU inside dG
    assert _gbwd(lib, dXr=A + 0x7000) == mt.E_ALIAS   # dX partial over dY
    assert _gbwd(lib, dWu=C) == mt.E_ALIAS            # two weight gradients on one buffer


def _bias_act(lib, **kw):
    a = dict(Z=A, b=B, H=C, N=4, F=16, T=2, dtype=mt.BF16, act=mt.ACT["gelu_tanh"])
    a.update(kw)
    return lib.mlp_tp_bias_act(a["Z"], a["b"], a["H"], a["N"], a["F"], a["T"], a["dtype"],
                               a["act"], S)


def test_bias_act_argument_checks(lib):
    # The up-projection's epilogue on its own [Z 02], [Z 05].
    assert _bias_act(lib, Z=None) == mt.E_NULL
    assert _bias_act(lib, H=None) == mt.E_NULL
    assert _bias_act(lib, N=-1) == mt.E_SHAPE
    assert _bias_act(lib, T=0) == mt.E_SHAPE
    assert _bias_act(lib, T=3) == mt.E_INDIVISIBLE
    assert _bias_act(lib, dtype=7) == mt.E_DTYPE
    assert _bias_act(lib, act=99) == mt.E_ACT
    assert _bias_act(lib, H=C + 4) == mt.E_ALIGN
    assert _bias_act(lib, b=B + 8) == mt.E_ALIGN
    assert _bias_act(lib, H=A + 16) == mt.E_ALIAS   # H inside Z
    assert _bias_act(lib, H=B) == mt.E_ALIAS        # H over the bias
    assert _bias_act(lib, N=0) == mt.OK             # nothing to do, no launch
    assert _bias_act(lib, N=0, b=None) == mt.OK


def test_header_has_no_torch_or_hip_types():
    with open(mt.HEADER) as f:
        text = f.read()
    assert "torch" not in text.lower().replace("torch's", "")
    assert "hipStream_t" not in text.split("*/", 1)[1]  # streams travel as void*
    assert 'extern "C"' in text


def _overlap(lib, ptrs, r=1, T=None, b2=None, Y=G, N=4, D=8, F=16, chunk=2, H=A, W2r=B):
    import ctypes
    T = len(ptrs) if T is None else T
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    return lib.mlp_tp_down_proj_overlap_tail(H, W2r, ctypes.cast(arr, ctypes.c_void_p), T, r, b2,
                                             mt.F32, Y, N, D, F, mt.BF16, chunk, S, S)


def test_overlap_tail_checks(lib):
    """[F 4.4.2] the tail overlapped with the last shard's GEMM: host-side argument checks."""
    import ctypes
    assert lib.mlp_tp_down_proj_overlap_tail(A, B, None, 2, 1, None, mt.F32, G, 4, 8, 16,
                                             mt.BF16, 2, S, S) == mt.E_NULL
    assert _overlap(lib, [C, E], r=2) == mt.E_SHAPE                  # r outside [0, T)
    assert _overlap(lib, [C, E], r=-1) == mt.E_SHAPE
    assert _overlap(lib, [C, E], chunk=0) == mt.E_SHAPE
    assert _overlap(lib, [C, E], N=1000, chunk=1) == mt.E_SHAPE      # more than 256 chunks
    assert _overlap(lib, [C, None]) == mt.E_NULL
    assert _overlap(lib, [C, E], F=15) == mt.E_INDIVISIBLE
    assert _overlap(lib, [C, E + 4]) == mt.E_ALIGN
    assert _overlap(lib, [C, E], Y=A) == mt.E_ALIAS                  # Y over H
    assert _overlap(lib, [C, C + 64]) == mt.E_ALIAS                  # partials overlap
    assert _overlap(lib, [C, E], Y=E + 16) == mt.E_ALIAS             # Y partly over P[1]
    assert _overlap(lib, [C, E], Y=E, N=0) == mt.OK                  # exact alias, no rows
    assert _overlap(lib, [C, E], N=0) == mt.OK
    del ctypes


def test_tile_chooser_puts_edge_cases_on_their_tiles():
    """The GPU edge tests run shapes meant to exercise a ragged edge (or two rounds) of each
    256-class tile; the library's own chooser must send each product there on a 256-CU GPU."""
    from tile_cases import EDGE_CASES, MI355X_CUS
    for w, expect in EDGE_CASES:
        for prod, tile in expect.items():
            got = mt.mlp_tp_shard_tile(prod, w.N, w.D, w.F, w.T, MI355X_CUS)
            assert got == (*tile, 0), (w.name, prod, got)


def test_tile_chooser_headline_and_small_shapes():
    # The Llama shard [Z 07 shapes]: 16 x 16 tiles of 256 x 224 up, 16 x 32 of 256 x 256 down.
    assert mt.mlp_tp_shard_tile("up", 4096, 8192, 28672, 8, 256) == (256, 224, 0)
    assert mt.mlp_tp_shard_tile("down", 4096, 8192, 28672, 8, 256) == (256, 256, 0)
    # small products take the 128 x 128 tile; leading dimensions not multiples of 8 the
    # register-staged kernel
    assert mt.mlp_tp_shard_tile("down", 256, 4096, 11008, 1, 256) == (128, 128, 0)
    assert mt.mlp_tp_shard_tile("up", 77, 200, 300, 3, 256) == (128, 128, 1)


def test_shard_tile_checks(lib):
    import ctypes
    r = ctypes.c_int32()
    rp = ctypes.cast(ctypes.byref(r), ctypes.c_void_p)
    assert lib.mlp_tp_shard_tile(6, 4, 8, 16, 2, 256, rp, None, None) == mt.E_DTYPE
    assert lib.mlp_tp_shard_tile(-1, 4, 8, 16, 2, 256, rp, None, None) == mt.E_DTYPE
    assert lib.mlp_tp_shard_tile(0, 0, 8, 16, 2, 256, rp, None, None) == mt.E_SHAPE
    assert lib.mlp_tp_shard_tile(0, 4, 8, 16, 2, 0, rp, None, None) == mt.E_SHAPE
    assert lib.mlp_tp_shard_tile(0, 4, 8, 18, 4, 256, rp, None, None) == mt.E_INDIVISIBLE
    assert lib.mlp_tp_shard_tile(0, 4, 8, 16, 2, 256, None, None, None) == mt.OK


def test_bias_share_checks(lib):
    """[Z 05] b2/T per rank: the down-projection's checks plus those of the bias."""
    f = lib.mlp_tp_down_proj_bias_share
    assert f(A, B, C, mt.F32, None, 4, 8, 16, 2, mt.BF16, S) == mt.E_NULL
    assert f(A, B, C, mt.F32, E, 4, 8, 16, 3, mt.BF16, S) == mt.E_INDIVISIBLE
    assert f(A, B, C, 7, E, 4, 8, 16, 2, mt.BF16, S) == mt.E_DTYPE
    assert f(A, B, C + 4, mt.F32, E, 4, 8, 16, 2, mt.BF16, S) == mt.E_ALIGN
    assert f(A, B, E, mt.F32, E, 4, 8, 16, 2, mt.BF16, S) == mt.E_ALIAS     # P over b2
    assert f(A, B, C, mt.F32, A, 4, 8, 16, 2, mt.BF16, S) == mt.E_ALIAS     # P over H
    assert f(A, B, C, mt.F32, E, 0, 8, 16, 2, mt.BF16, S) == mt.OK          # no tokens
    assert f(A, B, None, 7, E, 0, 8, 16, 2, mt.BF16, S) == mt.OK            # no bias: dtype unused


def test_binding_rejects_tensors_the_library_cannot_read():
    """Marshalling checks of the binding, before the library is called: a column slice
    W1[:, c0:c1] is not contiguous (read with the shard's own row stride it would give wrong
    results), a tensor of another element type than the call's dtype code, a tensor in host
    memory, and a partial list whose length is not T."""
    import torch
    W1 = torch.zeros((8, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="contiguous"):
        mt.mlp_tp_up_proj(A, W1[:, 0:8], None, None, Dp, 4, 8, 16, 2, mt.BF16, "relu")
    with pytest.raises(ValueError, match="dtype"):
        mt.mlp_tp_up_proj(A, W1.float(), None, None, Dp, 4, 8, 16, 1, mt.BF16, "relu")
    with pytest.raises(ValueError, match="GPU"):
        mt.mlp_tp_up_proj(A, W1, None, None, Dp, 4, 8, 16, 1, mt.BF16, "relu")
    with pytest.raises(ValueError, match="dtype"):
        mt.mlp_tp_down_proj(A, B, torch.zeros((4, 8), dtype=torch.bfloat16), 4, 8, 16, 2, mt.BF16)
    with pytest.raises(ValueError, match="T = 3"):
        mt.mlp_tp_partial_reduce([A, B], 3, None, mt.F32, G, 4, 8)
    with pytest.raises(ValueError, match="T = 1"):
        mt.mlp_tp_partial_reduce_scatter([A, B], 1, 0, None, mt.F32, G, 4, 8)
    with pytest.raises(ValueError, match="T = 4"):
        mt.mlp_tp_down_proj_overlap_tail(A, B, [C, E], 4, 1, None, mt.F32, G, 4, 8, 16, mt.BF16,
                                         2, stream=0)


def test_noalloc_backward_checks(lib):
    """The allocation-free backward takes the backward's checks, and rejects on the host,
    before any HIP call, sizes whose column-sum workspace exceeds its buffer."""
    f = lib.mlp_tp_shard_bwd_noalloc

    def call(**kw):
        a = dict(X=A, W1r=A + 0x1000, W2r=A + 0x2000, Z=A + 0x3000, H=A + 0x4000,
                 dY=A + 0x5000, dZ=B, dW1r=C, db1r=Dp, dW2r=E, dXr=G, N=4, D=8, F=16, T=2,
                 dtype=mt.BF16, act=mt.ACT["gelu_tanh"])
        a.update(kw)
        return f(a["X"], a["W1r"], a["W2r"], a["Z"], a["H"], a["dY"], a["dZ"], a["dW1r"],
                 a["db1r"], a["dW2r"], a["dXr"], a["N"], a["D"], a["F"], a["T"], a["dtype"],
                 a["act"], S)

    assert call(dY=None) == mt.E_NULL
    assert call(T=3) == mt.E_INDIVISIBLE
    assert call(act=9) == mt.E_ACT
    assert call(dZ=A + 0x3000) == mt.E_ALIAS
    # 32776 tokens of Fs = 4096: 513 slabs x 4096 x 4 bytes > 8 MiB
    big = dict(X=A, W1r=B, W2r=B + (1 << 22), Z=C, H=C + (1 << 27), dY=Dp, dZ=E,
               dW1r=G, db1r=G + (1 << 22), dW2r=G + (1 << 23), dXr=G + (1 << 24),
               N=32776, D=64, F=4096, T=1)
    assert mt.mlp_tp_shard_bwd_workspace_bytes(32776, 64, 4096, 1) > mt.NOALLOC_SCRATCH_BYTES
    assert call(**big) == mt.E_WORKSPACE


def test_split_forward_workspace_query_and_checks(lib):
    """The split-contraction forward [Z 04]: the workspace query (this container has no GPU, so
    the library sizes for 256 compute units) and the host checks of mlp_tp_shard_fwd_ws."""
    # the pages' example shape at T = 1: the down-projection's 64 tiles of 128 x 128 split
    # 8 ways (8 fp32 planes of [256, 4096]); the Llama shard fills the GPU and never splits
    assert mt.mlp_tp_shard_fwd_workspace_bytes(256, 4096, 11008, 1) == 8 * 256 * 4096 * 4
    assert mt.mlp_tp_shard_fwd_workspace_bytes(4096, 8192, 28672, 8) == 0
    assert mt.mlp_tp_shard_fwd_workspace_bytes(0, 4096, 11008, 1) == 0
    assert lib.mlp_tp_shard_fwd_workspace_bytes(4, 8, 18, 4) == mt.E_INDIVISIBLE
    f = lib.mlp_tp_shard_fwd_ws

    def call(**kw):
        a = dict(X=A, W1r=B, b1r=None, W2r=C, H=Dp, Z=None, P=E, ws=G, wsb=1 << 20, N=4, D=8,
                 F=16, T=2, dtype=mt.BF16, act=mt.ACT["gelu_tanh"])
        a.update(kw)
        return f(a["X"], a["W1r"], a["b1r"], a["W2r"], a["H"], a["Z"], a["P"], a["ws"],
                 a["wsb"], a["N"], a["D"], a["F"], a["T"], a["dtype"], a["act"], S)

    assert call(X=None) == mt.E_NULL
    assert call(F=18, T=4) == mt.E_INDIVISIBLE
    assert call(ws=G + 8) == mt.E_ALIGN
    assert call(ws=E) == mt.E_ALIAS          # workspace over P
    assert call(ws=A + 16) == mt.E_ALIAS     # workspace over X
    assert call(H=A) == mt.E_ALIAS
    assert call(N=0) == mt.OK
    assert call(N=0, ws=None, wsb=0) == mt.OK
