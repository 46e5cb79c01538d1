"""ctypes binding of libmlptp.so: the C entry points of include/mlp_tp.h under the same names.

Argument marshalling only: tensors become device pointers (``data_ptr()``), ``None`` becomes
NULL, and the stream defaults to torch's current stream on the current device. Every step of
the computation runs in the HIP library. A non-zero return code raises ``MlpTpError``
carrying the code and the library's message.

The library is loaded on first use. If it has not been built, the first call raises: there is
no fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmlptp.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "mlp_tp.h")

# Return codes, dtypes and activations (the values of include/mlp_tp.h).
OK = 0
E_NULL, E_SHAPE, E_INDIVISIBLE, E_DTYPE, E_ACT, E_ALIGN, E_WORKSPACE, E_HIP, E_ALIAS = (
    -1, -2, -3, -4, -5, -6, -7, -8, -9)
F32, BF16 = 0, 1
ACT = {"identity": 0, "relu": 1, "gelu_tanh": 2, "gelu_erf": 3, "gelu_sigmoid": 4}
MAX_REDUCE_T = 64

_lib = None


class MlpTpError(RuntimeError):
    def __init__(self, code: int, func: str):
        self.code = code
        super().__init__(f"{func} failed with {code}: {strerror(code)}")


def load() -> ctypes.CDLL:
    """Loads libmlptp.so; raises if it is missing (build it with tensor_mlp_block_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m tensor_mlp_block_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sigs = {
        "mlp_tp_up_proj": ([vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp], ctypes.c_int),
        "mlp_tp_down_proj": ([vp, vp, vp, i64, i64, i64, i32, i32, vp], ctypes.c_int),
        "mlp_tp_shard_fwd": ([vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp],
                             ctypes.c_int),
        "mlp_tp_partial_reduce": ([vp, i32, vp, i32, vp, i64, i64, vp], ctypes.c_int),
        "mlp_tp_shard_bwd_workspace_bytes": ([i64, i64, i64, i32], ctypes.c_int64),
        "mlp_tp_shard_bwd": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                              i64, i64, i64, i32, i32, i32, vp], ctypes.c_int),
        "mlp_tp_token_slice": ([i64, i32, i32, vp, vp], ctypes.c_int),
        "mlp_tp_partial_reduce_scatter": ([vp, i32, i32, vp, i32, vp, i64, i64, vp],
                                          ctypes.c_int),
        "mlp_tp_down_proj_accumulate": ([vp, vp, vp, i64, i64, i64, i32, i32, vp], ctypes.c_int),
        "mlp_tp_down_proj_overlap_tail": ([vp, vp, vp, i32, i32, vp, i32, vp, i64, i64, i64, i32,
                                           i64, vp, vp], ctypes.c_int),
        "mlp_tp_swiglu_up_proj": ([vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp],
                                  ctypes.c_int),
        "mlp_tp_swiglu_shard_fwd": ([vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32,
                                     vp], ctypes.c_int),
        "mlp_tp_swiglu_shard_bwd": ([vp] * 14 + [i64, i64, i64, i32, i32, vp], ctypes.c_int),
        "mlp_tp_bias_act": ([vp, vp, vp, i64, i64, i32, i32, i32, vp], ctypes.c_int),
        "mlp_tp_strerror": ([ctypes.c_int], ctypes.c_char_p),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def declared_functions() -> list[str]:
    """Names of the functions include/mlp_tp.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mlp_tp_\w+)\s*\(", text)))


def strerror(code: int) -> str:
    return load().mlp_tp_strerror(int(code)).decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _act(act):
    return ACT[act] if isinstance(act, str) else int(act)


def _check(rc: int, func: str) -> int:
    if rc != OK:
        raise MlpTpError(rc, func)
    return rc


def mlp_tp_up_proj(X, W1r, b1r, Z, H, N, D, F, T, dtype, act, stream=None):
    rc = load().mlp_tp_up_proj(_ptr(X), _ptr(W1r), _ptr(b1r), _ptr(Z), _ptr(H), N, D, F, T,
                               dtype, _act(act), _stream(stream))
    return _check(rc, "mlp_tp_up_proj")


def mlp_tp_down_proj(H, W2r, P, N, D, F, T, dtype, stream=None):
    rc = load().mlp_tp_down_proj(_ptr(H), _ptr(W2r), _ptr(P), N, D, F, T, dtype,
                                 _stream(stream))
    return _check(rc, "mlp_tp_down_proj")


def mlp_tp_shard_fwd(X, W1r, b1r, W2r, H, Z, P, N, D, F, T, dtype, act, stream=None):
    rc = load().mlp_tp_shard_fwd(_ptr(X), _ptr(W1r), _ptr(b1r), _ptr(W2r), _ptr(H), _ptr(Z),
                                 _ptr(P), N, D, F, T, dtype, _act(act), _stream(stream))
    return _check(rc, "mlp_tp_shard_fwd")


def mlp_tp_partial_reduce(P, T, b2, b2_dtype, Y, N, D, stream=None):
    """P: a sequence of T device tensors/pointers (passed as a host array of pointers)."""
    ptrs = (ctypes.c_void_p * max(1, len(P)))(*[_ptr(p) for p in P])
    rc = load().mlp_tp_partial_reduce(ctypes.cast(ptrs, ctypes.c_void_p), T, _ptr(b2), b2_dtype,
                                      _ptr(Y), N, D, _stream(stream))
    return _check(rc, "mlp_tp_partial_reduce")


def mlp_tp_token_slice(N, T, r):
    """(first row, row count) of token slice r in the reduce-scatter layout."""
    row0, rows = ctypes.c_int64(), ctypes.c_int64()
    rc = load().mlp_tp_token_slice(N, T, r, ctypes.cast(ctypes.byref(row0), ctypes.c_void_p),
                                   ctypes.cast(ctypes.byref(rows), ctypes.c_void_p))
    _check(rc, "mlp_tp_token_slice")
    return row0.value, rows.value


def mlp_tp_partial_reduce_scatter(P, T, r, b2, b2_dtype, Yr, N, D, stream=None):
    """Token slice r of the block tail into Yr [rows, D]; P as for mlp_tp_partial_reduce."""
    ptrs = (ctypes.c_void_p * max(1, len(P)))(*[_ptr(p) for p in P])
    rc = load().mlp_tp_partial_reduce_scatter(ctypes.cast(ptrs, ctypes.c_void_p), T, r, _ptr(b2),
                                              b2_dtype, _ptr(Yr), N, D, _stream(stream))
    return _check(rc, "mlp_tp_partial_reduce_scatter")


def mlp_tp_down_proj_accumulate(H, W2r, P, N, D, F, T, dtype, stream=None):
    rc = load().mlp_tp_down_proj_accumulate(_ptr(H), _ptr(W2r), _ptr(P), N, D, F, T, dtype,
                                            _stream(stream))
    return _check(rc, "mlp_tp_down_proj_accumulate")


def mlp_tp_down_proj_overlap_tail(H, W2r, P, T, r, b2, b2_dtype, Y, N, D, F, dtype, chunk_rows,
                                  stream=None, tail_stream=None):
    """P[r] = H W2r in token chunks on `stream`, the block tail of each finished chunk on
    `tail_stream` (default: the same stream)."""
    ptrs = (ctypes.c_void_p * max(1, len(P)))(*[_ptr(p) for p in P])
    s0 = _stream(stream)
    s1 = _stream(tail_stream) if tail_stream is not None else s0
    rc = load().mlp_tp_down_proj_overlap_tail(_ptr(H), _ptr(W2r), ctypes.cast(ptrs, ctypes.c_void_p),
                                              T, r, _ptr(b2), b2_dtype, _ptr(Y), N, D, F, dtype,
                                              chunk_rows, s0, s1)
    return _check(rc, "mlp_tp_down_proj_overlap_tail")


def mlp_tp_swiglu_up_proj(X, Wgr, Wur, G, U, H, N, D, F, T, dtype, stream=None):
    rc = load().mlp_tp_swiglu_up_proj(_ptr(X), _ptr(Wgr), _ptr(Wur), _ptr(G), _ptr(U), _ptr(H),
                                      N, D, F, T, dtype, _stream(stream))
    return _check(rc, "mlp_tp_swiglu_up_proj")


def mlp_tp_swiglu_shard_fwd(X, Wgr, Wur, W2r, G, U, H, P, N, D, F, T, dtype, stream=None):
    rc = load().mlp_tp_swiglu_shard_fwd(_ptr(X), _ptr(Wgr), _ptr(Wur), _ptr(W2r), _ptr(G),
                                        _ptr(U), _ptr(H), _ptr(P), N, D, F, T, dtype,
                                        _stream(stream))
    return _check(rc, "mlp_tp_swiglu_shard_fwd")


def mlp_tp_shard_bwd_workspace_bytes(N, D, F, T) -> int:
    n = load().mlp_tp_shard_bwd_workspace_bytes(N, D, F, T)
    if n < 0:
        raise MlpTpError(int(n), "mlp_tp_shard_bwd_workspace_bytes")
    return int(n)


def mlp_tp_shard_bwd(X, W1r, W2r, Z, H, dY, dZ, dW1r, db1r, dW2r, dXr, workspace,
                     workspace_bytes, N, D, F, T, dtype, act, stream=None):
    rc = load().mlp_tp_shard_bwd(_ptr(X), _ptr(W1r), _ptr(W2r), _ptr(Z), _ptr(H), _ptr(dY),
                                 _ptr(dZ), _ptr(dW1r), _ptr(db1r), _ptr(dW2r), _ptr(dXr),
                                 _ptr(workspace), int(workspace_bytes), N, D, F, T, dtype,
                                 _act(act), _stream(stream))
    return _check(rc, "mlp_tp_shard_bwd")


def mlp_tp_swiglu_shard_bwd(X, Wgr, Wur, W2r, G, U, H, dY, dG, dU, dWgr, dWur, dW2r, dXr, N, D, F,
                            T, dtype, stream=None):
    rc = load().mlp_tp_swiglu_shard_bwd(_ptr(X), _ptr(Wgr), _ptr(Wur), _ptr(W2r), _ptr(G), _ptr(U),
                                        _ptr(H), _ptr(dY), _ptr(dG), _ptr(dU), _ptr(dWgr),
                                        _ptr(dWur), _ptr(dW2r), _ptr(dXr), N, D, F, T, dtype,
                                        _stream(stream))
    return _check(rc, "mlp_tp_swiglu_shard_bwd")


def mlp_tp_bias_act(Z, b1r, H, N, F, T, dtype, act, stream=None):
    rc = load().mlp_tp_bias_act(_ptr(Z), _ptr(b1r), _ptr(H), N, F, T, dtype, _act(act),
                                _stream(stream))
    return _check(rc, "mlp_tp_bias_act")


def mlp_tp_strerror(code: int) -> str:
    return strerror(code)
