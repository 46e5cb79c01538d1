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
NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024
PROD = {"up": 0, "down": 1, "dh": 2, "dw2": 3, "dw1": 4, "dx": 5}

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
        "mlp_tp_shard_fwd_workspace_bytes": ([i64, i64, i64, i32], ctypes.c_int64),
        "mlp_tp_shard_fwd_ws": ([vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64, i32, i32, i32,
                                 vp], ctypes.c_int),
        "mlp_tp_partial_reduce": ([vp, i32, vp, i32, vp, i64, i64, vp], ctypes.c_int),
        "mlp_tp_shard_bwd_workspace_bytes": ([i64, i64, i64, i32], ctypes.c_int64),
        "mlp_tp_shard_bwd": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                              i64, i64, i64, i32, i32, i32, vp], ctypes.c_int),
        "mlp_tp_token_slice": ([i64, i32, i32, vp, vp], ctypes.c_int),
        "mlp_tp_partial_reduce_scatter": ([vp, i32, i32, vp, i32, vp, i64, i64, vp],
                                          ctypes.c_int),
        "mlp_tp_down_proj_accumulate": ([vp, vp, vp, i64, i64, i64, i32, i32, vp], ctypes.c_int),
        "mlp_tp_down_proj_bias_share": ([vp, vp, vp, i32, vp, i64, i64, i64, i32, i32, vp],
                                        ctypes.c_int),
        "mlp_tp_shard_tile": ([i32, i64, i64, i64, i32, i32, vp, vp, vp], ctypes.c_int),
        "mlp_tp_down_proj_overlap_tail": ([vp, vp, vp, i32, i32, vp, i32, vp, i64, i64, i64, i32,
                                           i64, vp, vp], ctypes.c_int),
        "mlp_tp_swiglu_up_proj": ([vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp],
                                  ctypes.c_int),
        "mlp_tp_swiglu_shard_fwd": ([vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32,
                                     vp], ctypes.c_int),
        "mlp_tp_shard_bwd_noalloc": ([vp] * 11 + [i64, i64, i64, i32, i32, i32, vp],
                                     ctypes.c_int),
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


_TORCH_DTYPES = {}


def _torch_dtype(code):
    """torch dtype of a dtype code (F32 or BF16); None for an unknown code (the library then
    rejects the call with E_DTYPE)."""
    if not _TORCH_DTYPES:
        import torch
        _TORCH_DTYPES.update({F32: torch.float32, BF16: torch.bfloat16})
    return _TORCH_DTYPES.get(code)


def _ptr(x, dtype=None, name="tensor"):
    """Device address of x: None -> NULL, an int is taken as an address, a torch tensor must be
    contiguous (row-major, no padding: a column slice such as W1[:, c0:c1] is not), of the
    element type `dtype` (a dtype code; None skips the check, e.g. for a byte workspace), and
    in GPU memory. Marshalling checks only: they raise ValueError before the library is
    called."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major, no padding); pass "
                         f"a .contiguous() copy")
    if dtype is not None:
        want = _torch_dtype(dtype)
        if want is not None and x.dtype != want:
            raise ValueError(f"{name} has dtype {x.dtype}, the call's dtype code {dtype} "
                             f"needs {want}")
    if not x.is_cuda:
        raise ValueError(f"{name} must be in GPU memory")
    return x.data_ptr()


def _ptr_array(P, T, name="P"):
    """Host array of the T device pointers of the partials (float32 tensors or addresses)."""
    if len(P) != T:
        raise ValueError(f"{name} holds {len(P)} partials but T = {T}")
    ptrs = [_ptr(p, F32, f"{name}[{i}]") for i, p in enumerate(P)]
    return (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)


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
    rc = load().mlp_tp_up_proj(_ptr(X, dtype, "X"), _ptr(W1r, dtype, "W1r"),
                               _ptr(b1r, dtype, "b1r"), _ptr(Z, dtype, "Z"), _ptr(H, dtype, "H"),
                               N, D, F, T, dtype, _act(act), _stream(stream))
    return _check(rc, "mlp_tp_up_proj")


def mlp_tp_down_proj(H, W2r, P, N, D, F, T, dtype, stream=None):
    rc = load().mlp_tp_down_proj(_ptr(H, dtype, "H"), _ptr(W2r, dtype, "W2r"),
                                 _ptr(P, F32, "P"), N, D, F, T, dtype, _stream(stream))
    return _check(rc, "mlp_tp_down_proj")


def mlp_tp_shard_fwd(X, W1r, b1r, W2r, H, Z, P, N, D, F, T, dtype, act, stream=None):
    rc = load().mlp_tp_shard_fwd(_ptr(X, dtype, "X"), _ptr(W1r, dtype, "W1r"),
                                 _ptr(b1r, dtype, "b1r"), _ptr(W2r, dtype, "W2r"),
                                 _ptr(H, dtype, "H"), _ptr(Z, dtype, "Z"), _ptr(P, F32, "P"),
                                 N, D, F, T, dtype, _act(act), _stream(stream))
    return _check(rc, "mlp_tp_shard_fwd")


def mlp_tp_shard_fwd_workspace_bytes(N, D, F, T) -> int:
    n = load().mlp_tp_shard_fwd_workspace_bytes(N, D, F, T)
    if n < 0:
        raise MlpTpError(int(n), "mlp_tp_shard_fwd_workspace_bytes")
    return int(n)


def mlp_tp_shard_fwd_ws(X, W1r, b1r, W2r, H, Z, P, workspace, workspace_bytes, N, D, F, T, dtype,
                        act, stream=None):
    rc = load().mlp_tp_shard_fwd_ws(_ptr(X, dtype, "X"), _ptr(W1r, dtype, "W1r"),
                                    _ptr(b1r, dtype, "b1r"), _ptr(W2r, dtype, "W2r"),
                                    _ptr(H, dtype, "H"), _ptr(Z, dtype, "Z"), _ptr(P, F32, "P"),
                                    _ptr(workspace, None, "workspace"), int(workspace_bytes),
                                    N, D, F, T, dtype, _act(act), _stream(stream))
    return _check(rc, "mlp_tp_shard_fwd_ws")


def mlp_tp_partial_reduce(P, T, b2, b2_dtype, Y, N, D, stream=None):
    """P: a sequence of exactly T float32 device tensors or addresses (passed as a host array
    of pointers)."""
    ptrs = _ptr_array(P, T)
    rc = load().mlp_tp_partial_reduce(ctypes.cast(ptrs, ctypes.c_void_p), T,
                                      _ptr(b2, b2_dtype, "b2"), b2_dtype, _ptr(Y, F32, "Y"), N, D,
                                      _stream(stream))
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
    ptrs = _ptr_array(P, T)
    rc = load().mlp_tp_partial_reduce_scatter(ctypes.cast(ptrs, ctypes.c_void_p), T, r,
                                              _ptr(b2, b2_dtype, "b2"), b2_dtype,
                                              _ptr(Yr, F32, "Yr"), N, D, _stream(stream))
    return _check(rc, "mlp_tp_partial_reduce_scatter")


def mlp_tp_down_proj_accumulate(H, W2r, P, N, D, F, T, dtype, stream=None):
    rc = load().mlp_tp_down_proj_accumulate(_ptr(H, dtype, "H"), _ptr(W2r, dtype, "W2r"),
                                            _ptr(P, F32, "P"), N, D, F, T, dtype,
                                            _stream(stream))
    return _check(rc, "mlp_tp_down_proj_accumulate")


def mlp_tp_down_proj_bias_share(H, W2r, b2, b2_dtype, P, N, D, F, T, dtype, stream=None):
    """P = H W2r + b2 / T: rank r's partial carrying its 1/T share of the full bias b2."""
    rc = load().mlp_tp_down_proj_bias_share(_ptr(H, dtype, "H"), _ptr(W2r, dtype, "W2r"),
                                            _ptr(b2, b2_dtype, "b2"), b2_dtype,
                                            _ptr(P, F32, "P"), N, D, F, T, dtype,
                                            _stream(stream))
    return _check(rc, "mlp_tp_down_proj_bias_share")


def mlp_tp_shard_tile(product, N, D, F, T, compute_units):
    """(tile rows, tile cols, staged) of a bf16 product of the shard; product is a PROD key or
    code. A host query: no GPU needed."""
    code = PROD[product] if isinstance(product, str) else int(product)
    rows, cols, staged = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    rc = load().mlp_tp_shard_tile(code, N, D, F, T, compute_units,
                                  ctypes.cast(ctypes.byref(rows), ctypes.c_void_p),
                                  ctypes.cast(ctypes.byref(cols), ctypes.c_void_p),
                                  ctypes.cast(ctypes.byref(staged), ctypes.c_void_p))
    _check(rc, "mlp_tp_shard_tile")
    return rows.value, cols.value, staged.value


def mlp_tp_down_proj_overlap_tail(H, W2r, P, T, r, b2, b2_dtype, Y, N, D, F, dtype, chunk_rows,
                                  stream=None, tail_stream=None):
    """P[r] = H W2r in token chunks on `stream`, the block tail of each finished chunk on
    `tail_stream` (default: the same stream)."""
    ptrs = _ptr_array(P, T)
    s0 = _stream(stream)
    s1 = _stream(tail_stream) if tail_stream is not None else s0
    rc = load().mlp_tp_down_proj_overlap_tail(_ptr(H, dtype, "H"), _ptr(W2r, dtype, "W2r"),
                                              ctypes.cast(ptrs, ctypes.c_void_p), T, r,
                                              _ptr(b2, b2_dtype, "b2"), b2_dtype,
                                              _ptr(Y, F32, "Y"), N, D, F, dtype, chunk_rows,
                                              s0, s1)
    return _check(rc, "mlp_tp_down_proj_overlap_tail")


def mlp_tp_swiglu_up_proj(X, Wgr, Wur, G, U, H, N, D, F, T, dtype, stream=None):
    rc = load().mlp_tp_swiglu_up_proj(_ptr(X, dtype, "X"), _ptr(Wgr, dtype, "Wgr"),
                                      _ptr(Wur, dtype, "Wur"), _ptr(G, dtype, "G"),
                                      _ptr(U, dtype, "U"), _ptr(H, dtype, "H"), N, D, F, T,
                                      dtype, _stream(stream))
    return _check(rc, "mlp_tp_swiglu_up_proj")


def mlp_tp_swiglu_shard_fwd(X, Wgr, Wur, W2r, G, U, H, P, N, D, F, T, dtype, stream=None):
    rc = load().mlp_tp_swiglu_shard_fwd(_ptr(X, dtype, "X"), _ptr(Wgr, dtype, "Wgr"),
                                        _ptr(Wur, dtype, "Wur"), _ptr(W2r, dtype, "W2r"),
                                        _ptr(G, dtype, "G"), _ptr(U, dtype, "U"),
                                        _ptr(H, dtype, "H"), _ptr(P, F32, "P"), N, D, F, T,
                                        dtype, _stream(stream))
    return _check(rc, "mlp_tp_swiglu_shard_fwd")


def mlp_tp_shard_bwd_workspace_bytes(N, D, F, T) -> int:
    n = load().mlp_tp_shard_bwd_workspace_bytes(N, D, F, T)
    if n < 0:
        raise MlpTpError(int(n), "mlp_tp_shard_bwd_workspace_bytes")
    return int(n)


def mlp_tp_shard_bwd(X, W1r, W2r, Z, H, dY, dZ, dW1r, db1r, dW2r, dXr, workspace,
                     workspace_bytes, N, D, F, T, dtype, act, stream=None):
    rc = load().mlp_tp_shard_bwd(_ptr(X, dtype, "X"), _ptr(W1r, dtype, "W1r"),
                                 _ptr(W2r, dtype, "W2r"), _ptr(Z, dtype, "Z"),
                                 _ptr(H, dtype, "H"), _ptr(dY, dtype, "dY"),
                                 _ptr(dZ, dtype, "dZ"), _ptr(dW1r, F32, "dW1r"),
                                 _ptr(db1r, F32, "db1r"), _ptr(dW2r, F32, "dW2r"),
                                 _ptr(dXr, F32, "dXr"), _ptr(workspace, None, "workspace"),
                                 int(workspace_bytes), N, D, F, T, dtype, _act(act),
                                 _stream(stream))
    return _check(rc, "mlp_tp_shard_bwd")


def mlp_tp_shard_bwd_noalloc(X, W1r, W2r, Z, H, dY, dZ, dW1r, db1r, dW2r, dXr, N, D, F, T,
                             dtype, act, stream=None):
    """mlp_tp_shard_bwd with the library's own per-GPU device buffer as the workspace (for
    callers that cannot allocate; calls that overlap on one GPU race on that buffer)."""
    rc = load().mlp_tp_shard_bwd_noalloc(_ptr(X, dtype, "X"), _ptr(W1r, dtype, "W1r"),
                                         _ptr(W2r, dtype, "W2r"), _ptr(Z, dtype, "Z"),
                                         _ptr(H, dtype, "H"), _ptr(dY, dtype, "dY"),
                                         _ptr(dZ, dtype, "dZ"), _ptr(dW1r, F32, "dW1r"),
                                         _ptr(db1r, F32, "db1r"), _ptr(dW2r, F32, "dW2r"),
                                         _ptr(dXr, F32, "dXr"), N, D, F, T, dtype, _act(act),
                                         _stream(stream))
    return _check(rc, "mlp_tp_shard_bwd_noalloc")


def mlp_tp_swiglu_shard_bwd(X, Wgr, Wur, W2r, G, U, H, dY, dG, dU, dWgr, dWur, dW2r, dXr, N, D, F,
                            T, dtype, stream=None):
    rc = load().mlp_tp_swiglu_shard_bwd(_ptr(X, dtype, "X"), _ptr(Wgr, dtype, "Wgr"),
                                        _ptr(Wur, dtype, "Wur"), _ptr(W2r, dtype, "W2r"),
                                        _ptr(G, dtype, "G"), _ptr(U, dtype, "U"),
                                        _ptr(H, dtype, "H"), _ptr(dY, dtype, "dY"),
                                        _ptr(dG, dtype, "dG"), _ptr(dU, dtype, "dU"),
                                        _ptr(dWgr, F32, "dWgr"), _ptr(dWur, F32, "dWur"),
                                        _ptr(dW2r, F32, "dW2r"), _ptr(dXr, F32, "dXr"), N, D, F,
                                        T, dtype, _stream(stream))
    return _check(rc, "mlp_tp_swiglu_shard_bwd")


def mlp_tp_bias_act(Z, b1r, H, N, F, T, dtype, act, stream=None):
    rc = load().mlp_tp_bias_act(_ptr(Z, F32, "Z"), _ptr(b1r, dtype, "b1r"), _ptr(H, dtype, "H"),
                                N, F, T, dtype, _act(act), _stream(stream))
    return _check(rc, "mlp_tp_bias_act")


def mlp_tp_strerror(code: int) -> str:
    return strerror(code)
