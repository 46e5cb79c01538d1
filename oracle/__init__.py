"""Python wrapper of the fp64 CPU oracle (``mlp_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the benchmark's
CPU-baseline leg, never by the GPU library or its binding. It shares no code with them.

Every function takes array-likes (numpy arrays or CPU torch tensors of any float dtype),
widens them to contiguous fp64 (exact for bf16 and fp32 inputs) and returns fp64 numpy
arrays. Shapes follow the oracle's C header comment: X [N,D], W1, Wg, Wu [D,F], b1 [F], W2 [F,D],
b2 [D], dY [N,D]; shard outputs are [N, F/T] and [N, D].

Parity status of each function is pinned by the tests under ``tests/test_oracle_*.py``:
activation values and derivatives, the shard forward, the block tail, the dense forward,
the shard backward and the dense backward each have at least one pin that does not re-run
the oracle's own formula.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from ._build import LIB_PATH, build_oracle

ACT = {"identity": 0, "relu": 1, "gelu_tanh": 2, "gelu_erf": 3, "gelu_sigmoid": 4}

_lib = None
_dp = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build_oracle()
        lib = ctypes.CDLL(LIB_PATH)
        i64, i32, ci = ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        vp = ctypes.c_void_p
        lib.oracle_act_vec.argtypes = [ci, vp, vp, i64]
        lib.oracle_act_deriv_vec.argtypes = [ci, vp, vp, i64]
        lib.oracle_shard_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, ci, vp, vp, vp]
        lib.oracle_partial_sum.argtypes = [vp, i32, vp, i64, i64, vp]
        lib.oracle_partial_sum_bias_share.argtypes = [vp, i32, i32, vp, i64, i64, vp]
        lib.oracle_block_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, ci, vp]
        lib.oracle_dense_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci, vp]
        lib.oracle_shard_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, ci,
                                         vp, vp, vp, vp, vp]
        lib.oracle_dense_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci,
                                         vp, vp, vp, vp, vp]
        lib.oracle_num_threads.argtypes = []
        lib.oracle_token_slice.argtypes = [i64, i32, i32, vp, vp]
        lib.oracle_partial_reduce_scatter.argtypes = [vp, i32, i32, vp, i64, i64, vp]
        lib.oracle_silu_vec.argtypes = [vp, vp, i64, ci]
        lib.oracle_swiglu_shard_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32,
                                                vp, vp, vp, vp]
        lib.oracle_swiglu_dense_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
        lib.oracle_swiglu_shard_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32,
                                                vp, vp, vp, vp, vp, vp]
        for name in ("oracle_act_vec", "oracle_act_deriv_vec", "oracle_shard_fwd",
                     "oracle_partial_sum", "oracle_partial_sum_bias_share", "oracle_block_fwd", "oracle_dense_fwd",
                     "oracle_shard_bwd", "oracle_dense_bwd", "oracle_num_threads",
                     "oracle_token_slice", "oracle_partial_reduce_scatter", "oracle_silu_vec",
                     "oracle_swiglu_shard_fwd", "oracle_swiglu_dense_fwd",
                     "oracle_swiglu_shard_bwd"):
            getattr(lib, name).restype = ci
        _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _f64(a):
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


def _act_code(act):
    if act not in ACT:
        raise OracleError(f"unknown activation {act!r}")
    return ACT[act]


def act(name, z):
    z = _f64(z)
    out = np.empty_like(z)
    _check(_load().oracle_act_vec(_act_code(name), _p(z), _p(out), z.size), "oracle_act_vec")
    return out


def act_deriv(name, z):
    z = _f64(z)
    out = np.empty_like(z)
    _check(_load().oracle_act_deriv_vec(_act_code(name), _p(z), _p(out), z.size),
           "oracle_act_deriv_vec")
    return out


def _dims(X, W1, W2):
    N, D = X.shape
    D1, F = W1.shape
    if D1 != D or W2.shape != (F, D):
        raise OracleError(f"shape mismatch X{X.shape} W1{W1.shape} W2{W2.shape}")
    return N, D, F


def shard_fwd(X, W1, b1, W2, T, r, act="gelu_tanh"):
    """(Z, H, P) of shard r of T; W1, b1, W2 are the full weights."""
    X, W1, b1, W2 = _f64(X), _f64(W1), _f64(b1), _f64(W2)
    N, D, F = _dims(X, W1, W2)
    fs = F // T if T > 0 else 0
    Z = np.empty((N, fs)); H = np.empty((N, fs)); P = np.empty((N, D))
    _check(_load().oracle_shard_fwd(_p(X), _p(W1), _p(b1), _p(W2), N, D, F, T, r,
                                    _act_code(act), _p(Z), _p(H), _p(P)), "oracle_shard_fwd")
    return Z, H, P


def partial_sum(partials, b2=None):
    """Y = ((P0 + P1) + ...) + b2 over the list of [N, D] partials."""
    Ps = [_f64(p) for p in partials]
    T = len(Ps)
    N, D = Ps[0].shape
    for p in Ps:
        if p.shape != (N, D):
            raise OracleError("partials differ in shape")
    b2 = _f64(b2)
    arr = (ctypes.c_void_p * T)(*[p.ctypes.data for p in Ps])
    Y = np.empty((N, D))
    _check(_load().oracle_partial_sum(ctypes.cast(arr, ctypes.c_void_p), T, _p(b2), N, D,
                                      _p(Y)), "oracle_partial_sum")
    return Y


def partial_sum_bias_share(partials, b2, T):
    """b2 split over the ranks [Z 05]: Y = ((P0 + b2/T) + (P1 + b2/T)) + ... over the given
    [N, D] partials (all T of them for the tail, or one rank's for its contribution)."""
    Ps = [_f64(p) for p in partials]
    N, D = Ps[0].shape
    for p in Ps:
        if p.shape != (N, D):
            raise OracleError("partials differ in shape")
    b2 = _f64(b2)
    arr = (ctypes.c_void_p * len(Ps))(*[p.ctypes.data for p in Ps])
    Y = np.empty((N, D))
    _check(_load().oracle_partial_sum_bias_share(ctypes.cast(arr, ctypes.c_void_p), len(Ps), T,
                                                 _p(b2), N, D, _p(Y)),
           "oracle_partial_sum_bias_share")
    return Y


def block_fwd(X, W1, b1, W2, b2, T, act="gelu_tanh"):
    X, W1, b1, W2, b2 = _f64(X), _f64(W1), _f64(b1), _f64(W2), _f64(b2)
    N, D, F = _dims(X, W1, W2)
    Y = np.empty((N, D))
    _check(_load().oracle_block_fwd(_p(X), _p(W1), _p(b1), _p(W2), _p(b2), N, D, F, T,
                                    _act_code(act), _p(Y)), "oracle_block_fwd")
    return Y


def dense_fwd(X, W1, b1, W2, b2, act="gelu_tanh"):
    X, W1, b1, W2, b2 = _f64(X), _f64(W1), _f64(b1), _f64(W2), _f64(b2)
    N, D, F = _dims(X, W1, W2)
    Y = np.empty((N, D))
    _check(_load().oracle_dense_fwd(_p(X), _p(W1), _p(b1), _p(W2), _p(b2), N, D, F,
                                    _act_code(act), _p(Y)), "oracle_dense_fwd")
    return Y


def shard_bwd(X, W1, b1, W2, dY, T, r, act="gelu_tanh", want=("dZ", "dW1", "db1", "dW2", "dX")):
    """Gradients of shard r: dict with dZ [N,Fs], dW1 [D,Fs], db1 [Fs], dW2 [Fs,D], dX [N,D]."""
    X, W1, b1, W2, dY = _f64(X), _f64(W1), _f64(b1), _f64(W2), _f64(dY)
    N, D, F = _dims(X, W1, W2)
    fs = F // T if T > 0 else 0
    out = {"dZ": np.empty((N, fs))}
    out["dW1"] = np.empty((D, fs)) if "dW1" in want else None
    out["db1"] = np.empty((fs,)) if "db1" in want else None
    out["dW2"] = np.empty((fs, D)) if "dW2" in want else None
    out["dX"] = np.empty((N, D)) if "dX" in want else None
    _check(_load().oracle_shard_bwd(_p(X), _p(W1), _p(b1), _p(W2), _p(dY), N, D, F, T, r,
                                    _act_code(act), _p(out["dZ"]), _p(out["dW1"]),
                                    _p(out["db1"]), _p(out["dW2"]), _p(out["dX"])),
           "oracle_shard_bwd")
    return {k: v for k, v in out.items() if v is not None}


def dense_bwd(X, W1, b1, W2, dY, act="gelu_tanh"):
    """Unsharded gradients: dict with dW1 [D,F], db1 [F], dW2 [F,D], db2 [D], dX [N,D]."""
    X, W1, b1, W2, dY = _f64(X), _f64(W1), _f64(b1), _f64(W2), _f64(dY)
    N, D, F = _dims(X, W1, W2)
    out = {"dW1": np.empty((D, F)), "db1": np.empty((F,)), "dW2": np.empty((F, D)),
           "db2": np.empty((D,)), "dX": np.empty((N, D))}
    _check(_load().oracle_dense_bwd(_p(X), _p(W1), _p(b1), _p(W2), _p(dY), N, D, F,
                                    _act_code(act), _p(out["dW1"]), _p(out["db1"]),
                                    _p(out["dW2"]), _p(out["db2"]), _p(out["dX"])),
           "oracle_dense_bwd")
    return out


def token_slice(N, T, r):
    """(first row, row count) of token slice r of T in the reduce-scatter layout."""
    row0, rows = ctypes.c_int64(), ctypes.c_int64()
    _check(_load().oracle_token_slice(N, T, r, ctypes.byref(row0), ctypes.byref(rows)),
           "oracle_token_slice")
    return row0.value, rows.value


def partial_reduce_scatter(partials, r, b2=None):
    """Token slice r of ((P0 + P1) + ...) + b2: the rows token_slice(N, T, r) of the tail."""
    Ps = [_f64(p) for p in partials]
    T = len(Ps)
    N, D = Ps[0].shape
    for p in Ps:
        if p.shape != (N, D):
            raise OracleError("partials differ in shape")
    b2 = _f64(b2)
    arr = (ctypes.c_void_p * T)(*[p.ctypes.data for p in Ps])
    _, rows = token_slice(N, T, r) if 0 <= r < T else (0, 0)
    Yr = np.empty((rows, D))
    _check(_load().oracle_partial_reduce_scatter(ctypes.cast(arr, ctypes.c_void_p), T, r,
                                                 _p(b2), N, D, _p(Yr)),
           "oracle_partial_reduce_scatter")
    return Yr


def silu(z):
    z = _f64(z)
    out = np.empty_like(z)
    _check(_load().oracle_silu_vec(_p(z), _p(out), z.size, 0), "oracle_silu_vec")
    return out


def silu_deriv(z):
    z = _f64(z)
    out = np.empty_like(z)
    _check(_load().oracle_silu_vec(_p(z), _p(out), z.size, 1), "oracle_silu_vec")
    return out


def _gated_dims(X, Wg, Wu, W2):
    N, D = X.shape
    D1, F = Wg.shape
    if D1 != D or Wu.shape != (D, F) or W2.shape != (F, D):
        raise OracleError(f"shape mismatch X{X.shape} Wg{Wg.shape} Wu{Wu.shape} W2{W2.shape}")
    return N, D, F


def swiglu_shard_fwd(X, Wg, Wu, W2, T, r):
    """(G, U, H, P) of gated shard r of T; Wg, Wu, W2 are the full weights."""
    X, Wg, Wu, W2 = _f64(X), _f64(Wg), _f64(Wu), _f64(W2)
    N, D, F = _gated_dims(X, Wg, Wu, W2)
    fs = F // T if T > 0 else 0
    G = np.empty((N, fs)); U = np.empty((N, fs)); H = np.empty((N, fs)); P = np.empty((N, D))
    _check(_load().oracle_swiglu_shard_fwd(_p(X), _p(Wg), _p(Wu), _p(W2), N, D, F, T, r,
                                           _p(G), _p(U), _p(H), _p(P)),
           "oracle_swiglu_shard_fwd")
    return G, U, H, P


def swiglu_dense_fwd(X, Wg, Wu, W2):
    X, Wg, Wu, W2 = _f64(X), _f64(Wg), _f64(Wu), _f64(W2)
    N, D, F = _gated_dims(X, Wg, Wu, W2)
    Y = np.empty((N, D))
    _check(_load().oracle_swiglu_dense_fwd(_p(X), _p(Wg), _p(Wu), _p(W2), N, D, F, _p(Y)),
           "oracle_swiglu_dense_fwd")
    return Y


def swiglu_shard_bwd(X, Wg, Wu, W2, dY, T, r):
    """Gradients of gated shard r: dict with dG, dU [N,Fs], dWg, dWu [D,Fs], dW2 [Fs,D],
    dX [N,D]."""
    X, Wg, Wu, W2, dY = _f64(X), _f64(Wg), _f64(Wu), _f64(W2), _f64(dY)
    N, D, F = _gated_dims(X, Wg, Wu, W2)
    fs = F // T if T > 0 else 0
    out = {"dG": np.empty((N, fs)), "dU": np.empty((N, fs)), "dWg": np.empty((D, fs)),
           "dWu": np.empty((D, fs)), "dW2": np.empty((fs, D)), "dX": np.empty((N, D))}
    _check(_load().oracle_swiglu_shard_bwd(_p(X), _p(Wg), _p(Wu), _p(W2), _p(dY), N, D, F, T,
                                           r, _p(out["dG"]), _p(out["dU"]), _p(out["dWg"]),
                                           _p(out["dWu"]), _p(out["dW2"]), _p(out["dX"])),
           "oracle_swiglu_shard_bwd")
    return out


def num_threads() -> int:
    return int(_load().oracle_num_threads())
