"""Seeded synthetic inputs for the MLP shard. Holds none of the method's arithmetic.

Both the GPU tests/benchmark and the CPU oracle tests draw their inputs from here and nowhere
else, so the two sides always see the same values.

Recipe. Every tensor of the block is a fixed function of ``(seed, tensor tag)`` and its full
(global) shape. Each is cut into blocks of ``BLOCK`` rows or columns along one axis, and each
block is drawn from its own ``torch.Generator('cpu')`` seeded with a splitmix64 hash of
``(seed, tag, block index)``:

* X [N, D] and dY [N, D]: blocks of ``BLOCK`` token rows;
* W1 [D, F] and b1 [F]: blocks of ``BLOCK`` columns, so a column shard W1[:, r*Fs:(r+1)*Fs]
  is bit-identical to the same slice of the full weight, and computing it does not require
  drawing the other shards ("slice one fixed full weight", not a seed per rank: zwjcode.cn,
  "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约", section 09);
* Wg [D, F] and Wu [D, F] (the gated form's gate and up weights): as W1, blocks of ``BLOCK``
  columns, each under its own tag;
* W2 [F, D]: blocks of ``BLOCK`` rows (the row shard is a slice of the full weight);
* b2 [D]: a single block.

Distributions: ``"normal"`` draws fp32 N(0, 1) values and scales them by the tensor's std,
then rounds to bf16 with round-to-nearest-even (torch's ``.to(torch.bfloat16)``); ``"int"``
draws uniform integers in [-2, 2] and stores them exactly in fp32.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import torch

from .workloads import Workload

BLOCK = 128

TAG_X, TAG_W1, TAG_B1, TAG_W2, TAG_B2, TAG_DY, TAG_WG, TAG_WU = 1, 2, 3, 4, 5, 6, 7, 8

_MASK64 = (1 << 64) - 1


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _MASK64
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & _MASK64
    return x ^ (x >> 31)


def block_seed(seed: int, tag: int, index: int) -> int:
    h = _splitmix64(seed & _MASK64)
    h = _splitmix64(h ^ tag)
    h = _splitmix64(h ^ index)
    return h & ((1 << 63) - 1)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw_block(out: torch.Tensor, seed: int, kind: str, std: float) -> None:
    g = torch.Generator("cpu")
    g.manual_seed(seed)
    if kind == "normal":
        torch.randn(out.shape, generator=g, out=out)
        if std != 1.0:
            out.mul_(std)
    elif kind == "int":
        out.copy_(torch.randint(-2, 3, out.shape, generator=g, dtype=torch.int32))
    else:
        raise ValueError(f"unknown distribution {kind!r}")


def blocked_slice(seed: int, tag: int, full_shape: tuple, axis: int, lo: int, hi: int,
                  kind: str, std: float) -> torch.Tensor:
    """fp32 slice [lo, hi) along ``axis`` of the blocked tensor of ``full_shape``."""
    full_shape = tuple(int(s) for s in full_shape)
    extent = full_shape[axis]
    if not (0 <= lo <= hi <= extent):
        raise ValueError(f"slice [{lo},{hi}) outside axis of length {extent}")
    b0, b1 = lo // BLOCK, (hi + BLOCK - 1) // BLOCK
    cover_lo, cover_hi = b0 * BLOCK, min(b1 * BLOCK, extent)
    shape = list(full_shape)
    shape[axis] = cover_hi - cover_lo
    buf = torch.empty(shape, dtype=torch.float32)

    def one(b: int) -> None:
        s, e = b * BLOCK, min((b + 1) * BLOCK, extent)
        view = buf.narrow(axis, s - cover_lo, e - s)
        tmp = torch.empty(view.shape, dtype=torch.float32)
        _draw_block(tmp, block_seed(seed, tag, b), kind, std)
        view.copy_(tmp)

    blocks = range(b0, b1)
    if len(blocks) > 1 and buf.numel() > (1 << 20):
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, blocks))
    else:
        for b in blocks:
            one(b)
    return buf.narrow(axis, lo - cover_lo, hi - lo).contiguous()


def _finish(t: torch.Tensor, w: Workload) -> torch.Tensor:
    if w.dtype == "bf16":
        return t.to(torch.bfloat16)
    if w.dtype == "f32":
        return t
    raise ValueError(f"unknown dtype {w.dtype!r}")


def gen_X(w: Workload) -> torch.Tensor:
    return _finish(blocked_slice(w.seed, TAG_X, (w.N, w.D), 0, 0, w.N, w.dist, w.x_std), w)


def gen_W1(w: Workload, c0: int = 0, c1: int | None = None) -> torch.Tensor:
    c1 = w.F if c1 is None else c1
    return _finish(blocked_slice(w.seed, TAG_W1, (w.D, w.F), 1, c0, c1, w.dist, w.w_std), w)


def gen_Wg(w: Workload, c0: int = 0, c1: int | None = None) -> torch.Tensor:
    c1 = w.F if c1 is None else c1
    return _finish(blocked_slice(w.seed, TAG_WG, (w.D, w.F), 1, c0, c1, w.dist, w.w_std), w)


def gen_Wu(w: Workload, c0: int = 0, c1: int | None = None) -> torch.Tensor:
    c1 = w.F if c1 is None else c1
    return _finish(blocked_slice(w.seed, TAG_WU, (w.D, w.F), 1, c0, c1, w.dist, w.w_std), w)


def gen_b1(w: Workload, c0: int = 0, c1: int | None = None) -> torch.Tensor:
    c1 = w.F if c1 is None else c1
    return _finish(blocked_slice(w.seed, TAG_B1, (w.F,), 0, c0, c1, w.dist, w.b_std), w)


def gen_W2(w: Workload, r0: int = 0, r1: int | None = None) -> torch.Tensor:
    r1 = w.F if r1 is None else r1
    return _finish(blocked_slice(w.seed, TAG_W2, (w.F, w.D), 0, r0, r1, w.dist, w.w_std), w)


def gen_b2(w: Workload) -> torch.Tensor:
    return _finish(blocked_slice(w.seed, TAG_B2, (w.D,), 0, 0, w.D, w.dist, w.b_std), w)


def gen_dY(w: Workload) -> torch.Tensor:
    seed = w.dy_seed if w.dy_seed is not None else w.seed
    return _finish(blocked_slice(seed, TAG_DY, (w.N, w.D), 0, 0, w.N, w.dist, w.dy_std), w)

