"""Shapes that put each large tile of the bf16 GEMMs under test: a ragged row or column edge
of every 256-class tile, and grids of two rounds of workgroups.

Each case names the tile every product of interest is meant to take on an MI355X (256 compute
units), as the library's own chooser (``mlp_tp_shard_tile``) reports it. A CPU test pins
those choices, so the GPU tests that run these shapes really cover the tiles they name. The
contractions are kept short (K = 64 or 72: one full and one partial 64-deep stage for 72) so
the fp64 oracle compares every element in about a second.

zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约", section 10 asks for exactly this:
evidence that the implementation is not silently wrong at the places a fast path could be.
"""
from tensor_mlp_block_amd.workloads import Workload

MI355X_CUS = 256


def _w(name, N, D, F, seed):
    return Workload(name, N=N, D=D, F=F, T=1, act="gelu_tanh", dtype="bf16", seed=seed,
                    dist="normal")


# (workload, {product: (tile rows, tile cols)}) for T = 1 (the shard is the whole layer).
EDGE_CASES = [
    # up-projection and dH on 256 x 224 over 4000 tokens: the last row tile holds 160 rows
    (_w("edge224_n4000_d72_f3584", 4000, 72, 3584, 7201), {"up": (256, 224), "dh": (256, 224)}),
    # up-projection and dH on 256 x 192 over 2000 tokens (the last row tile holds 208)
    (_w("edge192_n2000_d72_f6144", 2000, 72, 6144, 7202), {"up": (256, 192), "dh": (256, 192)}),
    # down-projection and dX on 256 x 256, ragged in both directions (4000 = 15 x 256 + 160)
    (_w("edge256_n4000_d4000_f64", 4000, 4000, 64, 7203), {"down": (256, 256), "dx": (256, 256)}),
    # down-projection and dX on 224 x 256 over 3584 tokens, ragged columns
    (_w("edge224m_n3584_d4000_f64", 3584, 4000, 64, 7204), {"down": (224, 256), "dx": (224, 256)}),
    # weight gradients (both operands token-major) on 256 x 256, ragged in both directions
    (_w("wgrad256_n72_d4000_f4000", 72, 4000, 4000, 7205), {"dw2": (256, 256), "dw1": (256, 256)}),
    # weight gradients on 224 x 256 (dW2, ragged columns) and 256 x 224 (dW1, ragged rows)
    (_w("wgrad224_n72_d4000_f3584", 72, 4000, 3584, 7206), {"dw2": (224, 256), "dw1": (256, 224)}),
    # two rounds of 256 workgroups: 512 tiles of 256 x 256 (down-projection and dX)
    (_w("round2_n4096_d8192_f64", 4096, 8192, 64, 7207), {"down": (256, 256), "dx": (256, 256)}),
    # two rounds of 256 x 192 tiles, the GPT-3-175B shard's down-projection grid
    (_w("round2_n2048_d12288_f64", 2048, 12288, 64, 7208), {"down": (256, 192), "dx": (256, 192)}),
]
