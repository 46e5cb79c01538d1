"""Named synthetic workloads: shapes, dtypes, activations, seeds and value distributions.

Shapes follow the models the pages use as examples; the values are seeded synthetic draws
(see ``synth``), never real weights or data.

N = B * L tokens (the [B, L, D] activation flattened to [N, D] row-major), D the model width,
F the FFN width, T the shard count; each shard owns F / T hidden columns.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    D: int
    F: int
    T: int
    act: str                    # "relu" | "gelu_tanh" | "gelu_erf" | "identity" | "swiglu"
    dtype: str                  # "f32" (exact integer data) | "bf16"
    seed: int
    dist: str                   # "int": uniform integers in [-2, 2]; "normal": N(0, std^2)
    x_std: float = 1.0
    w_std: float = 0.02
    b_std: float = 0.02
    dy_std: float = 1.0
    dy_seed: int | None = None
    bias: bool = True

    @property
    def Fs(self) -> int:
        return self.F // self.T

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# Integer-valued fp32 case: every product and sum is an integer below 2^24, so any
# summation order gives the same fp32 result and the GPU must match the oracle exactly.
INT_EXACT = Workload("int_exact_n64_d64_f256_t2", N=64, D=64, F=256, T=2, act="relu",
                     dtype="f32", seed=101, dist="int")

# GPT-2-medium-sized MLP (D=1024, F=4D) on 8 x 512 tokens, two shards.
GPT2_MEDIUM_T2 = Workload("gpt2_medium_n4096_d1024_f4096_t2", N=4096, D=1024, F=4096, T=2,
                          act="gelu_tanh", dtype="bf16", seed=202, dist="normal")

# Llama-3-70B FFN width (W1 [8192, 28672]) split 8 ways: one rank's shard F/T = 3584 on
# 4 x 1024 tokens. The output is that rank's fp32 partial.
LLAMA70B_SHARD_T8 = Workload("llama3_70b_ffn_shard_n4096_d8192_f28672_t8", N=4096, D=8192,
                             F=28672, T=8, act="gelu_tanh", dtype="bf16", seed=303,
                             dist="normal")

# GPT-3-175B MLP (12288 -> 49152 -> 12288) as 8 shards of 6144 run one after another on one
# GPU over 2048 tokens, then the 8 partials are summed with b2 added once.
GPT3_175B_T8 = Workload("gpt3_175b_mlp_n2048_d12288_f49152_t8", N=2048, D=12288, F=49152,
                        T=8, act="gelu_tanh", dtype="bf16", seed=404, dist="normal")

# Backward of the Llama-3-70B shard with a seeded upstream gradient dY ~ N(0, 1).
LLAMA70B_SHARD_T8_BWD = LLAMA70B_SHARD_T8.with_(
    name="llama3_70b_ffn_shard_bwd_n4096_d8192_f28672_t8", dy_seed=505)

# The gated (SwiGLU) form of the same Llama-3-70B FFN shard: gate and up weights [8192, 28672]
# cut 8 ways at the same columns, no biases.
LLAMA70B_SWIGLU_SHARD_T8 = Workload("llama3_70b_swiglu_shard_n4096_d8192_f28672_t8", N=4096,
                                    D=8192, F=28672, T=8, act="swiglu", dtype="bf16",
                                    seed=606, dist="normal", bias=False)

# The MLP shape of the pages' PyTorch example (d_model = 4096, d_ff = 11008, x [2, 128, 4096]),
# for the shard-count sweep: T = 1, 2, 4, 8 all divide 11008.
PAGE_EXAMPLE_MLP = Workload("page_example_mlp_n256_d4096_f11008", N=256, D=4096, F=11008, T=1,
                            act="gelu_tanh", dtype="bf16", seed=707, dist="normal")

ALL = (INT_EXACT, GPT2_MEDIUM_T2, LLAMA70B_SHARD_T8, GPT3_175B_T8, LLAMA70B_SHARD_T8_BWD,
       LLAMA70B_SWIGLU_SHARD_T8, PAGE_EXAMPLE_MLP)

BY_NAME = {w.name: w for w in ALL}
