// epilogue.hpp -- fused GEMM epilogues of the MLP shard (bf16 or fp32 storage).
//
// Pages cited, as [tag section]:
//   [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
//   [U] unpurerationalist.github.io, "LLM Systems 16: Model Parallel Training"
//
// Each functor receives four consecutive fp32 results C[row, col .. col+3] (col % 4 == 0) and
// the GEMM extent; it writes nothing outside [0, M) x [0, N). `vec` says the output row
// stride allows one vector store per four elements.
#pragma once

#include "common.hpp"

namespace mlptp {

__device__ __forceinline__ f32x4 load4(const float* p, int n, bool vec)
{
    if (vec && n == 4) return *reinterpret_cast<const f32x4*>(p);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < n) v[e] = p[e];
    return v;
}

__device__ __forceinline__ f32x4 load4(const uint16_t* p, int n, bool vec)
{
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (vec && n == 4) {
        uint2 w = *reinterpret_cast<const uint2*>(p);
        v[0] = bf16_bits_to_f32(w.x & 0xffffu);
        v[1] = bf16_bits_to_f32(w.x >> 16);
        v[2] = bf16_bits_to_f32(w.y & 0xffffu);
        v[3] = bf16_bits_to_f32(w.y >> 16);
        return v;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < n) v[e] = bf16_bits_to_f32(p[e]);
    return v;
}

__device__ __forceinline__ void store4(float* p, f32x4 v, int n, bool vec)
{
    if (vec && n == 4) {
        *reinterpret_cast<f32x4*>(p) = v;
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < n) p[e] = v[e];
}

__device__ __forceinline__ void store4(uint16_t* p, f32x4 v, int n, bool vec)
{
    if (vec && n == 4) {
        *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < n) p[e] = f32_to_bf16_bits(v[e]);
}

__device__ __forceinline__ int valid4(int64_t row, int64_t col, int64_t M, int64_t N)
{
    if (row >= M || col >= N) return 0;
    const int64_t n = N - col;
    return n < 4 ? (int)n : 4;
}

// Plain fp32 store: the row-parallel partial P^(r) (no b2 [Z 05]), weight gradients, dX^(r).
struct EpiStoreF32 {
    float* C;
    int64_t ldc;
    int vec;
    __device__ __forceinline__ void operator()(int64_t row, int64_t col, f32x4 v, int64_t M,
                                               int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        if (n) store4(C + row * ldc + col, v, n, vec);
    }
};

// Up-projection epilogue [Z 02], [Z 05]: z = acc + b1^(r)[col] (the bias slice that travels
// with W1's columns), optional store of Z for the backward, H = phi(z). One HBM write each.
template <class T, int ACT>
struct EpiBiasAct {
    const T* bias;  // [N] or nullptr
    T* Z;           // [M, N] or nullptr
    T* H;           // [M, N]
    int64_t ldc;
    int vec;
    __device__ __forceinline__ void operator()(int64_t row, int64_t col, f32x4 v, int64_t M,
                                               int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        if (!n) return;
        if (bias) v += load4(bias + col, n, true);
        if (Z) store4(Z + row * ldc + col, v, n, vec);
        f32x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = act_fwd<ACT>(v[e]);
        store4(H + row * ldc + col, h, n, vec);
    }
};

// Backward through the local activation [Z 06], [U 3.6.1]: dZ = dH * phi'(Z), where the
// GEMM produced dH = dY W2^(r)^T.
template <class T, int ACT>
struct EpiActGrad {
    const T* Z;  // [M, N]
    T* dZ;       // [M, N]
    int64_t ldc;
    int vec;
    __device__ __forceinline__ void operator()(int64_t row, int64_t col, f32x4 v, int64_t M,
                                               int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        if (!n) return;
        const f32x4 z = load4(Z + row * ldc + col, n, vec);
        f32x4 d;
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = v[e] * act_grad<ACT>(z[e]);
        store4(dZ + row * ldc + col, d, n, vec);
    }
};

}  // namespace mlptp
