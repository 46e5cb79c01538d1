// epilogue.hpp -- fused GEMM epilogues of the MLP shard (bf16 or fp32 storage).
//
// Pages cited, as [tag section]:
//   [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
//   [U] unpurerationalist.github.io, "LLM Systems 16: Model Parallel Training"
//
// Each functor handles four consecutive fp32 results C[row, col .. col+3] (col % 4 == 0) and
// writes nothing outside [0, M) x [0, N); `vec` says the output row stride allows one vector
// store per four elements. The work is split in three so that a kernel can issue every load an
// epilogue needs before its first store:
//   col_load(col, N)          data that depends on the column only (a bias slice);
//   elem_load(row, col, M, N) data per element (a saved activation input);
//   apply(row, col, v, c, e, M, N) the arithmetic and the stores.
// operator() runs the three in order, for kernels that do not stage the loads.
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

// Four bf16 values kept packed (two dwords) between a load and its use.
struct Bf16x4 {
    uint32_t lo, hi;
};

__device__ __forceinline__ Bf16x4 load4_raw(const uint16_t* p, int n, bool vec)
{
    if (vec && n == 4) {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        return Bf16x4{w.x, w.y};
    }
    uint16_t e[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (i < n) e[i] = p[i];
    return Bf16x4{(uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16)};
}

__device__ __forceinline__ f32x4 unpack4(Bf16x4 w)
{
    return f32x4{bf16_bits_to_f32(w.lo & 0xffffu), bf16_bits_to_f32(w.lo >> 16),
                 bf16_bits_to_f32(w.hi & 0xffffu), bf16_bits_to_f32(w.hi >> 16)};
}

// Storage of four staged values of type T: packed bf16, or fp32.
template <class T> struct Staged4;
template <> struct Staged4<uint16_t> {
    Bf16x4 raw;
    __device__ __forceinline__ static Staged4 load(const uint16_t* p, int n, bool vec)
    {
        return Staged4{load4_raw(p, n, vec)};
    }
    __device__ __forceinline__ f32x4 get() const { return unpack4(raw); }
};
template <> struct Staged4<float> {
    f32x4 raw;
    __device__ __forceinline__ static Staged4 load(const float* p, int n, bool vec)
    {
        return Staged4{load4(p, n, vec)};
    }
    __device__ __forceinline__ f32x4 get() const { return raw; }
};

struct NoData {};

__device__ __forceinline__ int valid4(int64_t row, int64_t col, int64_t M, int64_t N)
{
    if (row >= M || col >= N) return 0;
    const int64_t n = N - col;
    return n < 4 ? (int)n : 4;
}

// Plain store as T: the row-parallel partial P^(r) in fp32 (no b2 [Z 05]), weight gradients,
// dX^(r); in bf16, a staged gate pre-activation.
template <class T>
struct EpiStore {
    T* C;
    int64_t ldc;
    int vec;
    using ColData = NoData;
    using ElemData = NoData;
    static constexpr bool kColData = false, kElemData = false;
    __device__ __forceinline__ ColData col_load(int64_t, int64_t) const { return {}; }
    __device__ __forceinline__ ElemData elem_load(int64_t, int64_t, int64_t, int64_t) const
    {
        return {};
    }
    __device__ __forceinline__ void apply(int64_t row, int64_t col, f32x4 v, ColData, ElemData,
                                          int64_t M, int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        if (!n) return;
        // fp32 results (a partial, a gradient) are written once and read later by another
        // kernel, usually after far more other traffic than the caches hold: stream them past
        // the caches, so they do not evict operands that are read again.
        if (std::is_same<T, float>::value && vec && n == 4)
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(C + row * ldc + col));
        else
            store4(C + row * ldc + col, v, n, vec);
    }
    __device__ __forceinline__ void operator()(int64_t row, int64_t col, f32x4 v, int64_t M,
                                               int64_t N) const
    {
        apply(row, col, v, {}, {}, M, N);
    }
};
using EpiStoreF32 = EpiStore<float>;

// Row-parallel partial with this rank's share of b2 [Z 05]: C = v + b2[col] / T in fp32, the
// alternative to adding b2 once after the sum. b2 (of type TB, the full bias) is divided by T
// per column once, before the main loop; the division is IEEE (correctly rounded), so for T a
// power of two the share is exact.
template <class TB>
struct EpiBiasShare {
    float* C;
    const TB* b2;  // [N] or nullptr
    float T;
    int64_t ldc;
    int vec;
    using ColData = f32x4;  // b2[col .. col+3] / T, zero past N or without a bias
    using ElemData = NoData;
    static constexpr bool kColData = true, kElemData = false;
    __device__ __forceinline__ ColData col_load(int64_t col, int64_t N) const
    {
        const int64_t left = N - col;
        const int n = left <= 0 ? 0 : (left < 4 ? (int)left : 4);
        f32x4 b = {0.f, 0.f, 0.f, 0.f};
        if (!b2 || !n) return b;
        b = load4(b2 + col, n, true);
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = b[e] / T;
        return b;
    }
    __device__ __forceinline__ ElemData elem_load(int64_t, int64_t, int64_t, int64_t) const
    {
        return {};
    }
    __device__ __forceinline__ void apply(int64_t row, int64_t col, f32x4 v, ColData b, ElemData,
                                          int64_t M, int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        if (!n) return;
        v += b;
        if (vec && n == 4)
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(C + row * ldc + col));
        else
            store4(C + row * ldc + col, v, n, vec);
    }
    __device__ __forceinline__ void operator()(int64_t row, int64_t col, f32x4 v, int64_t M,
                                               int64_t N) const
    {
        apply(row, col, v, col_load(col, N), {}, M, N);
    }
};

// One split of a split contraction: the fp32 partial of split blockIdx.y goes to its own plane
// C + blockIdx.y * plane (ldc N) of a workspace, stored normally so that the pass summing the
// planes, which follows at once, finds them in the caches.
struct EpiSplitF32 {
    float* C;
    int64_t plane;
    int64_t ldc;
    int vec;
    using ColData = NoData;
    using ElemData = NoData;
    static constexpr bool kColData = false, kElemData = false;
    __device__ __forceinline__ ColData col_load(int64_t, int64_t) const { return {}; }
    __device__ __forceinline__ ElemData elem_load(int64_t, int64_t, int64_t, int64_t) const
    {
        return {};
    }
    __device__ __forceinline__ void apply(int64_t row, int64_t col, f32x4 v, ColData, ElemData,
                                          int64_t M, int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        if (n) store4(C + (int64_t)blockIdx.y * plane + row * ldc + col, v, n, vec);
    }
    __device__ __forceinline__ void operator()(int64_t row, int64_t col, f32x4 v, int64_t M,
                                               int64_t N) const
    {
        apply(row, col, v, {}, {}, M, N);
    }
};

// fp32 accumulation C += v: a down-projection adding its partial into one running buffer,
// the sequential one-GPU form of the block-tail sum [Z 02]. Each element is read and written
// by the same lane, so the update needs no atomics.
struct EpiAccumF32 {
    float* C;
    int64_t ldc;
    int vec;
    using ColData = NoData;
    using ElemData = Staged4<float>;
    static constexpr bool kColData = false, kElemData = true;
    __device__ __forceinline__ ColData col_load(int64_t, int64_t) const { return {}; }
    __device__ __forceinline__ ElemData elem_load(int64_t row, int64_t col, int64_t M,
                                                  int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        return n ? ElemData::load(C + row * ldc + col, n, vec) : ElemData::load(C, 0, false);
    }
    __device__ __forceinline__ void apply(int64_t row, int64_t col, f32x4 v, ColData, ElemData c,
                                          int64_t M, int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        if (n) store4(C + row * ldc + col, c.get() + v, n, vec);
    }
    __device__ __forceinline__ void operator()(int64_t row, int64_t col, f32x4 v, int64_t M,
                                               int64_t N) const
    {
        apply(row, col, v, {}, elem_load(row, col, M, N), M, N);
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
    using ColData = Staged4<T>;  // b1^(r)[col .. col+3], zero past N or without a bias
    using ElemData = NoData;
    static constexpr bool kColData = true, kElemData = false;
    __device__ __forceinline__ ColData col_load(int64_t col, int64_t N) const
    {
        const int64_t left = N - col;
        const int n = left <= 0 ? 0 : (left < 4 ? (int)left : 4);
        // The bias row is contiguous: a whole group of four is one aligned vector load
        // whenever the caller's pointer is 16-byte aligned, which the library requires.
        return (bias && n) ? ColData::load(bias + col, n, true) : ColData::load(bias, 0, false);
    }
    __device__ __forceinline__ ElemData elem_load(int64_t, int64_t, int64_t, int64_t) const
    {
        return {};
    }
    __device__ __forceinline__ void apply(int64_t row, int64_t col, f32x4 v, ColData b, ElemData,
                                          int64_t M, int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        if (!n) return;
        v += b.get();
        if (Z) store4(Z + row * ldc + col, v, n, vec);
        f32x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = act_fwd<ACT>(v[e]);
        store4(H + row * ldc + col, h, n, vec);
    }
    __device__ __forceinline__ void operator()(int64_t row, int64_t col, f32x4 v, int64_t M,
                                               int64_t N) const
    {
        apply(row, col, v, col_load(col, N), {}, M, N);
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
    using ColData = NoData;
    using ElemData = Staged4<T>;  // Z[row, col .. col+3], zero outside the matrix
    static constexpr bool kColData = false, kElemData = true;
    __device__ __forceinline__ ColData col_load(int64_t, int64_t) const { return {}; }
    __device__ __forceinline__ ElemData elem_load(int64_t row, int64_t col, int64_t M,
                                                  int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        return n ? ElemData::load(Z + row * ldc + col, n, vec) : ElemData::load(Z, 0, false);
    }
    __device__ __forceinline__ void apply(int64_t row, int64_t col, f32x4 v, ColData, ElemData z,
                                          int64_t M, int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        if (!n) return;
        const f32x4 zv = z.get();
        f32x4 d;
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = v[e] * act_grad<ACT>(zv[e]);
        store4(dZ + row * ldc + col, d, n, vec);
    }
    __device__ __forceinline__ void operator()(int64_t row, int64_t col, f32x4 v, int64_t M,
                                               int64_t N) const
    {
        apply(row, col, v, {}, elem_load(row, col, M, N), M, N);
    }
};

// Gated MLP [Z 08], fused form: the GEMM produced the gate g = X Wg^(r) and the up value
// u = X Wu^(r) of the same four columns (the two projections are cut at the same columns);
// H = SiLU(g) * u. G and U keep the pre-activations for the backward when non-null.
template <class T>
struct EpiSwiGLU {
    T* H;  // [M, N]
    T* G;  // [M, N] or nullptr
    T* U;  // [M, N] or nullptr
    int64_t ldc;
    int vec;
    static constexpr bool kDual = true;
    using ColData = NoData;
    static constexpr bool kColData = false;
    __device__ __forceinline__ void apply_dual(int64_t row, int64_t col, f32x4 g, f32x4 u,
                                               int64_t M, int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        if (!n) return;
        if (G) store4(G + row * ldc + col, g, n, vec);
        if (U) store4(U + row * ldc + col, u, n, vec);
        f32x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = silu_f(g[e]) * u[e];
        store4(H + row * ldc + col, h, n, vec);
    }
};

// Gated MLP, second pass of the two-GEMM form: the GEMM produced u = X Wu^(r); the gate
// values g were stored by the first pass in `gate` (which may be H itself: each element is
// read before it is overwritten, by the same lane). H = SiLU(g) * u.
template <class T>
struct EpiGateMul {
    const T* gate;  // [M, N]
    T* U;           // [M, N] or nullptr
    T* H;           // [M, N]
    int64_t ldc;
    int vec;
    using ColData = NoData;
    using ElemData = Staged4<T>;
    static constexpr bool kColData = false, kElemData = true;
    __device__ __forceinline__ ColData col_load(int64_t, int64_t) const { return {}; }
    __device__ __forceinline__ ElemData elem_load(int64_t row, int64_t col, int64_t M,
                                                  int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        return n ? ElemData::load(gate + row * ldc + col, n, vec) : ElemData::load(gate, 0, false);
    }
    __device__ __forceinline__ void apply(int64_t row, int64_t col, f32x4 u, ColData, ElemData g,
                                          int64_t M, int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        if (!n) return;
        if (U) store4(U + row * ldc + col, u, n, vec);
        const f32x4 gv = g.get();
        f32x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = silu_f(gv[e]) * u[e];
        store4(H + row * ldc + col, h, n, vec);
    }
    __device__ __forceinline__ void operator()(int64_t row, int64_t col, f32x4 u, int64_t M,
                                               int64_t N) const
    {
        apply(row, col, u, {}, elem_load(row, col, M, N), M, N);
    }
};

// Gated MLP backward [Z 08], through H = SiLU(g) * u by the product rule: the GEMM produced
// dh = dY W2^(r)^T for four columns; with s = sigmoid(g), dU = dh * SiLU(g) and
// dG = dh * u * SiLU'(g), where SiLU'(g) = s * (1 + g * (1 - s)). G and U are the stored
// pre-activations of the forward; dG and dU are written in the same dtype.
template <class T>
struct EpiSwiGLUGrad {
    const T* G;  // [M, N]
    const T* U;  // [M, N]
    T* dG;       // [M, N]
    T* dU;       // [M, N]
    int64_t ldc;
    int vec;
    using ColData = NoData;
    struct ElemData {
        Staged4<T> g, u;
    };
    static constexpr bool kColData = false, kElemData = true;
    __device__ __forceinline__ ColData col_load(int64_t, int64_t) const { return {}; }
    __device__ __forceinline__ ElemData elem_load(int64_t row, int64_t col, int64_t M,
                                                  int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        if (!n) return {Staged4<T>::load(G, 0, false), Staged4<T>::load(U, 0, false)};
        return {Staged4<T>::load(G + row * ldc + col, n, vec),
                Staged4<T>::load(U + row * ldc + col, n, vec)};
    }
    __device__ __forceinline__ void apply(int64_t row, int64_t col, f32x4 dh, ColData,
                                          ElemData gu, int64_t M, int64_t N) const
    {
        const int n = valid4(row, col, M, N);
        if (!n) return;
        const f32x4 g = gu.g.get(), u = gu.u.get();
        f32x4 dg, du;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float s = sigmoidf_(g[e]);
            du[e] = dh[e] * (g[e] * s);
            dg[e] = dh[e] * u[e] * (s * (1.0f + g[e] * (1.0f - s)));
        }
        store4(dG + row * ldc + col, dg, n, vec);
        store4(dU + row * ldc + col, du, n, vec);
    }
    __device__ __forceinline__ void operator()(int64_t row, int64_t col, f32x4 dh, int64_t M,
                                               int64_t N) const
    {
        apply(row, col, dh, {}, elem_load(row, col, M, N), M, N);
    }
};

}  // namespace mlptp
