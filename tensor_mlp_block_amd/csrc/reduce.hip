// reduce.hip -- block-tail reduction of the row-parallel partials on one GPU.
//
// Pages cited, as [tag section]:
//   [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
//   [U] unpurerationalist.github.io, "LLM Systems 16: Model Parallel Training"
//
// Y = (((P0 + P1) + ...) + P_{T-1}) + b2: the element-wise sum an all-reduce of the
// row-parallel outputs performs [Z 02], [Z 04], with b2 added exactly once after the sum
// [Z 05], [U 3.8]. The work is pure streaming: T fp32 reads and one fp32 write per element,
// so it is bound by HBM bandwidth. Each thread handles 16-byte vectors; the T loads of one
// vector are issued back to back, for several vectors per thread, so many independent 16-byte
// requests are in flight per thread, and the streaming loads/stores are marked non-temporal so
// they do not evict anything useful from the caches.
#include "common.hpp"
#include "launch.hpp"

#include <string.h>

#define MLP_TP_MAX_REDUCE_T_INTERNAL 64

namespace mlptp {

struct PartialPtrs {
    const float* p[MLP_TP_MAX_REDUCE_T_INTERNAL];
};

__device__ __forceinline__ f32x4 ld_nt(const float* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

__device__ __forceinline__ void st_nt(float* p, f32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

__device__ __forceinline__ float bias_at(const void* b2, int b2_dtype, int64_t c)
{
    return b2_dtype == kBF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(b2)[c])
                             : static_cast<const float*>(b2)[c];
}

// b2[c .. c+3] widened to fp32 (c % 4 == 0).
__device__ __forceinline__ f32x4 bias4(const void* b2, int b2_dtype, int64_t c)
{
    if (b2_dtype == kBF16) {
        const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(b2) + c);
        return f32x4{bf16_bits_to_f32(w.x & 0xffffu), bf16_bits_to_f32(w.x >> 16),
                     bf16_bits_to_f32(w.y & 0xffffu), bf16_bits_to_f32(w.y >> 16)};
    }
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(b2) + c);
}

// Vector path: D % 4 == 0, so the 4 elements of a vector share one row of b2's index space.
// Each thread owns VECS vectors spaced kBlock apart (so every load instruction of a wave is
// one contiguous 1 KB run) and issues all T x VECS loads before the first add: enough bytes
// in flight per CU to cover HBM latency without a grid-stride loop. Four vectors per thread
// where that still gives at least kMinGroups4 workgroups, two below (more workgroups for a
// short sum). Measured at T = 8 (one MI355X, bit-identical): a 256-row slice of a
// [2048, 12288] tail 23.4 -> 18.0 us with two; the whole [2048, 12288] tail 142.3 us with four
// against 146.1 with two, and a [4096, 8192] sum 184.1 against 194.8.
constexpr int kBlock = 256;
constexpr int64_t kMinGroups4 = 2048;

template <int TT, int VECS>
__global__ __launch_bounds__(kBlock) void partial_reduce_vec(PartialPtrs P, int T, const void* b2,
                                                             int b2_dtype, float* Y, int64_t nvec,
                                                             int64_t D, int64_t v0)
{
    constexpr int kVecs = VECS;
    const int nt = TT > 0 ? TT : T;
    const int64_t base = v0 + (int64_t)blockIdx.x * (kBlock * kVecs) + threadIdx.x;
    f32x4 s[kVecs];
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
        const int64_t v = base + u * kBlock;
        s[u] = v < nvec ? ld_nt(P.p[0] + v * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int r = 1; r < (TT > 0 ? TT : MLP_TP_MAX_REDUCE_T_INTERNAL); ++r) {
        if (r >= nt) break;
#pragma unroll
        for (int u = 0; u < kVecs; ++u) {
            const int64_t v = base + u * kBlock;
            if (v < nvec) s[u] += ld_nt(P.p[r] + v * 4);
        }
    }
    if (b2) {
        // Column of the thread's first vector, then advanced by 4 kBlock elements per vector
        // (one 64-bit remainder per thread, not per vector). The 4 bias values of a vector are
        // contiguous and 8- or 16-byte aligned (b2 is 16-byte aligned and c % 4 == 0).
        int64_t c = (base * 4) % D;
#pragma unroll
        for (int u = 0; u < kVecs; ++u) {
            if (u > 0) {
                c += 4 * kBlock;
                while (c >= D) c -= D;
            }
            s[u] += bias4(b2, b2_dtype, c);
        }
    }
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
        const int64_t v = base + u * kBlock;
        if (v < nvec) st_nt(Y + v * 4, s[u]);
    }
}

// Element path for D % 4 != 0.
__global__ __launch_bounds__(256) void partial_reduce_scalar(PartialPtrs P, int T, const void* b2,
                                                             int b2_dtype, float* Y, int64_t n,
                                                             int64_t D)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
        float s = P.p[0][e];
        for (int r = 1; r < T; ++r) s += P.p[r][e];
        if (b2) s += bias_at(b2, b2_dtype, e % D);
        Y[e] = s;
    }
}

void launch_partial_reduce(const float* const* P, int T, const void* b2, int b2_dtype, float* Y,
                           int64_t N, int64_t D, hipStream_t s)
{
    PartialPtrs pp;
    memset(&pp, 0, sizeof(pp));
    for (int r = 0; r < T; ++r) pp.p[r] = P[r];
    const int64_t n = N * D;
    // The element path grid-strides over at most this many workgroups.
    const int64_t max_groups = 256 * 16;
    if (D % 4 == 0) {
        // One launch per chunk of at most 2^30 workgroups (2^40 elements), so the grid size
        // always fits; a single launch covers anything that fits in one GPU's memory.
        const int64_t nvec = n / 4;
        const int vecs = ceil_div(nvec, (int64_t)kBlock * 4) >= kMinGroups4 ? 4 : 2;
        const int64_t per_group = (int64_t)kBlock * vecs;
        const int64_t max_launch = int64_t(1) << 30;
        for (int64_t g0 = 0; g0 < ceil_div(nvec, per_group); g0 += max_launch) {
            const int64_t groups = ceil_div(nvec, per_group) - g0;
            const dim3 grid((uint32_t)(groups < max_launch ? groups : max_launch)), block(kBlock);
            const int64_t v0 = g0 * per_group;
            auto launch = [&](auto tt, auto vv) {
                hipLaunchKernelGGL((partial_reduce_vec<decltype(tt)::value, decltype(vv)::value>), grid,
                                   block, 0, s, pp, T, b2, b2_dtype, Y, nvec, D, v0);
            };
            auto with_t = [&](auto vv) {
                switch (T) {
                case 1: launch(std::integral_constant<int, 1>{}, vv); break;
                case 2: launch(std::integral_constant<int, 2>{}, vv); break;
                case 4: launch(std::integral_constant<int, 4>{}, vv); break;
                case 8: launch(std::integral_constant<int, 8>{}, vv); break;
                default: launch(std::integral_constant<int, 0>{}, vv); break;
                }
            };
            if (vecs == 4)
                with_t(std::integral_constant<int, 4>{});
            else
                with_t(std::integral_constant<int, 2>{});
        }
    } else {
        const int64_t groups = ceil_div(n, 256) < max_groups ? ceil_div(n, 256) : max_groups;
        hipLaunchKernelGGL(partial_reduce_scalar, dim3((uint32_t)groups), dim3(256), 0, s, pp, T, b2,
                           b2_dtype, Y, n, D);
    }
}

}  // namespace mlptp
