// elementwise.hip -- bias and activation over an fp32 pre-activation: the up-projection's
// epilogue [Z 02], [Z 05] as a kernel of its own.
//
// Pages cited, as [tag section]:
//   [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
//
// H = phi(Z + b1^(r)) over a shard's [N, Fs] block: b1^(r) is the bias slice that travels with
// W1's columns [Z 05], and phi is elementwise, so each shard applies it to its own columns with
// no exchange [Z 02]. The up-projection fuses exactly this into its GEMM; the standalone form
// takes the GEMM's fp32 result from elsewhere. It is bound by HBM: 4 bytes read and 2 (bf16) or
// 4 (fp32) written per element, plus the bias, which stays in cache.
#include "common.hpp"
#include "launch.hpp"

namespace mlptp {

namespace {

constexpr int kEwBlock = 256, kEwVecs = 4;

template <class T>
__device__ __forceinline__ f32x4 bias4_at(const T* b, int64_t c);
template <>
__device__ __forceinline__ f32x4 bias4_at<uint16_t>(const uint16_t* b, int64_t c)
{
    const uint2 w = *reinterpret_cast<const uint2*>(b + c);
    return f32x4{bf16_bits_to_f32(w.x & 0xffffu), bf16_bits_to_f32(w.x >> 16),
                 bf16_bits_to_f32(w.y & 0xffffu), bf16_bits_to_f32(w.y >> 16)};
}
template <>
__device__ __forceinline__ f32x4 bias4_at<float>(const float* b, int64_t c)
{
    return *reinterpret_cast<const f32x4*>(b + c);
}

template <class T>
__device__ __forceinline__ void store4_to(T* p, f32x4 v);
template <>
__device__ __forceinline__ void store4_to<uint16_t>(uint16_t* p, f32x4 v)
{
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
template <>
__device__ __forceinline__ void store4_to<float>(float* p, f32x4 v)
{
    *reinterpret_cast<f32x4*>(p) = v;
}

template <class T>
__device__ __forceinline__ float load1(const T* b, int64_t c);
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t* b, int64_t c) { return bf16_bits_to_f32(b[c]); }
template <>
__device__ __forceinline__ float load1<float>(const float* b, int64_t c) { return b[c]; }

template <class T>
__device__ __forceinline__ void store1(T* p, float v);
template <>
__device__ __forceinline__ void store1<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
template <>
__device__ __forceinline__ void store1<float>(float* p, float v) { *p = v; }

// Vector path (Fs % 4 == 0): four 16-byte vectors of Z per thread, kEwBlock apart, all loaded
// before the first is processed; the 4 values of a vector share one bias row position. The
// bias column of the first vector is one 64-bit remainder per thread; the next vectors' columns
// are 4 kEwBlock elements further on, so each follows by one add and at most one subtraction
// (`step` = 4 kEwBlock mod Fs, from the host).
// Z holds S planes `plane` elements apart (S > 1: the fp32 partials of a split contraction),
// summed in plane order before the bias; Zout, when non-null, keeps the pre-activation.
template <class T, int ACT>
__global__ __launch_bounds__(kEwBlock) void bias_act_vec(const float* __restrict__ Z, int S,
                                                         int64_t plane, const T* __restrict__ b,
                                                         T* __restrict__ Zout,
                                                         T* __restrict__ H, int64_t nvec,
                                                         int64_t Fs, int64_t v0, int64_t step)
{
    const int64_t base = v0 + (int64_t)blockIdx.x * (kEwBlock * kEwVecs) + threadIdx.x;
    int64_t col = b ? (base * 4) % Fs : 0;
    f32x4 z[kEwVecs];
#pragma unroll
    for (int u = 0; u < kEwVecs; ++u) {
        const int64_t v = base + u * kEwBlock;
        z[u] = v < nvec ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Z) + v)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int p = 1; p < S; ++p) {
        const f32x4* Zp = reinterpret_cast<const f32x4*>(Z + p * plane);
#pragma unroll
        for (int u = 0; u < kEwVecs; ++u) {
            const int64_t v = base + u * kEwBlock;
            if (v < nvec) z[u] += __builtin_nontemporal_load(Zp + v);
        }
    }
#pragma unroll
    for (int u = 0; u < kEwVecs; ++u) {
        const int64_t v = base + u * kEwBlock;
        if (v >= nvec) continue;
        f32x4 x = z[u];
        if (b) {
            x += bias4_at<T>(b, col);
            col += step;
            if (col >= Fs) col -= Fs;
        }
        if (Zout) store4_to<T>(Zout + v * 4, x);
        f32x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = act_fwd<ACT>(x[e]);
        store4_to<T>(H + v * 4, h);
    }
}

// Element path for Fs % 4 != 0.
template <class T, int ACT>
__global__ __launch_bounds__(256) void bias_act_scalar(const float* __restrict__ Z, int S,
                                                       int64_t plane, const T* __restrict__ b,
                                                       T* __restrict__ Zout, T* __restrict__ H,
                                                       int64_t n, int64_t Fs)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
        float x = Z[e];
        for (int p = 1; p < S; ++p) x += Z[p * plane + e];
        if (b) x += load1<T>(b, e % Fs);
        if (Zout) store1<T>(Zout + e, x);
        store1<T>(H + e, act_fwd<ACT>(x));
    }
}

template <class T, int ACT>
void launch_typed(const float* Z, int S, int64_t plane, const T* b, T* Zout, T* H, int64_t N,
                  int64_t Fs, hipStream_t s)
{
    const int64_t n = N * Fs;
    if (Fs % 4 == 0) {
        const int64_t nvec = n / 4, per_group = (int64_t)kEwBlock * kEwVecs;
        const int64_t max_launch = int64_t(1) << 30;
        for (int64_t g0 = 0; g0 < ceil_div(nvec, per_group); g0 += max_launch) {
            const int64_t groups = ceil_div(nvec, per_group) - g0;
            hipLaunchKernelGGL((bias_act_vec<T, ACT>),
                               dim3((uint32_t)(groups < max_launch ? groups : max_launch)),
                               dim3(kEwBlock), 0, s, Z, S, plane, b, Zout, H, nvec, Fs,
                               g0 * per_group, (int64_t)(4 * kEwBlock) % Fs);
        }
    } else {
        const int64_t groups = ceil_div(n, 256) < 4096 ? ceil_div(n, 256) : 4096;
        hipLaunchKernelGGL((bias_act_scalar<T, ACT>), dim3((uint32_t)groups), dim3(256), 0, s, Z,
                           S, plane, b, Zout, H, n, Fs);
    }
}

template <class F>
void with_dtype_act(int dtype, int act, F&& f)
{
    with_act(act, [&](auto a) {
        if (dtype == kBF16)
            f(a, uint16_t{});
        else
            f(a, float{});
    });
}

}  // namespace

void launch_bias_act(const float* Z, const void* b1r, void* H, int64_t N, int64_t Fs, int dtype,
                     int act, hipStream_t s)
{
    launch_split_bias_act(Z, 1, 0, b1r, nullptr, H, N, Fs, dtype, act, s);
}

void launch_split_bias_act(const float* planes, int S, int64_t plane, const void* b1r, void* Z,
                           void* H, int64_t N, int64_t Fs, int dtype, int act, hipStream_t s)
{
    with_dtype_act(dtype, act, [&](auto a, auto t) {
        constexpr int ACT = decltype(a)::value;
        using T = decltype(t);
        launch_typed<T, ACT>(planes, S, plane, static_cast<const T*>(b1r), static_cast<T*>(Z),
                             static_cast<T*>(H), N, Fs, s);
    });
}

}  // namespace mlptp
