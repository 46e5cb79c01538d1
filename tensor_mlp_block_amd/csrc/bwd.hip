// bwd.hip -- backward shard kernels.
//
// Pages cited, as [tag section]:
//   [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
//   [U] unpurerationalist.github.io, "LLM Systems 16: Model Parallel Training"
//   [C] charliedreemur.github.io, "TP:Column / Row Parallel Linear 怎么切? MLP 和 attention 怎么切?"
#include "dispatch.hpp"
#include "launch.hpp"

#include <mutex>

namespace mlptp {

// Device buffer of the allocation-free backward: the db1 column sum's workspace, for callers
// that cannot allocate (HIP graph capture, serving loops). One copy per GPU, resident until
// the process ends. In host code `scratch` names a host-side stand-in, not a device address:
// kernels and copies get the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

int noalloc_scratch(void** ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        // The device is current here, so this is that GPU's copy of the array.
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return -1;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return 0;
}

// dH = dY W2^(r)^T (no exchange in the row-parallel backward), then dZ = dH * phi'(Z)
// [Z 06], [U 3.6.1]. GEMM view: M = N tokens, N = Fs, K = D; A = dY (k-contiguous),
// B(k = d, n = j) = W2r[j, d] (k-contiguous).
void launch_bwd_dz(const void* dY, const void* W2r, const void* Z, void* dZ, int64_t N, int64_t D,
                   int64_t Fs, int dtype, int act, hipStream_t s)
{
    const int vec = (Fs % 4 == 0);
    with_act(act, [&](auto a) {
        constexpr int ACT = decltype(a)::value;
        if (dtype == kBF16) {
            EpiActGrad<uint16_t, ACT> epi{static_cast<const uint16_t*>(Z),
                                          static_cast<uint16_t*>(dZ), Fs, vec};
            run_bf16<true, true>(dY, W2r, N, Fs, D, D, D, epi, s);
        } else {
            EpiActGrad<float, ACT> epi{static_cast<const float*>(Z), static_cast<float*>(dZ), Fs,
                                       vec};
            run_simt<true, true>(dY, W2r, N, Fs, D, D, D, epi, s);
        }
    });
}

// Gated form [Z 08]: the same dH = dY W2^(r)^T product, with the product rule through
// H = SiLU(G) * U in its epilogue, so dG and dU each take one HBM write and G, U one read.
void launch_swiglu_bwd_dgu(const void* dY, const void* W2r, const void* G, const void* U, void* dG,
                           void* dU, int64_t N, int64_t D, int64_t Fs, int dtype, hipStream_t s)
{
    const int vec = (Fs % 4 == 0);
    if (dtype == kBF16) {
        EpiSwiGLUGrad<uint16_t> epi{static_cast<const uint16_t*>(G),
                                    static_cast<const uint16_t*>(U), static_cast<uint16_t*>(dG),
                                    static_cast<uint16_t*>(dU), Fs, vec};
        run_bf16<true, true>(dY, W2r, N, Fs, D, D, D, epi, s);
    } else {
        EpiSwiGLUGrad<float> epi{static_cast<const float*>(G), static_cast<const float*>(U),
                                 static_cast<float*>(dG), static_cast<float*>(dU), Fs, vec};
        run_simt<true, true>(dY, W2r, N, Fs, D, D, D, epi, s);
    }
}

// Local weight gradients [Z 06], [U 3.6.1]: C = A^T B, both operands stored token-major
// ([K, M] and [K, N]), so both are transposed into LDS.
void launch_wgrad(const void* A, const void* B, float* C, int64_t M, int64_t N, int64_t K,
                  int64_t lda, int64_t ldb, int dtype, hipStream_t s)
{
    EpiStoreF32 epi{C, N, (int)(N % 4 == 0)};
    if (dtype == kBF16)
        run_bf16<false, false>(A, B, M, N, K, lda, ldb, epi, s);
    else
        run_simt<false, false>(A, B, M, N, K, lda, ldb, epi, s);
}

// dX^(r) = dZ W1^(r)^T, this rank's partial of the input gradient [Z 06 equation],
// [C 推导 / 关键公式]. GEMM view: M = N tokens, N = D, K = Fs; A = dZ (k-contiguous),
// B(k = j, n = d) = W1r[d, j] (k-contiguous).
void launch_dx(const void* dZ, const void* W1r, float* dX, int64_t N, int64_t D, int64_t Fs,
               int dtype, hipStream_t s)
{
    EpiStoreF32 epi{dX, D, (int)(D % 4 == 0)};
    if (dtype == kBF16)
        run_bf16<true, true>(dZ, W1r, N, D, Fs, Fs, Fs, epi, s);
    else
        run_simt<true, true>(dZ, W1r, N, D, Fs, Fs, Fs, epi, s);
}

// dX^(r) += dZ W1^(r)^T: the gated form's second input-gradient term, dU Wu^(r)^T added to
// dG Wg^(r)^T [Z 08].
void launch_dx_accumulate(const void* dZ, const void* W1r, float* dX, int64_t N, int64_t D,
                          int64_t Fs, int dtype, hipStream_t s)
{
    EpiAccumF32 epi{dX, D, (int)(D % 4 == 0)};
    if (dtype == kBF16)
        run_bf16<true, true>(dZ, W1r, N, D, Fs, Fs, Fs, epi, s);
    else
        run_simt<true, true>(dZ, W1r, N, D, Fs, Fs, Fs, epi, s);
}

// db1^(r)[j] = sum over tokens of dZ[n, j]. Pass 1: each workgroup sums a slab of kColsumRows
// tokens of one column block into ws[slab, :]; pass 2 adds the slabs in a fixed order. No atomics,
// so the result is the same on every run.
constexpr int kColsumRows = 64;

template <class T>
__device__ __forceinline__ float as_f32(T v);
template <>
__device__ __forceinline__ float as_f32<uint16_t>(uint16_t v) { return bf16_bits_to_f32(v); }
template <>
__device__ __forceinline__ float as_f32<float>(float v) { return v; }

// Element e of a 16-byte vector of T.
template <class T>
__device__ __forceinline__ float vec_elem(const uint4& v, int e);
template <>
__device__ __forceinline__ float vec_elem<uint16_t>(const uint4& v, int e)
{
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return bf16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFFu));
}
template <>
__device__ __forceinline__ float vec_elem<float>(const uint4& v, int e)
{
    const uint32_t w = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
    return __uint_as_float(w);
}

// Vector form, for rows that are whole 16-byte vectors (Fs a multiple of 16 / sizeof(T); the base
// pointer is 16-byte aligned). 32 threads span a row of the column block (one vector each) and the
// 8 groups of 32 take tokens r0 + g, r0 + g + 8, ...: every load instruction of a wave reads two
// contiguous row runs, and all of a thread's loads are issued before its first add. The 8 group
// sums of a column are then added in group order through LDS.
template <class T>
__global__ __launch_bounds__(256) void colsum_slabs_vec(const T* __restrict__ dZ,
                                                        float* __restrict__ ws, int64_t N,
                                                        int64_t Fs)
{
    constexpr int VEC = 16 / (int)sizeof(T);
    constexpr int COLS = 32 * VEC;
    constexpr int PER = kColsumRows / 8;
    __shared__ float part[8][COLS];
    const int tx = threadIdx.x & 31, g = threadIdx.x >> 5;
    const int64_t c0 = (int64_t)blockIdx.x * COLS + tx * VEC;
    const int64_t r0 = (int64_t)blockIdx.y * kColsumRows + g;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    if (c0 < Fs) {
        uint4 v[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int64_t r = r0 + 8 * i;
            v[i] = r < N ? *reinterpret_cast<const uint4*>(dZ + r * Fs + c0) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < PER; ++i)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] += vec_elem<T>(v[i], e);
    }
    // Column tx * VEC + e sits at part[g][e * 32 + tx], so the 32 lanes of a store hit 32 banks.
#pragma unroll
    for (int e = 0; e < VEC; ++e) part[g][e * 32 + tx] = acc[e];
    __syncthreads();
    const int t = threadIdx.x;
    const int64_t col = (int64_t)blockIdx.x * COLS + t;
    if (t < COLS && col < Fs) {
        const int idx = (t % VEC) * 32 + t / VEC;
        float sum = part[0][idx];
#pragma unroll
        for (int j = 1; j < 8; ++j) sum += part[j][idx];
        ws[(int64_t)blockIdx.y * Fs + col] = sum;
    }
}

// Element form, for any Fs: one column per thread, tokens in order.
template <class T>
__global__ __launch_bounds__(256) void colsum_slabs(const T* __restrict__ dZ, float* __restrict__ ws,
                                                    int64_t N, int64_t Fs)
{
    const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (col >= Fs) return;
    const int64_t r0 = (int64_t)blockIdx.y * kColsumRows;
    const int64_t r1 = (r0 + kColsumRows < N) ? r0 + kColsumRows : N;
    float acc = 0.f;
    for (int64_t r = r0; r < r1; ++r) acc += as_f32<T>(dZ[r * Fs + col]);
    ws[(int64_t)blockIdx.y * Fs + col] = acc;
}

// Pass 2: 64 columns per workgroup; the 4 groups of 64 threads add slabs q, q + 4, q + 8, ... and
// their 4 sums are added in group order.
__global__ __launch_bounds__(256) void colsum_finish(const float* __restrict__ ws,
                                                     float* __restrict__ out, int64_t slabs,
                                                     int64_t Fs)
{
    __shared__ float part[4][64];
    const int tx = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int64_t col = (int64_t)blockIdx.x * 64 + tx;
    float acc = 0.f;
    if (col < Fs) {
#pragma unroll 8
        for (int64_t b = q; b < slabs; b += 4) acc += ws[b * Fs + col];
    }
    part[q][tx] = acc;
    __syncthreads();
    if (q == 0 && col < Fs) out[col] = ((part[0][tx] + part[1][tx]) + part[2][tx]) + part[3][tx];
}

int64_t colsum_workspace_bytes(int64_t N, int64_t Fs)
{
    return ceil_div(N, kColsumRows) * Fs * (int64_t)sizeof(float);
}

void launch_colsum(const void* dZ, float* ws, float* db1, int64_t N, int64_t Fs, int dtype,
                   hipStream_t s)
{
    const int64_t slabs = ceil_div(N, kColsumRows);
    const int64_t es = dtype == kBF16 ? 2 : 4;
    const int64_t vec = 16 / es;
    if (slabs == 0) {
        // no tokens: the finishing pass writes zeros
    } else if (Fs % vec == 0) {
        const dim3 grid((uint32_t)ceil_div(Fs, 32 * vec), (uint32_t)slabs);
        if (dtype == kBF16)
            hipLaunchKernelGGL(colsum_slabs_vec<uint16_t>, grid, dim3(256), 0, s,
                               static_cast<const uint16_t*>(dZ), ws, N, Fs);
        else
            hipLaunchKernelGGL(colsum_slabs_vec<float>, grid, dim3(256), 0, s,
                               static_cast<const float*>(dZ), ws, N, Fs);
    } else {
        const dim3 grid((uint32_t)ceil_div(Fs, 256), (uint32_t)slabs);
        if (dtype == kBF16)
            hipLaunchKernelGGL(colsum_slabs<uint16_t>, grid, dim3(256), 0, s,
                               static_cast<const uint16_t*>(dZ), ws, N, Fs);
        else
            hipLaunchKernelGGL(colsum_slabs<float>, grid, dim3(256), 0, s,
                               static_cast<const float*>(dZ), ws, N, Fs);
    }
    hipLaunchKernelGGL(colsum_finish, dim3((uint32_t)ceil_div(Fs, 64)), dim3(256), 0, s, ws, db1,
                       slabs, Fs);
}

}  // namespace mlptp
