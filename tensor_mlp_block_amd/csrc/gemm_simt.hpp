// gemm_simt.hpp -- fp32 GEMM on the vector ALUs, for the fp32 storage type.
//
// The fp32 path exists for exact results on integer-valued data: every product and partial
// sum is an integer below 2^24, so fp32 FMA in any order reproduces the exact value. On
// MI355X fp32 matrix throughput equals the vector fp32 rate, so MFMA would buy nothing here.
//
// 64x64 block tile, 256 threads, 4x4 outputs per thread, BK = 16 staged through LDS. Layout
// flags as in gemm_mfma.hpp. All loads are bounds-checked element loads.
#pragma once

#include "common.hpp"

namespace mlptp {

template <bool A_KC, bool B_KC, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_simt(const float* __restrict__ A,
                                                     const float* __restrict__ B, int64_t M,
                                                     int64_t N, int64_t K, int64_t lda,
                                                     int64_t ldb, Epi epi)
{
    constexpr int BM = 64, BN = 64, BK = 16;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];

    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    const int64_t tiles_n = ceil_div(N, BN);
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM;
    const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * BN;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int64_t k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int id = p * 256 + tid;
            int m, k;
            if (A_KC) { m = id / BK; k = id % BK; } else { k = id / BM; m = id % BM; }
            const int64_t gm = m0 + m, gk = k0 + k;
            float a = 0.f;
            if (gm < M && gk < K) a = A_KC ? A[gm * lda + gk] : A[gk * lda + gm];
            As[k][m] = a;
            int n, kb;
            if (B_KC) { n = id / BK; kb = id % BK; } else { kb = id / BN; n = id % BN; }
            const int64_t gn = n0 + n, gkb = k0 + kb;
            float b = 0.f;
            if (gn < N && gkb < K) b = B_KC ? B[gn * ldb + gkb] : B[gkb * ldb + gn];
            Bs[kb][n] = b;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x4 v = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
        epi(m0 + ty * 4 + i, n0 + tx * 4, v, M, N);
    }
}

}  // namespace mlptp
