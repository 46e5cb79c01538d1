// dispatch.hpp -- host helpers that size grids and launch the GEMM templates.
#pragma once

#include "epilogue.hpp"
#include "gemm_mfma.hpp"
#include "gemm_simt.hpp"

namespace mlptp {

// Tile for every bf16 product: 128 x 128 per workgroup, 4 waves of 64 x 64.
using DefaultTile = MfmaTile<128, 128, 2, 2>;

template <class Cfg, bool A_KC, bool B_KC, class Epi>
inline void run_mfma(const void* A, const void* B, int64_t M, int64_t N, int64_t K, int64_t lda,
                     int64_t ldb, Epi epi, hipStream_t s)
{
    const int64_t tiles = ceil_div(M, Cfg::BM) * ceil_div(N, Cfg::BN);
    const int vecA = (lda % 8 == 0), vecB = (ldb % 8 == 0);
    hipLaunchKernelGGL((gemm_bf16_mfma<Cfg, A_KC, B_KC, Epi>), dim3((uint32_t)tiles),
                       dim3(Cfg::NTHREADS), 0, s, static_cast<const uint16_t*>(A),
                       static_cast<const uint16_t*>(B), M, N, K, lda, ldb, vecA, vecB, epi);
}

template <bool A_KC, bool B_KC, class Epi>
inline void run_simt(const void* A, const void* B, int64_t M, int64_t N, int64_t K, int64_t lda,
                     int64_t ldb, Epi epi, hipStream_t s)
{
    const int64_t tiles = ceil_div(M, 64) * ceil_div(N, 64);
    hipLaunchKernelGGL((gemm_f32_simt<A_KC, B_KC, Epi>), dim3((uint32_t)tiles), dim3(256), 0, s,
                       static_cast<const float*>(A), static_cast<const float*>(B), M, N, K, lda,
                       ldb, epi);
}

}  // namespace mlptp
