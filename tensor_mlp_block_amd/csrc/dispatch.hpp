// dispatch.hpp -- host helpers that size grids and launch the GEMM templates.
#pragma once

#include "epilogue.hpp"
#include "gemm_dma.hpp"
#include "gemm_mfma.hpp"
#include "gemm_simt.hpp"

namespace mlptp {

// Fallback tile for bf16 products the direct-to-LDS kernel cannot take: 128 x 128 per
// workgroup, 4 waves of 64 x 64.
using DefaultTile = MfmaTile<128, 128, 2, 2>;

// Main bf16 tiles: 8 waves per workgroup (two per SIMD). 256 x 256 (waves of 64 x 128) by
// default; 256 x 224 (64 x 112) and 224 x 256 (112 x 64) when an extent is a multiple of 224 and
// that tile count fills the GPU's compute units better (e.g. F/T = 3584 = 16 x 224: 256 tiles
// instead of 224 on 256 CUs); 256 x 192 likewise for multiples of 192.
using DmaTile256x256 = DmaTile<256, 256, 4, 2>;
using DmaTile256x224 = DmaTile<256, 224, 4, 2>;
using DmaTile224x256 = DmaTile<224, 256, 2, 4>;
using DmaTile256x192 = DmaTile<256, 192, 4, 2>;
// For products with too few 256-wide tiles to fill the GPU: 128 x 128, 4 waves of 64 x 64, two
// workgroups per CU.
using DmaTile128x128 = DmaTile<128, 128, 2, 2>;

int compute_units();  // of the current device, queried once

// Tiles of the bf16 GEMMs, as the chooser names them.
enum TileKind : int {
    kTile256x256 = 0,
    kTile256x224 = 1,
    kTile224x256 = 2,
    kTile256x192 = 3,
    kTile128x128 = 4,
    kTileRegStaged = 5,  // register-staged fallback, 128 x 128 (shapes the direct kernel rejects)
};

// Estimated time of a tile shape: rounds of workgroups over the CU slots, times the tile area
// over the tile's throughput relative to one 8-wave 256-class tile per CU. Measured (bf16, the
// Llama-shape and GPT-2-medium-shape projections): a 128 x 128 workgroup runs at about 0.42 of a
// 256-class one when two share a CU, so the small tile wins when it fills the GPU in one round
// and the large tiles do not (a GPT-2-medium shard's down-projection: 553 instead of 350
// TFLOP/s; a 256-token batch: 161 instead of 108) and loses otherwise (the Llama shard: 950
// instead of 1210).
inline int64_t tile_cost(int64_t M, int64_t N, int bm, int bn, int64_t cus, int per_cu = 1,
                         int rate_pct = 100)
{
    const int64_t tiles = ceil_div(M, bm) * ceil_div(N, bn);
    return ceil_div(tiles, cus * per_cu) * bm * bn * 100 / rate_pct;
}

// The direct-to-LDS kernel loads whole 16-byte chunks and addresses a tile with 32-bit byte
// offsets: every leading dimension and K must be multiples of 8 elements, the contiguous extent
// of an m/n-contiguous operand too, and one tile's offsets must stay below 2 GiB.
inline bool dma_eligible(bool a_kc, bool b_kc, int64_t M, int64_t N, int64_t K, int64_t lda,
                         int64_t ldb)
{
    if (lda % 8 || ldb % 8 || K % 8) return false;
    if (!a_kc && M % 8) return false;
    if (!b_kc && N % 8) return false;
    const int64_t limit = int64_t(1) << 31;
    const int64_t span_a = a_kc ? 256 * lda * 2 : 64 * lda * 2;
    const int64_t span_b = b_kc ? 256 * ldb * 2 : 64 * ldb * 2;
    return span_a < limit && span_b < limit;
}

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

// N counts output columns; a dual epilogue takes two B operands (B2 non-null) whose tiles
// share the workgroup's B region, so each tile covers BN / 2 output columns.
template <class Cfg, bool A_KC, bool B_KC, class Epi>
inline void run_dma(const void* A, const void* B, int64_t M, int64_t N, int64_t K, int64_t lda,
                    int64_t ldb, Epi epi, hipStream_t s, const void* B2 = nullptr)
{
    constexpr int BNO = EpiIsDual<Epi>::value ? Cfg::BN / 2 : Cfg::BN;
    const int64_t tiles = ceil_div(M, Cfg::BM) * ceil_div(N, BNO);
    hipLaunchKernelGGL((gemm_bf16_dma<Cfg, A_KC, B_KC, Epi>), dim3((uint32_t)tiles),
                       dim3(Cfg::NTHREADS), 0, s, static_cast<const uint16_t*>(A),
                       static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(B2), M, N,
                       K, lda, ldb, epi);
}

// The tile a bf16 product of M x N outputs (contraction K, leading dimensions lda, ldb) runs
// on over `cus` compute units: the register-staged kernel when the direct-to-LDS kernel cannot
// take the shape, else the candidate of lowest cost, in order of preference (larger tiles
// first, the first of the lowest cost wins); the narrower 256-class tiles only where they
// divide the extent exactly. A pure function of its arguments (no HIP call).
inline TileKind choose_tile(bool a_kc, bool b_kc, int64_t M, int64_t N, int64_t K, int64_t lda,
                            int64_t ldb, int64_t cus)
{
    if (!dma_eligible(a_kc, b_kc, M, N, K, lda, ldb)) return kTileRegStaged;
    constexpr int kCands = 5;
    const int64_t cost[kCands] = {tile_cost(M, N, 256, 256, cus),
                                  (N % 224 == 0) ? tile_cost(M, N, 256, 224, cus) : INT64_MAX,
                                  (M % 224 == 0) ? tile_cost(M, N, 224, 256, cus) : INT64_MAX,
                                  (N % 192 == 0) ? tile_cost(M, N, 256, 192, cus) : INT64_MAX,
                                  tile_cost(M, N, 128, 128, cus, 2, 42)};
    int best = 0;
    for (int c = 1; c < kCands; ++c)
        if (cost[c] < cost[best]) best = c;
    return static_cast<TileKind>(best);
}

// Every bf16 product goes through here: the tile choose_tile picks for the current device.
template <bool A_KC, bool B_KC, class Epi>
inline void run_bf16(const void* A, const void* B, int64_t M, int64_t N, int64_t K, int64_t lda,
                     int64_t ldb, Epi epi, hipStream_t s)
{
    switch (choose_tile(A_KC, B_KC, M, N, K, lda, ldb, compute_units())) {
    case kTile256x224: run_dma<DmaTile256x224, A_KC, B_KC>(A, B, M, N, K, lda, ldb, epi, s); break;
    case kTile224x256: run_dma<DmaTile224x256, A_KC, B_KC>(A, B, M, N, K, lda, ldb, epi, s); break;
    case kTile256x192: run_dma<DmaTile256x192, A_KC, B_KC>(A, B, M, N, K, lda, ldb, epi, s); break;
    case kTile128x128: run_dma<DmaTile128x128, A_KC, B_KC>(A, B, M, N, K, lda, ldb, epi, s); break;
    case kTileRegStaged: run_mfma<DefaultTile, A_KC, B_KC>(A, B, M, N, K, lda, ldb, epi, s); break;
    default: run_dma<DmaTile256x256, A_KC, B_KC>(A, B, M, N, K, lda, ldb, epi, s); break;
    }
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
