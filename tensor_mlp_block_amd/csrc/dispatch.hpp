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
// `splits` > 1 cuts the contraction into ranges of kc (a multiple of 64), one grid row each.
template <class Cfg, bool A_KC, bool B_KC, class Epi>
inline void run_dma(const void* A, const void* B, int64_t M, int64_t N, int64_t K, int64_t lda,
                    int64_t ldb, Epi epi, hipStream_t s, const void* B2 = nullptr,
                    int splits = 1, int64_t kc = 0)
{
    constexpr int BNO = EpiIsDual<Epi>::value ? Cfg::BN / 2 : Cfg::BN;
    const int64_t tiles = ceil_div(M, Cfg::BM) * ceil_div(N, BNO);
    hipLaunchKernelGGL((gemm_bf16_dma<Cfg, A_KC, B_KC, Epi>), dim3((uint32_t)tiles, splits),
                       dim3(Cfg::NTHREADS), 0, s, static_cast<const uint16_t*>(A),
                       static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(B2), M, N,
                       K, lda, ldb, epi, splits > 1 ? kc : K);
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

// A split of the contraction for products with fewer 128 x 128 tiles than compute units: each
// split's workgroups write an fp32 partial plane of the whole [M, N] product into a caller-owned
// workspace, and a second, streaming pass sums the planes in split order and applies the
// product's epilogue. Deterministic (no atomics); only the order of the fp32 additions differs
// from the unsplit product. S = min(8, 2 CUs / tiles, K / 1024): at most two workgroups per CU,
// and each split at least 1024 deep (sixteen 64-deep stages), so the extra launch and the planes'
// traffic stay small beside the GEMM. Measured (one MI355X, GEMM plus the sum of the planes, us):
// the pages' example shape's products (256 tokens) 57 -> 46 (up, T = 1, S = 2), 134 -> 42
// (down, T = 1, S = 8), 53 -> 33 (up, T = 2, S = 4), 53 -> 24 (up, T = 8, S = 4); a 1024-token
// Llama-width up-projection (224 tiles) 101 -> 72 (S = 2). Products with as many tiles as CUs
// lost (GPT-2-medium's down-projection, 256 tiles: 29 -> 32 at S = 2), and so did splits below
// 1024 (T = 8 down-projection, K = 1376: 17.1 -> 18.4 at S = 2).
struct SplitPlan {
    int splits;
    int64_t kc;  // contraction length per split (a multiple of 64)
};

inline SplitPlan split_plan(bool a_kc, bool b_kc, int64_t M, int64_t N, int64_t K, int64_t lda,
                            int64_t ldb, int64_t cus)
{
    const SplitPlan none{1, K};
    if (choose_tile(a_kc, b_kc, M, N, K, lda, ldb, cus) != kTile128x128) return none;
    const int64_t tiles = ceil_div(M, 128) * ceil_div(N, 128);
    if (tiles >= cus) return none;
    int64_t S = 2 * cus / tiles;
    if (S > 8) S = 8;
    if (S > K / 1024) S = K / 1024;
    if (S < 2) return none;
    const int64_t kc = ceil_div(ceil_div(K, S), 64) * 64;
    return SplitPlan{(int)ceil_div(K, kc), kc};
}

// Workspace bytes of a split product: one fp32 [M, N] plane per split.
inline int64_t split_workspace_bytes(const SplitPlan& p, int64_t M, int64_t N)
{
    return p.splits > 1 ? (int64_t)p.splits * M * N * 4 : 0;
}

// The split GEMM: fp32 planes ws[s][M, N] on the 128 x 128 tile.
template <bool A_KC, bool B_KC>
inline void run_split(const void* A, const void* B, int64_t M, int64_t N, int64_t K, int64_t lda,
                      int64_t ldb, const SplitPlan& p, float* ws, hipStream_t s)
{
    EpiSplitF32 epi{ws, M * N, N, (int)(N % 4 == 0)};
    run_dma<DmaTile128x128, A_KC, B_KC>(A, B, M, N, K, lda, ldb, epi, s, nullptr, p.splits, p.kc);
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
