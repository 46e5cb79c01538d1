// gemm_mfma.hpp -- bf16 MFMA GEMM core for gfx950 (CDNA4), fp32 accumulation.
//
// Computes C[M, N] = sum_k A(m, k) B(k, n) and hands each fp32 result to an epilogue functor.
// Used for every dense contraction of the MLP shard: the column-parallel up-projection, the
// row-parallel down-projection and the four backward products.
//
// Operand layouts (template flags):
//   A_KC: A(m, k) at A[m * lda + k]  (k contiguous)   else at A[k * lda + m]  (m contiguous)
//   B_KC: B(k, n) at B[n * ldb + k]  (k contiguous)   else at B[k * ldb + n]  (n contiguous)
//
// Design (written for 64-wide wavefronts and the 16x16x32 bf16 MFMA):
//   * A block tile is BM x BN, with BK = 64 along k per stage; the waves tile it WAVES_M x
//     WAVES_N, and each wave owns a (BM/WAVES_M) x (BN/WAVES_N) slab of 16x16 MFMA tiles.
//   * Both operands live in LDS k-contiguous ([row][BK], rows = m for A and n for B), so
//     every MFMA operand is one 16-byte ds_read_b128 per lane. The 16-byte chunks of a row
//     are XOR-swizzled with bits of the row index to spread a fragment read (16 rows, same
//     chunk) and a tile write over distinct banks.
//   * Global -> LDS goes through registers with 16-byte loads. A k-contiguous operand is
//     copied as is; an m/n-contiguous operand (the row-major weights W1^(r) [D, Fs] and
//     W2^(r) [Fs, D], and both operands of the weight gradients) is loaded as 8x8 blocks
//     and transposed in registers with v_perm_b32 before the LDS write.
//   * Two LDS stages: the global loads of stage k+1 are issued before the MFMAs of stage k
//     and written to the other buffer after them; one barrier per stage.
//   * The MFMA is issued with its operands swapped (B fragment first), so it produces the
//     transposed tile: each lane then holds 4 consecutive columns of one row, which the
//     epilogue writes with one vector store.
//   * Tiles are mapped XCD-aware: the hardware deals consecutive workgroups round-robin
//     over the 8 XCDs, so the block index is remapped to give each XCD a contiguous range of
//     tiles, ordered in groups of GROUP_M row-tiles so that concurrent tiles on one XCD share
//     A row-panels and B column-panels in that XCD's L2.
//   * Ragged M, N and K are handled by zero-filled masked loads and masked stores; a leading
//     dimension that is not a multiple of 8 elements falls back to element loads.
#pragma once

#include "common.hpp"
#include "lds_dma.hpp"

namespace mlptp {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int GROUP_M_ = 4>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = 64;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NTHREADS = WAVES_M * WAVES_N * 64;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static constexpr int KCH = BK / 8;   // 16-byte chunks per LDS row
    static constexpr int KSUB = BK / 32; // MFMA k-steps per stage
    static constexpr int GROUP_M = GROUP_M_;
    static constexpr int STAGE_ELEMS = (BM + BN) * BK;
    static constexpr int LDS_BYTES = 2 * STAGE_ELEMS * 2;
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(BM % 8 == 0 && BN % 8 == 0, "tile must be a multiple of 8");
};

// Physical 16-byte chunk of logical chunk c in LDS row `row` (see header comment).
__device__ __forceinline__ int lds_swizzle(int row, int c)
{
    return c ^ (((row >> 1) & 7) ^ ((row & 1) << 2));
}

// Loads 8 consecutive bf16 starting at src, keeping only the first `nvalid` (zeros after).
__device__ __forceinline__ uint4 load8_masked(const uint16_t* src, int64_t nvalid)
{
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (e < nvalid) w[e >> 1] |= (uint32_t)src[e] << ((e & 1) * 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// 8x8 transpose of bf16: in[j] holds row j (8 elements); out[i] receives column i.
__device__ __forceinline__ void transpose8x8(const uint4* in, uint4* out)
{
    const uint32_t* w = reinterpret_cast<const uint32_t*>(in);  // w[j*4 + q]
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        const int q = i >> 1;
        uint32_t d0 = __builtin_amdgcn_perm(w[1 * 4 + q], w[0 * 4 + q], sel);
        uint32_t d1 = __builtin_amdgcn_perm(w[3 * 4 + q], w[2 * 4 + q], sel);
        uint32_t d2 = __builtin_amdgcn_perm(w[5 * 4 + q], w[4 * 4 + q], sel);
        uint32_t d3 = __builtin_amdgcn_perm(w[7 * 4 + q], w[6 * 4 + q], sel);
        out[i] = make_uint4(d0, d1, d2, d3);
    }
}

// Global -> register -> LDS loader of one operand tile: ROWS rows (m or n) by BK along k.
template <int ROWS, int BK, int NT, bool KC>
struct TileLoader {
    static constexpr int KCH = BK / 8;
    // KC: one unit is a 16-byte chunk (row, k-chunk). Otherwise: an 8x8 block (8 rows, 8 k).
    static constexpr int TOTAL = KC ? ROWS * KCH : (ROWS / 8) * KCH;
    static constexpr int PER = (TOTAL + NT - 1) / NT;
    static constexpr int REGS = KC ? PER : PER * 8;
    uint4 r[REGS];

    __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t ld,
                                         int64_t row0, int64_t rows_lim, int64_t k0, int64_t K,
                                         bool vec, int tid)
    {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int id = p * NT + tid;
            if (TOTAL % NT != 0 && id >= TOTAL) continue;
            if (KC) {
                const int row = id / KCH, c = id % KCH;
                const int64_t grow = row0 + row, gk = k0 + c * 8;
                const uint16_t* src = base + grow * ld + gk;
                if (vec && grow < rows_lim && gk + 8 <= K)
                    r[p] = *reinterpret_cast<const uint4*>(src);
                else
                    r[p] = load8_masked(src, grow < rows_lim ? K - gk : 0);
            } else {
                const int kb = id % KCH, rb = id / KCH;
                const int64_t grow0 = row0 + rb * 8;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int64_t gk = k0 + kb * 8 + j;
                    const uint16_t* src = base + gk * ld + grow0;
                    if (vec && gk < K && grow0 + 8 <= rows_lim)
                        r[p * 8 + j] = *reinterpret_cast<const uint4*>(src);
                    else
                        r[p * 8 + j] = load8_masked(src, gk < K ? rows_lim - grow0 : 0);
                }
            }
        }
    }

    __device__ __forceinline__ void store(uint16_t* lds, int tid) const
    {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int id = p * NT + tid;
            if (TOTAL % NT != 0 && id >= TOTAL) continue;
            if (KC) {
                const int row = id / KCH, c = id % KCH;
                *reinterpret_cast<uint4*>(lds + row * BK + lds_swizzle(row, c) * 8) = r[p];
            } else {
                const int kb = id % KCH, rb = id / KCH;
                uint4 t[8];
                transpose8x8(&r[p * 8], t);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int row = rb * 8 + e;
                    *reinterpret_cast<uint4*>(lds + row * BK + lds_swizzle(row, kb) * 8) = t[e];
                }
            }
        }
    }
};

template <class Cfg, bool A_KC, bool B_KC, class Epi>
__global__ __launch_bounds__(Cfg::NTHREADS, 1) void gemm_bf16_mfma(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int64_t M, int64_t N,
    int64_t K, int64_t lda, int64_t ldb, int vecA, int vecB, Epi epi)
{
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Cfg::STAGE_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % Cfg::WAVES_M, wn = wave / Cfg::WAVES_M;

    const int64_t tiles_m = ceil_div(M, Cfg::BM), tiles_n = ceil_div(N, Cfg::BN);
    int64_t tm, tn;
    tile_coords<Cfg::GROUP_M>(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;

    TileLoader<Cfg::BM, Cfg::BK, Cfg::NTHREADS, A_KC> la;
    TileLoader<Cfg::BN, Cfg::BK, Cfg::NTHREADS, B_KC> lb;

    f32x4 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t nk = ceil_div(K, Cfg::BK);
    uint16_t* const stage0 = smem;
    uint16_t* const stage1 = smem + Cfg::STAGE_ELEMS;

    la.load(A, lda, m0, M, 0, K, vecA, tid);
    lb.load(B, ldb, n0, N, 0, K, vecB, tid);
    la.store(stage0, tid);
    lb.store(stage0 + Cfg::BM * Cfg::BK, tid);
    __syncthreads();

    const int frow = lane & 15;  // row of the fragment inside a 16-row MFMA tile
    const int fchunk = lane >> 4; // which of the 4 k-chunks of an MFMA k-step

    for (int64_t kt = 0; kt < nk; ++kt) {
        uint16_t* const cur = (kt & 1) ? stage1 : stage0;
        uint16_t* const nxt = (kt & 1) ? stage0 : stage1;
        const bool more = kt + 1 < nk;
        if (more) {
            la.load(A, lda, m0, M, (kt + 1) * Cfg::BK, K, vecA, tid);
            lb.load(B, ldb, n0, N, (kt + 1) * Cfg::BK, K, vecB, tid);
        }
        const uint16_t* As = cur;
        const uint16_t* Bs = cur + Cfg::BM * Cfg::BK;
#pragma unroll
        for (int ks = 0; ks < Cfg::KSUB; ++ks) {
            const int c = ks * 4 + fchunk;
            bf16x8 af[Cfg::FM], bfr[Cfg::FN];
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i) {
                const int row = wm * Cfg::WTM + i * 16 + frow;
                af[i] = *reinterpret_cast<const bf16x8*>(As + row * Cfg::BK +
                                                         lds_swizzle(row, c) * 8);
            }
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) {
                const int row = wn * Cfg::WTN + j * 16 + frow;
                bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + row * Cfg::BK +
                                                          lds_swizzle(row, c) * 8);
            }
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j],
                                                                        0, 0, 0);
        }
        if (more) {
            la.store(nxt, tid);
            lb.store(nxt + Cfg::BM * Cfg::BK, tid);
        }
        __syncthreads();
    }

    // acc[i][j][q] is C[row, col + q] with the row/col below (the swapped-operand layout).
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
        const int64_t row = m0 + wm * Cfg::WTM + i * 16 + frow;
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) {
            const int64_t col = n0 + wn * Cfg::WTN + j * 16 + 4 * fchunk;
            epi(row, col, acc[i][j], M, N);
        }
    }
}

}  // namespace mlptp
