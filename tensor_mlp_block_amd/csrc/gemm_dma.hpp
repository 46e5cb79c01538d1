// gemm_dma.hpp -- bf16 MFMA GEMM for gfx950 with direct global->LDS loads and LDS transpose
// reads, fp32 accumulation.
//
// Same contract as gemm_mfma.hpp (C[M, N] = sum_k A(m, k) B(k, n), layouts A_KC / B_KC,
// results handed to an epilogue functor), for the common case where every leading dimension,
// K, and the m/n extent of an m/n-contiguous operand are multiples of 8.
//
// How the operands reach the matrix cores:
//   * Global -> LDS with `buffer_load_dwordx4 ... lds` (lds_dma.hpp): 1 KB per wave
//     instruction, no register round trip, zeros for out-of-range lanes.
//   * A k-contiguous operand is stored [rows][64 k] (128 bytes per row); an m/n-contiguous one
//     keeps its global orientation, [64 k][rows]. In both, 16-byte chunks are XOR-swizzled with
//     bits of the row (k) index; the swizzle is applied on the global side by choosing which
//     chunk each lane fetches, since the LDS side of the load is fixed by the lane number.
//   * MFMA operands (16 rows x 32 k, 8 k-values per lane) are read with one ds_read_b128 from a
//     k-contiguous tile, or with two ds_read_b64_tr_b16 from a [k][rows] tile: in each 16-lane
//     group the transpose read returns lane i the i-th element of the four 16-element rows the
//     group's lanes address, i.e. 4 consecutive k of one output row.
//   * Two LDS stages: the loads of stage k+1 are issued while the MFMAs of stage k run; a vmcnt
//     wait and one barrier end each stage. Within a stage the loads and the LDS reads are
//     interleaved with the MFMAs, the B reads two fragments ahead of their use and the second
//     k-substep's A reads spread over the first substep (dma_step).
#pragma once

#include "lds_dma.hpp"

namespace mlptp {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int GROUP_M_ = 4>
struct DmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = 64;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NWAVES = WAVES_M * WAVES_N;
    static constexpr int NTHREADS = NWAVES * 64;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static constexpr int KSUB = BK / 32;
    static constexpr int GROUP_M = GROUP_M_;
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    // Waves per SIMD the kernel must leave room for: a 4-wave tile asks for 2, so that two
    // workgroups (and their two LDS double buffers) can share a CU.
    static constexpr int MIN_WAVES_PER_SIMD = NWAVES >= 8 ? 1 : 2;
    // Who issues a stage's global->LDS loads, and when. On the 256 x 224 and 256 x 192 tiles,
    // waves 0-3 (one per SIMD) issue all of them at the start of the stage while their SIMD
    // partners, waves 4-7, keep the matrix cores busy: +4% and up to +2% against every wave
    // issuing its share spread over the stage, which the 256 x 256 tile keeps (-2% otherwise).
    static constexpr bool LOADERS_UP_FRONT = NWAVES == 8 && BM == 256 && BN < 256;
    static constexpr int NLOAD = LOADERS_UP_FRONT ? 4 : NWAVES;  // waves that issue loads
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "tiles move in 1 KB wave loads");
    static_assert(2 * STAGE_BYTES <= 160 * 1024, "two stages must fit in LDS");
};

// k-contiguous tile [rows][64]: chunk c (8 elements) of row r sits at physical chunk
// c ^ kc_swz(r). Spreads 16 consecutive rows of one chunk over distinct banks.
__device__ __forceinline__ int kc_swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// [64][rows] tile: 16-byte chunk c of k-row k sits at c ^ mc_swz(k). A transpose read touches
// four consecutive k rows (32 bytes each) per 16-lane group, and the next group reads the rows
// 8 below; the swizzle puts all of them on distinct banks.
//   * ROWS a power of two >= 128: rows are a multiple of 256 bytes apart, so every k row starts
//     on the same bank; XOR the chunk pair with k mod 4 and flip bit 3 with bit 3 of k.
//   * ROWS = 224: a 448-byte row pitch already spreads 4 consecutive rows over distinct banks;
//     only rows 8 apart collide, so flip chunk bit 1 with bit 3 of k (stays inside the row's
//     28 chunks, since it permutes within aligned groups of 4).
//   * ROWS = 192: a 384-byte pitch puts odd k rows half a bank period from even ones, so rows
//     2 apart collide; bit 1 of k flips chunk bit 1 and bit 3 of k chunk bit 2, which gives the
//     8 rows one half-wave reads 8 distinct bank groups and stays inside aligned groups of 8
//     of the row's 24 chunks.
template <int ROWS>
__device__ __forceinline__ int mc_swz(int k)
{
    if constexpr (ROWS == 224)
        return ((k >> 3) & 1) << 1;
    else if constexpr (ROWS == 192)
        return (((k >> 1) & 1) << 1) | (((k >> 3) & 1) << 2);
    else if constexpr (ROWS >= 128)
        return ((k & 3) << 1) | (((k >> 3) & 1) << 3);
    else
        return (k & 3) << 1;
}

// Issues load q of this wave's share of the global->LDS copy of one operand tile (ROWS x 64 k),
// shared among NLOAD waves (wave < NLOAD).
//   KC: element (row, k) at src[row * ld + k]; LDS [ROWS][64].
//   MC: element (row, k) at src[k * ld + row]; LDS [64][ROWS].
// `src` already points at (row0, k0); rows >= rows_left or k >= k_left load zeros. One buffer
// resource covers the tile; the first row (KC) or k row (MC) of each 1 KB load travels in the
// scalar offset operand, so the per-lane offset only holds the row within the load and the
// swizzled chunk. (Out-of-range lanes carry an offset of 2^31 in the vector operand, past the
// resource's range whether or not the hardware adds the scalar offset before its check.)
template <int ROWS, int NLOAD, bool KC>
__device__ __forceinline__ void dma_load_one(const uint16_t* src, int64_t ld, int rows_left,
                                             int k_left, MLPTP_LDS uint8_t* lds, int wave, int lane,
                                             int q)
{
    constexpr int kInstr = ROWS * 64 * 2 / 1024;  // 1 KB wave loads per tile
    const int qi = q * NLOAD + wave;
    if (kInstr % NLOAD != 0 && qi >= kInstr) return;  // wave-uniform
    const i32x4 rsrc = make_buffer_rsrc(src);
    int off;
    int first;  // first row (KC) or k row (MC) of this load
    if (KC) {
        first = qi * 8;
        const int rl = lane >> 3;
        const int c = (lane & 7) ^ kc_swz(first + rl);
        const bool ok = rl < rows_left - first && c * 8 < k_left;
        off = ok ? (int)(rl * ld * 2 + c * 16) : kOutOfRange;
    } else {
        // Chunk index idx = 64 qi + lane lands at byte 16 idx = k * 2 ROWS + 16 p.
        constexpr int kChunks = ROWS / 8;
        first = (qi * 64) / kChunks;
        const int idx = qi * 64 + lane;
        const int k = idx / kChunks;
        const int c = (idx % kChunks) ^ mc_swz<ROWS>(k);
        const bool ok = k < k_left && c * 8 < rows_left;
        off = ok ? (int)((k - first) * ld * 2 + c * 16) : kOutOfRange;
    }
    const int soff = __builtin_amdgcn_readfirstlane((int)(first * ld * 2));
    llvm_amdgcn_raw_buffer_load_lds(rsrc, reinterpret_cast<MLPTP_LDS uint32_t*>(lds + qi * 1024), 16,
                                    off, soff, 0, 0);
}

// Loads per wave for one operand tile of ROWS x 64 k.
template <int ROWS, int NWAVES>
constexpr int dma_loads_per_wave()
{
    return (ROWS * 64 * 2 / 1024 + NWAVES - 1) / NWAVES;
}

// One MFMA operand fragment (16 rows x 32 k) for k-step ks from a KC tile.
template <int ROWS>
__device__ __forceinline__ bf16x8 frag_kc(const MLPTP_LDS uint8_t* lds, int row0, int ks, int lane)
{
    const int r = row0 + (lane & 15);
    const int c = (ks * 4 + (lane >> 4)) ^ kc_swz(r);
    return *reinterpret_cast<const MLPTP_LDS bf16x8*>(lds + r * 128 + c * 16);
}

// The same fragment from an MC tile [64][ROWS] with two transpose reads: lane (16 g + i) gets
// k = 32 ks + 8 g + {0..3} from the first read and {4..7} from the second, of row row0 + i.
template <int ROWS>
__device__ __forceinline__ bf16x8 frag_mc(const MLPTP_LDS uint8_t* lds, int row0, int ks, int lane)
{
    const int g = lane >> 4, i = lane & 15;
    const int n = row0 + 4 * (i & 3);
    s16x4 h[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int k = ks * 32 + 8 * g + 4 * t + (i >> 2);
        const int c = (n >> 3) ^ mc_swz<ROWS>(k);
        const MLPTP_LDS uint8_t* p = lds + k * (ROWS * 2) + c * 16 + (n & 7) * 2;
        h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<MLPTP_LDS s16x4*>(const_cast<MLPTP_LDS uint8_t*>(p)));
    }
    s16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf16x8, v);
}

struct DmaCtx {
    const uint16_t* A;
    const uint16_t* B;
    const uint16_t* B2;  // dual form only: the second B, loaded beside the first
    int64_t M, N, K, lda, ldb, m0, n0;
    int m_left, n_left, wave, lane;
};

// Global sources of stage kt's tiles. In the dual form the B tile is two tiles of BN/2 columns,
// the same output columns of B and of B2, side by side in LDS. k_left = K - 64 kt is not clamped
// to the stage: the loads only compare it with k indices below 64, and a kt past the last stage
// (k_left <= 0) gives an empty k range, so every lane of its loads takes the out-of-range offset
// and loads zeros.
struct StageSrc {
    const uint16_t* a;
    const uint16_t* b;
    const uint16_t* b2;
    int k_left;
};

template <class Cfg, bool A_KC, bool B_KC, bool DUAL>
__device__ __forceinline__ StageSrc stage_src(const DmaCtx& c, int64_t kt)
{
    const int64_t k0 = kt * Cfg::BK;
    StageSrc t;
    t.k_left = (int)(c.K - k0);
    t.a = A_KC ? c.A + c.m0 * c.lda + k0 : c.A + k0 * c.lda + c.m0;
    t.b = B_KC ? c.B + c.n0 * c.ldb + k0 : c.B + k0 * c.ldb + c.n0;
    t.b2 = DUAL ? (B_KC ? c.B2 + c.n0 * c.ldb + k0 : c.B2 + k0 * c.ldb + c.n0) : nullptr;
    return t;
}

// From stage kt's sources to stage kt + 1's: pointer increments instead of the products
// stage_src forms, so the step after a barrier starts with its reads, not with address work.
template <class Cfg, bool A_KC, bool B_KC, bool DUAL>
__device__ __forceinline__ void advance_src(const DmaCtx& c, StageSrc& t)
{
    t.a += A_KC ? (int64_t)Cfg::BK : Cfg::BK * c.lda;
    t.b += B_KC ? (int64_t)Cfg::BK : Cfg::BK * c.ldb;
    if constexpr (DUAL) t.b2 += B_KC ? (int64_t)Cfg::BK : Cfg::BK * c.ldb;
    t.k_left -= Cfg::BK;
}

// Loads per wave for a whole stage: the A tile's, then the B tile's (both halves in the dual form).
template <class Cfg, bool DUAL>
struct StageLoads {
    static constexpr int QA = dma_loads_per_wave<Cfg::BM, Cfg::NLOAD>();
    static constexpr int QH = dma_loads_per_wave<Cfg::BN / 2, Cfg::NLOAD>();
    static constexpr int QB = DUAL ? 2 * QH : dma_loads_per_wave<Cfg::BN, Cfg::NLOAD>();
    static constexpr int Q = QA + QB;
};

// Load q (0 <= q < StageLoads::Q) of this wave's share of a stage (waves below Cfg::NLOAD).
template <class Cfg, bool A_KC, bool B_KC, bool DUAL>
__device__ __forceinline__ void stage_load(const DmaCtx& c, const StageSrc& t,
                                           MLPTP_LDS uint8_t* base, int q)
{
    using SL = StageLoads<Cfg, DUAL>;
    if (q < SL::QA) {
        dma_load_one<Cfg::BM, Cfg::NLOAD, A_KC>(t.a, c.lda, c.m_left, t.k_left, base, c.wave,
                                                 c.lane, q);
    } else if constexpr (!DUAL) {
        dma_load_one<Cfg::BN, Cfg::NLOAD, B_KC>(t.b, c.ldb, c.n_left, t.k_left,
                                                 base + Cfg::A_BYTES, c.wave, c.lane, q - SL::QA);
    } else {
        constexpr int HB = Cfg::BN / 2;
        if (q < SL::QA + SL::QH)
            dma_load_one<HB, Cfg::NLOAD, B_KC>(t.b, c.ldb, c.n_left, t.k_left,
                                                base + Cfg::A_BYTES, c.wave, c.lane, q - SL::QA);
        else
            dma_load_one<HB, Cfg::NLOAD, B_KC>(t.b2, c.ldb, c.n_left, t.k_left,
                                                base + Cfg::A_BYTES + Cfg::B_BYTES / 2, c.wave,
                                                c.lane, q - SL::QA - SL::QH);
    }
}

// All loads of stage kt (the pipeline's first stage).
template <class Cfg, bool A_KC, bool B_KC, bool DUAL>
__device__ __forceinline__ void dma_issue(const DmaCtx& c, int64_t kt, MLPTP_LDS uint8_t* base)
{
    const StageSrc t = stage_src<Cfg, A_KC, B_KC, DUAL>(c, kt);
    if (Cfg::NLOAD < Cfg::NWAVES && c.wave >= Cfg::NLOAD) return;
#pragma unroll
    for (int q = 0; q < StageLoads<Cfg, DUAL>::Q; ++q) stage_load<Cfg, A_KC, B_KC, DUAL>(c, t, base, q);
}

// One pipeline step: the MFMAs of the stage held in `cur`, and the loads of the next stage (from
// `src`) into `nxt` (past the last stage: loads of an empty k range). `cur` and `nxt` are distinct stages; the
// __restrict__ qualifiers tell the compiler so, which lets it read `cur` while the loads into
// `nxt` are still in flight instead of waiting for them first.
//
// The order is written out, because the compiler keeps LDS reads after an LDS-writing load that
// precedes them in the source: the MFMAs go B fragment by B fragment (each meets the wave's FM A
// fragments, in alternating directions); after each group of FM MFMAs come one of the wave's
// loads of the next stage, the reads of the B fragment two places ahead and, within the first
// k-substep, some of the second substep's A fragments. Left to itself the compiler put every load and all 30-40 reads of a stage
// ahead of its first MFMA: a wave tracks at most 15 outstanding LDS reads, so that MFMA waited for
// about half of them, and both waves of every SIMD did this at the same moment after the barrier.
template <class Cfg, bool A_KC, bool B_KC, bool DUAL>
__device__ __attribute__((always_inline)) inline void dma_step(
    const DmaCtx& c, const StageSrc& src, const MLPTP_LDS uint8_t* __restrict__ cur,
    MLPTP_LDS uint8_t* __restrict__ nxt, f32x4 (&acc)[Cfg::FM][Cfg::FN], int wm, int wn)
{
    using SL = StageLoads<Cfg, DUAL>;
    const MLPTP_LDS uint8_t* As = cur;
    const MLPTP_LDS uint8_t* Bs = cur + Cfg::A_BYTES;
    constexpr int G = Cfg::KSUB * Cfg::FN, L = 2;
    bf16x8 af[Cfg::KSUB][Cfg::FM], bfr[G];
    auto read_a = [&](int ks, int i) {
        const int row = wm * Cfg::WTM + i * 16;
        af[ks][i] = A_KC ? frag_kc<Cfg::BM>(As, row, ks, c.lane) : frag_mc<Cfg::BM>(As, row, ks, c.lane);
    };
    auto read_b = [&](int f) {
        const int ks = f / Cfg::FN, j = f % Cfg::FN;
        if constexpr (!DUAL) {
            const int row = wn * Cfg::WTN + j * 16;
            bfr[f] = B_KC ? frag_kc<Cfg::BN>(Bs, row, ks, c.lane)
                          : frag_mc<Cfg::BN>(Bs, row, ks, c.lane);
        } else {
            // Fragments 0 .. FN/2-1 from the first B tile, the rest from the second, at the same
            // columns: acc[i][j] and acc[i][j + FN/2] hold the same outputs of B and B2.
            constexpr int HB = Cfg::BN / 2, HF = Cfg::FN / 2;
            const MLPTP_LDS uint8_t* Bh = Bs + (j / HF) * (Cfg::B_BYTES / 2);
            const int row = wn * (Cfg::WTN / 2) + (j % HF) * 16;
            bfr[f] = B_KC ? frag_kc<HB>(Bh, row, ks, c.lane) : frag_mc<HB>(Bh, row, ks, c.lane);
        }
    };
    // Placement of the next stage's loads. With loader waves (Cfg::LOADERS_UP_FRONT) all of them
    // before the stage's first reads. Otherwise kPerGroup after each MFMA group, from the first;
    // with a transposed A (the weight-gradient products, whose strided operand loads take longer)
    // two per group, so they are all in flight within the first half of the stage. Measured on
    // the bench's rows against loads all up front: one per group was +1-2% on the forward, two
    // per group +2% on the GPT-3-175B layer, and either was within 1% on the rest.
    constexpr int kUpFront = Cfg::LOADERS_UP_FRONT ? SL::Q : 0;
    constexpr int kPerGroup = Cfg::LOADERS_UP_FRONT ? 0 : (A_KC ? 1 : 2);
    // A compile-time true when every wave loads: a runtime test would put a branch around each of
    // the stage's loads (measured: 2-8% on the tiles where every wave loads, bit-identical).
    const bool loader = Cfg::NLOAD == Cfg::NWAVES || c.wave < Cfg::NLOAD;
    // A scheduling barrier closes each group: without it the compiler, knowing the loads do not
    // alias the reads, sank all of a 256x192 tile's loads to the end of the stage, in front of the
    // wait for them (the GPT-3-175B layer ran 20% slower).
    constexpr bool kPin = true;
#pragma unroll
    for (int q = 0; q < kUpFront && q < SL::Q; ++q)
        if (loader) stage_load<Cfg, A_KC, B_KC, DUAL>(c, src, nxt, q);
    // B fragment 0 first: the first MFMA needs it and A fragment 0 only (3 reads, not 6).
    read_b(0);
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) read_a(0, i);
#pragma unroll
    for (int f = 1; f < L && f < G; ++f) read_b(f);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int ks = g / Cfg::FN, j = g % Cfg::FN;
        // Odd groups walk the A fragments backwards (a serpentine), so no two consecutive MFMAs
        // change both operands: fewer operand bits toggle, and the clock, which under this load
        // follows the power drawn, runs a little higher. Each accumulator's order of additions is
        // unchanged (bit-identical); measured 0.9% on the Llama shard's step, 0.4-0.9% on the
        // backward's dH, dX and dW1 products, a wash on dW2.
#pragma unroll
        for (int ii = 0; ii < Cfg::FM; ++ii) {
            const int i = (g & 1) ? Cfg::FM - 1 - ii : ii;
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[g], af[ks][i], acc[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kPerGroup; ++u) {
            const int q = kUpFront + g * kPerGroup + u;
            if (q < SL::Q && loader) stage_load<Cfg, A_KC, B_KC, DUAL>(c, src, nxt, q);
        }
        const int f = g + L;
        // The next k-substep's A fragments are spread over this substep's groups (fragment i
        // after group j with i % FN == j) rather than read all at once at the substep boundary:
        // measured 1-2% faster on the forward, dH and dW2 products (same box, interleaved runs),
        // bit-identical.
        if (ks + 1 < Cfg::KSUB) {
#pragma unroll
            for (int i = j; i < Cfg::FM; i += Cfg::FN) read_a(ks + 1, i);
        }
        if (f < G) read_b(f);
        if constexpr (kPin) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = kUpFront + G * kPerGroup; q < SL::Q; ++q)
        if (loader) stage_load<Cfg, A_KC, B_KC, DUAL>(c, src, nxt, q);
}

// For a pair of accumulator fragments a (columns c..c+15) and b (columns c+16..c+31) of the
// same 16 rows, where lane 16 g + r holds row r, columns 4 g..4 g+3 of each: x gets a on lanes
// r < 8 and, on lanes r >= 8, b of lane r - 8 (row r - 8); y gets a on lanes r >= 8 and, on
// lanes r < 8, b of lane r + 8 (row r + 8). Two DPP row shifts by 8 with bank masks (a bank is 4
// lanes of a 16-lane row; the masked-off lanes keep a).
__device__ __forceinline__ void swap_row_halves(const f32x4& a, const f32x4& b, f32x4& x, f32x4& y)
{
    // Each element is copied to a scalar before its bit pattern is taken: a bit cast of a vector
    // element expression reads the vector's first element, whichever element is named.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float ae = a[e], be = b[e];
        const int ai = __float_as_int(ae), bi = __float_as_int(be);
        x[e] = __int_as_float(__builtin_amdgcn_update_dpp(ai, bi, 0x118, 0xF, 0xC, false));
        y[e] = __int_as_float(__builtin_amdgcn_update_dpp(ai, bi, 0x108, 0xF, 0x3, false));
    }
}

// Whether an epilogue takes the dual form (two results per output element, from B and B2).
template <class E, class = void>
struct EpiIsDual : std::false_type {};
template <class E>
struct EpiIsDual<E, std::void_t<decltype(E::kDual)>> : std::bool_constant<E::kDual> {};

// C[M, N] = A B, or in the dual form the pair (A B, A B2) handed to epi.apply_dual: one A tile
// in LDS feeds both products, as the gated MLP's gate and up projections need [Z 08].
// With a grid of more than one row (gridDim.y = S), the contraction is split: workgroup
// (x, s) sums k in [s kc, min(K, (s + 1) kc)) only (kc a multiple of 64) and its epilogue
// tells the splits apart by blockIdx.y.
template <class Cfg, bool A_KC, bool B_KC, class Epi>
__global__ __launch_bounds__(Cfg::NTHREADS, Cfg::MIN_WAVES_PER_SIMD) void gemm_bf16_dma(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const uint16_t* __restrict__ B2, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
    Epi epi, int64_t kc)
{
    if (gridDim.y > 1) {
        const int64_t k0 = (int64_t)blockIdx.y * kc;
        K = (K - k0) < kc ? (K - k0) : kc;
        A += A_KC ? k0 : k0 * lda;
        B += B_KC ? k0 : k0 * ldb;
        if (B2) B2 += B_KC ? k0 : k0 * ldb;
    }
    constexpr bool DUAL = EpiIsDual<Epi>::value;
    constexpr int BNO = DUAL ? Cfg::BN / 2 : Cfg::BN;    // output columns per tile
    constexpr int WTNO = DUAL ? Cfg::WTN / 2 : Cfg::WTN;  // output columns per wave
    static_assert(!DUAL || (Cfg::FN % 2 == 0 && (Cfg::BN / 2) % 128 == 0),
                  "dual tiles are two halves of 128k columns");
    __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[2 * Cfg::STAGE_BYTES];
    // C-style cast: generic -> LDS address space (smem_raw is an LDS variable).
    MLPTP_LDS uint8_t* smem = (MLPTP_LDS uint8_t*)(smem_raw);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % Cfg::WAVES_M, wn = wave / Cfg::WAVES_M;

    const int64_t tiles_m = ceil_div(M, Cfg::BM), tiles_n = ceil_div(N, BNO);
    int64_t tm, tn;
    tile_coords<Cfg::GROUP_M>(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = tm * Cfg::BM, n0 = tn * BNO;
    const int m_left = (int)((M - m0) < Cfg::BM ? (M - m0) : Cfg::BM);
    const int n_left = (int)((N - n0) < BNO ? (N - n0) : BNO);

    f32x4 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Per-column epilogue data (the bias) is fetched before the main loop, so its latency hides
    // under the MFMAs instead of stalling the epilogue between stores.
    const int frow = lane & 15, fchunk = lane >> 4;
    typename Epi::ColData cdat[Cfg::FN];
    if constexpr (!DUAL && Epi::kColData) {
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
            cdat[j] = epi.col_load(n0 + wn * Cfg::WTN + j * 16 + 4 * fchunk, N);
    }

    const int64_t nk = ceil_div(K, Cfg::BK);
    const DmaCtx ctx{A, B, B2, M, N, K, lda, ldb, m0, n0, m_left, n_left, wave, lane};

    dma_issue<Cfg, A_KC, B_KC, DUAL>(ctx, 0, smem);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    // Two steps per trip, so both stages' LDS addresses are fixed in the code. The next stage's
    // sources advance before the wait and the barrier (pinned there by the scheduling barrier):
    // after the barrier a step starts with its fragment reads. Measured against one step per trip
    // with the sources recomputed from kt: +2.5% on the Llama down-projection, +3-6% on 128x128
    // tiles, bit-identical.
    StageSrc nsrc = stage_src<Cfg, A_KC, B_KC, DUAL>(ctx, 1);
    MLPTP_LDS uint8_t* s0 = smem;
    MLPTP_LDS uint8_t* s1 = smem + Cfg::STAGE_BYTES;
    for (int64_t kt = 0; kt < nk; kt += 2) {
        dma_step<Cfg, A_KC, B_KC, DUAL>(ctx, nsrc, s0, s1, acc, wm, wn);
        advance_src<Cfg, A_KC, B_KC, DUAL>(ctx, nsrc);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of the next stage
        __syncthreads();
        if (kt + 1 >= nk) break;
        dma_step<Cfg, A_KC, B_KC, DUAL>(ctx, nsrc, s1, s0, acc, wm, wn);
        advance_src<Cfg, A_KC, B_KC, DUAL>(ctx, nsrc);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
        const int64_t row = m0 + wm * Cfg::WTM + i * 16 + frow;
        if constexpr (DUAL) {
            // As below for the single form, per half: fragments j and j+1 of each half are 32
            // adjacent output columns.
            constexpr int HF = Cfg::FN / 2;
            const bool hi = frow >= 8;
            const int64_t row_lo = m0 + wm * Cfg::WTM + i * 16 + (frow & 7);
#pragma unroll
            for (int j = 0; j + 1 < HF; j += 2) {
                const int64_t c0 = n0 + wn * WTNO + j * 16 + 4 * fchunk;
                f32x4 gx, gy, ux, uy;
                swap_row_halves(acc[i][j], acc[i][j + 1], gx, gy);
                swap_row_halves(acc[i][HF + j], acc[i][HF + j + 1], ux, uy);
                epi.apply_dual(row_lo, c0 + (hi ? 16 : 0), gx, ux, M, N);
                epi.apply_dual(row_lo + 8, c0 + (hi ? 0 : 16), gy, uy, M, N);
            }
            if constexpr (HF % 2 != 0) {
                constexpr int j = HF - 1;
                const int64_t col = n0 + wn * WTNO + j * 16 + 4 * fchunk;
                epi.apply_dual(row, col, acc[i][j], acc[i][j + HF], M, N);
            }
        } else {
            // Fragments j and j+1 are 32 adjacent columns of the same 16 rows. Handed out as
            // they are, each store instruction would write 16 rows x 16 columns: half of each
            // row's 128-byte line in fp32, and a streaming store then reaches HBM as separate
            // partial-line writes. Instead lanes 8-15 of every 16-lane row swap their fragment
            // j+1 values with lanes 0-7's fragment j+1 values: the first store covers rows
            // 0-7 and the second rows 8-15, each row's 32 columns whole.
            const bool hi = frow >= 8;
            const int64_t row_lo = m0 + wm * Cfg::WTM + i * 16 + (frow & 7);
#pragma unroll
            for (int j = 0; j + 1 < Cfg::FN; j += 2) {
                const int64_t c0 = n0 + wn * Cfg::WTN + j * 16 + 4 * fchunk;
                f32x4 x, y;
                swap_row_halves(acc[i][j], acc[i][j + 1], x, y);
                const int64_t cx = c0 + (hi ? 16 : 0), cy = c0 + (hi ? 0 : 16);
                if constexpr (Epi::kColData) {
                    epi.apply(row_lo, cx, x, hi ? cdat[j + 1] : cdat[j], {}, M, N);
                    epi.apply(row_lo + 8, cy, y, hi ? cdat[j] : cdat[j + 1], {}, M, N);
                } else {
                    epi(row_lo, cx, x, M, N);
                    epi(row_lo + 8, cy, y, M, N);
                }
            }
            if constexpr (Cfg::FN % 2 != 0) {
                constexpr int j = Cfg::FN - 1;
                const int64_t col = n0 + wn * Cfg::WTN + j * 16 + 4 * fchunk;
                if constexpr (Epi::kColData)
                    epi.apply(row, col, acc[i][j], cdat[j], {}, M, N);
                else
                    epi(row, col, acc[i][j], M, N);
            }
        }
    }
}

}  // namespace mlptp
