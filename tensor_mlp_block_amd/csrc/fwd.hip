// fwd.hip -- forward shard kernels: column-parallel up-projection with fused bias and
// activation, and row-parallel down-projection to the fp32 partial.
//
// Also the gated (SwiGLU) up-projection and the accumulating form of the down-projection.
//
// Pages cited, as [tag section]:
//   [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
//   [J] jwzheng96.github.io, "张量并行 TP 与列并行 / 行并行的实现" (Megatron-LM tutorial ch. 7)
#include "dispatch.hpp"
#include "launch.hpp"

#include <atomic>

namespace mlptp {

int compute_units()
{
    // Queried once (the first device asked sizes every launch). Atomic, so host threads that
    // launch at the same time read either 0 (and query) or the stored count.
    static std::atomic<int> cus{0};
    int n = cus.load(std::memory_order_relaxed);
    if (n == 0) {
        int dev = 0, c = 0;
        n = (hipGetDevice(&dev) == hipSuccess &&
             hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
             c > 0)
                ? c
                : 256;
        cus.store(n, std::memory_order_relaxed);
    }
    return n;
}

// Z^(r) = X W1^(r) + b1^(r), H^(r) = phi(Z^(r)) [Z 02], [J 7.2 列并行].
// GEMM view: M = N tokens, N = Fs, K = D; A = X (k-contiguous), B = W1r [D, Fs]
// (n-contiguous, transposed into LDS).
void launch_up_proj(const void* X, const void* W1r, const void* b1r, void* Z, void* H, int64_t N,
                    int64_t D, int64_t Fs, int dtype, int act, hipStream_t s, float* ws,
                    int64_t ws_bytes)
{
    if (ws && dtype == kBF16) {
        const SplitPlan p = split_plan(true, false, N, Fs, D, D, Fs, compute_units());
        if (p.splits > 1 && split_workspace_bytes(p, N, Fs) <= ws_bytes) {
            // fp32 planes of X W1r over the contraction's ranges, then bias and phi over their
            // sum: the same epilogue arithmetic as the fused form.
            run_split<true, false>(X, W1r, N, Fs, D, D, Fs, p, ws, s);
            launch_split_bias_act(ws, p.splits, N * Fs, b1r, Z, H, N, Fs, dtype, act, s);
            return;
        }
    }
    const int vec = (Fs % 4 == 0);
    with_act(act, [&](auto a) {
        constexpr int ACT = decltype(a)::value;
        if (dtype == kBF16) {
            EpiBiasAct<uint16_t, ACT> epi{static_cast<const uint16_t*>(b1r),
                                          static_cast<uint16_t*>(Z), static_cast<uint16_t*>(H),
                                          Fs, vec};
            run_bf16<true, false>(X, W1r, N, Fs, D, D, Fs, epi, s);
        } else {
            EpiBiasAct<float, ACT> epi{static_cast<const float*>(b1r), static_cast<float*>(Z),
                                       static_cast<float*>(H), Fs, vec};
            run_simt<true, false>(X, W1r, N, Fs, D, D, Fs, epi, s);
        }
    });
}

// P^(r) = H^(r) W2^(r), fp32, no b2 [Z 02], [Z 05], [J 7.2 行并行].
// GEMM view: M = N tokens, N = D, K = Fs; A = H (k-contiguous), B = W2r [Fs, D]
// (n-contiguous).
void launch_down_proj(const void* H, const void* W2r, float* P, int64_t N, int64_t D, int64_t Fs,
                      int dtype, hipStream_t s, float* ws, int64_t ws_bytes)
{
    if (ws && dtype == kBF16) {
        const SplitPlan p = split_plan(true, false, N, D, Fs, Fs, D, compute_units());
        if (p.splits > 1 && split_workspace_bytes(p, N, D) <= ws_bytes) {
            // fp32 planes of H W2r over the contraction's ranges, summed in order into P.
            run_split<true, false>(H, W2r, N, D, Fs, Fs, D, p, ws, s);
            const float* planes[8];
            for (int i = 0; i < p.splits; ++i) planes[i] = ws + (int64_t)i * N * D;
            launch_partial_reduce(planes, p.splits, nullptr, kF32, P, N, D, s);
            return;
        }
    }
    EpiStoreF32 epi{P, D, (int)(D % 4 == 0)};
    if (dtype == kBF16)
        run_bf16<true, false>(H, W2r, N, D, Fs, Fs, D, epi, s);
    else
        run_simt<true, false>(H, W2r, N, D, Fs, Fs, D, epi, s);
}

int64_t fwd_split_workspace_bytes(int64_t N, int64_t D, int64_t Fs, int dtype)
{
    if (dtype != kBF16 || N == 0) return 0;
    const int64_t cus = compute_units();
    const int64_t up =
        split_workspace_bytes(split_plan(true, false, N, Fs, D, D, Fs, cus), N, Fs);
    const int64_t down =
        split_workspace_bytes(split_plan(true, false, N, D, Fs, Fs, D, cus), N, D);
    return up > down ? up : down;
}

// P^(r) = H^(r) W2^(r) + b2 / T: each rank adds its 1/T share of b2 to its own partial, so the
// plain sum of the partials carries b2 once [Z 05].
void launch_down_proj_bias_share(const void* H, const void* W2r, const void* b2, int b2_dtype,
                                 float* P, int64_t N, int64_t D, int64_t Fs, int T, int dtype,
                                 hipStream_t s)
{
    auto run = [&](auto epi) {
        if (dtype == kBF16)
            run_bf16<true, false>(H, W2r, N, D, Fs, Fs, D, epi, s);
        else
            run_simt<true, false>(H, W2r, N, D, Fs, Fs, D, epi, s);
    };
    const int vec = (int)(D % 4 == 0);
    if (b2_dtype == kBF16)
        run(EpiBiasShare<uint16_t>{P, static_cast<const uint16_t*>(b2), (float)T, D, vec});
    else
        run(EpiBiasShare<float>{P, static_cast<const float*>(b2), (float)T, D, vec});
}

// The tile each product of the shard takes, from the same chooser its launcher runs
// (run_bf16), with the GEMM views of the launchers in this file and in bwd.hip.
void shard_tile(int product, int64_t N, int64_t D, int64_t Fs, int64_t cus, int& rows, int& cols,
                int& staged)
{
    TileKind t = kTile256x256;
    switch (product) {
    case 0: t = choose_tile(true, false, N, Fs, D, D, Fs, cus); break;    // X . W1r
    case 1: t = choose_tile(true, false, N, D, Fs, Fs, D, cus); break;    // H . W2r
    case 2: t = choose_tile(true, true, N, Fs, D, D, D, cus); break;      // dY . W2r^T
    case 3: t = choose_tile(false, false, Fs, D, N, Fs, D, cus); break;   // H^T . dY
    case 4: t = choose_tile(false, false, D, Fs, N, D, Fs, cus); break;   // X^T . dZ
    default: t = choose_tile(true, true, N, D, Fs, Fs, Fs, cus); break;   // dZ . W1r^T
    }
    static const int kRows[] = {256, 256, 224, 256, 128, 128};
    static const int kCols[] = {256, 224, 256, 192, 128, 128};
    rows = kRows[t];
    cols = kCols[t];
    staged = t == kTileRegStaged ? 1 : 0;
}

// P += H^(r) W2^(r): the shards of one GPU adding their partials into one running fp32 buffer
// in turn, the sequential form of the block-tail sum [Z 02].
void launch_down_proj_accumulate(const void* H, const void* W2r, float* P, int64_t N, int64_t D,
                                 int64_t Fs, int dtype, hipStream_t s)
{
    EpiAccumF32 epi{P, D, (int)(D % 4 == 0)};
    if (dtype == kBF16)
        run_bf16<true, false>(H, W2r, N, D, Fs, Fs, D, epi, s);
    else
        run_simt<true, false>(H, W2r, N, D, Fs, Fs, D, epi, s);
}

// Gated up-projection [Z 08]: G = X Wg^(r), U = X Wu^(r) over the same columns,
// H = SiLU(G) * U. GEMM view as the plain up-projection (A = X, B = the [D, Fs] weight).
//   * bf16, shapes the direct-to-LDS kernel takes: one fused GEMM whose B tile holds 128
//     columns of Wg^(r) and the same 128 columns of Wu^(r), so each X tile in LDS feeds both
//     products and G, U never leave registers unless the caller keeps them.
//   * otherwise two GEMMs: the gate goes to G (or, when the caller does not keep G, to H as a
//     staging buffer), then the up GEMM's epilogue reads it back and writes H in place.
template <class T>
static void swiglu_up_typed(const void* X, const void* Wg, const void* Wu, void* G, void* U,
                            void* H, int64_t N, int64_t D, int64_t Fs, hipStream_t s)
{
    const int vec = (Fs % 4 == 0);
    T* h = static_cast<T*>(H);
    T* g = static_cast<T*>(G);
    T* u = static_cast<T*>(U);
    if constexpr (sizeof(T) == 2) {
        if (dma_eligible(true, false, N, Fs, D, D, Fs)) {
            EpiSwiGLU<T> epi{h, g, u, Fs, vec};
            run_dma<DmaTile256x256, true, false>(X, Wg, N, Fs, D, D, Fs, epi, s, Wu);
            return;
        }
    }
    T* gate = g ? g : h;
    EpiStore<T> first{gate, Fs, vec};
    EpiGateMul<T> second{gate, u, h, Fs, vec};
    if constexpr (sizeof(T) == 2) {
        run_bf16<true, false>(X, Wg, N, Fs, D, D, Fs, first, s);
        run_bf16<true, false>(X, Wu, N, Fs, D, D, Fs, second, s);
    } else {
        run_simt<true, false>(X, Wg, N, Fs, D, D, Fs, first, s);
        run_simt<true, false>(X, Wu, N, Fs, D, D, Fs, second, s);
    }
}

void launch_swiglu_up(const void* X, const void* Wg, const void* Wu, void* G, void* U, void* H,
                      int64_t N, int64_t D, int64_t Fs, int dtype, hipStream_t s)
{
    if (dtype == kBF16)
        swiglu_up_typed<uint16_t>(X, Wg, Wu, G, U, H, N, D, Fs, s);
    else
        swiglu_up_typed<float>(X, Wg, Wu, G, U, H, N, D, Fs, s);
}

}  // namespace mlptp
