// host_check.cpp -- CPU-only checks of the library's host code and of the oracle, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitized_host.py builds and
// runs it; no GPU, no HIP runtime).
//
// The C entry points (api.hip, compiled here as plain C++) run for real; the kernel launchers
// they call and the few HIP runtime functions they use are replaced by recording stubs, so
// every argument check, the derived shard width, the order of launches, the host arrays of
// partial pointers and the HIP error handling can be exercised without a GPU. The oracle runs
// on small cases, the pages' worked example among them.
//
// Pages cited:
//   [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
//   [C] charliedreemur.github.io, "TP:Column / Row Parallel Linear 怎么切? MLP 和 attention 怎么切?"
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "launch.hpp"
#include "mlp_tp.h"

// ------------------------------------------------------------------------------------------
// Stubs: the HIP runtime functions the entry points call, and the kernel launchers
// ------------------------------------------------------------------------------------------

static hipError_t g_pending = hipSuccess;  // the thread's pending "last error"
static int g_fail_launch = -1;             // launch index that "fails" (sets an error)
static std::vector<std::string> g_calls;   // launches, in order
static int g_events_made = 0;

static void record(const std::string& s)
{
    if ((int)g_calls.size() == g_fail_launch) g_pending = hipErrorLaunchFailure;
    g_calls.push_back(s);
}

extern "C" {
hipError_t hipPeekAtLastError(void) { return g_pending; }
hipError_t hipGetLastError(void)
{
    const hipError_t e = g_pending;
    g_pending = hipSuccess;
    return e;
}
hipError_t hipGetDevice(int* d)
{
    *d = 0;
    return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned)
{
    static char storage[1024];
    *e = reinterpret_cast<hipEvent_t>(storage + (g_events_made++ % 1024));
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t)
{
    record("event_record");
    return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int)
{
    record("stream_wait");
    return hipSuccess;
}
}

static std::string fmt(const char* name, int64_t a, int64_t b, int64_t c)
{
    char buf[160];
    std::snprintf(buf, sizeof buf, "%s %lld %lld %lld", name, (long long)a, (long long)b,
                  (long long)c);
    return buf;
}

namespace mlptp {
void launch_up_proj(const void*, const void*, const void*, void*, void*, int64_t N, int64_t D,
                    int64_t Fs, int, int, hipStream_t, float* ws, int64_t ws_bytes)
{
    record(fmt("up", N, D, Fs) + (ws ? " ws" + std::to_string(ws_bytes) : ""));
}
void launch_down_proj(const void*, const void*, float*, int64_t N, int64_t D, int64_t Fs, int,
                      hipStream_t, float* ws, int64_t ws_bytes)
{
    record(fmt("down", N, D, Fs) + (ws ? " ws" + std::to_string(ws_bytes) : ""));
}
int64_t fwd_split_workspace_bytes(int64_t N, int64_t D, int64_t Fs, int)
{
    return N * (D > Fs ? D : Fs) * 4;
}
void launch_down_proj_accumulate(const void*, const void*, float*, int64_t N, int64_t D,
                                 int64_t Fs, int, hipStream_t)
{
    record(fmt("down_acc", N, D, Fs));
}
void launch_down_proj_bias_share(const void*, const void*, const void*, int, float*, int64_t N,
                                 int64_t D, int64_t Fs, int T, int, hipStream_t)
{
    record(fmt("down_share", N, D, Fs) + " T" + std::to_string(T));
}
void shard_tile(int product, int64_t, int64_t, int64_t, int64_t cus, int& rows, int& cols,
                int& staged)
{
    rows = 100 + product;
    cols = (int)cus;
    staged = 0;
}
void launch_swiglu_up(const void*, const void*, const void*, void*, void*, void*, int64_t N,
                      int64_t D, int64_t Fs, int, hipStream_t)
{
    record(fmt("swiglu_up", N, D, Fs));
}
void launch_bwd_dz(const void*, const void*, const void*, void*, int64_t N, int64_t D,
                   int64_t Fs, int, int, hipStream_t)
{
    record(fmt("dz", N, D, Fs));
}
void launch_swiglu_bwd_dgu(const void*, const void*, const void*, const void*, void*, void*,
                           int64_t N, int64_t D, int64_t Fs, int, hipStream_t)
{
    record(fmt("dgu", N, D, Fs));
}
void launch_wgrad(const void*, const void*, float*, int64_t M, int64_t N, int64_t K, int64_t,
                  int64_t, int, hipStream_t)
{
    record(fmt("wgrad", M, N, K));
}
void launch_dx(const void*, const void*, float*, int64_t N, int64_t D, int64_t Fs, int,
               hipStream_t)
{
    record(fmt("dx", N, D, Fs));
}
void launch_dx_accumulate(const void*, const void*, float*, int64_t N, int64_t D, int64_t Fs,
                          int, hipStream_t)
{
    record(fmt("dx_acc", N, D, Fs));
}
// The column sum's workspace as the library sizes it: one fp32 row of Fs per 64 tokens.
int64_t colsum_workspace_bytes(int64_t N, int64_t Fs) { return (N + 63) / 64 * Fs * 4; }
static const void* g_last_ws = nullptr;
void launch_colsum(const void*, float* ws, float*, int64_t N, int64_t Fs, int, hipStream_t)
{
    g_last_ws = ws;
    record(fmt("colsum", N, Fs, 0));
}
void launch_bias_act(const float*, const void*, void*, int64_t N, int64_t Fs, int, int,
                     hipStream_t)
{
    record(fmt("bias_act", N, Fs, 0));
}
static std::vector<const float*> g_reduce_ptrs;
void launch_partial_reduce(const float* const* P, int T, const void*, int, float*, int64_t N,
                           int64_t D, hipStream_t)
{
    g_reduce_ptrs.assign(P, P + T);  // reads the whole host array: ASan checks its bounds
    record(fmt("reduce", T, N, D));
}
static char g_scratch_stand_in[16] __attribute__((aligned(256)));
int noalloc_scratch(void** ptr)
{
    *ptr = g_scratch_stand_in;
    return 0;
}
}  // namespace mlptp

// ------------------------------------------------------------------------------------------
// Oracle entry points (mlp_oracle.c)
// ------------------------------------------------------------------------------------------

extern "C" {
int oracle_shard_fwd(const double*, const double*, const double*, const double*, int64_t, int64_t,
                     int64_t, int32_t, int32_t, int, double*, double*, double*);
int oracle_partial_sum(const double* const*, int32_t, const double*, int64_t, int64_t, double*);
int oracle_partial_sum_bias_share(const double* const*, int32_t, int32_t, const double*, int64_t,
                                  int64_t, double*);
int oracle_block_fwd(const double*, const double*, const double*, const double*, const double*,
                     int64_t, int64_t, int64_t, int32_t, int, double*);
int oracle_dense_fwd(const double*, const double*, const double*, const double*, const double*,
                     int64_t, int64_t, int64_t, int, double*);
int oracle_shard_bwd(const double*, const double*, const double*, const double*, const double*,
                     int64_t, int64_t, int64_t, int32_t, int32_t, int, double*, double*, double*,
                     double*, double*);
int oracle_dense_bwd(const double*, const double*, const double*, const double*, const double*,
                     int64_t, int64_t, int64_t, int, double*, double*, double*, double*, double*);
int oracle_partial_reduce_scatter(const double* const*, int32_t, int32_t, const double*, int64_t,
                                  int64_t, double*);
int oracle_swiglu_shard_fwd(const double*, const double*, const double*, const double*, int64_t,
                            int64_t, int64_t, int32_t, int32_t, double*, double*, double*,
                            double*);
int oracle_swiglu_shard_bwd(const double*, const double*, const double*, const double*,
                            const double*, int64_t, int64_t, int64_t, int32_t, int32_t, double*,
                            double*, double*, double*, double*, double*);
}

// ------------------------------------------------------------------------------------------
// Checks
// ------------------------------------------------------------------------------------------

static int g_failed = 0;
#define CHECK(cond)                                                                   \
    do {                                                                              \
        if (!(cond)) {                                                                \
            std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);   \
            ++g_failed;                                                               \
        }                                                                             \
    } while (0)

static void reset()
{
    g_calls.clear();
    g_pending = hipSuccess;
    g_fail_launch = -1;
}

// Fake device addresses: aligned, never dereferenced (the launchers are stubs).
static void* addr(uintptr_t a) { return reinterpret_cast<void*>(a); }
static float* faddr(uintptr_t a) { return reinterpret_cast<float*>(a); }

static void check_forward_calls()
{
    // The library derives Fs = F / T from the global sizes [Z 07], then launches up and down.
    reset();
    CHECK(mlp_tp_shard_fwd(addr(0x10000), addr(0x200000), nullptr, addr(0x400000),
                           addr(0x600000), nullptr, faddr(0x800000), 4, 8, 16, 2, MLP_TP_BF16,
                           MLP_TP_ACT_GELU_TANH, nullptr) == MLP_TP_OK);
    CHECK(g_calls.size() == 2 && g_calls[0] == "up 4 8 8" && g_calls[1] == "down 4 8 8");
    // argument errors launch nothing
    reset();
    CHECK(mlp_tp_shard_fwd(addr(0x10000), addr(0x200000), nullptr, addr(0x400000),
                           addr(0x600000), nullptr, faddr(0x800000), 4, 8, 18, 4, MLP_TP_BF16,
                           MLP_TP_ACT_GELU_TANH, nullptr) == MLP_TP_E_INDIVISIBLE);
    CHECK(g_calls.empty());
    // the split-contraction forward: the caller's workspace reaches both products; without
    // one it is exactly the plain forward
    reset();
    CHECK(mlp_tp_shard_fwd_workspace_bytes(4, 8, 16, 2) == 4 * 8 * 4);
    CHECK(mlp_tp_shard_fwd_ws(addr(0x10000), addr(0x200000), nullptr, addr(0x400000),
                              addr(0x600000), nullptr, faddr(0x800000), addr(0x900000), 128, 4, 8,
                              16, 2, MLP_TP_BF16, MLP_TP_ACT_GELU_TANH, nullptr) == MLP_TP_OK);
    CHECK(g_calls.size() == 2 && g_calls[0] == "up 4 8 8 ws128" &&
          g_calls[1] == "down 4 8 8 ws128");
    reset();
    CHECK(mlp_tp_shard_fwd_ws(addr(0x10000), addr(0x200000), nullptr, addr(0x400000),
                              addr(0x600000), nullptr, faddr(0x800000), nullptr, 0, 4, 8, 16, 2,
                              MLP_TP_BF16, MLP_TP_ACT_GELU_TANH, nullptr) == MLP_TP_OK);
    CHECK(g_calls.size() == 2 && g_calls[0] == "up 4 8 8" && g_calls[1] == "down 4 8 8");
    // a workspace below the query's size: neither product gets it
    reset();
    CHECK(mlp_tp_shard_fwd_ws(addr(0x10000), addr(0x200000), nullptr, addr(0x400000),
                              addr(0x600000), nullptr, faddr(0x800000), addr(0x900000), 127, 4, 8,
                              16, 2, MLP_TP_BF16, MLP_TP_ACT_GELU_TANH, nullptr) == MLP_TP_OK);
    CHECK(g_calls.size() == 2 && g_calls[0] == "up 4 8 8" && g_calls[1] == "down 4 8 8");
    reset();
    CHECK(mlp_tp_shard_fwd_ws(addr(0x10000), addr(0x200000), nullptr, addr(0x400000),
                              addr(0x600000), nullptr, faddr(0x800000), addr(0x800010), 128, 4, 8,
                              16, 2, MLP_TP_BF16, MLP_TP_ACT_GELU_TANH,
                              nullptr) == MLP_TP_E_ALIAS);  // workspace over P
    CHECK(g_calls.empty());
    // b2 share: the rank count travels to the epilogue [Z 05]
    reset();
    CHECK(mlp_tp_down_proj_bias_share(addr(0x10000), addr(0x200000), addr(0x300000), MLP_TP_F32,
                                      faddr(0x800000), 4, 8, 24, 3, MLP_TP_BF16,
                                      nullptr) == MLP_TP_OK);
    CHECK(g_calls.size() == 1 && g_calls[0] == "down_share 4 8 8 T3");
}

static void check_hip_error_handling()
{
    // An error pending before the call is not the call's: nothing launches, the error stays.
    reset();
    g_pending = hipErrorInvalidValue;
    CHECK(mlp_tp_up_proj(addr(0x10000), addr(0x200000), nullptr, nullptr, addr(0x600000), 4, 8,
                         16, 2, MLP_TP_BF16, MLP_TP_ACT_RELU, nullptr) == MLP_TP_E_HIP);
    CHECK(g_calls.empty());
    CHECK(g_pending == hipErrorInvalidValue);
    // A failure of the call's own launch is reported and cleared; the second launch of the
    // forward is not issued after the first fails.
    reset();
    g_fail_launch = 0;
    CHECK(mlp_tp_shard_fwd(addr(0x10000), addr(0x200000), nullptr, addr(0x400000),
                           addr(0x600000), nullptr, faddr(0x800000), 4, 8, 16, 2, MLP_TP_BF16,
                           MLP_TP_ACT_GELU_TANH, nullptr) == MLP_TP_E_HIP);
    CHECK(g_calls.size() == 1);
    CHECK(g_pending == hipSuccess);
    // N == 0 is a host no-op even with an error pending: no HIP call at all.
    reset();
    g_pending = hipErrorInvalidValue;
    CHECK(mlp_tp_down_proj(addr(0x10000), addr(0x200000), faddr(0x800000), 0, 8, 16, 2,
                           MLP_TP_BF16, nullptr) == MLP_TP_OK);
    CHECK(g_pending == hipErrorInvalidValue);
}

static void check_reduce_host_arrays()
{
    // The host array of partial pointers is read for exactly T entries (heap-allocated at its
    // exact size, so ASan reports any read past it).
    for (int T : {1, 3, MLP_TP_MAX_REDUCE_T}) {
        reset();
        const float** P = static_cast<const float**>(std::malloc(sizeof(float*) * T));
        for (int r = 0; r < T; ++r) P[r] = faddr(0x1000000 + (uintptr_t)r * 0x10000);
        CHECK(mlp_tp_partial_reduce(P, T, nullptr, MLP_TP_F32, faddr(0x100000000ull), 16, 64,
                                    nullptr) == MLP_TP_OK);
        CHECK(g_calls.size() == 1 && (int)mlptp::g_reduce_ptrs.size() == T);
        // token slice r of the reduce-scatter layout: pointers offset by its first row [Z 04]
        reset();
        CHECK(mlp_tp_partial_reduce_scatter(P, T, 0, nullptr, MLP_TP_F32, faddr(0x100000000ull),
                                            16, 64, nullptr) == MLP_TP_OK);
        std::free(P);
    }
    const float* P65[65];
    for (int r = 0; r < 65; ++r) P65[r] = faddr(0x1000000 + (uintptr_t)r * 0x10000);
    CHECK(mlp_tp_partial_reduce(P65, 65, nullptr, MLP_TP_F32, faddr(0x100000000ull), 16, 64,
                                nullptr) == MLP_TP_E_SHAPE);
    // the overlapped tail: chunks of the down-projection, each followed by its tail
    reset();
    const float* P2[2] = {faddr(0x1000000), faddr(0x2000000)};
    CHECK(mlp_tp_down_proj_overlap_tail(addr(0x10000), addr(0x200000), P2, 2, 1, nullptr,
                                        MLP_TP_F32, faddr(0x3000000), 10, 8, 16, MLP_TP_BF16, 4,
                                        nullptr, addr(0x8)) == MLP_TP_OK);
    // 3 chunks: (down, record, wait, reduce) x 3, then record + wait to join
    CHECK(g_calls.size() == 14);
    CHECK(g_calls[0] == "down 4 8 8" && g_calls[8] == "down 2 8 8");
}

static void check_backward_calls()
{
    auto bwd = [](int64_t N, void* ws, size_t wsb, float* db1) {
        return mlp_tp_shard_bwd(addr(0x10000), addr(0x20000), addr(0x30000), addr(0x40000),
                                addr(0x50000), addr(0x60000), addr(0x1000000), faddr(0x2000000),
                                db1, faddr(0x3000000), faddr(0x4000000), ws, wsb, N, 8, 16, 2,
                                MLP_TP_BF16, MLP_TP_ACT_GELU_TANH, nullptr);
    };
    reset();
    CHECK(bwd(300, addr(0x5000000), 5 * 8 * 4, faddr(0x6000000)) == MLP_TP_OK);
    CHECK(g_calls.size() == 5 && g_calls[0] == "dz 300 8 8" && g_calls[1] == "wgrad 8 8 300" &&
          g_calls[3] == "colsum 300 8 0" && g_calls[4] == "dx 300 8 8");
    reset();
    CHECK(bwd(300, addr(0x5000000), 5 * 8 * 4 - 1, faddr(0x6000000)) == MLP_TP_E_WORKSPACE);
    CHECK(g_calls.empty());
    // the allocation-free form: the library's own buffer stands in for the workspace
    reset();
    CHECK(mlp_tp_shard_bwd_noalloc(addr(0x10000), addr(0x20000), addr(0x30000), addr(0x40000),
                                   addr(0x50000), addr(0x60000), addr(0x1000000),
                                   faddr(0x2000000), faddr(0x6000000), faddr(0x3000000),
                                   faddr(0x4000000), 300, 8, 16, 2, MLP_TP_BF16,
                                   MLP_TP_ACT_GELU_TANH, nullptr) == MLP_TP_OK);
    CHECK(g_calls.size() == 5 && mlptp::g_last_ws == mlptp::g_scratch_stand_in);
    reset();
    // 32776 tokens of Fs = 4096: 513 slabs x 4096 x 4 bytes of workspace, above 8 MiB
    // (buffers 512 MiB apart, so no output overlaps an input)
    const uintptr_t g = uintptr_t(1) << 29;
    CHECK(mlp_tp_shard_bwd_noalloc(addr(1 * g), addr(2 * g), addr(3 * g), addr(4 * g),
                                   addr(5 * g), addr(6 * g), addr(7 * g), faddr(8 * g),
                                   faddr(9 * g), faddr(10 * g), faddr(11 * g), 32776, 64, 4096, 1,
                                   MLP_TP_BF16, MLP_TP_ACT_GELU_TANH,
                                   nullptr) == MLP_TP_E_WORKSPACE);
    CHECK(g_calls.empty());
    // the tile query writes only the outputs it is given
    int32_t rows = 0, cols = 0;
    CHECK(mlp_tp_shard_tile(MLP_TP_PROD_DX, 4, 8, 16, 2, 256, &rows, &cols, nullptr) ==
          MLP_TP_OK);
    CHECK(rows == 100 + MLP_TP_PROD_DX && cols == 256);
    for (int code = 1; code >= -10; --code) CHECK(mlp_tp_strerror(code) != nullptr);
}

// ---- the oracle on small cases ----

static void check_oracle()
{
    // [Z 03]: x = [1, 2] through the 2x4 W1 and the 4x2 W2 under ReLU, two shards: [4, 5].
    const double x[2] = {1, 2};
    const double W1[8] = {1, 0, 1, 2, 0, 1, 1, -1};
    const double W2[8] = {1, 0, 0, 1, 1, 1, 2, -1};
    double Z[2], H[2], P0[2], P1[2], Y[2];
    CHECK(oracle_shard_fwd(x, W1, nullptr, W2, 1, 2, 4, 2, 0, 1, Z, H, P0) == 0);
    CHECK(oracle_shard_fwd(x, W1, nullptr, W2, 1, 2, 4, 2, 1, 1, Z, H, P1) == 0);
    const double* parts[2] = {P0, P1};
    CHECK(oracle_partial_sum(parts, 2, nullptr, 1, 2, Y) == 0);
    CHECK(Y[0] == 4 && Y[1] == 5);
    const double b2[2] = {1, -1};
    CHECK(oracle_partial_sum_bias_share(parts, 2, 2, b2, 1, 2, Y) == 0);
    CHECK(Y[0] == 5 && Y[1] == 4);

    // A ragged case through every entry point: N = 7, D = 5, F = 12, T = 3 (and the tail's
    // token slices with N not a multiple of T), pseudo-random values.
    const int64_t N = 7, D = 5, F = 12;
    const int T = 3;
    std::vector<double> X(N * D), A1(D * F), bb1(F), A2(F * D), bb2(D), dY(N * D), Wu(D * F);
    uint64_t s = 12345;
    auto rnd = [&s]() {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return (double)((s >> 33) % 2001) / 1000.0 - 1.0;
    };
    for (auto* v : {&X, &A1, &bb1, &A2, &bb2, &dY, &Wu})
        for (double& e : *v) e = rnd();
    std::vector<double> Yb(N * D), Yd(N * D);
    for (int act = 0; act <= 4; ++act) {
        CHECK(oracle_block_fwd(X.data(), A1.data(), bb1.data(), A2.data(), bb2.data(), N, D, F,
                               T, act, Yb.data()) == 0);
        CHECK(oracle_dense_fwd(X.data(), A1.data(), bb1.data(), A2.data(), bb2.data(), N, D, F,
                               act, Yd.data()) == 0);
        for (int64_t i = 0; i < N * D; ++i) CHECK(std::fabs(Yb[i] - Yd[i]) < 1e-12);
    }
    const int64_t Fs = F / T;
    std::vector<double> dZ(N * Fs), dW1(D * Fs), db1(Fs), dW2(Fs * D), dX(N * D);
    std::vector<std::vector<double>> dXp(T, std::vector<double>(N * D));
    for (int r = 0; r < T; ++r)
        CHECK(oracle_shard_bwd(X.data(), A1.data(), bb1.data(), A2.data(), dY.data(), N, D, F, T,
                               r, 2, dZ.data(), dW1.data(), db1.data(), dW2.data(),
                               dXp[r].data()) == 0);
    std::vector<double> gW1(D * F), gb1(F), gW2(F * D), gb2(D), gX(N * D);
    CHECK(oracle_dense_bwd(X.data(), A1.data(), bb1.data(), A2.data(), dY.data(), N, D, F, 2,
                           gW1.data(), gb1.data(), gW2.data(), gb2.data(), gX.data()) == 0);
    const double* dxparts[3] = {dXp[0].data(), dXp[1].data(), dXp[2].data()};
    CHECK(oracle_partial_sum(dxparts, T, nullptr, N, D, dX.data()) == 0);
    for (int64_t i = 0; i < N * D; ++i) CHECK(std::fabs(dX[i] - gX[i]) < 1e-12);  // [Z 06]
    // token slices of the reduce-scatter layout [Z 04] (S = ceil(7 / 3) = 3 rows: 3, 3, 1)
    // put together give the full tail
    std::vector<double> Yfull(N * D);
    CHECK(oracle_partial_sum(dxparts, T, bb2.data(), N, D, Yfull.data()) == 0);
    const int64_t S = (N + T - 1) / T;
    for (int r = 0; r < T; ++r) {
        const int64_t row0 = r * S, rows = (row0 + S <= N) ? S : N - row0;
        std::vector<double> Yr(rows * D);
        CHECK(oracle_partial_reduce_scatter(dxparts, T, r, bb2.data(), N, D, Yr.data()) == 0);
        for (int64_t i = 0; i < rows * D; ++i) CHECK(Yr[i] == Yfull[row0 * D + i]);
    }
    std::vector<double> G(N * Fs), U(N * Fs), Hg(N * Fs), Pg(N * D);
    CHECK(oracle_swiglu_shard_fwd(X.data(), A1.data(), Wu.data(), A2.data(), N, D, F, T, 1,
                                  G.data(), U.data(), Hg.data(), Pg.data()) == 0);
    std::vector<double> dG(N * Fs), dU(N * Fs), dWg(D * Fs), dWu(D * Fs), dW2g(Fs * D),
        dXg(N * D);
    CHECK(oracle_swiglu_shard_bwd(X.data(), A1.data(), Wu.data(), A2.data(), dY.data(), N, D, F,
                                  T, 2, dG.data(), dU.data(), dWg.data(), dWu.data(),
                                  dW2g.data(), dXg.data()) == 0);
}

int main()
{
    check_forward_calls();
    check_hip_error_handling();
    check_reduce_host_arrays();
    check_backward_calls();
    check_oracle();
    if (g_failed) {
        std::fprintf(stderr, "%d check(s) failed\n", g_failed);
        return 1;
    }
    std::printf("host_check: all checks passed\n");
    return 0;
}
