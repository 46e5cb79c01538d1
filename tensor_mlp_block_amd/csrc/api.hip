// api.hip -- the extern "C" entry points of libmlptp.so (declared in include/mlp_tp.h).
//
// Each entry point validates every argument on the host before any HIP call, derives the
// shard width Fs = F / T from the global sizes, then enqueues its kernels on the caller's
// stream. Nothing here allocates, frees or synchronises.
//
// Pages cited, as [tag section]:
//   [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
//   [U] unpurerationalist.github.io, "LLM Systems 16: Model Parallel Training"
//   [F] 5688vip.com, "4、张量并行原理：张量切分方式（行并行、列并行）…"
#include "../../include/mlp_tp.h"
#include "launch.hpp"

#include <stdint.h>

#include <map>
#include <mutex>
#include <vector>

namespace {

using mlptp::kBF16;
using mlptp::kF32;

// Sizes above this are rejected so byte counts and grid sizes cannot overflow.
constexpr int64_t kMaxDim = INT32_MAX;
constexpr int64_t kMaxElems = int64_t(1) << 56;

struct Span {
    const void* p;
    int64_t bytes;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(Span a, Span b)
{
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

int elem_size(int32_t dtype) { return dtype == MLP_TP_BF16 ? 2 : 4; }

bool dtype_ok(int32_t dtype) { return dtype == MLP_TP_F32 || dtype == MLP_TP_BF16; }

bool act_ok(int32_t act) { return act >= MLP_TP_ACT_IDENTITY && act <= MLP_TP_ACT_GELU_SIGMOID; }

// Shape rules shared by the shard calls: N >= 0, D > 0, F > 0, T >= 1, T | F [U 3.8].
int check_shard_shape(int64_t N, int64_t D, int64_t F, int32_t T)
{
    if (N < 0 || D <= 0 || F <= 0 || T < 1) return MLP_TP_E_SHAPE;
    if (N > kMaxDim || D > kMaxDim || F > kMaxDim) return MLP_TP_E_SHAPE;
    if (F % T != 0) return MLP_TP_E_INDIVISIBLE;
    const int64_t Fs = F / T;
    if (N * Fs > kMaxElems || N * D > kMaxElems || D * Fs > kMaxElems) return MLP_TP_E_SHAPE;
    // Grid sizes: one workgroup per 64 x 64 tile or larger, for every product of the shard.
    const int64_t tn = (N + 63) / 64, td = (D + 63) / 64, tf = (Fs + 63) / 64;
    if (tn * td > INT32_MAX || tn * tf > INT32_MAX || td * tf > INT32_MAX) return MLP_TP_E_SHAPE;
    return MLP_TP_OK;
}

int all_aligned(std::initializer_list<const void*> ps)
{
    for (const void* p : ps)
        if (p && !aligned16(p)) return MLP_TP_E_ALIGN;
    return MLP_TP_OK;
}

// Every span in `outs` must be disjoint from every span in `ins` and from the other outs.
int disjoint(std::initializer_list<Span> outs, std::initializer_list<Span> ins)
{
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Span& i : ins)
            if (overlap(*o, i)) return MLP_TP_E_ALIAS;
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlap(*o, *o2)) return MLP_TP_E_ALIAS;
    }
    return MLP_TP_OK;
}

// HIP keeps one pending "last error" per host thread. An error already pending when a call is
// about to launch belongs to earlier work (the caller's, or another library's): the call then
// launches nothing and returns MLP_TP_E_HIP, and leaves that error pending for the caller to
// read. Checked once per call, just before its first HIP call.
int hip_clean()
{
    return hipPeekAtLastError() == hipSuccess ? MLP_TP_OK : MLP_TP_E_HIP;
}

// After this call's own launches (which started with no error pending): an error now came from
// them; it is reported as MLP_TP_E_HIP and cleared, so later work is not blamed for it.
int launch_status()
{
    return hipGetLastError() == hipSuccess ? MLP_TP_OK : MLP_TP_E_HIP;
}

// Cross-stream ordering of the overlapped block tail needs HIP events. They are synchronisation
// objects, not device memory: a pool per device, created on first use (timing disabled) and
// kept until the process ends. Calls hold the mutex while they enqueue, so calls from several
// host threads never share an event between a record and its wait.
std::mutex g_event_mu;
std::map<int, std::vector<hipEvent_t>> g_events;

// n events of the current device in *out; MLP_TP_E_HIP if HIP cannot create them.
int pooled_events(int n, hipEvent_t** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MLP_TP_E_HIP;
    std::vector<hipEvent_t>& pool = g_events[dev];
    while ((int)pool.size() < n) {
        hipEvent_t e;
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return MLP_TP_E_HIP;
        pool.push_back(e);
    }
    *out = pool.data();
    return MLP_TP_OK;
}

int check_up(const void* X, const void* W1r, const void* b1r, void* Z, void* H, int64_t N,
             int64_t D, int64_t F, int32_t T, int32_t dtype, int32_t act)
{
    if (!X || !W1r || !H) return MLP_TP_E_NULL;
    if (int rc = check_shard_shape(N, D, F, T)) return rc;
    if (!dtype_ok(dtype)) return MLP_TP_E_DTYPE;
    if (!act_ok(act)) return MLP_TP_E_ACT;
    if (int rc = all_aligned({X, W1r, b1r, Z, H})) return rc;
    const int64_t es = elem_size(dtype), Fs = F / T;
    return disjoint({{H, N * Fs * es}, {Z, N * Fs * es}},
                    {{X, N * D * es}, {W1r, D * Fs * es}, {b1r, Fs * es}});
}

int check_down(const void* H, const void* W2r, const float* P, int64_t N, int64_t D, int64_t F,
               int32_t T, int32_t dtype)
{
    if (!H || !W2r || !P) return MLP_TP_E_NULL;
    if (int rc = check_shard_shape(N, D, F, T)) return rc;
    if (!dtype_ok(dtype)) return MLP_TP_E_DTYPE;
    if (int rc = all_aligned({H, W2r, P})) return rc;
    const int64_t es = elem_size(dtype), Fs = F / T;
    return disjoint({{P, N * D * 4}}, {{H, N * Fs * es}, {W2r, Fs * D * es}});
}

int check_swiglu_up(const void* X, const void* Wg, const void* Wu, void* G, void* U, void* H,
                    int64_t N, int64_t D, int64_t F, int32_t T, int32_t dtype)
{
    if (!X || !Wg || !Wu || !H) return MLP_TP_E_NULL;
    if (int rc = check_shard_shape(N, D, F, T)) return rc;
    if (!dtype_ok(dtype)) return MLP_TP_E_DTYPE;
    if (int rc = all_aligned({X, Wg, Wu, G, U, H})) return rc;
    const int64_t es = elem_size(dtype), Fs = F / T;
    return disjoint({{H, N * Fs * es}, {G, N * Fs * es}, {U, N * Fs * es}},
                    {{X, N * D * es}, {Wg, D * Fs * es}, {Wu, D * Fs * es}});
}

// The reduce's own checks (shared by the full and the token-slice forms), except aliasing.
// Y may be NULL only where the caller allows it (an empty token slice).
int check_reduce(const float* const* P, int32_t T, const void* b2, int32_t b2_dtype,
                 const float* Y, int64_t N, int64_t D, bool y_optional = false)
{
    if (!P || (!Y && !y_optional)) return MLP_TP_E_NULL;
    if (T < 1 || T > MLP_TP_MAX_REDUCE_T || N < 0 || D <= 0 || N > kMaxDim || D > kMaxDim ||
        N * D > kMaxElems)
        return MLP_TP_E_SHAPE;
    for (int32_t r = 0; r < T; ++r)
        if (!P[r]) return MLP_TP_E_NULL;
    if (b2 && !dtype_ok(b2_dtype)) return MLP_TP_E_DTYPE;
    if ((Y && !aligned16(Y)) || (b2 && !aligned16(b2))) return MLP_TP_E_ALIGN;
    for (int32_t r = 0; r < T; ++r)
        if (!aligned16(P[r])) return MLP_TP_E_ALIGN;
    return MLP_TP_OK;
}

// Token slice r of N rows over T ranks: S = ceil(N / T) rows per slice [Z 04].
void token_slice(int64_t N, int32_t T, int32_t r, int64_t& row0, int64_t& rows)
{
    const int64_t S = (N + T - 1) / T;
    int64_t a = (int64_t)r * S, b = a + S;
    row0 = a < N ? a : N;
    rows = (b < N ? b : N) - row0;
}

}  // namespace

extern "C" {

int mlp_tp_up_proj(const void* X, const void* W1r, const void* b1r, void* Z, void* H, int64_t N,
                   int64_t D, int64_t F, int32_t T, int32_t dtype, int32_t act, void* stream)
{
    if (int rc = check_up(X, W1r, b1r, Z, H, N, D, F, T, dtype, act)) return rc;
    if (N == 0) return MLP_TP_OK;
    if (int rc = hip_clean()) return rc;
    mlptp::launch_up_proj(X, W1r, b1r, Z, H, N, D, F / T, dtype, act,
                          static_cast<hipStream_t>(stream));
    return launch_status();
}

int mlp_tp_down_proj(const void* H, const void* W2r, float* P, int64_t N, int64_t D, int64_t F,
                     int32_t T, int32_t dtype, void* stream)
{
    if (int rc = check_down(H, W2r, P, N, D, F, T, dtype)) return rc;
    if (N == 0) return MLP_TP_OK;
    if (int rc = hip_clean()) return rc;
    mlptp::launch_down_proj(H, W2r, P, N, D, F / T, dtype, static_cast<hipStream_t>(stream));
    return launch_status();
}

int mlp_tp_shard_fwd(const void* X, const void* W1r, const void* b1r, const void* W2r, void* H,
                     void* Z, float* P, int64_t N, int64_t D, int64_t F, int32_t T,
                     int32_t dtype, int32_t act, void* stream)
{
    if (int rc = check_up(X, W1r, b1r, Z, H, N, D, F, T, dtype, act)) return rc;
    if (int rc = check_down(H, W2r, P, N, D, F, T, dtype)) return rc;
    {
        const int64_t es = elem_size(dtype), Fs = F / T;
        // P is written after H is complete; it must still not clobber any input or Z.
        if (int rc = disjoint({{P, N * D * 4}}, {{X, N * D * es}, {W1r, D * Fs * es},
                                                  {b1r, Fs * es}, {Z, N * Fs * es}}))
            return rc;
        if (int rc = disjoint({{H, N * Fs * es}, {Z, N * Fs * es}}, {{W2r, Fs * D * es}}))
            return rc;
    }
    if (N == 0) return MLP_TP_OK;
    if (int rc = hip_clean()) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    mlptp::launch_up_proj(X, W1r, b1r, Z, H, N, D, F / T, dtype, act, s);
    if (int rc = launch_status()) return rc;
    mlptp::launch_down_proj(H, W2r, P, N, D, F / T, dtype, s);
    return launch_status();
}

int64_t mlp_tp_shard_fwd_workspace_bytes(int64_t N, int64_t D, int64_t F, int32_t T)
{
    if (int rc = check_shard_shape(N, D, F, T)) return rc;
    if (N == 0) return 0;
    return mlptp::fwd_split_workspace_bytes(N, D, F / T, MLP_TP_BF16);
}

int mlp_tp_shard_fwd_ws(const void* X, const void* W1r, const void* b1r, const void* W2r, void* H,
                        void* Z, float* P, void* workspace, size_t workspace_bytes, int64_t N,
                        int64_t D, int64_t F, int32_t T, int32_t dtype, int32_t act, void* stream)
{
    if (int rc = check_up(X, W1r, b1r, Z, H, N, D, F, T, dtype, act)) return rc;
    if (int rc = check_down(H, W2r, P, N, D, F, T, dtype)) return rc;
    if (workspace && !aligned16(workspace)) return MLP_TP_E_ALIGN;
    const int64_t wsb = workspace ? (int64_t)workspace_bytes : 0;
    if (wsb < 0) return MLP_TP_E_WORKSPACE;
    {
        const int64_t es = elem_size(dtype), Fs = F / T;
        if (int rc = disjoint({{P, N * D * 4}}, {{X, N * D * es}, {W1r, D * Fs * es},
                                                  {b1r, Fs * es}, {Z, N * Fs * es}}))
            return rc;
        if (int rc = disjoint({{H, N * Fs * es}, {Z, N * Fs * es}}, {{W2r, Fs * D * es}}))
            return rc;
        if (int rc = disjoint({{workspace, wsb}},
                              {{X, N * D * es}, {W1r, D * Fs * es}, {b1r, Fs * es},
                               {W2r, Fs * D * es}, {H, N * Fs * es}, {Z, N * Fs * es},
                               {P, N * D * 4}}))
            return rc;
    }
    if (N == 0) return MLP_TP_OK;
    if (int rc = hip_clean()) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // Both products split as planned, or neither: a workspace below the query's size (the
    // larger product's planes) leaves the shard exactly mlp_tp_shard_fwd.
    const int64_t need = mlptp::fwd_split_workspace_bytes(N, D, F / T, dtype);
    float* ws = (need > 0 && wsb >= need) ? static_cast<float*>(workspace) : nullptr;
    mlptp::launch_up_proj(X, W1r, b1r, Z, H, N, D, F / T, dtype, act, s, ws, wsb);
    if (int rc = launch_status()) return rc;
    mlptp::launch_down_proj(H, W2r, P, N, D, F / T, dtype, s, ws, wsb);
    return launch_status();
}

int mlp_tp_partial_reduce(const float* const* P, int32_t T, const void* b2, int32_t b2_dtype,
                          float* Y, int64_t N, int64_t D, void* stream)
{
    if (int rc = check_reduce(P, T, b2, b2_dtype, Y, N, D)) return rc;
    const int64_t bytes = N * D * 4;
    for (int32_t r = 0; r < T; ++r)
        if (P[r] != Y && overlap({Y, bytes}, {P[r], bytes})) return MLP_TP_E_ALIAS;
    if (b2 && overlap({Y, bytes}, {b2, D * elem_size(b2_dtype)})) return MLP_TP_E_ALIAS;
    if (N == 0) return MLP_TP_OK;
    if (int rc = hip_clean()) return rc;
    mlptp::launch_partial_reduce(P, T, b2, b2_dtype, Y, N, D, static_cast<hipStream_t>(stream));
    return launch_status();
}

int mlp_tp_token_slice(int64_t N, int32_t T, int32_t r, int64_t* row0, int64_t* rows)
{
    if (!row0 || !rows) return MLP_TP_E_NULL;
    if (N < 0 || T < 1 || r < 0 || r >= T) return MLP_TP_E_SHAPE;
    token_slice(N, T, r, *row0, *rows);
    return MLP_TP_OK;
}

int mlp_tp_partial_reduce_scatter(const float* const* P, int32_t T, int32_t r, const void* b2,
                                  int32_t b2_dtype, float* Yr, int64_t N, int64_t D, void* stream)
{
    // An empty slice has no rows to write: Yr may then be NULL (an empty tensor's pointer).
    const bool slice_ok = T >= 1 && r >= 0 && r < T && N >= 0;
    int64_t row0 = 0, rows = 0;
    if (slice_ok) token_slice(N, T, r, row0, rows);
    if (int rc = check_reduce(P, T, b2, b2_dtype, Yr, N, D, slice_ok && rows == 0)) return rc;
    if (r < 0 || r >= T) return MLP_TP_E_SHAPE;
    if (rows == 0) return MLP_TP_OK;
    const int64_t bytes = rows * D * 4, full = N * D * 4;
    for (int32_t s = 0; s < T; ++s)
        if (Yr != P[s] + row0 * D && overlap({Yr, bytes}, {P[s], full})) return MLP_TP_E_ALIAS;
    if (b2 && overlap({Yr, bytes}, {b2, D * elem_size(b2_dtype)})) return MLP_TP_E_ALIAS;
    // The slice's rows of every partial, reduced as a [rows, D] block tail. With D % 4 == 0 the
    // offset keeps each pointer 16-byte aligned; otherwise the reduce takes its element path.
    if (int rc = hip_clean()) return rc;
    const float* Ps[MLP_TP_MAX_REDUCE_T];
    for (int32_t s = 0; s < T; ++s) Ps[s] = P[s] + row0 * D;
    mlptp::launch_partial_reduce(Ps, T, b2, b2_dtype, Yr, rows, D,
                                 static_cast<hipStream_t>(stream));
    return launch_status();
}

int mlp_tp_down_proj_bias_share(const void* H, const void* W2r, const void* b2, int32_t b2_dtype,
                                float* P, int64_t N, int64_t D, int64_t F, int32_t T,
                                int32_t dtype, void* stream)
{
    if (int rc = check_down(H, W2r, P, N, D, F, T, dtype)) return rc;
    if (b2 && !dtype_ok(b2_dtype)) return MLP_TP_E_DTYPE;
    if (b2 && !aligned16(b2)) return MLP_TP_E_ALIGN;
    if (b2 && overlap({P, N * D * 4}, {b2, D * elem_size(b2_dtype)})) return MLP_TP_E_ALIAS;
    if (N == 0) return MLP_TP_OK;
    if (int rc = hip_clean()) return rc;
    mlptp::launch_down_proj_bias_share(H, W2r, b2, b2_dtype, P, N, D, F / T, T, dtype,
                                       static_cast<hipStream_t>(stream));
    return launch_status();
}

int mlp_tp_down_proj_accumulate(const void* H, const void* W2r, float* P, int64_t N, int64_t D,
                                int64_t F, int32_t T, int32_t dtype, void* stream)
{
    if (int rc = check_down(H, W2r, P, N, D, F, T, dtype)) return rc;
    if (N == 0) return MLP_TP_OK;
    if (int rc = hip_clean()) return rc;
    mlptp::launch_down_proj_accumulate(H, W2r, P, N, D, F / T, dtype,
                                       static_cast<hipStream_t>(stream));
    return launch_status();
}

int mlp_tp_down_proj_overlap_tail(const void* H, const void* W2r, const float* const* P,
                                  int32_t T, int32_t r, const void* b2, int32_t b2_dtype, float* Y,
                                  int64_t N, int64_t D, int64_t F, int32_t dtype,
                                  int64_t chunk_rows, void* stream, void* tail_stream)
{
    if (!P) return MLP_TP_E_NULL;
    if (T < 1 || T > MLP_TP_MAX_REDUCE_T || r < 0 || r >= T) return MLP_TP_E_SHAPE;
    if (int rc = check_down(H, W2r, P[r], N, D, F, T, dtype)) return rc;
    if (int rc = check_reduce(P, T, b2, b2_dtype, Y, N, D)) return rc;
    if (chunk_rows <= 0) return MLP_TP_E_SHAPE;
    const int64_t chunks = (N + chunk_rows - 1) / chunk_rows;
    if (chunks > MLP_TP_MAX_TAIL_CHUNKS) return MLP_TP_E_SHAPE;
    const int64_t es = elem_size(dtype), Fs = F / T, bytes = N * D * 4;
    for (int32_t s = 0; s < T; ++s) {
        if (P[s] != Y && overlap({Y, bytes}, {P[s], bytes})) return MLP_TP_E_ALIAS;
        if (s != r && overlap({P[r], bytes}, {P[s], bytes})) return MLP_TP_E_ALIAS;
    }
    if (int rc = disjoint({{Y, bytes}}, {{H, N * Fs * es}, {W2r, Fs * D * es}})) return rc;
    if (b2 && overlap({Y, bytes}, {b2, D * elem_size(b2_dtype)})) return MLP_TP_E_ALIAS;
    if (N == 0) return MLP_TP_OK;
    if (int rc = hip_clean()) return rc;

    const hipStream_t s0 = static_cast<hipStream_t>(stream);
    const hipStream_t s1 = static_cast<hipStream_t>(tail_stream);
    std::lock_guard<std::mutex> lock(g_event_mu);
    hipEvent_t* ev = nullptr;
    if (int rc = pooled_events((int)chunks + 1, &ev)) return rc;
    float* Pr = const_cast<float*>(P[r]);
    const char* Hb = static_cast<const char*>(H);
    const float* Ps[MLP_TP_MAX_REDUCE_T];
    for (int64_t c = 0; c < chunks; ++c) {
        const int64_t row0 = c * chunk_rows;
        const int64_t rows = (N - row0) < chunk_rows ? (N - row0) : chunk_rows;
        // P[r] rows [row0, row0 + rows) on the compute stream ...
        mlptp::launch_down_proj(Hb + row0 * Fs * es, W2r, Pr + row0 * D, rows, D, Fs, dtype, s0);
        if (hipEventRecord(ev[c], s0) != hipSuccess) return MLP_TP_E_HIP;
        // ... then the block tail of those rows on the tail stream once they are written.
        if (hipStreamWaitEvent(s1, ev[c], 0) != hipSuccess) return MLP_TP_E_HIP;
        for (int32_t s = 0; s < T; ++s) Ps[s] = P[s] + row0 * D;
        mlptp::launch_partial_reduce(Ps, T, b2, b2_dtype, Y + row0 * D, rows, D, s1);
    }
    // Chunked tail on its own stream, each chunk started as soon as it is computed [F 4.4.2].
    // Join: work queued on the compute stream after this call sees Y complete.
    if (hipEventRecord(ev[chunks], s1) != hipSuccess) return MLP_TP_E_HIP;
    if (hipStreamWaitEvent(s0, ev[chunks], 0) != hipSuccess) return MLP_TP_E_HIP;
    return launch_status();
}

int mlp_tp_swiglu_up_proj(const void* X, const void* Wgr, const void* Wur, void* G, void* U,
                          void* H, int64_t N, int64_t D, int64_t F, int32_t T, int32_t dtype,
                          void* stream)
{
    if (int rc = check_swiglu_up(X, Wgr, Wur, G, U, H, N, D, F, T, dtype)) return rc;
    if (N == 0) return MLP_TP_OK;
    if (int rc = hip_clean()) return rc;
    mlptp::launch_swiglu_up(X, Wgr, Wur, G, U, H, N, D, F / T, dtype,
                            static_cast<hipStream_t>(stream));
    return launch_status();
}

int mlp_tp_swiglu_shard_fwd(const void* X, const void* Wgr, const void* Wur, const void* W2r,
                            void* G, void* U, void* H, float* P, int64_t N, int64_t D, int64_t F,
                            int32_t T, int32_t dtype, void* stream)
{
    if (int rc = check_swiglu_up(X, Wgr, Wur, G, U, H, N, D, F, T, dtype)) return rc;
    if (int rc = check_down(H, W2r, P, N, D, F, T, dtype)) return rc;
    {
        const int64_t es = elem_size(dtype), Fs = F / T;
        if (int rc = disjoint({{P, N * D * 4}}, {{X, N * D * es}, {Wgr, D * Fs * es},
                                                  {Wur, D * Fs * es}, {G, N * Fs * es},
                                                  {U, N * Fs * es}}))
            return rc;
        if (int rc = disjoint({{H, N * Fs * es}, {G, N * Fs * es}, {U, N * Fs * es}},
                              {{W2r, Fs * D * es}}))
            return rc;
    }
    if (N == 0) return MLP_TP_OK;
    if (int rc = hip_clean()) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    mlptp::launch_swiglu_up(X, Wgr, Wur, G, U, H, N, D, F / T, dtype, s);
    if (int rc = launch_status()) return rc;
    mlptp::launch_down_proj(H, W2r, P, N, D, F / T, dtype, s);
    return launch_status();
}

int64_t mlp_tp_shard_bwd_workspace_bytes(int64_t N, int64_t D, int64_t F, int32_t T)
{
    if (int rc = check_shard_shape(N, D, F, T)) return rc;
    if (N == 0) return 0;
    return mlptp::colsum_workspace_bytes(N, F / T);
}

}  // extern "C"

namespace {

// The backward's checks except those of the workspace; *ws_need receives the bytes of
// workspace the column sum needs (0 without db1r or without tokens).
int check_bwd(const void* X, const void* W1r, const void* W2r, const void* Z, const void* H,
              const void* dY, const void* dZ, const float* dW1r, const float* db1r,
              const float* dW2r, const float* dXr, int64_t N, int64_t D, int64_t F, int32_t T,
              int32_t dtype, int32_t act, int64_t* ws_need)
{
    if (!X || !W1r || !W2r || !Z || !H || !dY || !dZ || !dW1r || !dW2r || !dXr)
        return MLP_TP_E_NULL;
    if (int rc = check_shard_shape(N, D, F, T)) return rc;
    if (!dtype_ok(dtype)) return MLP_TP_E_DTYPE;
    if (!act_ok(act)) return MLP_TP_E_ACT;
    if (int rc = all_aligned({X, W1r, W2r, Z, H, dY, dZ, dW1r, db1r, dW2r, dXr})) return rc;
    const int64_t es = elem_size(dtype), Fs = F / T;
    *ws_need = (db1r && N > 0) ? mlptp::colsum_workspace_bytes(N, Fs) : 0;
    return disjoint({{dZ, N * Fs * es}, {dW1r, D * Fs * 4}, {db1r, Fs * 4}, {dW2r, Fs * D * 4},
                     {dXr, N * D * 4}},
                    {{X, N * D * es}, {W1r, D * Fs * es}, {W2r, Fs * D * es}, {Z, N * Fs * es},
                     {H, N * Fs * es}, {dY, N * D * es}});
}

// The backward's launches on stream s [Z 06], [U 3.6.1]; `workspace` holds the column sum's
// workspace (every byte the column sum reads it writes first, so nothing needs clearing).
int run_bwd(const void* X, const void* W1r, const void* W2r, const void* Z, const void* H,
            const void* dY, void* dZ, float* dW1r, float* db1r, float* dW2r, float* dXr,
            void* workspace, int64_t N, int64_t D, int64_t Fs, int32_t dtype, int32_t act,
            hipStream_t s)
{
    // With N == 0 tokens dZ and dXr are empty, and the weight gradients are empty sums: the
    // K = 0 products and the column sum below then write zeros.
    if (N > 0) {
        // dZ = (dY W2r^T) * phi'(Z)  [Z 06]
        mlptp::launch_bwd_dz(dY, W2r, Z, dZ, N, D, Fs, dtype, act, s);
        if (int rc = launch_status()) return rc;
    }
    // dW2r = H^T dY   [U 3.6.1]: C [Fs, D], A = H stored [N, Fs], B = dY stored [N, D]
    mlptp::launch_wgrad(H, dY, dW2r, Fs, D, N, Fs, D, dtype, s);
    if (int rc = launch_status()) return rc;
    // dW1r = X^T dZ:  C [D, Fs], A = X stored [N, D], B = dZ stored [N, Fs]
    mlptp::launch_wgrad(X, dZ, dW1r, D, Fs, N, D, Fs, dtype, s);
    if (int rc = launch_status()) return rc;
    if (db1r) {
        mlptp::launch_colsum(dZ, static_cast<float*>(workspace), db1r, N, Fs, dtype, s);
        if (int rc = launch_status()) return rc;
    }
    if (N > 0) {
        // dXr = dZ W1r^T: this rank's partial of dX [Z 06 equation]
        mlptp::launch_dx(dZ, W1r, dXr, N, D, Fs, dtype, s);
    }
    return launch_status();
}

}  // namespace

extern "C" {

int mlp_tp_shard_bwd(const void* X, const void* W1r, const void* W2r, const void* Z,
                     const void* H, const void* dY, void* dZ, float* dW1r, float* db1r,
                     float* dW2r, float* dXr, void* workspace, size_t workspace_bytes,
                     int64_t N, int64_t D, int64_t F, int32_t T, int32_t dtype, int32_t act,
                     void* stream)
{
    int64_t ws_need = 0;
    if (int rc = check_bwd(X, W1r, W2r, Z, H, dY, dZ, dW1r, db1r, dW2r, dXr, N, D, F, T, dtype,
                           act, &ws_need))
        return rc;
    if (workspace && !aligned16(workspace)) return MLP_TP_E_ALIGN;
    if (ws_need > 0 && (!workspace || (int64_t)workspace_bytes < ws_need))
        return MLP_TP_E_WORKSPACE;
    {
        const int64_t es = elem_size(dtype), Fs = F / T;
        if (int rc = disjoint({{workspace, ws_need}},
                              {{dZ, N * Fs * es}, {dW1r, D * Fs * 4}, {db1r, Fs * 4},
                               {dW2r, Fs * D * 4}, {dXr, N * D * 4}, {X, N * D * es},
                               {W1r, D * Fs * es}, {W2r, Fs * D * es}, {Z, N * Fs * es},
                               {H, N * Fs * es}, {dY, N * D * es}}))
            return rc;
    }
    if (int rc = hip_clean()) return rc;
    return run_bwd(X, W1r, W2r, Z, H, dY, dZ, dW1r, db1r, dW2r, dXr, workspace, N, D, F / T,
                   dtype, act, static_cast<hipStream_t>(stream));
}

int mlp_tp_shard_bwd_noalloc(const void* X, const void* W1r, const void* W2r, const void* Z,
                             const void* H, const void* dY, void* dZ, float* dW1r, float* db1r,
                             float* dW2r, float* dXr, int64_t N, int64_t D, int64_t F, int32_t T,
                             int32_t dtype, int32_t act, void* stream)
{
    static_assert(MLP_TP_NOALLOC_SCRATCH_BYTES == mlptp::kNoallocScratchBytes,
                  "the header states the buffer's size");
    int64_t ws_need = 0;
    if (int rc = check_bwd(X, W1r, W2r, Z, H, dY, dZ, dW1r, db1r, dW2r, dXr, N, D, F, T, dtype,
                           act, &ws_need))
        return rc;
    if (ws_need > MLP_TP_NOALLOC_SCRATCH_BYTES) return MLP_TP_E_WORKSPACE;
    if (int rc = hip_clean()) return rc;
    // The library's own device buffer of the current GPU stands in for the workspace argument;
    // only its address (looked up once per device) is used, nothing is allocated.
    void* scratch = nullptr;
    if (ws_need > 0 && mlptp::noalloc_scratch(&scratch) != 0) return MLP_TP_E_HIP;
    return run_bwd(X, W1r, W2r, Z, H, dY, dZ, dW1r, db1r, dW2r, dXr, scratch, N, D, F / T, dtype,
                   act, static_cast<hipStream_t>(stream));
}

int mlp_tp_swiglu_shard_bwd(const void* X, const void* Wgr, const void* Wur, const void* W2r,
                            const void* G, const void* U, const void* H, const void* dY, void* dG,
                            void* dU, float* dWgr, float* dWur, float* dW2r, float* dXr,
                            int64_t N, int64_t D, int64_t F, int32_t T, int32_t dtype,
                            void* stream)
{
    if (!X || !Wgr || !Wur || !W2r || !G || !U || !H || !dY || !dG || !dU || !dWgr || !dWur ||
        !dW2r || !dXr)
        return MLP_TP_E_NULL;
    if (int rc = check_shard_shape(N, D, F, T)) return rc;
    if (!dtype_ok(dtype)) return MLP_TP_E_DTYPE;
    if (int rc = all_aligned({X, Wgr, Wur, W2r, G, U, H, dY, dG, dU, dWgr, dWur, dW2r, dXr}))
        return rc;
    const int64_t es = elem_size(dtype), Fs = F / T;
    if (int rc = disjoint({{dG, N * Fs * es}, {dU, N * Fs * es}, {dWgr, D * Fs * 4},
                           {dWur, D * Fs * 4}, {dW2r, Fs * D * 4}, {dXr, N * D * 4}},
                          {{X, N * D * es}, {Wgr, D * Fs * es}, {Wur, D * Fs * es},
                           {W2r, Fs * D * es}, {G, N * Fs * es}, {U, N * Fs * es},
                           {H, N * Fs * es}, {dY, N * D * es}}))
        return rc;
    if (int rc = hip_clean()) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // With N == 0 tokens the weight gradients are empty sums: the K = 0 products write zeros.
    if (N > 0) {
        // dG, dU from dH = dY W2r^T and the product rule through SiLU(G) * U  [Z 08]
        mlptp::launch_swiglu_bwd_dgu(dY, W2r, G, U, dG, dU, N, D, Fs, dtype, s);
        if (int rc = launch_status()) return rc;
    }
    // dW2r = H^T dY   [U 3.6.1]
    mlptp::launch_wgrad(H, dY, dW2r, Fs, D, N, Fs, D, dtype, s);
    if (int rc = launch_status()) return rc;
    // dWgr = X^T dG, dWur = X^T dU
    mlptp::launch_wgrad(X, dG, dWgr, D, Fs, N, D, Fs, dtype, s);
    if (int rc = launch_status()) return rc;
    mlptp::launch_wgrad(X, dU, dWur, D, Fs, N, D, Fs, dtype, s);
    if (int rc = launch_status()) return rc;
    if (N > 0) {
        // dXr = dG Wgr^T + dU Wur^T: the two input-gradient terms of the gated shard
        mlptp::launch_dx(dG, Wgr, dXr, N, D, Fs, dtype, s);
        if (int rc = launch_status()) return rc;
        mlptp::launch_dx_accumulate(dU, Wur, dXr, N, D, Fs, dtype, s);
    }
    return launch_status();
}

int mlp_tp_bias_act(const float* Z, const void* b1r, void* H, int64_t N, int64_t F, int32_t T,
                    int32_t dtype, int32_t act, void* stream)
{
    if (!Z || !H) return MLP_TP_E_NULL;
    // D does not enter; 1 stands in for it in the shared shape check.
    if (int rc = check_shard_shape(N, 1, F, T)) return rc;
    if (!dtype_ok(dtype)) return MLP_TP_E_DTYPE;
    if (!act_ok(act)) return MLP_TP_E_ACT;
    if (int rc = all_aligned({Z, b1r, H})) return rc;
    const int64_t es = elem_size(dtype), Fs = F / T;
    if (int rc = disjoint({{H, N * Fs * es}}, {{Z, N * Fs * 4}, {b1r, Fs * es}})) return rc;
    if (N == 0) return MLP_TP_OK;
    if (int rc = hip_clean()) return rc;
    mlptp::launch_bias_act(Z, b1r, H, N, Fs, dtype, act, static_cast<hipStream_t>(stream));
    return launch_status();
}

int mlp_tp_shard_tile(int32_t product, int64_t N, int64_t D, int64_t F, int32_t T,
                      int32_t compute_units, int32_t* tile_rows, int32_t* tile_cols,
                      int32_t* staged)
{
    if (product < MLP_TP_PROD_UP || product > MLP_TP_PROD_DX) return MLP_TP_E_DTYPE;
    if (int rc = check_shard_shape(N, D, F, T)) return rc;
    if (N == 0 || compute_units < 1) return MLP_TP_E_SHAPE;
    int rows = 0, cols = 0, st = 0;
    mlptp::shard_tile(product, N, D, F / T, compute_units, rows, cols, st);
    if (tile_rows) *tile_rows = rows;
    if (tile_cols) *tile_cols = cols;
    if (staged) *staged = st;
    return MLP_TP_OK;
}

const char* mlp_tp_strerror(int code)
{
    switch (code) {
    case MLP_TP_OK: return "success";
    case MLP_TP_E_NULL: return "a required pointer is NULL";
    case MLP_TP_E_SHAPE: return "invalid size (N < 0, D <= 0, F <= 0, T out of range, or too large)";
    case MLP_TP_E_INDIVISIBLE: return "the shard count T does not divide F";
    case MLP_TP_E_DTYPE: return "unknown dtype code";
    case MLP_TP_E_ACT: return "unknown activation code";
    case MLP_TP_E_ALIGN: return "a pointer is not 16-byte aligned";
    case MLP_TP_E_WORKSPACE: return "workspace missing or too small";
    case MLP_TP_E_HIP: return "a HIP kernel launch failed";
    case MLP_TP_E_ALIAS: return "an output overlaps an input or another output";
    default: return "unknown error code";
    }
}

}  // extern "C"
