/*
 * mlp_tp.h -- C ABI of libmlptp.so: one rank's tensor-parallel MLP shard on an MI355X (gfx950).
 *
 * Pages cited, as [tag section]:
 *   [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
 *   [C] charliedreemur.github.io, "TP:Column / Row Parallel Linear 怎么切? MLP 和 attention 怎么切?"
 *   [U] unpurerationalist.github.io, "LLM Systems 16: Model Parallel Training"
 *   [J] jwzheng96.github.io, "张量并行 TP 与列并行 / 行并行的实现" (Megatron-LM tutorial ch. 7)
 *   [F] 5688vip.com, "4、张量并行原理：张量切分方式（行并行、列并行）…"
 *
 * The method. An MLP H = phi(X W1 + b1), Y = H W2 + b2 [Z 01] is split over T ranks: W1 by
 * columns and W2 by the matching rows [Z 02], [U 3.2], [J 7.2]. Rank r (Fs = F / T hidden
 * columns) computes
 *     Z^(r) = X W1^(r) + b1^(r),   H^(r) = phi(Z^(r)),   P^(r) = H^(r) W2^(r)
 * with no exchange; P^(r) is a full-shape [N, D] partial. The block tail sums the partials
 * and adds b2 exactly once: Y = sum_r P^(r) + b2 [Z 02], [Z 05], [U 3.8]. In the backward,
 * each rank forms its own weight gradients locally; the input gradient is a sum of per-rank
 * partials dX^(r) = dZ^(r) W1^(r)^T [Z 06], [U 3.6.1].
 *
 * Conventions shared by every entry point:
 *   - Shapes are GLOBAL: callers pass the full FFN width F and the shard count T; the library
 *     derives Fs = F / T itself and rejects F % T != 0 [U 3.8] ("local vs global shape": [Z 07]).
 *   - N (tokens, the [B, L, D] activation flattened to [N, D] row-major [Z 04]) may be 0: the
 *     call is then a no-op that returns MLP_TP_OK. D, F must be > 0 and T >= 1.
 *   - All tensors are dense row-major with no padding. Pointers are DEVICE pointers (HIP
 *     device memory of the current device) unless stated otherwise, each 16-byte aligned.
 *   - dtype selects the element type of X, W1^(r), b1^(r), W2^(r), H, Z, dY and dZ:
 *     MLP_TP_F32 (float) or MLP_TP_BF16 (bfloat16, stored as 16-bit words). Partials, Y and
 *     every gradient except dZ are always float. Products accumulate in fp32; bf16 results
 *     (H, Z, dZ) are rounded to nearest even once.
 *   - Every call is asynchronous on the caller's HIP stream (a hipStream_t passed as void*;
 *     NULL is the null stream). The library never allocates, frees or synchronises; the
 *     caller owns all memory and must keep it alive until the stream has run the work.
 *   - Every argument is validated on the host BEFORE any HIP call; a failed check returns its
 *     negative code and launches nothing.
 *   - MLP_TP_E_HIP has two sources. (a) A HIP error was already pending on the calling thread
 *     (left by earlier work) when the call was about to launch: nothing is launched and that
 *     error stays pending for the caller's hipGetLastError. (b) One of this call's own launches
 *     failed: the error is cleared, and the stream may hold part of the call's work.
 *   - Outputs must not overlap inputs or each other (MLP_TP_E_ALIAS), except where stated.
 */
#ifndef MLP_TP_H
#define MLP_TP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MLP_TP_OK 0
#define MLP_TP_E_NULL (-1)        /* a required pointer is NULL */
#define MLP_TP_E_SHAPE (-2)       /* N < 0, D <= 0, F <= 0, T < 1, or T above the limit */
#define MLP_TP_E_INDIVISIBLE (-3) /* F % T != 0 */
#define MLP_TP_E_DTYPE (-4)       /* unknown dtype code */
#define MLP_TP_E_ACT (-5)         /* unknown activation code */
#define MLP_TP_E_ALIGN (-6)       /* a pointer is not 16-byte aligned */
#define MLP_TP_E_WORKSPACE (-7)   /* workspace NULL or smaller than the query returns */
#define MLP_TP_E_HIP (-8)         /* a HIP launch failed */
#define MLP_TP_E_ALIAS (-9)       /* an output overlaps an input or another output */

/* Element types. */
#define MLP_TP_F32 0
#define MLP_TP_BF16 1

/* Activations phi. GELU_TANH is 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))); GELU_ERF is
   z Phi(z); GELU_SIGMOID is z / (1 + exp(-1.702 z)) (the form in [C 代码]); RELU'(0) = 0. */
#define MLP_TP_ACT_IDENTITY 0
#define MLP_TP_ACT_RELU 1
#define MLP_TP_ACT_GELU_TANH 2
#define MLP_TP_ACT_GELU_ERF 3
#define MLP_TP_ACT_GELU_SIGMOID 4

/* Largest shard count mlp_tp_partial_reduce accepts in one call. */
#define MLP_TP_MAX_REDUCE_T 64

/* Most token chunks one overlapped block-tail call splits its rows into. */
#define MLP_TP_MAX_TAIL_CHUNKS 256

/*
 * Column-parallel up-projection with fused bias and activation [Z 02], [Z 05], [U 3.8]:
 *     Z = X . W1r + b1r   (fp32 accumulate),   H = phi(Z).
 *   X   [N, D]   dtype, replicated input.
 *   W1r [D, Fs]  dtype, this rank's column slice W1[:, r*Fs:(r+1)*Fs], itself row-major.
 *   b1r [Fs]     dtype, the matching slice of b1; NULL means no bias.
 *   Z   [N, Fs]  dtype output, pre-activation kept for the backward; NULL skips it.
 *   H   [N, Fs]  dtype output, the activation.
 * Errors: E_NULL (X, W1r, H), E_SHAPE, E_INDIVISIBLE, E_DTYPE, E_ACT, E_ALIGN, E_ALIAS
 * (H or Z overlapping X, W1r, b1r or each other), E_HIP.
 */
int mlp_tp_up_proj(const void* X, const void* W1r, const void* b1r, void* Z, void* H,
                   int64_t N, int64_t D, int64_t F, int32_t T, int32_t dtype, int32_t act,
                   void* stream);

/*
 * Row-parallel down-projection to this rank's full-shape partial [Z 02], [J 7.2]:
 *     P = H . W2r   (fp32 accumulate and output, NO b2: b2 belongs to the block tail [Z 05]).
 *   H   [N, Fs]  dtype.   W2r [Fs, D] dtype, the row slice W2[r*Fs:(r+1)*Fs, :].
 *   P   [N, D]   float output.
 * Errors: E_NULL, E_SHAPE, E_INDIVISIBLE, E_DTYPE, E_ALIGN, E_ALIAS (P overlapping H or W2r),
 * E_HIP.
 */
int mlp_tp_down_proj(const void* H, const void* W2r, float* P, int64_t N, int64_t D, int64_t F,
                     int32_t T, int32_t dtype, void* stream);

/*
 * One rank's forward shard: mlp_tp_up_proj then mlp_tp_down_proj on the same stream [Z 02].
 * There is deliberately no b2 argument: adding b2 per rank would give Y + T b2 after the
 * sum [Z 05]; b2 is taken only by mlp_tp_partial_reduce.
 *   X [N, D], W1r [D, Fs], b1r [Fs] (nullable), W2r [Fs, D]: dtype inputs.
 *   H [N, Fs] dtype output; Z [N, Fs] dtype output (nullable, needed for the backward);
 *   P [N, D] float output.
 * Errors: those of the two calls; all arguments are checked before the first launch.
 */
int mlp_tp_shard_fwd(const void* X, const void* W1r, const void* b1r, const void* W2r, void* H,
                     void* Z, float* P, int64_t N, int64_t D, int64_t F, int32_t T,
                     int32_t dtype, int32_t act, void* stream);

/*
 * Bytes of device workspace mlp_tp_shard_fwd_ws uses for these sizes on the current device:
 * 0 when both products of the shard fill the GPU unsplit. Only bf16 products split (for
 * MLP_TP_F32 any workspace is unused). A negative MLP_TP_E_* code for invalid sizes.
 */
int64_t mlp_tp_shard_fwd_workspace_bytes(int64_t N, int64_t D, int64_t F, int32_t T);

/*
 * mlp_tp_shard_fwd for shards whose products have too few output tiles to fill the GPU (few
 * tokens, or a narrow Fs or D [Z 04]): given a workspace, such a product splits its contraction
 * over several workgroups per output tile. Each split writes an fp32 partial of the product into
 * the workspace, and one streaming pass sums the partials in a fixed order and applies the
 * product's own epilogue (bias and phi for the up-projection, the fp32 partial P for the
 * down-projection). Deterministic, no atomics; the results differ from mlp_tp_shard_fwd's only
 * in the order of the fp32 additions (both are within the same tolerance of the exact result).
 *   Arguments as mlp_tp_shard_fwd, plus:
 *   workspace        device scratch owned by the caller, contents not preserved; NULL with
 *                    workspace_bytes = 0 gives exactly mlp_tp_shard_fwd.
 *   workspace_bytes  its size. The products split only when it is at least
 *                    mlp_tp_shard_fwd_workspace_bytes(N, D, F, T); a smaller workspace leaves
 *                    both unsplit (the call is then exactly mlp_tp_shard_fwd).
 * Errors: those of mlp_tp_shard_fwd, E_ALIGN (workspace), E_ALIAS (workspace overlapping any
 * input or output).
 */
int mlp_tp_shard_fwd_ws(const void* X, const void* W1r, const void* b1r, const void* W2r, void* H,
                        void* Z, float* P, void* workspace, size_t workspace_bytes, int64_t N,
                        int64_t D, int64_t F, int32_t T, int32_t dtype, int32_t act,
                        void* stream);

/*
 * Block-tail reduction on one GPU [Z 02], [Z 04], [Z 05], [U 3.8]:
 *     Y = (((P[0] + P[1]) + ...) + P[T-1]) + b2     (fp32, shards summed in rank order,
 *                                                    b2 added exactly once, last).
 * This is the sum the all-reduce of the row-parallel output performs, over T partial buffers
 * resident in this GPU's memory. With b2 = NULL it is the plain sum, e.g. of the input-gradient
 * partials dX^(r) [Z 06].
 *   P   HOST array of T device pointers, each to a float [N, D] partial.
 *   T   1 <= T <= MLP_TP_MAX_REDUCE_T.
 *   b2  [D] of b2_dtype (MLP_TP_F32 or MLP_TP_BF16); NULL means no bias.
 *   Y   [N, D] float output. Y may be exactly equal to any P[r] (in-place); a partial overlap
 *       with any P[r] or with b2 is E_ALIAS.
 * Errors: E_NULL (P, any P[r], Y), E_SHAPE (N < 0, D <= 0, T outside the range), E_DTYPE,
 * E_ALIGN, E_ALIAS, E_HIP.
 */
int mlp_tp_partial_reduce(const float* const* P, int32_t T, const void* b2, int32_t b2_dtype,
                          float* Y, int64_t N, int64_t D, void* stream);

/*
 * Rows of token slice r in the reduce-scatter layout of the block tail [Z 04]: slices are
 * contiguous, S = ceil(N / T) rows each in rank order, the last ones shorter or empty.
 *   row0, rows  HOST pointers receiving the first row and the row count of slice r.
 * Errors: E_NULL (row0, rows), E_SHAPE (N < 0, T < 1, r outside [0, T)). Launches nothing.
 */
int mlp_tp_token_slice(int64_t N, int32_t T, int32_t r, int64_t* row0, int64_t* rows);

/*
 * Block-tail reduction in the reduce-scatter layout [Z 04], [Z 05]: only token slice r of
 *     Y = (((P[0] + P[1]) + ...) + P[T-1]) + b2
 * is formed, so the residual stream stays token-sharded. It is the share of the sum that the
 * reduce-scatter of the row-parallel output leaves on rank r, computed here over T partials
 * resident in this GPU's memory; b2 is added once, to that rank's rows only.
 *   P   HOST array of T device pointers, each to a float [N, D] partial (whole partials).
 *   r   the slice, 0 <= r < T; its rows are those mlp_tp_token_slice(N, T, r) returns.
 *   b2  [D] of b2_dtype; NULL means no bias.
 *   Yr  [rows, D] float output. Yr may be exactly equal to P[s] + row0 * D for any s (in place
 *       over that partial's own slice rows); any other overlap with a partial or b2 is E_ALIAS.
 *       When the slice is empty Yr is not touched and may be NULL.
 * Errors: as mlp_tp_partial_reduce, and E_SHAPE for r outside [0, T). An empty slice is a no-op.
 */
int mlp_tp_partial_reduce_scatter(const float* const* P, int32_t T, int32_t r, const void* b2,
                                  int32_t b2_dtype, float* Yr, int64_t N, int64_t D, void* stream);

/*
 * Row-parallel down-projection added into a running fp32 sum [Z 02]:
 *     P += H . W2r
 * The one-GPU, one-buffer form of the block tail: the T shards, computed in turn, add their
 * partials into P (which the caller zeroes or seeds first), so no T separate [N, D] partials
 * are kept. Shapes, dtypes and errors as mlp_tp_down_proj. Calls on one P must be ordered on
 * one stream; the fp32 sum then follows rank order exactly like mlp_tp_partial_reduce.
 */
int mlp_tp_down_proj_accumulate(const void* H, const void* W2r, float* P, int64_t N, int64_t D,
                                int64_t F, int32_t T, int32_t dtype, void* stream);

/*
 * Row-parallel down-projection of rank r overlapped with the block tail [F 4.4.2], [F 4.4.3]:
 * on one GPU, the last shard's GEMM and the reduction of the finished token rows run at the
 * same time, the local form of cutting the tail's all-reduce into chunks, each sent as soon as
 * it is computed, on a stream of its own. The token
 * rows are cut into chunks of chunk_rows:
 *     P[r][chunk]  = H[chunk] . W2r                                   on `stream`;
 *     Y[chunk]     = (((P[0] + P[1]) + ...) + P[T-1])[chunk] + b2      on `tail_stream`,
 * the reduction of chunk c waiting only for the GEMM of chunk c.
 *   H [N, Fs], W2r [Fs, D]: dtype; Fs = F / T as for mlp_tp_down_proj.
 *   P   HOST array of T device pointers to float [N, D] partials. P[r] is written here; every
 *       other partial must be complete before work queued after this call on either stream
 *       could read it (e.g. computed earlier on `stream`).
 *   b2  [D] of b2_dtype or NULL; Y [N, D] float, may be exactly equal to any P[s].
 *   chunk_rows > 0, at most MLP_TP_MAX_TAIL_CHUNKS chunks.
 *   stream, tail_stream  HIP streams (may be the same; then nothing overlaps). On return, work
 *       queued on `stream` after this call sees Y complete.
 * The library keeps a small pool of HIP events per device for the cross-stream waits
 * (created on first use, never device memory); calls from several host threads are
 * serialised while they enqueue.
 * Errors: those of mlp_tp_down_proj and mlp_tp_partial_reduce, E_SHAPE (r outside [0, T),
 * chunk_rows <= 0, too many chunks), E_ALIAS (partials overlapping each other, Y overlapping
 * H, W2r, b2 or a partial other than exactly), E_HIP.
 */
int mlp_tp_down_proj_overlap_tail(const void* H, const void* W2r, const float* const* P,
                                  int32_t T, int32_t r, const void* b2, int32_t b2_dtype, float* Y,
                                  int64_t N, int64_t D, int64_t F, int32_t dtype,
                                  int64_t chunk_rows, void* stream, void* tail_stream);

/*
 * Row-parallel down-projection with rank r's share of b2 [Z 05]:
 *     P = H . W2r + b2 / T        (fp32; b2[d] / T rounded once to fp32, then added)
 * The alternative [Z 05] names to adding b2 once after the sum: every rank adds b2 / T to its
 * own partial, so the plain sum of the T partials (mlp_tp_partial_reduce with b2 = NULL) holds
 * b2 once. For T a power of two, b2 / T is exact and the result equals the b2-once tail on
 * exactly representable data; for other T it differs by the rounding of b2 / T and of the
 * extra additions (mlp_tp_partial_reduce's b2 argument is the exact form).
 *   H [N, Fs], W2r [Fs, D]: dtype, as for mlp_tp_down_proj.
 *   b2 [D] of b2_dtype (MLP_TP_F32 or MLP_TP_BF16), the FULL bias; NULL adds nothing.
 *   P [N, D] float output.
 * Errors: those of mlp_tp_down_proj, E_DTYPE (b2_dtype), E_ALIGN (b2), E_ALIAS (P over b2).
 */
int mlp_tp_down_proj_bias_share(const void* H, const void* W2r, const void* b2, int32_t b2_dtype,
                                float* P, int64_t N, int64_t D, int64_t F, int32_t T,
                                int32_t dtype, void* stream);

/*
 * Gated (SwiGLU) up-projection [Z 08]: the gate and up projections are cut at the SAME columns,
 * so each rank multiplies matching channels locally:
 *     G = X . Wgr,   U = X . Wur   (fp32 accumulate),   H = SiLU(G) * U,   SiLU(z) = z sigmoid(z).
 *   X    [N, D]   dtype, replicated input.
 *   Wgr  [D, Fs]  dtype, the gate weight's column slice Wg[:, r*Fs:(r+1)*Fs].
 *   Wur  [D, Fs]  dtype, the up weight's slice over the same columns.
 *   G, U [N, Fs]  dtype outputs, the two projections kept for a backward; NULL skips each.
 *   H    [N, Fs]  dtype output.
 * As on the page, the gated form has no biases. In bf16, G and U are rounded once when stored.
 * When D and Fs are multiples of 8 (bf16), the gate and up products share one GEMM pass and H
 * is formed from their fp32 values; otherwise the gate is computed first, rounded to dtype,
 * and H is formed from that rounded gate.
 * Errors: E_NULL (X, Wgr, Wur, H), E_SHAPE, E_INDIVISIBLE, E_DTYPE, E_ALIGN, E_ALIAS (H, G or U
 * overlapping X, Wgr, Wur or each other), E_HIP.
 */
int mlp_tp_swiglu_up_proj(const void* X, const void* Wgr, const void* Wur, void* G, void* U,
                          void* H, int64_t N, int64_t D, int64_t F, int32_t T, int32_t dtype,
                          void* stream);

/*
 * One rank's gated forward shard: mlp_tp_swiglu_up_proj then mlp_tp_down_proj on one stream
 * [Z 08]. No b2, as for mlp_tp_shard_fwd.
 *   X [N, D], Wgr, Wur [D, Fs], W2r [Fs, D]: dtype inputs.
 *   G, U [N, Fs] dtype outputs (nullable); H [N, Fs] dtype output; P [N, D] float output.
 * Errors: those of the two calls; all arguments are checked before the first launch.
 */
int mlp_tp_swiglu_shard_fwd(const void* X, const void* Wgr, const void* Wur, const void* W2r,
                            void* G, void* U, void* H, float* P, int64_t N, int64_t D, int64_t F,
                            int32_t T, int32_t dtype, void* stream);

/*
 * Bytes of device workspace mlp_tp_shard_bwd needs for these sizes (0 if none); a negative
 * MLP_TP_E_* code for invalid sizes.
 */
int64_t mlp_tp_shard_bwd_workspace_bytes(int64_t N, int64_t D, int64_t F, int32_t T);

/*
 * Backward of one rank's shard for the upstream gradient dY of the block output [Z 06],
 * [U 3.6.1], [C 推导 / 关键公式]:
 *     dH   = dY . W2r^T                 (no exchange: the row-parallel backward is local)
 *     dZ   = dH (.) phi'(Z)             (through the local activation)
 *     dW2r = H^T . dY      dW1r = X^T . dZ      db1r = sum over tokens of dZ
 *     dXr  = dZ . W1r^T                 (this rank's partial of dX; the sum over ranks,
 *                                        e.g. by mlp_tp_partial_reduce with b2 = NULL, is dX)
 *   Inputs (dtype): X [N, D], W1r [D, Fs], W2r [Fs, D], Z [N, Fs] and H [N, Fs] as saved by the
 *   forward, dY [N, D].
 *   Outputs: dZ [N, Fs] dtype; dW1r [D, Fs], db1r [Fs] (nullable), dW2r [Fs, D] and
 *   dXr [N, D], all float.
 *   workspace: device scratch of at least mlp_tp_shard_bwd_workspace_bytes(N, D, F, T)
 *   bytes (ignored when that is 0), owned by the caller, contents not preserved.
 * Errors: E_NULL, E_SHAPE, E_INDIVISIBLE, E_DTYPE, E_ACT, E_ALIGN, E_WORKSPACE, E_ALIAS
 * (any output overlapping an input, another output or the workspace), E_HIP.
 */
int mlp_tp_shard_bwd(const void* X, const void* W1r, const void* W2r, const void* Z,
                     const void* H, const void* dY, void* dZ, float* dW1r, float* db1r,
                     float* dW2r, float* dXr, void* workspace, size_t workspace_bytes,
                     int64_t N, int64_t D, int64_t F, int32_t T, int32_t dtype, int32_t act,
                     void* stream);

/*
 * mlp_tp_shard_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same computation and
 * results, with the column-sum workspace taken from a library-owned device buffer of
 * MLP_TP_NOALLOC_SCRATCH_BYTES per GPU (a static device array, resident until the process
 * ends) instead of an argument. The call allocates nothing.
 *   Arguments and outputs as mlp_tp_shard_bwd, without workspace and workspace_bytes.
 *   Every call on one GPU shares that GPU's buffer: calls that can overlap on one GPU (other
 *   streams, other host threads) race on it and must be ordered by the caller.
 * Errors: those of mlp_tp_shard_bwd, and E_WORKSPACE when db1r is requested and
 * mlp_tp_shard_bwd_workspace_bytes(N, D, F, T) exceeds MLP_TP_NOALLOC_SCRATCH_BYTES;
 * E_HIP also when the buffer's device address cannot be obtained.
 */
#define MLP_TP_NOALLOC_SCRATCH_BYTES (8 * 1024 * 1024)
int mlp_tp_shard_bwd_noalloc(const void* X, const void* W1r, const void* W2r, const void* Z,
                             const void* H, const void* dY, void* dZ, float* dW1r, float* db1r,
                             float* dW2r, float* dXr, int64_t N, int64_t D, int64_t F, int32_t T,
                             int32_t dtype, int32_t act, void* stream);

/*
 * Backward of one rank's gated (SwiGLU) shard [Z 08] for the upstream gradient dY, by the
 * same rules as mlp_tp_shard_bwd [Z 06], [U 3.6.1] with the product rule through
 * H = SiLU(G) * U:
 *     dH   = dY . W2r^T                    (local, as in the plain shard)
 *     dU   = dH (.) SiLU(G)                dG = dH (.) U (.) SiLU'(G),
 *                                          SiLU'(g) = s (1 + g (1 - s)), s = sigmoid(g)
 *     dW2r = H^T . dY      dWgr = X^T . dG      dWur = X^T . dU
 *     dXr  = dG . Wgr^T + dU . Wur^T       (this rank's partial of dX)
 *   Inputs (dtype): X [N, D], Wgr, Wur [D, Fs], W2r [Fs, D], G, U and H [N, Fs] as stored by
 *   mlp_tp_swiglu_shard_fwd, dY [N, D].
 *   Outputs: dG, dU [N, Fs] dtype (rounded once when stored; the weight and input gradients are
 *   formed from the stored values); dWgr, dWur [D, Fs], dW2r [Fs, D] and dXr [N, D], float.
 *   No workspace: the gated form has no bias, so no column sum.
 * Errors: E_NULL (any pointer), E_SHAPE, E_INDIVISIBLE, E_DTYPE, E_ALIGN, E_ALIAS (any output
 * overlapping an input or another output), E_HIP.
 */
int mlp_tp_swiglu_shard_bwd(const void* X, const void* Wgr, const void* Wur, const void* W2r,
                            const void* G, const void* U, const void* H, const void* dY, void* dG,
                            void* dU, float* dWgr, float* dWur, float* dW2r, float* dXr,
                            int64_t N, int64_t D, int64_t F, int32_t T, int32_t dtype,
                            void* stream);

/*
 * The up-projection's epilogue on its own [Z 02], [Z 05]: H = phi(Z + b1r) for a shard's
 * fp32 pre-activation, the same arithmetic the fused up-projection applies to its GEMM result
 * (bias add in fp32, phi, one rounding to dtype). For a pre-activation computed elsewhere, and
 * as the unfused reference that shows what the fusion saves.
 *   Z    [N, Fs] float, row-major, Fs = F / T.
 *   b1r  [Fs] dtype, the bias slice; NULL for no bias.
 *   H    [N, Fs] dtype output.
 * Errors: E_NULL (Z, H), E_SHAPE, E_INDIVISIBLE, E_DTYPE, E_ACT, E_ALIGN, E_ALIAS (H overlapping
 * Z or b1r), E_HIP. N = 0 is a no-op.
 */
int mlp_tp_bias_act(const float* Z, const void* b1r, void* H, int64_t N, int64_t F, int32_t T,
                    int32_t dtype, int32_t act, void* stream);

/* Products of one rank's shard, named for mlp_tp_shard_tile. */
#define MLP_TP_PROD_UP 0   /* X . W1r       [N, Fs]  up-projection             [Z 02] */
#define MLP_TP_PROD_DOWN 1 /* H . W2r       [N, D]   down-projection           [Z 02] */
#define MLP_TP_PROD_DH 2   /* dY . W2r^T    [N, Fs]  backward through W2r      [Z 06] */
#define MLP_TP_PROD_DW2 3  /* H^T . dY      [Fs, D]  weight gradient of W2r    [Z 06] */
#define MLP_TP_PROD_DW1 4  /* X^T . dZ      [D, Fs]  weight gradient of W1r    [Z 06] */
#define MLP_TP_PROD_DX 5   /* dZ . W1r^T    [N, D]   input-gradient partial    [Z 06] */

/*
 * The output tile a bf16 product of one rank's shard runs on, on a GPU of compute_units
 * compute units: *tile_rows x *tile_cols results of the product per workgroup; *staged is 1
 * when the shape takes the register-staged kernel (a leading dimension, K, or an m/n-contiguous
 * extent not a multiple of 8) and 0 for the direct-to-LDS kernel. A host query for tuning and
 * tests: it calls no HIP function and launches nothing.
 *   product  one of MLP_TP_PROD_*; N, D, F, T as for the shard calls (N > 0 here).
 *   tile_rows, tile_cols, staged  HOST pointers (each may be NULL if not wanted).
 * Errors: E_SHAPE (sizes as for the shard calls, N == 0, or compute_units < 1),
 * E_INDIVISIBLE, E_DTYPE (product outside the list).
 */
int mlp_tp_shard_tile(int32_t product, int64_t N, int64_t D, int64_t F, int32_t T,
                      int32_t compute_units, int32_t* tile_rows, int32_t* tile_cols,
                      int32_t* staged);

/* Static description of a return code; never NULL. */
const char* mlp_tp_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MLP_TP_H */
