// launch.hpp -- internal host launchers of libmlptp.so (not part of the C ABI).
//
// Every launcher assumes its arguments were validated by the C entry points (non-null,
// 16-byte aligned, positive sizes, N > 0) and only enqueues kernels on `s`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlptp {

// dtype codes as in the C header.
constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// Z = X W1r + b1r; H = phi(Z). X [N, D], W1r [D, Fs], b1r [Fs] or null, Z/H [N, Fs].
// With a workspace `ws` of at least fwd_split_workspace_bytes bytes, a product with too few
// tiles to fill the GPU splits its contraction (fp32 planes in ws, then a streaming pass).
void launch_up_proj(const void* X, const void* W1r, const void* b1r, void* Z, void* H, int64_t N,
                    int64_t D, int64_t Fs, int dtype, int act, hipStream_t s,
                    float* ws = nullptr, int64_t ws_bytes = 0);

// P = H W2r. H [N, Fs], W2r [Fs, D], P [N, D] fp32. Workspace as for launch_up_proj.
void launch_down_proj(const void* H, const void* W2r, float* P, int64_t N, int64_t D, int64_t Fs,
                      int dtype, hipStream_t s, float* ws = nullptr, int64_t ws_bytes = 0);

// Workspace bytes the split forms of the forward's two products use on the current device (the
// larger of the two, since they run one after the other); 0 when neither splits.
int64_t fwd_split_workspace_bytes(int64_t N, int64_t D, int64_t Fs, int dtype);

// P = H W2r + b2 / T: rank r's partial carrying its share of b2. b2 [D] of b2_dtype, nullable.
void launch_down_proj_bias_share(const void* H, const void* W2r, const void* b2, int b2_dtype,
                                 float* P, int64_t N, int64_t D, int64_t Fs, int T, int dtype,
                                 hipStream_t s);

// The output tile (rows, cols) and kernel (staged = 1: register-staged) of a bf16 product of a
// shard (product codes as MLP_TP_PROD_* in the C header) on `cus` compute units. Host only.
void shard_tile(int product, int64_t N, int64_t D, int64_t Fs, int64_t cus, int& rows,
                int& cols, int& staged);

// P += H W2r (fp32 accumulation into an existing partial).
void launch_down_proj_accumulate(const void* H, const void* W2r, float* P, int64_t N, int64_t D,
                                 int64_t Fs, int dtype, hipStream_t s);

// Gated up-projection: G = X Wg, U = X Wu (same columns), H = SiLU(G) * U. X [N, D], Wg/Wu
// [D, Fs], G/U (nullable)/H [N, Fs].
void launch_swiglu_up(const void* X, const void* Wg, const void* Wu, void* G, void* U, void* H,
                      int64_t N, int64_t D, int64_t Fs, int dtype, hipStream_t s);

// dZ = (dY W2r^T) * phi'(Z). dY [N, D], W2r [Fs, D], Z/dZ [N, Fs].
void launch_bwd_dz(const void* dY, const void* W2r, const void* Z, void* dZ, int64_t N, int64_t D,
                   int64_t Fs, int dtype, int act, hipStream_t s);

// Gated backward through the activation: dH = dY W2r^T, then dG = dH * U * SiLU'(G) and
// dU = dH * SiLU(G). dY [N, D], W2r [Fs, D], G/U/dG/dU [N, Fs].
void launch_swiglu_bwd_dgu(const void* dY, const void* W2r, const void* G, const void* U, void* dG,
                           void* dU, int64_t N, int64_t D, int64_t Fs, int dtype, hipStream_t s);

// C [M, N] fp32 = A^T B with A stored [K, M] (lda) and B stored [K, N] (ldb): the weight
// gradients dW2r = H^T dY and dW1r = X^T dZ.
void launch_wgrad(const void* A, const void* B, float* C, int64_t M, int64_t N, int64_t K,
                  int64_t lda, int64_t ldb, int dtype, hipStream_t s);

// dX = dZ W1r^T. dZ [N, Fs], W1r [D, Fs], dX [N, D] fp32.
void launch_dx(const void* dZ, const void* W1r, float* dX, int64_t N, int64_t D, int64_t Fs,
               int dtype, hipStream_t s);

// dX += dZ W1r^T (fp32 accumulation into an existing dX).
void launch_dx_accumulate(const void* dZ, const void* W1r, float* dX, int64_t N, int64_t D,
                          int64_t Fs, int dtype, hipStream_t s);

// Size of the library-owned device buffer of the allocation-free backward (per GPU).
constexpr int64_t kNoallocScratchBytes = int64_t(8) << 20;

// Device address of that buffer on the current device in *ptr (looked up once per device);
// 0, or -1 when HIP cannot provide it. Nothing is allocated.
int noalloc_scratch(void** ptr);

// db1 [Fs] = column sums of dZ [N, Fs], deterministic two-pass through `ws`.
int64_t colsum_workspace_bytes(int64_t N, int64_t Fs);
void launch_colsum(const void* dZ, float* ws, float* db1, int64_t N, int64_t Fs, int dtype,
                   hipStream_t s);

// H = phi(Z + b1r): Z [N, Fs] fp32, b1r [Fs] (dtype, nullable), H [N, Fs] dtype.
void launch_bias_act(const float* Z, const void* b1r, void* H, int64_t N, int64_t Fs, int dtype,
                     int act, hipStream_t s);

// The same over the sum of S fp32 planes [N, Fs] `plane` elements apart (the partials of a split
// contraction, summed in plane order), keeping the pre-activation in Z when non-null.
void launch_split_bias_act(const float* planes, int S, int64_t plane, const void* b1r, void* Z,
                           void* H, int64_t N, int64_t Fs, int dtype, int act, hipStream_t s);

// Y = ((P[0] + P[1]) + ...) + b2 over T fp32 [N, D] partials (P is a host array).
void launch_partial_reduce(const float* const* P, int T, const void* b2, int b2_dtype, float* Y,
                           int64_t N, int64_t D, hipStream_t s);

}  // namespace mlptp
