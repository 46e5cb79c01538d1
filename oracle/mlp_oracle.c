/*
 * mlp_oracle.c -- plain fp64 CPU oracle of the tensor-parallel MLP shard.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's CPU-baseline
 * leg are the only callers. The GPU library never links, loads or calls this code, and the
 * two share no source, header, helper or table.
 *
 * Sources (web pages), cited as [tag section]:
 *   [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
 *   [C] charliedreemur.github.io, "TP:Column / Row Parallel Linear 怎么切? MLP 和 attention 怎么切?"
 *   [U] unpurerationalist.github.io, "LLM Systems 16: Model Parallel Training"
 *   [J] jwzheng96.github.io, "张量并行 TP 与列并行 / 行并行的实现" (Megatron-LM tutorial ch. 7)
 *
 * What is computed (the plain definitions, no blocking, no fusion, no reordering):
 *   shard r of T, Fs = F / T, columns c in [r*Fs, (r+1)*Fs):
 *     Z^(r) = X . W1[:, c] + b1[c]          column-parallel up-projection   [Z 02], [U 3.2]
 *     H^(r) = phi(Z^(r))                     activation, local per shard     [Z 02], [C MLP 为什么先 column 后 row]
 *     P^(r) = H^(r) . W2[c, :]               row-parallel down-projection    [Z 02], [J 7.2]
 *     Y     = ((P^(0) + P^(1)) + ...) + b2   block-tail sum, b2 added once   [Z 02], [Z 05], [U 3.8]
 *     or, b2 split over the ranks: Y = ((P^(0) + b2/T) + (P^(1) + b2/T)) + ...      [Z 05]
 *   backward of shard r for an upstream gradient dY of Y:
 *     dH^(r)  = dY . W2[c, :]^T              no exchange                     [Z 06], [U 3.6.1]
 *     dZ^(r)  = dH^(r) (.) phi'(Z^(r))       through the local activation    [Z 06]
 *     dW2^(r) = H^(r)^T . dY                                                 [Z 06], [U 3.6.1]
 *     dW1^(r) = X^T . dZ^(r)                                                 [U 3.6.1]
 *     db1^(r) = sum over tokens of dZ^(r)
 *     dX^(r)  = dZ^(r) . W1[:, c]^T          a partial; the sum over r is dX  [Z 06 equation], [C 推导 / 关键公式]
 *
 * Readings where the pages are silent (each is restated in the design notes):
 *   - GELU forms. The pages name GELU without a formula; one page's code uses the sigmoid
 *     approximation z / (1 + exp(-1.702 z)) [C 代码]. The oracle offers the exact erf form
 *     z * Phi(z), the tanh form 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) of Hendrycks
 *     and Gimpel (2016), and the sigmoid form.
 *   - ReLU'(0) = 0: the gradient passes only where Z > 0.
 *   - b1 is added before the activation; b2 is added once, after the sum over shards.
 *   - SiLU, named by the gated form without a formula, is z * sigmoid(z) = z / (1 + exp(-z));
 *     the gated form as the page writes it has no biases.
 *   - The token slices of the reduce-scatter layout are contiguous and as equal as possible,
 *     the first ones full: S = ceil(N / T) rows each, the last ones shorter or empty.
 *
 * Layout: every array is fp64, row-major and contiguous. X [N,D]; W1, Wg, Wu [D,F]; b1 [F];
 * W2 [F,D]; b2 [D]; Z, G, U, H, dZ [N,Fs]; P, Y, dX [N,D]; dW1 [D,Fs]; db1 [Fs]; dW2 [Fs,D].
 * Each output element accumulates its reduction index in ascending order. OpenMP only
 * splits independent output rows (or columns) across threads; no element's arithmetic
 * changes with the thread count.
 *
 * Return value of every entry point: 0 on success, -1 on a null required pointer, -2 on a
 * non-positive size or T < 1 or r outside [0,T), -3 when T does not divide F, -4 on an
 * unknown activation code.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum {
    ORACLE_ACT_IDENTITY = 0,
    ORACLE_ACT_RELU = 1,
    ORACLE_ACT_GELU_TANH = 2,
    ORACLE_ACT_GELU_ERF = 3,
    ORACLE_ACT_GELU_SIGMOID = 4,
};

static const double kSqrt2OverPi = 0.79788456080286535587989211986876; /* sqrt(2/pi) */
static const double kInvSqrt2 = 0.70710678118654752440084436210485;    /* 1/sqrt(2) */
static const double kInvSqrt2Pi = 0.39894228040143267793994605993438;  /* 1/sqrt(2 pi) */
static const double kTanhCubic = 0.044715;
static const double kSigmoidScale = 1.702;

static int act_known(int act)
{
    return act >= ORACLE_ACT_IDENTITY && act <= ORACLE_ACT_GELU_SIGMOID;
}

/* phi(z): the elementwise activation applied to each shard's own columns [Z 02]. */
double oracle_act(int act, double z)
{
    switch (act) {
    case ORACLE_ACT_IDENTITY:
        return z;
    case ORACLE_ACT_RELU:
        return z > 0.0 ? z : 0.0;
    case ORACLE_ACT_GELU_TANH: {
        double u = kSqrt2OverPi * (z + kTanhCubic * z * z * z);
        return 0.5 * z * (1.0 + tanh(u));
    }
    case ORACLE_ACT_GELU_ERF:
        return 0.5 * z * (1.0 + erf(z * kInvSqrt2));
    case ORACLE_ACT_GELU_SIGMOID:
        return z / (1.0 + exp(-kSigmoidScale * z));
    default:
        return NAN;
    }
}

/* phi'(z), by differentiating each form above by hand. */
double oracle_act_deriv(int act, double z)
{
    switch (act) {
    case ORACLE_ACT_IDENTITY:
        return 1.0;
    case ORACLE_ACT_RELU:
        return z > 0.0 ? 1.0 : 0.0;
    case ORACLE_ACT_GELU_TANH: {
        /* phi = 0.5 z (1 + t), t = tanh(u), u = c (z + a z^3)
           phi' = 0.5 (1 + t) + 0.5 z (1 - t^2) c (1 + 3 a z^2) */
        double u = kSqrt2OverPi * (z + kTanhCubic * z * z * z);
        double t = tanh(u);
        double du = kSqrt2OverPi * (1.0 + 3.0 * kTanhCubic * z * z);
        return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * du;
    }
    case ORACLE_ACT_GELU_ERF: {
        /* phi = z Phi(z)  ->  phi' = Phi(z) + z pdf(z) */
        double cdf = 0.5 * (1.0 + erf(z * kInvSqrt2));
        double pdf = kInvSqrt2Pi * exp(-0.5 * z * z);
        return cdf + z * pdf;
    }
    case ORACLE_ACT_GELU_SIGMOID: {
        /* phi = z s(k z)  ->  phi' = s + k z s (1 - s) */
        double s = 1.0 / (1.0 + exp(-kSigmoidScale * z));
        return s + kSigmoidScale * z * s * (1.0 - s);
    }
    default:
        return NAN;
    }
}

int oracle_act_vec(int act, const double* z, double* out, int64_t n)
{
    if (!act_known(act)) return -4;
    if (n < 0) return -2;
    if (n > 0 && (!z || !out)) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_act(act, z[i]);
    return 0;
}

int oracle_act_deriv_vec(int act, const double* z, double* out, int64_t n)
{
    if (!act_known(act)) return -4;
    if (n < 0) return -2;
    if (n > 0 && (!z || !out)) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_act_deriv(act, z[i]);
    return 0;
}

static int check_shard_args(int64_t N, int64_t D, int64_t F, int32_t T, int32_t r, int act)
{
    if (N <= 0 || D <= 0 || F <= 0 || T < 1 || r < 0 || r >= T) return -2;
    if (F % T != 0) return -3; /* the shard count must divide F [U 3.8] */
    if (!act_known(act)) return -4;
    return 0;
}

/* Z^(r)[n,j] = sum_k X[n,k] W1[k, r Fs + j] + b1[r Fs + j];  H^(r) = phi(Z^(r)).
   Column slice of W1 and of b1 for shard r [Z 02], [Z 05: the up-projection bias splits with
   the columns]. */
static void up_projection(const double* X, const double* W1, const double* b1, int64_t N,
                          int64_t D, int64_t F, int64_t Fs, int64_t c0, int act, double* Z,
                          double* H)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double* z = Z + n * Fs;
        for (int64_t j = 0; j < Fs; ++j) z[j] = 0.0;
        /* k outermost over a row of W1: each z[j] still sums k = 0, 1, ..., D-1 in order. */
        for (int64_t k = 0; k < D; ++k) {
            double x = X[n * D + k];
            const double* w = W1 + k * F + c0;
            for (int64_t j = 0; j < Fs; ++j) z[j] += x * w[j];
        }
        if (b1)
            for (int64_t j = 0; j < Fs; ++j) z[j] += b1[c0 + j];
        if (H)
            for (int64_t j = 0; j < Fs; ++j) H[n * Fs + j] = oracle_act(act, z[j]);
    }
}

/* P^(r)[n,d] = sum_j H^(r)[n,j] W2[r Fs + j, d]: row slice of W2 [Z 02], [J 7.2]. */
static void down_projection(const double* H, const double* W2, int64_t N, int64_t D,
                            int64_t Fs, int64_t c0, double* P)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double* p = P + n * D;
        for (int64_t d = 0; d < D; ++d) p[d] = 0.0;
        for (int64_t j = 0; j < Fs; ++j) {
            double h = H[n * Fs + j];
            const double* w = W2 + (c0 + j) * D;
            for (int64_t d = 0; d < D; ++d) p[d] += h * w[d];
        }
    }
}

/*
 * One rank's forward shard: column-parallel up-projection with its b1 slice, local
 * activation, row-parallel down-projection to a full-shape partial with NO b2 [Z 02], [Z 05],
 * [U 3.8]. W1, b1 and W2 are the FULL weights; the oracle slices shard r itself.
 * Z, H: [N, F/T] (Z may be NULL); P: [N, D]. b1 may be NULL (no bias).
 */
int oracle_shard_fwd(const double* X, const double* W1, const double* b1, const double* W2,
                     int64_t N, int64_t D, int64_t F, int32_t T, int32_t r, int act, double* Z,
                     double* H, double* P)
{
    int rc = check_shard_args(N, D, F, T, r, act);
    if (rc) return rc;
    if (!X || !W1 || !W2 || !H || !P) return -1;
    int64_t Fs = F / T, c0 = (int64_t)r * Fs;
    double* z = Z ? Z : (double*)malloc((size_t)(N * Fs) * sizeof(double));
    if (!z) return -1;
    up_projection(X, W1, b1, N, D, F, Fs, c0, act, z, H);
    down_projection(H, W2, N, D, Fs, c0, P);
    if (!Z) free(z);
    return 0;
}

/*
 * Block tail: Y = (((P^(0) + P^(1)) + ...) + P^(T-1)) + b2, shards summed in rank order and
 * b2 added exactly once after the sum [Z 02], [Z 05], [U 3.8]. P is an array of T pointers
 * to [N, D] partials; b2 may be NULL (e.g. the sum of input-gradient partials [Z 06]).
 */
int oracle_partial_sum(const double* const* P, int32_t T, const double* b2, int64_t N,
                       int64_t D, double* Y)
{
    if (N <= 0 || D <= 0 || T < 1) return -2;
    if (!P || !Y) return -1;
    for (int32_t r = 0; r < T; ++r)
        if (!P[r]) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t d = 0; d < D; ++d) {
            double s = P[0][n * D + d];
            for (int32_t r = 1; r < T; ++r) s += P[r][n * D + d];
            if (b2) s += b2[d];
            Y[n * D + d] = s;
        }
    }
    return 0;
}

/*
 * Block tail with b2 split over the ranks, the alternative [Z 05] offers to adding b2 once:
 * every rank adds b2 / T to its own partial before the exchange, and the exchange sums those:
 *     Y = ((P^(0) + b2/T) + (P^(1) + b2/T)) + ...
 * over the nparts partials given (nparts = T for the whole tail; nparts = 1 gives one rank's
 * contribution P^(r) + b2/T). Each contribution is formed first, then the contributions are
 * summed in rank order. b2 may be NULL (then this is the plain sum).
 */
int oracle_partial_sum_bias_share(const double* const* P, int32_t nparts, int32_t T,
                                  const double* b2, int64_t N, int64_t D, double* Y)
{
    if (N <= 0 || D <= 0 || T < 1 || nparts < 1) return -2;
    if (!P || !Y) return -1;
    for (int32_t r = 0; r < nparts; ++r)
        if (!P[r]) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t d = 0; d < D; ++d) {
            const double share = b2 ? b2[d] / (double)T : 0.0;
            double s = P[0][n * D + d] + share;
            for (int32_t r = 1; r < nparts; ++r) s += P[r][n * D + d] + share;
            Y[n * D + d] = s;
        }
    }
    return 0;
}

/* The whole block as T shards: every shard forward in rank order, then the block tail. */
int oracle_block_fwd(const double* X, const double* W1, const double* b1, const double* W2,
                     const double* b2, int64_t N, int64_t D, int64_t F, int32_t T, int act,
                     double* Y)
{
    int rc = check_shard_args(N, D, F, T, 0, act);
    if (rc) return rc;
    if (!X || !W1 || !W2 || !Y) return -1;
    int64_t Fs = F / T;
    double* H = (double*)malloc((size_t)(N * Fs) * sizeof(double));
    double** P = (double**)calloc((size_t)T, sizeof(double*));
    if (!H || !P) {
        free(H);
        free(P);
        return -1;
    }
    rc = 0;
    for (int32_t r = 0; r < T && rc == 0; ++r) {
        P[r] = (double*)malloc((size_t)(N * D) * sizeof(double));
        if (!P[r]) rc = -1;
        else rc = oracle_shard_fwd(X, W1, b1, W2, N, D, F, T, r, act, NULL, H, P[r]);
    }
    if (rc == 0) rc = oracle_partial_sum((const double* const*)P, T, b2, N, D, Y);
    for (int32_t r = 0; r < T; ++r) free(P[r]);
    free(P);
    free(H);
    return rc;
}

/* The unsharded MLP: Y = phi(X W1 + b1) W2 + b2 [Z 01], [C 推导 / 关键公式]. */
int oracle_dense_fwd(const double* X, const double* W1, const double* b1, const double* W2,
                     const double* b2, int64_t N, int64_t D, int64_t F, int act, double* Y)
{
    int rc = check_shard_args(N, D, F, 1, 0, act);
    if (rc) return rc;
    if (!X || !W1 || !W2 || !Y) return -1;
    double* A = (double*)malloc((size_t)(N * F) * sizeof(double));
    double* H = (double*)malloc((size_t)(N * F) * sizeof(double));
    if (!A || !H) {
        free(A);
        free(H);
        return -1;
    }
    up_projection(X, W1, b1, N, D, F, F, 0, act, A, H);
    down_projection(H, W2, N, D, F, 0, Y);
    if (b2)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t d = 0; d < D; ++d) Y[n * D + d] += b2[d];
    free(A);
    free(H);
    return 0;
}

/*
 * Backward of shard r for the upstream gradient dY [N, D] of the block output Y [Z 06],
 * [U 3.6.1]. Recomputes Z^(r) and H^(r) from X and the weights in fp64. Outputs:
 *   dZ [N,Fs], dW1r [D,Fs], db1r [Fs] (may be NULL), dW2r [Fs,D], dXr [N,D] (the shard's
 *   partial of dX; the sum over shards is the input gradient [Z 06 equation]).
 * Any output pointer except dZ may be NULL to skip that output.
 */
int oracle_shard_bwd(const double* X, const double* W1, const double* b1, const double* W2,
                     const double* dY, int64_t N, int64_t D, int64_t F, int32_t T, int32_t r,
                     int act, double* dZ, double* dW1r, double* db1r, double* dW2r, double* dXr)
{
    int rc = check_shard_args(N, D, F, T, r, act);
    if (rc) return rc;
    if (!X || !W1 || !W2 || !dY || !dZ) return -1;
    int64_t Fs = F / T, c0 = (int64_t)r * Fs;
    double* Z = (double*)malloc((size_t)(N * Fs) * sizeof(double));
    double* H = (double*)malloc((size_t)(N * Fs) * sizeof(double));
    if (!Z || !H) {
        free(Z);
        free(H);
        return -1;
    }
    up_projection(X, W1, b1, N, D, F, Fs, c0, act, Z, H);

    /* dH[n,j] = sum_d dY[n,d] W2[c0+j, d];  dZ = dH * phi'(Z). */
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < Fs; ++j) {
            const double* w = W2 + (c0 + j) * D;
            double s = 0.0;
            for (int64_t d = 0; d < D; ++d) s += dY[n * D + d] * w[d];
            dZ[n * Fs + j] = s * oracle_act_deriv(act, Z[n * Fs + j]);
        }
    }

    /* dW2r[j,d] = sum_n H[n,j] dY[n,d]  (row j of the shard's W2 gradient). */
    if (dW2r) {
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < Fs; ++j) {
            double* g = dW2r + j * D;
            for (int64_t d = 0; d < D; ++d) g[d] = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double h = H[n * Fs + j];
                const double* dy = dY + n * D;
                for (int64_t d = 0; d < D; ++d) g[d] += h * dy[d];
            }
        }
    }

    /* dW1r[k,j] = sum_n X[n,k] dZ[n,j]. */
    if (dW1r) {
#pragma omp parallel for schedule(static)
        for (int64_t k = 0; k < D; ++k) {
            double* g = dW1r + k * Fs;
            for (int64_t j = 0; j < Fs; ++j) g[j] = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double x = X[n * D + k];
                const double* dz = dZ + n * Fs;
                for (int64_t j = 0; j < Fs; ++j) g[j] += x * dz[j];
            }
        }
    }

    /* db1r[j] = sum_n dZ[n,j]. */
    if (db1r) {
        for (int64_t j = 0; j < Fs; ++j) db1r[j] = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t j = 0; j < Fs; ++j) db1r[j] += dZ[n * Fs + j];
    }

    /* dXr[n,k] = sum_j dZ[n,j] W1[k, c0+j]. */
    if (dXr) {
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < D; ++k) {
                const double* w = W1 + k * F + c0;
                double s = 0.0;
                for (int64_t j = 0; j < Fs; ++j) s += dZ[n * Fs + j] * w[j];
                dXr[n * D + k] = s;
            }
        }
    }
    free(Z);
    free(H);
    return 0;
}

/*
 * Backward of the unsharded MLP for the upstream gradient dY: the full parameter gradients
 * dW1 [D,F], db1 [F], dW2 [F,D], db2 [D] and the input gradient dX [N,D]. This is the shard
 * backward with T = 1 plus db2 = sum over tokens of dY. Any output may be NULL.
 */
int oracle_dense_bwd(const double* X, const double* W1, const double* b1, const double* W2,
                     const double* dY, int64_t N, int64_t D, int64_t F, int act, double* dW1,
                     double* db1, double* dW2, double* db2, double* dX)
{
    int rc = check_shard_args(N, D, F, 1, 0, act);
    if (rc) return rc;
    if (!dY) return -1;
    double* dZ = (double*)malloc((size_t)(N * F) * sizeof(double));
    if (!dZ) return -1;
    rc = oracle_shard_bwd(X, W1, b1, W2, dY, N, D, F, 1, 0, act, dZ, dW1, db1, dW2, dX);
    free(dZ);
    if (rc) return rc;
    if (db2) {
        for (int64_t d = 0; d < D; ++d) db2[d] = 0.0;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t d = 0; d < D; ++d) db2[d] += dY[n * D + d];
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* Reduce-scatter layout of the block tail [Z 04].                                           */

/* First row and row count of token slice r: S = ceil(N / T) rows per slice. */
int oracle_token_slice(int64_t N, int32_t T, int32_t r, int64_t* row0, int64_t* rows)
{
    if (N < 0 || T < 1 || r < 0 || r >= T) return -2;
    if (!row0 || !rows) return -1;
    int64_t S = (N + T - 1) / T;
    int64_t a = (int64_t)r * S, b = a + S;
    if (a > N) a = N;
    if (b > N) b = N;
    *row0 = a;
    *rows = b - a;
    return 0;
}

/*
 * Token slice r of the block tail: Yr[i,d] = (sum_s P^(s)[row0 + i, d]) + b2[d] for the rows of
 * slice r, shards summed in rank order, b2 added once [Z 04], [Z 05]. Yr is [rows, D].
 */
int oracle_partial_reduce_scatter(const double* const* P, int32_t T, int32_t r,
                                  const double* b2, int64_t N, int64_t D, double* Yr)
{
    if (N <= 0 || D <= 0 || T < 1 || r < 0 || r >= T) return -2;
    if (!P || !Yr) return -1;
    for (int32_t s = 0; s < T; ++s)
        if (!P[s]) return -1;
    int64_t row0, rows;
    oracle_token_slice(N, T, r, &row0, &rows);
    for (int64_t i = 0; i < rows; ++i) {
        int64_t n = row0 + i;
        for (int64_t d = 0; d < D; ++d) {
            double v = P[0][n * D + d];
            for (int32_t s = 1; s < T; ++s) v += P[s][n * D + d];
            if (b2) v += b2[d];
            Yr[i * D + d] = v;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* Gated (SwiGLU) MLP [Z 08].                                                                */

/* SiLU(z) = z * sigmoid(z). */
double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* SiLU'(z) = s (1 + z (1 - s)), s = sigmoid(z), by the product rule. */
double oracle_silu_deriv(double z)
{
    double s = 1.0 / (1.0 + exp(-z));
    return s * (1.0 + z * (1.0 - s));
}

int oracle_silu_vec(const double* z, double* out, int64_t n, int deriv)
{
    if (!z || !out) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = deriv ? oracle_silu_deriv(z[i]) : oracle_silu(z[i]);
    return 0;
}

/* A[n,j] = sum_k X[n,k] W[k, c0 + j], k ascending: one column slice of a [D,F] weight. */
static void column_slice_product(const double* X, const double* W, int64_t N, int64_t D,
                                 int64_t F, int64_t Fs, int64_t c0, double* A)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double* a = A + n * Fs;
        for (int64_t j = 0; j < Fs; ++j) a[j] = 0.0;
        for (int64_t k = 0; k < D; ++k) {
            double x = X[n * D + k];
            const double* w = W + k * F + c0;
            for (int64_t j = 0; j < Fs; ++j) a[j] += x * w[j];
        }
    }
}

/*
 * One rank's gated shard: gate and up projections with the SAME column slice of Wg and Wu,
 * H = SiLU(G) (.) U locally, then the row slice of W2 to a full-shape partial [Z 08]. Wg, Wu,
 * W2 are the FULL weights. G, U may be NULL; H [N,Fs] and P [N,D] are required.
 */
int oracle_swiglu_shard_fwd(const double* X, const double* Wg, const double* Wu,
                            const double* W2, int64_t N, int64_t D, int64_t F, int32_t T,
                            int32_t r, double* G, double* U, double* H, double* P)
{
    int rc = check_shard_args(N, D, F, T, r, 0);
    if (rc) return rc;
    if (!X || !Wg || !Wu || !W2 || !H || !P) return -1;
    int64_t Fs = F / T, c0 = (int64_t)r * Fs;
    double* g = G ? G : (double*)malloc((size_t)(N * Fs) * sizeof(double));
    double* u = U ? U : (double*)malloc((size_t)(N * Fs) * sizeof(double));
    if (!g || !u) {
        if (!G) free(g);
        if (!U) free(u);
        return -1;
    }
    column_slice_product(X, Wg, N, D, F, Fs, c0, g);
    column_slice_product(X, Wu, N, D, F, Fs, c0, u);
    for (int64_t i = 0; i < N * Fs; ++i) H[i] = oracle_silu(g[i]) * u[i];
    down_projection(H, W2, N, D, Fs, c0, P);
    if (!G) free(g);
    if (!U) free(u);
    return 0;
}

/* The unsharded gated MLP: Y = (SiLU(X Wg) (.) (X Wu)) W2 [Z 08]. */
int oracle_swiglu_dense_fwd(const double* X, const double* Wg, const double* Wu,
                            const double* W2, int64_t N, int64_t D, int64_t F, double* Y)
{
    int rc = check_shard_args(N, D, F, 1, 0, 0);
    if (rc) return rc;
    if (!X || !Wg || !Wu || !W2 || !Y) return -1;
    double* H = (double*)malloc((size_t)(N * F) * sizeof(double));
    if (!H) return -1;
    rc = oracle_swiglu_shard_fwd(X, Wg, Wu, W2, N, D, F, 1, 0, NULL, NULL, H, Y);
    free(H);
    return rc;
}

/*
 * Backward of the gated shard r for dY [N,D]. Recomputes G, U and H in fp64. Outputs (any
 * may be NULL except dG and dU): dG, dU [N,Fs]; dWg, dWu [D,Fs]; dW2r [Fs,D]; dXr [N,D].
 */
int oracle_swiglu_shard_bwd(const double* X, const double* Wg, const double* Wu,
                            const double* W2, const double* dY, int64_t N, int64_t D, int64_t F,
                            int32_t T, int32_t r, double* dG, double* dU, double* dWg,
                            double* dWu, double* dW2r, double* dXr)
{
    int rc = check_shard_args(N, D, F, T, r, 0);
    if (rc) return rc;
    if (!X || !Wg || !Wu || !W2 || !dY || !dG || !dU) return -1;
    int64_t Fs = F / T, c0 = (int64_t)r * Fs;
    double* G = (double*)malloc((size_t)(N * Fs) * sizeof(double));
    double* U = (double*)malloc((size_t)(N * Fs) * sizeof(double));
    double* H = (double*)malloc((size_t)(N * Fs) * sizeof(double));
    if (!G || !U || !H) {
        free(G);
        free(U);
        free(H);
        return -1;
    }
    column_slice_product(X, Wg, N, D, F, Fs, c0, G);
    column_slice_product(X, Wu, N, D, F, Fs, c0, U);
    for (int64_t i = 0; i < N * Fs; ++i) H[i] = oracle_silu(G[i]) * U[i];

    /* dH[n,j] = sum_d dY[n,d] W2[c0+j, d]; then the product rule through H = SiLU(G) U. */
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < Fs; ++j) {
            const double* w = W2 + (c0 + j) * D;
            double s = 0.0;
            for (int64_t d = 0; d < D; ++d) s += dY[n * D + d] * w[d];
            double g = G[n * Fs + j], u = U[n * Fs + j];
            dG[n * Fs + j] = s * u * oracle_silu_deriv(g);
            dU[n * Fs + j] = s * oracle_silu(g);
        }
    }

    /* dW2r[j,d] = sum_n H[n,j] dY[n,d]. */
    if (dW2r) {
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < Fs; ++j) {
            double* g = dW2r + j * D;
            for (int64_t d = 0; d < D; ++d) g[d] = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double h = H[n * Fs + j];
                for (int64_t d = 0; d < D; ++d) g[d] += h * dY[n * D + d];
            }
        }
    }

    /* dWg[k,j] = sum_n X[n,k] dG[n,j];  dWu[k,j] = sum_n X[n,k] dU[n,j]. */
    for (int pass = 0; pass < 2; ++pass) {
        double* out = pass == 0 ? dWg : dWu;
        const double* dA = pass == 0 ? dG : dU;
        if (!out) continue;
#pragma omp parallel for schedule(static)
        for (int64_t k = 0; k < D; ++k) {
            double* g = out + k * Fs;
            for (int64_t j = 0; j < Fs; ++j) g[j] = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double x = X[n * D + k];
                for (int64_t j = 0; j < Fs; ++j) g[j] += x * dA[n * Fs + j];
            }
        }
    }

    /* dXr[n,k] = sum_j dG[n,j] Wg[k,c0+j] + sum_j dU[n,j] Wu[k,c0+j]. */
    if (dXr) {
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < D; ++k) {
                const double* wg = Wg + k * F + c0;
                const double* wu = Wu + k * F + c0;
                double s = 0.0;
                for (int64_t j = 0; j < Fs; ++j) s += dG[n * Fs + j] * wg[j];
                for (int64_t j = 0; j < Fs; ++j) s += dU[n * Fs + j] * wu[j];
                dXr[n * D + k] = s;
            }
        }
    }
    free(G);
    free(U);
    free(H);
    return 0;
}

/* Threads an OpenMP region in this library would use (reported beside the CPU timing). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
