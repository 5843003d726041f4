/*
 * Plain fp64 CPU oracle for the Gaussian Mixture Attention (GMA) forward mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or constant with the HIP kernels.
 *
 * Source: "Gaussian Mixture Attention: Linear-Time Sequence Mixing via
 * Probabilistic Latent Routing" (Huang, Raza; arXiv 2606.18283), as summarised on
 * gist.science (ja/de pages, section "Core mechanism") and in the arXiv abstract.
 *
 * What is computed, per batch element b and head h (parameters are per head):
 *   var_kd   = softplus(var_raw_kd) + var_floor            (Core mechanism 3:
 *                                                          softplus keeps variances valid)
 *   log pi_k = p_k - logsumexp_j p_j                       (Core mechanism 3: softmax priors)
 *   l_k(x)   = log pi_k + log N(x; mu_k, diag var_k)       (Core mechanism 1: standard
 *                                                          GMM posterior p(z=k|x))
 *   gamma_k  = exp(l_k - max l) / sum_j exp(l_j - max l)
 *   Bidirectional (Core mechanism 2, write/read equations):
 *     Vt = Gamma_K^T V,  Z = Gamma_K^T 1,  O = Gamma_Q Vt / (Gamma_Q Z + eps)
 *   Causal (Core mechanism 3): prefix sums of the memory and the normaliser, so that
 *     O_i uses only positions j <= i (inclusive of i).
 *   Cross (the German page's closing paragraph names cross-attention as future work):
 *     the bidirectional equations with Gamma_K, V over Nk key rows and Gamma_Q, O over
 *     Nq query rows; Nk = Nq is self-mixing.
 *   Decode (Core mechanism 3 read as a recurrence): the causal memory after positions
 *     0..t-1 is the state [S | z] (K x (d_v+1)); one step adds gamma_K,t (x) [v_t | 1] and
 *     reads O_t = gamma_Q,t S / (gamma_Q,t . z + eps), which is row t of the causal forward.
 *     The memory of a prefix is the write phase over its positions.
 *   Backward: the gradients of a loss with respect to every input (the pages train the
 *     mixture end to end by backpropagation), the chain rule of the above written out.
 *   Responsibility statistics (the pages' interpretability analysis of learned
 *     responsibilities: components used, usage entropy, hard assignments): per head, over
 *     the rows of the batch, hard assignments (argmax), their histogram, the soft usage
 *     sum of gamma, the number of components used and the normalised usage entropy.
 *
 * Readings of points the pages leave open: the log-density keeps every constant
 * (log 2 pi and the prior's log-sum-exp); eps is added once per output row after
 * the product Gamma_Q Z; softplus is the exact log1p(exp(r)) with no linear
 * threshold; the same K Gaussians serve queries and keys of one head.
 *
 * Everything is double precision, sums run in ascending index order, and the loops
 * follow the definitions directly: no blocking, fusion or reordering.  OpenMP only
 * spreads independent (b, h) slices and independent rows over threads.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)
#define ORACLE_NO_MEM (-2)

static const double LOG_2PI = 1.8378770664093454835606594728112; /* log(2*pi) */

/* softplus(r) = log(1 + e^r), written in the overflow-free form max(r,0)+log1p(e^-|r|). */
static double softplus(double r) { return fmax(r, 0.0) + log1p(exp(-fabs(r))); }

int gma_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Log joint l_k(x_i) = log pi_k + log N(x_i; mu_k, diag(var_k)) for the N rows of x.
 *   x            [N, d]   routing vectors of one head
 *   mu, var_raw  [K, d]   parameters of that head
 *   prior_logits [K]
 *   out          [N, K]
 */
int gma_oracle_log_joint(const double* x, int N, int d, const double* mu,
                         const double* var_raw, const double* prior_logits, int K,
                         double var_floor, double* out) {
    if (!x || !mu || !var_raw || !prior_logits || !out || N < 0 || d < 1 || K < 1)
        return ORACLE_BAD_ARG;
    double* var = (double*)malloc(sizeof(double) * (size_t)K * d);
    double* logvar = (double*)malloc(sizeof(double) * (size_t)K * d);
    double* logpi = (double*)malloc(sizeof(double) * (size_t)K);
    if (!var || !logvar || !logpi) { free(var); free(logvar); free(logpi); return ORACLE_NO_MEM; }

    for (int k = 0; k < K; ++k)
        for (int j = 0; j < d; ++j) {
            var[(size_t)k * d + j] = softplus(var_raw[(size_t)k * d + j]) + var_floor;
            logvar[(size_t)k * d + j] = log(var[(size_t)k * d + j]);
        }

    /* log softmax of the prior logits */
    double pmax = prior_logits[0];
    for (int k = 1; k < K; ++k) pmax = fmax(pmax, prior_logits[k]);
    double psum = 0.0;
    for (int k = 0; k < K; ++k) psum += exp(prior_logits[k] - pmax);
    double lse = pmax + log(psum);
    for (int k = 0; k < K; ++k) logpi[k] = prior_logits[k] - lse;

#pragma omp parallel for schedule(static)
    for (int i = 0; i < N; ++i) {
        const double* xi = x + (size_t)i * d;
        for (int k = 0; k < K; ++k) {
            const double* mk = mu + (size_t)k * d;
            const double* vk = var + (size_t)k * d;
            const double* lvk = logvar + (size_t)k * d;
            double quad = 0.0;
            for (int j = 0; j < d; ++j) {
                double diff = xi[j] - mk[j];
                quad += LOG_2PI + lvk[j] + diff * diff / vk[j];
            }
            out[(size_t)i * K + k] = logpi[k] - 0.5 * quad;
        }
    }
    free(var);
    free(logvar);
    free(logpi);
    return ORACLE_OK;
}

/* Posterior responsibilities gamma [N, K] = row-wise softmax of the log joint. */
int gma_oracle_responsibilities(const double* x, int N, int d, const double* mu,
                                const double* var_raw, const double* prior_logits, int K,
                                double var_floor, double* gamma) {
    int st = gma_oracle_log_joint(x, N, d, mu, var_raw, prior_logits, K, var_floor, gamma);
    if (st != ORACLE_OK) return st;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < N; ++i) {
        double* row = gamma + (size_t)i * K;
        double m = row[0];
        for (int k = 1; k < K; ++k) m = fmax(m, row[k]);
        double s = 0.0;
        for (int k = 0; k < K; ++k) { row[k] = exp(row[k] - m); s += row[k]; }
        for (int k = 0; k < K; ++k) row[k] /= s;
    }
    return ORACLE_OK;
}

/* Bidirectional write then read for one head: the memory Vt = Gamma_K^T V, Z = Gamma_K^T 1
 * over the Nk key rows, read by the Nq query rows.  gq [Nq, K], gk [Nk, K], v [Nk, dv]
 * -> o [Nq, dv].  Self-mixing is Nq = Nk with queries and keys of the same positions. */
static int mix_bidirectional(const double* gq, int Nq, const double* gk, const double* v, int Nk, int K,
                             int dv, double eps, double* o) {
    double* vt = (double*)calloc((size_t)K * dv, sizeof(double)); /* Gamma_K^T V */
    double* z = (double*)calloc((size_t)K, sizeof(double));       /* Gamma_K^T 1 */
    if (!vt || !z) { free(vt); free(z); return ORACLE_NO_MEM; }
    for (int j = 0; j < Nk; ++j)
        for (int k = 0; k < K; ++k) {
            double g = gk[(size_t)j * K + k];
            z[k] += g;
            for (int c = 0; c < dv; ++c) vt[(size_t)k * dv + c] += g * v[(size_t)j * dv + c];
        }
    for (int i = 0; i < Nq; ++i) {
        double den = 0.0;
        for (int k = 0; k < K; ++k) den += gq[(size_t)i * K + k] * z[k];
        for (int c = 0; c < dv; ++c) {
            double num = 0.0;
            for (int k = 0; k < K; ++k) num += gq[(size_t)i * K + k] * vt[(size_t)k * dv + c];
            o[(size_t)i * dv + c] = num / (den + eps);
        }
    }
    free(vt);
    free(z);
    return ORACLE_OK;
}

/* Causal variant for one head: inclusive prefix sums S_i = sum_{j<=i} gk_j v_j^T,
 * z_i = sum_{j<=i} gk_j, and O_i = gq_i S_i / (gq_i . z_i + eps). */
static int mix_causal(const double* gq, const double* gk, const double* v, int N, int K, int dv,
                      double eps, double* o) {
    double* s = (double*)calloc((size_t)K * dv, sizeof(double));
    double* z = (double*)calloc((size_t)K, sizeof(double));
    if (!s || !z) { free(s); free(z); return ORACLE_NO_MEM; }
    for (int i = 0; i < N; ++i) {
        for (int k = 0; k < K; ++k) {
            double g = gk[(size_t)i * K + k];
            z[k] += g;
            for (int c = 0; c < dv; ++c) s[(size_t)k * dv + c] += g * v[(size_t)i * dv + c];
        }
        double den = 0.0;
        for (int k = 0; k < K; ++k) den += gq[(size_t)i * K + k] * z[k];
        for (int c = 0; c < dv; ++c) {
            double num = 0.0;
            for (int k = 0; k < K; ++k) num += gq[(size_t)i * K + k] * s[(size_t)k * dv + c];
            o[(size_t)i * dv + c] = num / (den + eps);
        }
    }
    free(s);
    free(z);
    return ORACLE_OK;
}

/* One forward over all (b, h) slices with Nq query rows and Nk key rows (causal needs
 * Nq == Nk).  Slices are independent and run in parallel; inside a slice everything is
 * sequential in index order. */
static int forward_slices(const double* qr, const double* kr, const double* v, const double* mu,
                          const double* var_raw, const double* prior_logits, int B, int H, int Nq, int Nk,
                          int d_r, int d_v, int K, int causal, double eps, double var_floor, double* out,
                          double* gamma_q, double* gamma_k) {
    const size_t nqk = (size_t)Nq * K, nkk = (size_t)Nk * K;
    int status = ORACLE_OK;

#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; ++bh) {
        const int h = bh % H;
        double* gq = gamma_q ? gamma_q + (size_t)bh * nqk : (double*)malloc(sizeof(double) * (nqk ? nqk : 1));
        double* gk = gamma_k ? gamma_k + (size_t)bh * nkk : (double*)malloc(sizeof(double) * (nkk ? nkk : 1));
        int st = (gq && gk) ? ORACLE_OK : ORACLE_NO_MEM;
        const double* mu_h = mu + (size_t)h * K * d_r;
        const double* vr_h = var_raw + (size_t)h * K * d_r;
        const double* p_h = prior_logits + (size_t)h * K;
        const double* q_bh = qr + (size_t)bh * Nq * d_r;
        const double* k_bh = kr + (size_t)bh * Nk * d_r;
        const double* v_bh = v + (size_t)bh * Nk * d_v;
        double* o_bh = out + (size_t)bh * Nq * d_v;
        if (st == ORACLE_OK)
            st = gma_oracle_responsibilities(q_bh, Nq, d_r, mu_h, vr_h, p_h, K, var_floor, gq);
        if (st == ORACLE_OK)
            st = gma_oracle_responsibilities(k_bh, Nk, d_r, mu_h, vr_h, p_h, K, var_floor, gk);
        if (st == ORACLE_OK)
            st = causal ? mix_causal(gq, gk, v_bh, Nq, K, d_v, eps, o_bh)
                        : mix_bidirectional(gq, Nq, gk, v_bh, Nk, K, d_v, eps, o_bh);
        if (!gamma_q) free(gq);
        if (!gamma_k) free(gk);
        if (st != ORACLE_OK) {
#pragma omp critical
            status = st;
        }
    }
    return status;
}

/*
 * Full forward.  All arrays are contiguous double:
 *   qr, kr [B,H,N,d_r]; v, out [B,H,N,d_v]; mu, var_raw [H,K,d_r]; prior_logits [H,K];
 *   gamma_q, gamma_k (each nullable) [B,H,N,K].
 */
int gma_oracle_forward(const double* qr, const double* kr, const double* v, const double* mu,
                       const double* var_raw, const double* prior_logits, int B, int H, int N,
                       int d_r, int d_v, int K, int causal, double eps, double var_floor,
                       double* out, double* gamma_q, double* gamma_k) {
    if (!qr || !kr || !v || !mu || !var_raw || !prior_logits || !out) return ORACLE_BAD_ARG;
    if (B < 1 || H < 1 || N < 0 || d_r < 1 || d_v < 1 || K < 1) return ORACLE_BAD_ARG;
    if (causal != 0 && causal != 1) return ORACLE_BAD_ARG;
    return forward_slices(qr, kr, v, mu, var_raw, prior_logits, B, H, N, N, d_r, d_v, K, causal, eps,
                          var_floor, out, gamma_q, gamma_k);
}

/*
 * Cross variant (bidirectional): queries and keys of different lengths, the memory formed
 * over the Nk key rows of each (b, h) and read by its Nq query rows.
 *   qr [B,H,Nq,d_r]; kr [B,H,Nk,d_r]; v [B,H,Nk,d_v]; out [B,H,Nq,d_v];
 *   gamma_q [B,H,Nq,K], gamma_k [B,H,Nk,K] (each nullable).
 */
int gma_oracle_forward_cross(const double* qr, const double* kr, const double* v, const double* mu,
                             const double* var_raw, const double* prior_logits, int B, int H, int Nq, int Nk,
                             int d_r, int d_v, int K, double eps, double var_floor, double* out,
                             double* gamma_q, double* gamma_k) {
    if (!qr || !kr || !v || !mu || !var_raw || !prior_logits || !out) return ORACLE_BAD_ARG;
    if (B < 1 || H < 1 || Nq < 0 || Nk < 0 || d_r < 1 || d_v < 1 || K < 1) return ORACLE_BAD_ARG;
    return forward_slices(qr, kr, v, mu, var_raw, prior_logits, B, H, Nq, Nk, d_r, d_v, K, 0, eps, var_floor,
                          out, gamma_q, gamma_k);
}

/*
 * Memory [S | z] of the first N positions of every (b, h): S[k][c] = sum_j gamma_K[j][k] v[j][c],
 * z[k] = sum_j gamma_K[j][k], summed in position order.
 *   kr [B,H,N,d_r]; v [B,H,N,d_v]; state [B,H,K,d_v+1] (row k: S[k][0..d_v-1], z[k]).
 */
int gma_oracle_memory(const double* kr, const double* v, const double* mu, const double* var_raw,
                      const double* prior_logits, int B, int H, int N, int d_r, int d_v, int K,
                      double var_floor, double* state) {
    if (!kr || !v || !mu || !var_raw || !prior_logits || !state) return ORACLE_BAD_ARG;
    if (B < 1 || H < 1 || N < 0 || d_r < 1 || d_v < 1 || K < 1) return ORACLE_BAD_ARG;
    const int W = d_v + 1;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; ++bh) {
        const int h = bh % H;
        double* gk = (double*)malloc(sizeof(double) * ((size_t)N * K + 1));
        double* st_bh = state + (size_t)bh * K * W;
        int st = gk ? ORACLE_OK : ORACLE_NO_MEM;
        if (st == ORACLE_OK)
            st = gma_oracle_responsibilities(kr + (size_t)bh * N * d_r, N, d_r, mu + (size_t)h * K * d_r,
                                             var_raw + (size_t)h * K * d_r, prior_logits + (size_t)h * K, K,
                                             var_floor, gk);
        if (st == ORACLE_OK) {
            for (size_t i = 0; i < (size_t)K * W; ++i) st_bh[i] = 0.0;
            const double* v_bh = v + (size_t)bh * N * d_v;
            for (int j = 0; j < N; ++j)
                for (int k = 0; k < K; ++k) {
                    const double g = gk[(size_t)j * K + k];
                    st_bh[(size_t)k * W + d_v] += g;
                    for (int c = 0; c < d_v; ++c) st_bh[(size_t)k * W + c] += g * v_bh[(size_t)j * d_v + c];
                }
        }
        free(gk);
        if (st != ORACLE_OK) {
#pragma omp critical
            status = st;
        }
    }
    return status;
}

/*
 * One causal decode step for every (b, h): with the state [S | z] of the positions before
 * this one, add this position's gamma_K (x) [v | 1] (the sum is inclusive) and read
 * out = gamma_Q S / (gamma_Q . z + eps).
 *   qr, kr [B,H,d_r]; v, out [B,H,d_v]; state [B,H,K,d_v+1] (updated in place).
 */
int gma_oracle_decode_step(const double* qr, const double* kr, const double* v, const double* mu,
                           const double* var_raw, const double* prior_logits, int B, int H, int d_r,
                           int d_v, int K, double eps, double var_floor, double* state, double* out) {
    if (!qr || !kr || !v || !mu || !var_raw || !prior_logits || !state || !out) return ORACLE_BAD_ARG;
    if (B < 1 || H < 1 || d_r < 1 || d_v < 1 || K < 1) return ORACLE_BAD_ARG;
    const int W = d_v + 1;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; ++bh) {
        const int h = bh % H;
        double* gq = (double*)malloc(sizeof(double) * (size_t)K);
        double* gk = (double*)malloc(sizeof(double) * (size_t)K);
        int st = (gq && gk) ? ORACLE_OK : ORACLE_NO_MEM;
        const double* mu_h = mu + (size_t)h * K * d_r;
        const double* vr_h = var_raw + (size_t)h * K * d_r;
        const double* p_h = prior_logits + (size_t)h * K;
        if (st == ORACLE_OK)
            st = gma_oracle_responsibilities(qr + (size_t)bh * d_r, 1, d_r, mu_h, vr_h, p_h, K, var_floor, gq);
        if (st == ORACLE_OK)
            st = gma_oracle_responsibilities(kr + (size_t)bh * d_r, 1, d_r, mu_h, vr_h, p_h, K, var_floor, gk);
        if (st == ORACLE_OK) {
            double* s = state + (size_t)bh * K * W;
            const double* vt = v + (size_t)bh * d_v;
            for (int k = 0; k < K; ++k) {
                s[(size_t)k * W + d_v] += gk[k];
                for (int c = 0; c < d_v; ++c) s[(size_t)k * W + c] += gk[k] * vt[c];
            }
            double den = 0.0;
            for (int k = 0; k < K; ++k) den += gq[k] * s[(size_t)k * W + d_v];
            for (int c = 0; c < d_v; ++c) {
                double num = 0.0;
                for (int k = 0; k < K; ++k) num += gq[k] * s[(size_t)k * W + c];
                out[(size_t)bh * d_v + c] = num / (den + eps);
            }
        }
        free(gq);
        free(gk);
        if (st != ORACLE_OK) {
#pragma omp critical
            status = st;
        }
    }
    return status;
}

/*
 * Responsibility statistics of the routing rows x [B,H,N,d_r] (queries or keys), per head,
 * pooled over the batch and the positions: the quantities of the pages' interpretability
 * analysis of learned responsibilities (components used, usage entropy, hard assignments).
 * Readings (the pages name the quantities but do not define them):
 *   hard    [B,H,N]  hard assignment: argmax_k of the log joint (= of gamma), the lowest k
 *                    among equal maxima
 *   counts  [H,K]    number of rows (b, n) whose hard assignment is k
 *   usage   [H,K]    soft usage: sum over the rows (b, n) of gamma_k
 *   used    [H]      number of components with counts > 0
 *   entropy [H]      usage entropy: -sum_k p_k ln p_k / ln K with p_k = counts_k / (B N) and
 *                    0 ln 0 = 0, i.e. the Shannon entropy of the hard-usage frequencies
 *                    normalised to [0, 1]; 0 when K = 1 or B N = 0
 * Rows are visited in the order b, then n; sums follow that order.
 */
int gma_oracle_resp_stats(const double* x, const double* mu, const double* var_raw, const double* prior_logits,
                          int B, int H, int N, int d_r, int K, double var_floor, int* hard, long long* counts,
                          double* usage, int* used, double* entropy) {
    if (!x || !mu || !var_raw || !prior_logits || !hard || !counts || !usage || !used || !entropy)
        return ORACLE_BAD_ARG;
    if (B < 0 || H < 1 || N < 0 || d_r < 1 || K < 1) return ORACLE_BAD_ARG;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < H; ++h) {
        long long* ch = counts + (size_t)h * K;
        double* uh = usage + (size_t)h * K;
        for (int k = 0; k < K; ++k) { ch[k] = 0; uh[k] = 0.0; }
        const size_t n_alloc = (size_t)(N > 0 ? N : 1) * K;
        double* lj = (double*)malloc(sizeof(double) * n_alloc);
        double* g = (double*)malloc(sizeof(double) * n_alloc);
        int st = (lj && g) ? ORACLE_OK : ORACLE_NO_MEM;
        const double* mu_h = mu + (size_t)h * K * d_r;
        const double* vr_h = var_raw + (size_t)h * K * d_r;
        const double* p_h = prior_logits + (size_t)h * K;
        for (int b = 0; b < B && st == ORACLE_OK && N > 0; ++b) {
            const double* xb = x + ((size_t)b * H + h) * N * d_r;
            st = gma_oracle_log_joint(xb, N, d_r, mu_h, vr_h, p_h, K, var_floor, lj);
            if (st == ORACLE_OK) st = gma_oracle_responsibilities(xb, N, d_r, mu_h, vr_h, p_h, K, var_floor, g);
            if (st != ORACLE_OK) break;
            for (int i = 0; i < N; ++i) {
                const double* li = lj + (size_t)i * K;
                int best = 0;
                for (int k = 1; k < K; ++k)
                    if (li[k] > li[best]) best = k;
                hard[((size_t)b * H + h) * N + i] = best;
                ch[best] += 1;
                for (int k = 0; k < K; ++k) uh[k] += g[(size_t)i * K + k];
            }
        }
        int nu = 0;
        double ent = 0.0;
        const double rows = (double)B * (double)N;
        for (int k = 0; k < K; ++k) {
            if (ch[k] > 0) {
                ++nu;
                const double p = (double)ch[k] / rows;
                ent -= p * log(p);
            }
        }
        used[h] = nu;
        entropy[h] = (K > 1 && rows > 0) ? ent / log((double)K) : 0.0;
        free(lj);
        free(g);
        if (st != ORACLE_OK) {
#pragma omp critical
            status = st;
        }
    }
    return status;
}

/*
 * Backward of the forward mixer (bidirectional or causal): the gradients of a scalar loss L
 * with respect to every input, given dout = dL/dO [B,H,N,d_v].  The pages train the mixture
 * parameters end to end by backpropagation (Core mechanism 3) and analyse the gradients'
 * structure; the gradients here are the chain rule of the forward above, written out:
 *   num_i = gamma_Q,i Vt_i, den_i = gamma_Q,i . Z_i + eps, O_i = num_i / den_i, where
 *   (Vt_i, Z_i) are the totals (bidirectional) or the inclusive prefix sums up to i (causal)
 *   g_num_i = dO_i / den_i,  g_den_i = -(dO_i . O_i) / den_i
 *   dgamma_Q,i[k] = g_num_i . Vt_i[k,:] + g_den_i Z_i[k]
 *   R_j[k,:] = sum_i gamma_Q,i[k] g_num_i,  r_j[k] = sum_i gamma_Q,i[k] g_den_i, over all i
 *              (bidirectional) or over i >= j (causal: the positions that read j)
 *   dv_j = sum_k gamma_K,j[k] R_j[k,:],  dgamma_K,j[k] = v_j . R_j[k,:] + r_j[k]
 *   softmax:  dl_k = gamma_k (dgamma_k - sum_m gamma_m dgamma_m)
 *   log joint l_k(x) = log pi_k - 1/2 sum_d (log 2 pi + log var_kd + (x_d - mu_kd)^2 / var_kd):
 *     dx_d      = -sum_k dl_k (x_d - mu_kd) / var_kd
 *     dmu_kd   += dl_k (x_d - mu_kd) / var_kd
 *     dvar_kd  += dl_k (-1/2) (1 / var_kd - (x_d - mu_kd)^2 / var_kd^2)
 *     dlogpi_k += dl_k
 *   var = softplus(var_raw) + floor:  dvar_raw = dvar * sigmoid(var_raw)
 *   log pi = p - logsumexp(p):        dp_j = dlogpi_j - pi_j sum_k dlogpi_k
 * Parameter gradients sum over both sides, all rows and the batch (b ascending).
 *   dqr, dkr [B,H,N,d_r]; dv [B,H,N,d_v]; dmu, dvar_raw [H,K,d_r]; dprior [H,K].
 */
int gma_oracle_backward(const double* qr, const double* kr, const double* v, const double* mu,
                        const double* var_raw, const double* prior_logits, const double* dout, int B, int H,
                        int N, int d_r, int d_v, int K, int causal, double eps, double var_floor, double* dqr,
                        double* dkr, double* dv, double* dmu, double* dvar_raw, double* dprior) {
    if (!qr || !kr || !v || !mu || !var_raw || !prior_logits || !dout || !dqr || !dkr || !dv || !dmu ||
        !dvar_raw || !dprior)
        return ORACLE_BAD_ARG;
    if (B < 1 || H < 1 || N < 0 || d_r < 1 || d_v < 1 || K < 1 || (causal != 0 && causal != 1))
        return ORACLE_BAD_ARG;
    const size_t BH = (size_t)B * H;
    const size_t nkd = (size_t)K * d_r;
    /* per-(b,h) contributions to the parameter gradients, summed over b afterwards */
    double* cmu = (double*)calloc(BH * nkd, sizeof(double));
    double* cvar = (double*)calloc(BH * nkd, sizeof(double));
    double* cpi = (double*)calloc(BH * (size_t)K, sizeof(double));
    if (!cmu || !cvar || !cpi) {
        free(cmu);
        free(cvar);
        free(cpi);
        return ORACLE_NO_MEM;
    }
    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < (int)BH; ++bh) {
        const int h = bh % H;
        const size_t nN = (size_t)(N > 0 ? N : 1);
        double* gq = (double*)malloc(sizeof(double) * nN * K);
        double* gk = (double*)malloc(sizeof(double) * nN * K);
        double* dgq = (double*)calloc(nN * K, sizeof(double));
        double* dgk = (double*)calloc(nN * K, sizeof(double));
        double* gnum = (double*)malloc(sizeof(double) * nN * d_v);
        double* gden = (double*)malloc(sizeof(double) * nN);
        double* S = (double*)calloc((size_t)K * d_v, sizeof(double));
        double* z = (double*)calloc((size_t)K, sizeof(double));
        double* var = (double*)malloc(sizeof(double) * nkd);
        double* o = (double*)malloc(sizeof(double) * d_v);
        int st = (gq && gk && dgq && dgk && gnum && gden && S && z && var && o) ? ORACLE_OK : ORACLE_NO_MEM;
        const double* mu_h = mu + (size_t)h * nkd;
        const double* vr_h = var_raw + (size_t)h * nkd;
        const double* p_h = prior_logits + (size_t)h * K;
        const double* q_bh = qr + (size_t)bh * N * d_r;
        const double* k_bh = kr + (size_t)bh * N * d_r;
        const double* v_bh = v + (size_t)bh * N * d_v;
        const double* do_bh = dout + (size_t)bh * N * d_v;
        double* dq_bh = dqr + (size_t)bh * N * d_r;
        double* dk_bh = dkr + (size_t)bh * N * d_r;
        double* dv_bh = dv + (size_t)bh * N * d_v;
        if (st == ORACLE_OK && N > 0)
            st = gma_oracle_responsibilities(q_bh, N, d_r, mu_h, vr_h, p_h, K, var_floor, gq);
        if (st == ORACLE_OK && N > 0)
            st = gma_oracle_responsibilities(k_bh, N, d_r, mu_h, vr_h, p_h, K, var_floor, gk);
        if (st == ORACLE_OK) {
            for (size_t i = 0; i < nkd; ++i) var[i] = softplus(vr_h[i]) + var_floor;
            /* bidirectional: the totals of the memory first */
            if (!causal)
                for (int j = 0; j < N; ++j)
                    for (int k = 0; k < K; ++k) {
                        const double g = gk[(size_t)j * K + k];
                        z[k] += g;
                        for (int c = 0; c < d_v; ++c) S[(size_t)k * d_v + c] += g * v_bh[(size_t)j * d_v + c];
                    }
            /* rows in order: (causal) add row i to the prefix, then the read and its gradient */
            for (int i = 0; i < N; ++i) {
                if (causal)
                    for (int k = 0; k < K; ++k) {
                        const double g = gk[(size_t)i * K + k];
                        z[k] += g;
                        for (int c = 0; c < d_v; ++c) S[(size_t)k * d_v + c] += g * v_bh[(size_t)i * d_v + c];
                    }
                const double* gqi = gq + (size_t)i * K;
                double den = eps;
                for (int k = 0; k < K; ++k) den += gqi[k] * z[k];
                double dot = 0.0;
                for (int c = 0; c < d_v; ++c) {
                    double num = 0.0;
                    for (int k = 0; k < K; ++k) num += gqi[k] * S[(size_t)k * d_v + c];
                    o[c] = num / den;
                    dot += do_bh[(size_t)i * d_v + c] * o[c];
                }
                gden[i] = -dot / den;
                for (int c = 0; c < d_v; ++c) gnum[(size_t)i * d_v + c] = do_bh[(size_t)i * d_v + c] / den;
                for (int k = 0; k < K; ++k) {
                    double a = gden[i] * z[k];
                    for (int c = 0; c < d_v; ++c) a += gnum[(size_t)i * d_v + c] * S[(size_t)k * d_v + c];
                    dgq[(size_t)i * K + k] = a;
                }
            }
            /* R, r: sums of gamma_Q (x) [g_num | g_den] over the rows that read row j */
            for (size_t t = 0; t < (size_t)K * d_v; ++t) S[t] = 0.0; /* S reused as R */
            for (int k = 0; k < K; ++k) z[k] = 0.0;                 /* z reused as r */
            if (!causal)
                for (int i = 0; i < N; ++i)
                    for (int k = 0; k < K; ++k) {
                        const double g = gq[(size_t)i * K + k];
                        z[k] += g * gden[i];
                        for (int c = 0; c < d_v; ++c) S[(size_t)k * d_v + c] += g * gnum[(size_t)i * d_v + c];
                    }
            for (int j = N - 1; j >= 0; --j) {
                if (causal)
                    for (int k = 0; k < K; ++k) {
                        const double g = gq[(size_t)j * K + k];
                        z[k] += g * gden[j];
                        for (int c = 0; c < d_v; ++c) S[(size_t)k * d_v + c] += g * gnum[(size_t)j * d_v + c];
                    }
                const double* gkj = gk + (size_t)j * K;
                for (int c = 0; c < d_v; ++c) {
                    double a = 0.0;
                    for (int k = 0; k < K; ++k) a += gkj[k] * S[(size_t)k * d_v + c];
                    dv_bh[(size_t)j * d_v + c] = a;
                }
                for (int k = 0; k < K; ++k) {
                    double a = z[k];
                    for (int c = 0; c < d_v; ++c) a += v_bh[(size_t)j * d_v + c] * S[(size_t)k * d_v + c];
                    dgk[(size_t)j * K + k] = a;
                }
            }
            /* softmax backward, then the log joint's, for both sides */
            for (int side = 0; side < 2; ++side) {
                const double* g = side == 0 ? gq : gk;
                double* dg = side == 0 ? dgq : dgk;
                const double* x = side == 0 ? q_bh : k_bh;
                double* dx = side == 0 ? dq_bh : dk_bh;
                for (int i = 0; i < N; ++i) {
                    double s = 0.0;
                    for (int k = 0; k < K; ++k) s += g[(size_t)i * K + k] * dg[(size_t)i * K + k];
                    for (int k = 0; k < K; ++k) dg[(size_t)i * K + k] = g[(size_t)i * K + k] * (dg[(size_t)i * K + k] - s);
                    const double* xi = x + (size_t)i * d_r;
                    for (int d = 0; d < d_r; ++d) dx[(size_t)i * d_r + d] = 0.0;
                    for (int k = 0; k < K; ++k) {
                        const double dl = dg[(size_t)i * K + k];
                        cpi[(size_t)bh * K + k] += dl;
                        for (int d = 0; d < d_r; ++d) {
                            const size_t kd = (size_t)k * d_r + d;
                            const double diff = xi[d] - mu_h[kd];
                            dx[(size_t)i * d_r + d] -= dl * diff / var[kd];
                            cmu[(size_t)bh * nkd + kd] += dl * diff / var[kd];
                            cvar[(size_t)bh * nkd + kd] += dl * -0.5 * (1.0 / var[kd] - diff * diff / (var[kd] * var[kd]));
                        }
                    }
                }
            }
        }
        free(gq);
        free(gk);
        free(dgq);
        free(dgk);
        free(gnum);
        free(gden);
        free(S);
        free(z);
        free(var);
        free(o);
        if (st != ORACLE_OK) {
#pragma omp critical
            status = st;
        }
    }
    if (status == ORACLE_OK) {
        for (int h = 0; h < H; ++h) {
            const double* p_h = prior_logits + (size_t)h * K;
            double m = p_h[0];
            for (int k = 1; k < K; ++k) m = fmax(m, p_h[k]);
            double se = 0.0;
            for (int k = 0; k < K; ++k) se += exp(p_h[k] - m);
            double tot = 0.0;
            for (int k = 0; k < K; ++k) {
                double a = 0.0;
                for (int b = 0; b < B; ++b) a += cpi[((size_t)b * H + h) * K + k];
                dprior[(size_t)h * K + k] = a;
                tot += a;
            }
            for (int k = 0; k < K; ++k) dprior[(size_t)h * K + k] -= exp(p_h[k] - m) / se * tot;
            for (size_t kd = 0; kd < nkd; ++kd) {
                double am = 0.0, av = 0.0;
                for (int b = 0; b < B; ++b) {
                    am += cmu[((size_t)b * H + h) * nkd + kd];
                    av += cvar[((size_t)b * H + h) * nkd + kd];
                }
                const double r = var_raw[(size_t)h * nkd + kd];
                dmu[(size_t)h * nkd + kd] = am;
                dvar_raw[(size_t)h * nkd + kd] = av / (1.0 + exp(-r));
            }
        }
    }
    free(cmu);
    free(cvar);
    free(cpi);
    return status;
}
