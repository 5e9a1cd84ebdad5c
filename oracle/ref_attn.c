/*
 * Reference implementation of exact softmax attention, fp64, CPU only.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links or calls this
 * file; it exists so the HIP kernels can be checked against the plain
 * definition.  It shares no code, header or table with them.
 *
 * What it computes is the definition of attention that FlashAttention keeps
 * exactly ("FlashAttention: Fast and Memory-Efficient Exact Attention with
 * IO-Awareness" section 1.1, Attn = softmax(QK^T)V, with the numerically
 * stable softmax of its section 2.4), with a scale on the scores and two masks
 * ("FlashAttention 深度解析" section 五 names the causal mask as built in;
 * the block-sparse variant of the IO-Awareness page section 4 attends only the
 * kept 128x128 blocks).  For every (batch, head) it materializes the full
 * score matrix S and probability matrix P ("FlashAttention 深度解析"
 * section 一 describes exactly this standard route), then O = P V.
 *
 * Layout: q, k, v, o, dO, dq, dk, dv are [B][H][N][d] row-major doubles;
 * lse is [B][H][N]; mask (optional) is [nb][nb] uint8 with nb = ceil(N/128),
 * shared by all (b, h); nonzero = block kept.
 *
 * Conventions (choices where the pages are silent):
 *   S_ij = scale * sum_k q_ik k_jk - slope_h |i - j|   (slope_h = 0 without ALiBi)
 *   allowed(i, j) = (!causal || j <= i) && (mask == NULL || mask[i/128][j/128])
 *                   && (wl < 0 || j >= i - wl) && (wr < 0 || j <= i + wr)
 *   The window (wl, wr) and the per-head ALiBi slopes are the two further
 *   built-in variants "FlashAttention 深度解析" section 五 names beside the
 *   causal mask; the `_ex` entry points take them, the others use none.
 *   m_i = max over allowed j of S_ij;  Z_i = sum over allowed j of exp(S_ij - m_i)
 *   P_ij = exp(S_ij - m_i) / Z_i if allowed else 0
 *   O_i = sum_j P_ij v_j;  lse_i = m_i + log(Z_i)
 *   a row with no allowed key: O_i = 0, lse_i = -inf.
 *
 * The backward is the chain rule of the same definition (the recompute
 * backward of "FlashAttention原理概览" section 3.2 and the IO-Awareness page
 * section 2.5 produces the same numbers without storing P):
 *   dV = P^T dO;  dP = dO V^T;  D_i = sum_j P_ij dP_ij;
 *   dS_ij = P_ij (dP_ij - D_i);  dQ = scale * dS K;  dK = scale * dS^T Q.
 *
 * An online-softmax variant (the running max / running sum loop of
 * "FlashAttention 深度解析" section 二) is provided separately so tests can
 * check that chunked evaluation reaches the one-shot result.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define REF_MASK_BLOCK 128

int ref_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Local-window bounds (negative = unbounded) and the ALiBi slope of the head. */
typedef struct {
    long wl, wr;
    double slope;
} ref_var;

static const ref_var REF_PLAIN = {-1, -1, 0.0};

static int ref_allowed(long i, long j, int causal, const uint8_t* mask, long nb, const ref_var* var) {
    if (causal && j > i) return 0;
    if (mask && !mask[(i / REF_MASK_BLOCK) * nb + (j / REF_MASK_BLOCK)]) return 0;
    if (var->wl >= 0 && j < i - var->wl) return 0;
    if (var->wr >= 0 && j > i + var->wr) return 0;
    return 1;
}

/* The ALiBi term of S_ij. */
static double ref_bias(long i, long j, const ref_var* var) {
    return var->slope == 0.0 ? 0.0 : -var->slope * (double)(i > j ? i - j : j - i);
}

/* Variant of head bh (slopes indexed by h = bh mod H). */
static ref_var ref_var_of(long bh, int H, int wl, int wr, const double* slopes) {
    ref_var v;
    v.wl = wl;
    v.wr = wr;
    v.slope = slopes ? slopes[bh % H] : 0.0;
    return v;
}

/* Scores, probabilities and lse of one head.  S and P are N*N doubles each. */
static void ref_head_probs(const double* q, const double* k, long N, long d, double scale,
                           int causal, const uint8_t* mask, const ref_var* var, double* S, double* P,
                           double* lse) {
    long nb = (N + REF_MASK_BLOCK - 1) / REF_MASK_BLOCK;
#pragma omp parallel for schedule(static)
    for (long i = 0; i < N; i++) {
        /* 1. scores */
        for (long j = 0; j < N; j++) {
            double acc = 0.0;
            for (long c = 0; c < d; c++) acc += q[i * d + c] * k[j * d + c];
            S[i * N + j] = scale * acc + ref_bias(i, j, var);
        }
        /* 2. stable softmax over the allowed keys */
        double m = -INFINITY;
        long count = 0;
        for (long j = 0; j < N; j++)
            if (ref_allowed(i, j, causal, mask, nb, var)) {
                if (S[i * N + j] > m) m = S[i * N + j];
                count++;
            }
        if (count == 0) {
            for (long j = 0; j < N; j++) P[i * N + j] = 0.0;
            lse[i] = -INFINITY;
            continue;
        }
        double z = 0.0;
        for (long j = 0; j < N; j++)
            if (ref_allowed(i, j, causal, mask, nb, var)) z += exp(S[i * N + j] - m);
        for (long j = 0; j < N; j++)
            P[i * N + j] = ref_allowed(i, j, causal, mask, nb, var) ? exp(S[i * N + j] - m) / z : 0.0;
        lse[i] = m + log(z);
    }
}

/* O = P V for one head. */
static void ref_head_pv(const double* P, const double* v, long N, long d, double* o) {
#pragma omp parallel for schedule(static)
    for (long i = 0; i < N; i++) {
        for (long c = 0; c < d; c++) o[i * d + c] = 0.0;
        for (long j = 0; j < N; j++) {
            double p = P[i * N + j];
            if (p == 0.0) continue;
            for (long c = 0; c < d; c++) o[i * d + c] += p * v[j * d + c];
        }
    }
}

/* Probabilities of a single head (exposed so tests can inspect P). */
int ref_attn_probs(const double* q, const double* k, int N, int d, double scale, int causal,
                   const uint8_t* mask, double* P, double* lse) {
    double* S = (double*)malloc(sizeof(double) * (size_t)N * N);
    if (!S) return 1;
    ref_head_probs(q, k, N, d, scale, causal, mask, &REF_PLAIN, S, P, lse);
    free(S);
    return 0;
}

int ref_attn_fwd_ex(const double* q, const double* k, const double* v, int B, int H, int N, int d,
                    double scale, int causal, const uint8_t* mask, int wl, int wr, const double* slopes,
                    double* o, double* lse) {
    size_t nn = (size_t)N * N, nd = (size_t)N * d;
    double* S = (double*)malloc(sizeof(double) * nn);
    double* P = (double*)malloc(sizeof(double) * nn);
    if (!S || !P) { free(S); free(P); return 1; }
    for (long bh = 0; bh < (long)B * H; bh++) {
        const ref_var var = ref_var_of(bh, H, wl, wr, slopes);
        ref_head_probs(q + bh * nd, k + bh * nd, N, d, scale, causal, mask, &var, S, P, lse + bh * N);
        ref_head_pv(P, v + bh * nd, N, d, o + bh * nd);
    }
    free(S);
    free(P);
    return 0;
}

int ref_attn_fwd(const double* q, const double* k, const double* v, int B, int H, int N, int d,
                 double scale, int causal, const uint8_t* mask, double* o, double* lse) {
    return ref_attn_fwd_ex(q, k, v, B, H, N, d, scale, causal, mask, -1, -1, NULL, o, lse);
}

/*
 * Selected rows only: rows[r] = {bh, i}.  Each row's scores, probabilities and
 * output follow the same definition; nothing is shared between rows.
 */
int ref_attn_fwd_rows_ex(const double* q, const double* k, const double* v, int B, int H, int N,
                         int d, double scale, int causal, const uint8_t* mask, int wl, int wr,
                         const double* slopes, const int64_t* rows, int nrows, double* o_rows,
                         double* lse_rows) {
    size_t nd = (size_t)N * d;
    long nb = (N + REF_MASK_BLOCK - 1) / REF_MASK_BLOCK;
    int err = 0;
    (void)B;
#pragma omp parallel
    {
        double* srow = (double*)malloc(sizeof(double) * (size_t)N);
        double* prow = (double*)malloc(sizeof(double) * (size_t)N);
        if (!srow || !prow) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int r = 0; r < nrows; r++) {
                long bh = rows[2 * r], i = rows[2 * r + 1];
                const ref_var vv = ref_var_of(bh, H, wl, wr, slopes);
                const ref_var* var = &vv;
                const double* qi = q + bh * nd + i * d;
                const double* kh = k + bh * nd;
                const double* vh = v + bh * nd;
                for (long j = 0; j < N; j++) {
                    double acc = 0.0;
                    for (long c = 0; c < d; c++) acc += qi[c] * kh[j * d + c];
                    srow[j] = scale * acc + ref_bias(i, j, var);
                }
                double m = -INFINITY;
                long count = 0;
                for (long j = 0; j < N; j++)
                    if (ref_allowed(i, j, causal, mask, nb, var)) {
                        if (srow[j] > m) m = srow[j];
                        count++;
                    }
                double* orow = o_rows + (size_t)r * d;
                for (long c = 0; c < d; c++) orow[c] = 0.0;
                if (count == 0) { lse_rows[r] = -INFINITY; continue; }
                double z = 0.0;
                for (long j = 0; j < N; j++)
                    if (ref_allowed(i, j, causal, mask, nb, var)) z += exp(srow[j] - m);
                for (long j = 0; j < N; j++) {
                    prow[j] = ref_allowed(i, j, causal, mask, nb, var) ? exp(srow[j] - m) / z : 0.0;
                    if (prow[j] == 0.0) continue;
                    for (long c = 0; c < d; c++) orow[c] += prow[j] * vh[j * d + c];
                }
                lse_rows[r] = m + log(z);
            }
        }
        free(srow);
        free(prow);
    }
    return err;
}

int ref_attn_fwd_rows(const double* q, const double* k, const double* v, int B, int H, int N, int d,
                      double scale, int causal, const uint8_t* mask, const int64_t* rows, int nrows,
                      double* o_rows, double* lse_rows) {
    return ref_attn_fwd_rows_ex(q, k, v, B, H, N, d, scale, causal, mask, -1, -1, NULL, rows, nrows,
                                o_rows, lse_rows);
}

/*
 * Online softmax ("FlashAttention 深度解析" section 二): scan the keys of each
 * row in chunks of `chunk`; keep the running max m, the running sum l and the
 * unnormalized output o; when the max grows, rescale l and o by exp(m - m_new);
 * divide once at the end.  Keys a mask removes are skipped.
 */
int ref_attn_fwd_online_ex(const double* q, const double* k, const double* v, int B, int H, int N,
                           int d, double scale, int causal, const uint8_t* mask, int wl, int wr,
                           const double* slopes, int chunk, double* o, double* lse) {
    if (chunk < 1) return 1;
    size_t nd = (size_t)N * d;
    long nb = (N + REF_MASK_BLOCK - 1) / REF_MASK_BLOCK;
    int err = 0;
    for (long bh = 0; bh < (long)B * H; bh++) {
        const double* qh = q + bh * nd;
        const double* kh = k + bh * nd;
        const double* vh = v + bh * nd;
        const ref_var vv = ref_var_of(bh, H, wl, wr, slopes);
        const ref_var* var = &vv;
#pragma omp parallel
        {
            double* sblk = (double*)malloc(sizeof(double) * (size_t)chunk);
            if (!sblk) {
#pragma omp atomic write
                err = 1;
            }
#pragma omp for schedule(static)
            for (long i = 0; i < N; i++) {
                if (!sblk) continue;
                double m = -INFINITY, l = 0.0;
                double* oi = o + bh * nd + i * d;
                for (long c = 0; c < d; c++) oi[c] = 0.0;
                for (long j0 = 0; j0 < N; j0 += chunk) {
                    long j1 = j0 + chunk < N ? j0 + chunk : N;
                    /* scores of this chunk and the chunk's max over allowed keys */
                    double bmax = -INFINITY;
                    for (long j = j0; j < j1; j++) {
                        double acc = 0.0;
                        for (long c = 0; c < d; c++) acc += qh[i * d + c] * kh[j * d + c];
                        sblk[j - j0] = scale * acc + ref_bias(i, j, var);
                        if (ref_allowed(i, j, causal, mask, nb, var) && sblk[j - j0] > bmax) bmax = sblk[j - j0];
                    }
                    if (bmax == -INFINITY) continue; /* nothing allowed in this chunk */
                    double m_new = m > bmax ? m : bmax;
                    double corr = exp(m - m_new); /* 0 while m is still -inf */
                    l *= corr;
                    for (long c = 0; c < d; c++) oi[c] *= corr;
                    for (long j = j0; j < j1; j++) {
                        if (!ref_allowed(i, j, causal, mask, nb, var)) continue;
                        double p = exp(sblk[j - j0] - m_new);
                        l += p;
                        for (long c = 0; c < d; c++) oi[c] += p * vh[j * d + c];
                    }
                    m = m_new;
                }
                if (l == 0.0) {
                    lse[bh * N + i] = -INFINITY;
                    continue;
                }
                for (long c = 0; c < d; c++) oi[c] /= l;
                lse[bh * N + i] = m + log(l);
            }
            free(sblk);
        }
    }
    return err;
}

int ref_attn_fwd_online(const double* q, const double* k, const double* v, int B, int H, int N,
                        int d, double scale, int causal, const uint8_t* mask, int chunk,
                        double* o, double* lse) {
    return ref_attn_fwd_online_ex(q, k, v, B, H, N, d, scale, causal, mask, -1, -1, NULL, chunk, o, lse);
}

/*
 * Backward of the definition above for every (b, h).  Optionally returns the
 * forward's O and lse and the row terms D (pointers may be NULL).
 */
int ref_attn_bwd_ex(const double* q, const double* k, const double* v, const double* dO, int B, int H,
                    int N, int d, double scale, int causal, const uint8_t* mask, int wl, int wr,
                    const double* slopes, double* dq, double* dk, double* dv, double* o_out,
                    double* lse_out, double* D_out) {
    size_t nn = (size_t)N * N, nd = (size_t)N * d;
    double* S = (double*)malloc(sizeof(double) * nn);
    double* P = (double*)malloc(sizeof(double) * nn);
    double* dP = (double*)malloc(sizeof(double) * nn);
    double* lse = (double*)malloc(sizeof(double) * (size_t)N);
    double* D = (double*)malloc(sizeof(double) * (size_t)N);
    if (!S || !P || !dP || !lse || !D) {
        free(S); free(P); free(dP); free(lse); free(D);
        return 1;
    }
    double* dS = S; /* S is not needed once P exists */
    for (long bh = 0; bh < (long)B * H; bh++) {
        const double* qh = q + bh * nd;
        const double* kh = k + bh * nd;
        const double* vh = v + bh * nd;
        const double* doh = dO + bh * nd;
        const ref_var var = ref_var_of(bh, H, wl, wr, slopes);
        ref_head_probs(qh, kh, N, d, scale, causal, mask, &var, S, P, lse);
        if (o_out) ref_head_pv(P, vh, N, d, o_out + bh * nd);
        if (lse_out) memcpy(lse_out + bh * N, lse, sizeof(double) * (size_t)N);
        /* dP = dO V^T */
#pragma omp parallel for schedule(static)
        for (long i = 0; i < N; i++)
            for (long j = 0; j < N; j++) {
                double acc = 0.0;
                for (long c = 0; c < d; c++) acc += doh[i * d + c] * vh[j * d + c];
                dP[i * N + j] = acc;
            }
        /* D_i = sum_j P_ij dP_ij;  dS = P o (dP - D) */
#pragma omp parallel for schedule(static)
        for (long i = 0; i < N; i++) {
            double acc = 0.0;
            for (long j = 0; j < N; j++) acc += P[i * N + j] * dP[i * N + j];
            D[i] = acc;
            for (long j = 0; j < N; j++) dS[i * N + j] = P[i * N + j] * (dP[i * N + j] - acc);
        }
        if (D_out) memcpy(D_out + bh * N, D, sizeof(double) * (size_t)N);
        /* dQ = scale * dS K */
        double* dqh = dq + bh * nd;
#pragma omp parallel for schedule(static)
        for (long i = 0; i < N; i++) {
            for (long c = 0; c < d; c++) dqh[i * d + c] = 0.0;
            for (long j = 0; j < N; j++) {
                double s = dS[i * N + j];
                if (s == 0.0) continue;
                for (long c = 0; c < d; c++) dqh[i * d + c] += s * kh[j * d + c];
            }
            for (long c = 0; c < d; c++) dqh[i * d + c] *= scale;
        }
        /* dV = P^T dO and dK = scale * dS^T Q; each thread owns a range of keys j
         * and sums over i in increasing order. */
        double* dvh = dv + bh * nd;
        double* dkh = dk + bh * nd;
#pragma omp parallel
        {
            long nt = 1, t = 0;
#ifdef _OPENMP
            nt = omp_get_num_threads();
            t = omp_get_thread_num();
#endif
            long j0 = (long)N * t / nt, j1 = (long)N * (t + 1) / nt;
            for (long j = j0; j < j1; j++)
                for (long c = 0; c < d; c++) dvh[j * d + c] = dkh[j * d + c] = 0.0;
            for (long i = 0; i < N; i++)
                for (long j = j0; j < j1; j++) {
                    double p = P[i * N + j], s = dS[i * N + j];
                    if (p != 0.0)
                        for (long c = 0; c < d; c++) dvh[j * d + c] += p * doh[i * d + c];
                    if (s != 0.0)
                        for (long c = 0; c < d; c++) dkh[j * d + c] += s * qh[i * d + c];
                }
            for (long j = j0; j < j1; j++)
                for (long c = 0; c < d; c++) dkh[j * d + c] *= scale;
        }
    }
    free(S); free(P); free(dP); free(lse); free(D);
    return 0;
}

int ref_attn_bwd(const double* q, const double* k, const double* v, const double* dO, int B, int H,
                 int N, int d, double scale, int causal, const uint8_t* mask, double* dq, double* dk,
                 double* dv, double* o_out, double* lse_out, double* D_out) {
    return ref_attn_bwd_ex(q, k, v, dO, B, H, N, d, scale, causal, mask, -1, -1, NULL, dq, dk, dv, o_out,
                           lse_out, D_out);
}

/*
 * Attention of a few new queries over a paged KV cache (decode).
 * "FlashAttention 深度解析" section 五: since version 2.5 FlashAttention reads
 * the KV cache straight from the paged layout that PagedAttention manages;
 * "FlashAttention原理概览" section 3.2 notes that inference needs no score
 * matrix, only the cache.  The result is the same exact attention as above,
 * taken over the keys the page table names.
 *
 * Layout (choices where the pages are silent):
 *   q, o: [B][H][Nq][d]; lse: [B][H][Nq];
 *   k_cache, v_cache: [num_pages][page_size][Hkv][d];
 *   block_table: [B][max_pages] int32, logical page p of sequence b is the
 *     physical page block_table[b * max_pages + p];
 *   seqlens: [B] int32, sequence b holds keys at positions 0 .. L_b - 1, the
 *     key at position t in row t % page_size of logical page t / page_size.
 *   Query head h reads KV head h / (H / Hkv) (grouped heads, H % Hkv == 0).
 *   The Nq queries are the last Nq positions L_b - Nq .. L_b - 1: with causal,
 *   query i sees positions t <= L_b - Nq + i, otherwise all L_b keys.
 *   A query with no key: O = 0, lse = -inf.
 * Returns 0, or -1 (bad sizes), -2 (a page index outside [0, num_pages)),
 * -3 (a length outside [0, max_pages * page_size]).
 */
int ref_attn_paged_fwd(const double* q, const double* k_cache, const double* v_cache,
                       const int32_t* block_table, const int32_t* seqlens, int B, int H, int Hkv, int Nq,
                       int d, int num_pages, int page_size, int max_pages, double scale, int causal,
                       double* o, double* lse) {
    if (B < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || Nq < 1 || d < 1 || num_pages < 1 || page_size < 1 ||
        max_pages < 1)
        return -1;
    for (long b = 0; b < B; b++) {
        long L = seqlens[b];
        if (L < 0 || L > (long)max_pages * page_size) return -3;
        for (long p = 0; p < (L + page_size - 1) / page_size; p++) {
            int32_t pg = block_table[b * max_pages + p];
            if (pg < 0 || pg >= num_pages) return -2;
        }
    }
    const long group = H / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (long b = 0; b < B; b++)
        for (long h = 0; h < H; h++) {
            const long L = seqlens[b], hk = h / group;
            double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
            for (long i = 0; i < Nq; i++) {
                const double* qi = q + ((b * H + h) * Nq + i) * d;
                double* oi = o + ((b * H + h) * Nq + i) * d;
                /* keys 0 .. n-1 are allowed */
                long n = causal ? L - Nq + i + 1 : L;
                if (n > L) n = L;
                for (long c = 0; c < d; c++) oi[c] = 0.0;
                if (n <= 0) {
                    lse[(b * H + h) * Nq + i] = -INFINITY;
                    continue;
                }
                double m = -INFINITY;
                for (long t = 0; t < n; t++) {
                    const long pg = block_table[b * max_pages + t / page_size];
                    const double* kt = k_cache + ((pg * page_size + t % page_size) * Hkv + hk) * d;
                    double acc = 0.0;
                    for (long c = 0; c < d; c++) acc += qi[c] * kt[c];
                    s[t] = scale * acc;
                    if (s[t] > m) m = s[t];
                }
                double z = 0.0;
                for (long t = 0; t < n; t++) z += exp(s[t] - m);
                for (long t = 0; t < n; t++) {
                    const long pg = block_table[b * max_pages + t / page_size];
                    const double* vt = v_cache + ((pg * page_size + t % page_size) * Hkv + hk) * d;
                    const double p = exp(s[t] - m) / z;
                    for (long c = 0; c < d; c++) oi[c] += p * vt[c];
                }
                lse[(b * H + h) * Nq + i] = m + log(z);
            }
            free(s);
        }
    return 0;
}

/*
 * FP8 forward with block quantization and incoherent processing ("FlashAttention
 * 深度解析" section 四 names both for FlashAttention-3: FP8 block quantization,
 * with incoherent processing, gives 2.6x lower error than plain FP8).  The pages
 * give no formulas; the readings taken:
 *   format      FP8 E4M3 (OCP E4M3FN): 1 sign, 4 exponent bits (bias 7), 3
 *               mantissa bits, subnormals, largest finite 448, no infinities;
 *               encoding rounds to nearest, ties to even, and saturates at 448;
 *   blocks      each (b, h) slice of Q, K and V is cut into blocks of `block`
 *               rows (the last may be short); a block gets the power-of-two
 *               scale 2^e, e = the smallest integer with amax / 2^e <= 448
 *               (e = 0 for an all-zero block; e kept within [-127, 127], the
 *               range of an E8M0 scale), and codes = E4M3(x / 2^e);
 *   incoherent  Q and K are first multiplied along the head dimension by the
 *               same random orthogonal map: x -> H (sigma o x), H the Sylvester
 *               Hadamard matrix of order d and sigma a vector of random signs,
 *               with a factor 1/d on K only, so that (Q M)(K M')^T = Q K^T
 *               exactly (H H^T = d I);
 *   attention   exact attention (as above, fp64) of the dequantized Q, K, V.
 * The kernels' own rounding of P to FP8 before P V is an extra error the
 * oracle does not model (its scale depends on the kernel's running max).
 */
static double ref_e4m3_value(int code) {
    const int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);  /* (1 + m/8) 2^(e-7) */
    return s ? -v : v;
}

/* Nearest E4M3 code (ties to even code), saturating to +-448. */
static int ref_e4m3_code(double x) {
    int sign = 0;
    if (x < 0 || (x == 0 && signbit(x))) { sign = 0x80; x = -x; }
    if (x >= 448.0) return sign | 0x7E;
    /* candidates are the 127 non-negative finite codes 0x00 .. 0x7E, increasing in value */
    int lo = 0, hi = 0x7E;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (ref_e4m3_value(mid) <= x) lo = mid; else hi = mid;
    }
    double dl = x - ref_e4m3_value(lo), dh = ref_e4m3_value(hi) - x;
    int c;
    if (ref_e4m3_value(hi) <= x) c = hi;
    else if (dl < dh) c = lo;
    else if (dh < dl) c = hi;
    else c = (lo & 1) ? hi : lo;  /* tie: the even code */
    return sign | c;
}

int ref_e4m3_encode(const double* x, long n, uint8_t* codes) {
    for (long i = 0; i < n; i++) codes[i] = (uint8_t)ref_e4m3_code(x[i]);
    return 0;
}

int ref_e4m3_decode(const uint8_t* codes, long n, double* x) {
    for (long i = 0; i < n; i++) x[i] = ref_e4m3_value(codes[i]);
    return 0;
}

/* y = H (sigma o x) for one row of length d (d a power of two), by the
 * definition H_ij = (-1)^popcount(i & j); times 1/d when `inverse_side`. */
static void ref_hadamard_row(const double* x, const double* sigma, long d, int inverse_side, double* y) {
    for (long i = 0; i < d; i++) {
        double acc = 0.0;
        for (long j = 0; j < d; j++) {
            double t = sigma[j] * x[j];
            acc += (__builtin_popcountl((unsigned long)(i & j)) & 1) ? -t : t;
        }
        y[i] = inverse_side ? acc / (double)d : acc;
    }
}

/* Quantize rows [rows][d] in blocks of `block` rows: codes and block exponents. */
static void ref_quant_blocks(const double* x, long rows, long d, long block, uint8_t* codes, int8_t* exps) {
    for (long b0 = 0, bi = 0; b0 < rows; b0 += block, bi++) {
        long b1 = b0 + block < rows ? b0 + block : rows;
        double amax = 0.0;
        for (long i = b0 * d; i < b1 * d; i++) amax = fmax(amax, fabs(x[i]));
        int e = 0;
        if (amax > 0.0) {
            e = (int)ceil(log2(amax / 448.0));
            while (ldexp(amax, -e) > 448.0) e++;      /* guard the log2 rounding */
            while (ldexp(amax, -(e - 1)) <= 448.0) e--;
        }
        if (e < -127) e = -127;  /* the range of an E8M0 block scale */
        if (e > 127) e = 127;
        exps[bi] = (int8_t)e;
        for (long i = b0 * d; i < b1 * d; i++) codes[i] = (uint8_t)ref_e4m3_code(ldexp(x[i], -e));
    }
}

/*
 * Quantize one [B][H][N][d] tensor: codes [B][H][N][d], exps [B][H][ceil(N/block)].
 * sigma (length d, entries +-1) or NULL; inverse_side = 1 applies the 1/d (K).
 */
int ref_fp8_quantize(const double* x, int B, int H, int N, int d, int block, const double* sigma, int inverse_side,
                     uint8_t* codes, int8_t* exps) {
    if (block < 1 || (sigma && (d & (d - 1)))) return -1;
    const long nd = (long)N * d, nblk = (N + block - 1) / block;
    double* t = (double*)malloc(sizeof(double) * (size_t)nd);
    if (!t) return -1;
    for (long bh = 0; bh < (long)B * H; bh++) {
        const double* xh = x + bh * nd;
        if (sigma)
            for (long i = 0; i < N; i++) ref_hadamard_row(xh + i * d, sigma, d, inverse_side, t + i * d);
        else
            memcpy(t, xh, sizeof(double) * (size_t)nd);
        ref_quant_blocks(t, N, d, block, codes + bh * nd, exps + bh * nblk);
    }
    free(t);
    return 0;
}

/* The incoherent map alone, for rows [rows][d]: y = H (sigma o x) (x 1/d if inverse_side). */
int ref_hadamard(const double* x, long rows, int d, const double* sigma, int inverse_side, double* y) {
    if (d < 1 || (d & (d - 1))) return -1;
    for (long i = 0; i < rows; i++) ref_hadamard_row(x + i * d, sigma, d, inverse_side, y + i * d);
    return 0;
}
