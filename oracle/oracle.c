/*
 * Plain fp64 CPU oracle for one rank's share of Ulysses sequence parallelism.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do. It shares no code, header or table with the HIP library.
 *
 * What it computes, and where that is stated:
 *
 *  O1  The sequence<->head layout swap. "Ulysses sequence parallelism"
 *      (HF Transformers docs), intro and its two-GPU diagram: each GPU first
 *      holds a contiguous token range with all heads; after the all-to-all it
 *      holds all tokens for a contiguous range of heads; a second all-to-all
 *      returns to the token split. "Ulysses Sequence Parallelism for
 *      Million-Token Context Training", "How Ulysses Sequence Parallelism
 *      Works", steps 1, 3 and 5 restate the same three layouts.
 *  O2  Softmax attention over the full sequence for the local heads (same
 *      page, step 4; "The Challenge of Long Sequence Training": tiled
 *      FlashAttention saves memory but computes the exact O(n^2) result, so
 *      the oracle is the plain definition). Causal masking follows from the
 *      causal-LM training the pages benchmark; packed documents must not
 *      attend across their boundaries ("Ulysses sequence parallelism",
 *      Configure, on sp_attn_implementation and packed samples).
 *  O3  The textbook gradient of O2 (the pages do not spell it out).
 *
 * Readings where the pages are silent: query head h uses KV head
 * floor(h / G), G = hq / hkv (contiguous GQA groups, the only grouping that
 * survives a contiguous head split); causal means key j <= query i, diagonal
 * included, on positions 0..N-1; the softmax uses the natural exponential and
 * LSE is natural-log.
 *
 * All floating point is double. Inputs arrive as doubles already decoded
 * exactly from bf16 by the caller.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- O1 ---- */

/*
 * Global (fused) head index of local head c on rank r. The fused head axis is
 * [q heads | k heads | v heads] = seg_heads[0] | seg_heads[1] | ...; rank r
 * owns the contiguous block [r*seg/P, (r+1)*seg/P) of every segment, in
 * segment order.
 */
static int64_t orc_global_head(int r, int c, int P, int nseg, const int32_t *seg_heads) {
    int64_t base = 0;
    for (int k = 0; k < nseg; ++k) {
        int local = seg_heads[k] / P;
        if (c < local) return base + (int64_t)r * local + c;
        c -= local;
        base += seg_heads[k];
    }
    return -1;
}

/*
 * Pack: x_seq [n][H][d] (H = sum of seg_heads) -> send [P][n][H/P][d], where
 * send[p][t][c][e] = x_seq[t][global_head(p, c)][e]. Chunk p is what this
 * rank sends to rank p in the sequence-to-head all-to-all.
 */
void orc_seq_to_head(const uint16_t *x_seq, uint16_t *send, int64_t n, int32_t P,
                     int32_t nseg, const int32_t *seg_heads, int32_t d) {
    int64_t H = 0;
    for (int k = 0; k < nseg; ++k) H += seg_heads[k];
    int64_t h = H / P;
    for (int p = 0; p < P; ++p)
        for (int64_t t = 0; t < n; ++t)
            for (int c = 0; c < h; ++c) {
                int64_t g = orc_global_head(p, c, P, nseg, seg_heads);
                for (int e = 0; e < d; ++e)
                    send[((p * n + t) * h + c) * d + e] = x_seq[(t * H + g) * d + e];
            }
}

/* Unpack: the inverse of orc_seq_to_head, recv [P][n][H/P][d] -> x_seq [n][H][d]. */
void orc_head_to_seq(const uint16_t *recv, uint16_t *x_seq, int64_t n, int32_t P,
                     int32_t nseg, const int32_t *seg_heads, int32_t d) {
    int64_t H = 0;
    for (int k = 0; k < nseg; ++k) H += seg_heads[k];
    int64_t h = H / P;
    for (int p = 0; p < P; ++p)
        for (int64_t t = 0; t < n; ++t)
            for (int c = 0; c < h; ++c) {
                int64_t g = orc_global_head(p, c, P, nseg, seg_heads);
                for (int e = 0; e < d; ++e)
                    x_seq[(t * H + g) * d + e] = recv[((p * n + t) * h + c) * d + e];
            }
}

/* ---------------------------------------------------------- masks ------ */

/* Document index of token t under cu (cu[0]=0 < cu[1] < ... < cu[nseq]=N). */
static int orc_doc_of(int64_t t, const int32_t *cu, int nseq) {
    if (!cu) return 0;
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/* Allowed keys A(i) form one contiguous range [*j0, *j1). */
static void orc_key_range(int64_t i, int64_t N, int causal, const int32_t *cu, int nseq,
                          int64_t *j0, int64_t *j1) {
    int64_t lo = 0, hi = N;
    if (cu) {
        int b = orc_doc_of(i, cu, nseq);
        lo = cu[b];
        hi = cu[b + 1];
    }
    if (causal) hi = i + 1;
    *j0 = lo;
    *j1 = hi;
}

/* --------------------------------------------------------------- O2 ---- */

static int orc_thread(void) {
#ifdef _OPENMP
    return omp_get_thread_num();
#else
    return 0;
#endif
}

static int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * One query row of one head: writes o[d] and returns LSE. Steps in order:
 * s_j = scale * q.k_j on A(i); m = max s_j; l = sum exp(s_j - m);
 * LSE = m + ln l; p_j = exp(s_j - LSE); o = sum p_j v_j.
 * s is caller scratch of length N.
 */
static double orc_row_fwd(const double *q, const double *k, const double *v, int64_t i, int h,
                          int64_t N, int hq, int hkv, int d, double scale, int causal,
                          const int32_t *cu, int nseq, double *s, double *o) {
    int G = hq / hkv;
    int g = h / G;
    int64_t j0, j1;
    (void)N;
    orc_key_range(i, N, causal, cu, nseq, &j0, &j1);
    const double *qi = q + (i * hq + h) * d;
    double m = -INFINITY;
    for (int64_t j = j0; j < j1; ++j) {
        const double *kj = k + (j * hkv + g) * d;
        double acc = 0.0;
        for (int e = 0; e < d; ++e) acc += qi[e] * kj[e];
        s[j] = scale * acc;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = j0; j < j1; ++j) l += exp(s[j] - m);
    double lse = m + log(l);
    for (int e = 0; e < d; ++e) o[e] = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
        double p = exp(s[j] - lse);
        const double *vj = v + (j * hkv + g) * d;
        for (int e = 0; e < d; ++e) o[e] += p * vj[e];
    }
    return lse;
}

/*
 * Attention forward for selected query rows.
 * q [N][hq][d], k, v [N][hkv][d] (contiguous doubles); rows[0..nrows) are the
 * query positions to compute (rows == NULL means all N in order).
 * o [nrows][hq][d], lse [hq][nrows].
 * cu == NULL: one document. Returns 0, -1 on a bad argument, -2 when out of
 * host memory.
 */
int orc_attn_fwd(const double *q, const double *k, const double *v, int64_t N, int32_t hq,
                 int32_t hkv, int32_t d, double scale, int32_t causal, const int32_t *cu,
                 int32_t nseq, const int64_t *rows, int64_t nrows, double *o, double *lse) {
    if (hq <= 0 || hkv <= 0 || hq % hkv || d <= 0 || N <= 0) return -1;
    if (!rows) nrows = N;
    int64_t total = nrows * hq;
    int nt = orc_max_threads();
    double *scratch = (double *)malloc(sizeof(double) * N * nt);
    if (!scratch) return -2;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t w = 0; w < total; ++w) {
        double *s = scratch + (int64_t)orc_thread() * N;
        int64_t r = w / hq;
        int h = (int)(w % hq);
        int64_t i = rows ? rows[r] : r;
        lse[h * nrows + r] = orc_row_fwd(q, k, v, i, h, N, hq, hkv, d, scale, causal, cu, nseq, s,
                                         o + (r * hq + h) * d);
    }
    free(scratch);
    return 0;
}

/* --------------------------------------------------------------- O3 ---- */

/*
 * Attention backward (loss L = sum dO * O), textbook form:
 *   D_i   = sum_e dO_ie O_ie                    (O from the oracle's own O2)
 *   dp_ij = dO_i . v_j
 *   ds_ij = p_ij (dp_ij - D_i)
 *   dQ_i  = scale * sum_j ds_ij k_j
 *   dK_j  = scale * sum_{h in group} sum_i ds^h_ij q^h_i
 *   dV_j  = sum_{h in group} sum_i p^h_ij dO^h_i
 *
 * dQ is produced for rows[0..nrows) (rows == NULL: all N), dq [nrows][hq][d].
 * dK/dV are produced for keys [key_lo, key_hi), dk, dv [key_hi-key_lo][hkv][d].
 * Any output pointer may be NULL to skip that part.
 */
int orc_attn_bwd(const double *q, const double *k, const double *v, const double *dout,
                 int64_t N, int32_t hq, int32_t hkv, int32_t d, double scale, int32_t causal,
                 const int32_t *cu, int32_t nseq, const int64_t *rows, int64_t nrows,
                 int64_t key_lo, int64_t key_hi, double *dq, double *dk, double *dv) {
    if (hq <= 0 || hkv <= 0 || hq % hkv || d <= 0 || N <= 0) return -1;
    if (key_lo < 0 || key_hi > N || key_lo > key_hi) return -1;
    int G = hq / hkv;
    if (!rows) nrows = N;
    int nt = orc_max_threads();
    double *scratch = (double *)malloc(sizeof(double) * (N + d) * nt);
    if (!scratch) return -2;

    /* dQ rows: every row is self-contained. */
    if (dq) {
        int64_t total = nrows * hq;
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t w = 0; w < total; ++w) {
            double *s = scratch + (int64_t)orc_thread() * (N + d);
            double *o = s + N;
            int64_t r = w / hq;
            int h = (int)(w % hq);
            int g = h / G;
            int64_t i = rows ? rows[r] : r;
            double lse = orc_row_fwd(q, k, v, i, h, N, hq, hkv, d, scale, causal, cu, nseq, s, o);
            const double *doi = dout + (i * hq + h) * d;
            double D = 0.0;
            for (int e = 0; e < d; ++e) D += doi[e] * o[e];
            double *dqi = dq + (r * hq + h) * d;
            for (int e = 0; e < d; ++e) dqi[e] = 0.0;
            int64_t j0, j1;
            orc_key_range(i, N, causal, cu, nseq, &j0, &j1);
            for (int64_t j = j0; j < j1; ++j) {
                double p = exp(s[j] - lse);
                const double *vj = v + (j * hkv + g) * d;
                const double *kj = k + (j * hkv + g) * d;
                double dp = 0.0;
                for (int e = 0; e < d; ++e) dp += doi[e] * vj[e];
                double ds = p * (dp - D);
                for (int e = 0; e < d; ++e) dqi[e] += scale * ds * kj[e];
            }
        }
    }

    if ((dk || dv) && key_hi > key_lo) {
        /* Queries that can see a key in [key_lo, key_hi): under the causal
         * mask only i >= key_lo; with documents only those of the documents
         * the key range overlaps. Their LSE and D come first, row by row. */
        int64_t qlo, qhi;
        if (cu) {
            int b0 = orc_doc_of(key_lo, cu, nseq), b1 = orc_doc_of(key_hi - 1, cu, nseq);
            qlo = causal ? key_lo : cu[b0];
            qhi = cu[b1 + 1];
        } else {
            qlo = causal ? key_lo : 0;
            qhi = N;
        }
        int64_t nq = qhi - qlo;
        double *LSE = (double *)malloc(sizeof(double) * nq * hq);
        double *Dv = (double *)malloc(sizeof(double) * nq * hq);
        if (!LSE || !Dv) {
            free(LSE);
            free(Dv);
            free(scratch);
            return -2;
        }
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t w = 0; w < nq * hq; ++w) {
            double *s = scratch + (int64_t)orc_thread() * (N + d);
            double *o = s + N;
            int64_t i = qlo + w / hq;
            int h = (int)(w % hq);
            double lse = orc_row_fwd(q, k, v, i, h, N, hq, hkv, d, scale, causal, cu, nseq, s, o);
            const double *doi = dout + (i * hq + h) * d;
            double D = 0.0;
            for (int e = 0; e < d; ++e) D += doi[e] * o[e];
            LSE[w] = lse;
            Dv[w] = D;
        }
        int64_t nk = key_hi - key_lo;
#pragma omp parallel for schedule(dynamic, 4)
        for (int64_t w = 0; w < nk * hkv; ++w) {
            int64_t j = key_lo + w / hkv;
            int g = (int)(w % hkv);
            const double *kj = k + (j * hkv + g) * d;
            const double *vj = v + (j * hkv + g) * d;
            double *dkj = dk ? dk + ((j - key_lo) * hkv + g) * d : NULL;
            double *dvj = dv ? dv + ((j - key_lo) * hkv + g) * d : NULL;
            for (int e = 0; e < d; ++e) {
                if (dkj) dkj[e] = 0.0;
                if (dvj) dvj[e] = 0.0;
            }
            for (int64_t i = qlo; i < qhi; ++i) {
                int64_t a0, a1;
                orc_key_range(i, N, causal, cu, nseq, &a0, &a1);
                if (j < a0 || j >= a1) continue;
                for (int hh = 0; hh < G; ++hh) {
                    int h = g * G + hh;
                    const double *qi = q + (i * hq + h) * d;
                    const double *doi = dout + (i * hq + h) * d;
                    double sdot = 0.0, dp = 0.0;
                    for (int e = 0; e < d; ++e) {
                        sdot += qi[e] * kj[e];
                        dp += doi[e] * vj[e];
                    }
                    int64_t w2 = (i - qlo) * hq + h;
                    double p = exp(scale * sdot - LSE[w2]);
                    double ds = p * (dp - Dv[w2]);
                    for (int e = 0; e < d; ++e) {
                        if (dkj) dkj[e] += scale * ds * qi[e];
                        if (dvj) dvj[e] += p * doi[e];
                    }
                }
            }
        }
        free(LSE);
        free(Dv);
    }
    free(scratch);
    return 0;
}

/* Threads an OpenMP parallel region of this library uses (1 without OpenMP). */
int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
