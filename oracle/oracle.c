/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow fp64 CPU reference for exact attention and for flash-decoding
 * partials.  Only tests/, the smoke check and the bench's CPU-baseline leg may
 * load it.  It shares no code, header, table or constant with the HIP library
 * under exact_attention_fa2_amd/csrc, and it includes nothing from there.
 *
 * Every function computes the plain definition with sequential fp64 loops:
 *
 *   "Flash attention, f32" (phobos-lang.dev), opening paragraph:
 *       O = softmax(Q K^T * scale) V, rows of Q against rows of K.
 *   "Flash Attention" (aarnphm.xyz), Definition 1 and Proposition 1 (safe
 *       softmax): subtracting the row maximum leaves the softmax unchanged and
 *       keeps every exponent non-positive.
 *   "Flash Attention", section FlashAttention 2: the per-row statistic kept for
 *       the backward pass is the log-sum-exp L = m + log(l); here in natural
 *       log of the *scaled* scores.
 *   "06: Fused attention" (phobos-lang.dev tutorial), attn_fwd: causal keeps
 *       key j for query i only when j <= i.  Masked keys are left out of the
 *       sum entirely (no finite stand-in for -infinity is used here).
 *   "Flash decoding" (linearalgebraforprogrammers.com), Overview of the
 *       algorithm: split s covers keys [n_s, n_{s+1}); it holds
 *       m_s = max_j s_j, l_s = sum_j exp(s_j - m_s), O_s = sum_j exp(s_j - m_s) V_j
 *       (unnormalised); combine takes m_g = max_s m_s,
 *       l_g = sum_s exp(m_s - m_g) l_s, O = sum_s exp(m_s - m_g) O_s / l_g.
 *       Scores include the scale factor (the page's split kernel multiplies
 *       the dot product by `scale`; its equations omit it).  Split size is
 *       S = ceil(N / n_splits); a split with no keys holds (-inf, 0, 0).
 *   Backward pass ("Flash Attention", section IO complexity, the paragraph on
 *       the backward pass; "06: Fused attention", the backward kernels): with
 *       P = softmax(scale Q K^T) (masked keys left out) and the upstream
 *       gradient dO of O = P V,
 *         dV = P^T dO,   dP = dO V^T,   D_i = rowsum(dO o O)_i,
 *         dS = P o (dP - D_i),   dQ = scale dS K,   dK = scale dS^T Q.
 *       D_i equals sum_j P_ij dP_ij, the term the softmax Jacobian reduces to.
 *
 * Layouts (all contiguous row-major, fp64):
 *   q [B,H,Nq,D], k and v [B,H,Nk,D], o [rows,D], lse [rows].
 *   A "row id" is r = (b*H + h)*Nq + i.
 *   Backward: dout [B,H,Nq,D]; for each selected head t: dq [t][Nq][D],
 *   dk and dv [t][Nk][D], delta [t][Nq].
 *
 * Return value: 0 on success, -1 on an invalid argument.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One output row of exact attention: O[i,:] and LSE[i] for query i of one
 * (b,h) slice.  qrow [D]; kh, vh [Nk,D] of the same (b,h). */
static void one_row(const double *qrow, const double *kh, const double *vh,
                    int Nk, int D, double scale, int nlive, double *orow,
                    double *lse, double *s /* scratch [Nk] */) {
    /* scores s_j = scale * <q_i, k_j> for live keys j < nlive */
    double mx = -INFINITY;
    for (int j = 0; j < nlive; ++j) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qrow[d] * kh[(size_t)j * D + d];
        s[j] = scale * acc;
        if (s[j] > mx) mx = s[j];
    }
    (void)Nk;
    /* safe softmax: e_j = exp(s_j - max), Z = sum e_j */
    double z = 0.0;
    for (int j = 0; j < nlive; ++j) {
        s[j] = exp(s[j] - mx);
        z += s[j];
    }
    /* O = sum_j e_j V_j / Z */
    for (int d = 0; d < D; ++d) orow[d] = 0.0;
    for (int j = 0; j < nlive; ++j) {
        const double w = s[j];
        const double *vr = vh + (size_t)j * D;
        for (int d = 0; d < D; ++d) orow[d] += w * vr[d];
    }
    for (int d = 0; d < D; ++d) orow[d] /= z;
    if (lse) *lse = mx + log(z);
}

/* Exact attention for a list of rows (or every row when rows == NULL).
 * o must hold nrows*D values and lse nrows values (lse may be NULL).
 * nthreads <= 0 lets OpenMP choose. */
int oracle_attn_rows(const double *q, const double *k, const double *v,
                     int B, int H, int Nq, int Nk, int D, double scale, int causal,
                     const long long *rows, long long nrows,
                     double *o, double *lse, int nthreads) {
    if (!q || !k || !v || !o || B < 1 || H < 1 || Nq < 1 || Nk < 1 || D < 1) return -1;
    if (causal && Nq != Nk) return -1;
    const long long total = (long long)B * H * Nq;
    if (!rows) nrows = total;
    if (nrows < 0) return -1;
    for (long long t = 0; t < nrows && rows; ++t)
        if (rows[t] < 0 || rows[t] >= total) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Nk);
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (long long t = 0; t < nrows; ++t) {
            if (!s) continue;
            const long long r = rows ? rows[t] : t;
            const long long bh = r / Nq;
            const int i = (int)(r % Nq);
            const double *qrow = q + (size_t)r * D;
            const double *kh = k + (size_t)bh * Nk * D;
            const double *vh = v + (size_t)bh * Nk * D;
            const int nlive = causal ? i + 1 : Nk;
            one_row(qrow, kh, vh, Nk, D, scale, nlive, o + (size_t)t * D,
                    lse ? lse + t : NULL, s);
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/* Flash-decoding partials, one query row per (b,h).
 * q [B,H,D]; k, v [B,H,N,D]; o_part [B,H,n_splits,D]; m_part, l_part [B,H,n_splits]. */
int oracle_decode_split(const double *q, const double *k, const double *v,
                        int B, int H, int N, int D, double scale, int n_splits,
                        double *o_part, double *m_part, double *l_part) {
    if (!q || !k || !v || !o_part || !m_part || !l_part) return -1;
    if (B < 1 || H < 1 || N < 1 || D < 1 || n_splits < 1) return -1;
    const long long S = ((long long)N + n_splits - 1) / n_splits;
    double *s = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    if (!s) return -1;
    for (long long bh = 0; bh < (long long)B * H; ++bh) {
        const double *qr = q + (size_t)bh * D;
        const double *kh = k + (size_t)bh * N * D;
        const double *vh = v + (size_t)bh * N * D;
        for (int sp = 0; sp < n_splits; ++sp) {
            const long long n0 = (long long)sp * S;
            const long long n1 = n0 + S < N ? n0 + S : N;
            double *op = o_part + ((size_t)bh * n_splits + sp) * D;
            double mx = -INFINITY, l = 0.0;
            for (int d = 0; d < D; ++d) op[d] = 0.0;
            for (long long j = n0; j < n1; ++j) {
                double acc = 0.0;
                for (int d = 0; d < D; ++d) acc += qr[d] * kh[(size_t)j * D + d];
                s[j - n0] = scale * acc;
                if (s[j - n0] > mx) mx = s[j - n0];
            }
            for (long long j = n0; j < n1; ++j) {
                const double w = exp(s[j - n0] - mx);
                l += w;
                for (int d = 0; d < D; ++d) op[d] += w * vh[(size_t)j * D + d];
            }
            m_part[(size_t)bh * n_splits + sp] = mx; /* -inf for an empty split */
            l_part[(size_t)bh * n_splits + sp] = l;  /* 0 for an empty split */
        }
    }
    free(s);
    return 0;
}

/* Merge of flash-decoding partials.  o [B,H,D]. */
int oracle_decode_combine(const double *o_part, const double *m_part,
                          const double *l_part, int B, int H, int D, int n_splits,
                          double *o) {
    if (!o_part || !m_part || !l_part || !o || B < 1 || H < 1 || D < 1 || n_splits < 1)
        return -1;
    for (long long bh = 0; bh < (long long)B * H; ++bh) {
        const double *mp = m_part + (size_t)bh * n_splits;
        const double *lp = l_part + (size_t)bh * n_splits;
        double mg = -INFINITY;
        for (int sp = 0; sp < n_splits; ++sp)
            if (mp[sp] > mg) mg = mp[sp];
        double lg = 0.0;
        /* a split with m_s = -inf carries no keys: its weight is exactly zero */
        for (int sp = 0; sp < n_splits; ++sp)
            if (mp[sp] != -INFINITY) lg += exp(mp[sp] - mg) * lp[sp];
        double *orow = o + (size_t)bh * D;
        for (int d = 0; d < D; ++d) {
            double a = 0.0;
            for (int sp = 0; sp < n_splits; ++sp)
                if (mp[sp] != -INFINITY)
                    a += exp(mp[sp] - mg) * o_part[((size_t)bh * n_splits + sp) * D + d];
            orow[d] = a / lg;
        }
    }
    return 0;
}

/* Gradients of O = softmax(scale Q K^T) V for the heads listed in `heads`
 * (indices b*H + h; every head when heads == NULL).  Per head the whole
 * probability matrix is formed in fp64 (Nq x Nk doubles of scratch). */
int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dout,
                    int B, int H, int Nq, int Nk, int D, double scale, int causal,
                    const long long *heads, long long nheads,
                    double *dq, double *dk, double *dv, double *delta, int nthreads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv || !delta) return -1;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || D < 1) return -1;
    if (causal && Nq != Nk) return -1;
    const long long total = (long long)B * H;
    if (!heads) nheads = total;
    if (nheads < 0) return -1;
    for (long long t = 0; t < nheads && heads; ++t)
        if (heads[t] < 0 || heads[t] >= total) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int bad = 0;
#pragma omp parallel
    {
        double *P = (double *)malloc(sizeof(double) * (size_t)Nq * Nk);
        double *O = (double *)malloc(sizeof(double) * (size_t)Nq * D);
        if (!P || !O) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long long t = 0; t < nheads; ++t) {
            if (!P || !O) continue;
            const long long bh = heads ? heads[t] : t;
            const double *qh = q + (size_t)bh * Nq * D;
            const double *kh = k + (size_t)bh * Nk * D;
            const double *vh = v + (size_t)bh * Nk * D;
            const double *gh = dout + (size_t)bh * Nq * D;
            double *dqh = dq + (size_t)t * Nq * D;
            double *dkh = dk + (size_t)t * Nk * D;
            double *dvh = dv + (size_t)t * Nk * D;
            double *dlt = delta + (size_t)t * Nq;
            /* P: the softmax of each row over its live keys, 0 for masked keys */
            for (int i = 0; i < Nq; ++i) {
                const int nlive = causal ? i + 1 : Nk;
                double *pr = P + (size_t)i * Nk;
                double mx = -INFINITY;
                for (int j = 0; j < nlive; ++j) {
                    double acc = 0.0;
                    for (int d = 0; d < D; ++d) acc += qh[(size_t)i * D + d] * kh[(size_t)j * D + d];
                    pr[j] = scale * acc;
                    if (pr[j] > mx) mx = pr[j];
                }
                double z = 0.0;
                for (int j = 0; j < nlive; ++j) {
                    pr[j] = exp(pr[j] - mx);
                    z += pr[j];
                }
                for (int j = 0; j < nlive; ++j) pr[j] /= z;
                for (int j = nlive; j < Nk; ++j) pr[j] = 0.0;
            }
            /* O = P V and D_i = rowsum(dO o O) */
            for (int i = 0; i < Nq; ++i) {
                double di = 0.0;
                for (int d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int j = 0; j < Nk; ++j) acc += P[(size_t)i * Nk + j] * vh[(size_t)j * D + d];
                    O[(size_t)i * D + d] = acc;
                    di += gh[(size_t)i * D + d] * acc;
                }
                dlt[i] = di;
            }
            /* dV = P^T dO */
            for (int j = 0; j < Nk; ++j)
                for (int d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int i = 0; i < Nq; ++i) acc += P[(size_t)i * Nk + j] * gh[(size_t)i * D + d];
                    dvh[(size_t)j * D + d] = acc;
                }
            /* dS = P o (dO V^T - D_i), stored over P */
            for (int i = 0; i < Nq; ++i)
                for (int j = 0; j < Nk; ++j) {
                    double dp = 0.0;
                    for (int d = 0; d < D; ++d) dp += gh[(size_t)i * D + d] * vh[(size_t)j * D + d];
                    P[(size_t)i * Nk + j] *= dp - dlt[i];
                }
            /* dQ = scale dS K,  dK = scale dS^T Q */
            for (int i = 0; i < Nq; ++i)
                for (int d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int j = 0; j < Nk; ++j) acc += P[(size_t)i * Nk + j] * kh[(size_t)j * D + d];
                    dqh[(size_t)i * D + d] = scale * acc;
                }
            for (int j = 0; j < Nk; ++j)
                for (int d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int i = 0; i < Nq; ++i) acc += P[(size_t)i * Nk + j] * qh[(size_t)i * D + d];
                    dkh[(size_t)j * D + d] = scale * acc;
                }
        }
        free(P);
        free(O);
    }
    return bad ? -1 : 0;
}
