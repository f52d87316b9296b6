/*
 * abi_caller.c -- a plain C program that uses libfa2.so through include/fa2.h
 * alone: device buffers from hipMalloc, results copied back with hipMemcpy,
 * no Python and no torch.  Built by __graft_entry__.build() with gcc; run by
 * tests/test_gpu_c_caller.py.  Exit status 0 and "abi_caller: ok" when every
 * check passes.
 *
 * The inputs make the answer a closed form, so no reference implementation is
 * needed here: with K = 0 every score is 0 and every live key weighs the
 * same, so O is the mean of the live rows of V and LSE = ln(number of live
 * keys) (the definition of attn_fwd in include/fa2.h with all s_ij = 0).
 * V holds small integers, so the means are computed exactly in double on the
 * host.  Error paths: an unsupported head dimension, a NULL pointer and a
 * misaligned pointer are refused before anything is enqueued.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "fa2.h"

static int failures = 0;

static void check(int ok, const char *what) {
    if (!ok) {
        printf("FAIL %s\n", what);
        failures++;
    }
}

static void *dev_alloc(size_t bytes) {
    void *p = NULL;
    if (hipMalloc(&p, bytes) != hipSuccess) {
        printf("hipMalloc of %zu bytes failed\n", bytes);
        exit(2);
    }
    return p;
}

static void to_dev(void *d, const void *h, size_t bytes) {
    if (hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) exit(2);
}

static void to_host(void *h, const void *d, size_t bytes) {
    if (hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost) != hipSuccess) exit(2);
}

/* V[bh][j][d]: small integers in [-5, 5] */
static float vval(int bh, int j, int d) { return (float)((bh * 5 + j * 7 + d * 3) % 11 - 5); }

/* forward on B*H heads of [N, D] float32 with K = 0; causal or not */
static void forward_case(int B, int H, int Nq, int Nk, int D, int causal) {
    const size_t nq = (size_t)B * H * Nq * D, nk = (size_t)B * H * Nk * D;
    float *q = malloc(nq * 4), *k = calloc(nk, 4), *v = malloc(nk * 4), *o = malloc(nq * 4);
    float *lse = malloc((size_t)B * H * Nq * 4);
    unsigned s = 12345u;
    for (size_t i = 0; i < nq; ++i) {
        s = s * 1664525u + 1013904223u;
        q[i] = (float)((s >> 8) & 0xFFFF) / 65536.0f - 0.5f;
    }
    for (int bh = 0; bh < B * H; ++bh)
        for (int j = 0; j < Nk; ++j)
            for (int d = 0; d < D; ++d) v[((size_t)bh * Nk + j) * D + d] = vval(bh, j, d);
    void *dq = dev_alloc(nq * 4), *dk = dev_alloc(nk * 4), *dv = dev_alloc(nk * 4);
    void *dout = dev_alloc(nq * 4), *dlse = dev_alloc((size_t)B * H * Nq * 4);
    to_dev(dq, q, nq * 4);
    to_dev(dk, k, nk * 4);
    to_dev(dv, v, nk * 4);
    fa2_status st = attn_fwd(dq, dk, dv, dout, (float *)dlse, B, H, Nq, Nk, D, 0.125f, causal,
                             FA2_F32, NULL);
    check(st == FA2_OK, "attn_fwd status");
    check(hipDeviceSynchronize() == hipSuccess, "synchronize after attn_fwd");
    to_host(o, dout, nq * 4);
    to_host(lse, dlse, (size_t)B * H * Nq * 4);
    double worst = 0.0, worst_lse = 0.0;
    for (int bh = 0; bh < B * H; ++bh)
        for (int i = 0; i < Nq; ++i) {
            const int live = causal ? i + 1 : Nk;
            for (int d = 0; d < D; ++d) {
                double mean = 0.0;
                for (int j = 0; j < live; ++j) mean += vval(bh, j, d);
                mean /= live;
                const double e = fabs(o[((size_t)bh * Nq + i) * D + d] - mean);
                if (e > worst) worst = e;
            }
            const double el = fabs(lse[(size_t)bh * Nq + i] - log((double)live));
            if (el > worst_lse) worst_lse = el;
        }
    printf("attn_fwd f32 B%d H%d Nq%d Nk%d D%d causal %d: max|O - mean V| %.2e, max|LSE - ln n| %.2e\n",
           B, H, Nq, Nk, D, causal, worst, worst_lse);
    check(worst <= 1e-4, "attn_fwd O");
    check(worst_lse <= 1e-4, "attn_fwd LSE");
    hipFree(dq);
    hipFree(dk);
    hipFree(dv);
    hipFree(dout);
    hipFree(dlse);
    free(q);
    free(k);
    free(v);
    free(o);
    free(lse);
}

/* flash-decoding: split then combine, one query row per head, K = 0 */
static void decode_case(int B, int H, int N, int D, int n_splits) {
    const size_t nq = (size_t)B * H * D, nk = (size_t)B * H * N * D;
    const size_t np = (size_t)B * H * n_splits;
    float *q = malloc(nq * 4), *k = calloc(nk, 4), *v = malloc(nk * 4), *o = malloc(nq * 4);
    for (size_t i = 0; i < nq; ++i) q[i] = (float)(i % 13) * 0.1f - 0.6f;
    for (int bh = 0; bh < B * H; ++bh)
        for (int j = 0; j < N; ++j)
            for (int d = 0; d < D; ++d) v[((size_t)bh * N + j) * D + d] = vval(bh, j, d);
    void *dq = dev_alloc(nq * 4), *dk = dev_alloc(nk * 4), *dv = dev_alloc(nk * 4);
    void *dout = dev_alloc(nq * 4);
    float *op = dev_alloc(np * D * 4), *mp = dev_alloc(np * 4), *lp = dev_alloc(np * 4);
    to_dev(dq, q, nq * 4);
    to_dev(dk, k, nk * 4);
    to_dev(dv, v, nk * 4);
    fa2_status st = attn_decode_split(dq, dk, dv, op, mp, lp, B, H, N, D, 0.09f, n_splits,
                                      FA2_F32, NULL);
    check(st == FA2_OK, "attn_decode_split status");
    st = attn_decode_combine(op, mp, lp, dout, B, H, D, n_splits, FA2_F32, NULL);
    check(st == FA2_OK, "attn_decode_combine status");
    check(hipDeviceSynchronize() == hipSuccess, "synchronize after decode");
    to_host(o, dout, nq * 4);
    double worst = 0.0;
    for (int bh = 0; bh < B * H; ++bh)
        for (int d = 0; d < D; ++d) {
            double mean = 0.0;
            for (int j = 0; j < N; ++j) mean += vval(bh, j, d);
            mean /= N;
            const double e = fabs(o[(size_t)bh * D + d] - mean);
            if (e > worst) worst = e;
        }
    printf("attn_decode f32 B%d H%d N%d D%d splits %d: max|O - mean V| %.2e\n", B, H, N, D,
           n_splits, worst);
    check(worst <= 1e-4, "attn_decode O");
    hipFree(dq);
    hipFree(dk);
    hipFree(dv);
    hipFree(dout);
    hipFree(op);
    hipFree(mp);
    hipFree(lp);
    free(q);
    free(k);
    free(v);
    free(o);
}

static void error_paths(void) {
    float *buf = dev_alloc(1 << 20);
    float *lse = dev_alloc(1 << 16);
    check(attn_fwd(buf, buf, buf, buf, lse, 1, 1, 8, 8, 96, 0.1f, 0, FA2_F32, NULL) ==
              FA2_ERR_UNSUPPORTED,
          "D = 96 refused");
    check(attn_fwd(NULL, buf, buf, buf, lse, 1, 1, 8, 8, 64, 0.1f, 0, FA2_F32, NULL) == FA2_ERR_NULL,
          "NULL q refused");
    check(attn_fwd((char *)buf + 4, buf, buf, buf, lse, 1, 1, 8, 8, 64, 0.1f, 0, FA2_F32, NULL) ==
              FA2_ERR_ALIGN,
          "misaligned q refused");
    check(attn_decode_split(buf, buf, buf, buf, lse, lse, 1, 1, 8, 64, 0.1f, 0, FA2_F32, NULL) !=
              FA2_OK,
          "zero splits refused");
    check(fa2_status_string(FA2_ERR_ALIGN) != NULL, "status string");
    hipFree(buf);
    hipFree(lse);
}

int main(void) {
    forward_case(1, 2, 100, 300, 64, 0);
    forward_case(2, 3, 77, 77, 64, 1);
    forward_case(1, 2, 130, 50, 128, 0);
    decode_case(2, 4, 1000, 128, 7);
    decode_case(1, 3, 5, 64, 16);
    error_paths();
    if (failures) {
        printf("abi_caller: %d failures\n", failures);
        return 1;
    }
    printf("abi_caller: ok\n");
    return 0;
}
