/* Drives the double-precision oracle (oracle/ne_oracle.c, linked in) on small shapes under
 * AddressSanitizer and UndefinedBehaviorSanitizer: every buffer is allocated at its exact size,
 * so any read or write past an array ends the run with a report.  Returns 0 when every call
 * succeeds and a few exact properties hold (T = 1: O = V; RoPE at position 0 is the identity;
 * the inverse rotation undoes the forward one), 1 otherwise. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int ora_attn(int B, int Hq, int Hkv, int T, int D, double theta, double scale, const double* q,
             const double* k, const double* v, const double* dO, double* o, double* L, double* dq,
             double* dk, double* dv, const unsigned char* group_mask, int nthreads);
void ora_rope(int B, int H, int T, int D, double theta, int pos_offset, int inverse, const double* x,
              double* y);

static double* filled(long n, unsigned seed) {
    double* p = malloc(sizeof(double) * (size_t)n);
    for (long i = 0; i < n; ++i) {
        seed = seed * 1103515245u + 12345u;
        p[i] = ((seed >> 8) & 0xffff) / 32768.0 - 1.0;
    }
    return p;
}

static int run(int B, int Hq, int Hkv, int T, int D, double theta, int backward, int mask_half) {
    const long nq = (long)B * Hq * T * D, nk = (long)B * Hkv * T * D;
    double *q = filled(nq, 1), *k = filled(nk, 2), *v = filled(nk, 3), *dO = filled(nq, 4);
    double *o = malloc(sizeof(double) * nq), *L = malloc(sizeof(double) * (size_t)B * Hq * T);
    double *dq = malloc(sizeof(double) * nq), *dk = malloc(sizeof(double) * nk), *dv = malloc(sizeof(double) * nk);
    unsigned char* gm = NULL;
    if (mask_half) {
        gm = malloc((size_t)B * Hkv);
        for (int i = 0; i < B * Hkv; ++i) gm[i] = (unsigned char)(i % 2);
    }
    int bad = ora_attn(B, Hq, Hkv, T, D, theta, 0.0, q, k, v, backward ? dO : NULL, o, L, dq, dk, dv, gm, 2) != 0;
    if (!bad && T == 1 && !mask_half) {               /* a single key: O = V of the group */
        const int G = Hq / Hkv;
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < Hq; ++h)
                for (int d = 0; d < D; ++d)
                    if (fabs(o[((long)b * Hq + h) * D + d] - v[((long)b * Hkv + h / G) * D + d]) > 1e-12) bad = 1;
    }
    free(q); free(k); free(v); free(dO); free(o); free(L); free(dq); free(dk); free(dv); free(gm);
    if (bad) fprintf(stderr, "attention B%d Hq%d Hkv%d T%d D%d failed\n", B, Hq, Hkv, T, D);
    return bad;
}

static int rope_roundtrip(int B, int H, int T, int D, int pos_offset) {
    const long n = (long)B * H * T * D;
    double *x = filled(n, 5), *y = malloc(sizeof(double) * n), *z = malloc(sizeof(double) * n);
    ora_rope(B, H, T, D, 10000.0, pos_offset, 0, x, y);
    ora_rope(B, H, T, D, 10000.0, pos_offset, 1, y, z);
    int bad = 0;
    for (long i = 0; i < n; ++i)
        if (fabs(z[i] - x[i]) > 1e-12) bad = 1;
    if (pos_offset == 0)                              /* row 0 of every head is not rotated */
        for (long r = 0; r < (long)B * H; ++r)
            for (int d = 0; d < D; ++d)
                if (y[r * T * D + d] != x[r * T * D + d]) bad = 1;
    free(x); free(y); free(z);
    if (bad) fprintf(stderr, "rope B%d H%d T%d D%d offset %d failed\n", B, H, T, D, pos_offset);
    return bad;
}

int main(void) {
    int bad = 0;
    bad |= run(1, 2, 1, 1, 4, 10000.0, 1, 0);
    bad |= run(2, 4, 2, 7, 8, 10.0, 1, 0);
    bad |= run(1, 3, 3, 13, 6, 0.0, 1, 0);
    bad |= run(2, 6, 2, 33, 32, 10000.0, 1, 1);       /* half of the kv groups selected */
    bad |= run(1, 4, 2, 65, 64, 10000.0, 0, 0);       /* forward only (dO = NULL) */
    bad |= run(1, 1, 1, 1, 2, 10000.0, 1, 0);
    bad |= ora_attn(0, 2, 1, 4, 4, 1.0, 0.0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1) != -1;
    bad |= ora_attn(1, 3, 2, 4, 4, 1.0, 0.0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1) != -1;
    bad |= rope_roundtrip(2, 3, 9, 8, 0);
    bad |= rope_roundtrip(1, 2, 5, 64, 37);
    printf(bad ? "FAILED\n" : "ok\n");
    return bad;
}
