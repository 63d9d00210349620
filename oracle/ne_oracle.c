/*
 * ne_oracle.c -- plain, slow, obviously correct causal GQA attention with RoPE, in double.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity oracle for the HIP library.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.  It shares no source,
 * header, table or helper with the GPU path.
 *
 * What it computes (the plain definition; FlashAttention reaches the same result up to rounding
 * order, because tiling plus online softmax is an exact reordering -- agentlenshq page
 * "NanoEuler: C와 CUDA로 밑바닥부터 구축한 GPT-2 규모의 LLM", section "커널 구현"):
 *
 *   RoPE on queries and keys (same page, section "기술 사양"; byte-level GPT page, "Core
 *   Mechanics"): pairs (x[2i], x[2i+1]) at position t are rotated by the angle t * w_i with
 *   w_i = theta^(-2i/D).  theta <= 0 switches RoPE off (identity).
 *   Grouped-query attention (page 3, "기술 사양"): query head h reads kv head h / (Hq/Hkv).
 *   Causal self-attention (byte-level GPT page, "Core Mechanics"): query i sees keys j <= i.
 *   S_ij = s <q~_i, k~_j>, P = row softmax over j <= i (P_ij = 0 exactly above the diagonal),
 *   L_i = m_i + ln l_i (natural log), O_i = sum_j P_ij v_j.
 *   Backward for the loss <dO, O> (hand-written backward, page 1 "Core Mechanics"):
 *   dP_ij = <dO_i, v_j>, D_i = <dO_i, O_i>, dS_ij = P_ij (dP_ij - D_i),
 *   dq~_i = s sum_j dS_ij k~_j, dk~_j = s sum_i dS_ij q~_i, dv_j = sum_i P_ij dO_i,
 *   then dq = R^T dq~, dk = sum over the group's heads of R^T dk~, dv = sum over the heads.
 *
 * The T x T matrices P and dS are stored in full, on purpose: this is the definition, not a
 * fast kernel.  Parallelism is OpenMP over independent (batch, kv group) pairs only, in the
 * style of the CPU engine the pages describe (libm + OpenMP, page 1 "Core Mechanics").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int ora_version(void) { return 1; }

int ora_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Rotate one row x[0..D) at absolute position pos; inverse applies R^T (angle -a). */
static void rope_row(const double* x, double* y, int D, double theta, long pos, int inverse) {
    if (theta <= 0.0) {
        for (int d = 0; d < D; ++d) y[d] = x[d];
        return;
    }
    for (int i = 0; i < D / 2; ++i) {
        double w = pow(theta, -(2.0 * i) / (double)D);
        double a = (double)pos * w;
        double c = cos(a), s = sin(a);
        if (inverse) s = -s;
        double x0 = x[2 * i], x1 = x[2 * i + 1];
        y[2 * i] = x0 * c - x1 * s;
        y[2 * i + 1] = x0 * s + x1 * c;
    }
}

/* y[b,h,t,:] = R_(t+pos_offset) x[b,h,t,:]  (or R^T when inverse != 0). */
void ora_rope(int B, int H, int T, int D, double theta, int pos_offset, int inverse,
              const double* x, double* y) {
    long rows = (long)B * H * T;
    for (long r = 0; r < rows; ++r) {
        long t = r % T;
        rope_row(x + r * D, y + r * D, D, theta, t + pos_offset, inverse);
    }
}

static double dot(const double* a, const double* b, int n) {
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += a[i] * b[i];
    return s;
}

/*
 * Forward (and, when dO != NULL, backward) for every (b, g) selected by group_mask
 * (NULL = all).  Layout [B, H, T, D] contiguous for q, k, v, dO, o, dq, dk, dv; L is [B, Hq, T].
 * scale <= 0 means 1/sqrt(D).  Outputs of unselected groups are left untouched.
 * Returns 0, or -1 on a bad shape, -2 when memory runs out.
 */
int ora_attn(int B, int Hq, int Hkv, int T, int D, double theta, double scale,
             const double* q, const double* k, const double* v, const double* dO,
             double* o, double* L, double* dq, double* dk, double* dv,
             const unsigned char* group_mask, int nthreads) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0 || D <= 0 || (D % 2) || (Hq % Hkv)) return -1;
    const int G = Hq / Hkv;
    const double s = scale > 0.0 ? scale : 1.0 / sqrt((double)D);
    const long TD = (long)T * D;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (long bg = 0; bg < (long)B * Hkv; ++bg) {
        if (group_mask && !group_mask[bg]) continue;
        const long b = bg / Hkv, g = bg % Hkv;
        double* kr = malloc(sizeof(double) * TD);
        double* qr = malloc(sizeof(double) * TD);
        double* P = calloc((size_t)T * T, sizeof(double));
        double* dS = calloc((size_t)T * T, sizeof(double));
        double* dqr = malloc(sizeof(double) * TD);
        double* dkr = malloc(sizeof(double) * TD);
        double* tmp = malloc(sizeof(double) * D);
        double* Srow = malloc(sizeof(double) * T);
        if (!kr || !qr || !P || !dS || !dqr || !dkr || !tmp || !Srow) {
            failed = 1;
            goto done;
        }
        const double* kg = k + (b * Hkv + g) * TD;
        const double* vg = v + (b * Hkv + g) * TD;
        for (int t = 0; t < T; ++t) rope_row(kg + (long)t * D, kr + (long)t * D, D, theta, t, 0);
        if (dO) {
            memset(dk + (b * Hkv + g) * TD, 0, sizeof(double) * TD);
            memset(dv + (b * Hkv + g) * TD, 0, sizeof(double) * TD);
        }
        for (int hh = 0; hh < G; ++hh) {
            const long h = g * G + hh;
            const long off = (b * Hq + h) * TD;
            const double* qh = q + off;
            double* oh = o + off;
            double* Lh = L + (b * Hq + h) * (long)T;
            for (int t = 0; t < T; ++t) rope_row(qh + (long)t * D, qr + (long)t * D, D, theta, t, 0);
            /* forward: scores, masked softmax, L, O */
            for (int i = 0; i < T; ++i) {
                double m = -INFINITY;
                for (int j = 0; j <= i; ++j) {
                    Srow[j] = s * dot(qr + (long)i * D, kr + (long)j * D, D);
                    if (Srow[j] > m) m = Srow[j];
                }
                double l = 0.0;
                for (int j = 0; j <= i; ++j) l += exp(Srow[j] - m);
                for (int j = 0; j <= i; ++j) P[(long)i * T + j] = exp(Srow[j] - m) / l;
                Lh[i] = m + log(l);
                for (int d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int j = 0; j <= i; ++j) acc += P[(long)i * T + j] * vg[(long)j * D + d];
                    oh[(long)i * D + d] = acc;
                }
            }
            if (!dO) continue;
            /* backward */
            const double* dOh = dO + off;
            for (int i = 0; i < T; ++i) {
                double Di = dot(dOh + (long)i * D, oh + (long)i * D, D);
                for (int j = 0; j <= i; ++j) {
                    double dP = dot(dOh + (long)i * D, vg + (long)j * D, D);
                    dS[(long)i * T + j] = P[(long)i * T + j] * (dP - Di);
                }
            }
            for (int i = 0; i < T; ++i)
                for (int d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int j = 0; j <= i; ++j) acc += dS[(long)i * T + j] * kr[(long)j * D + d];
                    dqr[(long)i * D + d] = s * acc;
                }
            for (int j = 0; j < T; ++j)
                for (int d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int i = j; i < T; ++i) acc += dS[(long)i * T + j] * qr[(long)i * D + d];
                    dkr[(long)j * D + d] = s * acc;
                }
            for (int t = 0; t < T; ++t) {
                rope_row(dqr + (long)t * D, dq + off + (long)t * D, D, theta, t, 1);
                rope_row(dkr + (long)t * D, tmp, D, theta, t, 1);
                double* dkt = dk + (b * Hkv + g) * TD + (long)t * D;
                for (int d = 0; d < D; ++d) dkt[d] += tmp[d];
            }
            for (int j = 0; j < T; ++j) {
                double* dvj = dv + (b * Hkv + g) * TD + (long)j * D;
                for (int d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int i = j; i < T; ++i) acc += P[(long)i * T + j] * dOh[(long)i * D + d];
                    dvj[d] += acc;
                }
            }
        }
    done:
        free(kr); free(qr); free(P); free(dS); free(dqr); free(dkr); free(tmp); free(Srow);
    }
    return failed ? -2 : 0;
}
