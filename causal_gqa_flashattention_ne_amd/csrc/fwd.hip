// fwd.hip -- causal GQA FlashAttention forward for gfx950.
//
// One workgroup (4 waves) owns BM = 128 queries of one (batch, query head); wave w owns queries
// [32w, 32w + 32) of that block.  Keys/values stream through LDS in tiles of BN = 64, only up
// to the block's last query (tiles above the causal diagonal are never loaded).  RoPE is applied
// while tiles are loaded (queries once into registers, keys into LDS).
//
// The scores are formed transposed, S^T = K Q^T, so one lane owns one query column: the row
// max, the running sum l and the rescale of the output accumulator are all per lane, and the
// only cross-lane step is one exchange between the two lane halves (permlane32 swap).  The
// output is accumulated transposed as well, O^T += V^T P^T, with P^T taken straight from the
// score registers (its K index order is the accumulator's row order, and V^T is read from LDS
// in that same order).  exp2 with scale*log2(e) folded in; L = ln(sum) is written per row.
//
// Tiling plus an online softmax keeps the T x T matrix out of memory entirely (agentlenshq
// NanoEuler page, section "커널 구현").
#include "common.hpp"
#include "kernels.hpp"

namespace ne {

namespace {

constexpr int kFwdBM = 128;
constexpr int kFwdBN = 64;
constexpr int kThreads = 256;

__device__ inline float partner_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float partner_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdArgs a) {
    using M = Mfma<T>;
    constexpr int KW = M::KW;
    constexpr int NCH = D / (2 * KW);          // MFMA chunks over head_dim
    constexpr int KPAD = 16 / sizeof(T);       // row padding (elements) against bank conflicts
    constexpr int VPAD = 16 / sizeof(T);
    constexpr int VEC = 16 / sizeof(T);        // elements per 16-byte global access
    constexpr int NDT = D / 32;                // 32-row tiles of O^T

    __shared__ __attribute__((aligned(16))) T Ks[kFwdBN][D + KPAD];
    __shared__ __attribute__((aligned(16))) T Vt[D][kFwdBN + VPAD];

    const int T_ = a.T;
    const int nqt = (T_ + kFwdBM - 1) / kFwdBM;
    const int BH = a.B * a.Hq;
    // heaviest query blocks (largest causal extent) are dispatched first
    const int qt = nqt - 1 - (int)(blockIdx.x / BH);
    const int bh = (int)(blockIdx.x % BH);
    const int b = bh / a.Hq, h = bh % a.Hq;
    const int g = h / (a.Hq / a.Hkv);
    const int i0 = qt * kFwdBM;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int col = lane & 31, half = lane >> 5;

    const T* __restrict__ q = reinterpret_cast<const T*>(a.q) + ((size_t)(b * a.Hq + h) * T_) * D;
    const T* __restrict__ k = reinterpret_cast<const T*>(a.k) + ((size_t)(b * a.Hkv + g) * T_) * D;
    const T* __restrict__ v = reinterpret_cast<const T*>(a.v) + ((size_t)(b * a.Hkv + g) * T_) * D;
    const float* __restrict__ cs = a.rope_cs;

    // ---- this lane's query column: rotated, held as B operands of S^T = K Q^T ----
    const int qrow = i0 + 32 * w + col;
    typename M::op qop[NCH];
    {
        float x[D / 2];
        load_row_slots<T, D>(q + (size_t)qrow * D, cs, qrow, half, qrow < T_, x);
        slots_to_ops<T, D / 2>(x, qop);
    }

    f32x16 oacc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;   // running max, log2 units
    float l_run = 0.f;         // this lane's share of the running sum
    const float sl2 = a.scale * kLog2e;

    const int kv_end = min(T_, i0 + kFwdBM);
    const int wq_lo = i0 + 32 * w;      // wave's first query
    for (int j0 = 0; j0 < kv_end; j0 += kFwdBN) {
        __syncthreads();
        // ---- K tile -> LDS (rotated), V tile -> LDS transposed ----
        constexpr int CPR = D / VEC;                   // 16-byte chunks per row
        for (int ch = tid; ch < kFwdBN * CPR; ch += kThreads) {
            const int r = ch / CPR, d0 = (ch % CPR) * VEC;
            const int key = j0 + r;
            float kx[VEC], vx[VEC];
            if (key < T_) {
                load16<T>(k + (size_t)key * D + d0, kx);
                load16<T>(v + (size_t)key * D + d0, vx);
                if (cs) rope_rotate(kx, VEC, cs, D, key, d0, false);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) { kx[e] = 0.f; vx[e] = 0.f; }
            }
            store16<T>(&Ks[r][d0], kx);
#pragma unroll
            for (int e = 0; e < VEC; ++e) Vt[d0 + e][r] = from_f32<T>(vx[e]);
        }
        __syncthreads();
        if (j0 > wq_lo + 31) continue;   // every key of the tile is after every query of the wave

        // ---- S^T = K Q^T for the 64 keys: two 32x32 tiles ----
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            s[kt] = f32x16{};
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                typename M::op kop;
                if constexpr (KW == 8) {
                    kop = *reinterpret_cast<const bf16x8*>(&Ks[32 * kt + col][dslot<T, D>(c, half, 0)]);
                } else {
                    kop = Ks[32 * kt + col][dslot<T, D>(c, half, 0)];
                }
                s[kt] = M::mma(kop, qop[c], s[kt]);
            }
        }
        // ---- online softmax (per lane = per query) ----
        const bool diag = (j0 + kFwdBN - 1 > wq_lo);
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = s[kt][r] * sl2;
                if (diag && (j0 + 32 * kt + acc_row(r, half) > qrow)) x = -INFINITY;
                s[kt][r] = x;
                mx = fmaxf(mx, x);
            }
        mx = partner_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = exp2f(s[kt][r] - m_new);
                s[kt][r] = p;
                ls += p;
            }
        l_run = l_run * alpha + ls;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;

        // ---- O^T += V^T P^T ----
        constexpr int PCH = 64 / (2 * KW);   // MFMA chunks over the 64 keys
#pragma unroll
        for (int pc = 0; pc < PCH; ++pc) {
            typename M::op pop;
            const int kt = (pc * KW) / 16;
            const int r0 = (pc * KW) % 16;
            if constexpr (KW == 8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) pop[e] = (bf16)s[kt][r0 + e];
            } else {
                pop = s[kt][r0];
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                typename M::op vop;
                if constexpr (KW == 8) {
                    const int k0 = 32 * kt + acc_row(r0, half);       // 4 keys, then 4 more at +8
                    bf16x4 lo = *reinterpret_cast<const bf16x4*>(&Vt[32 * dt + col][k0]);
                    bf16x4 hi = *reinterpret_cast<const bf16x4*>(&Vt[32 * dt + col][k0 + 8]);
                    vop = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                } else {
                    vop = Vt[32 * dt + col][32 * kt + acc_row(r0, half)];
                }
                oacc[dt] = M::mma(vop, pop, oacc[dt]);
            }
        }
    }

    // ---- epilogue: O = O^T / l, L = ln(sum) ----
    const float l_tot = partner_sum(l_run);
    if (qrow < T_) {
        const float inv = 1.f / l_tot;
        T* __restrict__ o = reinterpret_cast<T*>(a.o) + ((size_t)(b * a.Hq + h) * T_ + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                const int d = 32 * dt + acc_row(r, half);
                store4<T>(o + d, oacc[dt][r] * inv, oacc[dt][r + 1] * inv, oacc[dt][r + 2] * inv,
                          oacc[dt][r + 3] * inv);
            }
        if (half == 0) a.lse[(size_t)(b * a.Hq + h) * T_ + qrow] = (m_run + log2f(l_tot)) * kLn2;
    }
}

}  // namespace

template <typename T, int D>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
    const int nqt = (a.T + kFwdBM - 1) / kFwdBM;
    const long blocks = (long)nqt * a.B * a.Hq;
    hipLaunchKernelGGL((fwd_kernel<T, D>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template hipError_t launch_fwd<float, 64>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<float, 32>(const FwdArgs&, hipStream_t);

}  // namespace ne
