// bwd.hip -- causal GQA FlashAttention backward for gfx950 (hand-written backward of the forward
// in fwd.hip; ai-paper-delta NanoEuler page, "Core Mechanics").
//
// Three launches:
//   1. bwd_pre:  delta_i = sum_d dO_id * O_id  (float32).
//   2. bwd_main: key/value-tile major.  A workgroup owns BN = 128 keys of one (batch, kv head)
//      and one contiguous share of that tile's steps; wave w owns keys [32w, 32w + 32).  The
//      steps are every (query head of the kv group, query tile at or after the tile's first key)
//      (tiles wholly before the diagonal are skipped); a tile's steps are cut into as many shares
//      as make about a thousand workgroups (one share at long sequences), so that short
//      sequences still fill the GPU (bwd_f32_splits).  Each step recomputes
//          S = Q~ K~^T,  P = exp(scale*S - L),  dP = dO V^T,  dS = P * (dP - delta),
//          dV^T += dO^T P,  dK~^T += Q~^T dS,  dQ~_tile = dS K~ (scale applied).
//      S is formed untransposed here, so one lane owns one key: P and dS are then the B operands
//      of the dV^T / dK^T products directly from the accumulator registers (the K order of those
//      products is the accumulator's row order, and Q^T / dO^T are read from LDS in that order).
//      dS goes through LDS once per step so that all four waves' keys feed the dQ product.
//      dK~ and dV of the share are summed in registers (the group sum over query heads) and
//      stored into the share's own workspace slice; an empty share stores zeros.  A key tile's
//      contribution to dQ~ of the step's queries is stored (plain stores) into that key tile's own
//      dQ slice: each element of a slice has exactly one writer (one step of one share, one wave).
//   3. bwd_dq:   dQ = R^T (sum of the dQ~ slices of key tiles 0 .. the row's own), and
//      dK = R^T (scale sum of the dK~ slices) and dV = sum of the dV slices, converted to the
//      element type (R^T is linear, so un-rotating the sum equals summing the un-rotated parts).
//      Every sum is taken in slice order, so dQ, dK and dV are deterministic (no atomics).
#include "common.hpp"
#include "kernels.hpp"

namespace ne {

namespace {

constexpr int kThreads = 256;
constexpr int kBwdBN = 128;

template <typename T> struct BwdTile { static constexpr int BM = 64; };
template <> struct BwdTile<float> { static constexpr int BM = 32; };

// K index (key within the 128-key tile) of (chunk c, half h, item e) for the dQ product.
template <typename T>
__device__ constexpr inline int kslot(int c, int h, int e) {
    if constexpr (Mfma<T>::KW == 8) return 16 * c + 8 * h + e;
    else return c + h * (kBwdBN / 2);
}

// ---------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdArgs a) {
    constexpr int VEC = 16 / sizeof(T);
    constexpr int TPR = D / VEC;                       // threads per row (power of two)
    const long rows = (long)a.B * a.Hq * a.T;
    const long gid = (long)blockIdx.x * kThreads + threadIdx.x;
    const long row = gid / TPR;
    const int part = (int)(gid % TPR);
    float sum = 0.f;
    if (row < rows) {
        float o[VEC], d[VEC];
        load16<T>(reinterpret_cast<const T*>(a.o) + row * D + part * VEC, o);
        load16<T>(reinterpret_cast<const T*>(a.dout) + row * D + part * VEC, d);
#pragma unroll
        for (int e = 0; e < VEC; ++e) sum += o[e] * d[e];
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) sum += __shfl_xor(sum, off, 64);
    if (row < rows && part == 0) a.delta[row] = sum;
}

// ---------------------------------------------------------------------------------------------
template <typename T, int D>
struct BwdSmem {
    static constexpr int BM = BwdTile<T>::BM;
    static constexpr int PAD = 16 / sizeof(T);
    static constexpr int KT = 0;                                          // [D][BN + PAD]
    static constexpr int QS = KT + D * (kBwdBN + PAD) * (int)sizeof(T);   // [BM][D + PAD]
    static constexpr int QT = QS + BM * (D + PAD) * (int)sizeof(T);       // [D][BM + PAD]
    static constexpr int DOS = QT + D * (BM + PAD) * (int)sizeof(T);      // [BM][D + PAD]
    static constexpr int DOT = DOS + BM * (D + PAD) * (int)sizeof(T);     // [D][BM + PAD]
    static constexpr int DSS = DOT + D * (BM + PAD) * (int)sizeof(T);     // [BM][BN + PAD]
    static constexpr int LS = DSS + BM * (kBwdBN + PAD) * (int)sizeof(T); // [BM] float
    static constexpr int DL = LS + BM * 4;                                 // [BM] float
    static constexpr int BYTES = DL + BM * 4;
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_main_kernel(BwdArgs a) {
    using M = Mfma<T>;
    using L = BwdSmem<T, D>;
    constexpr int KW = M::KW;
    constexpr int BM = L::BM;
    constexpr int NQT = BM / 32;                 // 32-query tiles per step
    constexpr int NDT = D / 32;                  // 32-row tiles over head_dim
    constexpr int NCH = D / (2 * KW);            // chunks over head_dim
    constexpr int PCH = BM / (2 * KW);           // chunks over the step's queries
    constexpr int QCH = kBwdBN / (2 * KW);       // chunks over the tile's keys
    constexpr int PAD = L::PAD;
    constexpr int VEC = 16 / sizeof(T);
    constexpr int KTS = kBwdBN + PAD, RS = D + PAD, TS = BM + PAD, SS = kBwdBN + PAD;

    extern __shared__ __attribute__((aligned(16))) char smem[];
    T* Kt_s = reinterpret_cast<T*>(smem + L::KT);
    T* Q_s = reinterpret_cast<T*>(smem + L::QS);
    T* Qt_s = reinterpret_cast<T*>(smem + L::QT);
    T* dO_s = reinterpret_cast<T*>(smem + L::DOS);
    T* dOt_s = reinterpret_cast<T*>(smem + L::DOT);
    T* dS_s = reinterpret_cast<T*>(smem + L::DSS);
    float* L_s = reinterpret_cast<float*>(smem + L::LS);
    float* D_s = reinterpret_cast<float*>(smem + L::DL);

    const int T_ = a.T;
    const int BG = a.B * a.Hkv;
    const int nkt = (T_ + kBwdBN - 1) / kBwdBN;
    const int nsplit = a.nsplit;                 // shares per key tile
    const int unit = (int)(blockIdx.x % (unsigned)(nkt * BG));
    const int sp = (int)(blockIdx.x / (unsigned)(nkt * BG));
    const int jt = unit / BG;                    // first blocks own the earliest keys (most work)
    const int bg = unit % BG;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int G = a.Hq / a.Hkv;
    const int j0 = jt * kBwdBN;
    const int nq = (T_ - j0 + BM - 1) / BM;      // query tiles at or after the first key
    const long s_tot = (long)G * nq;
    const int s_begin = (int)(s_tot * sp / nsplit), s_end = (int)(s_tot * (sp + 1) / nsplit);

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int kw0 = j0 + 32 * w;                 // wave's first key
    const int key = kw0 + col;                   // this lane's key
    const float* __restrict__ cs = a.rope_cs;
    const float sl2 = a.scale * kLog2e;

    // ---- this lane's key row: rotated K and V as B operands; K~^T into LDS for dQ ----
    typename M::op kop[NCH], vop[NCH];
    {
        const size_t base = ((size_t)(b * a.Hkv + g) * T_ + key) * D;
        float kx[D / 2], vx[D / 2];
        load_row_slots<T, D>(reinterpret_cast<const T*>(a.k) + base, cs, key, half, key < T_, kx);
        load_row_slots<T, D>(reinterpret_cast<const T*>(a.v) + base, nullptr, key, half, key < T_, vx);
        slots_to_ops<T, D / 2>(kx, kop);
        slots_to_ops<T, D / 2>(vx, vop);
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int e = 0; e < KW; ++e)
                Kt_s[dslot<T, D>(c, half, e) * KTS + 32 * w + col] = from_f32<T>(kx[c * KW + e]);
    }

    f32x16 dkt[NDT], dvt[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) { dkt[i] = f32x16{}; dvt[i] = f32x16{}; }

    for (int st = s_begin; st < s_end; ++st) {
        const int hh = st / nq;
        const int i0 = j0 + (st % nq) * BM;
        const int h = g * G + hh;
        const size_t hrow = (size_t)(b * a.Hq + h) * T_;
        const T* __restrict__ q = reinterpret_cast<const T*>(a.q) + hrow * D;
        const T* __restrict__ dout = reinterpret_cast<const T*>(a.dout) + hrow * D;
        {
            __syncthreads();
            // ---- Q~ and dO tiles -> LDS, row-major and transposed; L (log2 units), delta ----
            constexpr int CPR = D / VEC;
            for (int ch = tid; ch < BM * CPR; ch += kThreads) {
                const int r = ch / CPR, d0 = (ch % CPR) * VEC;
                const int qi = i0 + r;
                float qx[VEC], gx[VEC];
                if (qi < T_) {
                    load16<T>(q + (size_t)qi * D + d0, qx);
                    load16<T>(dout + (size_t)qi * D + d0, gx);
                    if (cs) rope_rotate(qx, VEC, cs, D, qi, d0, false);
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) { qx[e] = 0.f; gx[e] = 0.f; }
                }
                store16<T>(Q_s + r * RS + d0, qx);
                store16<T>(dO_s + r * RS + d0, gx);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    Qt_s[(d0 + e) * TS + r] = from_f32<T>(qx[e]);
                    dOt_s[(d0 + e) * TS + r] = from_f32<T>(gx[e]);
                }
            }
            for (int r = tid; r < BM; r += kThreads) {
                const int qi = i0 + r;
                L_s[r] = qi < T_ ? a.lse[hrow + qi] * kLog2e : INFINITY;
                D_s[r] = qi < T_ ? a.delta[hrow + qi] : 0.f;
            }
            __syncthreads();

            const bool active = (kw0 < T_) && (kw0 <= i0 + BM - 1);
            if (active) {
                f32x16 s[NQT], dp[NQT];
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) {
                    s[qt] = f32x16{};
                    dp[qt] = f32x16{};
#pragma unroll
                    for (int c = 0; c < NCH; ++c) {
                        typename M::op qa, ga;
                        if constexpr (KW == 8) {
                            qa = *reinterpret_cast<const bf16x8*>(Q_s + (32 * qt + col) * RS + dslot<T, D>(c, half, 0));
                            ga = *reinterpret_cast<const bf16x8*>(dO_s + (32 * qt + col) * RS + dslot<T, D>(c, half, 0));
                        } else {
                            qa = Q_s[(32 * qt + col) * RS + dslot<T, D>(c, half, 0)];
                            ga = dO_s[(32 * qt + col) * RS + dslot<T, D>(c, half, 0)];
                        }
                        s[qt] = M::mma(qa, kop[c], s[qt]);
                        dp[qt] = M::mma(ga, vop[c], dp[qt]);
                    }
                }
                // P = exp2(S*scale*log2e - L*log2e), dS = P * (dP - delta)
                const bool diag = (kw0 + 31 > i0);
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int qr = 32 * qt + acc_row(r, half);
                        float p = exp2f(s[qt][r] * sl2 - L_s[qr]);
                        if (diag && key > i0 + qr) p = 0.f;
                        s[qt][r] = p;
                        dp[qt][r] = p * (dp[qt][r] - D_s[qr]);
                    }
                // dV^T += dO^T P,  dK~^T += Q~^T dS   (K = the step's queries)
#pragma unroll
                for (int pc = 0; pc < PCH; ++pc) {
                    const int qt = (pc * KW) / 16;
                    const int r0 = (pc * KW) % 16;
                    typename M::op pb, sb;
                    if constexpr (KW == 8) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) { pb[e] = (bf16)s[qt][r0 + e]; sb[e] = (bf16)dp[qt][r0 + e]; }
                    } else {
                        pb = s[qt][r0];
                        sb = dp[qt][r0];
                    }
                    const int q0 = 32 * qt + acc_row(r0, half);
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        typename M::op ga, qa;
                        if constexpr (KW == 8) {
                            bf16x4 g0 = *reinterpret_cast<const bf16x4*>(dOt_s + (32 * dt + col) * TS + q0);
                            bf16x4 g1 = *reinterpret_cast<const bf16x4*>(dOt_s + (32 * dt + col) * TS + q0 + 8);
                            bf16x4 a0 = *reinterpret_cast<const bf16x4*>(Qt_s + (32 * dt + col) * TS + q0);
                            bf16x4 a1 = *reinterpret_cast<const bf16x4*>(Qt_s + (32 * dt + col) * TS + q0 + 8);
                            ga = bf16x8{g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
                            qa = bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                        } else {
                            ga = dOt_s[(32 * dt + col) * TS + q0];
                            qa = Qt_s[(32 * dt + col) * TS + q0];
                        }
                        dvt[dt] = M::mma(ga, pb, dvt[dt]);
                        dkt[dt] = M::mma(qa, sb, dkt[dt]);
                    }
                }
                // dS -> LDS [query][key] for the dQ product
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dS_s[(32 * qt + acc_row(r, half)) * SS + 32 * w + col] = from_f32<T>(dp[qt][r]);
            } else {
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dS_s[(32 * qt + acc_row(r, half)) * SS + 32 * w + col] = from_f32<T>(0.f);
            }
            __syncthreads();

            // ---- dQ~ (BM x D) += scale * dS K~ : one 32x32 output tile per wave ----
            if (w < NQT * NDT) {
                const int qt = w / NDT, dt = w % NDT;
                // keys past the step's last query carry dS = 0: skip their chunks
                const int live = min(kBwdBN, i0 + BM - j0);
                const int nch = (KW == 8) ? (live + 15) / 16 : QCH;
                f32x16 acc = f32x16{};
                for (int c = 0; c < nch; ++c) {
                    typename M::op sa, kb;
                    if constexpr (KW == 8) {
                        sa = *reinterpret_cast<const bf16x8*>(dS_s + (32 * qt + col) * SS + kslot<T>(c, half, 0));
                        kb = *reinterpret_cast<const bf16x8*>(Kt_s + (32 * dt + col) * KTS + kslot<T>(c, half, 0));
                    } else {
                        sa = dS_s[(32 * qt + col) * SS + kslot<T>(c, half, 0)];
                        kb = Kt_s[(32 * dt + col) * KTS + kslot<T>(c, half, 0)];
                    }
                    acc = M::mma(sa, kb, acc);
                }
                // this key tile's slice of the dQ~ parts (rows at or after the tile's first key)
                float* __restrict__ dqa = a.dq_acc + (size_t)jt * a.B * a.Hq * T_ * D + (hrow + i0) * D + 32 * dt + col;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qr = 32 * qt + acc_row(r, half);
                    if (i0 + qr < T_) dqa[(size_t)qr * D] = acc[r] * a.scale;
                }
            }
        }
    }

    // ---- epilogue: this share's dK~ / scale and dV into its slice (lane owns one key) ----
    if (key < T_) {
        const size_t base = (size_t)sp * a.B * a.Hkv * T_ * D + ((size_t)(b * a.Hkv + g) * T_ + key) * D;
        float* __restrict__ dka = a.dk_acc + base;
        float* __restrict__ dva = a.dv_acc + base;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                const int d = 32 * dt + acc_row(r, half);
                *reinterpret_cast<f32x4*>(dka + d) = f32x4{dkt[dt][r], dkt[dt][r + 1], dkt[dt][r + 2], dkt[dt][r + 3]};
                *reinterpret_cast<f32x4*>(dva + d) = f32x4{dvt[dt][r], dvt[dt][r + 1], dvt[dt][r + 2], dvt[dt][r + 3]};
            }
    }
}

// ---------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(BwdArgs a) {
    const long n4 = (long)a.B * a.Hq * a.T * (D / 4);
    const long gid = (long)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= n4) {                                   // dK = R^T (scale dK~) and dV
        const long k4 = gid - n4;
        if (k4 >= (long)a.B * a.Hkv * a.T * (D / 4)) return;
        const long row = k4 / (D / 4);
        const int d0 = (int)(k4 % (D / 4)) * 4;
        const size_t slice = (size_t)a.B * a.Hkv * a.T * D;
        f32x4 kv = *reinterpret_cast<const f32x4*>(a.dk_acc + row * D + d0);
        f32x4 vv = *reinterpret_cast<const f32x4*>(a.dv_acc + row * D + d0);
        for (int sp = 1; sp < a.nsplit; ++sp) {
            kv += *reinterpret_cast<const f32x4*>(a.dk_acc + sp * slice + row * D + d0);
            vv += *reinterpret_cast<const f32x4*>(a.dv_acc + sp * slice + row * D + d0);
        }
        float x[4] = {kv[0] * a.scale, kv[1] * a.scale, kv[2] * a.scale, kv[3] * a.scale};
        if (a.rope_cs) rope_rotate(x, 4, a.rope_cs, D, (int)(row % a.T), d0, true);
        store4<T>(reinterpret_cast<T*>(a.dk) + row * D + d0, x[0], x[1], x[2], x[3]);
        store4<T>(reinterpret_cast<T*>(a.dv) + row * D + d0, vv[0], vv[1], vv[2], vv[3]);
        return;
    }
    const long row = gid / (D / 4);
    const int d0 = (int)(gid % (D / 4)) * 4;
    // the dQ~ parts of key tiles 0 .. the row's own tile, in tile order
    const int last = (int)(row % a.T) / kBwdBN;
    const size_t slice = (size_t)a.B * a.Hq * a.T * D;
    f32x4 v = *reinterpret_cast<const f32x4*>(a.dq_acc + row * D + d0);
    for (int kt = 1; kt <= last; ++kt) v += *reinterpret_cast<const f32x4*>(a.dq_acc + kt * slice + row * D + d0);
    float x[4] = {v[0], v[1], v[2], v[3]};
    if (a.rope_cs) rope_rotate(x, 4, a.rope_cs, D, (int)(row % a.T), d0, true);
    store4<T>(reinterpret_cast<T*>(a.dq) + row * D + d0, x[0], x[1], x[2], x[3]);
}

}  // namespace

template <typename T, int D>
hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t stream) {
    constexpr int VEC = 16 / sizeof(T);
    const long threads = (long)a.B * a.Hq * a.T * (D / VEC);
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)((threads + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_main(const BwdArgs& a, hipStream_t stream) {
    using L = BwdSmem<T, D>;
    // opt in to more than 64 KiB of dynamic LDS, once per device
    static bool attr_set[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !attr_set[dev]) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_main_kernel<T, D>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) attr_set[dev] = true;
    }
    static_assert(kBwdBN == kBwdF32Keys && BwdTile<float>::BM == kBwdF32Queries, "share count assumes these tiles");
    const long units = (long)((a.T + kBwdBN - 1) / kBwdBN) * a.B * a.Hkv;
    hipLaunchKernelGGL((bwd_main_kernel<T, D>), dim3((unsigned)(units * a.nsplit)), dim3(kThreads), L::BYTES, stream, a);
    return launch_bwd_dq<T, D>(a, stream);
}

template <typename T, int D>
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
    const long threads = ((long)a.B * a.Hq * a.T + (long)a.B * a.Hkv * a.T) * (D / 4);
    hipLaunchKernelGGL((bwd_dq_kernel<T, D>), dim3((unsigned)((threads + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template hipError_t launch_bwd_dq<float, 64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<float, 32>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_pre<float, 64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_main<float, 64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_pre<float, 32>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_main<float, 32>(const BwdArgs&, hipStream_t);

}  // namespace ne
