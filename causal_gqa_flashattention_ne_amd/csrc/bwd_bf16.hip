// bwd_bf16.hip -- bf16 backward for gfx950 (the float32 path lives in bwd.hip).
//
// Mathematics (hand-written backward of the forward; ai-paper-delta NanoEuler page, "Core
// Mechanics"), with R the RoPE rotation, Q~ = R q and K~ = R k:
//     S = Q~ K~^T, P = exp(scale*S - L), dP = dO V^T, dS = P * (dP - delta),
//     dV = P^T dO,  dK = R^T (scale * dS^T Q~),  dQ = R^T (scale * dS K~),
// where delta_i = sum_d dO_id O_id.  The kernels work with P' = scale * P and dS' = scale * dS:
// the factor enters through the exponent (log2(scale) is folded into L), so dS' feeds dK and dQ
// directly and dV is divided by scale once at the end.
//
// The rotated queries are carried as two bf16 parts, Q~ = hi + lo, in every score product (the
// forward does the same): S then carries only the rounding of the rotated keys, which keeps the
// byte-level workload (keys scaled x8) inside the bf16 error bar; Q~^T in the dK product uses hi.
//
// Two launches:
//   bwd_pre_bf16:  delta (float32), Q~ (hi and lo) and K~ (bf16, rotated once) into the workspace.
//   bwd_bf16:      one grid, two kinds of workgroups, no atomics and no float32 scratch:
//     dK/dV blocks (key-tile major): a block owns 64 keys of one (batch, kv head); its 4 waves
//       split every 64-query step 2 x 2 (wave w: keys 32*(w&1).., queries 32*(w>>1)..), keep
//       dK^T / dV^T of their 32 keys in registers across all query heads of the group and all
//       query tiles at or after the diagonal, and add the two query halves through LDS at the
//       end.  S = Q~ K~^T is formed so that a lane owns one key: P' and dS' are then the B
//       operands of dV^T += dO^T P' and dK^T += Q~^T dS' straight from the accumulator
//       registers (K order = accumulator row order; dO^T and Q~^T are read in that order).
//     dQ blocks (query-tile major): a block owns 128 queries of one query head, wave w the
//       queries 32w..32w+31, one lane per query.  Key/value tiles of 64 stream through LDS;
//       S^T = K~ Q~^T and dP^T = V dO^T put one query per lane, and dQ^T += K~^T dS'^T takes
//       dS'^T straight from the registers.  dQ is un-rotated and written once.
//   Tiles are double-buffered in LDS; the next tile is loaded from global memory (clamped,
//   unconditional loads) while the current one is used.  Every LDS tile is row-major, written
//   with 16-byte stores; transposed operands come from ds_read_b64_tr_b16, which transposes
//   16-bit elements across each 16-lane group.  Blocks are ordered heaviest causal work first;
//   tiles wholly above the diagonal are never visited.  The two roles recompute S and dP
//   separately (7 products per score instead of 5) in exchange for having no cross-XCD
//   float32 atomics, which on this machine go out to the memory fabric.
#include "common.hpp"
#include "kernels.hpp"

namespace ne {

namespace {

constexpr int kTile = 64;     // keys per dK/dV block, queries per step; keys per dQ step
constexpr int kQBlk = 128;    // queries per dQ block
constexpr int kThreads = 256;
constexpr int kXcds = 8;      // accelerator complex dies of the MI355X, each with its own L2

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b16: inside each 16-lane group, lane i receives element (i % 4) of the 8-byte
// rows read by lanes (i / 4) + 4k, k = 0..3.
__device__ inline bf16x4 tr_read(const bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// A-operand fragment (32 rows m x 16 k) of the 32x32x16 MFMA taken from a row-major LDS tile
// X[k][m] (so A[m][k] = X[k][m]): lane (m = l%32, half h) receives X[k][m] for the k rows
// kb0 + 0..3 and kb1 + 0..3 (kb0 / kb1 chosen per half by the caller).  rs = row stride.
__device__ inline bf16x8 tr_frag(const bf16* X, int rs, int m0, int kb0, int kb1, int lane) {
    const int s = lane & 15;
    const int m = m0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
    const bf16x4 lo = tr_read(X + (kb0 + (s >> 2)) * rs + m);
    const bf16x4 hi = tr_read(X + (kb1 + (s >> 2)) * rs + m);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even)
__device__ inline bf16x2 cvt2(float x, float y) { return __builtin_convertvector(f32x2{x, y}, bf16x2); }

__device__ inline bf16x4 cvt4(const float* x) {
    return __builtin_shufflevector(cvt2(x[0], x[1]), cvt2(x[2], x[3]), 0, 1, 2, 3);
}

template <int D>
struct alignas(16) DkdvLds {
    static constexpr int RS = D + 8;
    alignas(16) bf16 q[2][kTile * RS];    // Q~ tiles [query][d] (hi part)
    alignas(16) bf16 ql[2][kTile * RS];   // Q~ remainder tiles (lo part)
    alignas(16) bf16 g[2][kTile * RS];    // dO tiles
    alignas(16) float l[2][kTile];        // L*log2(e) - log2(scale)  (+inf past the sequence end)
    alignas(16) float dl[2][kTile];       // delta
};

template <int D>
struct alignas(16) DqLds {
    static constexpr int RS = D + 8;
    alignas(16) bf16 k[2][kTile * RS];    // K~ tiles [key][d]
    alignas(16) bf16 v[2][kTile * RS];    // V tiles
};

template <int D>
union alignas(16) BwdLds {
    DkdvLds<D> kv;
    DqLds<D> q;
};

// Prefetch of NT 64-row x D tiles: rows clamped into [0, T), loads unconditional, so the
// destination registers are not touched again before the store to LDS.
template <int D, int NT>
struct TileSet {
    static constexpr int NU = (kTile * D / 8) / kThreads;
    static_assert((kTile * D / 8) % kThreads == 0, "tile chunks must cover the workgroup evenly");
    bf16x8 x[NT][NU];

    __device__ inline void load(const bf16* const* src, int last, int tid) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int ch = tid + u * kThreads;
            const int off = min(ch / (D / 8), last) * D + (ch % (D / 8)) * 8;
#pragma unroll
            for (int t = 0; t < NT; ++t) x[t][u] = *reinterpret_cast<const bf16x8*>(src[t] + off);
        }
    }
    __device__ inline void store(bf16* const* dst, int tid) const {
        constexpr int RS = D + 8;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int ch = tid + u * kThreads;
            const int o = (ch / (D / 8)) * RS + (ch % (D / 8)) * 8;
#pragma unroll
            for (int t = 0; t < NT; ++t) *reinterpret_cast<bf16x8*>(dst[t] + o) = x[t][u];
        }
    }
};

// One 32 x 32 dK/dV block: P' and dS' for this wave's keys (lane) and queries (registers),
// packed to bf16 as B operands of the dV / dK products.
template <bool MASKED>
__device__ inline void kv_softmax(const f32x16& s, const f32x16& dp, const float* lsc, const float* dl,
                                  float sl2, int kloc, int qbase, int half, bf16x8* pb, bf16x8* sb) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
        const int q0 = qbase + 8 * rg + 4 * half;
        const f32x4 lv = *reinterpret_cast<const f32x4*>(lsc + q0);
        const f32x4 dv = *reinterpret_cast<const f32x4*>(dl + q0);
        float p[4], d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * rg + e;
            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -lv[e]));
            if (MASKED && kloc > q0 + e) p[e] = 0.f;
            d[e] = p[e] * (dp[r] - dv[e]);
        }
        const bf16x4 p4 = cvt4(p), d4 = cvt4(d);
        if (rg & 1) {
            pb[rg >> 1] = __builtin_shufflevector(pb[rg >> 1].lo, p4, 0, 1, 2, 3, 4, 5, 6, 7);
            sb[rg >> 1] = __builtin_shufflevector(sb[rg >> 1].lo, d4, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
            pb[rg >> 1] = __builtin_shufflevector(p4, p4, 0, 1, 2, 3, 4, 5, 6, 7);
            sb[rg >> 1] = __builtin_shufflevector(d4, d4, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
}

// ---------------------------------------------------------------------------------------------
// dK/dV block: keys [j0, j0 + 64) of kv head (b, g).
template <int D>
__device__ void dkdv_block(const BwdArgs& a, DkdvLds<D>& S, int jt, int bg) {
    using M = Mfma<bf16>;
    constexpr int NCH = D / 16, NDT = D / 32, RS = DkdvLds<D>::RS;
    const int T_ = a.T;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int G = a.Hq / a.Hkv;
    const int j0 = jt * kTile;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform across the wave
    const int col = lane & 31, half = lane >> 5;
    const int kh = w & 1, qh = w >> 1;
    const int kloc = 32 * kh + col;
    const int key = j0 + kloc;
    const float sl2 = a.scale * kLog2e;
    const float log2_scale = __log2f(a.scale);
    const bf16* __restrict__ qrot = reinterpret_cast<const bf16*>(a.qrot);
    const bf16* __restrict__ qrot_lo = reinterpret_cast<const bf16*>(a.qrot_lo);
    const bf16* __restrict__ dout = reinterpret_cast<const bf16*>(a.dout);

    // this lane's key row: K~ and V as B operands
    bf16x8 kop[NCH], vop[NCH];
    {
        const size_t off = ((size_t)bg * T_ + min(key, T_ - 1)) * D + 8 * half;
        const bf16* kr = reinterpret_cast<const bf16*>(a.krot) + off;
        const bf16* vr = reinterpret_cast<const bf16*>(a.v) + off;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            kop[c] = *reinterpret_cast<const bf16x8*>(kr + 16 * c);
            vop[c] = *reinterpret_cast<const bf16x8*>(vr + 16 * c);
        }
    }

    const int nsph = (T_ - j0 + kTile - 1) / kTile;   // query steps per head
    const int nsteps = G * nsph;
    const size_t hrow0 = (size_t)(b * a.Hq + g * G) * T_;
    TileSet<D, 3> pf;
    float px = 0.f;
    auto load = [&](int hh, int i0) {
        const size_t hrow = hrow0 + (size_t)hh * T_;
        const bf16* src[3] = {qrot + (hrow + i0) * D, qrot_lo + (hrow + i0) * D, dout + (hrow + i0) * D};
        pf.load(src, T_ - 1 - i0, tid);
        const int r = min(tid & (kTile - 1), T_ - 1 - i0);
        if (w == 0) px = a.lse[hrow + i0 + r];
        else if (w == 1) px = a.delta[hrow + i0 + r];
    };
    auto store = [&](int buf, int i0) {
        bf16* dst[3] = {S.q[buf], S.ql[buf], S.g[buf]};
        pf.store(dst, tid);
        const bool in = i0 + (tid & (kTile - 1)) < T_;
        if (w == 0) S.l[buf][tid] = in ? px * kLog2e - log2_scale : INFINITY;
        else if (w == 1) S.dl[buf][tid - kTile] = px;
    };
    load(0, j0);
    store(0, j0);
    __syncthreads();

    f32x16 dkt[NDT], dvt[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) { dkt[i] = f32x16{}; dvt[i] = f32x16{}; }

    int hh = 0, i0 = j0;
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        int nhh = hh, ni0 = i0 + kTile;
        if (ni0 >= T_) { ni0 = j0; ++nhh; }
        const bool more = st + 1 < nsteps;
        if (more) load(nhh, ni0);
        const bf16* Qs = S.q[buf];
        const bf16* Gs = S.g[buf];
        const bool first = (i0 == j0);
        if (!(first && kh > qh)) {            // blocks wholly above the diagonal are skipped
            // query (hi, lo) / dO fragments first, then the two independent chains interleaved
            const bf16* Ql = S.ql[buf];
            bf16x8 qf[NCH], qlf[NCH], gf[NCH];
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                qf[c] = *reinterpret_cast<const bf16x8*>(&Qs[(32 * qh + col) * RS + 16 * c + 8 * half]);
                qlf[c] = *reinterpret_cast<const bf16x8*>(&Ql[(32 * qh + col) * RS + 16 * c + 8 * half]);
                gf[c] = *reinterpret_cast<const bf16x8*>(&Gs[(32 * qh + col) * RS + 16 * c + 8 * half]);
            }
            f32x16 sacc = M::mma(qf[0], kop[0], f32x16{});
            f32x16 dp = M::mma(gf[0], vop[0], f32x16{});
            sacc = M::mma(qlf[0], kop[0], sacc);
#pragma unroll
            for (int c = 1; c < NCH; ++c) {
                sacc = M::mma(qf[c], kop[c], sacc);
                dp = M::mma(gf[c], vop[c], dp);
                sacc = M::mma(qlf[c], kop[c], sacc);
            }
            bf16x8 pb[2], sb[2];
            if (first && kh == qh)
                kv_softmax<true>(sacc, dp, S.l[buf], S.dl[buf], sl2, kloc, 32 * qh, half, pb, sb);
            else
                kv_softmax<false>(sacc, dp, S.l[buf], S.dl[buf], sl2, kloc, 32 * qh, half, pb, sb);
            bf16x8 gt[2][NDT], qtf[2][NDT];
#pragma unroll
            for (int pc = 0; pc < 2; ++pc) {
                const int kb0 = 32 * qh + 16 * pc + 4 * half;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    gt[pc][dt] = tr_frag(Gs, RS, 32 * dt, kb0, kb0 + 8, lane);
                    qtf[pc][dt] = tr_frag(Qs, RS, 32 * dt, kb0, kb0 + 8, lane);
                }
            }
#pragma unroll
            for (int pc = 0; pc < 2; ++pc)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    dvt[dt] = M::mma(gt[pc][dt], pb[pc], dvt[dt]);
                    dkt[dt] = M::mma(qtf[pc][dt], sb[pc], dkt[dt]);
                }
        }
        if (more) store(buf ^ 1, ni0);
        __syncthreads();
        hh = nhh;
        i0 = ni0;
    }

    // add the two query halves' partial dK^T / dV^T through LDS (reuses the tile buffers)
    float* red = reinterpret_cast<float*>(&S.q[0][0]);   // [dk|dv][kh][NDT][16 regs][64 lanes]
    static_assert(sizeof(S.q) + sizeof(S.ql) + sizeof(S.g) >= 2 * 2 * NDT * 16 * 64 * 4, "reduction buffer too small");
    if (qh == 1) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                red[((kh * NDT + dt) * 16 + r) * 64 + lane] = dkt[dt][r];
                red[(((2 + kh) * NDT + dt) * 16 + r) * 64 + lane] = dvt[dt][r];
            }
    }
    __syncthreads();
    if (qh == 0 && key < T_) {
        const float inv_scale = 1.f / a.scale;     // dV was accumulated from P' = scale * P
        const size_t base = ((size_t)bg * T_ + key) * D;
        bf16* __restrict__ dk = reinterpret_cast<bf16*>(a.dk) + base;
        bf16* __restrict__ dv = reinterpret_cast<bf16*>(a.dv) + base;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                float x[4], y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = dkt[dt][r + e] + red[((kh * NDT + dt) * 16 + r + e) * 64 + lane];
                    y[e] = (dvt[dt][r + e] + red[(((2 + kh) * NDT + dt) * 16 + r + e) * 64 + lane]) * inv_scale;
                }
                const int d = 32 * dt + acc_row(r, half);
                if (a.rope_cs) rope_rotate(x, 4, a.rope_cs, D, key, d, true);
                *reinterpret_cast<bf16x4*>(dk + d) = cvt4(x);
                *reinterpret_cast<bf16x4*>(dv + d) = cvt4(y);
            }
    }
}

// ---------------------------------------------------------------------------------------------
// dQ block: queries [i0, i0 + 128) of query head (b, h).
template <int D>
__device__ void dq_block(const BwdArgs& a, DqLds<D>& S, int qt, int bh) {
    using M = Mfma<bf16>;
    constexpr int NCH = D / 16, NDT = D / 32, RS = DqLds<D>::RS;
    const int T_ = a.T;
    const int b = bh / a.Hq, h = bh % a.Hq;
    const int bg = b * a.Hkv + h / (a.Hq / a.Hkv);
    const int i0 = qt * kQBlk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform across the wave
    const int col = lane & 31, half = lane >> 5;
    const int wq0 = i0 + 32 * w;            // wave's first query
    const int qrow = wq0 + col;             // this lane's query
    const size_t qoff = ((size_t)bh * T_ + min(qrow, T_ - 1)) * D;
    const float sl2 = a.scale * kLog2e;

    // this lane's query row: Q~ (hi and lo) and dO as B operands, L and delta
    bf16x8 qop[NCH], qlo[NCH], gop[NCH];
    {
        const bf16* qr = reinterpret_cast<const bf16*>(a.qrot) + qoff + 8 * half;
        const bf16* ql = reinterpret_cast<const bf16*>(a.qrot_lo) + qoff + 8 * half;
        const bf16* gr = reinterpret_cast<const bf16*>(a.dout) + qoff + 8 * half;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            qop[c] = *reinterpret_cast<const bf16x8*>(qr + 16 * c);
            qlo[c] = *reinterpret_cast<const bf16x8*>(ql + 16 * c);
            gop[c] = *reinterpret_cast<const bf16x8*>(gr + 16 * c);
        }
    }
    const size_t rowi = (size_t)bh * T_ + min(qrow, T_ - 1);
    const float lsc = a.lse[rowi] * kLog2e - __log2f(a.scale);
    const float dlt = a.delta[rowi];

    const bf16* __restrict__ kbase = reinterpret_cast<const bf16*>(a.krot) + (size_t)bg * T_ * D;
    const bf16* __restrict__ vbase = reinterpret_cast<const bf16*>(a.v) + (size_t)bg * T_ * D;
    const int kv_end = min(T_, i0 + kQBlk);
    const int nsteps = (kv_end + kTile - 1) / kTile;
    TileSet<D, 2> pf;
    {
        const bf16* src[2] = {kbase, vbase};
        bf16* dst[2] = {S.k[0], S.v[0]};
        pf.load(src, T_ - 1, tid);
        pf.store(dst, tid);
    }
    __syncthreads();

    f32x16 dqt[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) dqt[i] = f32x16{};

    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        const int j0 = st * kTile;
        const bool more = st + 1 < nsteps;
        if (more) {
            const bf16* src[2] = {kbase + (size_t)(j0 + kTile) * D, vbase + (size_t)(j0 + kTile) * D};
            pf.load(src, T_ - 1 - j0 - kTile, tid);
        }
        if (j0 <= wq0 + 31) {               // some key of the tile is at or before some query of the wave
            const bf16* Ks = S.k[buf];
            const bf16* Vs = S.v[buf];
            // key / value fragments first, then four independent chains interleaved
            bf16x8 kf[2][NCH], vf[2][NCH];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    kf[kt][c] = *reinterpret_cast<const bf16x8*>(&Ks[(32 * kt + col) * RS + 16 * c + 8 * half]);
                    vf[kt][c] = *reinterpret_cast<const bf16x8*>(&Vs[(32 * kt + col) * RS + 16 * c + 8 * half]);
                }
            f32x16 sT[2], dpT[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                sT[kt] = M::mma(kf[kt][0], qop[0], f32x16{});
                dpT[kt] = M::mma(vf[kt][0], gop[0], f32x16{});
                sT[kt] = M::mma(kf[kt][0], qlo[0], sT[kt]);
            }
#pragma unroll
            for (int c = 1; c < NCH; ++c)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    sT[kt] = M::mma(kf[kt][c], qop[c], sT[kt]);
                    dpT[kt] = M::mma(vf[kt][c], gop[c], dpT[kt]);
                    sT[kt] = M::mma(kf[kt][c], qlo[c], sT[kt]);
                }
            // dS'^T = P' (dP^T - delta), packed as B operands (4 chunks of 16 keys)
            bf16x8 sb[4];
            const bool diag = j0 + kTile - 1 > wq0;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    float d[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * rg + e;
                        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sT[kt][r], sl2, -lsc));
                        if (diag && j0 + 32 * kt + acc_row(r, half) > qrow) p = 0.f;
                        d[e] = p * (dpT[kt][r] - dlt);
                    }
                    const bf16x4 d4 = cvt4(d);
                    const int pc = 2 * kt + (rg >> 1);
                    if (rg & 1) sb[pc] = __builtin_shufflevector(sb[pc].lo, d4, 0, 1, 2, 3, 4, 5, 6, 7);
                    else sb[pc] = __builtin_shufflevector(d4, d4, 0, 1, 2, 3, 4, 5, 6, 7);
                }
            // dQ~^T (D x 32 queries) += K~^T dS'^T  (K = the tile's keys, accumulator order)
            bf16x8 ktf[4][NDT];
#pragma unroll
            for (int pc = 0; pc < 4; ++pc) {
                const int kb0 = 32 * (pc >> 1) + 16 * (pc & 1) + 4 * half;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) ktf[pc][dt] = tr_frag(Ks, RS, 32 * dt, kb0, kb0 + 8, lane);
            }
#pragma unroll
            for (int pc = 0; pc < 4; ++pc)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) dqt[dt] = M::mma(ktf[pc][dt], sb[pc], dqt[dt]);
        }
        if (more) {
            bf16* dst[2] = {S.k[buf ^ 1], S.v[buf ^ 1]};
            pf.store(dst, tid);
        }
        __syncthreads();
    }

    // dQ = R^T dQ~ ; lane owns one query, 4 consecutive d per register group
    if (qrow < T_) {
        bf16* __restrict__ dq = reinterpret_cast<bf16*>(a.dq) + ((size_t)bh * T_ + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                float x[4] = {dqt[dt][r], dqt[dt][r + 1], dqt[dt][r + 2], dqt[dt][r + 3]};
                const int d = 32 * dt + acc_row(r, half);
                if (a.rope_cs) rope_rotate(x, 4, a.rope_cs, D, qrow, d, true);
                *reinterpret_cast<bf16x4*>(dq + d) = cvt4(x);
            }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_bf16_kernel(BwdArgs a) {
    __shared__ BwdLds<D> S;
    const int BG = a.B * a.Hkv, G = a.Hq / a.Hkv;
    const int nkv = (a.T + kTile - 1) / kTile;
    const int nqt = (a.T + kQBlk - 1) / kQBlk;
    if (BG % kXcds == 0) {
        // workgroups are dispatched round-robin over the XCDs: block i runs on XCD i % 8.  All
        // blocks of kv group bg (its dK/dV tiles and the dQ tiles of its query heads) go to XCD
        // bg % 8, so the group's Q~, dO, K~ and V are fetched into one L2 only.  Within an XCD:
        // dK/dV blocks first (key tile 0 carries the most causal work), then dQ blocks (last
        // query tile first).
        const int x = (int)(blockIdx.x % kXcds), j = (int)(blockIdx.x / kXcds);
        const int gpx = BG / kXcds;                     // kv groups per XCD
        if (j < nkv * gpx) {
            dkdv_block<D>(a, S.kv, j / gpx, (j % gpx) * kXcds + x);
        } else {
            const int r = j - nkv * gpx;
            const int per = gpx * G;
            const int bg = ((r % per) / G) * kXcds + x;
            dq_block<D>(a, S.q, nqt - 1 - r / per, bg * G + (r % per) % G);
        }
    } else {
        const int BH = a.B * a.Hq;
        const int ndk = nkv * BG;
        const int blk = (int)blockIdx.x;
        if (blk < ndk) dkdv_block<D>(a, S.kv, blk / BG, blk % BG);
        else dq_block<D>(a, S.q, nqt - 1 - (blk - ndk) / BH, (blk - ndk) % BH);
    }
}

// delta_i = sum_d dO_id O_id; Q~ = R q (bf16 hi + lo) and K~ = R k (bf16) into the workspace.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_bf16_kernel(BwdArgs a) {
    constexpr int TPR = D / 8;
    const long qrows = (long)a.B * a.Hq * a.T;
    const long krows = (long)a.B * a.Hkv * a.T;
    const long gid = (long)blockIdx.x * kThreads + threadIdx.x;
    const long row = gid / TPR;
    const int part = (int)(gid % TPR);
    if (row < qrows) {
        const size_t off = (size_t)row * D + part * 8;
        float o[8], d[8], q[8];
        load16<bf16>(reinterpret_cast<const bf16*>(a.o) + off, o);
        load16<bf16>(reinterpret_cast<const bf16*>(a.dout) + off, d);
        load16<bf16>(reinterpret_cast<const bf16*>(a.q) + off, q);
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += o[e] * d[e];
        if (a.rope_cs) rope_rotate(q, 8, a.rope_cs, D, (int)(row % a.T), part * 8, false);
        const bf16x8 hi = __builtin_shufflevector(cvt4(q), cvt4(q + 4), 0, 1, 2, 3, 4, 5, 6, 7);
        float r[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = q[e] - (float)hi[e];
        *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.qrot) + off) = hi;
        *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.qrot_lo) + off) =
            __builtin_shufflevector(cvt4(r), cvt4(r + 4), 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int o2 = 1; o2 < TPR; o2 <<= 1) sum += __shfl_xor(sum, o2, 64);
        if (part == 0) a.delta[row] = sum;
    } else if (row < qrows + krows) {
        const long kr = row - qrows;
        const size_t off = (size_t)kr * D + part * 8;
        float k[8];
        load16<bf16>(reinterpret_cast<const bf16*>(a.k) + off, k);
        if (a.rope_cs) rope_rotate(k, 8, a.rope_cs, D, (int)(kr % a.T), part * 8, false);
        store16<bf16>(reinterpret_cast<bf16*>(a.krot) + off, k);
    }
}

}  // namespace

template <int D>
hipError_t launch_bwd_pre_bf16(const BwdArgs& a, hipStream_t stream) {
    const long rows = (long)a.B * (a.Hq + a.Hkv) * a.T;
    const long threads = rows * (D / 8);
    hipLaunchKernelGGL((bwd_pre_bf16_kernel<D>), dim3((unsigned)((threads + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_main_bf16(const BwdArgs& a, hipStream_t stream) {
    const long ndk = (long)((a.T + kTile - 1) / kTile) * a.B * a.Hkv;
    const long ndq = (long)((a.T + kQBlk - 1) / kQBlk) * a.B * a.Hq;
    hipLaunchKernelGGL((bwd_bf16_kernel<D>), dim3((unsigned)(ndk + ndq)), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template hipError_t launch_bwd_pre_bf16<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_pre_bf16<32>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_main_bf16<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_main_bf16<32>(const BwdArgs&, hipStream_t);

}  // namespace ne
