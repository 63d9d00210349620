// fwd_bf16.hip -- bf16 causal GQA FlashAttention forward for gfx950 (float32 path: fwd.hip).
//
// Tiling plus an online softmax, so the T x T matrix is never stored (agentlenshq NanoEuler page,
// section "커널 구현"); RoPE is applied to the queries as they are loaded and to the keys once
// per call (same page, "기술 사양").
//
// A workgroup owns 128 queries of one (batch, query head); wave w owns queries 32w..32w+31,
// one lane per query.  The keys arrive already rotated (K~ = R k, written once per call by the
// RoPE kernel, so no query head of a group rotates them again).  Key/value tiles of 64 rows reach
// LDS through the copy pipeline of tiles.hpp with two stages (buffer_load ... lds one step ahead
// of use, swizzled unpadded tiles).  Only tiles at or before the block's last query are visited.
// Each step works in two 32-key halves (key fragments, then P^T and the V^T fragments of the PV
// product), so that the fragments of only one half are live at a time: with two stages this
// keeps three workgroups per CU at head_dim 64 and makes two fit at 128.
//   S^T = K~ Q~^T        (A = key rows from LDS, B = this lane's rotated query in registers,
//                         split into bf16 hi + lo so that only the keys' rounding enters S)
//   P^T = exp2(S^T * scale*log2(e) - m)
//   O^T += V^T P^T       (A = V^T read with ds_read_b64_tr_b16 from the row-major V tile,
//                         B = P^T straight from the score registers; K order = accumulator order)
// The running max m only moves when a row's tile maximum exceeds it by more than 2^8: until then
// P is computed against the stale m (values up to 256, exact in the float32 sums and harmless in
// bf16), and O and l are rescaled only on the rare wave-uniform branch where some row moved.
// L = (m + log2 l) * ln 2 is the natural-log row logsumexp.
#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace ne {

namespace {

constexpr int kTile = kTileRows;       // keys per step
constexpr int kFS = 2;                 // LDS stages: a tile is fetched one step before its use
// workgroups per CU the kernel is compiled for (registers: 133 at head_dim 64, 219 at 128)
template <int D> struct FwdOcc { static constexpr int MINB = 3; };
template <> struct FwdOcc<128> { static constexpr int MINB = 2; };
constexpr int kQBlk = 128;             // queries per workgroup
constexpr int kThreads = kBlockThreads;
constexpr float kRescale = 8.f;        // log2 units of headroom before the running max is moved
constexpr int kXcds = 8;               // accelerator complex dies of the MI355X, each with its own L2
constexpr int kSaveStep = 2;           // step after whose tile copies the training forward stores Q~

__device__ inline float partner_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float partner_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct alignas(16) FwdLds {
    alignas(16) bf16 k[kFS][kTile * D];    // K~ tiles [key][d] (swizzled)
    alignas(16) bf16 v[kFS][kTile * D];    // V tiles
};

template <int D, bool SAVE>
__global__ __launch_bounds__(kThreads, FwdOcc<D>::MINB) void fwd_bf16_kernel(FwdArgs a) {
    using M = Mfma<bf16>;
    constexpr int NCH = D / 16, NDT = D / 32;
    __shared__ FwdLds<D> S;

    const int T_ = a.T;
    const int nqt = (T_ + kQBlk - 1) / kQBlk;
    const int G = a.Hq / a.Hkv;
    const int BG = a.B * a.Hkv;
    int qt, bg, hh;
    if (BG % kXcds == 0) {
        // workgroups are dispatched round-robin over the XCDs: block i runs on XCD i % 8.  Every
        // query head of kv group bg is placed on XCD bg % 8, so the group's K/V tiles are fetched
        // into one L2 only; within an XCD the blocks run most causal work first.
        const int x = (int)(blockIdx.x % kXcds), j = (int)(blockIdx.x / kXcds);
        const int per = (BG / kXcds) * G;               // blocks of one query tile on one XCD
        qt = nqt - 1 - j / per;
        bg = ((j % per) / G) * kXcds + x;
        hh = (j % per) % G;
    } else {
        const int BH = a.B * a.Hq;
        qt = nqt - 1 - (int)(blockIdx.x / BH);          // most causal work first
        const int bhh = (int)(blockIdx.x % BH);
        bg = bhh / G;
        hh = bhh % G;
    }
    const int bh = bg * G + hh;                         // = b * Hq + h
    const int i0 = qt * kQBlk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform across the wave
    const int col = lane & 31, half = lane >> 5;
    const int wq0 = i0 + 32 * w;
    const int qrow = wq0 + col;
    const float* __restrict__ cs = a.rope_cs;
    const float c2 = a.scale * kLog2e;

    const int kv_end = min(T_, i0 + kQBlk);
    const int nsteps = (kv_end + kTile - 1) / kTile;
    // buffers over kv head bg (key rows past T read as zeros; they are causally masked)
    const unsigned hbytes = (unsigned)T_ * (unsigned)(D * 2);
    const i32x4 rk = buffer_rsrc(reinterpret_cast<const bf16*>(a.k) + (size_t)bg * T_ * D, hbytes);
    const i32x4 rv = buffer_rsrc(reinterpret_cast<const bf16*>(a.v) + (size_t)bg * T_ * D, hbytes);
    const unsigned lk = lds_addr(&S.k[0][0]), lv = lds_addr(&S.v[0][0]);
    TileCopy<D> tc;
    tc.init(w, lane);
    auto issue = [&](int st, int buf) {
        const unsigned row0 = (unsigned)(st * kTile) * (unsigned)(D * 2), so = (unsigned)buf * TileCopy<D>::kBytes;
        tc.copy(rk, row0, lk + so, w);
        tc.copy(rv, row0, lv + so, w);
    };
    issue(0, 0);

    // this lane's query, rotated in float32 and held as two bf16 B operands (hi + lo) of
    // S^T = K~ Q~^T: the rotated query is then exact to ~2^-16 in the score product, and only the
    // rounding of the rotated keys remains (the dominant bf16 error once keys are large)
    bf16x8 qhi[NCH], qlo[NCH];
    row_operands<D>(reinterpret_cast<const bf16*>(a.q) + ((size_t)bh * T_ + min(qrow, T_ - 1)) * D, cs,
                    min(qrow, T_ - 1), half, qhi, qlo);

    wait_vmcnt<0>();   // query operands and the first tile (see copy16_to_lds)

    // per-lane LDS offsets of the key row fragments (row 32*kt + col, chunks 2c + half)
    int roff[2][NCH];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int c = 0; c < NCH; ++c) roff[kt][c] = Swz<D>::at(32 * kt + col, 16 * c + 8 * half);
    // per-lane bases of the transposed V fragment reads (one per 32 columns of d)
    int vtb[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vtb[dt] = tr_base<D>(32 * dt, lane);

    f32x16 oacc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;   // reference max, log2 units
    float l_run = 0.f;         // this lane's share of the row sum (against m_run)

    int buf = 0;                                      // stage of the current step
    for (int st = 0; st < nsteps; ++st) {
        wait_vmcnt<0>();                     // this wave's copies of tile st, the only ones in flight
        step_barrier();                      // tile st is complete; the other stage is free
        if (st + 1 < nsteps) issue(st + 1, buf ^ 1);
        if constexpr (SAVE) {
            // the training forward keeps the rotated query for the backward, in the same two bf16
            // parts (this lane's slots: d = 16 c + 8 half + 0..7).  Stored once, right after the
            // copies of step kSaveStep (or of the last step of a shorter block): issued before the
            // first tiles they would delay them, and after the epilogue they would lengthen the
            // tail of the blocks with the most steps
            if (st == min(kSaveStep, nsteps - 1) && qrow < T_) {
                const size_t off = ((size_t)bh * T_ + qrow) * D + 8 * half;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.qrot) + off + 16 * c) = qhi[c];
                    *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.qrot_lo) + off + 16 * c) = qlo[c];
                }
            }
        }
        const int j0 = st * kTile;
        if (j0 <= wq0 + 31) {               // some key of the tile is at or before some query of the wave
            const bf16* Ks = S.k[buf];
            const bf16* Vs = S.v[buf];
            // per 32-key half: its key fragments as one batch, then one accumulation chain (dependent
            // MFMAs issue back to back on gfx950, so the halves need not be interleaved)
            f32x16 sT[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                bf16x8 kf[NCH];
#pragma unroll
                for (int c = 0; c < NCH; ++c) kf[c] = *reinterpret_cast<const bf16x8*>(Ks + roff[kt][c]);
                __builtin_amdgcn_sched_barrier(0);
                sT[kt] = M::mma(kf[0], qhi[0], f32x16{});
                sT[kt] = M::mma(kf[0], qlo[0], sT[kt]);
#pragma unroll
                for (int c = 1; c < NCH; ++c) {
                    sT[kt] = M::mma(kf[c], qhi[c], sT[kt]);
                    sT[kt] = M::mma(kf[c], qlo[c], sT[kt]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (j0 + kTile - 1 > wq0) {     // diagonal tile for this wave: keys after the query
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (j0 + 32 * kt + acc_row(r, half) > qrow) sT[kt][r] = -INFINITY;
            }
            float mx = sT[0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sT[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sT[1][r]);
            mx = partner_max(mx) * c2;
            if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescale) != 0) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
                m_run = m_new;
            }
            // per 32-key half: V^T fragments, P^T (B operands, 2 chunks of 16 keys) and the row sum,
            // then O^T += V^T P^T
            float ls = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                bf16x8 vf[2][NDT];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) vf[h2][dt] = tr_frag_at<D>(Vs, vtb[dt], 32 * kt + 16 * h2);
                bf16x8 pb[2];
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    float p[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sT[kt][4 * rg + e], c2, -m_run));
                        ls += p[e];
                    }
                    const bf16x4 p4 = cvt4(p);
                    if (rg & 1) pb[rg >> 1] = __builtin_shufflevector(pb[rg >> 1].lo, p4, 0, 1, 2, 3, 4, 5, 6, 7);
                    else pb[rg >> 1] = __builtin_shufflevector(p4, p4, 0, 1, 2, 3, 4, 5, 6, 7);
                }
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = M::mma(vf[h2][dt], pb[h2], oacc[dt]);
            }
            l_run += ls;
        }
        buf ^= 1;
    }

    // epilogue: O = O^T / l, L = (m + log2 l) ln 2
    const float l_tot = partner_sum(l_run);
    if (qrow < T_) {
        const float inv = 1.f / l_tot;
        bf16* __restrict__ o = reinterpret_cast<bf16*>(a.o) + ((size_t)bh * T_ + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                const float x[4] = {oacc[dt][r] * inv, oacc[dt][r + 1] * inv, oacc[dt][r + 2] * inv,
                                    oacc[dt][r + 3] * inv};
                *reinterpret_cast<bf16x4*>(o + 32 * dt + acc_row(r, half)) = cvt4(x);
            }
        if (half == 0) a.lse[(size_t)bh * T_ + qrow] = (m_run + __log2f(l_tot)) * kLn2;
    }
}

}  // namespace

template <int D>
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
    const long blocks = (long)((a.T + kQBlk - 1) / kQBlk) * a.B * a.Hq;
    if (a.qrot) hipLaunchKernelGGL((fwd_bf16_kernel<D, true>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((fwd_bf16_kernel<D, false>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template hipError_t launch_fwd_bf16<128>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_bf16<64>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_bf16<32>(const FwdArgs&, hipStream_t);

}  // namespace ne
