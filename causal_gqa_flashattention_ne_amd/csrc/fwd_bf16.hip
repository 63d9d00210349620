// fwd_bf16.hip -- bf16 causal GQA FlashAttention forward for gfx950 (float32 path: fwd.hip).
//
// Tiling plus an online softmax, so the T x T matrix is never stored (agentlenshq NanoEuler page,
// section "커널 구현"); RoPE is applied to the queries as they are loaded and to the keys once
// per call (same page, "기술 사양").
//
// A workgroup owns 128 queries of one (batch, query head); wave w owns queries 32w..32w+31,
// one lane per query.  The keys arrive already rotated (K~ = R k, written once per call by
// key_rot_kernel below, so no query head of a group rotates them again).  Key/value tiles of 64
// rows reach LDS through the copy pipeline of tiles.hpp with two stages (buffer_load ... lds one
// step ahead of use, swizzled unpadded tiles).  Only tiles at or before the block's last query
// are visited.  Each step works in two 32-key halves (key fragments, then P^T and the V^T
// fragments of the PV product), so that the fragments of only one half are live at a time.
//   S'^T = K~ Q~'^T - m  (A = key rows from LDS, B = this lane's rotated query in registers,
//                         pre-multiplied by scale*log2(e) so that S' is in log2 units; the
//                         accumulator starts at -m, the lane's running max, so the product
//                         itself subtracts it)
//   P^T = exp2(S'^T - m)
//   O^T += V^T P^T       (A = V^T read with ds_read_b64_tr_b16 from the row-major V tile,
//                         B = P^T straight from the score registers; K order = accumulator order)
// The running max m only moves when a row's tile maximum exceeds it by more than 2^8: until then
// P is computed against the stale m (values up to 256, exact in the float32 sums and harmless in
// bf16), and O and l are rescaled only on the rare wave-uniform branch where some row moved.
// L = (m + log2 l) * ln 2 is the natural-log row logsumexp.
//
// Precision: the rotated query is rounded to bf16 (hi); blocks whose score bound exceeds
// kLoBound (kernels.hpp) carry the remainder as a second bf16 operand (lo) in every score
// product, so that only the keys' rounding enters S there.  The decision is made per workgroup
// from exact maxima of the raw inputs, and the backward makes the same one.
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
    float red[kThreads / 64];              // per-wave maxima of the block's raw queries
};

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// The block's work once its precision is known.  qraw: this lane's raw query values (chunk c holds
// d = 16c + 8*half + 0..7, row min(qrow, T-1)).
template <int D, bool SAVE, bool LO>
__device__ void fwd_block(const FwdArgs& a, FwdLds<D>& S, const bf16x8* qh_, const bf16x8* ql_, int bg, int bh,
                          int i0) {
    using M = Mfma<bf16>;
    constexpr int NCH = D / 16, NDT = D / 32;
    const int T_ = a.T;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform across the wave
    const int col = lane & 31, half = lane >> 5;
    const int wq0 = i0 + 32 * w;
    const int qrow = wq0 + col;

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

    // this lane's query as the bf16 B operand(s) of S'^T = K~ Q~'^T (qh_ and, with LO, the
    // remainder ql_: the rotated query is then exact to ~2^-16 in the score product, and only the
    // rounding of the rotated keys remains)
    bf16x8 qhi[NCH], qlo[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        qhi[c] = qh_[c];
        if constexpr (LO) qlo[c] = ql_[c];
    }

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
    float m_run = 0.f;         // running max, log2 units (set by the first step)
    float l_run = 0.f;         // this lane's share of the row sum (against m_run)

    // One step: S'^T - m for the tile (first: from 0, and m is then set to the tile's row max),
    // the causal mask on the diagonal tile, the lazy max update, P^T and O^T += V^T P^T.
    auto step = [&](int st, int buf, bool first) {
        const int j0 = st * kTile;
        const bf16* Ks = S.k[buf];
        const bf16* Vs = S.v[buf];
        // per 32-key half: its key fragments as one batch, then one accumulation chain (dependent
        // MFMAs issue back to back on gfx950, so the halves need not be interleaved)
        const float minit = first ? 0.f : -m_run;
        f32x16 sT[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            bf16x8 kf[NCH];
#pragma unroll
            for (int c = 0; c < NCH; ++c) kf[c] = *reinterpret_cast<const bf16x8*>(Ks + roff[kt][c]);
            __builtin_amdgcn_sched_barrier(0);
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = minit;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                acc = M::mma(kf[c], qhi[c], acc);
                if constexpr (LO) acc = M::mma(kf[c], qlo[c], acc);
            }
            sT[kt] = acc;
            __builtin_amdgcn_sched_barrier(0);
        }
        if (j0 + kTile - 1 > wq0) {         // diagonal tile for this wave: keys after the query
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
        mx = partner_max(mx);
        // On the common path the scores are used as they come out of the product.  The first step
        // sets the reference max to the tile's row max (key 0 is visible to every query, so it is
        // finite); later, a lane whose row max grew by more than 2^8 moves it (wave-uniform branch)
        // and O and l are rescaled; the scores are then shifted by how far it moved.
        if (first || __builtin_amdgcn_ballot_w64(mx > kRescale) != 0) {
            const float shift = first ? mx : (mx > kRescale ? mx : 0.f);
            if (!first) {
                const float alpha = __builtin_amdgcn_exp2f(-shift);
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
            }
            m_run += shift;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) sT[kt][r] -= shift;
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
                    p[e] = __builtin_amdgcn_exp2f(sT[kt][4 * rg + e]);
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
    };

    // the training forward keeps the scaled rotated query for the backward, in the same bf16
    // parts (this lane's slots: d = 16 c + 8 half + 0..7).  Stored once, right after the copies
    // of step kSaveStep (or of the last step of a shorter block): issued before the first tiles
    // they would delay them, and after the epilogue they would lengthen the tail of the blocks
    // with the most steps
    auto save = [&](int st) {
        if constexpr (SAVE) {
            if (st == min(kSaveStep, nsteps - 1) && qrow < T_) {
                const size_t off = ((size_t)bh * T_ + qrow) * D + 8 * half;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.qrot) + off + 16 * c) = qhi[c];
                    if constexpr (LO)
                        *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.qrot_lo) + off + 16 * c) = qlo[c];
                }
            }
        }
    };

    // step 0 (key 0 is visible to every query of the block: every wave has work), then the rest
    wait_vmcnt<0>();                         // this wave's copies of tile 0, the only ones in flight
    step_barrier();                          // tile 0 is complete
    if (nsteps > 1) issue(1, 1);
    save(0);
    step(0, 0, true);
    int buf = 1;                                      // stage of the current step
    for (int st = 1; st < nsteps; ++st) {
        wait_vmcnt<0>();                     // this wave's copies of tile st, the only ones in flight
        step_barrier();                      // tile st is complete; the other stage is free
        if (st + 1 < nsteps) issue(st + 1, buf ^ 1);
        save(st);
        if (st * kTile <= wq0 + 31) step(st, buf, false);   // some key of the tile at or before a query
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

template <int D, bool SAVE>
__global__ __launch_bounds__(kThreads, FwdOcc<D>::MINB) void fwd_bf16_kernel(FwdArgs a) {
    constexpr int NCH = D / 16;
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
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;
    const int qrow = i0 + 32 * w + col;
    const int kv_end = min(T_, i0 + kQBlk);
    const int nsteps = (kv_end + kTile - 1) / kTile;

    // this lane's raw query values and the block's precision: max |q| over the block's rows (a
    // wave reduction, then the 4 waves through LDS) against the largest max |k| of the key
    // tiles the block visits.  Up to head_dim 64 the 128 rows are copied whole into the second
    // stage (unused until step 1) and read from there into the operand layout (copies of
    // contiguous rows take a quarter of the memory requests of per-lane row loads; rows past T
    // read as zeros, which leave max |q| unchanged and whose outputs are not stored), together
    // with the first key / value tile and this lane's RoPE table entries in the query-operand
    // order (one 16-byte piece per chunk and p): one round trip.  At head_dim 128 those entries,
    // held through the barrier, would not fit the registers: the rows are loaded per lane and the
    // tile and the entries follow the block maximum, as two round trips.
    TileCopy<D> tc;
    tc.init(w, lane);
    const unsigned hbytes = (unsigned)T_ * (unsigned)(D * 2);
    auto issue_tile0 = [&]() {
        const i32x4 rk = buffer_rsrc(reinterpret_cast<const bf16*>(a.k) + (size_t)bg * T_ * D, hbytes);
        const i32x4 rv = buffer_rsrc(reinterpret_cast<const bf16*>(a.v) + (size_t)bg * T_ * D, hbytes);
        tc.copy(rk, 0u, lds_addr(&S.k[0][0]), w);
        tc.copy(rv, 0u, lds_addr(&S.v[0][0]), w);
    };
    f32x4 tq[NCH][2];
    auto load_tq = [&]() {
        if (a.rope_cs) {
            const f32x4* qcs = reinterpret_cast<const f32x4*>(a.qcs);
            const int pos = min(qrow, T_ - 1);
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int p = 0; p < 2; ++p) tq[c][p] = qcs[rope_qcs_index(pos, c, p, half, NCH)];
        }
    };
    bf16x8 qraw[NCH];
    float km = 0.f;
    if constexpr (D <= 64) {
        const i32x4 rq = buffer_rsrc(reinterpret_cast<const bf16*>(a.q) + (size_t)bh * T_ * D, hbytes);
        tc.copy(rq, (unsigned)i0 * (unsigned)(D * 2), lds_addr(&S.k[1][0]), w);
        tc.copy(rq, (unsigned)(i0 + kTile) * (unsigned)(D * 2), lds_addr(&S.v[1][0]), w);
        issue_tile0();
        load_tq();
        for (int j = lane; j < nsteps; j += 64) km = fmaxf(km, a.ak[(size_t)bg * ((T_ + kTile - 1) / kTile) + j]);
        wait_vmcnt<0>();
        step_barrier();                                 // every wave's copies have landed
        const bf16* xq = (w >> 1) ? &S.v[1][0] : &S.k[1][0];
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            qraw[c] = *reinterpret_cast<const bf16x8*>(xq + Swz<D>::at(32 * (w & 1) + col, 16 * c + 8 * half));
    } else {
        const bf16* qr = reinterpret_cast<const bf16*>(a.q) + ((size_t)bh * T_ + min(qrow, T_ - 1)) * D + 8 * half;
#pragma unroll
        for (int c = 0; c < NCH; ++c) qraw[c] = *reinterpret_cast<const bf16x8*>(qr + 16 * c);
        for (int j = lane; j < nsteps; j += 64) km = fmaxf(km, a.ak[(size_t)bg * ((T_ + kTile - 1) / kTile) + j]);
    }
    float qm = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) qm = fmaxf(qm, fabsf((float)qraw[c][e]));
    qm = wave_max(qm);
    km = wave_max(km);
    if (lane == 0) S.red[w] = qm;
    __syncthreads();
    float aq = S.red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) aq = fmaxf(aq, S.red[i]);
    if constexpr (D > 64) {
        issue_tile0();
        load_tq();
    }

    const bool lo = __builtin_amdgcn_readfirstlane((int)(a.scale * (float)D * aq * km > kLoBound)) != 0;
    if constexpr (SAVE) {
        if (tid == 0) a.lof[(size_t)bh * nqt + qt] = lo ? 1 : 0;
    }
    // the query rotated in float32 and multiplied by scale*log2(e), as a bf16 part and, where the
    // block's flag asks for it, its bf16 remainder
    bf16x8 qhi[NCH], qlo[NCH];
    {
        const float c2 = a.scale * kLog2e;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (float)qraw[c][e];
            if (a.rope_cs) {
                const f32x4 t0 = tq[c][0], t1 = tq[c][1];
                const float cc[4] = {t0[0], t0[2], t1[0], t1[2]}, ss[4] = {t0[1], t0[3], t1[1], t1[3]};
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {
                    const float x0 = x[2 * pr], x1 = x[2 * pr + 1];
                    x[2 * pr] = x0 * cc[pr] - x1 * ss[pr];
                    x[2 * pr + 1] = x0 * ss[pr] + x1 * cc[pr];
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= c2;
            qhi[c] = cvt8(x);
            if (lo) qlo[c] = remainder8(x, qhi[c]);
        }
    }
    if (lo) fwd_block<D, SAVE, true>(a, S, qhi, qlo, bg, bh, i0);
    else fwd_block<D, SAVE, false>(a, S, qhi, qlo, bg, bh, i0);
}

// Keys of one 64-row tile of (batch, kv head): K~ = R k (a copy without RoPE; nothing when krot is
// null) and the tile's max |k| over the raw values.  Each thread moves D * 64 / (8 * 256) chunks of 8 values, all
// loads issued before any is used.
template <int D>
__global__ __launch_bounds__(kThreads) void key_rot_kernel(KeyRotArgs a) {
    constexpr int CPR = D / 8, NU = kTile * CPR / kThreads;
    static_assert(NU >= 1 && kTile * CPR % kThreads == 0, "chunks must cover the threads evenly");
    __shared__ float red[kThreads / 64];
    const int ntile = (a.T + kTile - 1) / kTile;
    // the tiles of kv group bgi go to XCD bgi % 8, where the forward's blocks of that group read
    // them
    int bgi, t;
    if (a.BH % kXcds == 0) {
        const int x = (int)blockIdx.x % kXcds, j = (int)blockIdx.x / kXcds;
        bgi = (j / ntile) * kXcds + x;
        t = j % ntile;
    } else {
        bgi = (int)blockIdx.x / ntile;
        t = (int)blockIdx.x % ntile;
    }
    const int tid = threadIdx.x;
    const size_t base = ((size_t)bgi * a.T + (size_t)t * kTile) * D;
    const bf16* __restrict__ k = reinterpret_cast<const bf16*>(a.k) + base;
    bf16* __restrict__ kr = a.krot ? reinterpret_cast<bf16*>(a.krot) + base : nullptr;
    bf16x8 x[NU];
    f32x4 c[NU][2];
    bool ok[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int idx = u * kThreads + tid, r = idx / CPR, part = idx % CPR;
        ok[u] = t * kTile + r < a.T;
        if (ok[u]) {
            x[u] = *reinterpret_cast<const bf16x8*>(k + (size_t)r * D + part * 8);
            if (a.rope_cs && a.krot) {
                const f32x4* cs = reinterpret_cast<const f32x4*>(a.rope_cs + (size_t)(t * kTile + r) * D + part * 8);
                c[u][0] = cs[0];
                c[u][1] = cs[1];
            }
        }
    }
    float m = 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        if (!ok[u]) continue;
        const int idx = u * kThreads + tid, r = idx / CPR, part = idx % CPR;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            y[e] = (float)x[u][e];
            m = fmaxf(m, fabsf(y[e]));
        }
        if (a.rope_cs && a.krot) {
            if (a.qcs && bgi == 0) {      // chunk `part` = operand chunk part / 2, lane half part % 2
                const int row = t * kTile + r;
                f32x4* q4 = reinterpret_cast<f32x4*>(a.qcs);
                q4[rope_qcs_index(row, part >> 1, 0, part & 1, D / 16)] = c[u][0];
                q4[rope_qcs_index(row, part >> 1, 1, part & 1, D / 16)] = c[u][1];
            }
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
                const float cc = c[u][pr / 2][2 * (pr % 2)], sn = c[u][pr / 2][2 * (pr % 2) + 1];
                const float y0 = y[2 * pr], y1 = y[2 * pr + 1];
                y[2 * pr] = y0 * cc - y1 * sn;
                y[2 * pr + 1] = y0 * sn + y1 * cc;
            }
            *reinterpret_cast<bf16x8*>(kr + (size_t)r * D + part * 8) = cvt8(y);
        } else if (a.krot) {
            *reinterpret_cast<bf16x8*>(kr + (size_t)r * D + part * 8) = x[u];
        }
    }
    m = wave_max(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) {
        float mm = red[0];
#pragma unroll
        for (int i = 1; i < kThreads / 64; ++i) mm = fmaxf(mm, red[i]);
        a.ak[(size_t)bgi * ntile + t] = mm;
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

template <int D>
hipError_t launch_key_rot(const KeyRotArgs& a, hipStream_t stream) {
    const long blocks = (long)a.BH * ((a.T + kTile - 1) / kTile);
    hipLaunchKernelGGL((key_rot_kernel<D>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template hipError_t launch_key_rot<128>(const KeyRotArgs&, hipStream_t);
template hipError_t launch_key_rot<64>(const KeyRotArgs&, hipStream_t);
template hipError_t launch_key_rot<32>(const KeyRotArgs&, hipStream_t);
template hipError_t launch_fwd_bf16<128>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_bf16<64>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_bf16<32>(const FwdArgs&, hipStream_t);

}  // namespace ne
