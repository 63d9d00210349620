// bwd_bf16.hip -- bf16 backward for gfx950 (the float32 path lives in bwd.hip).
//
// Mathematics (hand-written backward of the forward; ai-paper-delta NanoEuler page, "Core
// Mechanics"), with R the RoPE rotation, Q~ = R q and K~ = R k:
//     S = Q~ K~^T, P = exp(scale*S - L), dP = dO V^T, dS = P * (dP - delta),
//     dV = P^T dO,  dK = R^T (scale * dS^T Q~),  dQ = R^T (scale * dS K~),
// where delta_i = sum_d dO_id O_id.  The kernels work with P' = scale * P and dS' = scale * dS:
// the factor enters through the exponent (l' = L log2(e) - log2(scale) is what the kernels
// subtract), so dS' feeds dK and dQ directly and dV is divided by scale once at the end.  The
// rotated queries are stored multiplied by c = scale * log2(e), Q~' = c Q~, so that Q~' K~^T is
// the score in log2 units; dK, formed from Q~', is divided by c once at the end.
//
// The rotated queries are rounded to bf16 (hi).  For the 128-query blocks whose score bound
// exceeds kLoBound the forward also keeps the remainder (lo) and adds its products to every score
// of the block, so that S carries only the rounding of the rotated keys there (this keeps the
// byte-level workload, keys scaled x8, inside the bf16 error bar); the backward follows the
// forward's per-block flags (lof), so that P is formed from the same products in both.  Q~'^T in
// the dK product uses hi.
//
// Launches:
//   bwd_pre_bf16:  per query row -l' and -delta (float32, padded per head to whole 64-row tiles:
//     -inf / 0 past the sequence end, so padded rows get P = 0); in the plain backward also Q~'
//     (hi, and lo for the flagged blocks) and the flags.  K~ comes from key_rot_kernel.
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
//   The l' and delta of a step's rows are the starting values of its S and dP accumulators in the
//   dK/dV role (stored negated), so the products themselves subtract them.
//   Tiles reach LDS through the copy pipeline of tiles.hpp with two stages (buffer_load ... lds
//   one step ahead, swizzled unpadded tiles, one wait and one barrier per step; a third stage
//   measured no faster and costs 25 KB of LDS per dK/dV workgroup).  Blocks are ordered
//   heaviest causal work first; tiles wholly above the diagonal are never visited.  The two roles
//   recompute S and dP separately in exchange for having no cross-XCD float32 atomics, which on
//   this machine go out to the memory fabric.
#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

#include <type_traits>

namespace ne {

namespace {

constexpr int kTile = kTileRows;       // keys per dK/dV block, queries per step; keys per dQ step
constexpr int kQBlk = 128;             // queries per dQ block
constexpr int kThreads = kBlockThreads;
constexpr int kXcds = 8;               // accelerator complex dies of the MI355X, each with its own L2
constexpr int kBS = 2;                 // LDS stages: a tile is fetched one step before its use

// (l', delta) of a 64-row query tile, stored in the workspace exactly as in LDS: 4 groups of 16
// rows [l' x 16 | delta x 16] (512 bytes per tile); wave w copies group w with 8 lanes.
__device__ inline int ld_lsc(int q) { return (q >> 4) * 32 + (q & 15); }
__device__ inline int ld_dlt(int q) { return (q >> 4) * 32 + 16 + (q & 15); }

template <int D>
struct alignas(16) DkdvLds {
    alignas(16) bf16 q[kBS][kTile * D];    // Q~ tiles [query][d] (hi part)
    alignas(16) bf16 ql[kBS][kTile * D];   // Q~ remainder tiles (lo part)
    alignas(16) bf16 g[kBS][kTile * D];    // dO tiles
    alignas(16) float ld[kBS][2 * kTile];  // l' and delta, see ld_lsc
};

template <int D>
struct alignas(16) DqLds {
    alignas(16) bf16 k[kBS][kTile * D];    // K~ tiles [key][d]
    alignas(16) bf16 v[kBS][kTile * D];    // V tiles
    alignas(16) bf16 xq[2][kTile * D];     // the block's Q~' rows in the prologue (two 64-row tiles)
};

template <int D>
union alignas(16) BwdLds {
    DkdvLds<D> kv;
    DqLds<D> q;
};

typedef const __attribute__((address_space(4))) int cint;   // loads through it are scalar loads

// ---------------------------------------------------------------------------------------------
// dK/dV block: keys [j0, j0 + 64) of kv head (b, g).
//
// Prologue: every load the block needs before its first step goes out together (the low-part
// flags of the query blocks it meets, this lane's K~ / V rows, the first tiles), so that the block
// waits for one memory round trip; only a block that uses the low part then fetches its first
// remainder tile.
template <int D>
__device__ void dkdv_block(const BwdArgs& a, DkdvLds<D>& S, int jt, int bg) {
    using M = Mfma<bf16>;
    constexpr int NCH = D / 16, NDT = D / 32;
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
    const bf16* __restrict__ qrot = reinterpret_cast<const bf16*>(a.qrot);
    const bf16* __restrict__ qrot_lo = reinterpret_cast<const bf16*>(a.qrot_lo);
    const bf16* __restrict__ dout = reinterpret_cast<const bf16*>(a.dout);

    const int nsph = (T_ - j0 + kTile - 1) / kTile;   // query steps per head
    const int nsteps = G * nsph;
    const int hq0 = b * a.Hq + g * G;                 // first query head of the group
    const int ntile = a.Tp / kTile;                   // (l', delta) tiles per head
    const int nblk = (T_ + kQBlk - 1) / kQBlk;        // 128-row query blocks per head (flags)
    // the low-part flags of the query blocks the key tile meets: head hh, blocks I0 + i; lane
    // hh * nI + i loads one (the load stays in flight until the ballot below)
    const int I0 = jt / 2, nI = nblk - I0, nfl = G * nI;
    const int* lofh = a.lof + (size_t)hq0 * nblk;
    const int f0 = lane < nfl ? lofh[(lane / nI) * nblk + I0 + lane % nI] : 0;
    // buffers over the group's query heads; step st covers query tile jt + st % nsph of head
    // hq0 + st / nsph (tile rows past T read another head's rows or zeros: l' = +inf there)
    const size_t hoff = (size_t)hq0 * T_ * D;
    const unsigned gbytes = (unsigned)(G * T_) * (unsigned)(D * 2);   // < 2^32: at most 2^31 - 1 elements
    const i32x4 rq = buffer_rsrc(qrot + hoff, gbytes);
    const i32x4 rql = buffer_rsrc(qrot_lo + hoff, gbytes);
    const i32x4 rg = buffer_rsrc(dout + hoff, gbytes);
    const i32x4 rld = buffer_rsrc(a.ld + (size_t)hq0 * ntile * 2 * kTile, (unsigned)(G * ntile) * (unsigned)(2 * kTile * 4));
    const unsigned lq = lds_addr(&S.q[0][0]), lql = lds_addr(&S.ql[0][0]), lg = lds_addr(&S.g[0][0]);
    const unsigned lld = lds_addr(&S.ld[0][0]);
    TileCopy<D> tc;
    tc.init(w, lane);
    // the tiles of step (head hh, query tile jt + t) that every block reads: Q~ hi, dO, (l', delta)
    auto issue = [&](int hh, int t, int buf) {
        const unsigned row0 = (unsigned)(hh * T_ + j0 + t * kTile) * (unsigned)(D * 2);
        const unsigned so = (unsigned)buf * TileCopy<D>::kBytes;
        tc.copy(rq, row0, lq + so, w);
        tc.copy(rg, row0, lg + so, w);
        if (lane < 8)
            copy16_to_lds(rld, (unsigned)(w * 128 + lane * 16), (unsigned)(hh * ntile + jt + t) * 512u,
                          lld + (unsigned)(buf * 512 + w * 128));
    };
    // a step's low-part tile: the query block's own remainder where the forward used it (flag f),
    // else the same buffer with size 0, whose reads land in LDS as zeros (those scores then equal
    // the forward's)
    auto issue_lo = [&](int hh, int t, int buf, int f) {
        const unsigned row0 = (unsigned)(hh * T_ + j0 + t * kTile) * (unsigned)(D * 2);
        i32x4 r = rql;
        r[2] = __builtin_amdgcn_readfirstlane(f ? r[2] : 0);
        tc.copy(r, row0, lql + (unsigned)buf * TileCopy<D>::kBytes, w);
    };
    issue(0, 0, 0);
    // the block's 64 K~ and V rows, copied whole into the second stage's Q~ and dO tiles (unused
    // until the second step's copies) and read from there into the operand layout: copies of
    // contiguous rows take a quarter of the memory requests of per-lane row loads.  Rows past T
    // read as zeros (those keys' results are not stored).
    {
        const unsigned kvbytes = (unsigned)T_ * (unsigned)(D * 2);
        const size_t kvoff = (size_t)bg * T_ * D;
        tc.copy(buffer_rsrc(reinterpret_cast<const bf16*>(a.krot) + kvoff, kvbytes), (unsigned)j0 * (unsigned)(D * 2),
                lq + TileCopy<D>::kBytes, w);
        tc.copy(buffer_rsrc(reinterpret_cast<const bf16*>(a.v) + kvoff, kvbytes), (unsigned)j0 * (unsigned)(D * 2),
                lg + TileCopy<D>::kBytes, w);
    }
    // A block uses the low-part tiles when any query block it meets has its flag set; its other
    // steps then read zeros there.  With at most 64 such blocks their flags are one wave-uniform
    // mask (bit hh * nI + i); beyond that a step reads its flag with a scalar load (these do not
    // share the vector-memory counter with the tile copies in flight: a vector load in the loop
    // would be waited for with vmcnt(0), i.e. after every copy issued so far).
    int fl = f0;
    for (int idx = lane + 64; idx < nfl; idx += 64) fl |= lofh[(idx / nI) * nblk + I0 + idx % nI];
    const unsigned long long fmask = __builtin_amdgcn_ballot_w64(f0 != 0);
    const bool lo = __builtin_amdgcn_ballot_w64(fl != 0) != 0;
    cint* lofs = (cint*)(unsigned long long)lofh;
    auto flag = [&](int hh, int t) -> int {
        const int i = (jt + t) / 2 - I0;
        if (nfl <= 64) return (int)((fmask >> (hh * nI + i)) & 1ull);
        return lofs[__builtin_amdgcn_readfirstlane(hh * nblk + I0 + i)];
    };
    if (lo) issue_lo(0, 0, 0, flag(0, 0));
    wait_vmcnt<0>();   // the key / value rows and the first tiles (see copy16_to_lds)
    step_barrier();    // every wave's copies have landed

    // this lane's key row: K~ and V as B operands
    bf16x8 kop[NCH], vop[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int o = Swz<D>::at(kloc, 16 * c + 8 * half);
        kop[c] = *reinterpret_cast<const bf16x8*>(&S.q[1][0] + o);
        vop[c] = *reinterpret_cast<const bf16x8*>(&S.g[1][0] + o);
    }
    __syncthreads();   // every wave has its rows before the second step's copies overwrite them

    // per-lane LDS offsets of the row fragments (query row 32*qh + col, chunks 2c + half)
    int roff[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) roff[c] = Swz<D>::at(32 * qh + col, 16 * c + 8 * half);
    // per-lane bases of the transposed dO / Q~ fragment reads (rows of this wave's query half)
    int trb[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) trb[dt] = tr_base<D>(32 * dt, lane) + 32 * qh * D;

    f32x16 dkt[NDT], dvt[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) { dkt[i] = f32x16{}; dvt[i] = f32x16{}; }

    // the step loop, with and without the low-part products
    auto run = [&](auto lo_c) {
        constexpr bool LO = decltype(lo_c)::value;
        int ih = 0, it = 1;                           // head / tile of the next step to issue
        if (it == nsph) { it = 0; ++ih; }
        int buf = 0, ct = 0;                          // stage and query tile of the current step
        for (int st = 0; st < nsteps; ++st) {
            wait_vmcnt<0>();                 // this wave's copies of tile st, the only ones in flight
            step_barrier();                  // tile st is complete; the other stage is free
            if (st + 1 < nsteps) {
                issue(ih, it, buf ^ 1);
                if constexpr (LO) issue_lo(ih, it, buf ^ 1, flag(ih, it));
                if (++it == nsph) { it = 0; ++ih; }
            }
            const bf16* Qs = S.q[buf];
            const bf16* Ql = S.ql[buf];
            const bf16* Gs = S.g[buf];
            const float* Ld = S.ld[buf];
            const bool first = ct == 0;
            if (!(first && kh > qh)) {        // blocks wholly above the diagonal are skipped
                // All LDS reads of a product are issued together ahead of it (sched_barrier keeps
                // the scheduler from sinking them next to their uses, which would expose the LDS
                // latency on every MFMA): row fragments and the accumulators' starting values (-l'
                // and -delta of the rows: register group rg holds 4 consecutive queries), then S /
                // dP; the transposed fragments of the dV / dK products are read while the softmax
                // waits for S and dP.
                bf16x8 qf[NCH], qlf[NCH], gf[NCH];
                f32x16 sacc, dp;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    qf[c] = *reinterpret_cast<const bf16x8*>(Qs + roff[c]);
                    if constexpr (LO) qlf[c] = *reinterpret_cast<const bf16x8*>(Ql + roff[c]);
                    gf[c] = *reinterpret_cast<const bf16x8*>(Gs + roff[c]);
                }
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int q0 = 32 * qh + 8 * rg + 4 * half;
                    const f32x4 nl = *reinterpret_cast<const f32x4*>(Ld + ld_lsc(q0));
                    const f32x4 nd = *reinterpret_cast<const f32x4*>(Ld + ld_dlt(q0));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sacc[4 * rg + e] = nl[e];
                        dp[4 * rg + e] = nd[e];
                    }
                }
                if (first && kh == qh) {      // diagonal block: keys after the query are masked
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (kloc > 32 * qh + acc_row(r, half)) sacc[r] = -INFINITY;
                }
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    sacc = M::mma(qf[c], kop[c], sacc);
                    dp = M::mma(gf[c], vop[c], dp);
                    if constexpr (LO) sacc = M::mma(qlf[c], kop[c], sacc);
                }
                __builtin_amdgcn_s_setprio(0);
                __builtin_amdgcn_sched_barrier(0);
                bf16x8 gt[2][NDT], qtf[2][NDT];
#pragma unroll
                for (int pc = 0; pc < 2; ++pc)
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        gt[pc][dt] = tr_frag_at<D>(Gs, trb[dt], 16 * pc);
                        qtf[pc][dt] = tr_frag_at<D>(Qs, trb[dt], 16 * pc);
                    }
                __builtin_amdgcn_sched_barrier(0);
                // P' = exp2(S' - l') and dS' = P' (dP - delta) for this wave's keys (lane) and
                // queries (registers), packed to bf16 as B operands of the dV / dK products
                bf16x8 pb[2], sb[2];
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    float p[4], d[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        p[e] = __builtin_amdgcn_exp2f(sacc[4 * rg + e]);
                        d[e] = p[e] * dp[4 * rg + e];
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
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int pc = 0; pc < 2; ++pc)
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        dvt[dt] = M::mma(gt[pc][dt], pb[pc], dvt[dt]);
                        dkt[dt] = M::mma(qtf[pc][dt], sb[pc], dkt[dt]);
                    }
                __builtin_amdgcn_s_setprio(0);
            }
            buf ^= 1;
            if (++ct == nsph) ct = 0;
        }
    };
    if (lo) run(std::true_type{});
    else run(std::false_type{});

    // the RoPE entries of the key rows this wave stores, issued first so that they arrive during
    // the reduction below (whose barriers are bare: __syncthreads would wait for these loads)
    const bool rope = a.rope_cs != nullptr;
    f32x4 cs[NDT][4];
    if (rope && qh == 0) load_acc_qcs<D>(a.qcs, min(key, T_ - 1), half, cs);
    // add the two query halves' partial dK^T / dV^T through LDS (reuses the tile buffers once
    // every wave is past its last step: the loop's LDS reads have all been consumed by then)
    step_barrier();
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
    step_barrier();   // (it waits for this wave's LDS writes, not for the loads above)
    if (qh == 0 && key < T_) {
        const float inv_scale = 1.f / a.scale;     // dV was accumulated from P' = scale * P
        const float inv_c = 1.f / (a.scale * kLog2e);   // dK from Q~' = scale * log2(e) * Q~
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
                    x[e] = (dkt[dt][r + e] + red[((kh * NDT + dt) * 16 + r + e) * 64 + lane]) * inv_c;
                    y[e] = (dvt[dt][r + e] + red[(((2 + kh) * NDT + dt) * 16 + r + e) * 64 + lane]) * inv_scale;
                }
                const int d = 32 * dt + acc_row(r, half);
                if (rope) unrotate4(x, cs[dt][r / 4]);
                *reinterpret_cast<bf16x4*>(dk + d) = cvt4(x);
                *reinterpret_cast<bf16x4*>(dv + d) = cvt4(y);
            }
    }
}

// ---------------------------------------------------------------------------------------------
// dQ block: queries [i0, i0 + 128) of query head (b, h).  As in the dK/dV block, the prologue's
// loads (the block's low-part flag, the first key / value tiles, this lane's Q~' and dO rows and
// (l', delta)) go out together; a block that uses the low part (as the forward did for it) then
// loads its remainder rows.
template <int D>
__device__ void dq_block(const BwdArgs& a, DqLds<D>& S, int qt, int bh) {
    using M = Mfma<bf16>;
    constexpr int NCH = D / 16, NDT = D / 32;
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
    const int nblk = (T_ + kQBlk - 1) / kQBlk;
    const int flag = ((cint*)(unsigned long long)a.lof)[(size_t)bh * nblk + qt];   // scalar load

    const int kv_end = min(T_, i0 + kQBlk);
    const int nsteps = (kv_end + kTile - 1) / kTile;
    // buffers over kv head bg (key rows past T read as zeros; they are causally masked)
    const unsigned hbytes = (unsigned)T_ * (unsigned)(D * 2);
    const i32x4 rk = buffer_rsrc(reinterpret_cast<const bf16*>(a.krot) + (size_t)bg * T_ * D, hbytes);
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
    // the block's 128 Q~' (hi) and dO rows, copied whole (Q~' into xq, dO into the second stage,
    // unused until the second step's copies) and read from there into the operand layout, as the
    // dK/dV block does with its key rows.  Rows past T read as zeros (not stored).
    {
        const unsigned qbytes = (unsigned)T_ * (unsigned)(D * 2);
        const size_t hoff = (size_t)bh * T_ * D;
        const i32x4 rq = buffer_rsrc(reinterpret_cast<const bf16*>(a.qrot) + hoff, qbytes);
        const i32x4 rg = buffer_rsrc(reinterpret_cast<const bf16*>(a.dout) + hoff, qbytes);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const unsigned row0 = (unsigned)(i0 + t * kTile) * (unsigned)(D * 2);
            tc.copy(rq, row0, lds_addr(&S.xq[t][0]), w);
            tc.copy(rg, row0, t == 0 ? lk + TileCopy<D>::kBytes : lv + TileCopy<D>::kBytes, w);
        }
    }

    // this lane's query row: Q~' (hi, and lo for a flagged block) and dO as B operands, -l' and -delta
    bf16x8 qop[NCH], qlo[NCH], gop[NCH];
    const int rowc = min(qrow, T_ - 1);
    const float* ldt = a.ld + ((size_t)bh * (a.Tp / kTile) + rowc / kTile) * 2 * kTile;
    const float nlsc = ldt[ld_lsc(rowc % kTile)];      // -l'
    const float ndlt = ldt[ld_dlt(rowc % kTile)];      // -delta
    const bool lo = flag != 0;
    if (lo) {
        const bf16* ql = reinterpret_cast<const bf16*>(a.qrot_lo) + qoff + 8 * half;
#pragma unroll
        for (int c = 0; c < NCH; ++c) qlo[c] = *reinterpret_cast<const bf16x8*>(ql + 16 * c);
    }
    wait_vmcnt<0>();   // the rows, (l', delta) and the first tile (see copy16_to_lds)
    step_barrier();    // every wave's copies have landed
    {
        const bf16* xq = &S.xq[w >> 1][0];
        const bf16* xg = (w >> 1) ? &S.v[1][0] : &S.k[1][0];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int o = Swz<D>::at(32 * (w & 1) + col, 16 * c + 8 * half);
            qop[c] = *reinterpret_cast<const bf16x8*>(xq + o);
            gop[c] = *reinterpret_cast<const bf16x8*>(xg + o);
        }
    }
    __syncthreads();   // every wave has its rows before the second step's copies overwrite them

    // per-lane LDS offsets of the key / value row fragments (row 32*kt + col, chunks 2c + half)
    int roff[2][NCH];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int c = 0; c < NCH; ++c) roff[kt][c] = Swz<D>::at(32 * kt + col, 16 * c + 8 * half);
    // per-lane bases of the transposed K~ fragment reads (one per 32 columns of d)
    int ktb[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) ktb[dt] = tr_base<D>(32 * dt, lane);

    f32x16 dqt[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) dqt[i] = f32x16{};
    // -l' as the starting value of the score products (one query per lane), so that the products
    // themselves subtract it
    f32x16 nl16;
#pragma unroll
    for (int r = 0; r < 16; ++r) nl16[r] = nlsc;

    // the step loop, with and without the low-part products
    auto run = [&](auto lo_c) {
        constexpr bool LO = decltype(lo_c)::value;
        int buf = 0;                                  // stage of the current step
        for (int st = 0; st < nsteps; ++st) {
            wait_vmcnt<0>();                 // this wave's copies of tile st, the only ones in flight
            step_barrier();                  // tile st is complete; the other stage is free
            if (st + 1 < nsteps) issue(st + 1, buf ^ 1);
            const int j0 = st * kTile;
            // the step's work; DIAG: the tile reaches past the wave's first query, so some of its
            // keys come after some of the wave's queries and are masked (only there: the compare
            // and select of the mask cost as many vector instructions as the softmax itself)
            auto body = [&](auto diag_c) {
                constexpr bool DIAG = decltype(diag_c)::value;
                const bf16* Ks = S.k[buf];
                const bf16* Vs = S.v[buf];
                // Per 32-key half (kt): its key / value row fragments, then its score and dP products,
                // the scores starting from -l' (the masked keys of a diagonal tile from -inf).  L
                // and delta are known, so a half's dS' needs only its own products: the fragments of
                // half 1 are read while the products of half 0 run, the softmax of half 0 is slotted
                // between the products of half 1, and that of half 1 between the dQ products of half
                // 0, so that vector work and matrix products of one wave overlap
                auto sinit = [&](int kt) {
                    if constexpr (DIAG) {
                        f32x16 m;
#pragma unroll
                        for (int r = 0; r < 16; ++r) m[r] = j0 + 32 * kt + acc_row(r, half) > qrow ? -INFINITY : nlsc;
                        return m;
                    } else {
                        return nl16;
                    }
                };
                bf16x8 kf0[NCH], vf0[NCH];
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    kf0[c] = *reinterpret_cast<const bf16x8*>(Ks + roff[0][c]);
                    vf0[c] = *reinterpret_cast<const bf16x8*>(Vs + roff[0][c]);
                }
                __builtin_amdgcn_sched_barrier(0);
                f32x16 sT[2], dpT[2];
                sT[0] = M::mma(kf0[0], qop[0], sinit(0));
                dpT[0] = M::mma(vf0[0], gop[0], f32x16{});
                if constexpr (LO) sT[0] = M::mma(kf0[0], qlo[0], sT[0]);
#pragma unroll
                for (int c = 1; c < NCH; ++c) {
                    sT[0] = M::mma(kf0[c], qop[c], sT[0]);
                    dpT[0] = M::mma(vf0[c], gop[c], dpT[0]);
                    if constexpr (LO) sT[0] = M::mma(kf0[c], qlo[c], sT[0]);
                }
                __builtin_amdgcn_sched_barrier(0);
                bf16x8 kf1[NCH], vf1[NCH], ktf[4][NDT];
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    kf1[c] = *reinterpret_cast<const bf16x8*>(Ks + roff[1][c]);
                    vf1[c] = *reinterpret_cast<const bf16x8*>(Vs + roff[1][c]);
                }
#pragma unroll
                for (int pc = 0; pc < 4; ++pc)
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) ktf[pc][dt] = tr_frag_at<D>(Ks, ktb[dt], 16 * pc);
                __builtin_amdgcn_sched_barrier(0);
                // dS'^T = P' (dP^T - delta) of register group rg of half kt, packed into the B
                // operand chunk 2 kt + rg / 2 (4 chunks of 16 keys)
                bf16x8 sb[4];
                auto ds_group = [&](int kt, int rg) {
                    float d[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * rg + e;
                        d[e] = __builtin_amdgcn_exp2f(sT[kt][r]) * (dpT[kt][r] + ndlt);
                    }
                    const bf16x4 d4 = cvt4(d);
                    const int pc = 2 * kt + (rg >> 1);
                    if (rg & 1) sb[pc] = __builtin_shufflevector(sb[pc].lo, d4, 0, 1, 2, 3, 4, 5, 6, 7);
                    else sb[pc] = __builtin_shufflevector(d4, d4, 0, 1, 2, 3, 4, 5, 6, 7);
                };
                // products of half 1, chunk by chunk, each followed by its share of half 0's groups
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    sT[1] = M::mma(kf1[c], qop[c], c == 0 ? sinit(1) : sT[1]);
                    dpT[1] = M::mma(vf1[c], gop[c], c == 0 ? f32x16{} : dpT[1]);
                    if constexpr (LO) sT[1] = M::mma(kf1[c], qlo[c], sT[1]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int rg = c * 4 / NCH; rg < (c + 1) * 4 / NCH; ++rg) ds_group(0, rg);
                    __builtin_amdgcn_sched_barrier(0);
                }
                // dQ~^T (D x 32 queries) += K~^T dS'^T (K = the tile's keys, accumulator order):
                // the chunks of half 0, each followed by two of half 1's groups, then those of half 1
#pragma unroll
                for (int pc = 0; pc < 2; ++pc) {
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) dqt[dt] = M::mma(ktf[pc][dt], sb[pc], dqt[dt]);
                    __builtin_amdgcn_sched_barrier(0);
                    ds_group(1, 2 * pc);
                    ds_group(1, 2 * pc + 1);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int pc = 2; pc < 4; ++pc)
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) dqt[dt] = M::mma(ktf[pc][dt], sb[pc], dqt[dt]);
            };
            if (j0 + kTile - 1 <= wq0) body(std::false_type{});
            else if (j0 <= wq0 + 31) body(std::true_type{});   // some key at or before some query of the wave
            buf ^= 1;
        }
    };
    if (lo) run(std::true_type{});
    else run(std::false_type{});

    // dQ = R^T dQ~ ; lane owns one query, 4 consecutive d per register group
    if (qrow < T_) {
        const bool rope = a.rope_cs != nullptr;
        f32x4 cs[NDT][4];
        if (rope) load_acc_qcs<D>(a.qcs, qrow, half, cs);
        bf16* __restrict__ dq = reinterpret_cast<bf16*>(a.dq) + ((size_t)bh * T_ + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                float x[4] = {dqt[dt][r], dqt[dt][r + 1], dqt[dt][r + 2], dqt[dt][r + 3]};
                const int d = 32 * dt + acc_row(r, half);
                if (rope) unrotate4(x, cs[dt][r / 4]);
                *reinterpret_cast<bf16x4*>(dq + d) = cvt4(x);
            }
    }
}

// workgroups per CU the kernel is compiled for: two (≤ 256 registers per wave) up to head_dim 64;
// at 128 a dK/dV wave needs more than 256, so one
template <int D> struct BwdOcc { static constexpr int MINB = 2; };
template <> struct BwdOcc<128> { static constexpr int MINB = 1; };

// block -> (key tile, kv group) of a dK/dV block, and -> (query tile, query head) of a dQ block.
// Workgroups are dispatched round-robin over the XCDs: block i runs on XCD i % 8.  When the kv
// groups divide evenly, all blocks of kv group bg (its dK/dV tiles and the dQ tiles of its query
// heads) go to XCD bg % 8, so that the group's Q~, dO, K~ and V are fetched into one L2 only.
// dK/dV blocks come key tile 0 first (it carries the most causal work), dQ blocks last query tile
// first.
__device__ inline void dkdv_index(int blk, int BG, int& jt, int& bg) {
    if (BG % kXcds == 0) {
        const int x = blk % kXcds, j = blk / kXcds, gpx = BG / kXcds;
        jt = j / gpx;
        bg = (j % gpx) * kXcds + x;
    } else {
        jt = blk / BG;
        bg = blk % BG;
    }
}
__device__ inline void dq_index(int blk, int BG, int G, int nqt, int& qt, int& bh) {
    if (BG % kXcds == 0) {
        const int x = blk % kXcds, r = blk / kXcds, per = BG / kXcds * G;
        const int bg = ((r % per) / G) * kXcds + x;
        qt = nqt - 1 - r / per;
        bh = bg * G + (r % per) % G;
    } else {
        const int BH = BG * G;
        qt = nqt - 1 - blk / BH;
        bh = blk % BH;
    }
}

// The two roles in one grid: the dK/dV blocks first, then the dQ blocks (each XCD gets its groups'
// blocks of both roles in this order).
template <int D>
__global__ __launch_bounds__(kThreads, BwdOcc<D>::MINB) void bwd_bf16_kernel(BwdArgs a) {
    __shared__ BwdLds<D> S;
    const int BG = a.B * a.Hkv, G = a.Hq / a.Hkv;
    const int nkv = (a.T + kTile - 1) / kTile;
    const int nqt = (a.T + kQBlk - 1) / kQBlk;
    const int ndk = nkv * BG;
    int blk = (int)blockIdx.x;
    if (BG % kXcds == 0) {
        // per XCD: its dK/dV blocks, then its dQ blocks
        const int x = blk % kXcds, j = blk / kXcds, dpx = ndk / kXcds;
        if (j < dpx) {
            int jt, bg;
            dkdv_index(j * kXcds + x, BG, jt, bg);
            dkdv_block<D>(a, S.kv, jt, bg);
        } else {
            int qt, bh;
            dq_index((j - dpx) * kXcds + x, BG, G, nqt, qt, bh);
            dq_block<D>(a, S.q, qt, bh);
        }
    } else if (blk < ndk) {
        int jt, bg;
        dkdv_index(blk, BG, jt, bg);
        dkdv_block<D>(a, S.kv, jt, bg);
    } else {
        int qt, bh;
        dq_index(blk - ndk, BG, G, nqt, qt, bh);
        dq_block<D>(a, S.q, qt, bh);
    }
}

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// Per 128-row query block of one head (b, h): -l' and -delta of its rows (delta = sum_d dO O,
// l' = L log2(e) - log2(scale)) into the tile layout of ld_lsc, rows past T up to the end of their
// 64-row tile getting -inf and 0.  ROT (the plain backward, whose forward kept nothing): also the
// block's low-part flag, made as the forward makes it (max |q| over the block's raw rows against
// the largest max |k| of the key tiles the block sees, written beforehand by key_rot_kernel), and
// Q~' = scale log2(e) R q as bf16 hi, with the remainder lo for a flagged block.  All loads of a
// thread are issued before any is used.
template <int D, bool ROT>
__global__ __launch_bounds__(kThreads) void bwd_pre_bf16_kernel(BwdArgs a) {
    constexpr int CPR = D / 8, NU = kQBlk * CPR / kThreads;   // 16-byte chunks per row / per thread
    static_assert(NU >= 1 && kQBlk * CPR % kThreads == 0, "chunks must cover the threads evenly");
    __shared__ float red[kThreads / 64];
    const int T_ = a.T;
    const int nblk = (T_ + kQBlk - 1) / kQBlk;
    long bh;
    int I;
    {
        // the rows of kv group bg go to XCD bg % 8, as the main kernel's blocks of that group do,
        // so that the dO rows read here are still in that XCD's L2 when the main kernel runs
        const int BG = a.B * a.Hkv, G = a.Hq / a.Hkv;
        const int blk = (int)blockIdx.x;
        if (BG % kXcds == 0) {
            const int x = blk % kXcds, j = blk / kXcds, per = G * nblk;
            bh = (long)((j / per) * kXcds + x) * G + (j % per) / nblk;
            I = (j % per) % nblk;
        } else {
            bh = blk / nblk;
            I = blk % nblk;
        }
    }
    const int tid = threadIdx.x;
    const size_t hbase = (size_t)bh * T_ * D;
    const bf16* __restrict__ o = reinterpret_cast<const bf16*>(a.o) + hbase;
    const bf16* __restrict__ g = reinterpret_cast<const bf16*>(a.dout) + hbase;
    const bf16* __restrict__ q = reinterpret_cast<const bf16*>(a.q) + hbase;
    bf16x8 xo[NU], xg[NU], xq[NU];
    f32x4 cs[NU][2];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int idx = u * kThreads + tid, r = idx / CPR, part = idx % CPR, t = I * kQBlk + r;
        if (t < T_) {
            xo[u] = *reinterpret_cast<const bf16x8*>(o + (size_t)t * D + part * 8);
            xg[u] = *reinterpret_cast<const bf16x8*>(g + (size_t)t * D + part * 8);
            if constexpr (ROT) {
                xq[u] = *reinterpret_cast<const bf16x8*>(q + (size_t)t * D + part * 8);
                if (a.rope_cs) {
                    const f32x4* c = reinterpret_cast<const f32x4*>(a.rope_cs + (size_t)t * D + part * 8);
                    cs[u][0] = c[0];
                    cs[u][1] = c[1];
                }
            }
        }
    }
    const float nlog2s = __log2f(a.scale);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int idx = u * kThreads + tid, r = idx / CPR, part = idx % CPR, t = I * kQBlk + r;
        float sum = 0.f;
        if (t < T_) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sum += (float)xo[u][e] * (float)xg[u][e];
        }
#pragma unroll
        for (int o2 = 1; o2 < CPR; o2 <<= 1) sum += __shfl_xor(sum, o2, 64);   // the row's CPR chunks
        if (part == 0 && t < a.Tp) {
            float* ldt = a.ld + ((size_t)bh * (a.Tp / kTile) + t / kTile) * 2 * kTile;
            ldt[ld_lsc(t % kTile)] = t < T_ ? nlog2s - a.lse[(size_t)bh * T_ + t] * kLog2e : -INFINITY;
            ldt[ld_dlt(t % kTile)] = -sum;
        }
    }
    if constexpr (ROT) {
        float m = 0.f;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int idx = u * kThreads + tid, t = I * kQBlk + idx / CPR;
            if (t < T_) {
#pragma unroll
                for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)xq[u][e]));
            }
        }
        m = wave_max(m);
        if ((tid & 63) == 0) red[tid >> 6] = m;
        const int G = a.Hq / a.Hkv;
        const long bg = bh / a.Hq * a.Hkv + bh % a.Hq / G;
        const int ntk = (T_ + kTile - 1) / kTile;
        const int nvis = min(2 * I + 2, ntk);
        float km = 0.f;
        for (int j = tid & 63; j < nvis; j += 64) km = fmaxf(km, a.ak[bg * ntk + j]);
        km = wave_max(km);
        __syncthreads();
        float aq = red[0];
#pragma unroll
        for (int i = 1; i < kThreads / 64; ++i) aq = fmaxf(aq, red[i]);
        const bool lo = a.scale * (float)D * aq * km > kLoBound;
        if (tid == 0) a.lof[bh * nblk + I] = lo ? 1 : 0;
        const float c = a.scale * kLog2e;
        bf16* __restrict__ qh = reinterpret_cast<bf16*>(a.qrot) + hbase;
        bf16* __restrict__ ql = reinterpret_cast<bf16*>(a.qrot_lo) + hbase;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int idx = u * kThreads + tid, r = idx / CPR, part = idx % CPR, t = I * kQBlk + r;
            if (t >= T_) continue;
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = (float)xq[u][e];
            if (a.rope_cs) {
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {
                    const float cc = cs[u][pr / 2][2 * (pr % 2)], sn = cs[u][pr / 2][2 * (pr % 2) + 1];
                    const float y0 = y[2 * pr], y1 = y[2 * pr + 1];
                    y[2 * pr] = y0 * cc - y1 * sn;
                    y[2 * pr + 1] = y0 * sn + y1 * cc;
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= c;
            const bf16x8 hi = cvt8(y);
            *reinterpret_cast<bf16x8*>(qh + (size_t)t * D + part * 8) = hi;
            if (lo) *reinterpret_cast<bf16x8*>(ql + (size_t)t * D + part * 8) = remainder8(y, hi);
        }
    }
}

}  // namespace

template <int D>
hipError_t launch_bwd_pre_bf16(const BwdArgs& a, hipStream_t stream, bool rotate) {
    const dim3 grid((unsigned)((long)a.B * a.Hq * ((a.T + kQBlk - 1) / kQBlk)));
    if (rotate) hipLaunchKernelGGL((bwd_pre_bf16_kernel<D, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((bwd_pre_bf16_kernel<D, false>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_main_bf16(const BwdArgs& a, hipStream_t stream) {
    const long ndk = (long)((a.T + kTile - 1) / kTile) * a.B * a.Hkv;
    const long ndq = (long)((a.T + kQBlk - 1) / kQBlk) * a.B * a.Hq;
    hipLaunchKernelGGL((bwd_bf16_kernel<D>), dim3((unsigned)(ndk + ndq)), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template hipError_t launch_bwd_pre_bf16<128>(const BwdArgs&, hipStream_t, bool);
template hipError_t launch_bwd_pre_bf16<64>(const BwdArgs&, hipStream_t, bool);
template hipError_t launch_bwd_pre_bf16<32>(const BwdArgs&, hipStream_t, bool);
template hipError_t launch_bwd_main_bf16<128>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_main_bf16<64>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_main_bf16<32>(const BwdArgs&, hipStream_t);

}  // namespace ne
