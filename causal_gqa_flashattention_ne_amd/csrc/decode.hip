// decode.hip -- decode-time attention on gfx950: n new tokens per sequence against a KV cache.
//
// The attention of the forward (tiling plus an online softmax; agentlenshq NanoEuler page,
// section "커널 구현"), for the generation path where a few new tokens attend to every cached
// position (the chat / token-by-token inference the NanoEuler pages describe).  The cache holds
// keys already rotated at their own positions (RoPE, same page, "기술 사양", is applied to each
// key once, when it is appended); token i of sequence b is rotated at position kv_len[b] - n + i
// and sees the keys 0 .. kv_len[b] - n + i.
//
// Split-KV: a sequence's key range is cut into chunks of `chunk` keys.  One wave per (batch,
// kv head, chunk) runs the online softmax over its chunk for all G * n query columns of the kv
// group at once (G query heads x n tokens, at most 32: one lane per column as in the forward, so
// every key / value tile is read once per kv group), and writes the chunk's normalised O and its
// L.  Tiles reach LDS through the copy pipeline of tiles.hpp (three stages, two tiles ahead).
// decode_merge then combines the chunks by log-sum-exp:
//     L = log sum_s exp(L_s),   O = sum_s exp(L_s - L) O_s.
// The work is a stream over the cache: HBM-bound, the matrix cores idle most of the time.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace ne {

namespace {

constexpr int kTile = kTileRows;       // keys per step
constexpr float kRescale = 8.f;        // log2 units of headroom before the running max is moved

__device__ inline float partner_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float partner_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct alignas(16) DecLds {
    alignas(16) bf16 k[kStages][kTile * D];    // K~ tiles [key][d] (swizzled)
    alignas(16) bf16 v[kStages][kTile * D];    // V tiles
};

// One wave: chunk s of kv head (b, g).
template <int D>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
    using M = Mfma<bf16>;
    using TC = TileCopy<D, 1>;
    constexpr int NCH = D / 16, NDT = D / 32;
    constexpr int kCopies = 2 * TC::NU;           // copies per tile pair (K~ and V)
    __shared__ DecLds<D> S;

    const int lane = threadIdx.x, col = lane & 31, half = lane >> 5;
    const int s = (int)blockIdx.x % a.nsplit, bg = (int)blockIdx.x / a.nsplit;
    const int b = bg / a.Hkv, g = bg % a.Hkv, G = a.Hq / a.Hkv;
    const int ncol = G * a.n;
    const int lb = min(max(a.kv_len[b], a.n), a.Tc);   // valid cache rows (clamped into [n, Tc])
    const int k0 = s * a.chunk, k1 = min(k0 + a.chunk, lb);
    float* __restrict__ po = a.part_o + ((size_t)bg * a.nsplit + s) * 32 * D;
    float* __restrict__ pl = a.part_l + ((size_t)bg * a.nsplit + s) * 32;
    if (k0 >= k1) {                                  // chunk past the sequence: weight 0 in the merge
        if (half == 0) pl[col] = -INFINITY;
        return;
    }

    // buffers over this kv head's cache rows 0 .. lb - 1 (rows past lb read as zeros)
    const unsigned hbytes = (unsigned)lb * (unsigned)(D * 2);
    const i32x4 rk = buffer_rsrc(reinterpret_cast<const bf16*>(a.kc) + (size_t)bg * a.Tc * D, hbytes);
    const i32x4 rv = buffer_rsrc(reinterpret_cast<const bf16*>(a.vc) + (size_t)bg * a.Tc * D, hbytes);
    const unsigned lk = lds_addr(&S.k[0][0]), lv = lds_addr(&S.v[0][0]);
    TC tc;
    tc.init(0, lane);
    const int ntile = (k1 - k0 + kTile - 1) / kTile;
    auto issue = [&](int t) {
        const unsigned row0 = (unsigned)(k0 + t * kTile) * (unsigned)(D * 2);
        const unsigned so = (unsigned)(t % kStages) * TC::kBytes;
        tc.copy(rk, row0, lk + so, 0);
        tc.copy(rv, row0, lv + so, 0);
    };
    issue(0);
    if (ntile > 1) issue(1);

    // this lane's query column: head g*G + hh, token ti at position lb - n + ti (columns past
    // G * n repeat column 0 and are never stored)
    const int c = col < ncol ? col : 0;
    const int hh = c / a.n, ti = c % a.n;
    const int pos = lb - a.n + ti;
    const float* __restrict__ cs = a.rope_cs;
    bf16x8 qhi[NCH], qlo[NCH];
    row_operands<D>(reinterpret_cast<const bf16*>(a.q) + (((size_t)b * a.Hq + g * G + hh) * a.n + ti) * D, cs, pos,
                    half, qhi, qlo);
    wait_vmcnt<0>();   // query operands and the first two tiles (see copy16_to_lds)

    int roff[2][NCH];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) roff[kt][ch] = Swz<D>::at(32 * kt + col, 16 * ch + 8 * half);

    const float c2 = a.scale * kLog2e;
    f32x16 oacc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    for (int t = 0; t < ntile; ++t) {
        if (t + 1 < ntile) wait_vmcnt<kCopies>();
        else wait_vmcnt<0>();
        if (t + 2 < ntile) issue(t + 2);      // stage (t + 2) % 3 was last read in step t - 1
        const int buf = t % kStages;
        const int j0 = k0 + t * kTile;
        const bf16* Ks = S.k[buf];
        const bf16* Vs = S.v[buf];
        bf16x8 kf[2][NCH];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) kf[kt][ch] = *reinterpret_cast<const bf16x8*>(Ks + roff[kt][ch]);
        f32x16 sT[2];
        sT[0] = M::mma(kf[0][0], qhi[0], f32x16{});
        sT[1] = M::mma(kf[1][0], qhi[0], f32x16{});
        sT[0] = M::mma(kf[0][0], qlo[0], sT[0]);
        sT[1] = M::mma(kf[1][0], qlo[0], sT[1]);
#pragma unroll
        for (int ch = 1; ch < NCH; ++ch) {
            sT[0] = M::mma(kf[0][ch], qhi[ch], sT[0]);
            sT[1] = M::mma(kf[1][ch], qhi[ch], sT[1]);
            sT[0] = M::mma(kf[0][ch], qlo[ch], sT[0]);
            sT[1] = M::mma(kf[1][ch], qlo[ch], sT[1]);
        }
        bf16x8 vf[4][NDT];
#pragma unroll
        for (int pc = 0; pc < 4; ++pc) {
            const int kb0 = 32 * (pc >> 1) + 16 * (pc & 1) + 4 * half;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) vf[pc][dt] = tr_frag_swz<D>(Vs, 32 * dt, kb0, kb0 + 8, lane);
        }
        // keys past the chunk or after this column's token are invisible: S = -inf for the max,
        // P = 0 (a column may see no key of a whole tile, or of the whole chunk)
        const bool edge = j0 + kTile > k1 || j0 + kTile - 1 > lb - a.n;
        unsigned long long vis = ~0ull;               // bit 16 kt + r: key visible
        if (edge) {
            vis = 0;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = j0 + 32 * kt + acc_row(r, half);
                    if (j < k1 && j <= pos) vis |= 1ull << (16 * kt + r);
                    else sT[kt][r] = -INFINITY;
                }
        }
        float mx = sT[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sT[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sT[1][r]);
        mx = partner_max(mx) * c2;
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescale) != 0) {
            const float m_new = fmaxf(m_run, mx);
            // 0 when this lane's first visible key arrives; 1 while it has seen none (m_new = -inf)
            const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
            m_run = m_new;
        }
        bf16x8 pb[4];
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * rg + e;
                    p[e] = (vis >> (16 * kt + r)) & 1 ? __builtin_amdgcn_exp2f(__builtin_fmaf(sT[kt][r], c2, -m_run)) : 0.f;
                    ls += p[e];
                }
                const bf16x4 p4 = cvt4(p);
                const int pc = 2 * kt + (rg >> 1);
                if (rg & 1) pb[pc] = __builtin_shufflevector(pb[pc].lo, p4, 0, 1, 2, 3, 4, 5, 6, 7);
                else pb[pc] = __builtin_shufflevector(p4, p4, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        l_run += ls;
#pragma unroll
        for (int pc = 0; pc < 4; ++pc)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) oacc[dt] = M::mma(vf[pc][dt], pb[pc], oacc[dt]);
    }

    // the chunk's normalised O and L; a column that saw no key here gets L = -inf
    const float l_tot = partner_sum(l_run);
    if (col < ncol) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float* __restrict__ orow = po + (size_t)col * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                const f32x4 x = {oacc[dt][r] * inv, oacc[dt][r + 1] * inv, oacc[dt][r + 2] * inv, oacc[dt][r + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + 32 * dt + acc_row(r, half)) = x;
            }
        if (half == 0) pl[col] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

// One wave per (kv head, query column): lane s < nsplit holds L_s; lane d the output element d.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
    const int G = a.Hq / a.Hkv, ncol = G * a.n;
    const int bg = (int)blockIdx.x / ncol, col = (int)blockIdx.x % ncol;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int lane = threadIdx.x;
    const float* __restrict__ pl = a.part_l + (size_t)bg * a.nsplit * 32 + col;
    const float Ls = lane < a.nsplit ? pl[(size_t)lane * 32] : -INFINITY;
    float mx = Ls;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    const float wgt = Ls == -INFINITY ? 0.f : __expf(Ls - mx);   // every column sees key 0: mx finite
    float sum = wgt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o, 64);
    float acc = 0.f;
    const float* __restrict__ po = a.part_o + (size_t)bg * a.nsplit * 32 * D + (size_t)col * D + lane;
    for (int sp = 0; sp < a.nsplit; ++sp) {
        const float ws = __shfl(wgt, sp, 64);
        if (ws != 0.f && lane < D) acc += ws * po[(size_t)sp * 32 * D];
    }
    const int hh = col / a.n, ti = col % a.n;
    const size_t row = ((size_t)b * a.Hq + g * G + hh) * a.n + ti;
    if (lane < D) reinterpret_cast<bf16*>(a.o)[row * D + lane] = (bf16)(acc / sum);
    if (lane == 0) a.lse[row] = mx + __logf(sum);
}

// ---------------------------------------------------------------------------------------------
// Balanced path for at most 16 query columns per kv group (G * n <= 16: the usual decode, where a
// kv head serves a few query heads and one or a few new tokens).
//
// The products use the 16 x 16 x 32 bf16 MFMA (result (i, j) in lane j + 16 (i / 4), register
// i % 4), so a 16-column group costs half the matrix work and half the softmax values of the
// 32-column layout.  Lane (c = lane % 16, g = lane / 16) owns query column c:
//   S^T = K~ Q~^T   A = K~ rows (key 16 kb + lane % 16, d = 32 ks + 8 g + 0..7), B = Q~ operands;
//                   lane (c, g) receives the scores of keys 16 kb + 4 g + 0..3;
//   O^T += V^T P^T  k slot 8 g + e of step k2 is key 32 k2 + 4 g + e (e < 4) or
//                   32 k2 + 16 + 4 g + e - 4 (e >= 4): exactly the scores lane (c, g) holds, so P^T
//                   is its own B operand; V^T comes from transposed LDS reads in the same order.
//
// Work split: the (batch, kv head) segments of valid tiles are laid end to end (sequence-major,
// kv head inside) and the W waves of the grid take equal shares [w T / W, (w + 1) T / W) of that
// line, T the total, whatever the mix of cache lengths.  A wave walks the segment pieces of its
// share.  A piece that is a whole segment writes O and L directly; otherwise it writes its
// normalised O and its L to partial slot w + segment (slots are unique along the line), and the
// last piece of the segment to arrive, counted on a per-segment arrival counter, merges all of
// them by log-sum-exp and resets the counter to zero for the next call.
template <int D, int TR, int NS>
struct alignas(16) Dec16Lds {
    alignas(16) bf16 k[NS][TR * D];    // K~ tiles [key][d] (swizzled)
    alignas(16) bf16 v[NS][TR * D];    // V tiles
};

__device__ inline float pair16_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair16_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// max / sum over the four lanes (c, g = 0..3) of a column
__device__ inline float col_max(float x) { return partner_max(pair16_max(x)); }
__device__ inline float col_sum(float x) { return partner_sum(pair16_sum(x)); }

__device__ inline f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline int wave_sum(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}
__device__ inline int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

// wait until at most `ahead` (0 .. MAXA) tiles of KC copies each are still in flight
template <int KC, int MAXA>
__device__ inline void wait_tiles(int ahead) {
    if constexpr (MAXA > 0) {
        if (ahead >= MAXA) {
            wait_vmcnt<MAXA * KC>();
            return;
        }
        wait_tiles<KC, MAXA - 1>(ahead);
    } else {
        wait_vmcnt<0>();
    }
}

// Q~ operands of one query row for the 16 x 16 x 32 layout: lane group g supplies
// d = 32 ks + 8 g + 0..7, rotated to R_pos q in float32 (ROPE) and split into bf16 hi + lo.  All
// loads are issued before any is used.
template <int D, bool ROPE>
__device__ inline void q_operands16(const bf16* rowp, const float* cs, int pos, int g, bf16x8* hi, bf16x8* lo) {
    constexpr int KS = D / 32;
    bf16x8 raw[KS];
    f32x4 cv[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) raw[ks] = *reinterpret_cast<const bf16x8*>(rowp + 32 * ks + 8 * g);
    if constexpr (ROPE) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                cv[ks][h] = *reinterpret_cast<const f32x4*>(cs + (size_t)pos * D + 32 * ks + 8 * g + 4 * h);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)raw[ks][e];
        if constexpr (ROPE) {
            // pairs (x[2p], x[2p+1]) with table entry (cos, sin) = cv[ks][p / 2][2 (p % 2) + 0..1]
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const float co = cv[ks][pp >> 1][2 * (pp & 1)], si = cv[ks][pp >> 1][2 * (pp & 1) + 1];
                const float x0 = x[2 * pp], x1 = x[2 * pp + 1];
                x[2 * pp] = x0 * co - x1 * si;
                x[2 * pp + 1] = x0 * si + x1 * co;
            }
        }
        hi[ks] = cvt8(x);
        lo[ks] = remainder8(x, hi[ks]);
    }
}

// a value every lane holds alike, moved to scalar registers
__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline long long uniform(long long x) {
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)x);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)((unsigned long long)x >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}

__device__ inline int valid_rows(const DecodeArgs& a, int b) { return min(max(a.kv_len[b], a.n), a.Tc); }
// through a read-only, unaliased kernel argument: a scalar load for a wave-uniform b
__device__ inline int valid_rows(const DecodeArgs& a, const int* __restrict__ kv_len, int b) {
    return min(max(kv_len[b], a.n), a.Tc);
}

// Wave w's share of the line is [floor(w T / W), floor((w + 1) T / W)); shares are empty only
// when T < W, and then every non-empty share is a single tile.
// the wave whose share holds line position x: the largest w with floor(w T / W) <= x
__device__ inline int wave_of(long long x, long long total, int W) {
    return (int)(((x + 1) * W - 1) / total);
}

// Piece results cross waves, and XCDs whose L2 caches are not coherent with each other, through
// device-scope (sc1) buffer stores and loads, coherent at that scope without the L2 write-back
// and invalidation of a device-scope fence.  Slot layout: O as [DB][64 lanes][4] floats (each
// instruction moves 1 KiB contiguously), L as [16 columns].
constexpr int kDeviceScope = 16;                 // buffer cache policy: sc1
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // the builtins' raw 128-bit data
template <int D>
__device__ inline __amdgpu_buffer_rsrc_t part_o_rsrc(const DecodeArgs& a, size_t slot) {
    return __builtin_amdgcn_make_buffer_rsrc(a.part_o + slot * 16 * D, 0, 16 * D * 4, 0x00020000);
}
__device__ inline __amdgpu_buffer_rsrc_t part_l_rsrc(const DecodeArgs& a, size_t slot) {
    return __builtin_amdgcn_make_buffer_rsrc(a.part_l + slot * 16, 0, 16 * 4, 0x00020000);
}
__device__ inline int part_o_off(int db, int lane) { return (db * 64 + lane) * 16; }

// Position on the tile line: tile t of segment (b, g); lb valid rows and nt tiles in sequence b,
// pb the line position of sequence b's first segment.  All fields are wave-uniform.
struct LineCursor {
    int b, g, t, lb, nt;
    long long pb;
    __device__ inline int seg(int Hkv) const { return b * Hkv + g; }
    // move to the next segment of the line (the caller knows there is one)
    __device__ inline void next_segment(const DecodeArgs& a, const int* __restrict__ kv_len, int TR) {
        t = 0;
        if (++g == a.Hkv) {
            g = 0;
            pb += (long long)a.Hkv * nt;
            ++b;
            lb = valid_rows(a, kv_len, b);
            nt = (lb + TR - 1) / TR;
        }
    }
};

// A piece whose segment other waves share: merged at the end of the share.
struct PendingPiece {
    int seg, npieces, wf;
    long long ps;
};

template <int D, int TR, int NS, bool ROPE>
__global__ __launch_bounds__(64) void decode16_kernel(DecodeArgs a, const int* __restrict__ kv_len) {
    constexpr int KB = TR / 16, KS = D / 32, DB = D / 16, K2 = TR / 32;
    using TC = TileCopy<D, 1, TR>;
    constexpr int kCopies = 2 * TC::NU;          // copies per tile (K~ and V)
    static_assert(NS >= 2 && (NS - 1) * kCopies < 64, "copies in flight must fit vmcnt");
    __shared__ Dec16Lds<D, TR, NS> S;

    const int lane = threadIdx.x, c = lane & 15, g4 = lane >> 4;
    const int W = a.nsplit, w = (int)blockIdx.x;
    const int G = a.Hq / a.Hkv, ncol = G * a.n;

    // ---- this wave's share of the tile line ----
    // tiles of sequence b0 + lane and their inclusive prefix over the chunk of 64 sequences
    auto chunk_tiles = [&](int b0, int& tl, int& incl) {
        tl = b0 + lane < a.B ? (valid_rows(a, kv_len, b0 + lane) + TR - 1) / TR : 0;
        incl = wave_incl_scan(tl, lane);
    };
    int tl, incl;
    chunk_tiles(0, tl, incl);
    long long total = __builtin_amdgcn_readlane(incl, 63);
    for (int b0 = 64; b0 < a.B; b0 += 64) {
        int t2, i2;
        chunk_tiles(b0, t2, i2);
        total += __builtin_amdgcn_readlane(i2, 63);
    }
    total = uniform(total * a.Hkv);
    const long long lo = (long long)w * total / W, hi = (long long)(w + 1) * total / W;
    if (lo >= hi) return;
    const int nsh = (int)(hi - lo);               // tiles in the share
    LineCursor cur;
    cur.b = 0;
    cur.pb = 0;
    for (int b0 = 0;; b0 += 64) {
        if (b0 > 0) chunk_tiles(b0, tl, incl);
        const unsigned long long m =
            __builtin_amdgcn_ballot_w64(b0 + lane < a.B && cur.pb + (long long)a.Hkv * incl > lo);
        if (m) {
            const int f = __builtin_ctzll(m);
            cur.b = b0 + f;
            cur.pb += (long long)a.Hkv * (__builtin_amdgcn_readlane(incl, f) - __builtin_amdgcn_readlane(tl, f));
            break;
        }
        cur.pb += (long long)a.Hkv * __builtin_amdgcn_readlane(incl, 63);
    }
    cur.b = uniform(cur.b);
    cur.pb = uniform(cur.pb);
    cur.lb = valid_rows(a, kv_len, cur.b);
    cur.nt = (cur.lb + TR - 1) / TR;
    cur.g = (int)((lo - cur.pb) / cur.nt);
    cur.t = (int)((lo - cur.pb) % cur.nt);

    // ---- one copy stream over the whole share, NS - 1 tiles ahead of the computation ----
    const unsigned lk = lds_addr(&S.k[0][0]), lv = lds_addr(&S.v[0][0]);
    TC tc;
    tc.init(0, lane);
    LineCursor icur = cur;                        // the next tile to fetch
    auto issue_next = [&](int i) {                // share tile i, at icur
        const size_t hoff = (size_t)icur.seg(a.Hkv) * a.Tc * D;
        const unsigned hbytes = (unsigned)icur.lb * (unsigned)(D * 2);
        const i32x4 rk = buffer_rsrc(reinterpret_cast<const bf16*>(a.kc) + hoff, hbytes);
        const i32x4 rv = buffer_rsrc(reinterpret_cast<const bf16*>(a.vc) + hoff, hbytes);
        const unsigned row0 = (unsigned)(icur.t * TR) * (unsigned)(D * 2);
        const unsigned so = (unsigned)(i % NS) * TC::kBytes;
        tc.copy(rk, row0, lk + so, 0);
        tc.copy(rv, row0, lv + so, 0);
        if (i + 1 < nsh && ++icur.t == icur.nt) icur.next_segment(a, kv_len, TR);
    };
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
        if (i < nsh) issue_next(i);

    int roff[KB][KS], voff[K2][2][DB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) roff[kb][ks] = Swz<D>::at(16 * kb + c, 32 * ks + 8 * g4);
#pragma unroll
    for (int k2 = 0; k2 < K2; ++k2)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                voff[k2][h][db] = Swz<D>::at(32 * k2 + 16 * h + 4 * g4 + (c >> 2), 16 * db + 4 * (c & 3));
    const float c2 = a.scale * kLog2e;
    const float* __restrict__ cs = a.rope_cs;
    // this lane's query column: head g G + hh, token ti (columns past G n repeat column 0 and are
    // never stored)
    const int cc = c < ncol ? c : 0;
    const int hh = cc / a.n, ti = cc % a.n;
    auto out_row = [&](int b, int g) { return ((size_t)b * a.Hq + g * G + hh) * a.n + ti; };

    PendingPiece pend[2];
    int npend = 0;
    for (int i = 0;;) {
        // ---- piece: tiles [cur.t, t1) of segment (cur.b, cur.g) ----
        const int t1 = min(cur.nt, cur.t + (nsh - i));
        const int seg = cur.seg(a.Hkv);
        const int lb = cur.lb, k1 = min(t1 * TR, lb);
        const int pos = lb - a.n + ti;
        bf16x8 qhi[KS], qlo[KS];
        q_operands16<D, ROPE>(reinterpret_cast<const bf16*>(a.q) + out_row(cur.b, cur.g) * D, cs, pos, g4, qhi, qlo);
        // The compiler waits for these loads with vmcnt(0) (it does not count the copies): pin the
        // operands here so that the wait comes before the next copy is issued, not after it.
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qhi[ks]), "+v"(qlo[ks]));

        f32x4 oacc[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = f32x4{};
        float m_run = -INFINITY, l_run = 0.f;

        for (int t = cur.t; t < t1; ++t, ++i) {
            wait_tiles<kCopies, NS - 2>(nsh - 1 - i);
            if (i + NS - 1 < nsh) issue_next(i + NS - 1);   // its stage was last read in step i - 1
            const int buf = i % NS;
            const int j0 = t * TR;
            const bf16* Ks = S.k[buf];
            const bf16* Vs = S.v[buf];
            bf16x8 kf[KB][KS];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) kf[kb][ks] = *reinterpret_cast<const bf16x8*>(Ks + roff[kb][ks]);
            f32x4 sc[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sc[kb] = mma16(kf[kb][0], qhi[0], f32x4{});
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sc[kb] = mma16(kf[kb][0], qlo[0], sc[kb]);
#pragma unroll
            for (int ks = 1; ks < KS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) sc[kb] = mma16(kf[kb][ks], qhi[ks], sc[kb]);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) sc[kb] = mma16(kf[kb][ks], qlo[ks], sc[kb]);
            }
            bf16x8 vf[K2][DB];
#pragma unroll
            for (int k2 = 0; k2 < K2; ++k2)
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    vf[k2][db] = __builtin_shufflevector(tr_read(Vs + voff[k2][0][db]), tr_read(Vs + voff[k2][1][db]),
                                                         0, 1, 2, 3, 4, 5, 6, 7);
            // keys past the piece or after this column's token are invisible (S = -inf for the
            // max, P = 0)
            const bool edge = j0 + TR > k1 || j0 + TR - 1 > lb - a.n;
            unsigned vis = ~0u;                         // bit 4 kb + e: key 16 kb + 4 g + e visible
            if (edge) {
                vis = 0;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = j0 + 16 * kb + 4 * g4 + e;
                        if (j < k1 && j <= pos) vis |= 1u << (4 * kb + e);
                        else sc[kb][e] = -INFINITY;
                    }
            }
            float mx = sc[0][0];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sc[kb][e]);
            mx = col_max(mx) * c2;
            if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescale) != 0) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
                m_run = m_new;
            }
            float ls = 0.f;
#pragma unroll
            for (int k2 = 0; k2 < K2; ++k2) {
                float p[8];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int kb = 2 * k2 + h;
                        p[4 * h + e] = (vis >> (4 * kb + e)) & 1
                                           ? __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][e], c2, -m_run)) : 0.f;
                        ls += p[4 * h + e];
                    }
                const bf16x8 pb = cvt8(p);
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db] = mma16(vf[k2][db], pb, oacc[db]);
            }
            l_run += ls;
        }

        // ---- the piece's result: final when the piece is its whole segment, else a partial ----
        const float l_tot = col_sum(l_run);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const float L = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
        const long long ps = cur.pb + (long long)cur.g * cur.nt;    // the segment on the line
        const int wf = wave_of(ps, total, W), wl = wave_of(ps + cur.nt - 1, total, W);
        const int npieces = total >= W ? wl - wf + 1 : cur.nt;     // waves holding part of it
        if (npieces == 1) {
            if (c < ncol) {
                const size_t orow = out_row(cur.b, cur.g);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const float y[4] = {oacc[db][0] * inv, oacc[db][1] * inv, oacc[db][2] * inv, oacc[db][3] * inv};
                    *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(a.o) + orow * D + 16 * db + 4 * g4) = cvt4(y);
                }
                if (g4 == 0) a.lse[orow] = L;
            }
        } else {
            const size_t slot = (size_t)w + seg;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const f32x4 y = oacc[db] * inv;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y), part_o_rsrc<D>(a, slot),
                                                       part_o_off(db, lane), 0, kDeviceScope);
            }
            if (g4 == 0)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(L), part_l_rsrc(a, slot), 4 * c, 0, kDeviceScope);
            // only the first and the last piece of a share can share their segment with others
            const PendingPiece pp{seg, npieces, wf, ps};
            if (npend == 0) pend[0] = pp;
            else pend[1] = pp;
            ++npend;
        }
        if (i >= nsh) break;
        cur.next_segment(a, kv_len, TR);
    }

    // ---- pieces of shared segments: count the arrival; the last one merges ----
    // Ordering across XCDs (whose L2 caches are not coherent with each other), with a relaxed
    // counter: (1) the pieces were stored with sc1 (agent scope), which writes through this XCD's
    // L2 to the memory side; (2) vmcnt(0) below waits until the memory side has acknowledged
    // those stores; (3) only then is the counter raised, and an agent-scope atomic is performed at
    // the memory side, after every earlier piece's own (1)-(2); (4) the wave that sees npieces - 1
    // issues its loads after comparing that value (the empty asm keeps the compiler from hoisting
    // them), and they are sc1 loads, which do not hit lines this XCD's L2 may hold from before.
    // This is the agent-scope release / acquire of this family with the L2 write-back and
    // invalidate replaced by the per-access sc1 policy on the lines that cross XCDs.
    wait_vmcnt<0>();
    int arrived[2] = {0, 0};                     // both counts raised before either is looked at
    if (lane == 0) {
        if (npend > 0) arrived[0] = __hip_atomic_fetch_add(a.ctr + pend[0].seg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (npend > 1) arrived[1] = __hip_atomic_fetch_add(a.ctr + pend[1].seg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    arrived[0] = uniform(arrived[0]);            // lane 0's values
    arrived[1] = uniform(arrived[1]);
    for (int k = 0; k < npend; ++k) {
        const PendingPiece pp = k == 0 ? pend[0] : pend[1];
        if ((k == 0 ? arrived[0] : arrived[1]) != pp.npieces - 1) continue;
        asm volatile("" ::: "memory");           // the loads below stay after the count
        // the waves holding the pieces, in line order: wf .. wf + npieces - 1 when no share is
        // empty, else one wave per tile
        const bool dense = total >= W;
        auto piece_wave = [&](int q) { return dense ? pp.wf + q : wave_of(pp.ps + q, total, W); };
        // running log-sum-exp over batches of kMergeBatch pieces, every load of a batch issued
        // before any is used (a batch past the last piece re-reads it with weight 0)
        constexpr int kMergeBatch = decode_merge_batch(D);
        float mx = -INFINITY, sum = 0.f;
        f32x4 acc[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = f32x4{};
        for (int q0 = 0; q0 < pp.npieces; q0 += kMergeBatch) {
            float lq[kMergeBatch];
            f32x4 ov[kMergeBatch][DB];
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {
                const size_t sl = (size_t)piece_wave(min(q0 + u, pp.npieces - 1)) + pp.seg;
                lq[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(part_l_rsrc(a, sl), 4 * c, 0, kDeviceScope));
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    ov[u][db] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                              part_o_rsrc<D>(a, sl), part_o_off(db, lane), 0, kDeviceScope));
            }
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u)
                if (q0 + u >= pp.npieces) lq[u] = -INFINITY;
            float bm = lq[0];
#pragma unroll
            for (int u = 1; u < kMergeBatch; ++u) bm = fmaxf(bm, lq[u]);
            const float m_new = fmaxf(mx, bm);
            if (m_new == -INFINITY) continue;          // no piece so far saw a key of this column
            const float sc = mx == -INFINITY ? 0.f : __expf(mx - m_new);
            sum *= sc;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] *= sc;
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {
                const float wt = lq[u] == -INFINITY ? 0.f : __expf(lq[u] - m_new);
                sum += wt;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db] += wt * ov[u][db];
            }
            mx = m_new;
        }
        if (c < ncol) {
            const size_t orow = out_row(pp.seg / a.Hkv, pp.seg % a.Hkv);
            const float is = 1.f / sum;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const float y[4] = {acc[db][0] * is, acc[db][1] * is, acc[db][2] * is, acc[db][3] * is};
                *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(a.o) + orow * D + 16 * db + 4 * g4) = cvt4(y);
            }
            if (g4 == 0) a.lse[orow] = mx + __logf(sum);
        }
        if (lane == 0) __hip_atomic_store(a.ctr + pp.seg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace

template <int D>
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    const unsigned nsplit_blocks = (unsigned)(a.B * a.Hkv * a.nsplit);
    hipLaunchKernelGGL((decode_split_kernel<D>), dim3(nsplit_blocks), dim3(64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned merge_blocks = (unsigned)(a.B * a.Hkv * (a.Hq / a.Hkv) * a.n);
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(merge_blocks), dim3(64), 0, stream, a);
    return hipGetLastError();
}

template <int D>
int decode16_slots() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&decode16_kernel<D, decode_tile_rows(D), kDecodeStages, true>), 64, 0) !=
        hipSuccess)
        return 0;
    const int v = std::max(1, cus * per_cu);
    if (dev < kMaxDevices) cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

template <int D>
hipError_t launch_decode16(const DecodeArgs& a, hipStream_t stream) {
    if (a.rope_cs)
        hipLaunchKernelGGL((decode16_kernel<D, decode_tile_rows(D), kDecodeStages, true>), dim3((unsigned)a.nsplit), dim3(64),
                           0, stream, a, a.kv_len);
    else
        hipLaunchKernelGGL((decode16_kernel<D, decode_tile_rows(D), kDecodeStages, false>), dim3((unsigned)a.nsplit),
                           dim3(64), 0, stream, a, a.kv_len);
    return hipGetLastError();
}

template int decode16_slots<128>();
template int decode16_slots<64>();
template int decode16_slots<32>();
template hipError_t launch_decode16<128>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode16<64>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode16<32>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode<64>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode<32>(const DecodeArgs&, hipStream_t);

}  // namespace ne
