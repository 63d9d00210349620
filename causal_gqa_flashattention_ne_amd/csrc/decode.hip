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

template hipError_t launch_decode<64>(const DecodeArgs&, hipStream_t);
template hipError_t launch_decode<32>(const DecodeArgs&, hipStream_t);

}  // namespace ne
