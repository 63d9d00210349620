// proj.hip -- the query/key/value projection of an attention block on gfx950, with RoPE in the
// epilogue and the outputs written straight into the attention layout [B, H, T, D].
//
// The model's linear maps carry no bias (agentlenshq NanoEuler page, "핵심 아키텍처 및 설계"); RoPE
// rotates the queries and keys ("기술 사양").  Output feature f of token m is x[m] . w[f], the
// features packed as [query heads | key heads | value heads], head-major, d fastest.
//
// GEMM in "TN" form: x [M, C] and w [N, C] both run along C, so every MFMA operand fragment is a
// row read of an LDS tile (8 consecutive k per lane, no transposes).  The product is formed
// feature-major, Y^T = W X^T: a lane of a 32 x 32 x 16 MFMA result holds one token and, per group
// of four registers, four consecutive features, so each RoPE pair sits in one lane.  A workgroup
// (4 waves, 2 x 2) owns 128 features x 192 tokens; k advances 64 per step through two LDS stages
// filled by buffer loads straight into LDS (tiles.hpp), one step ahead; at 80 KiB two workgroups
// share a CU and overlap each other's waits.  192 tokens make the 116M model's projection
// (8192 tokens x 1280 features) 430 tiles, one round of two workgroups on every CU: 128-token
// tiles (640) needed a second round for the last quarter, which measured 9% slower; three or four
// stages, k = 32 steps and three workgroups per CU measured no faster.  Results go through padded
// LDS rows to 16-byte stores, each a run of 8 features of one (head, token) row.
//
// Placement: workgroup i runs on XCD i % 8.  Each XCD takes a contiguous range of tiles in
// token-major order (features fastest), so the feature tiles of one token tile run back to back
// on one XCD and read their x rows from its L2; w (2 MB at the 116M model) stays in every L2.
#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace ne {

namespace {

constexpr int kXcds = 8;
constexpr int kFeat = 128;                 // features per output tile
constexpr int kWT = 3;                     // 32-token MFMA tiles per wave along tokens
constexpr int kTok = 2 * 32 * kWT;         // tokens per output tile
constexpr int kK = 64;                     // k per step
constexpr int kStagesP = 2;               // 80 KiB of LDS: two workgroups per CU
constexpr int kCPR = kK / 8;               // 16-byte chunks per tile row

struct alignas(16) ProjLds {
    alignas(16) bf16 w[kStagesP][kFeat * kK];   // [feature][k], swizzled
    alignas(16) bf16 x[kStagesP][kTok * kK];    // [token][k], swizzled
};
// epilogue staging: [token][feature] bf16 rows padded by 8 elements (conflict-free 8-byte writes)
constexpr int kOutPitch = kFeat + 8;
static_assert(kTok * kOutPitch * 2 <= (int)sizeof(ProjLds), "output staging must fit in the stage buffers");
static_assert(2 * sizeof(ProjLds) <= 160 * 1024, "two workgroups per CU");

// Copies of ROWS x 64 bf16 tiles of a row-major matrix with a row pitch of `pitch` bytes into
// swizzled LDS tiles, by the 4 waves of a workgroup (the tile copy of tiles.hpp with a run-time
// row pitch).  The per-lane offsets within a tile are loop-invariant; rows past the end of the
// buffer read as zeros.
template <int ROWS>
struct PitchCopy {
    static constexpr int NU = ROWS * kCPR / (64 * kBlockWaves);
    static_assert(NU >= 1 && (ROWS * kCPR) % (64 * kBlockWaves) == 0, "tile chunks must cover the waves");
    unsigned voff[NU];
    __device__ inline void init(int w, int lane, unsigned pitch) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int idx = (u * kBlockWaves + w) * 64 + lane;
            const int r = idx / kCPR, slot = idx % kCPR;
            voff[u] = (unsigned)r * pitch + (unsigned)((slot ^ Swz<kK>::f(r)) << 4);
        }
    }
    __device__ inline void copy(i32x4 rsrc, unsigned origin, unsigned lds, int w) const {
#pragma unroll
        for (int u = 0; u < NU; ++u) copy16_to_lds(rsrc, voff[u], origin, lds + (unsigned)(u * kBlockWaves + w) * 1024u);
    }
};

// q = m / d and r = m - q d for 0 <= m < 2^31, d >= 1: a double-precision estimate (exact to
// within one) corrected once each way
__device__ inline void divmod(int m, int d, double inv_d, int& q, int& r) {
    q = (int)((double)m * inv_d);
    r = m - q * d;
    if (r < 0) --q, r += d;
    else if (r >= d) ++q, r -= d;
}

template <bool ROPE>
__global__ __launch_bounds__(kBlockThreads, 2) void proj_kernel(ProjArgs a) {
    using M = Mfma<bf16>;
    using CW = PitchCopy<kFeat>;
    using CX = PitchCopy<kTok>;
    constexpr int kCopies = CW::NU + CX::NU;       // copies per wave per step
    __shared__ ProjLds S;

    // ---- tile of this workgroup ----
    const int xcd = (int)blockIdx.x % kXcds, local = (int)blockIdx.x / kXcds;
    const int tile = xcd * a.per_xcd + local;
    if (local >= a.per_xcd || tile >= a.tiles_m * a.tiles_n) return;
    const int tm = tile / a.tiles_n, tn = tile % a.tiles_n;
    const int m0 = tm * kTok, n0 = tn * kFeat;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int wf = w >> 1, wt = w & 1;              // wave: features wf*64.., tokens wt*(32 kWT)..

    // D is a power of two (32, 64 or 128): head and d by shift and mask
    const int lgD = __builtin_ctz(a.D);
    const int nq = a.Hq << lgD, nqk = (a.Hq + a.Hkv) << lgD;
    const double invT = 1.0 / (double)a.T;
    const unsigned pitch = (unsigned)a.C * 2u;
    const i32x4 rw = buffer_rsrc(a.w, (unsigned)a.N * pitch);
    const i32x4 rx = buffer_rsrc(a.x, (unsigned)a.M * pitch);
    const unsigned lw = lds_addr(&S.w[0][0]), lx = lds_addr(&S.x[0][0]);
    CW cw;
    CX cx;
    cw.init(w, lane, pitch);
    cx.init(w, lane, pitch);
    const int nk = a.C / kK;
    auto issue = [&](int t) {
        const unsigned st = (unsigned)(t % kStagesP);
        cw.copy(rw, (unsigned)n0 * pitch + (unsigned)(t * kK * 2), lw + st * (unsigned)(kFeat * kK * 2), w);
        cx.copy(rx, (unsigned)m0 * pitch + (unsigned)(t * kK * 2), lx + st * (unsigned)(kTok * kK * 2), w);
    };
#pragma unroll
    for (int i = 0; i < kStagesP - 1; ++i)
        if (i < nk) issue(i);
    // every table entry this lane needs, loaded as one batch after the main loop (no copy is in
    // flight then) and pinned, so that the compiler waits once for all of them; held through the
    // loop they would cost 96 registers
    f32x4 cs[2][kWT][4];
    bool rot[2];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb) rot[fb] = ROPE && n0 + wf * 64 + fb * 32 < nqk;   // whole 32-blocks
    auto load_cs = [&]() {
#pragma unroll
        for (int tb = 0; tb < kWT; ++tb) {
            const int m = m0 + wt * 32 * kWT + tb * 32 + col;
            int bq, pos;
            divmod(m < a.M ? m : 0, a.T, invT, bq, pos);
#pragma unroll
            for (int fb = 0; fb < 2; ++fb)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int d = (n0 + wf * 64 + fb * 32 + acc_row(4 * rq, half)) & (a.D - 1);
                    cs[fb][tb][rq] = *reinterpret_cast<const f32x4*>(a.rope_cs + (size_t)pos * a.D + d);
                }
        }
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
            for (int tb = 0; tb < kWT; ++tb)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) asm volatile("" : "+v"(cs[fb][tb][rq]));
    };


    int ra[2][4], rb[kWT][4];                       // fragment offsets: [block][k chunk of 16]
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) ra[fb][kc] = Swz<kK>::at(wf * 64 + fb * 32 + col, 16 * kc + 8 * half);
#pragma unroll
        for (int tb = 0; tb < kWT; ++tb) rb[tb][kc] = Swz<kK>::at(wt * 32 * kWT + tb * 32 + col, 16 * kc + 8 * half);
    }
    f32x16 acc[2][kWT];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int tb = 0; tb < kWT; ++tb) acc[fb][tb] = f32x16{};

    for (int t = 0; t < nk; ++t) {
        // this wave's copies of tile t have landed when at most the later tiles' are in flight
        static_assert(kStagesP == 2 || kStagesP == 3, "wait counts below are for two or three stages");
        if constexpr (kStagesP == 3) {
            if (t + 1 < nk) wait_vmcnt<(kStagesP - 2) * kCopies>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        step_barrier();                             // every wave's copies of tile t have landed
        if (t + kStagesP - 1 < nk) issue(t + kStagesP - 1);   // its stage was last read in step t - 1
        const bf16* Ws = S.w[t % kStagesP];
        const bf16* Xs = S.x[t % kStagesP];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            bf16x8 af[2], bfr[kWT];
#pragma unroll
            for (int fb = 0; fb < 2; ++fb) af[fb] = *reinterpret_cast<const bf16x8*>(Ws + ra[fb][kc]);
#pragma unroll
            for (int tb = 0; tb < kWT; ++tb) bfr[tb] = *reinterpret_cast<const bf16x8*>(Xs + rb[tb][kc]);
#pragma unroll
            for (int fb = 0; fb < 2; ++fb)
#pragma unroll
                for (int tb = 0; tb < kWT; ++tb) acc[fb][tb] = M::mma(af[fb], bfr[tb], acc[fb][tb]);
        }
    }

    // ---- epilogue: RoPE on query and key features, bf16, staged through LDS ----
    if constexpr (ROPE) load_cs();
    __syncthreads();                                // every wave is done with the stage buffers
    bf16* out = reinterpret_cast<bf16*>(&S);
#pragma unroll
    for (int fb = 0; fb < 2; ++fb) {
#pragma unroll
        for (int tb = 0; tb < kWT; ++tb) {
            const int tok = wt * 32 * kWT + tb * 32 + col;   // row within the tile
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                float y[4] = {acc[fb][tb][4 * rq], acc[fb][tb][4 * rq + 1], acc[fb][tb][4 * rq + 2],
                              acc[fb][tb][4 * rq + 3]};
                const int fl = wf * 64 + fb * 32 + acc_row(4 * rq, half);   // feature within the tile
                if constexpr (ROPE) {
                    const f32x4 c = cs[fb][tb][rq];
                    const float y0 = y[0], y1 = y[1], y2 = y[2], y3 = y[3];
                    const float r0 = y0 * c[0] - y1 * c[1], r1 = y0 * c[1] + y1 * c[0];
                    const float r2 = y2 * c[2] - y3 * c[3], r3 = y2 * c[3] + y3 * c[2];
                    if (rot[fb]) y[0] = r0, y[1] = r1, y[2] = r2, y[3] = r3;
                }
                *reinterpret_cast<bf16x4*>(out + tok * kOutPitch + fl) = cvt4(y);
            }
        }
    }
    __syncthreads();
    // 16-byte runs: 8 features of one token, inside one head (D is a multiple of 8)
    constexpr int kRuns = kTok * kFeat / 8;
    for (int i = threadIdx.x; i < kRuns; i += kBlockThreads) {
        const int tok = i / (kFeat / 8), f8 = (i % (kFeat / 8)) * 8;
        const int m = m0 + tok, n = n0 + f8;
        if (m >= a.M || n >= a.N) continue;
        const bf16x8 val = *reinterpret_cast<const bf16x8*>(out + tok * kOutPitch + f8);
        int b, tpos;
        divmod(m, a.T, invT, b, tpos);
        bf16* dst;
        if (n < nq) {
            dst = reinterpret_cast<bf16*>(a.q) + ((((size_t)b * a.Hq + (n >> lgD)) * a.T + tpos) << lgD) + (n & (a.D - 1));
        } else if (n < nqk) {
            const int nn = n - nq;
            dst = reinterpret_cast<bf16*>(a.k) + ((((size_t)b * a.Hkv + (nn >> lgD)) * a.T + tpos) << lgD) + (nn & (a.D - 1));
        } else {
            const int nn = n - nqk;
            dst = reinterpret_cast<bf16*>(a.v) + ((((size_t)b * a.Hkv + (nn >> lgD)) * a.T + tpos) << lgD) + (nn & (a.D - 1));
        }
        *reinterpret_cast<bf16x8*>(dst) = val;
    }
}

}  // namespace

int proj_tile_tokens() { return kTok; }

hipError_t launch_proj(const ProjArgs& a, hipStream_t stream) {
    if (a.rope_cs) hipLaunchKernelGGL(proj_kernel<true>, dim3((unsigned)(kXcds * a.per_xcd)), dim3(kBlockThreads), 0, stream, a);
    else hipLaunchKernelGGL(proj_kernel<false>, dim3((unsigned)(kXcds * a.per_xcd)), dim3(kBlockThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ne
