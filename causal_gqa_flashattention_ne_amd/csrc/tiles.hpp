// tiles.hpp -- LDS tile staging and operand helpers shared by the bf16 kernels (gfx950).
//
// Tiles of 64 rows x D (bf16, row-major, row stride D + 8 in LDS) are loaded by a 256-thread
// workgroup, 16 bytes per thread and chunk, with row indices clamped into the sequence so the
// loads are unconditional and nothing waits on them before the tile is stored.  The first tile
// of a set may be rotated by RoPE on its way to LDS (queries or keys: the rotation is applied in
// float32 and rounded to bf16 once), optionally split into a bf16 high part and a bf16 remainder.
#pragma once

#include "common.hpp"

namespace ne {

constexpr int kTileRows = 64;        // rows of one staged tile
constexpr int kBlockThreads = 256;   // threads of every bf16 attention workgroup

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

// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32 packs two per instruction)
__device__ inline bf16x2 cvt2(float x, float y) { return __builtin_convertvector(f32x2{x, y}, bf16x2); }
__device__ inline bf16x4 cvt4(const float* x) {
    return __builtin_shufflevector(cvt2(x[0], x[1]), cvt2(x[2], x[3]), 0, 1, 2, 3);
}
__device__ inline bf16x8 cvt8(const float* x) {
    return __builtin_shufflevector(cvt4(x), cvt4(x + 4), 0, 1, 2, 3, 4, 5, 6, 7);
}

// y = x - bf16(x) for 8 values whose bf16 rounding is hi: the remainder, itself rounded to bf16.
__device__ inline bf16x8 remainder8(const float* x, bf16x8 hi) {
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = x[e] - (float)hi[e];
    return cvt8(r);
}

// RoPE on 8 consecutive values (4 adjacent pairs) with their table entries (cos, sin) x 4.
__device__ inline void rot8(bf16x8 in, const f32x4* cs, float* y) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float c = cs[p >> 1][2 * (p & 1)], s = cs[p >> 1][2 * (p & 1) + 1];
        const float x0 = (float)in[2 * p], x1 = (float)in[2 * p + 1];
        y[2 * p] = x0 * c - x1 * s;
        y[2 * p + 1] = x0 * s + x1 * c;
    }
}

// Prefetch of NT tiles of 64 rows x D.  Tile 0 may be rotated on the store to LDS (positions of
// its rows come with the load); with SPLIT it is stored as two tiles, bf16(R x) to dst[0] and the
// bf16 remainder R x - bf16(R x) to dst[NT].
template <int D, int NT, bool SPLIT>
struct TileLoad {
    static constexpr int NU = (kTileRows * D / 8) / kBlockThreads;
    static constexpr int RS = D + 8;
    static_assert((kTileRows * D / 8) % kBlockThreads == 0, "tile chunks must cover the workgroup evenly");
    bf16x8 x[NT][NU];
    f32x4 cs[NU][2];

    // Rows r0 + (0..63) of each src[t] (row-major, D per row), clamped to r0 + last; the RoPE
    // table rows are pos0 + the same row offsets.
    __device__ inline void load(const bf16* const* src, const float* cs_tab, int pos0, int last, int tid) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int ch = tid + u * kBlockThreads;
            const int r = min(ch / (D / 8), last), d0 = (ch % (D / 8)) * 8;
#pragma unroll
            for (int t = 0; t < NT; ++t) x[t][u] = *reinterpret_cast<const bf16x8*>(src[t] + r * D + d0);
            if (cs_tab) {
                const f32x4* c = reinterpret_cast<const f32x4*>(cs_tab + (size_t)(pos0 + r) * D + d0);
                cs[u][0] = c[0];
                cs[u][1] = c[1];
            }
        }
    }

    __device__ inline void store(bf16* const* dst, bool rope, int tid) const {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int ch = tid + u * kBlockThreads;
            const int o = (ch / (D / 8)) * RS + (ch % (D / 8)) * 8;
            if (rope) {
                float y[8];
                rot8(x[0][u], cs[u], y);
                const bf16x8 hi = cvt8(y);
                *reinterpret_cast<bf16x8*>(dst[0] + o) = hi;
                if (SPLIT) *reinterpret_cast<bf16x8*>(dst[NT] + o) = remainder8(y, hi);
            } else {
                *reinterpret_cast<bf16x8*>(dst[0] + o) = x[0][u];
                if (SPLIT) *reinterpret_cast<bf16x8*>(dst[NT] + o) = bf16x8{};
            }
#pragma unroll
            for (int t = 1; t < NT; ++t) *reinterpret_cast<bf16x8*>(dst[t] + o) = x[t][u];
        }
    }
};

// (cos, sin) of the two RoPE pairs behind each 4-value group of a 32 x 32 accumulator column
// held by this lane (row pos of the table; d = 32 dt + acc_row(4 rq, half) + 0..3): one 16-byte
// load per group, all issued before any is used.
template <int D>
__device__ inline void load_acc_cs(const float* cs, int pos, int half, f32x4 (&c)[D / 32][4]) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
            c[dt][rq] = *reinterpret_cast<const f32x4*>(cs + (size_t)pos * D + 32 * dt + acc_row(4 * rq, half));
}

// x[0..3] = two adjacent RoPE pairs; apply R^T with their table entries c = (cos, sin, cos, sin).
__device__ inline void unrotate4(float* x, f32x4 c) {
    const float x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];
    x[0] = x0 * c[0] + x1 * c[1];
    x[1] = x1 * c[0] - x0 * c[1];
    x[2] = x2 * c[2] + x3 * c[3];
    x[3] = x3 * c[2] - x2 * c[3];
}

// This lane's slots of the row x (head_dim split as the bf16 MFMA operands: chunk c holds
// d = 16c + 8*half + 0..7), rotated to R_pos x in float32 and returned as bf16 hi + lo operand
// pairs (lo == nullptr: hi only).
template <int D>
__device__ inline void row_operands(const bf16* rowp, const float* cs, int pos, int half, bf16x8* hi,
                                    bf16x8* lo) {
    float x[D / 2];
    load_row_slots<bf16, D>(rowp, cs, pos, half, true, x);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        hi[c] = cvt8(x + 8 * c);
        if (lo) lo[c] = remainder8(x + 8 * c, hi[c]);
    }
}

}  // namespace ne
