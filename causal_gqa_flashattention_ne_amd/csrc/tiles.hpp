// tiles.hpp -- LDS tile staging and operand helpers shared by the bf16 kernels (gfx950).
//
// Tiles of 64 rows x D bf16 go from global memory straight into LDS (buffer_load_dwordx4 ... lds:
// no registers, no LDS store instructions) through LDS stages: kStages (three, tiles two steps
// ahead of their use) in decode, two (one step ahead) in the forward and backward.
// LDS tiles are unpadded and XOR-swizzled in 16-byte chunks (Swz) so that row reads
// (ds_read_b128) and transposed reads (ds_read_b64_tr_b16) stay conflict-free.  A step opens with
// an explicit wait for this wave's copies of the current tile and one barrier without a fence.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace ne {

constexpr int kTileRows = 64;                   // rows of one staged tile
constexpr int kBlockThreads = 256;              // threads of every bf16 attention workgroup
constexpr int kBlockWaves = kBlockThreads / 64;
constexpr int kStages = 3;                      // decode's LDS stages: a tile is fetched two steps before its use

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: inside each 16-lane group, lane i receives element (i % 4) of the 8-byte
// rows read by lanes (i / 4) + 4k, k = 0..3.
__device__ inline bf16x4 tr_read(const bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
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

// Unpadded LDS tile of 64 rows x D bf16.  The 16-byte chunk c of row r is stored at chunk
// position c ^ f(r): any 8 consecutive rows then put a given column chunk in 8 different bank
// groups, and the 4-row x 32-byte footprint of a transposed read is spread as well.
template <int D>
struct Swz {
    static constexpr int CPR = D / 8;                                  // chunks per row
    __device__ static inline int f(int r) { return (r * CPR / 8) & (CPR - 1); }
    // element offset of (row r, column col); a read of up to 8 elements starting at col must not
    // cross a chunk boundary
    __device__ static inline int at(int r, int col) { return r * D + (((col >> 3) ^ f(r)) << 3) + (col & 7); }
};

// A-operand fragment (32 rows m x 16 k) of the 32x32x16 MFMA taken from a swizzled LDS tile
// X[k][m] (so A[m][k] = X[k][m]): lane (m = l%32, half h) receives X[k][m] for the k rows
// kb0 + 0..3 and kb1 + 0..3 (kb0 / kb1 chosen per half by the caller).
template <int D>
__device__ inline bf16x8 tr_frag_swz(const bf16* X, int m0, int kb0, int kb1, int lane) {
    const int s = lane & 15;
    const int m = m0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
    const bf16x4 lo = tr_read(X + Swz<D>::at(kb0 + (s >> 2), m));
    const bf16x4 hi = tr_read(X + Swz<D>::at(kb1 + (s >> 2), m));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The same fragment with the address split into a per-lane base and a row block known at compile
// time.  The swizzle f(r) depends on r mod 8 only, so moving 8 rows down moves every chunk by 8 * D
// elements: tr_base gives the lane's element offset for the columns m0.. at rows 4 * half + s / 4,
// and tr_frag_at reads rows r0 + that and r0 + 8 + that (r0 a multiple of 8), the same values as
// tr_frag_swz(X, m0, r0 + 4 * half, r0 + 8 + 4 * half, lane) with only an immediate offset added.
template <int D>
__device__ inline int tr_base(int m0, int lane) {
    const int s = lane & 15;
    const int m = m0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
    return Swz<D>::at(4 * (lane >> 5) + (s >> 2), m);
}
template <int D>
__device__ inline bf16x8 tr_frag_at(const bf16* X, int base, int r0) {
    const bf16x4 lo = tr_read(X + base + r0 * D);
    const bf16x4 hi = tr_read(X + base + (r0 + 8) * D);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maxima: no wait on them).  The empty asm
// keeps the compiler from moving the LDS reads of the tile waited for above the wait.
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// Barrier between the waves of the workgroup without a memory fence (the fence of
// __syncthreads would also wait for the copies still in flight).  The empty asm keeps the
// compiler from moving LDS accesses across it, and the lgkmcnt(0) wait before it makes every LDS
// read this wave issued complete before any wave passes: the stage those reads came from is
// refilled by copies issued right after the barrier, and the compiler may otherwise place a
// read's consumer, and so the wait for it, after the barrier (vmcnt and expcnt not waited for).
__device__ inline void step_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Raw buffer descriptor (gfx9 family): base address, stride 0, size in bytes (reads at or past it
// return zeros), 32-bit data format.  All fields are wave-uniform.
__device__ inline i32x4 buffer_rsrc(const void* base, unsigned bytes) {
    const unsigned long long adr = reinterpret_cast<unsigned long long>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)adr);
    r[1] = __builtin_amdgcn_readfirstlane((int)((unsigned)(adr >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// LDS byte address of a __shared__ object (taken once per block; per-step addresses are offsets
// from it in scalar registers).
__device__ inline unsigned lds_addr(const void* p) { return (unsigned)(size_t)(lds_void*)p; }

// One 16-byte-per-lane copy from a buffer into LDS (buffer_load_dwordx4 ... lds): lane i reads at
// byte voff + soff of the buffer and writes bytes 16i..16i+15 after the wave-uniform LDS byte
// address lds.  Written as assembly so that the compiler does not track these copies: its
// automatic wait before a transposed LDS read would otherwise also wait for the copies of the
// tiles two steps ahead.  Every wait on them is the explicit wait_vmcnt at the top of a step; the
// per-lane operands a kernel loads before its step loop are waited for (vmcnt(0)) before the loop
// starts, so no other vector-memory load is in flight in it.
//
// Range.  soff is folded into the descriptor (base moved by soff, size cut by soff, never below
// zero) and the instruction's own scalar offset is 0: the hardware's range check then covers the
// whole offset voff + soff, so a read at or past the buffer's size writes zeros to LDS and never
// touches memory past the buffer, however the check treats a scalar offset.
//
// Wait states.  The descriptor words and M0 are scalar registers that a VALU instruction
// (v_readfirstlane) may have written just before this block, and the gfx9 family (gfx950
// included) requires 5 wait states between a VALU write of an SGPR and a vector-memory
// instruction that reads it; M0 written by a scalar move needs 1 before an LDS-direct load.  The
// compiler inserts these waits for the loads it emits itself but cannot see inside this
// assembly, so the block opens with s_nop 4 (5 wait states), which covers both whatever the
// compiler placed in front of it.
__device__ inline void copy16_to_lds(i32x4 rsrc, unsigned voff, unsigned soff, unsigned lds) {
    // soff and lds are wave-uniform; readfirstlane puts them in scalar registers even where the
    // compiler kept a uniform value in a vector register
    const unsigned so = __builtin_amdgcn_readfirstlane(soff), m0 = __builtin_amdgcn_readfirstlane(lds);
    const unsigned lo = (unsigned)rsrc[0] + so;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)lo);
    r[1] = __builtin_amdgcn_readfirstlane(rsrc[1] + (int)(lo < so));   // carry into address bits 32..47
    r[2] = __builtin_amdgcn_readfirstlane((unsigned)rsrc[2] > so ? (int)((unsigned)rsrc[2] - so) : 0);
    r[3] = rsrc[3];
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(voff), "s"(r), "{m0}"(m0)
                 : "memory");
}

// Copies of ROWS-row x D bf16 tiles of a row-major matrix into swizzled LDS tiles by the NW waves
// of a workgroup.  Each wave issues ROWS * D / (512 * NW) copies of 64 lanes x 16 bytes; the LDS
// side of one copy is a contiguous 1 KiB slice, so the swizzle is applied by choosing which chunk
// each lane fetches.  The per-lane byte offsets within a tile do not depend on the tile; rows
// past the end of the buffer read as zeros.
template <int D, int NW = kBlockWaves, int ROWS = kTileRows>
struct TileCopy {
    static constexpr int CPR = D / 8, NU = ROWS * CPR / (64 * NW);
    static_assert(NU >= 1 && (ROWS * CPR) % (64 * NW) == 0, "tile chunks must cover the waves evenly");
    static constexpr unsigned kBytes = ROWS * D * 2;        // one LDS tile
    unsigned voff[NU];
    __device__ inline void init(int w, int lane) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int idx = (u * NW + w) * 64 + lane;
            const int r = idx / CPR, p = idx % CPR;
            voff[u] = (unsigned)(r * D + ((p ^ Swz<D>::f(r)) << 3)) * 2u;
        }
    }
    // the tile whose first row starts at byte row0 of the buffer, into the LDS tile at byte lds
    __device__ inline void copy(i32x4 rsrc, unsigned row0, unsigned lds, int w) const {
#pragma unroll
        for (int u = 0; u < NU; ++u)
            copy16_to_lds(rsrc, voff[u], row0, lds + (unsigned)(u * NW + w) * 1024u);
    }
};

// (cos, sin) of the two RoPE pairs behind each 4-value group of a 32 x 32 accumulator column
// held by this lane (row pos of the table; d = 32 dt + acc_row(4 rq, half) + 0..3): one 16-byte
// load per group, all issued before any is used.
// The same entries from the table re-ordered by rope_qcs_index: group (dt, rq) of lane half h
// holds pairs 16 dt + 4 rq + 2 h + {0, 1}, the piece (chunk 2 dt + rq / 2, p = h, half rq % 2), so
// that the 32 lanes of a lane half read 512 contiguous bytes per load.
template <int D>
__device__ inline void load_acc_qcs(const float* qcs, int pos, int half, f32x4 (&c)[D / 32][4]) {
    const f32x4* q4 = reinterpret_cast<const f32x4*>(qcs);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) c[dt][rq] = q4[rope_qcs_index(pos, 2 * dt + rq / 2, half, rq % 2, D / 16)];
}

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
