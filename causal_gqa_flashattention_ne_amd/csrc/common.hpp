// common.hpp -- device helpers shared by the gfx950 attention kernels.
//
// Matrix-core convention used everywhere (verified lane layouts of the 32x32 MFMA family):
//   A (32 x K): row i of the tile lives in lane i + 32*h, where h = lane / 32 picks which half of
//               each K chunk the lane supplies;
//   B (K x 32): column j lives in lane j + 32*h;
//   C (32 x 32, 16 fp32 registers per lane): element (i, j) lives in lane j + 32*((i/4)%2),
//               register (i%4) + 4*(i/8).  Equivalently, register r of lane (j, h) holds row
//               8*(r/4) + 4*h + (r%4) of column j.
// bf16: v_mfma_f32_32x32x16_bf16, each lane supplies 8 consecutive K values per instruction.
// fp32: v_mfma_f32_32x32x2_f32, each lane supplies 1 K value per instruction.
// The K dimension of a product is a sum, so each kernel may assign K indices to (chunk, half,
// item) slots in any order as long as both operands use the same assignment.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ne {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Per-element-type constants of the 32x32 MFMA path.
template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
    static constexpr int KW = 8;           // K values one lane supplies per instruction
    typedef bf16x8 op;                     // operand register type
    __device__ static inline f32x16 mma(op a, op b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    static constexpr int KW = 1;
    typedef float op;
    __device__ static inline f32x16 mma(op a, op b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE on gfx950

// Row of the 32x32 accumulator tile held by register r of a lane in half h.
__device__ __host__ constexpr inline int acc_row(int r, int h) { return 8 * (r / 4) + 4 * h + (r % 4); }

__device__ inline float wave_xor32(float v) { return __shfl_xor(v, 32, 64); }

// 16-byte global load/store of VEC = 16/sizeof(T) elements.
template <typename T> struct Vec16 { static constexpr int N = 16 / sizeof(T); T v[N]; };

template <typename T>
__device__ inline void load16(const T* p, float* out) {
    if constexpr (sizeof(T) == 4) {
        f32x4 x = *reinterpret_cast<const f32x4*>(p);
        out[0] = x[0]; out[1] = x[1]; out[2] = x[2]; out[3] = x[3];
    } else {
        bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = (float)x[i];
    }
}

template <typename T>
__device__ inline void store16(T* p, const float* in) {
    if constexpr (sizeof(T) == 4) {
        f32x4 x = {in[0], in[1], in[2], in[3]};
        *reinterpret_cast<f32x4*>(p) = x;
    } else {
        bf16x8 x;
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (bf16)in[i];
        *reinterpret_cast<bf16x8*>(p) = x;
    }
}

// Store 4 consecutive elements (8 bytes for bf16, 16 for fp32).
template <typename T>
__device__ inline void store4(T* p, float a, float b, float c, float d) {
    if constexpr (sizeof(T) == 4) {
        f32x4 x = {a, b, c, d};
        *reinterpret_cast<f32x4*>(p) = x;
    } else {
        bf16x4 x = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
        *reinterpret_cast<bf16x4*>(p) = x;
    }
}

// Rotate the pairs of n consecutive values x[0..n) that start at an even column d0 of row pos,
// using the float32 (cos, sin) table cs[pos][D/2].  inverse applies R^T.
__device__ inline void rope_rotate(float* x, int n, const float* cs, int D, int pos, int d0,
                                   bool inverse) {
    const f32x2* row = reinterpret_cast<const f32x2*>(cs + (size_t)pos * D) + d0 / 2;
#pragma unroll
    for (int p = 0; p < n / 2; ++p) {
        f32x2 t = row[p];
        float c = t[0], s = inverse ? -t[1] : t[1];
        float x0 = x[2 * p], x1 = x[2 * p + 1];
        x[2 * p] = x0 * c - x1 * s;
        x[2 * p + 1] = x0 * s + x1 * c;
    }
}

// head_dim slot of (chunk c, half h, item e) for products whose K dimension is head_dim:
// bf16: 8 consecutive values per lane (d = 16c + 8h + e); fp32: lane half h owns the contiguous
// half [h*D/2, h*D/2 + D/2) (d = c + h*D/2).  Both keep RoPE pairs inside one lane.
template <typename T, int D>
__device__ constexpr inline int dslot(int c, int h, int e) {
    if constexpr (Mfma<T>::KW == 8) return 16 * c + 8 * h + e;
    else return c + h * (D / 2);
}

// out[c*KW + e] = (R_pos x)[dslot(c, half, e)] for the row x = rowp[0..D) (zeros when !valid);
// only this lane half's slots are read.  Register indices stay compile-time constants.
template <typename T, int D>
__device__ inline void load_row_slots(const T* rowp, const float* cs, int pos, int half, bool valid,
                                      float* out) {
    constexpr int KW = Mfma<T>::KW;
    constexpr int NSL = D / 2;                       // slots per lane
    if (!valid) {
#pragma unroll
        for (int i = 0; i < NSL; ++i) out[i] = 0.f;
        return;
    }
    if constexpr (KW == 8) {
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            const int d0 = 16 * c + 8 * half;
            load16<T>(rowp + d0, out + 8 * c);
            if (cs) rope_rotate(out + 8 * c, 8, cs, D, pos, d0, false);
        }
    } else {
        const int d0 = half * (D / 2);
#pragma unroll
        for (int j = 0; j < D / 2; j += 4) load16<T>(rowp + d0 + j, out + j);
        if (cs) rope_rotate(out, D / 2, cs, D, pos, d0, false);
    }
}

template <typename T, int NSL>
__device__ inline void slots_to_ops(const float* x, typename Mfma<T>::op* ops) {
    constexpr int KW = Mfma<T>::KW;
#pragma unroll
    for (int c = 0; c < NSL / KW; ++c) {
        if constexpr (KW == 8) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ops[c][e] = (bf16)x[8 * c + e];
        } else {
            ops[c] = x[c];
        }
    }
}

}  // namespace ne
