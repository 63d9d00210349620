// kernels.hpp -- argument blocks and launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ne {

// The rotated queries' low part (a second bf16 term, q~ = hi + lo) is used for a 128-query block I
// of head (b, h) when the bound scale * D * aq128[I] * max_{j in the block's key tiles} ak64[j] on
// its scores exceeds kLoBound: aq128 = max |q| over the block's raw query rows, ak64 = max |k| over
// a 64-row tile of raw keys (both exact maxima of the inputs, so every kernel that recomputes them
// reaches the same decision).  |scale q~.k~| <= scale ||q|| ||k|| <= scale * D * max|q| * max|k|.
constexpr float kLoBound = 400.f;

struct FwdArgs {
    const void* q;
    const void* k;          // bf16 kernel: keys already rotated (R k) when rope_cs is set
    const void* v;
    void* o;
    float* lse;
    const float* rope_cs;   // [T][D/2][2] or nullptr (bf16 kernel: used for the queries only)
    int B, Hq, Hkv, T;
    float scale;
    void* qrot;             // bf16 kernel, training variant: the rotated queries scaled by scale *
    void* qrot_lo;          // log2(e), hi and lo bf16 parts as the backward reads them ([B, Hq, T, D]
                            // each; lo only for the blocks that use it), or nullptr
    const float* ak;        // bf16 kernel: [B, Hkv, ceil(T/64)] max |k| per key tile
    int* lof;               // bf16 kernel, training variant: [B, Hq, ceil(T/128)] low-part flags
    const float* qcs;       // bf16 kernel with RoPE: the table's rows in the query-operand order
                            // (rope_qcs_index), written by key_rot_kernel
};

// The RoPE table re-ordered for the bf16 forward's query rotation: the lane holding row r of a
// 32-row wave (r % 32) in lane half h reads, for the 16 head_dim values of operand chunk c, the
// (cos, sin) of pairs 8c + 4h + 2p and +1 (p = 0, 1) as one 16-byte piece.  Pieces are ordered
// [r / 32][c][p][h][r % 32], so that each of a wave's loads reads 1 KB of contiguous memory;
// ceil(T / 64) * 64 rows (rows past T are never read).
inline constexpr size_t rope_qcs_index(int r, int c, int p, int h, int nch) {
    return ((((size_t)(r >> 5) * nch + c) * 2 + p) * 2 + h) * 32 + (r & 31);   // in 16-byte pieces
}

// bf16 key rotation: K~ = R k (or a copy without RoPE) and ak64 per 64-row tile
struct KeyRotArgs {
    const void* k;          // [B, Hkv, T, D] raw keys
    void* krot;             // [B, Hkv, T, D] rotated keys
    float* ak;              // [B, Hkv, ceil(T/64)] max |k| per tile
    const float* rope_cs;   // or nullptr
    int BH, T;
    float* qcs;             // or nullptr: the table in the query-operand order (rope_qcs_index),
                            // written by the blocks of kv group 0
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* delta;           // workspace (float32 path): [B, Hq, T] rowsum(dO * O)
    float* ld;              // workspace (bf16 path): per query head and 64-row tile, 4 groups of
                            // [-l' x 16 | -delta x 16] (l' = L log2(e) - log2(scale); rows >= T:
                            // -l' = -inf, -delta = 0)
    float* dq_acc;          // workspace (float32 path): [ceil(T/128)][B, Hq, T, D] rotated dQ parts,
                            // one slice per 128-key tile (rows at or after the tile's first key)
    float* dk_acc;          // workspace (float32 path): [nsplit][B, Hkv, T, D] per-share rotated dK / scale
    float* dv_acc;          // workspace (float32 path): [nsplit][B, Hkv, T, D] per-share dV
    void* qrot;             // workspace (bf16 path): [B, Hq, T, D] rotated Q times scale*log2(e),
                            // rounded to bf16 (hi part)
    void* qrot_lo;          // workspace (bf16 path): [B, Hq, T, D] its bf16 remainder (written for the
                            // blocks whose flag lof is set), hi + lo = scale*log2(e) * R q
    void* krot;             // workspace (bf16 path): [B, Hkv, T, D] rotated K, written by the preprocess
    const float* rope_cs;
    int B, Hq, Hkv, T;
    int Tp;                 // T rounded up to whole 64-row tiles
    float scale;
    int nsplit;             // float32 path: shares per key tile (bwd_f32_splits)
    int* lof;               // bf16 path: [B, Hq, ceil(T/128)] 1 where a 128-row query block uses the
                            // rotated queries' low part (the forward's decision, kLoBound)
    float* ak;              // bf16 path: [B, Hkv, ceil(T/64)] max |k| per 64-row key tile
    float* qcs;             // bf16 path with RoPE: the table in the query-operand order
                            // (rope_qcs_index), written by key_rot_kernel; the epilogues read it
};

// float32 backward: each workgroup owns 128 keys of one (batch, kv head) and one of nsplit
// contiguous shares of that tile's (query head, 32-query tile) steps.  Enough shares to make
// about a thousand workgroups at short sequences, at most one step per share, and one share
// once the key tiles alone are that many.  The workspace holds one dK / dV slice per share.
constexpr int kBwdF32Keys = 128, kBwdF32Queries = 32;
inline int bwd_f32_splits(int B, int Hq, int Hkv, int T) {
    const long units = (long)((T + kBwdF32Keys - 1) / kBwdF32Keys) * B * Hkv;
    const long steps = (long)(Hq / Hkv) * ((T + kBwdF32Queries - 1) / kBwdF32Queries);
    const long want = (1024 + units - 1) / units;
    return (int)(want < 1 ? 1 : (want < steps ? want : steps));
}

struct DecodeArgs {
    const void* q;          // [B, Hq, n, D] new tokens, un-rotated
    const void* kc;         // [B, Hkv, Tc, D] keys rotated at their positions
    const void* vc;         // [B, Hkv, Tc, D] values
    const int* kv_len;      // [B] valid cache rows, new tokens included (clamped into [n, Tc])
    void* o;                // [B, Hq, n, D]
    float* lse;             // [B, Hq, n]
    // workspace.  32-column path: part_o [B * Hkv][nsplit][32][D] chunk outputs, part_l
    // [B * Hkv][nsplit][32] chunk L (natural log).  16-column path: part_o [W + B * Hkv][16][D] and
    // part_l [W + B * Hkv][16] piece results, ctr [B * Hkv] arrival counters (zero between calls).
    float* part_o;
    float* part_l;
    int* ctr;
    const float* rope_cs;   // [rows][D/2][2] or nullptr
    int B, Hq, Hkv, n, Tc;
    int nsplit, chunk;      // 32-column path: chunks per sequence and keys per chunk (a multiple of
                            // 64); 16-column path: nsplit = W, the waves of the grid
    float scale;
};

// 16-column decode path: keys per staged tile (32 at D = 128, so that three stages stay at
// 48 KiB of LDS), LDS stages, the cap on the grid's waves, pieces merged per round of loads
constexpr int decode_tile_rows(int D) { return D == 128 ? 32 : 64; }
constexpr int kDecodeStages = 3;
constexpr int kDecodeMaxWaves = 4096;
constexpr int decode_merge_batch(int D) { return D == 128 ? 4 : 8; }

struct ProjArgs {
    const void* x;          // [M = B*T, C] bf16 activations, row-major
    const void* w;          // [N = (Hq + 2 Hkv) D, C] bf16 packed weights, row-major
    void* q;                // [B, Hq, T, D] rotated queries
    void* k;                // [B, Hkv, T, D] rotated keys
    void* v;                // [B, Hkv, T, D] values
    const float* rope_cs;   // [rows][D/2][2] or nullptr (no rotation)
    int B, T, C, Hq, Hkv, D;
    int M, N;               // token rows and output features
    int tiles_m, tiles_n;   // output tiles along tokens and features
    int per_xcd;            // tiles per XCD (the grid is 8 * per_xcd workgroups)
};

struct RopeArgs {
    const void* x;
    void* y;
    const float* rope_cs;
    int rows;               // B * H * T
    int T;
    int pos_offset;
    int inverse;
};

template <typename T, int D> hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// tokens per output tile of the projection (multiple of 64) and the launch
int proj_tile_tokens();
hipError_t launch_proj(const ProjArgs& a, hipStream_t stream);
template <typename T, int D> hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t stream);
template <typename T, int D> hipError_t launch_bwd_main(const BwdArgs& a, hipStream_t stream);
// a.qrot set: also writes the rotated queries (hi and lo parts) for the backward
template <int D> hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
template <int D> hipError_t launch_key_rot(const KeyRotArgs& a, hipStream_t stream);
// rotate == false: only the per-row (l', delta) data; the rotated queries and keys are already in
// the workspace (written by the training forward)
template <int D> hipError_t launch_bwd_pre_bf16(const BwdArgs& a, hipStream_t stream, bool rotate = true);
template <int D> hipError_t launch_bwd_main_bf16(const BwdArgs& a, hipStream_t stream);
template <typename T, int D> hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
template <typename T, int D> hipError_t launch_rope(const RopeArgs& a, hipStream_t stream);
template <int D> hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// waves of the 16-column decode grid that fit on the current device at once (CUs x resident
// waves per CU), or 0 when the query fails
template <int D> int decode16_slots();
template <int D> hipError_t launch_decode16(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_rope_table(int rows, int D, double theta, float* cs, hipStream_t stream);

}  // namespace ne
