// api.hip -- the extern "C" entry points declared in include/ne_attn.h: argument validation
// (before any launch) and dispatch on (dtype, head_dim) to the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "../../include/ne_attn.h"
#include "common.hpp"
#include "kernels.hpp"

namespace {

constexpr long kMaxElems = 0x7fffffffL;   // element counts index with 32-bit grid math

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_attn(const ne_attn_params* p) {
    if (!p) return NE_ERR_NULL;
    if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->T <= 0 || p->D <= 0) return NE_ERR_SHAPE;
    if (p->Hq % p->Hkv != 0) return NE_ERR_SHAPE;
    if (p->dtype != NE_DTYPE_F32 && p->dtype != NE_DTYPE_BF16) return NE_ERR_UNSUPPORTED;
    // head_dim 32 or 64; 128 on the bf16 path only (the fp32 tiles would not fit in LDS)
    if (p->D != 32 && p->D != 64 && !(p->D == 128 && p->dtype == NE_DTYPE_BF16)) return NE_ERR_UNSUPPORTED;
    if (p->causal != 1) return NE_ERR_UNSUPPORTED;
    if ((long)p->B * p->Hq * p->T * p->D > kMaxElems) return NE_ERR_SHAPE;
    if (!isfinite(p->scale)) return NE_ERR_SHAPE;
    if (p->rope_cs) {
        if (p->rope_rows < p->T) return NE_ERR_SHAPE;
        if (!aligned16(p->rope_cs)) return NE_ERR_ALIGN;
    }
    return NE_OK;
}

float eff_scale(const ne_attn_params* p) { return p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->D); }

int check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* x : ps)
        if (!x) return NE_ERR_NULL;
    for (const void* x : ps)
        if (!aligned16(x)) return NE_ERR_ALIGN;
    return NE_OK;
}

int padded_rows(int T) { return (T + 63) / 64 * 64; }

// per-row float32 data: float32 path delta [B, Hq, T]; bf16 path (l', delta) pairs for every row of
// whole 64-row tiles
size_t delta_bytes(const ne_attn_params* p) {
    size_t n = p->dtype == NE_DTYPE_BF16 ? (size_t)p->B * p->Hq * padded_rows(p->T) * 2 * sizeof(float)
                                         : (size_t)p->B * p->Hq * p->T * sizeof(float);
    return (n + 255) & ~(size_t)255;
}

// bf16: max |k| per 64-row key tile [B, Hkv, ceil(T/64)] and low-part flags per 128-row query
// block [B, Hq, ceil(T/128)]
size_t key_bound_bytes(const ne_attn_params* p) {
    return ((size_t)p->B * p->Hkv * ((p->T + 63) / 64) * sizeof(float) + 255) & ~(size_t)255;
}
// bf16 with RoPE: the table's rows in the forward's query-operand order (rope_qcs_index), for whole
// 64-row key tiles
size_t qcs_bytes(const ne_attn_params* p) {
    return p->rope_cs ? (size_t)((p->T + 63) / 64) * 64 * p->D * 2 * sizeof(float) : 0;
}
size_t lo_flag_bytes(const ne_attn_params* p) {
    return ((size_t)p->B * p->Hq * ((p->T + 127) / 128) * sizeof(int) + 255) & ~(size_t)255;
}

// the attention kernels: bf16 with D in {32, 64, 128}, fp32 with D in {32, 64}
template <typename F>
int dispatch(int dtype, int D, F&& f) {
    hipError_t e;
    if (dtype == NE_DTYPE_BF16)
        e = D == 128  ? f(ne::bf16{}, std::integral_constant<int, 128>{})
            : D == 64 ? f(ne::bf16{}, std::integral_constant<int, 64>{})
                      : f(ne::bf16{}, std::integral_constant<int, 32>{});
    else e = D == 64 ? f(float{}, std::integral_constant<int, 64>{}) : f(float{}, std::integral_constant<int, 32>{});
    return e == hipSuccess ? NE_OK : NE_ERR_HIP;
}

// the RoPE kernels: either dtype with D in {32, 64, 128}
template <typename F>
int dispatch_rope(int dtype, int D, F&& f) {
    auto by_d = [&](auto t) {
        return D == 128 ? f(t, std::integral_constant<int, 128>{})
               : D == 64 ? f(t, std::integral_constant<int, 64>{}) : f(t, std::integral_constant<int, 32>{});
    };
    const hipError_t e = dtype == NE_DTYPE_BF16 ? by_d(ne::bf16{}) : by_d(float{});
    return e == hipSuccess ? NE_OK : NE_ERR_HIP;
}

// Split-KV sizing of the decode path: enough (batch, kv head, chunk) waves to fill the chip
// (~1024), chunks of whole 64-key tiles, at most 64 chunks (one merge lane each).
void decode_split(const ne_decode_params* p, int* nsplit, int* chunk) {
    const long groups = (long)p->B * p->Hkv;
    const long want = std::min<long>(64, std::max<long>(1, (1024 + groups - 1) / groups));
    const int tiles = (p->cache_rows + 63) / 64;
    const int per = (int)std::max<long>(1, (tiles + want - 1) / want);      // tiles per chunk
    *chunk = per * 64;
    *nsplit = (tiles + per - 1) / per;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// at most 16 query columns per kv group: the balanced 16-column path
bool decode_narrow(const ne_decode_params* p) { return (long)(p->Hq / p->Hkv) * p->n <= 16; }

// Workspace of the 16-column path: arrival counters (zero between calls), then piece L and O for
// up to wcap waves plus one slot per segment.
struct Decode16Layout {
    long max_tiles;   // tiles when every cache is full
    int wcap;         // cap on the grid's waves
    size_t ctr, part_l, part_o, total;
    explicit Decode16Layout(const ne_decode_params* p) {
        const long nseg = (long)p->B * p->Hkv;
        max_tiles = nseg * ((p->cache_rows + ne::decode_tile_rows(p->D) - 1) / ne::decode_tile_rows(p->D));
        wcap = (int)std::min<long>(ne::kDecodeMaxWaves, max_tiles);
        const size_t slots = (size_t)wcap + nseg;
        ctr = 0;
        part_l = align256(nseg * sizeof(int));
        part_o = part_l + align256(slots * 16 * sizeof(float));
        total = part_o + slots * 16 * p->D * sizeof(float);
    }
};

// Waves of the 16-column grid (never more than fit at once): the fewest that minimise the
// estimated time with every cache full, a wave's tiles (one step each) plus the merge of a
// segment's pieces (one round of loads, costed like a step, per merge batch of pieces).
// Scans the tiles per wave k upward from the smallest feasible one; the cost is at least k.
long decode16_waves(const ne_decode_params* p, const Decode16Layout& L, int slots) {
    const long seg_tiles = (p->cache_rows + ne::decode_tile_rows(p->D) - 1) / ne::decode_tile_rows(p->D);
    const long wmax = std::max<long>(1, std::min<long>(L.wcap, slots));
    long best = 1, best_cost = -1;
    for (long k = (L.max_tiles + wmax - 1) / wmax; best_cost < 0 || k <= best_cost; ++k) {
        const long w = (L.max_tiles + k - 1) / k;                       // fewest waves with <= k tiles
        const long pieces = k >= seg_tiles ? 1 : (seg_tiles + k - 1) / k + 1;
        const long mb = ne::decode_merge_batch(p->D);
        const long cost = k + (pieces > 1 ? (pieces + mb - 1) / mb : 0);
        if (best_cost < 0 || cost <= best_cost) best = w, best_cost = cost;   // ties: fewer waves
    }
    return best;
}

int check_decode(const ne_decode_params* p) {
    if (!p) return NE_ERR_NULL;
    if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->n <= 0 || p->D <= 0 || p->cache_rows <= 0)
        return NE_ERR_SHAPE;
    if (p->Hq % p->Hkv != 0 || p->n > p->cache_rows) return NE_ERR_SHAPE;
    if (p->D != 32 && p->D != 64 && p->D != 128) return NE_ERR_UNSUPPORTED;
    if (p->dtype != NE_DTYPE_BF16) return NE_ERR_UNSUPPORTED;
    if ((long)(p->Hq / p->Hkv) * p->n > 32) return NE_ERR_UNSUPPORTED;
    if (p->D == 128 && (long)(p->Hq / p->Hkv) * p->n > 16) return NE_ERR_UNSUPPORTED;   // 16-column path only
    if ((long)p->B * p->Hkv * p->cache_rows * p->D > kMaxElems) return NE_ERR_SHAPE;
    if ((long)p->B * p->Hq * p->n * p->D > kMaxElems) return NE_ERR_SHAPE;
    if (!isfinite(p->scale)) return NE_ERR_SHAPE;
    if (p->rope_cs) {
        if (p->rope_rows < p->cache_rows) return NE_ERR_SHAPE;
        if (!aligned16(p->rope_cs)) return NE_ERR_ALIGN;
    }
    return NE_OK;
}

// Where the decode kernels keep their partial results.  16-column path: arrival counters (zero
// between calls), piece L and piece O for up to max_waves waves plus one slot per segment.
// 32-column path: chunk O then chunk L from part32.
struct DecodeSpace {
    char* ctr;
    char* part32_or_l;   // 32-column path: chunk outputs; 16-column path: piece L
    char* part_o;        // 16-column path: piece O
    long max_waves;      // 16-column path: cap on the grid's waves (the pieces' slots)
};

int decode_launch(const ne_decode_params* p, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* kv_len, void* o, float* lse, const DecodeSpace& sp, hipStream_t s) {
    const float scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->D);
    hipError_t e;
    if (decode_narrow(p)) {
        const Decode16Layout L(p);
        const int slots = p->D == 128 ? ne::decode16_slots<128>()
                          : p->D == 64 ? ne::decode16_slots<64>() : ne::decode16_slots<32>();
        if (slots <= 0) return NE_ERR_HIP;
        const long waves = decode16_waves(p, L, (int)std::min<long>(slots, sp.max_waves));
        ne::DecodeArgs a{q, k_cache, v_cache, kv_len, o, lse,
                         reinterpret_cast<float*>(sp.part_o), reinterpret_cast<float*>(sp.part32_or_l),
                         reinterpret_cast<int*>(sp.ctr), p->rope_cs, p->B, p->Hq, p->Hkv, p->n, p->cache_rows,
                         (int)std::max<long>(1, waves), 0, scale};
        e = p->D == 128 ? ne::launch_decode16<128>(a, s)
            : p->D == 64 ? ne::launch_decode16<64>(a, s) : ne::launch_decode16<32>(a, s);
    } else {
        int nsplit, chunk;
        decode_split(p, &nsplit, &chunk);
        const size_t parts = (size_t)p->B * p->Hkv * nsplit * 32;
        ne::DecodeArgs a{q, k_cache, v_cache, kv_len, o, lse, reinterpret_cast<float*>(sp.part32_or_l),
                         reinterpret_cast<float*>(sp.part32_or_l + align256(parts * p->D * sizeof(float))), nullptr,
                         p->rope_cs, p->B, p->Hq, p->Hkv, p->n, p->cache_rows, nsplit, chunk, scale};
        e = p->D == 64 ? ne::launch_decode<64>(a, s) : ne::launch_decode<32>(a, s);
    }
    return e == hipSuccess ? NE_OK : NE_ERR_HIP;
}

// ---- the allocation-free decode: partial results in a library-owned device array ----
//
// One array per device, in the library's code object (each GPU holds its own copy until the
// process ends).  Layout: arrival counters of the 16-column path in the first kStaticCtrBytes
// (zeroed once per device at set-up; every call leaves them at zero again), then the pieces of
// either path.  Calls on one GPU share it: calls that overlap in time on one GPU race.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
constexpr size_t kStaticCtrBytes = (size_t)64 << 10;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

__global__ void zero_words_kernel(unsigned* p, unsigned n) {
    const unsigned i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

constexpr int kMaxStaticDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxStaticDevices];

// The device address of this device's array (hipGetSymbolAddress with that device current; the
// name `scratch` itself is a host-side stand-in, never passed to a kernel), its counters zeroed
// on the first use on a device (a fill kernel on the caller's stream).
int static_scratch(hipStream_t s, char** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxStaticDevices) return NE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_static_mu);
    if (!g_static_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return NE_ERR_HIP;
        const unsigned words = (unsigned)(kStaticCtrBytes / 4);
        hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, s, static_cast<unsigned*>(ptr), words);
        if (hipGetLastError() != hipSuccess) return NE_ERR_HIP;
        g_static_ptr[dev] = ptr;
    }
    *out = static_cast<char*>(g_static_ptr[dev]);
    return NE_OK;
}

// Most waves whose pieces fit in the static array after the counters (16-column path), or -1 when
// not even one wave's do; bytes needed by the 32-column path.
long static_decode16_waves(const ne_decode_params* p) {
    const long nseg = (long)p->B * p->Hkv;
    if (nseg * (long)sizeof(int) > (long)kStaticCtrBytes) return -1;
    const size_t room = kStaticScratchBytes - kStaticCtrBytes;
    const size_t per_slot = 16 * sizeof(float) + 16 * (size_t)p->D * sizeof(float);
    const long slots = (long)((room - 256) / per_slot);      // align256 of the L part costs < 256 bytes
    return slots - nseg >= 1 ? slots - nseg : -1;
}
size_t static_decode32_bytes(const ne_decode_params* p) {
    int nsplit, chunk;
    decode_split(p, &nsplit, &chunk);
    const size_t parts = (size_t)p->B * p->Hkv * nsplit * 32;
    return align256(parts * p->D * sizeof(float)) + parts * sizeof(float);
}

}  // namespace

extern "C" {

int ne_abi_version(void) { return NE_ABI_VERSION; }

const char* ne_status_string(int status) {
    switch (status) {
        case NE_OK: return "ok";
        case NE_ERR_NULL: return "a required pointer is NULL";
        case NE_ERR_SHAPE: return "invalid shape (size <= 0, Hq % Hkv != 0, too large, or rope table too short)";
        case NE_ERR_UNSUPPORTED: return "unsupported configuration (head_dim not 32/64, dtype, or causal != 1)";
        case NE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case NE_ERR_WORKSPACE: return "workspace too small";
        case NE_ERR_HIP: return "HIP runtime error on launch";
        default: return "unknown status";
    }
}

int ne_rope_table(int32_t rows, int32_t D, double theta, float* cs, void* stream) {
    if (!cs) return NE_ERR_NULL;
    if (rows <= 0 || D <= 0 || (D % 2) != 0 || !(theta > 0.0) || !isfinite(theta)) return NE_ERR_SHAPE;
    if ((long)rows * D > kMaxElems) return NE_ERR_SHAPE;
    if (!aligned16(cs)) return NE_ERR_ALIGN;
    return ne::launch_rope_table(rows, D, theta, cs, static_cast<hipStream_t>(stream)) == hipSuccess
               ? NE_OK : NE_ERR_HIP;
}

int ne_rope_apply(const ne_rope_params* p, const void* x, void* y, int inverse, void* stream) {
    if (!p) return NE_ERR_NULL;
    if (p->B <= 0 || p->H <= 0 || p->T <= 0 || p->D <= 0 || p->pos_offset < 0) return NE_ERR_SHAPE;
    if (p->D != 32 && p->D != 64 && p->D != 128) return NE_ERR_UNSUPPORTED;
    if (p->dtype != NE_DTYPE_F32 && p->dtype != NE_DTYPE_BF16) return NE_ERR_UNSUPPORTED;
    if ((long)p->B * p->H * p->T * p->D > kMaxElems) return NE_ERR_SHAPE;
    if ((long)p->T + p->pos_offset > p->rope_rows) return NE_ERR_SHAPE;
    if (int rc = check_ptrs({x, y, p->rope_cs})) return rc;
    ne::RopeArgs a{x, y, p->rope_cs, p->B * p->H * p->T, p->T, p->pos_offset, inverse};
    hipStream_t s = static_cast<hipStream_t>(stream);
    return dispatch_rope(p->dtype, p->D, [&](auto t, auto d) {
        return ne::launch_rope<decltype(t), decltype(d)::value>(a, s);
    });
}

size_t ne_attn_fwd_workspace_bytes(const ne_attn_params* p) {
    if (check_attn(p) != NE_OK) return 0;
    if (p->dtype != NE_DTYPE_BF16) return 0;
    // bf16: max |k| per 64-row key tile, then (with RoPE) the rotated keys, written once and read by
    // every query head of their group, and the table in the query-operand order
    return key_bound_bytes(p) + (p->rope_cs ? (size_t)p->B * p->Hkv * p->T * p->D * 2 : 0) + qcs_bytes(p);
}

int ne_attn_fwd(const ne_attn_params* p, const void* q, const void* k, const void* v, void* o,
                float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    if (int rc = check_attn(p)) return rc;
    if (int rc = check_ptrs({q, k, v, o, lse})) return rc;
    const size_t need = ne_attn_fwd_workspace_bytes(p);
    if (need) {
        if (!workspace) return NE_ERR_NULL;
        if (!aligned16(workspace)) return NE_ERR_ALIGN;
        if (workspace_bytes < need) return NE_ERR_WORKSPACE;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    ne::FwdArgs a{q, k, v, o, lse, p->rope_cs, p->B, p->Hq, p->Hkv, p->T, eff_scale(p)};
    return dispatch(p->dtype, p->D, [&](auto t, auto d) {
        using T = decltype(t);
        constexpr int DD = decltype(d)::value;
        if constexpr (std::is_same<T, ne::bf16>::value) {
            char* ws = static_cast<char*>(workspace);
            float* ak = reinterpret_cast<float*>(ws);
            void* krot = p->rope_cs ? ws + key_bound_bytes(p) : nullptr;
            float* qcs = p->rope_cs ? reinterpret_cast<float*>(ws + key_bound_bytes(p) +
                                                               (size_t)p->B * p->Hkv * p->T * p->D * 2)
                                    : nullptr;
            const hipError_t e =
                ne::launch_key_rot<DD>(ne::KeyRotArgs{k, krot, ak, p->rope_cs, p->B * p->Hkv, p->T, qcs}, s);
            if (e != hipSuccess) return e;
            if (krot) a.k = krot;
            a.ak = ak;
            a.qcs = qcs;
            return ne::launch_fwd_bf16<DD>(a, s);
        } else {
            return ne::launch_fwd<T, DD>(a, s);
        }
    });
}

size_t ne_attn_decode_workspace_bytes(const ne_decode_params* p) {
    if (check_decode(p) != NE_OK) return 0;
    if (decode_narrow(p)) return Decode16Layout(p).total;
    int nsplit, chunk;
    decode_split(p, &nsplit, &chunk);
    const size_t parts = (size_t)p->B * p->Hkv * nsplit * 32;
    return align256(parts * p->D * sizeof(float)) + parts * sizeof(float);
}

int ne_attn_decode(const ne_decode_params* p, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* kv_len, void* o, float* lse, void* workspace, size_t workspace_bytes,
                   void* stream) {
    if (int rc = check_decode(p)) return rc;
    if (int rc = check_ptrs({q, k_cache, v_cache, kv_len, o, lse, workspace})) return rc;
    if (workspace_bytes < ne_attn_decode_workspace_bytes(p)) return NE_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    DecodeSpace sp;
    if (decode_narrow(p)) {
        const Decode16Layout L(p);
        sp = DecodeSpace{ws + L.ctr, ws + L.part_l, ws + L.part_o, L.wcap};
    } else {
        sp = DecodeSpace{nullptr, ws, nullptr, 0};
    }
    return decode_launch(p, q, k_cache, v_cache, kv_len, o, lse, sp, static_cast<hipStream_t>(stream));
}

int ne_qkv_proj(const ne_qkv_params* p, const void* x, const void* w, void* q, void* k, void* v, void* stream) {
    if (!p) return NE_ERR_NULL;
    if (p->B <= 0 || p->T <= 0 || p->C <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->D <= 0) return NE_ERR_SHAPE;
    if (p->dtype != NE_DTYPE_BF16) return NE_ERR_UNSUPPORTED;
    if (p->D != 32 && p->D != 64 && p->D != 128) return NE_ERR_UNSUPPORTED;
    if (p->C % 64 != 0) return NE_ERR_UNSUPPORTED;
    const long M = (long)p->B * p->T, N = (long)(p->Hq + 2L * p->Hkv) * p->D;
    // byte offsets of whole tiles (rows past M or N included) stay below 2^32
    const long pad = ne::proj_tile_tokens() > 128 ? ne::proj_tile_tokens() : 128;
    if ((M + pad) * p->C > kMaxElems || (N + pad) * p->C > kMaxElems || M * N > kMaxElems) return NE_ERR_SHAPE;
    if (p->rope_cs) {
        if (p->rope_rows < p->T) return NE_ERR_SHAPE;
        if (!aligned16(p->rope_cs)) return NE_ERR_ALIGN;
    }
    if (int rc = check_ptrs({x, w, q, k, v})) return rc;
    const int tm = (int)((M + ne::proj_tile_tokens() - 1) / ne::proj_tile_tokens());
    const int tn = (int)((N + 127) / 128);
    ne::ProjArgs a{x, w, q, k, v, p->rope_cs, p->B, p->T, p->C, p->Hq, p->Hkv, p->D, (int)M, (int)N,
                   tm, tn, (int)(((long)tm * tn + 7) / 8)};
    return ne::launch_proj(a, static_cast<hipStream_t>(stream)) == hipSuccess ? NE_OK : NE_ERR_HIP;
}

size_t ne_attn_bwd_workspace_bytes(const ne_attn_params* p) {
    if (check_attn(p) != NE_OK) return 0;
    const size_t qe = (size_t)p->B * p->Hq * p->T * p->D, ke = (size_t)p->B * p->Hkv * p->T * p->D;
    // float32: delta | dQ parts, one slice per 128-key tile | dK and dV slices, one per share of a
    // key tile
    // bf16: (-l', -delta) per row | low-part flags | max |k| per key tile | scaled rotated Q hi | lo |
    // rotated K | with RoPE, the table in the forward's query-operand order
    if (p->dtype == NE_DTYPE_BF16)
        return delta_bytes(p) + lo_flag_bytes(p) + key_bound_bytes(p) + 2 * ((qe * 2 + 255) & ~(size_t)255) + ke * 2 +
               qcs_bytes(p);
    const size_t ns = (size_t)ne::bwd_f32_splits(p->B, p->Hq, p->Hkv, p->T);
    const size_t nkt = (size_t)(p->T + ne::kBwdF32Keys - 1) / ne::kBwdF32Keys;
    return delta_bytes(p) + (nkt * qe + 2 * ns * ke) * sizeof(float);
}

namespace {
int bwd_args(const ne_attn_params* p, const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, ne::BwdArgs* a) {
    if (int rc = check_attn(p)) return rc;
    if (workspace_bytes < ne_attn_bwd_workspace_bytes(p)) return NE_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    const size_t qe = (size_t)p->B * p->Hq * p->T * p->D;
    float* delta = nullptr;
    float* ld = nullptr;
    float* dq_acc = nullptr;
    float* dk_acc = nullptr;
    float* dv_acc = nullptr;
    void* qrot = nullptr;
    void* qrot_lo = nullptr;
    void* krot = nullptr;
    int* lof = nullptr;
    float* ak = nullptr;
    float* qcs = nullptr;
    int nsplit = 1;
    if (p->dtype == NE_DTYPE_BF16) {
        const size_t qb = (qe * 2 + 255) & ~(size_t)255;
        char* x = ws;
        ld = reinterpret_cast<float*>(x);
        x += delta_bytes(p);
        lof = reinterpret_cast<int*>(x);
        x += lo_flag_bytes(p);
        ak = reinterpret_cast<float*>(x);
        x += key_bound_bytes(p);
        qrot = x;
        qrot_lo = x + qb;
        // without RoPE the kernels read the keys themselves
        krot = p->rope_cs ? x + 2 * qb : const_cast<void*>(k);
        // with RoPE the table in the query-operand order follows the rotated keys
        if (p->rope_cs) qcs = reinterpret_cast<float*>(x + 2 * qb + (size_t)p->B * p->Hkv * p->T * p->D * 2);
    } else {
        delta = reinterpret_cast<float*>(ws);
        const size_t ke = (size_t)p->B * p->Hkv * p->T * p->D;
        nsplit = ne::bwd_f32_splits(p->B, p->Hq, p->Hkv, p->T);
        dq_acc = reinterpret_cast<float*>(ws + delta_bytes(p));
        dk_acc = dq_acc + (size_t)((p->T + ne::kBwdF32Keys - 1) / ne::kBwdF32Keys) * qe;
        dv_acc = dk_acc + (size_t)nsplit * ke;
    }
    *a = ne::BwdArgs{q, k, v, o, lse, dout, dq, dk, dv, delta, ld, dq_acc, dk_acc, dv_acc, qrot, qrot_lo, krot, p->rope_cs,
                     p->B, p->Hq, p->Hkv, p->T, padded_rows(p->T), eff_scale(p), nsplit, lof, ak, qcs};
    return NE_OK;
}
}  // namespace

int ne_attn_bwd_preprocess(const ne_attn_params* p, const void* q, const void* k, const void* o,
                           const float* lse, const void* dout, void* workspace, size_t workspace_bytes,
                           void* stream) {
    if (int rc = check_attn(p)) return rc;
    if (int rc = check_ptrs({q, k, o, lse, dout, workspace})) return rc;
    ne::BwdArgs a;
    if (int rc = bwd_args(p, q, k, nullptr, o, lse, dout, nullptr, nullptr, nullptr,
                          workspace, workspace_bytes, &a)) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return dispatch(p->dtype, p->D, [&](auto t, auto d) {
        using T = decltype(t);
        constexpr int DD = decltype(d)::value;
        if constexpr (std::is_same<T, ne::bf16>::value) {
            const hipError_t e = ne::launch_key_rot<DD>(
                ne::KeyRotArgs{k, p->rope_cs ? a.krot : nullptr, a.ak, p->rope_cs, p->B * p->Hkv, p->T, a.qcs}, s);
            if (e != hipSuccess) return e;
            return ne::launch_bwd_pre_bf16<DD>(a, s);
        } else {
            return ne::launch_bwd_pre<T, DD>(a, s);
        }
    });
}

int ne_attn_fwd_train(const ne_attn_params* p, const void* q, const void* k, const void* v, void* o,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    if (int rc = check_attn(p)) return rc;
    if (p->dtype != NE_DTYPE_BF16) return ne_attn_fwd(p, q, k, v, o, lse, nullptr, 0, stream);
    if (int rc = check_ptrs({q, k, v, o, lse, workspace})) return rc;
    ne::BwdArgs b;
    if (int rc = bwd_args(p, q, k, v, o, lse, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes, &b))
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    ne::FwdArgs a{q, b.krot, v, o, lse, p->rope_cs, p->B, p->Hq, p->Hkv, p->T, eff_scale(p), b.qrot, b.qrot_lo,
                  b.ak, b.lof, b.qcs};
    return dispatch(p->dtype, p->D, [&](auto t, auto d) {
        using T = decltype(t);
        constexpr int DD = decltype(d)::value;
        if constexpr (std::is_same<T, ne::bf16>::value) {
            // the keys as the backward reads them (rotated once here; without RoPE the raw keys)
            // and their tile bounds
            const hipError_t e = ne::launch_key_rot<DD>(
                ne::KeyRotArgs{k, p->rope_cs ? b.krot : nullptr, b.ak, p->rope_cs, p->B * p->Hkv, p->T, b.qcs}, s);
            if (e != hipSuccess) return e;
            return ne::launch_fwd_bf16<DD>(a, s);
        } else {
            return hipErrorInvalidValue;            // not reached: float32 returned above
        }
    });
}

int ne_attn_bwd_train_preprocess(const ne_attn_params* p, const void* q, const void* k, const void* o,
                                 const float* lse, const void* dout, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    if (int rc = check_attn(p)) return rc;
    if (p->dtype != NE_DTYPE_BF16) return ne_attn_bwd_preprocess(p, q, k, o, lse, dout, workspace, workspace_bytes, stream);
    if (int rc = check_ptrs({q, k, o, lse, dout, workspace})) return rc;
    ne::BwdArgs a;
    if (int rc = bwd_args(p, q, k, nullptr, o, lse, dout, nullptr, nullptr, nullptr,
                          workspace, workspace_bytes, &a)) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return dispatch(p->dtype, p->D, [&](auto t, auto d) {
        using T = decltype(t);
        constexpr int DD = decltype(d)::value;
        if constexpr (std::is_same<T, ne::bf16>::value) return ne::launch_bwd_pre_bf16<DD>(a, s, false);
        else return hipErrorInvalidValue;        // not reached: float32 returned above
    });
}

int ne_attn_bwd_train(const ne_attn_params* p, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                      size_t workspace_bytes, void* stream) {
    if (int rc = check_attn(p)) return rc;
    if (int rc = check_ptrs({q, k, v, o, lse, dout, dq, dk, dv, workspace})) return rc;
    if (workspace_bytes < ne_attn_bwd_workspace_bytes(p)) return NE_ERR_WORKSPACE;
    if (int rc = ne_attn_bwd_train_preprocess(p, q, k, o, lse, dout, workspace, workspace_bytes, stream)) return rc;
    return ne_attn_bwd_main(p, q, k, v, lse, dout, dq, dk, dv, workspace, workspace_bytes, stream);
}

int ne_attn_bwd_main(const ne_attn_params* p, const void* q, const void* k, const void* v,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, void* stream) {
    if (int rc = check_attn(p)) return rc;
    if (int rc = check_ptrs({q, k, v, lse, dout, dq, dk, dv, workspace})) return rc;
    ne::BwdArgs a;
    if (int rc = bwd_args(p, q, k, v, nullptr, lse, dout, dq, dk, dv, workspace, workspace_bytes, &a))
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return dispatch(p->dtype, p->D, [&](auto t, auto d) {
        using T = decltype(t);
        constexpr int DD = decltype(d)::value;
        if constexpr (std::is_same<T, ne::bf16>::value) {
            return ne::launch_bwd_main_bf16<DD>(a, s);
        } else {
            return ne::launch_bwd_main<T, DD>(a, s);
        }
    });
}

int ne_attn_bwd(const ne_attn_params* p, const void* q, const void* k, const void* v, const void* o,
                const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, void* stream) {
    if (int rc = check_attn(p)) return rc;
    if (int rc = check_ptrs({q, k, v, o, lse, dout, dq, dk, dv, workspace})) return rc;
    if (workspace_bytes < ne_attn_bwd_workspace_bytes(p)) return NE_ERR_WORKSPACE;
    if (int rc = ne_attn_bwd_preprocess(p, q, k, o, lse, dout, workspace, workspace_bytes, stream)) return rc;
    return ne_attn_bwd_main(p, q, k, v, lse, dout, dq, dk, dv, workspace, workspace_bytes, stream);
}

size_t ne_attn_decode_static_max_bytes(void) { return kStaticScratchBytes; }

int ne_attn_decode_static(const ne_decode_params* p, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* kv_len, void* o, float* lse, void* stream) {
    if (int rc = check_decode(p)) return rc;
    if (int rc = check_ptrs({q, k_cache, v_cache, kv_len, o, lse})) return rc;
    const bool narrow = decode_narrow(p);
    const long wmax = narrow ? static_decode16_waves(p) : 0;
    if (narrow ? wmax < 1 : static_decode32_bytes(p) > kStaticScratchBytes - kStaticCtrBytes)
        return NE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = nullptr;
    if (int rc = static_scratch(s, &base)) return rc;
    DecodeSpace sp;
    if (narrow) {
        const long slots = wmax + (long)p->B * p->Hkv;
        char* pl = base + kStaticCtrBytes;
        sp = DecodeSpace{base, pl, pl + align256((size_t)slots * 16 * sizeof(float)), wmax};
    } else {
        sp = DecodeSpace{nullptr, base + kStaticCtrBytes, nullptr, 0};
    }
    return decode_launch(p, q, k_cache, v_cache, kv_len, o, lse, sp, s);
}

}  // extern "C"
