/*
 * ne_attn.h -- C ABI of the MI355X (gfx950) causal grouped-query FlashAttention library.
 *
 * The operation is the attention of a small decoder-only GPT as the NanoEuler pages describe it:
 * RoPE on queries and keys, grouped-query attention (a smaller set of key/value heads, each
 * shared by a contiguous group of query heads), causal self-attention, computed with tiling and
 * an online softmax so that the T x T score matrix is never stored, with a hand-written backward
 * pass.  (agentlenshq page "NanoEuler: C와 CUDA로 밑바닥부터 구축한 GPT-2 규모의 LLM", sections
 * "기술 사양" and "커널 구현"; byte-level GPT page "Tiny hackable CUDA language model
 * implementation", section "Core Mechanics"; ai-paper-delta NanoEuler page, "Core Mechanics".)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Layout: every activation is [B, H, T, D], contiguous, row-major (D fastest).
 *    q, o, dout, dq: H = Hq.  k, v, dk, dv: H = Hkv.  lse: [B, Hq, T] float32.
 *  * Query head h reads key/value head h / (Hq / Hkv).
 *  * Causal mask: query i sees keys j <= i (its own position included).
 *  * RoPE: adjacent pairs (x[2i], x[2i+1]) at position t are rotated by t * theta^(-2i/D):
 *    (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).  The rotation angles come from a table made
 *    by ne_rope_table (cos/sin evaluated in double, stored as float32).
 *  * Scores S_ij = scale * <R_i q_i, R_j k_j>; lse_i = ln sum_{j<=i} exp(S_ij) (natural log).
 *  * Element types: NE_DTYPE_F32 (float32 in/out, float32 arithmetic) or NE_DTYPE_BF16 (bfloat16
 *    in/out, bf16 matrix-core products with float32 accumulation).  lse is always float32; a
 *    workspace is opaque bytes whose size the matching *_workspace_bytes() call gives.
 *  * Memory: every pointer is device memory owned by the caller, 16-byte aligned.  The library
 *    allocates nothing and keeps no state beyond a cached device-property query.  Inputs are
 *    never written; outputs are fully overwritten (never accumulated into).
 *  * Streams: `stream` is a hipStream_t (NULL = the null stream).  Calls are asynchronous and
 *    never synchronise the host; device-side faults surface at the caller's next synchronisation.
 *  * Errors: 0 (NE_OK) or a negative NE_ERR_* code.  Arguments are validated before anything is
 *    launched; on an error nothing is launched and no output is touched.  No C++ exception
 *    crosses this interface.
 */
#ifndef NE_ATTN_H
#define NE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NE_ABI_VERSION 9

enum {
    NE_OK = 0,
    NE_ERR_NULL = -1,        /* a required pointer is NULL */
    NE_ERR_SHAPE = -2,       /* a size <= 0, Hq % Hkv != 0, rope table too short, ... */
    NE_ERR_UNSUPPORTED = -3, /* head_dim not supported (see each call), unknown dtype, causal != 1 */
    NE_ERR_ALIGN = -4,       /* a pointer that is not 16-byte aligned */
    NE_ERR_WORKSPACE = -5,   /* workspace smaller than the *_workspace_bytes() figure */
    NE_ERR_HIP = -6          /* the HIP runtime reported an error on launch */
};

enum { NE_DTYPE_F32 = 0, NE_DTYPE_BF16 = 1 };

typedef struct ne_attn_params {
    int32_t B, Hq, Hkv, T, D;   /* batch, query heads, kv heads, sequence length, head_dim:
                                   32 or 64, or 128 with NE_DTYPE_BF16 */
    int32_t dtype;              /* NE_DTYPE_F32 or NE_DTYPE_BF16 */
    int32_t causal;             /* must be 1 */
    float scale;                /* softmax scale; <= 0 means 1/sqrt(D) */
    const float* rope_cs;       /* device [rope_rows][D/2][2] (cos, sin) table, or NULL = no RoPE */
    int32_t rope_rows;          /* rows in rope_cs; must be >= T when rope_cs != NULL */
} ne_attn_params;

typedef struct ne_rope_params {
    int32_t B, H, T, D;
    int32_t dtype;              /* NE_DTYPE_F32 or NE_DTYPE_BF16 */
    int32_t pos_offset;         /* row t is rotated with the table row t + pos_offset (>= 0) */
    const float* rope_cs;       /* device [rope_rows][D/2][2] */
    int32_t rope_rows;          /* must be >= T + pos_offset */
} ne_rope_params;

/* NE_ABI_VERSION of the loaded library. */
int ne_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* ne_status_string(int status);

/*
 * Fill the RoPE table: cs[t][i] = (cos(t w_i), sin(t w_i)), w_i = theta^(-2i/D), for
 * t < rows and i < D/2, evaluated in double on the device and rounded to float32.
 * cs: device, rows * D * sizeof(float) bytes, written.  D even and >= 2, rows >= 1, theta > 0.
 * (RoPE on queries and keys: agentlenshq NanoEuler page, "기술 사양".)
 */
int ne_rope_table(int32_t rows, int32_t D, double theta, float* cs, void* stream);

/*
 * y = R x (inverse == 0) or y = R^T x (inverse != 0) for x, y of shape [B, H, T, D] in dtype;
 * row t uses the table row t + pos_offset.  x == y (in place) is allowed; other overlap is not.
 * D must be in {32, 64, 128}.  (Rotary embedding of queries and keys: agentlenshq NanoEuler page,
 * "기술 사양"; byte-level GPT page, "Core Mechanics".)
 */
int ne_rope_apply(const ne_rope_params* p, const void* x, void* y, int inverse, void* stream);

/*
 * Bytes of workspace ne_attn_fwd needs for these parameters (0 on a bad shape, and 0 on the
 * float32 path, which needs none).  bf16: the largest |k| of every 64-row key tile (float32,
 * B*Hkv*ceil(T/64), rounded up to 256 bytes; it decides, per 128-query block, whether the rotated
 * query's bf16 remainder enters the scores), then with RoPE the keys rotated once per call
 * (B*Hkv*T*D bf16) and the RoPE table's rows re-ordered for the query rotation (ceil(T/64)*64
 * rows of D/2 float32 (cos, sin) pairs).  The bf16 forward therefore always takes a workspace.
 */
size_t ne_attn_fwd_workspace_bytes(const ne_attn_params* p);

/*
 * Forward: o = softmax_causal(scale * (R q)(R k)^T) v and lse (natural log), per query head,
 * with kv head h / (Hq/Hkv).  q [B,Hq,T,D], k/v [B,Hkv,T,D], o [B,Hq,T,D] in dtype;
 * lse [B,Hq,T] float32.  Tiled with an online softmax: no T x T buffer exists at any point
 * (agentlenshq NanoEuler page, "커널 구현").  workspace: device, 16-byte aligned,
 * >= ne_attn_fwd_workspace_bytes(p) bytes, owned by the caller (may be NULL when that is 0);
 * contents on entry ignored, on exit unspecified.
 */
int ne_attn_fwd(const ne_attn_params* p, const void* q, const void* k, const void* v, void* o,
                float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace that ne_attn_bwd needs for these parameters (0 on a bad shape).  float32:
 * delta, the dQ parts (one float32 [B,Hq,T,D] slice per 128-key tile, summed in key order) and the
 * dK / dV parts (one slice per share of a key tile), so that the float32 backward is
 * deterministic.  bf16: the per-row exponent offsets and deltas, the per-128-query-block flags of
 * the query's low part, the largest |k| per 64-row key tile, the rotated queries scaled by
 * scale*log2(e) (two bf16 parts), the rotated keys and, with RoPE, the table rows re-ordered as in
 * ne_attn_fwd_workspace_bytes (read by ne_attn_fwd_train). */
size_t ne_attn_bwd_workspace_bytes(const ne_attn_params* p);

/*
 * Backward of ne_attn_fwd for the upstream gradient dout (hand-written backward: ai-paper-delta
 * NanoEuler page, "Core Mechanics"; agentlenshq NanoEuler page, "검증 및 안정성").
 * Inputs: q, k, v, o (the forward output), lse (the forward lse), dout [B,Hq,T,D].
 * Outputs: dq [B,Hq,T,D], dk, dv [B,Hkv,T,D], all in dtype.  dq and dk are gradients with
 * respect to the un-rotated q and k the caller passed; dk and dv are summed over the query heads
 * of each kv group.  workspace: device, >= ne_attn_bwd_workspace_bytes(p) bytes, owned by the
 * caller; its contents on entry are ignored and on exit are unspecified.
 */
int ne_attn_bwd(const ne_attn_params* p, const void* q, const void* k, const void* v,
                const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two halves of ne_attn_bwd, for callers that schedule them separately (for example to time
 * or overlap them).  ne_attn_bwd is exactly ne_attn_bwd_preprocess followed, on the same stream
 * and workspace, by ne_attn_bwd_main.
 *
 * ne_attn_bwd_preprocess: delta_i = sum_d dout_id * o_id (float32) for every query row, the
 * per-row term of the softmax backward dS = P * (dP - delta), written into the workspace, which
 * it also prepares for ne_attn_bwd_main (bf16: the rotated queries R q and keys R k, the low-part
 * flags made as the forward makes them and, from lse, the per-row exponent offset).  Reads q, k,
 * o, lse and dout; writes only the workspace.
 *
 * ne_attn_bwd_main: dq, dk, dv as ne_attn_bwd, from a workspace that ne_attn_bwd_preprocess filled
 * for the same parameters, o and dout (stream order), with no call on that workspace in between.
 */
int ne_attn_bwd_preprocess(const ne_attn_params* p, const void* q, const void* k, const void* o,
                           const float* lse, const void* dout, void* workspace, size_t workspace_bytes,
                           void* stream);
int ne_attn_bwd_main(const ne_attn_params* p, const void* q, const void* k, const void* v,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * The training pair: the same forward and backward as ne_attn_fwd / ne_attn_bwd, sharing one
 * workspace (>= ne_attn_bwd_workspace_bytes(p), owned by the caller).  o and lse are identical
 * bit for bit; the gradients agree up to float32 rounding (the rotation of q is evaluated by
 * another kernel, whose products the compiler contracts differently).
 * ne_attn_fwd_train also leaves in it what the backward would otherwise recompute from q and k:
 * on the bf16 path the rotated queries (as two bf16 parts) and the rotated keys.  The backward
 * preprocess then reads only O, dO and L.  Between the two calls the workspace must not be used
 * otherwise; q, k and the params must be the same.  On the float32 path the pair is ne_attn_fwd
 * followed by ne_attn_bwd.  Arguments, layouts and errors as for ne_attn_fwd / ne_attn_bwd.
 * (Keeping the forward's rotated operands for the backward instead of recomputing them: the
 * saved-activation pattern of the FlashAttention backward the NanoEuler pages build on,
 * agentlenshq NanoEuler page, "커널 구현".)
 */
int ne_attn_fwd_train(const ne_attn_params* p, const void* q, const void* k, const void* v, void* o,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream);
int ne_attn_bwd_train(const ne_attn_params* p, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                      size_t workspace_bytes, void* stream);
/* the first half of ne_attn_bwd_train (its second half is ne_attn_bwd_main) */
int ne_attn_bwd_train_preprocess(const ne_attn_params* p, const void* q, const void* k, const void* o,
                                 const float* lse, const void* dout, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Decode-time attention: n new tokens per sequence against a KV cache (the token-by-token
 * generation path of the NanoEuler pages; the same attention as ne_attn_fwd at the last n
 * positions: agentlenshq NanoEuler page, "커널 구현", RoPE as in "기술 사양").
 *   q        [B, Hq, n, D] dtype: the new tokens' queries, un-rotated.  Token i of sequence b sits at
 *            position kv_len[b] - n + i; it is rotated there and sees cache rows 0 .. kv_len[b] - n + i.
 *   k_cache  [B, Hkv, cache_rows, D] dtype: keys already rotated at their own positions (rotate
 *            each key once when appending it, e.g. ne_rope_apply with pos_offset); rows at or past
 *            kv_len[b] are not read.  The new tokens' keys and values must be in the cache.
 *   v_cache  [B, Hkv, cache_rows, D] dtype: values.
 *   kv_len   [B] int32, device: valid rows per sequence, the n new tokens included.  Values outside
 *            [n, cache_rows] are clamped into it (results are then meaningless, accesses stay in
 *            bounds).
 *   o [B, Hq, n, D] dtype, lse [B, Hq, n] float32 (natural log): outputs.
 *   workspace: device, 16-byte aligned, >= ne_attn_decode_workspace_bytes(p), owned by the caller.
 *            It must be zero-filled before its first use; every call leaves it ready for the
 *            next one (arrival counters back at zero).  Calls that share a workspace must not
 *            overlap in time.
 * bf16 only; D in {32, 64, 128}; (Hq/Hkv) * n <= 32 (the query columns of one kv group share its
 * key tiles), <= 16 when D = 128.  With (Hq/Hkv) * n <= 16: one launch on stream; the valid tiles of all (sequence, kv
 * head) pairs are split evenly over the waves that fit on the device, and the pieces of a pair
 * are merged by log-sum-exp inside the launch.  Otherwise two launches (fixed key chunks, then
 * the merge).  Returns NE_ERR_HIP if the device cannot be queried or a launch fails.
 */
typedef struct ne_decode_params {
    int32_t B, Hq, Hkv;
    int32_t n;             /* new tokens per sequence */
    int32_t D;
    int32_t dtype;         /* NE_DTYPE_BF16 */
    int32_t cache_rows;    /* rows allocated per (batch, kv head) in each cache */
    float scale;           /* <= 0: 1/sqrt(D) */
    const float* rope_cs;  /* device RoPE table with >= cache_rows rows, or NULL (no RoPE) */
    int32_t rope_rows;
} ne_decode_params;

size_t ne_attn_decode_workspace_bytes(const ne_decode_params* p);
int ne_attn_decode(const ne_decode_params* p, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* kv_len, void* o, float* lse, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * ne_attn_decode without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same operation,
 * arguments and results as ne_attn_decode, with the partial results kept in a device array that
 * the library itself holds (one per GPU, in the library's code object, until the process ends;
 * ne_attn_decode_static_max_bytes() bytes, 32 MiB).  The call allocates nothing.
 *   Its first call on a device zeroes the array's arrival counters with a small kernel on stream;
 *   every call leaves them at zero again.  All calls on one GPU share the array: calls that
 *   overlap in time on one GPU (same or different streams, host threads) race and must not.
 *   The 16-column path may run fewer waves than ne_attn_decode would (as many as the array holds
 *   the pieces of), so results agree with ne_attn_decode to rounding, not always bit for bit.
 * Returns NE_ERR_WORKSPACE, before any launch, when the partial results of this shape do not fit
 * (more than 16384 (sequence, kv head) pairs, or not even one wave's pieces); other errors as for
 * ne_attn_decode.
 */
size_t ne_attn_decode_static_max_bytes(void);
int ne_attn_decode_static(const ne_decode_params* p, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* kv_len, void* o, float* lse, void* stream);

/*
 * The query, key and value projections of an attention block, with RoPE on the queries and keys,
 * written straight into the attention layout (the bias-free linear maps before the attention:
 * agentlenshq NanoEuler page, "핵심 아키텍처 및 설계"; RoPE on queries and keys: "기술 사양").
 *   x  [B, T, C] bf16, row-major: the normalised activations of B sequences of T tokens.
 *   w  [(Hq + 2 Hkv) D, C] bf16, row-major: packed weights, output feature f = x . w[f]; the
 *      features are [query heads | key heads | value heads], head-major, d fastest in each head.
 *   q  [B, Hq, T, D] bf16: R_t (x W_q^T) for the token at position t (0-based within its sequence);
 *   k  [B, Hkv, T, D] bf16: R_t (x W_k^T);  v [B, Hkv, T, D] bf16: x W_v^T.  No RoPE when
 *      rope_cs is NULL.  Outputs are fully overwritten; x and w are not written.
 * bf16 only; D in {32, 64, 128}; C a multiple of 64; B*T*C and (Hq + 2 Hkv)*D*C below 2^31.
 * fp32 accumulation, one rounding to bf16 per output.  One launch on stream; no workspace.
 */
typedef struct ne_qkv_params {
    int32_t B, T, C;           /* sequences, tokens per sequence, model width */
    int32_t Hq, Hkv, D;        /* query heads, kv heads, head_dim */
    int32_t dtype;             /* NE_DTYPE_BF16 */
    const float* rope_cs;      /* device RoPE table with >= T rows (ne_rope_table), or NULL */
    int32_t rope_rows;
} ne_qkv_params;

int ne_qkv_proj(const ne_qkv_params* p, const void* x, const void* w, void* q, void* k, void* v,
                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NE_ATTN_H */
