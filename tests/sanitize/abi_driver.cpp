// Drives the C ABI of the library (include/ne_attn.h) through its argument validation under
// AddressSanitizer and UndefinedBehaviorSanitizer (host code instrumented): NULL and misaligned
// pointers, bad shapes, unsupported configurations, too-small workspaces, workspace-size queries
// and status strings.  Every call here is rejected before any launch, so no GPU is needed.
// Returns 0 when every call returns the documented status.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ne_attn.h"

static int failures = 0;
static void expect(int got, int want, const char* what) {
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}

int main() {
    alignas(16) static char buf[64];
    void* A = buf;                       // 16-byte aligned, never dereferenced: calls are rejected first
    void* M = buf + 4;                   // misaligned
    ne_attn_params p;
    memset(&p, 0, sizeof p);
    p.B = 2; p.Hq = 4; p.Hkv = 2; p.T = 16; p.D = 64; p.dtype = NE_DTYPE_BF16; p.causal = 1;
    expect(ne_attn_fwd(nullptr, A, A, A, A, (float*)A, A, 1 << 20, nullptr), NE_ERR_NULL, "fwd NULL params");
    expect(ne_attn_fwd(&p, nullptr, A, A, A, (float*)A, A, 1 << 20, nullptr), NE_ERR_NULL, "fwd NULL q");
    expect(ne_attn_fwd(&p, M, A, A, A, (float*)A, A, 1 << 20, nullptr), NE_ERR_ALIGN, "fwd misaligned q");
    expect(ne_attn_fwd(&p, A, A, A, A, (float*)A, nullptr, 0, nullptr), NE_ERR_NULL, "fwd NULL workspace");
    expect(ne_attn_fwd(&p, A, A, A, A, (float*)A, A, 1, nullptr), NE_ERR_WORKSPACE, "fwd small workspace");
    ne_attn_params s = p;
    s.Hq = 3;
    expect(ne_attn_fwd(&s, A, A, A, A, (float*)A, A, 1 << 20, nullptr), NE_ERR_SHAPE, "fwd Hq % Hkv");
    s = p; s.T = 0;
    expect(ne_attn_fwd(&s, A, A, A, A, (float*)A, A, 1 << 20, nullptr), NE_ERR_SHAPE, "fwd T = 0");
    s = p; s.D = 48;
    expect(ne_attn_fwd(&s, A, A, A, A, (float*)A, A, 1 << 20, nullptr), NE_ERR_UNSUPPORTED, "fwd D = 48");
    s = p; s.causal = 0;
    expect(ne_attn_fwd(&s, A, A, A, A, (float*)A, A, 1 << 20, nullptr), NE_ERR_UNSUPPORTED, "fwd causal = 0");
    s = p; s.dtype = NE_DTYPE_F32; s.D = 128;
    expect(ne_attn_fwd(&s, A, A, A, A, (float*)A, A, 1 << 20, nullptr), NE_ERR_UNSUPPORTED, "fwd f32 D = 128");
    s = p; s.B = 1 << 20; s.T = 1 << 12;
    expect(ne_attn_fwd(&s, A, A, A, A, (float*)A, A, 1 << 20, nullptr), NE_ERR_SHAPE, "fwd too large");
    s = p; s.rope_cs = (const float*)A; s.rope_rows = 15;
    expect(ne_attn_fwd(&s, A, A, A, A, (float*)A, A, 1 << 20, nullptr), NE_ERR_SHAPE, "fwd short rope table");
    const size_t need = ne_attn_bwd_workspace_bytes(&p);
    if (need == 0) { fprintf(stderr, "bwd workspace size 0\n"); ++failures; }
    expect(ne_attn_bwd(&p, A, A, A, A, (const float*)A, A, A, A, A, A, need - 1, nullptr), NE_ERR_WORKSPACE,
           "bwd small workspace");
    expect(ne_attn_bwd(&p, A, A, A, A, (const float*)A, A, nullptr, A, A, A, need, nullptr), NE_ERR_NULL, "bwd NULL dq");
    expect(ne_attn_bwd_main(&p, A, A, A, (const float*)A, A, A, A, M, A, need, nullptr), NE_ERR_ALIGN,
           "bwd main misaligned dv");
    expect(ne_attn_fwd_train(&p, A, A, A, A, (float*)A, A, need - 1, nullptr), NE_ERR_WORKSPACE, "fwd_train small");
    expect(ne_attn_bwd_train(&p, A, A, A, A, (const float*)A, A, A, A, A, nullptr, need, nullptr), NE_ERR_NULL,
           "bwd_train NULL workspace");
    s = p; s.D = 0;
    if (ne_attn_bwd_workspace_bytes(&s) != 0 || ne_attn_fwd_workspace_bytes(&s) != 0) {
        fprintf(stderr, "workspace size of an invalid shape is not 0\n");
        ++failures;
    }
    expect(ne_rope_table(0, 64, 10000.0, (float*)A, nullptr), NE_ERR_SHAPE, "rope table rows 0");
    expect(ne_rope_table(16, 63, 10000.0, (float*)A, nullptr), NE_ERR_SHAPE, "rope table odd D");
    expect(ne_rope_table(16, 64, -1.0, (float*)A, nullptr), NE_ERR_SHAPE, "rope table theta");
    expect(ne_rope_table(16, 64, 10000.0, (float*)M, nullptr), NE_ERR_ALIGN, "rope table misaligned");
    ne_rope_params rp;
    memset(&rp, 0, sizeof rp);
    rp.B = 1; rp.H = 2; rp.T = 8; rp.D = 64; rp.dtype = NE_DTYPE_BF16; rp.pos_offset = 4;
    rp.rope_cs = (const float*)A; rp.rope_rows = 11;
    expect(ne_rope_apply(&rp, A, A, 0, nullptr), NE_ERR_SHAPE, "rope apply table too short");
    rp.rope_rows = 12; rp.D = 16;
    expect(ne_rope_apply(&rp, A, A, 0, nullptr), NE_ERR_UNSUPPORTED, "rope apply D = 16");
    ne_decode_params dp;
    memset(&dp, 0, sizeof dp);
    dp.B = 2; dp.Hq = 4; dp.Hkv = 2; dp.n = 1; dp.D = 64; dp.dtype = NE_DTYPE_BF16; dp.cache_rows = 128;
    const size_t dneed = ne_attn_decode_workspace_bytes(&dp);
    expect(ne_attn_decode(&dp, A, A, A, (const int32_t*)A, A, (float*)A, A, dneed - 1, nullptr), NE_ERR_WORKSPACE,
           "decode small workspace");
    dp.n = 200;
    expect(ne_attn_decode(&dp, A, A, A, (const int32_t*)A, A, (float*)A, A, 1 << 30, nullptr), NE_ERR_SHAPE,
           "decode n > cache rows");
    dp.n = 1; dp.B = 10000;
    expect(ne_attn_decode_static(&dp, A, A, A, (const int32_t*)A, A, (float*)A, nullptr), NE_ERR_WORKSPACE,
           "static decode beyond its array");
    ne_qkv_params qp;
    memset(&qp, 0, sizeof qp);
    qp.B = 1; qp.T = 8; qp.C = 96; qp.Hq = 2; qp.Hkv = 1; qp.D = 64; qp.dtype = NE_DTYPE_BF16;
    expect(ne_qkv_proj(&qp, A, A, A, A, A, nullptr), NE_ERR_UNSUPPORTED, "projection C = 96");
    for (int st = 0; st >= -7; --st)
        if (!ne_status_string(st) || !ne_status_string(st)[0]) { fprintf(stderr, "status %d\n", st); ++failures; }
    if (ne_abi_version() != NE_ABI_VERSION) { fprintf(stderr, "ABI version\n"); ++failures; }
    printf(failures ? "FAILED (%d)\n" : "ok\n", failures);
    return failures != 0;
}
