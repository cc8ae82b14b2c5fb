// attn_abi.cpp -- the C ABI shim: argument validation, then one launcher call.
// Every check runs on the host before any HIP call; a rejected call launches nothing and
// writes nothing.  Unsupported inputs are reported, never routed to another code path
// [zwjcode.cn FlashAttention blog, sections 08 and 11: make "unsupported, fell back" an
// explicit error; LLM Internals 10.3.8 on silent fallback to the math path].
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/attn.h"
#include "attn_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

int attn::device_cu_count() {
    // per-device cache; a race between threads only repeats the same query
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev < 64) cached[dev] = n;
    return n;
}

hipError_t attn::report_launch(hipError_t e, const char* what) {
    if (e != hipSuccess && getenv("ATTN_DEBUG"))
        fprintf(stderr, "libattn: launching %s failed: %s\n", what, hipGetErrorString(e));
    return e;
}

extern "C" int attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                        int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                        int dtype, void* stream) {
    if (!Q || !K || !V || !O || !LSE) return ATTN_ERR_NULL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
    if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_SHAPE;
    // element counts must stay addressable with 64-bit offsets and the grid in 32 bits
    if ((long long)B * Hq * (long long)N * d > (1LL << 46)) return ATTN_ERR_SHAPE;
    // one head's rows are addressed with 32-bit byte offsets
    if ((long long)N * d * 2 > (1LL << 30)) return ATTN_ERR_SHAPE;
    if ((long long)((N + 127) / 128) * B * Hq > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
        !aligned(LSE, 16))
        return ATTN_ERR_ALIGN;
    attn::PrefillArgs a{Q, K, V, O, LSE, B, Hq, Hkv, N, d, causal != 0, dtype == ATTN_BF16,
                        scale, stream};
    return attn::launch_prefill(a) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_fwd_variant(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                int B, int Hq, int Hkv, int N, int d, int causal, int window,
                                float softcap, float scale, int dtype, void* stream) {
    if (!Q || !K || !V || !O || !LSE) return ATTN_ERR_NULL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
    if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_SHAPE;
    if (window < 0 || !(softcap >= 0.f) || !isfinite(softcap)) return ATTN_ERR_SHAPE;
    if ((long long)B * Hq * (long long)N * d > (1LL << 46)) return ATTN_ERR_SHAPE;
    if ((long long)N * d * 2 > (1LL << 30)) return ATTN_ERR_SHAPE;
    if ((long long)((N + 127) / 128) * B * Hq > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (window > 0 && !causal) return ATTN_ERR_UNSUPPORTED;   // the sliding window is causal
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
        !aligned(LSE, 16))
        return ATTN_ERR_ALIGN;
    attn::PrefillArgs a{Q, K, V, O, LSE, B, Hq, Hkv, N, d, causal != 0, dtype == ATTN_BF16,
                        scale, stream};
    return attn::launch_prefill_variant(a, window, softcap) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" size_t attn_decode_paged_workspace_bytes(int B, int Hq, int d, int page_size,
                                                    int max_pages_per_seq, int split_tokens) {
    if (B <= 0 || Hq <= 0 || d <= 0 || page_size <= 0 || max_pages_per_seq <= 0 ||
        split_tokens < 0)
        return 0;
    const long long S = attn::decode_max_splits(page_size, max_pages_per_seq, split_tokens);
    return attn::decode_workspace_bytes(B, Hq, d, S);
}

// Checks of a paged decode call (everything but the workspace).  On success *S_out is the
// number of partial states per (sequence, head).
int attn::check_decode_args(const void* q, const void* Kpages, const void* Vpages,
                            const int* block_table, const int* ctx_lens, const void* O,
                            const float* LSE, int B, int Hq, int Hkv, int d, int page_size,
                            int max_pages_per_seq, int split_tokens, float scale, int dtype,
                            long long* S_out) {
    if (!q || !Kpages || !Vpages || !block_table || !ctx_lens || !O) return ATTN_ERR_NULL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || page_size <= 0 || max_pages_per_seq <= 0 ||
        split_tokens < 0 || Hq % Hkv != 0)
        return ATTN_ERR_SHAPE;
    if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (page_size != 16) return ATTN_ERR_UNSUPPORTED;
    if (split_tokens % page_size != 0) return ATTN_ERR_UNSUPPORTED;   // 0 = balanced
    if (Hq / Hkv > 16) return ATTN_ERR_UNSUPPORTED;
    const long long S = attn::decode_max_splits(page_size, max_pages_per_seq, split_tokens);
    if (S > 65535 || (long long)max_pages_per_seq * page_size > 0x7fffffffLL ||
        (long long)B * Hq > 0x7fffffffLL || Hkv > 65535 || B > 65535)
        return ATTN_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(Kpages, 16) || !aligned(Vpages, 16) || !aligned(O, 16) ||
        !aligned(block_table, 4) || !aligned(ctx_lens, 4) || (LSE && !aligned(LSE, 4)))
        return ATTN_ERR_ALIGN;
    *S_out = S;
    return ATTN_OK;
}

extern "C" int attn_decode_paged(const void* q, const void* Kpages, const void* Vpages,
                                 const int* block_table, const int* ctx_lens, void* O, float* LSE,
                                 int B, int Hq, int Hkv, int d, int page_size,
                                 int max_pages_per_seq, int split_tokens, float scale, int dtype,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    long long S = 0;
    const int st = attn::check_decode_args(q, Kpages, Vpages, block_table, ctx_lens, O, LSE, B,
                                           Hq, Hkv, d, page_size, max_pages_per_seq,
                                           split_tokens, scale, dtype, &S);
    if (st != ATTN_OK) return st;
    if (!workspace) return ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_ERR_ALIGN;
    if (workspace_bytes < attn::decode_workspace_bytes(B, Hq, d, S)) return ATTN_ERR_WORKSPACE;
    attn::DecodeArgs a{q, Kpages, Vpages, block_table, ctx_lens, O, LSE, B, Hq, Hkv, d,
                       page_size, max_pages_per_seq, split_tokens, dtype == ATTN_BF16, scale,
                       workspace, stream};
    return attn::launch_decode(a) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" size_t attn_decode_cascade_workspace_bytes(int B, int Hq, int d, int page_size,
                                                      int max_pages_per_seq, int split_tokens,
                                                      int prefix_len) {
    if (B <= 0 || Hq <= 0 || d <= 0 || page_size <= 0 || max_pages_per_seq <= 0 ||
        split_tokens < 0 || prefix_len < 0)
        return 0;
    const long long S = attn::decode_max_splits(page_size, max_pages_per_seq, split_tokens) +
                        attn::cascade_chunks(prefix_len);
    return attn::decode_workspace_bytes(B, Hq, d, S);
}

extern "C" int attn_decode_cascade(const void* q, const void* Kprefix, const void* Vprefix,
                                   int prefix_len, const void* Kpages, const void* Vpages,
                                   const int* block_table, const int* ctx_lens, void* O,
                                   float* LSE, int B, int Hq, int Hkv, int d, int page_size,
                                   int max_pages_per_seq, int split_tokens, float scale,
                                   int dtype, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    if (!q || !Kpages || !Vpages || !block_table || !ctx_lens || !O) return ATTN_ERR_NULL;
    if (prefix_len < 0) return ATTN_ERR_SHAPE;
    if (prefix_len > 0 && (!Kprefix || !Vprefix)) return ATTN_ERR_NULL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || page_size <= 0 || max_pages_per_seq <= 0 ||
        split_tokens < 0 || Hq % Hkv != 0)
        return ATTN_ERR_SHAPE;
    if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (page_size != 16) return ATTN_ERR_UNSUPPORTED;
    if (split_tokens % page_size != 0) return ATTN_ERR_UNSUPPORTED;   // 0 = balanced
    if (Hq / Hkv > 16) return ATTN_ERR_UNSUPPORTED;
    const long long S = attn::decode_max_splits(page_size, max_pages_per_seq, split_tokens) +
                        attn::cascade_chunks(prefix_len);
    if (S > 65535 || (long long)max_pages_per_seq * page_size > 0x7fffffffLL ||
        (long long)B * Hq > 0x7fffffffLL || Hkv > 65535 || B > 65535)
        return ATTN_ERR_SHAPE;
    // q rows and one prefix head are addressed with 32-bit byte offsets
    if ((long long)B * Hq * d * 2 > (1LL << 30) || (long long)prefix_len * d * 2 > (1LL << 30))
        return ATTN_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(Kpages, 16) || !aligned(Vpages, 16) || !aligned(O, 16) ||
        !aligned(block_table, 4) || !aligned(ctx_lens, 4) || (LSE && !aligned(LSE, 4)) ||
        (prefix_len > 0 && (!aligned(Kprefix, 16) || !aligned(Vprefix, 16))))
        return ATTN_ERR_ALIGN;
    if (!workspace) return ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_ERR_ALIGN;
    if (workspace_bytes < attn::decode_workspace_bytes(B, Hq, d, S)) return ATTN_ERR_WORKSPACE;
    attn::DecodeArgs a{q, Kpages, Vpages, block_table, ctx_lens, O, LSE, B, Hq, Hkv, d,
                       page_size, max_pages_per_seq, split_tokens, dtype == ATTN_BF16, scale,
                       workspace, stream, Kprefix, Vprefix, prefix_len};
    return attn::launch_decode(a) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_prefill_paged(const void* q, const void* Kpages, const void* Vpages,
                                  const int* block_table, const int* cu_seqlens_q,
                                  const int* kv_lens, void* O, float* LSE, int B, int Hq,
                                  int Hkv, int d, int page_size, int max_pages_per_seq,
                                  int max_q_len, int causal, float scale, int dtype,
                                  void* stream) {
    if (!q || !Kpages || !Vpages || !block_table || !cu_seqlens_q || !kv_lens || !O)
        return ATTN_ERR_NULL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || page_size <= 0 || max_pages_per_seq <= 0 ||
        max_q_len < 0 || Hq % Hkv != 0)
        return ATTN_ERR_SHAPE;
    if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (page_size != 16) return ATTN_ERR_UNSUPPORTED;
    // one request's query rows are addressed with 32-bit byte offsets; the grid, the page
    // offsets within a request and the packed row indices stay in 32 bits
    if ((long long)max_q_len * Hq * d * 2 > (1LL << 30) ||
        (long long)max_pages_per_seq * page_size > 0x7fffffffLL ||
        (long long)B * Hkv > 0x7fffffffLL || (long long)Hkv * d * 2 * 16 > 0x7fffffffLL)
        return ATTN_ERR_SHAPE;
    const long long n_qtiles = ((long long)max_q_len * (Hq / Hkv) + 127) / 128;
    if (n_qtiles * B * Hkv > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(Kpages, 16) || !aligned(Vpages, 16) || !aligned(O, 16) ||
        !aligned(block_table, 4) || !aligned(cu_seqlens_q, 4) || !aligned(kv_lens, 4) ||
        (LSE && !aligned(LSE, 4)))
        return ATTN_ERR_ALIGN;
    if (max_q_len == 0) return ATTN_OK;   // no request has a new token: nothing to compute
    attn::PagedPrefillArgs a{q, Kpages, Vpages, block_table, cu_seqlens_q, kv_lens, O, LSE, B,
                             Hq, Hkv, d, max_pages_per_seq, max_q_len, causal != 0,
                             dtype == ATTN_BF16, scale, stream};
    return attn::launch_prefill_paged(a) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}
