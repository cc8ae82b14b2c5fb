// attn_internal.h -- launcher interface between the C ABI shim and the kernels.
// Arguments reaching these launchers have already been validated by the shim.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace attn {

struct PrefillArgs {
    const void* Q;
    const void* K;
    const void* V;
    void* O;
    float* LSE;
    int B, Hq, Hkv, N, d;
    bool causal, is_bf16;
    float scale;
    void* stream;
};

struct DecodeArgs {
    const void* q;
    const void* Kpages;
    const void* Vpages;
    const int* block_table;
    const int* ctx_lens;
    void* O;
    float* LSE;  // may be null
    int B, Hq, Hkv, d, page_size, max_pages, split_tokens;
    bool is_bf16;
    float scale;
    void* workspace;
    void* stream;
    // shared prefix (cascade decode): K/V [Hkv, prefix_len, d]; prefix_len 0 = none
    const void* Kprefix = nullptr;
    const void* Vprefix = nullptr;
    int prefix_len = 0;
};

// The prefix part of a cascade decode: partial states of every (request, query head) for
// each chunk of the shared prefix, written at split index s_base + chunk of the partial
// buffers (s_stride states per pair).
struct CascadePrefixArgs {
    const void* q;
    const void* Kprefix;
    const void* Vprefix;
    float* ws_o;
    float* ws_lse;
    int B, Hq, Hkv, d, prefix_len, chunk, n_chunks, s_stride, s_base;
    bool is_bf16;
    float scale;
    void* stream;
};

// Paged / varlen prefill: q [total_q, Hq, d] packed by cu_seqlens_q [B + 1], page pools
// [pages, 16, Hkv, d], block_table [B, max_pages], kv_lens [B] (cached tokens, new ones
// included), O [total_q, Hq, d], LSE [total_q, Hq] or null.
struct PagedPrefillArgs {
    const void* q;
    const void* Kpages;
    const void* Vpages;
    const int* block_table;
    const int* cu_seqlens_q;
    const int* kv_lens;
    void* O;
    float* LSE;
    int B, Hq, Hkv, d, max_pages, max_q_len;
    bool causal, is_bf16;
    float scale;
    void* stream;
};

// Launch through hipLaunchKernel so the status reflects this launch only (a sticky error
// left by some earlier, unrelated HIP call must not be reported as ours).  With
// ATTN_DEBUG set in the environment a failing launch prints the runtime's message.
hipError_t report_launch(hipError_t e, const char* what);

template <typename... KArgs>
hipError_t launch_exact(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                        const char* what, KArgs... args) {
    void* ptrs[] = {static_cast<void*>(&args)...};
    return report_launch(hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs,
                                         0, st),
                         what);
}

// Converts every argument to the kernel's exact parameter type before taking its address.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                         const char* what, Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    return launch_exact<KArgs...>(kern, grid, block, st, what, static_cast<KArgs>(args)...);
}

// Compute units of the current device (queried once per device, then cached).
int device_cu_count();

// Host-side checks of a paged decode call (all arguments but the workspace); returns an
// attn_status and, on success, the partial states per (sequence, head) in *S_out.
int check_decode_args(const void* q, const void* Kpages, const void* Vpages,
                      const int* block_table, const int* ctx_lens, const void* O,
                      const float* LSE, int B, int Hq, int Hkv, int d, int page_size,
                      int max_pages_per_seq, int split_tokens, float scale, int dtype,
                      long long* S_out);

hipError_t launch_prefill(const PrefillArgs& a);
// head size 128, long sequences: the 64-rows-per-wave kernel (attn_fwd_d128.hip), whose
// results equal those of the 32-rows-per-wave prefill kernel bit for bit
bool prefill_d128_applies(const PrefillArgs& a);
hipError_t launch_prefill_d128(const PrefillArgs& a);
hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_cascade_prefix(const CascadePrefixArgs& a);
hipError_t launch_prefill_paged(const PagedPrefillArgs& a);
// dense attention with a causal sliding window (window > 0) and/or logits soft-cap
// (softcap > 0); both off is plain launch_prefill
hipError_t launch_prefill_variant(const PrefillArgs& a, int window, float softcap);

// Prefix keys per partial state in a cascade decode.
constexpr int kCascadeChunk = 512;
inline long long cascade_chunks(int prefix_len) {
    return ((long long)prefix_len + kCascadeChunk - 1) / kCascadeChunk;
}

// Shortest split the device-side balanced choice (split_tokens == 0) can pick.
constexpr int kMinBalancedSplit = 256;

// Number of splits per sequence the workspace is sized for.
inline long long decode_max_splits(int page_size, int max_pages, int split_tokens) {
    const long long max_tokens = (long long)max_pages * page_size;
    const long long len = split_tokens > 0 ? split_tokens : kMinBalancedSplit;
    return (max_tokens + len - 1) / len;
}

// Workspace layout: the call's control block (work-queue counters, 256 bytes) first, at a
// fixed place whatever the split, then O partials [B][Hq][S][d] fp32, then LSE partials
// [B][Hq][S] fp32 (padded to 256 bytes).
constexpr size_t kDecodeCtrlBytes = 256;
inline size_t decode_workspace_bytes(int B, int Hq, int d, long long S) {
    const size_t o = (size_t)B * Hq * (size_t)S * d * sizeof(float);
    const size_t l = (size_t)B * Hq * (size_t)S * sizeof(float);
    return kDecodeCtrlBytes + o + ((l + 255) / 256) * 256;
}

}  // namespace attn
