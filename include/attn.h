/*
 * attn.h -- C ABI of the MI355X (gfx950) exact-attention library (libattn.so).
 *
 * Two compute calls follow the problem statement of the pages (two more serve requests that
 * share a prefix and chunks of new tokens over a paged cache):
 *   attn_fwd           exact scaled-dot-product attention forward (prefill), computed as a
 *                      tiled, fused kernel with online softmax: Q row-blocks stay on chip
 *                      while K/V column-blocks stream past, fully masked causal blocks are
 *                      skipped, and only O and the per-row LSE are written.
 *                      [LLM Internals 10.3.2, tiled forward in FlashAttention-2 loop order,
 *                      with "write back O_i = O~/l, LSE_i = m + ln l"; CS349D Lecture 4
 *                      notes 3.2-3.3; zwjcode.cn FlashAttention blog sections 02-06]
 *   attn_decode_paged  one query token per sequence against a paged KV cache, split along
 *                      the keys (Flash-Decoding / split-KV); each split writes a partial
 *                      state and the splits are merged with the LSE rule.
 *                      [CS349D Lecture 4 notes 4.2-4.3; LLM Internals 10.3.7; AI-infra
 *                      handbook "FlashAttention and inference operators", Flash-Decoding
 *                      split-K merge and the paged GQA decode kernel]
 *   attn_decode_cascade  decode for requests that share a prefix: the prefix is read once for
 *                      all of them, then merged with each request's own tokens by the LSE
 *                      rule [CS349D Lecture 4 notes 4.4, 5.3]
 *   attn_fwd_variant   attn_fwd with a causal sliding window and/or logits soft-cap
 *                      [CS349D Lecture 4 notes 5.4, attention variants]
 *   attn_prefill_paged  prefill of a chunk of new tokens per request over its paged KV
 *                      cache, requests packed end to end by cumulative lengths
 *                      [LLM Internals 10.3.8 variable-length batching, 10.3.7 block table;
 *                      CS349D Lecture 4 notes 5.1, incremental prefill]
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees, copies to the host or synchronises.  Work is enqueued on `stream`
 *     (a hipStream_t; NULL = the null stream) and is asynchronous: read results only after
 *     synchronising that stream.
 *   - Every argument is validated on the host before any HIP call; on error nothing is
 *     launched and nothing is written.  There is no fallback path: an unsupported input is
 *     an error, never a silent switch to slower code.
 *   - Device-resident block tables and context lengths are not read on the host and are
 *     not validated (see attn_decode_paged).
 *   - Results are bitwise deterministic for fixed inputs, shapes and split size: all
 *     reductions run in a fixed order.  (The decode's work queue takes tickets with an
 *     atomic counter; that decides only which workgroup computes an item, not how.)
 *   - The library is stateless (attn_decode_paged_noalloc excepted, by design: it keeps a
 *     fixed device buffer per GPU): it keeps no host state and no device state between calls.
 *     Everything a decode call needs beyond its inputs and outputs (partial states and the
 *     work-queue counters of its persistent grid) lives in the caller's workspace, so a call
 *     captured in a HIP graph touches only the buffers it was captured with.  Calls may be
 *     made from several host threads on different streams; calls that are in flight at the
 *     same time must not share a workspace.
 */
#ifndef EXACT_ATTENTION_ATTN_H
#define EXACT_ATTENTION_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (return values). */
enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,        /* a required pointer is NULL                                  */
    ATTN_ERR_SHAPE = -2,       /* a size is <= 0, Hq % Hkv != 0, sizes overflow, or scale is   */
                               /* not a finite positive number                                */
    ATTN_ERR_DTYPE = -3,       /* dtype is neither ATTN_BF16 nor ATTN_FP16                     */
    ATTN_ERR_UNSUPPORTED = -4, /* valid attention, but not built here: d not in {64, 128},     */
                               /* page_size != 16, split_tokens not 0 or a positive multiple  */
                               /* of page_size                                                 */
    ATTN_ERR_ALIGN = -5,       /* a tensor pointer is not 16-byte aligned                      */
    ATTN_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than the helper's size             */
    ATTN_ERR_HIP = -7,         /* the HIP runtime reported an error at launch                  */
    ATTN_ERR_TOO_LARGE = -8    /* attn_decode_paged_noalloc: the call needs more scratch than  */
                               /* the library's fixed buffer holds                             */
};

/* Element type of Q, K, V, O (and q, K/V pages, O for decode). */
enum attn_dtype { ATTN_BF16 = 0, ATTN_FP16 = 1 };

/*
 * attn_fwd -- prefill / full attention forward.
 *
 *   Q   [B, Hq,  N, d]  dtype, contiguous          (read)
 *   K   [B, Hkv, N, d]  dtype, contiguous          (read)
 *   V   [B, Hkv, N, d]  dtype, contiguous          (read)
 *   O   [B, Hq,  N, d]  dtype, contiguous          (written)
 *   LSE [B, Hq,  N]     float32                     (written; natural log of the row's
 *                        sum of exp(scale * q.k) over its visible keys)
 *
 *   O[b,h,i,:] = sum_j softmax_j(scale * Q[b,h,i,:].K[b,kvh,j,:]) V[b,kvh,j,:]
 *   with kvh = h / (Hq / Hkv) (query-head groups are contiguous) and, when causal != 0,
 *   only keys j <= i visible.  Scores, statistics and accumulation are fp32; the
 *   probabilities feeding the second product are rounded to dtype (round-to-nearest-even),
 *   as is O.
 *
 *   Supported: d in {64, 128}; dtype bf16 or fp16; N >= 1 with N * d * 2 <= 2^30 bytes per
 *   head (N <= 4194304 at d = 128); B >= 1, Hq % Hkv == 0; scale finite and > 0.  All five
 *   pointers must be 16-byte aligned.
 *   Returns ATTN_OK or a negative attn_status.
 */
int attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
             int B, int Hq, int Hkv, int N, int d, int causal, float scale,
             int dtype, void* stream);

/*
 * attn_fwd_variant -- attn_fwd with two attention variants [CS349D Lecture 4 notes 5.4]:
 *   window  > 0: sliding window (causal only): query i sees keys j with i - window < j <= i;
 *                0 = off
 *   softcap > 0: logits soft-cap: each scaled score s = scale * q.k becomes
 *                softcap * tanh(s / softcap) before the softmax (and in LSE); 0 = off
 * Both off is exactly attn_fwd.  Arguments, layouts and the rest as attn_fwd.
 *
 *   Supported: as attn_fwd; window > 0 requires causal (else ATTN_ERR_UNSUPPORTED);
 *   window < 0 or softcap < 0 or not finite is ATTN_ERR_SHAPE.  Returns ATTN_OK or a
 *   negative attn_status.
 */
int attn_fwd_variant(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     int B, int Hq, int Hkv, int N, int d, int causal, int window,
                     float softcap, float scale, int dtype, void* stream);

/*
 * attn_prefill_paged -- prefill of new tokens over a paged KV cache (chunked prefill)
 * [LLM Internals 10.3.8: sequences packed end to end with cumulative lengths; 10.3.7: the
 * block table and the [blocks, page, Hkv, d] cache; CS349D Lecture 4 notes 5.1: incremental
 * prefill, where each request brings a different number of new queries and KV length].
 * Request r brings q_len = cu_seqlens_q[r+1] - cu_seqlens_q[r] new tokens, whose queries
 * are rows cu_seqlens_q[r] .. cu_seqlens_q[r+1]-1 of q.  Its cache already holds kv_lens[r]
 * tokens, the new ones last (written there before the call), so new query i sits at
 * position kv_lens[r] - q_len + i.  With causal set it sees the keys at positions up to
 * its own (q_len = 1 is a decode step, q_len = kv_len ordinary causal prefill); without,
 * all kv_lens[r] keys.  A query that sees no key (kv_lens[r] < q_len) gets O = 0 and
 * LSE = -inf.
 *
 *   q             [total_q, Hq, d]   dtype, packed queries                     (read)
 *   Kpages,       [num_pages, page_size, Hkv, d]  dtype                       (read)
 *   Vpages
 *   block_table   [B, max_pages_per_seq] int32: physical page of each 16-token block of a
 *                 request's cache                                              (read)
 *   cu_seqlens_q  [B + 1] int32, cu_seqlens_q[0] = 0, non-decreasing          (read)
 *   kv_lens       [B] int32, cached tokens per request (new ones included)     (read)
 *   O             [total_q, Hq, d]   dtype; rows of requests are written, other rows are
 *                 left untouched                                               (write)
 *   LSE           [total_q, Hq] fp32, natural log, or NULL                     (write)
 *   max_q_len     host-side bound on every request's q_len; 0 launches nothing
 *   causal, scale, dtype, stream  as in attn_fwd
 *
 *   Supported: d in {64, 128}; page_size 16; max_q_len * Hq * d * 2 <= 2^30.  Device data
 *   are not validated: the caller guarantees cu_seqlens_q[B] <= total_q, q_len <= max_q_len,
 *   kv_lens[r] <= max_pages_per_seq * 16 and valid page indices for the pages a request's
 *   cache uses.  (Out-of-range lengths are clamped to those bounds; entries of unused
 *   pages, e.g. -1, are never read.)  Returns ATTN_OK or a negative attn_status.
 */
int attn_prefill_paged(const void* q, const void* Kpages, const void* Vpages,
                       const int* block_table, const int* cu_seqlens_q, const int* kv_lens,
                       void* O, float* LSE, int B, int Hq, int Hkv, int d, int page_size,
                       int max_pages_per_seq, int max_q_len, int causal, float scale, int dtype,
                       void* stream);

/*
 * attn_decode_paged -- one query token per sequence over a paged KV cache, split-KV.
 *
 *   q            [B, Hq, d]                         dtype          (read)
 *   Kpages       [num_pages, page_size, Hkv, d]     dtype          (read)
 *   Vpages       [num_pages, page_size, Hkv, d]     dtype          (read)
 *   block_table  [B, max_pages_per_seq]             int32, device  (read)
 *   ctx_lens     [B]                                int32, device  (read)
 *   O            [B, Hq, d]                         dtype          (written)
 *   LSE          [B, Hq] float32, or NULL            (written when not NULL)
 *   workspace    >= attn_decode_paged_workspace_bytes(...) bytes, 16-byte aligned,
 *                device memory owned by the caller: a 256-byte control block holding the
 *                call's work-queue counters, then the per-split partial states.  The control
 *                block (the first 256 bytes) must be zero before the first call that uses
 *                the workspace (zero-fill it once after allocating it: hipMemset, or a fill
 *                kernel); every call leaves it ready for the next call, whatever its split,
 *                so later calls need no reset.  A workspace serves one call at a time.
 *
 *   Token t of sequence r is slot t % page_size of physical page block_table[r][t /
 *   page_size]; kv head kvh = h / (Hq / Hkv).  All ctx_lens[r] tokens are visible.  The
 *   keys are cut into splits of split_tokens tokens starting at token 0; each split yields
 *   a partial (O_s normalised, LSE_s), and the splits of a sequence are merged in
 *   ascending order: LSE = ln sum_s e^{LSE_s}, O = sum_s e^{LSE_s - LSE} O_s.
 *   A sequence with ctx_lens[r] == 0 gets O = 0 and LSE = -inf.
 *
 *   split_tokens == 0 chooses the split on the device, balanced for the batch [CS349D
 *   Lecture 4 notes 5.6: the chunk length follows from the batch's total work over the
 *   workers]: with T = Hkv * sum(ctx_lens) and P = T / (compute units), the split is 256,
 *   512, 1024 or 2048 tokens for P up to 128, 3072, 10240 and beyond.  The choice is made
 *   from the device-resident lengths at run time, so a call captured in a HIP graph stays
 *   valid (and balanced) when the lengths change between replays.  Results are bitwise
 *   equal to a call with that split given explicitly.  The workspace helper sizes the
 *   workspace for the shortest (256-token) split when given split_tokens == 0.
 *
 *   Caller preconditions (device data, not checked): 0 <= ctx_lens[r] <=
 *   max_pages_per_seq * page_size, and every block_table entry a sequence uses
 *   (index < ceil(ctx/page_size)) is a valid page in [0, num_pages).  Entries past that are
 *   never read and may hold anything (e.g. -1).
 *
 *   Supported: d in {64, 128}; page_size == 16; split_tokens 0 (balanced) or a positive
 *   multiple of page_size; dtype bf16 or fp16; Hq % Hkv == 0 with Hq / Hkv <= 16.  q, Kpages, Vpages,
 *   O and workspace must be 16-byte aligned; block_table, ctx_lens and LSE 4-byte aligned.
 *   Returns ATTN_OK or a negative attn_status.
 */
int attn_decode_paged(const void* q, const void* Kpages, const void* Vpages,
                      const int* block_table, const int* ctx_lens, void* O, float* LSE,
                      int B, int Hq, int Hkv, int d, int page_size, int max_pages_per_seq,
                      int split_tokens, float scale, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_workspace_bytes -- host-only helper: the workspace attn_decode_paged
 * needs for these sizes (partial outputs and LSEs of every split of every (sequence,
 * head), after the 256-byte control block).  Returns 0 when the sizes are invalid.  Makes
 * no HIP call.
 */
size_t attn_decode_paged_workspace_bytes(int B, int Hq, int d, int page_size,
                                         int max_pages_per_seq, int split_tokens);

/*
 * attn_decode_paged_noalloc -- attn_decode_paged for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace and allocates nothing (no hipMalloc, no allocating
 * library routine): the partial states and the work-queue counters live in a fixed device
 * buffer of ATTN_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until
 * the process ends.  Arguments, results and errors as attn_decode_paged; same kernels, so
 * the output is bitwise equal to attn_decode_paged's for the same inputs and split.
 *
 *   Limit: the call's partial states, sized as attn_decode_paged_workspace_bytes(B, Hq, d,
 *   page_size, max_pages_per_seq, split_tokens) reports, must fit the buffer; a larger call
 *   is rejected with ATTN_ERR_TOO_LARGE before anything is launched.  (The 64-sequence,
 *   32-head, d = 128 batch with up to 2048 pages per sequence fits with 1024-token splits,
 *   not with the balanced split, which is sized for 256-token splits.)
 *   The first call on a device looks up the buffer's address (hipGetSymbolAddress) and
 *   enqueues a small kernel that clears its control block; every call leaves the block
 *   ready for the next.  All calls on one GPU share the buffer: calls that overlap in time
 *   on one GPU (different streams, or graphs replayed concurrently) race and give wrong
 *   results.  Serialise them, or use attn_decode_paged with a workspace per stream.
 *   The stream must belong to the device the data live on.  Returns ATTN_OK or a negative
 *   attn_status.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int attn_decode_paged_noalloc(const void* q, const void* Kpages, const void* Vpages,
                              const int* block_table, const int* ctx_lens, void* O, float* LSE,
                              int B, int Hq, int Hkv, int d, int page_size,
                              int max_pages_per_seq, int split_tokens, float scale, int dtype,
                              void* stream);

/*
 * attn_decode_cascade -- shared-prefix (cascade) decode [CS349D Lecture 4 notes, 4.4 and
 * 5.3]: every request r attends to the same prefix of prefix_len tokens followed by its own
 * ctx_lens[r] tokens in the paged pool; the result is standard attention over that key
 * sequence, computed as (a) the queries of all requests against the prefix, which is read
 * once, as matrix-matrix products in chunks of prefix keys, (b) each request's own tokens as
 * in attn_decode_paged, and (c) one merge of all partial states with the LSE rule in key
 * order (prefix chunks, then splits).
 *
 *   q          [B, Hq, d]               the query of each request, one token
 *   Kprefix,   [Hkv, prefix_len, d]     the shared prefix, head-major (as attn_fwd takes K
 *   Vprefix                              and V for one sequence); may be NULL if prefix_len
 *                                        is 0
 *   prefix_len >= 0 tokens; 0 makes the call equal to attn_decode_paged
 *   Kpages, Vpages, block_table, ctx_lens, O, LSE, sizes, split_tokens, scale, dtype,
 *   workspace, stream: as in attn_decode_paged (ctx_lens counts only a request's own
 *   tokens).  A request with no keys at all gets O = 0 and LSE = -inf.
 *   workspace  at least attn_decode_cascade_workspace_bytes(...) bytes; zero-filled once
 *              after allocation, one call at a time, as in attn_decode_paged
 *
 *   Supported: as attn_decode_paged; also B * Hq * d * 2 and prefix_len * d * 2 must not
 *   exceed 2^30 (32-bit addressing of q and of one prefix head).  Returns ATTN_OK or a
 *   negative attn_status.
 */
int attn_decode_cascade(const void* q, const void* Kprefix, const void* Vprefix, int prefix_len,
                        const void* Kpages, const void* Vpages, const int* block_table,
                        const int* ctx_lens, void* O, float* LSE, int B, int Hq, int Hkv, int d,
                        int page_size, int max_pages_per_seq, int split_tokens, float scale,
                        int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_cascade_workspace_bytes -- host-only helper: the workspace attn_decode_cascade
 * needs (the partial states of every split and every prefix chunk of every (request, head),
 * after the 256-byte control block).  Returns 0 when the sizes are invalid.  Makes no HIP
 * call.
 */
size_t attn_decode_cascade_workspace_bytes(int B, int Hq, int d, int page_size,
                                           int max_pages_per_seq, int split_tokens,
                                           int prefix_len);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ATTN_H */
