/*
 * oracle.c -- plain fp64 CPU reference for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls this file;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * What it computes (each function cites the passage it follows):
 *
 *   oracle_attention     Standard attention, "Algorithm 0": materialise one full row of
 *                        scores s_j = scale * q.k_j, take the safe softmax of the whole row
 *                        (subtract the row max), then O = P V and LSE = m + ln(l).
 *                        [CS349D Lecture 4 notes, section 2 (standard attention) and 3.2
 *                        (safe softmax); zwjcode.cn FlashAttention blog, section 01;
 *                        LLM Internals 10.3.2, "LSE" paragraph for LSE = m + ln l]
 *                        Causal rows see keys j <= i [zwjcode blog section 06; AI-infra
 *                        handbook "FlashAttention and inference operators", causal masking].
 *                        GQA maps query head h to kv head h / (Hq/Hkv) [same handbook,
 *                        paged decode kernel].
 *   oracle_attention_variant  Standard attention with two of the variants a template engine
 *                        supports [CS349D Lecture 4 notes 5.4]: logits soft-cap, where each
 *                        scaled score s becomes c * tanh(s / c) before the softmax, and a
 *                        sliding window, where query i sees only its last w keys
 *                        (i - w < j <= i).  Otherwise as oracle_attention.
 *   oracle_decode_paged  One query per request over a paged KV cache: token t of request r
 *                        lives in physical page block_table[r][t / page] at slot t % page
 *                        [handbook, PagedAttention section; LLM Internals 10.3.7].  All ctx
 *                        tokens are visible.  The row itself is the same standard attention.
 *   oracle_prefill_paged A chunk of new queries per request over its paged KV cache: the
 *                        requests' queries are packed end to end, request r owning rows
 *                        cu_seqlens_q[r] .. cu_seqlens_q[r+1]-1 [LLM Internals 10.3.8,
 *                        variable-length batching]; its cache holds kv_lens[r] tokens, the
 *                        last q_len of them being the new tokens themselves [LLM Internals
 *                        10.3.7; CS349D Lecture 4 section 5.1, incremental prefill].  Causal:
 *                        new query i sits at position kv_len - q_len + i and sees the keys at
 *                        positions up to its own, so q_len = 1 is a decode step and
 *                        q_len = kv_len is ordinary causal prefill.
 *   oracle_online_row    FlashAttention-2 loop order for one row: tiles of Bc scores, running
 *                        max m, exp-sum l and unnormalised output O~, each rescaled by
 *                        e^(m_old - m_new), one division at the end, LSE = m + ln l
 *                        [LLM Internals 10.3.2 tiled forward pseudocode; handbook recurrence
 *                        for m^(j), l^(j), O^(j)].  Exposes the per-tile (m, l, O~) trace.
 *   oracle_merge         The attention-state merge: with LSE_s per part and normalised O_s,
 *                        LSE = ln sum_s e^{LSE_s}, O = sum_s e^{LSE_s - LSE} O_s; parts with
 *                        LSE_s = -inf (no keys) are skipped.  Parts are taken in ascending
 *                        order [LLM Internals 10.3.2 "LSE" paragraph; handbook split-K merge
 *                        formula and exercise 2; CS349D Lecture 4 section 4.3].
 *   oracle_widen16       The exact widening of a bf16 / fp16 pattern to fp64 that every other
 *                        function applies to its inputs.
 *
 * All arithmetic is IEEE fp64 in program order (build with -ffp-contract=off, no fast-math).
 * Inputs are the same 16-bit patterns the GPU receives (dtype 0 = bf16, 1 = fp16).
 * Reading taken where the pages are silent: a row with no visible key gets O = 0 and
 * LSE = -inf (the configurations never produce one).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_BF16 0
#define OR_FP16 1

/* ------------------------------------------------------------------ exact 16-bit widening */
double oracle_widen16(uint16_t bits, int dtype)
{
    if (dtype == OR_BF16) {
        uint32_t u = (uint32_t)bits << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    /* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1F;
    int frac = bits & 0x3FF;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);                  /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), expo - 25);   /* (1 + frac/1024) * 2^(expo-15) */
    return sign ? -mag : mag;
}

static void widen_row(const uint16_t* src, int n, int dtype, double* dst)
{
    for (int i = 0; i < n; ++i) dst[i] = oracle_widen16(src[i], dtype);
}

/* ------------------------------------------------------------------ one standard-attention row
 * q[d] (already fp64), keys/values given as row pointers into 16-bit storage.
 * scratch must hold n doubles.  P (optional) receives the n softmax probabilities.        */
static void attend_row(const double* q, const uint16_t* const* krows,
                       const uint16_t* const* vrows, int n, int d, int dtype, double scale,
                       double* s, double* kv_tmp, double* out, double* lse, double* P)
{
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return;
    }
    /* S row: s_j = scale * sum_k q_k K_jk */
    for (int j = 0; j < n; ++j) {
        widen_row(krows[j], d, dtype, kv_tmp);
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += q[k] * kv_tmp[k];
        s[j] = scale * acc;
    }
    /* safe softmax over the complete row */
    double m = s[0];
    for (int j = 1; j < n; ++j)
        if (s[j] > m) m = s[j];
    double l = 0.0;
    for (int j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int j = 0; j < n; ++j) s[j] = s[j] / l;   /* P_ij */
    if (P)
        for (int j = 0; j < n; ++j) P[j] = s[j];
    /* O = P V */
    for (int j = 0; j < n; ++j) {
        widen_row(vrows[j], d, dtype, kv_tmp);
        for (int c = 0; c < d; ++c) out[c] += s[j] * kv_tmp[c];
    }
    *lse = m + log(l);
}

/* ------------------------------------------------------------------ dense (prefill) attention
 * Q [B,Hq,N,d], K,V [B,Hkv,N,d] (16-bit patterns).  rows: flat indices r = (b*Hq + h)*N + i
 * to evaluate (NULL = all B*Hq*N rows, in order).  O [n_rows, d], LSE [n_rows] fp64.
 * P (optional, tiny cases only) [n_rows, N]: probabilities, 0 for masked keys.
 * Returns 0, or -1 on bad arguments / allocation failure.                                   */
int oracle_attention(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int B, int Hq,
                     int Hkv, int N, int d, int causal, double scale, int dtype,
                     const int64_t* rows, int64_t n_rows, double* O, double* LSE, double* P)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || Hq % Hkv) return -1;
    const int64_t total = (int64_t)B * Hq * N;
    if (!rows) n_rows = total;
    const int group = Hq / Hkv;
    int err = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
        double* q = (double*)malloc(sizeof(double) * (size_t)d);
        double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
        const uint16_t** kr = (const uint16_t**)malloc(sizeof(void*) * (size_t)N);
        const uint16_t** vr = (const uint16_t**)malloc(sizeof(void*) * (size_t)N);
        double* prow = P ? (double*)malloc(sizeof(double) * (size_t)N) : NULL;
        const int ok = s && q && tmp && kr && vr && (!P || prow);
        /* every thread takes part in the work-shared loop; a thread without buffers only
         * flags the failure */
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < n_rows; ++t) {
            {
                int64_t r = rows ? rows[t] : t;
                if (!ok || r < 0 || r >= total) {
#pragma omp atomic write
                    err = 1;
                    continue;
                }
                int i = (int)(r % N);
                int h = (int)((r / N) % Hq);
                int b = (int)(r / ((int64_t)N * Hq));
                int kvh = h / group;
                const uint16_t* kbase = K + ((int64_t)b * Hkv + kvh) * N * d;
                const uint16_t* vbase = V + ((int64_t)b * Hkv + kvh) * N * d;
                int n = causal ? i + 1 : N;   /* visible keys j <= i */
                for (int j = 0; j < n; ++j) {
                    kr[j] = kbase + (int64_t)j * d;
                    vr[j] = vbase + (int64_t)j * d;
                }
                widen_row(Q + r * d, d, dtype, q);
                attend_row(q, kr, vr, n, d, dtype, scale, s, tmp, O + t * d, LSE + t,
                           P ? prow : NULL);
                if (P) {
                    for (int j = 0; j < N; ++j) P[t * N + j] = j < n ? prow[j] : 0.0;
                }
            }
        }
        free(s); free(q); free(tmp); free(kr); free(vr); free(prow);
    }
    return err ? -1 : 0;
}

/* ------------------------------------------------------------------ attention variants
 * As oracle_attention (same layouts, rows, outputs), with
 *   window  > 0: query i sees keys max(0, i - window + 1) .. i (requires causal); 0 = off;
 *   softcap > 0: each scaled score s = scale * q.k becomes softcap * tanh(s / softcap)
 *                before the softmax (and so in LSE); 0 = off.
 * Returns 0, or -1 on bad arguments / allocation failure.                                   */
int oracle_attention_variant(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int B,
                             int Hq, int Hkv, int N, int d, int causal, int window,
                             double softcap, double scale, int dtype, const int64_t* rows,
                             int64_t n_rows, double* O, double* LSE)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || Hq % Hkv) return -1;
    if (window < 0 || (window > 0 && !causal) || softcap < 0.0) return -1;
    const int64_t total = (int64_t)B * Hq * N;
    if (!rows) n_rows = total;
    const int group = Hq / Hkv;
    int err = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
        double* q = (double*)malloc(sizeof(double) * (size_t)d);
        double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
        const int ok = s && q && tmp;
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < n_rows; ++t) {
            int64_t r = rows ? rows[t] : t;
            if (!ok || r < 0 || r >= total) {
#pragma omp atomic write
                err = 1;
                continue;
            }
            int i = (int)(r % N);
            int h = (int)((r / N) % Hq);
            int b = (int)(r / ((int64_t)N * Hq));
            int kvh = h / group;
            const uint16_t* kbase = K + ((int64_t)b * Hkv + kvh) * N * d;
            const uint16_t* vbase = V + ((int64_t)b * Hkv + kvh) * N * d;
            int hi = causal ? i + 1 : N;                            /* keys j < hi ...      */
            int lo = window > 0 && i - window + 1 > 0 ? i - window + 1 : 0;   /* ... j >= lo */
            int n = hi - lo;
            double* out = O + t * d;
            for (int c = 0; c < d; ++c) out[c] = 0.0;
            widen_row(Q + r * d, d, dtype, q);
            /* scores of the visible keys, soft-capped if asked */
            for (int j = 0; j < n; ++j) {
                widen_row(kbase + (int64_t)(lo + j) * d, d, dtype, tmp);
                double acc = 0.0;
                for (int k = 0; k < d; ++k) acc += q[k] * tmp[k];
                s[j] = scale * acc;
                if (softcap > 0.0) s[j] = softcap * tanh(s[j] / softcap);
            }
            /* safe softmax over the visible keys, then O = P V and LSE = m + ln l */
            double m = s[0];
            for (int j = 1; j < n; ++j)
                if (s[j] > m) m = s[j];
            double l = 0.0;
            for (int j = 0; j < n; ++j) {
                s[j] = exp(s[j] - m);
                l += s[j];
            }
            for (int j = 0; j < n; ++j) {
                widen_row(vbase + (int64_t)(lo + j) * d, d, dtype, tmp);
                for (int c = 0; c < d; ++c) out[c] += (s[j] / l) * tmp[c];
            }
            LSE[t] = m + log(l);
        }
        free(s); free(q); free(tmp);
    }
    return err ? -1 : 0;
}

/* ------------------------------------------------------------------ paged decode
 * q [B,Hq,d]; Kp,Vp [num_pages, page_size, Hkv, d]; block_table [B, max_pages] int32;
 * ctx_lens [B].  pairs: flat (r*Hq + h) to evaluate, NULL = all.  O [n, d], LSE [n].
 * Returns 0, -1 on bad arguments, -2 if a needed table entry is outside [0, num_pages).   */
int oracle_decode_paged(const uint16_t* q, const uint16_t* Kp, const uint16_t* Vp,
                        const int32_t* block_table, const int32_t* ctx_lens, int B, int Hq,
                        int Hkv, int d, int page_size, int max_pages, int64_t num_pages,
                        double scale, int dtype, const int64_t* pairs, int64_t n_pairs,
                        double* O, double* LSE)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || page_size <= 0 || Hq % Hkv) return -1;
    const int64_t total = (int64_t)B * Hq;
    if (!pairs) n_pairs = total;
    int max_ctx = 0;
    for (int r = 0; r < B; ++r) {
        if (ctx_lens[r] < 0 || ctx_lens[r] > (int64_t)max_pages * page_size) return -1;
        if (ctx_lens[r] > max_ctx) max_ctx = ctx_lens[r];
    }
    const int group = Hq / Hkv;
    int err = 0;
#pragma omp parallel
    {
        int cap = max_ctx > 0 ? max_ctx : 1;
        double* s = (double*)malloc(sizeof(double) * (size_t)cap);
        double* qq = (double*)malloc(sizeof(double) * (size_t)d);
        double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
        const uint16_t** kr = (const uint16_t**)malloc(sizeof(void*) * (size_t)cap);
        const uint16_t** vr = (const uint16_t**)malloc(sizeof(void*) * (size_t)cap);
        const int ok = s && qq && tmp && kr && vr;
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n_pairs; ++t) {
            {
                int64_t p = pairs ? pairs[t] : t;
                if (!ok || p < 0 || p >= total) {
#pragma omp atomic write
                    err = -1;
                    continue;
                }
                int r = (int)(p / Hq), h = (int)(p % Hq), kvh = h / group;
                int ctx = ctx_lens[r];
                int bad = 0;
                for (int tok = 0; tok < ctx; ++tok) {
                    int32_t page = block_table[(int64_t)r * max_pages + tok / page_size];
                    int slot = tok % page_size;
                    if (page < 0 || page >= num_pages) { bad = 1; break; }
                    int64_t off = (((int64_t)page * page_size + slot) * Hkv + kvh) * d;
                    kr[tok] = Kp + off;
                    vr[tok] = Vp + off;
                }
                if (bad) {
#pragma omp atomic write
                    err = -2;
                    continue;
                }
                widen_row(q + p * d, d, dtype, qq);
                attend_row(qq, kr, vr, ctx, d, dtype, scale, s, tmp, O + t * d, LSE + t, NULL);
            }
        }
        free(s); free(qq); free(tmp); free(kr); free(vr);
    }
    return err;
}

/* ------------------------------------------------------------------ shared-prefix (cascade) decode
 * [CS349D Lecture 4 notes, 4.4 and 5.3: requests that share a prefix attend to the prefix
 * keys followed by their own keys; the cascade form is one way to compute the same result.]
 * What is computed is its definition: for request r and query head h, standard attention of
 * q[r,h] over the key sequence prefix (tokens 0..P-1 of Kpre/Vpre [Hkv, P, d], head h/G)
 * followed by the request's own ctx_lens[r] tokens in the paged pool (as in
 * oracle_decode_paged).  Same arguments as oracle_decode_paged plus the prefix.
 * Returns 0, -1 on bad arguments, -2 if a needed table entry is outside [0, num_pages).     */
int oracle_decode_cascade(const uint16_t* q, const uint16_t* Kpre, const uint16_t* Vpre,
                          int prefix_len, const uint16_t* Kp, const uint16_t* Vp,
                          const int32_t* block_table, const int32_t* ctx_lens, int B, int Hq,
                          int Hkv, int d, int page_size, int max_pages, int64_t num_pages,
                          double scale, int dtype, const int64_t* pairs, int64_t n_pairs,
                          double* O, double* LSE)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || page_size <= 0 || Hq % Hkv) return -1;
    if (prefix_len < 0 || (prefix_len > 0 && (!Kpre || !Vpre))) return -1;
    const int64_t total = (int64_t)B * Hq;
    if (!pairs) n_pairs = total;
    int max_ctx = 0;
    for (int r = 0; r < B; ++r) {
        if (ctx_lens[r] < 0 || ctx_lens[r] > (int64_t)max_pages * page_size) return -1;
        if (ctx_lens[r] > max_ctx) max_ctx = ctx_lens[r];
    }
    const int group = Hq / Hkv;
    int err = 0;
#pragma omp parallel
    {
        int cap = prefix_len + max_ctx > 0 ? prefix_len + max_ctx : 1;
        double* s = (double*)malloc(sizeof(double) * (size_t)cap);
        double* qq = (double*)malloc(sizeof(double) * (size_t)d);
        double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
        const uint16_t** kr = (const uint16_t**)malloc(sizeof(void*) * (size_t)cap);
        const uint16_t** vr = (const uint16_t**)malloc(sizeof(void*) * (size_t)cap);
        const int ok = s && qq && tmp && kr && vr;
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n_pairs; ++t) {
            int64_t p = pairs ? pairs[t] : t;
            if (!ok || p < 0 || p >= total) {
#pragma omp atomic write
                err = -1;
                continue;
            }
            int r = (int)(p / Hq), h = (int)(p % Hq), kvh = h / group;
            int n = 0;
            /* the shared prefix first ... */
            for (int tok = 0; tok < prefix_len; ++tok, ++n) {
                int64_t off = ((int64_t)kvh * prefix_len + tok) * d;   /* prefix head kvh */
                kr[n] = Kpre + off;
                vr[n] = Vpre + off;
            }
            /* ... then the request's own tokens */
            int bad = 0;
            for (int tok = 0; tok < ctx_lens[r]; ++tok, ++n) {
                int32_t pg = block_table[(int64_t)r * max_pages + tok / page_size];
                int in_page = tok % page_size;
                if (pg < 0 || pg >= num_pages) { bad = 1; break; }
                int64_t off = (((int64_t)pg * page_size + in_page) * Hkv + kvh) * d;
                kr[n] = Kp + off;
                vr[n] = Vp + off;
            }
            if (bad) {
#pragma omp atomic write
                err = -2;
                continue;
            }
            widen_row(q + p * d, d, dtype, qq);
            attend_row(qq, kr, vr, n, d, dtype, scale, s, tmp, O + t * d, LSE + t, NULL);
        }
        free(s); free(qq); free(tmp); free(kr); free(vr);
    }
    return err;
}

/* ------------------------------------------------------------------ paged / varlen prefill
 * q [total_q, Hq, d]: the new queries of all requests, packed (cu_seqlens_q [B+1], rows of
 * request r are cu_seqlens_q[r] .. cu_seqlens_q[r+1]-1).  The pools and block_table are as in
 * oracle_decode_paged; kv_lens[r] counts the cached tokens of request r, including its
 * q_len new ones.  rows: flat indices (token * Hq + h) to evaluate (NULL = all
 * total_q * Hq).  Returns 0, -1 on bad arguments, -2 if a needed table entry is outside
 * [0, num_pages).                                                                          */
int oracle_prefill_paged(const uint16_t* q, const uint16_t* Kp, const uint16_t* Vp,
                         const int32_t* block_table, const int32_t* cu_seqlens_q,
                         const int32_t* kv_lens, int B, int Hq, int Hkv, int d, int page_size,
                         int max_pages, int64_t num_pages, int total_q, int causal,
                         double scale, int dtype, const int64_t* rows, int64_t n_rows,
                         double* O, double* LSE)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || page_size <= 0 || Hq % Hkv) return -1;
    if (total_q < 0 || cu_seqlens_q[0] != 0 || cu_seqlens_q[B] > total_q) return -1;
    int max_kv = 0;
    for (int r = 0; r < B; ++r) {
        if (cu_seqlens_q[r + 1] < cu_seqlens_q[r]) return -1;
        if (kv_lens[r] < 0 || kv_lens[r] > (int64_t)max_pages * page_size) return -1;
        if (kv_lens[r] > max_kv) max_kv = kv_lens[r];
    }
    const int64_t total = (int64_t)total_q * Hq;
    if (!rows) n_rows = total;
    const int group = Hq / Hkv;
    int err = 0;
#pragma omp parallel
    {
        int cap = max_kv > 0 ? max_kv : 1;
        double* s = (double*)malloc(sizeof(double) * (size_t)cap);
        double* qq = (double*)malloc(sizeof(double) * (size_t)d);
        double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
        const uint16_t** kr = (const uint16_t**)malloc(sizeof(void*) * (size_t)cap);
        const uint16_t** vr = (const uint16_t**)malloc(sizeof(void*) * (size_t)cap);
        const int ok = s && qq && tmp && kr && vr;
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n_rows; ++t) {
            int64_t p = rows ? rows[t] : t;
            int tok = (int)(p / Hq), h = (int)(p % Hq);
            int r = -1;
            if (ok && p >= 0 && p < total)
                for (int k = 0; k < B; ++k)
                    if (cu_seqlens_q[k] <= tok && tok < cu_seqlens_q[k + 1]) { r = k; break; }
            if (r < 0) {     /* a padding row past the last request, or a bad index */
#pragma omp atomic write
                err = -1;
                continue;
            }
            int kvh = h / group;
            int q_len = cu_seqlens_q[r + 1] - cu_seqlens_q[r];
            int i = tok - cu_seqlens_q[r];
            int kv_len = kv_lens[r];
            /* keys visible to new query i: positions 0 .. kv_len - q_len + i (causal) */
            int n = kv_len;
            if (causal) {
                int last = kv_len - q_len + i;
                n = last + 1 < 0 ? 0 : (last + 1 < kv_len ? last + 1 : kv_len);
            }
            int bad = 0;
            for (int key = 0; key < n; ++key) {
                int32_t pg = block_table[(int64_t)r * max_pages + key / page_size];
                int in_page = key % page_size;
                if (pg < 0 || pg >= num_pages) { bad = 1; break; }
                int64_t off = (((int64_t)pg * page_size + in_page) * Hkv + kvh) * d;
                kr[key] = Kp + off;
                vr[key] = Vp + off;
            }
            if (bad) {
#pragma omp atomic write
                err = -2;
                continue;
            }
            widen_row(q + p * d, d, dtype, qq);
            attend_row(qq, kr, vr, n, d, dtype, scale, s, tmp, O + t * d, LSE + t, NULL);
        }
        free(s); free(qq); free(tmp); free(kr); free(vr);
    }
    return err;
}

/* ------------------------------------------------------------------ online softmax, one row
 * s[n] scores (already scaled), v[n, dv] values, tiles of bc scores in order.
 * Outputs O[dv] = O~/l, *m_out, *l_out, *lse_out.  Optional trace arrays, one entry per tile
 * (ceil(n/bc) of them): tm[t], tl[t], tacc[t*dv + c] = state after tile t.                */
int oracle_online_row(const double* s, const double* v, int n, int dv, int bc, double* O,
                      double* m_out, double* l_out, double* lse_out, double* tm, double* tl,
                      double* tacc)
{
    if (n < 0 || dv <= 0 || bc <= 0) return -1;
    double m = -INFINITY, l = 0.0;
    double* acc = (double*)calloc((size_t)dv, sizeof(double));
    if (!acc) return -1;
    int tile = 0;
    for (int j0 = 0; j0 < n; j0 += bc, ++tile) {
        int j1 = j0 + bc < n ? j0 + bc : n;
        double mb = -INFINITY;                       /* rowmax of this tile */
        for (int j = j0; j < j1; ++j)
            if (s[j] > mb) mb = s[j];
        double m_new = m > mb ? m : mb;
        double corr = (m == -INFINITY) ? 0.0 : exp(m - m_new);   /* e^(m_old - m_new) */
        double rowsum = 0.0;
        for (int c = 0; c < dv; ++c) acc[c] *= corr;
        for (int j = j0; j < j1; ++j) {
            double p = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m_new);
            rowsum += p;
            for (int c = 0; c < dv; ++c) acc[c] += p * v[(int64_t)j * dv + c];
        }
        l = l * corr + rowsum;
        m = m_new;
        if (tm) tm[tile] = m;
        if (tl) tl[tile] = l;
        if (tacc)
            for (int c = 0; c < dv; ++c) tacc[(int64_t)tile * dv + c] = acc[c];
    }
    for (int c = 0; c < dv; ++c) O[c] = (l > 0.0) ? acc[c] / l : 0.0;
    if (m_out) *m_out = m;
    if (l_out) *l_out = l;
    if (lse_out) *lse_out = (l > 0.0) ? m + log(l) : -INFINITY;
    free(acc);
    return 0;
}

/* ------------------------------------------------------------------ attention-state merge
 * O_s [S, dv] normalised part outputs, lse_s [S]; parts merged in ascending s.            */
int oracle_merge(const double* O_s, const double* lse_s, int S, int dv, double* O,
                 double* lse_out)
{
    if (S < 0 || dv <= 0) return -1;
    double M = -INFINITY;
    for (int s = 0; s < S; ++s)
        if (lse_s[s] > M) M = lse_s[s];
    for (int c = 0; c < dv; ++c) O[c] = 0.0;
    if (M == -INFINITY) {
        *lse_out = -INFINITY;
        return 0;
    }
    double wsum = 0.0;
    for (int s = 0; s < S; ++s) {
        if (lse_s[s] == -INFINITY) continue;     /* empty part: weight 0, skipped */
        double w = exp(lse_s[s] - M);
        wsum += w;
        for (int c = 0; c < dv; ++c) O[c] += w * O_s[(int64_t)s * dv + c];
    }
    for (int c = 0; c < dv; ++c) O[c] /= wsum;
    *lse_out = M + log(wsum);
    return 0;
}

/* ------------------------------------------------------------------ thread control */
int oracle_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
