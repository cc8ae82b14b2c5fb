// attn_decode.hip -- paged split-KV decode for gfx950.
//
// Method [CS349D Lecture 4 notes 4.1-4.3; LLM Internals 10.3.7; AI-infra handbook
// "FlashAttention and inference operators", Flash-Decoding / split-K and the paged GQA
// decode kernel with its four listed improvements]:
//   * one query token per sequence; the keys are cut into splits of split_tokens tokens;
//   * one work item per (sequence, kv head, split) serves all G = Hq/Hkv query heads of
//     that kv head, so each K/V byte is read from HBM once;
//   * token t lives in slot t % 16 of physical page block_table[r][t / 16];
//   * inside a split the running (m, l, O~) online softmax is used (no score buffer);
//   * each split writes its normalised O_s and LSE_s; a second kernel merges the splits
//     of a sequence in ascending order with LSE = ln sum e^{LSE_s},
//     O = sum e^{LSE_s - LSE} O_s.
//
// MI355X mapping:
//   * A fixed grid of 2 workgroups per CU walks the list of non-empty work items (the list
//     is derived on the fly from ctx_lens), so no workgroup is launched for a split past a
//     sequence's context.
//   * The G query heads are the columns of v_mfma_f32_16x16x32 (G <= 16), the 16 slots of
//     a page its rows: S^T = K Q^T runs on the matrix cores with K loaded from HBM straight
//     into the A operand.  The exponentiated scores of a page are exactly the B operand of
//     O^T = V^T P^T on v_mfma_f32_16x16x16, so P stays in registers.
//   * V is transposed through a small per-wave LDS slab (d-major); slots at or past the
//     context length are written as zeros, so poisoned slots never reach the sum.
//   * Each page is addressed through a buffer descriptor (page base in SGPRs, one VGPR of
//     per-lane offset); block-table entries are scalar loads.  Each wave keeps two pages in
//     flight ahead of the one it computes.
//   * The 4 waves of a workgroup take every 4th page of the item; their states are merged
//     through LDS at the end of the item.
#include <algorithm>

#include "attn_common.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kPage = 16;
constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;

template <int D, bool IS_BF16>
__global__ __launch_bounds__(kDecThreads, 2) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kp,
    const uint16_t* __restrict__ Vp, const int* __restrict__ block_table,
    const int* __restrict__ ctx_lens, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    int B, int Hq, int Hkv, int max_pages, int split_tokens, int S_max, float scale_log2) {
    using E = Elem<IS_BF16>;
    constexpr int NKS = D / 32;          // k-steps of S^T = K Q^T (32 dims each)
    constexpr int NDB = D / 16;          // 16-row d blocks of O^T
    constexpr int VSTR = 16 + 8;         // LDS row stride of a wave's V^T slab (elements)
    constexpr int KCH = D / 8;           // 16-byte chunks per K/V row
    static_assert(4 * KCH <= 64, "a page's V must fit one 4-slot unit per lane");
    constexpr int SLAB = D * VSTR;       // elements per wave slab
    constexpr int LDS_BYTES_V = kDecWaves * SLAB * 2;
    constexpr int LDS_BYTES_MERGE = kDecWaves * 16 * (D + 2) * 4;
    constexpr int LDS_BYTES = LDS_BYTES_V > LDS_BYTES_MERGE ? LDS_BYTES_V : LDS_BYTES_MERGE;
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int l16 = lane & 15;
    const int g4 = lane >> 4;                      // k-group of the 16-row MFMA operands
    const int G = Hq / Hkv;
    const int64_t row_stride = (int64_t)Hkv * D;   // elements between consecutive slots
    const int page_bytes = kPage * (int)row_stride * 2;
    const int slot_bytes = (int)row_stride * 2;
    uint16_t* slab = reinterpret_cast<uint16_t*>(lds) + wave * SLAB;

    // per-lane offsets inside a page (bytes): K as the A operand (slot l16, dims 8*g4 +
    // 32ks..), V as 4-slot units (slots 4*v_tg + e, dims 8*v_dc..+7; for d = 64 the upper
    // half of the wave repeats the lower half)
    const int vofs_k = (l16 * (int)row_stride + g4 * 8) * 2;
    const int v_tg = lane & 3;
    const int v_dc = (lane >> 2) & (KCH - 1);
    const int vofs_v = (4 * v_tg * (int)row_stride + v_dc * 8) * 2;

    // Work list.  The non-empty items (sequence r, split s, kv head) are numbered
    // f = t * Hkv + kvh, where t runs over the splits of sequence 0, then of sequence 1, ...
    // (ceil(ctx_r / split_tokens) splits each).  Workgroup b takes items b, b + gridDim.x,
    // ...; the loop ends for every wave once f passes the item count, so the grid always
    // drains.  Each wave derives the count and its item's (r, s) from ctx_lens with
    // wave-wide prefix sums over chunks of 64 sequences (all results are wave-uniform).
    auto n_split_of = [&](int rr) {
        return rr < B ? (ctx_lens[rr] + split_tokens - 1) / split_tokens : 0;
    };
    auto incl_scan = [&](int v) {
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_up(v, off, 64);
            v += (lane >= off) ? u : 0;
        }
        return v;
    };
    int total_splits = 0;
    for (int c0 = 0; c0 < B; c0 += 64) total_splits += __shfl(incl_scan(n_split_of(c0 + lane)), 63, 64);
    const int n_items = __builtin_amdgcn_readfirstlane(total_splits) * Hkv;

    for (int f = blockIdx.x; f < n_items; f += gridDim.x) {
        const int t_item = f / Hkv;
        const int kvh = f % Hkv;
        int r = 0, split = 0;
        {
            int base = 0;
            for (int c0 = 0; c0 < B; c0 += 64) {
                const int n = n_split_of(c0 + lane);
                const int inc = incl_scan(n);
                const int tot = __shfl(inc, 63, 64);
                if (t_item < base + tot) {
                    const int exc = base + inc - n;
                    const unsigned long long hit =
                        __ballot(n > 0 && exc <= t_item && t_item < base + inc);
                    const int lr = __builtin_ctzll(hit);
                    r = c0 + lr;
                    split = t_item - __shfl(exc, lr, 64);
                    break;
                }
                base += tot;
            }
        }
        r = __builtin_amdgcn_readfirstlane(r);
        split = __builtin_amdgcn_readfirstlane(split);
        const int ctx = ctx_lens[r];
        const int tok0 = split * split_tokens;
        const int tok_end = min(ctx, tok0 + split_tokens);
        const int page0 = tok0 / kPage;
        const int n_pages = (tok_end - tok0 + kPage - 1) / kPage;
        const int* bt = block_table + (int64_t)r * max_pages + page0;
        const uint16_t* Kh = Kp + (int64_t)kvh * D;   // kv-head column of the pools
        const uint16_t* Vh = Vp + (int64_t)kvh * D;

        // query heads of this kv head as the B operand (column = head l16); lanes past the
        // group read a valid head and are zeroed
        u32x4 qreg[NKS];
        {
            const int head = kvh * G + min(l16, G - 1);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const u32x4 t = ldg16(q + ((int64_t)r * Hq + head) * D + ks * 32 + g4 * 8);
                qreg[ks] = (l16 < G) ? t : zero4();
            }
        }

        // pages of this wave: lp = wave + 4*i, i < cnt
        const int cnt = wave < n_pages ? (n_pages - wave + kDecWaves - 1) / kDecWaves : 0;

        struct Page { u32x4 k[NKS]; u32x4 v[4]; };
        // Page i of this wave (clamped to the wave's last page, so a prefetch past the end
        // re-reads a page that is already cached).  Every load is inside the page.
        auto load_page = [&](Page& P, int i) {
            const int lp = __builtin_amdgcn_readfirstlane(wave + kDecWaves * min(i, cnt - 1));
            const int phys = bt[lp];
            const int64_t pofs = (int64_t)phys * kPage * row_stride;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(Kh + pofs), (short)0, page_bytes, 0x00020000);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(Vh + pofs), (short)0, page_bytes, 0x00020000);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                P.k[ks] = __builtin_amdgcn_raw_buffer_load_b128(rk, vofs_k, ks * 64, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                P.v[e] = __builtin_amdgcn_raw_buffer_load_b128(rv, vofs_v, e * slot_bytes, 0);
        };

        float m_run = -INFINITY, l_run = 0.f;
        f32x4 oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{};

        auto compute_page = [&](const Page& P, int i) {
            const int t_pg = tok0 + (wave + kDecWaves * i) * kPage;   // first token of the page
            const bool tail = t_pg + kPage > tok_end;                 // wave-uniform
            // S^T: rows = slots 4*g4 + v, column = head l16
            f32x4 s = f32x4{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) s = E::mfma16(P.k[ks], qreg[ks], s);
            if (tail) {
#pragma unroll
                for (int v = 0; v < 4; ++v) s[v] = (t_pg + 4 * g4 + v < tok_end) ? s[v] : -INFINITY;
            }
            // V^T into the slab (zeros for slots past the context)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = (!tail || t_pg + 4 * v_tg + e < tok_end) ? P.v[e][p] : 0u;
                const int d = v_dc * 8 + 2 * p;
                *reinterpret_cast<u32x2*>(&slab[d * VSTR + 4 * v_tg]) =
                    pack_col_lo(w[0], w[1], w[2], w[3]);
                *reinterpret_cast<u32x2*>(&slab[(d + 1) * VSTR + 4 * v_tg]) =
                    pack_col_hi(w[0], w[1], w[2], w[3]);
            }
            // online softmax for the page (per head = per column l16)
            float mloc = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
            mloc = fmaxf(mloc, xor_lanes(mloc, 16));
            mloc = fmaxf(mloc, xor_lanes(mloc, 32));
            const float m_new = fmaxf(m_run, mloc * scale_log2);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            float p[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) p[v] = fast_exp2(__builtin_fmaf(s[v], scale_log2, -m_use));
            l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
            if (__ballot(alpha != 1.f)) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
            }
            m_run = m_new;
            const u32x2 pb = {E::pack2(p[0], p[1]), E::pack2(p[2], p[3])};
            // slab writes land before other lanes of the wave read them
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const u32x2 a = *reinterpret_cast<const u32x2*>(&slab[(db * 16 + l16) * VSTR + 4 * g4]);
                oacc[db] = E::mfma16k16(a, pb, oacc[db]);
            }
            // every lane has read the slab before the next page overwrites it
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };

        // Page sweep: three register sets in rotation, two pages in flight ahead of the one
        // being computed.  The prefetch is unconditional (clamped), so the wait counter
        // sees the same outstanding loads on every path.
        if (cnt > 0) {
            Page b0, b1, b2;
            load_page(b0, 0);
            load_page(b1, 1);
            for (int i = 0;;) {
                load_page(b2, i + 2);
                compute_page(b0, i);
                if (++i >= cnt) break;
                load_page(b0, i + 2);
                compute_page(b1, i);
                if (++i >= cnt) break;
                load_page(b1, i + 2);
                compute_page(b2, i);
                if (++i >= cnt) break;
            }
        }

        // per-head totals of this wave: l over the 4 lane groups
        float l_w = l_run + xor_lanes(l_run, 16);
        l_w += xor_lanes(l_w, 32);

        // cross-wave merge through LDS (slabs are dead now)
        __syncthreads();
        float* mbuf = reinterpret_cast<float*>(lds);                 // [4][16]
        float* lbuf = mbuf + kDecWaves * 16;                          // [4][16]
        float* obuf = lbuf + kDecWaves * 16;                          // [4][16][D]
        if (g4 == 0) {
            mbuf[wave * 16 + l16] = m_run;
            lbuf[wave * 16 + l16] = l_w;
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                obuf[(wave * 16 + l16) * D + db * 16 + 4 * g4 + v] = oacc[db][v];
        __syncthreads();

        const int64_t part = ((int64_t)r * Hq + kvh * G) * S_max;   // (r, first head) partials
        for (int e = tid; e < G * D; e += kDecThreads) {
            const int hh = e / D, d = e % D;
            float m = -INFINITY;
#pragma unroll
            for (int w = 0; w < kDecWaves; ++w) m = fmaxf(m, mbuf[w * 16 + hh]);
            float lt = 0.f, ot = 0.f;
#pragma unroll
            for (int w = 0; w < kDecWaves; ++w) {
                const float wt = fast_exp2(mbuf[w * 16 + hh] - m);   // 0 for a wave without pages
                lt += wt * lbuf[w * 16 + hh];
                ot += wt * obuf[(w * 16 + hh) * D + d];
            }
            const int64_t pidx = part + (int64_t)hh * S_max + split;
            ws_o[pidx * D + d] = ot / lt;
            if (d == 0) ws_lse[pidx] = (m + fast_log2(lt)) * kLn2;
        }
        __syncthreads();   // merge buffers fully read before the next item reuses the LDS
    }
}

// a13: fixed-order merge of the splits of one (sequence, head); one thread per dim.
template <int D, bool IS_BF16>
__global__ __launch_bounds__(D) void decode_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    const int* __restrict__ ctx_lens, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int Hq, int split_tokens, int S_max) {
    using E = Elem<IS_BF16>;
    const int rh = blockIdx.x;                 // r * Hq + h
    const int r = rh / Hq;
    const int d = threadIdx.x;
    const int ctx = ctx_lens[r];
    const int n_split = (ctx + split_tokens - 1) / split_tokens;
    const float* lse_s = ws_lse + (int64_t)rh * S_max;
    const float* o_s = ws_o + (int64_t)rh * S_max * D;
    float M = -INFINITY;
    for (int s = 0; s < n_split; ++s) M = fmaxf(M, lse_s[s]);
    float wsum = 0.f, acc = 0.f;
    if (n_split > 0) {
        const float log2e = 1.4426950408889634f;
        for (int s = 0; s < n_split; ++s) {
            const float w = fast_exp2((lse_s[s] - M) * log2e);
            wsum += w;
            acc += w * o_s[(int64_t)s * D + d];
        }
    }
    const float out = (n_split > 0) ? acc / wsum : 0.f;
    // store as 16 bits (RNE); pairs of threads cooperate through a packed write
    const float other = __shfl_xor(out, 1, 64);
    if ((d & 1) == 0)
        *reinterpret_cast<uint32_t*>(O + (int64_t)rh * D + d) = E::pack2(out, other);
    if (LSE && d == 0) LSE[rh] = (n_split > 0) ? M + __logf(wsum) : -INFINITY;
}

template <int D, bool IS_BF16>
hipError_t launch_decode_t(const DecodeArgs& a) {
    const long long S = decode_max_splits(a.page_size, a.max_pages, a.split_tokens);
    float* ws_o = (float*)a.workspace;
    float* ws_lse = (float*)((char*)a.workspace + (size_t)a.B * a.Hq * (size_t)S * D * sizeof(float));
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    hipStream_t st = (hipStream_t)a.stream;
    const long long max_items = (long long)a.B * S * a.Hkv;
    const long long grid = std::min<long long>(max_items, 2LL * device_cu_count());
    hipError_t e = launch_kernel(decode_split_kernel<D, IS_BF16>, dim3((unsigned)grid),
                                 dim3(kDecThreads), st, "decode_split_kernel", a.q, a.Kpages,
                                 a.Vpages, a.block_table, a.ctx_lens, ws_o, ws_lse, a.B, a.Hq,
                                 a.Hkv, a.max_pages, a.split_tokens, (int)S, scale_log2);
    if (e != hipSuccess) return e;
    return launch_kernel(decode_merge_kernel<D, IS_BF16>, dim3((unsigned)(a.B * a.Hq)), dim3(D),
                         st, "decode_merge_kernel", ws_o, ws_lse, a.ctx_lens, a.O, a.LSE, a.Hq,
                         a.split_tokens, (int)S);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a) {
    if (a.d == 128) return a.is_bf16 ? launch_decode_t<128, true>(a) : launch_decode_t<128, false>(a);
    return a.is_bf16 ? launch_decode_t<64, true>(a) : launch_decode_t<64, false>(a);
}

}  // namespace attn
