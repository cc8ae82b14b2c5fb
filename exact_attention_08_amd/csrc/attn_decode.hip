// attn_decode.hip -- paged split-KV decode for gfx950.
//
// Method [CS349D Lecture 4 notes 4.1-4.3; LLM Internals 10.3.7; AI-infra handbook
// "FlashAttention and inference operators", Flash-Decoding / split-K and the paged GQA
// decode kernel with its four listed improvements]:
//   * one query token per sequence; the keys are cut into splits of split_tokens tokens;
//   * one workgroup per (sequence, kv head, split) serves all G = Hq/Hkv query heads of
//     that kv head, so each K/V byte is read from HBM once;
//   * token t lives in slot t % 16 of physical page block_table[r][t / 16];
//   * inside a split the running (m, l, O~) online softmax is used (no score buffer);
//   * each split writes its normalised O_s and LSE_s; a second kernel merges the splits
//     of a sequence in ascending order with LSE = ln sum e^{LSE_s},
//     O = sum e^{LSE_s - LSE} O_s, skipping nothing but splits past the context.
//
// MI355X mapping:
//   * The G query heads are the columns of v_mfma_f32_16x16x32 (G <= 16), a page of 16
//     tokens its rows: S^T = K Q^T runs on the matrix cores with 16-byte K loads straight
//     from HBM into the A operand.  The exponentiated scores of two pages (32 tokens) are
//     exactly the B operand of O^T = V^T P^T, so P stays in registers.
//   * V is transposed through a per-wave LDS slab (d-major, tokens permuted so each A
//     operand is one 16-byte read).  Tokens at or past the context length are zeroed on
//     the way in, so poisoned slots can never reach the sum.
//   * 4 waves per workgroup split the pages of a split round robin by page pair; the next
//     pair is fetched into registers while the current pair is in the matrix cores; the
//     four wave states are merged through LDS at the end.
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
    int Hq, int Hkv, int max_pages, int split_tokens, int S_max, float scale_log2) {
    using E = Elem<IS_BF16>;
    constexpr int NKS = D / 32;          // k-steps of S^T = K Q^T (32 dims each)
    constexpr int NDB = D / 16;          // 16-row d blocks of O^T
    constexpr int VSTR = 32 + 8;         // LDS row stride of the per-wave V^T slab (elements)
    constexpr int KCH = D / 8;           // 16-byte chunks per K/V row
    constexpr int VUNITS = 8 * KCH / 64; // V units (4 tokens x 8 dims) per lane per page pair
    static_assert(VUNITS * 64 == 8 * KCH, "V pair must split evenly over a wave");
    constexpr int SLAB = D * VSTR;       // elements per wave slab
    // LDS: 4 V^T slabs, reused after the sweep for the cross-wave merge
    constexpr int LDS_ELEMS_V = kDecWaves * SLAB;
    constexpr int LDS_BYTES_MERGE = kDecWaves * 16 * (D + 2) * 4;
    constexpr int LDS_BYTES = (LDS_ELEMS_V * 2 > LDS_BYTES_MERGE) ? LDS_ELEMS_V * 2 : LDS_BYTES_MERGE;
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

    const int split = blockIdx.x;
    const int kvh = blockIdx.y;
    const int r = blockIdx.z;
    const int ctx = ctx_lens[r];
    const int tok0 = split * split_tokens;
    if (tok0 >= ctx) return;                       // split past the context: nothing to do
    const int tok_end = min(ctx, tok0 + split_tokens);
    const int page0 = tok0 / kPage;
    const int n_pages = (tok_end - tok0 + kPage - 1) / kPage;
    const int n_pairs = (n_pages + 1) / 2;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;                      // k-group of the 16x16x32 operands
    const int G = Hq / Hkv;
    const int* bt = block_table + (int64_t)r * max_pages;
    const int64_t row_stride = (int64_t)Hkv * D;   // elements between consecutive slots
    uint16_t* slab = reinterpret_cast<uint16_t*>(lds) + wave * SLAB;

    // query heads of this kv head as the B operand (column = head l16, k = 32ks + 8g4..)
    u32x4 qreg[NKS];
    const int head = kvh * G + l16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        qreg[ks] = (l16 < G) ? ldg16(q + ((int64_t)r * Hq + head) * D + ks * 32 + g4 * 8)
                             : zero4();

    // one page pair in registers: K in A-operand layout, V as 4-token x 8-dim units
    struct Pair { u32x4 k[2][NKS]; u32x4 v[VUNITS][4]; };

    auto load_pair = [&](Pair& P, int pp) {
        const int pg = page0 + 2 * pp;             // first logical page of the pair
        const int tpair0 = pg * kPage;             // its first token
        const bool has1 = 2 * pp + 1 < n_pages;
        const int phys0 = bt[pg];
        const int phys1 = has1 ? bt[pg + 1] : 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int phys = h ? phys1 : phys0;
            const bool ok = (h == 0 || has1) && (tpair0 + h * kPage + l16 < tok_end);
            const uint16_t* base = Kp + ((int64_t)phys * kPage + l16) * row_stride +
                                   (int64_t)kvh * D + g4 * 8;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) P.k[h][ks] = ok ? ldg16(base + ks * 32) : zero4();
        }
#pragma unroll
        for (int u = 0; u < VUNITS; ++u) {
            const int unit = lane + 64 * u;
            const int tg = unit & 7;               // 4-token group within the 32-token pair
            const int dc = unit >> 3;              // 8-dim chunk
            const int phys = (tg < 4) ? phys0 : phys1;
            const bool page_ok = (tg < 4) || has1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int slot = (tg & 3) * 4 + e;
                const bool ok = page_ok && (tpair0 + (tg >> 2) * kPage + slot < tok_end);
                P.v[u][e] = ok ? ldg16(Vp + ((int64_t)phys * kPage + slot) * row_stride +
                                       (int64_t)kvh * D + dc * 8)
                               : zero4();
            }
        }
    };

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{};

    auto compute_pair = [&](const Pair& P, int pp) {
        const int tpair0 = (page0 + 2 * pp) * kPage;
        // V^T into the wave's slab: token t of the pair goes to column 8*(t/4 % 4) + 4*(t/16)
        // + t % 4, so lane group g4 later reads its 8 tokens {4g4..4g4+3, 16+4g4..+3}
        // as one 16-byte chunk.
#pragma unroll
        for (int u = 0; u < VUNITS; ++u) {
            const int unit = lane + 64 * u;
            const int tg = unit & 7, dc = unit >> 3;
            const int col = 8 * (tg & 3) + 4 * (tg >> 2);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int d = dc * 8 + 2 * p;
                *reinterpret_cast<u32x2*>(&slab[d * VSTR + col]) =
                    pack_col_lo(P.v[u][0][p], P.v[u][1][p], P.v[u][2][p], P.v[u][3][p]);
                *reinterpret_cast<u32x2*>(&slab[(d + 1) * VSTR + col]) =
                    pack_col_hi(P.v[u][0][p], P.v[u][1][p], P.v[u][2][p], P.v[u][3][p]);
            }
        }
        // S^T for both pages: rows = tokens 4*g4 + v (+16), column = head l16
        f32x4 s[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            s[h] = f32x4{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) s[h] = E::mfma16(P.k[h][ks], qreg[ks], s[h]);
        }
        // mask tokens past the context (select)
        float mloc = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = tpair0 + h * kPage + 4 * g4 + v;
                s[h][v] = (t < tok_end) ? s[h][v] : -INFINITY;
                mloc = fmaxf(mloc, s[h][v]);
            }
        mloc = fmaxf(mloc, xor_lanes(mloc, 16));
        mloc = fmaxf(mloc, xor_lanes(mloc, 32));
        const float m_new = fmaxf(m_run, mloc * scale_log2);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float p[8];
        float lsum = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                p[4 * h + v] = fast_exp2(__builtin_fmaf(s[h][v], scale_log2, -m_use));
                lsum += p[4 * h + v];
            }
        l_run = l_run * alpha + lsum;
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        }
        m_run = m_new;
        const u32x4 pb = {E::pack2(p[0], p[1]), E::pack2(p[2], p[3]), E::pack2(p[4], p[5]),
                          E::pack2(p[6], p[7])};
        // the slab writes above must land before other lanes read them (same wave)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(&slab[(db * 16 + l16) * VSTR + g4 * 8]);
            oacc[db] = E::mfma16(a, pb, oacc[db]);
        }
        // every lane has read the slab before the next pair overwrites it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // page-pair sweep, two register sets alternating (prefetch next while computing current)
    {
        Pair A, Bp;
        int pp = wave;
        if (pp < n_pairs) load_pair(A, pp);
        while (pp < n_pairs) {
            if (pp + kDecWaves < n_pairs) load_pair(Bp, pp + kDecWaves);
            compute_pair(A, pp);
            pp += kDecWaves;
            if (pp >= n_pairs) break;
            if (pp + kDecWaves < n_pairs) load_pair(A, pp + kDecWaves);
            compute_pair(Bp, pp);
            pp += kDecWaves;
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
        for (int v = 0; v < 4; ++v) obuf[(wave * 16 + l16) * D + db * 16 + 4 * g4 + v] = oacc[db][v];
    __syncthreads();

    const int64_t part = ((int64_t)r * Hq + kvh * G) * S_max;   // (r, first head) partial index
    for (int e = tid; e < G * D; e += kDecThreads) {
        const int hh = e / D, d = e % D;
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) m = fmaxf(m, mbuf[w * 16 + hh]);
        float lt = 0.f, ot = 0.f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) {
            const float wt = fast_exp2(mbuf[w * 16 + hh] - m);   // 0 for a wave without tokens
            lt += wt * lbuf[w * 16 + hh];
            ot += wt * obuf[(w * 16 + hh) * D + d];
        }
        const int64_t pidx = part + (int64_t)hh * S_max + split;
        ws_o[pidx * D + d] = ot / lt;
        if (d == 0) ws_lse[pidx] = (m + fast_log2(lt)) * kLn2;
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
    hipError_t e = launch_kernel(decode_split_kernel<D, IS_BF16>, dim3((unsigned)S, a.Hkv, a.B),
                                 dim3(kDecThreads), st, "decode_split_kernel", a.q, a.Kpages,
                                 a.Vpages, a.block_table, a.ctx_lens, ws_o, ws_lse, a.Hq, a.Hkv,
                                 a.max_pages, a.split_tokens, (int)S, scale_log2);
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
