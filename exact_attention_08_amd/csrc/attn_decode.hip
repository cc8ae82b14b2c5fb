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
//   * A fixed grid of one 8-wave workgroup per CU takes work items (sequence, split, kv head):
//     its first by its own index, the rest from an atomic ticket counter, full splits first
//     and the shorter last splits at the end, so faster workgroups take more items and the
//     grid finishes together.  No workgroup is
//     launched for a split past a sequence's context.
//   * The G query heads are the columns of v_mfma_f32_16x16x32 (G <= 16), the 16 slots of
//     a page its rows: S^T = K Q^T runs on the matrix cores.  The exponentiated scores of a
//     page are exactly the B operand of O^T = V^T P^T on v_mfma_f32_16x16x16, so P stays in
//     registers.
//   * A page's K and V rows of one kv head are loaded a few whole 256-byte rows per
//     instruction (a 64-byte piece of every row per instruction reaches far less of the HBM
//     bandwidth), then staged through a per-wave LDS slab in XOR-swizzled rows: K is read
//     back as the MFMA A operand, V^T with the transposing LDS read (ds_read_b64_tr_b16).
//     V rows at or past the context length are written as zeros, so poisoned slots never
//     reach the sum.
//   * Each page is addressed through a buffer descriptor (page base in SGPRs, one VGPR of
//     per-lane offset); block-table entries are scalar loads; K/V loads are non-temporal.
//     Two register sets per wave: a page's set is reloaded two pages ahead as soon as the
//     page is in the slab, so two pages stay in flight while one is computed.  For
//     1024-token splits the sweep is unrolled, so every wait on a load is counted exactly.
//     The next item's first pages are loaded while the current one is merged.
//   * The 8 waves of a workgroup take every 8th page of the item; their states are merged
//     through LDS at the end of the item.  One workgroup per CU (rather than two of four
//     waves) halves the time per item, so the queue's last items end closer together, and
//     no two workgroups on a CU compete.
#include <algorithm>

#include "attn_common.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kPage = 16;
constexpr int kLoadNT = 2;   // cache-policy operand of a buffer load: non-temporal
constexpr int kDecWaves = 8;         // one workgroup per CU, two waves per SIMD
constexpr int kDecThreads = 64 * kDecWaves;
// A wave's pages per item up to which the page sweep is unrolled (1024-token splits)
constexpr int kSweepUnroll = 8;

// The split kernel's work queue lives in the caller's workspace, in the control block at its
// start: [0] the next ticket, [1] the number of workgroups that have finished,
// [2] the split length the call used (read by the merge kernel when the length was chosen
// on the device).  Words 0 and 1 start at zero (the workspace is zero-filled once by its
// owner) and the last workgroup of a call to finish puts them back to zero, so the next call
// on the same workspace needs no reset.  Calls on different workspaces share nothing.
// Batches up to this size keep their per-sequence split counts in LDS (built once per
// workgroup), so finding an item's sequence needs no global loads.
constexpr int kSeqCache = 1024;

template <int D, bool IS_BF16>
__global__ __launch_bounds__(kDecThreads, 1) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kp,
    const uint16_t* __restrict__ Vp, const int* __restrict__ block_table,
    const int* __restrict__ ctx_lens, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    int B, int Hq, int Hkv, int max_pages, int split_tokens, int S_max, float scale_log2,
    unsigned* __restrict__ queue, int n_workers) {
    using E = Elem<IS_BF16>;
    constexpr int NKS = D / 32;          // k-steps of S^T = K Q^T (32 dims each)
    constexpr int NDB = D / 16;          // 16-row d blocks of O^T
    constexpr int RB = 2 * D;            // bytes per slot row
    constexpr int CH = D / 8;            // 16-byte chunks per row
    constexpr int RPI = 64 / CH;         // slot rows per load instruction
    constexpr int IPP = kPage / RPI;     // load instructions per page and tensor
    constexpr int SLAB_B = 2 * kPage * RB;   // a wave's slab: the page's K rows, then its V rows
    constexpr int LDS_BYTES_V = kDecWaves * SLAB_B;
    constexpr int LDS_BYTES_MERGE = kDecWaves * 16 * (D + 2) * 4;
    constexpr int LDS_BYTES = LDS_BYTES_V > LDS_BYTES_MERGE ? LDS_BYTES_V : LDS_BYTES_MERGE;
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    __shared__ int s_ticket;
    __shared__ int s_pref[2][kSeqCache];   // inclusive prefix sums: full splits, partial splits
    __shared__ int s_ctx[kSeqCache];
    __shared__ int s_porder[64];            // batches <= 64: partial splits, largest first
    __shared__ int s_split;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int l16 = lane & 15;
    const int g4 = lane >> 4;                      // k-group of the 16-row MFMA operands
    const int G = Hq / Hkv;
    const int64_t row_stride = (int64_t)Hkv * D;   // elements between consecutive slots
    const int page_bytes = kPage * (int)row_stride * 2;
    const int slot_bytes = (int)row_stride * 2;
    unsigned char* slab = lds + wave * SLAB_B;

    // Loads: instruction i of a page reads slot rows RPI*i .. RPI*i + RPI-1 whole, lane l the
    // 16-byte chunk l % CH of row RPI*i + l / CH (contiguous row pieces instead of a 64-byte
    // piece of every row).  In the slab, chunk c of slot row r sits in slot c ^ swz(r) of the
    // row; K is then read as the MFMA A operand (row l16, chunk 4ks + g4) and V^T with the
    // transposing read, both touching every LDS bank once per pass.
    auto k_swz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
    auto v_swz = [](int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); };
    const int ld_row = lane / CH, ld_ch = lane % CH;
    const int vofs_ld = (ld_row * (int)row_stride + ld_ch * 8) * 2;   // + i * RPI rows
    // slab byte offsets (K rows first, then V rows)
    auto kw_off = [&](int i) { const int r = RPI * i + ld_row; return r * RB + 16 * (ld_ch ^ k_swz(r)); };
    auto vw_off = [&](int i) {
        const int r = RPI * i + ld_row;
        return kPage * RB + r * RB + 16 * (ld_ch ^ v_swz(r));
    };
    auto kr_off = [&](int ks) { return l16 * RB + 16 * ((4 * ks + g4) ^ k_swz(l16)); };
    // V^T operand (16x16x16 A: row d = 16 db + l16, slots 4 g4 + e): source lane 16G + 4e + a of
    // the transposing read addresses slot row 4G + e, dims 16 db + 4a .. +3
    const int vt_row = 4 * (lane >> 4) + ((lane >> 2) & 3);
    const int vt_a = lane & 3;
    auto vr_off = [&](int db) {
        return kPage * RB + vt_row * RB + 16 * ((2 * db + (vt_a >> 1)) ^ v_swz(vt_row)) + 8 * (vt_a & 1);
    };

    // Balanced split length (split_tokens == 0) [CS349D Lecture 4 notes 5.6: the chunk
    // length follows from the batch's total work over the workers].  The total is
    // T = Hkv * sum(ctx) (token, kv head) pairs and P = T / n_workers the share of one
    // workgroup.  Each item also carries a fixed cost (loading q, merging the 8 waves'
    // states, writing its partial; about 256 pairs' worth here), so the best length grows
    // like sqrt(P) rather than P; the steps below are the measured best lengths on MI355X
    // for P up to 128, 3072, 10240 and beyond.  Every workgroup derives the same value from
    // the lengths on the device, so no host plan is needed and a captured graph stays valid
    // when the lengths change.
    if (split_tokens == 0) {
        if (wave == 0) {
            long long sum = 0;
            for (int rr = lane; rr < B; rr += 64) sum += max(ctx_lens[rr], 0);
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
            const long long per = sum * Hkv / n_workers;
            const int len = per <= 128 ? 256 : per <= 3072 ? 512 : per <= 10240 ? 1024 : 2048;
            if (lane == 0) {
                s_split = len;
                if (blockIdx.x == 0) queue[2] = (unsigned)len;
            }
        }
        __syncthreads();
        split_tokens = __builtin_amdgcn_readfirstlane(s_split);
    }

    // Work list.  The non-empty splits are numbered t = 0 .. n_full + n_part - 1: first the
    // full splits (split_tokens tokens) of sequence 0, 1, ..., then the shorter last split of
    // every sequence whose length is not a multiple of split_tokens, so the queue ends with
    // its lightest items.  Item f = t * Hkv + kvh.  Workgroups draw items from an atomic
    // ticket counter after their first (faster workgroups take more); a workgroup leaves once
    // its ticket passes the item count, so the grid always drains.  Each wave derives the counts and an item's
    // (r, split) from ctx_lens with wave-wide prefix sums over chunks of 64 sequences (all
    // results are wave-uniform).
    auto n_full_of = [&](int rr) { return rr < B ? ctx_lens[rr] / split_tokens : 0; };
    auto n_part_of = [&](int rr) { return rr < B && ctx_lens[rr] % split_tokens != 0 ? 1 : 0; };
    auto incl_scan = [&](int v) {
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_up(v, off, 64);
            v += (lane >= off) ? u : 0;
        }
        return v;
    };
    auto total_of = [&](auto count) {
        int tot = 0;
        for (int c0 = 0; c0 < B; c0 += 64) tot += __shfl(incl_scan(count(c0 + lane)), 63, 64);
        return __builtin_amdgcn_readfirstlane(tot);
    };
    // the sequence holding the t-th unit of `count`, and the unit's index inside it
    auto locate = [&](auto count, int t, int& r_out, int& k_out) {
        int base = 0;
        for (int c0 = 0; c0 < B; c0 += 64) {
            const int n = count(c0 + lane);
            const int inc = incl_scan(n);
            const int tot = __shfl(inc, 63, 64);
            if (t < base + tot) {
                const int exc = base + inc - n;
                const unsigned long long hit = __ballot(n > 0 && exc <= t && t < base + inc);
                const int lr = __builtin_ctzll(hit);
                r_out = c0 + lr;
                k_out = t - __shfl(exc, lr, 64);
                return;
            }
            base += tot;
        }
    };
    const int n_full = total_of(n_full_of);
    const int n_items = (n_full + total_of(n_part_of)) * Hkv;

    const bool cached = B <= kSeqCache;
    if (cached) {
        if (wave == 0) {
            int base_f = 0, base_p = 0;
            for (int c0 = 0; c0 < B; c0 += 64) {
                const int rr = c0 + lane;
                const int inc_f = incl_scan(n_full_of(rr)) + base_f;
                const int inc_p = incl_scan(n_part_of(rr)) + base_p;
                if (rr < B) {
                    s_pref[0][rr] = inc_f;
                    s_pref[1][rr] = inc_p;
                    s_ctx[rr] = ctx_lens[rr];
                }
                base_f = __shfl(inc_f, 63, 64);
                base_p = __shfl(inc_p, 63, 64);
            }
            // Batches of at most 64 sequences hand out the shorter last splits largest
            // first, so the final tickets are the smallest items.  Lane r ranks its last
            // split against all others (ties by sequence index), which every workgroup
            // computes identically.
            if (B <= 64) {
                const int key = lane < B ? ctx_lens[lane] % split_tokens : 0;
                int rank = 0;
                for (int j = 0; j < 64; ++j) {
                    const int kj = __shfl(key, j, 64);
                    rank += (kj > key || (kj == key && j < lane)) ? 1 : 0;
                }
                if (key > 0) s_porder[rank] = lane;
            }
        }
        __syncthreads();
    }
    // the sequence holding unit t of the cached prefix array pf (the first r with pf[r] > t)
    // Lane-dependent addresses in the two helpers below are rederived at each use (the empty
    // asm hides that the lane index is loop invariant): hoisted out of the item loop, they
    // would stay live across the page sweep and push its registers into scratch.
    auto fresh_tid = [] {
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        return t;
    };
    auto find_cached = [&](const int* pf, int t) {
        const int ln = fresh_tid() & 63;
        for (int c0 = 0;; c0 += 64) {
            const int v = c0 + ln < B ? pf[c0 + ln] : 0x7fffffff;
            const unsigned long long hit = __ballot(v > t);
            if (hit) return __builtin_amdgcn_readfirstlane(c0 + __builtin_ctzll(hit));
        }
    };

    // One work item: sequence r, split, kv head, and this wave's share of its pages.
    // An item past the end of the list (valid == false) reads nothing.
    struct Item {
        int r, split, kvh, tok0, tok_end, n_pages, cnt;
        bool valid;
        const int* bt;
    };
    auto setup = [&](int ff) {
        Item it;
        it.valid = ff < n_items;
        const int fv = it.valid ? ff : 0;
        const int t_item = fv / Hkv;
        it.kvh = fv % Hkv;
        // an item past the list (which may be empty) is sequence 0, split 0, no tokens: no
        // table is consulted, and its loads stay inside q (B >= 1) or read nothing
        int r = 0, split = 0, ctx = 0;
        if (it.valid && cached) {
            if (t_item < n_full) {
                r = find_cached(s_pref[0], t_item);
                split = t_item - (r > 0 ? s_pref[0][r - 1] : 0);
                ctx = (split + 1) * split_tokens;   // a full split: its end is inside ctx
            } else {
                r = B <= 64 ? s_porder[t_item - n_full] : find_cached(s_pref[1], t_item - n_full);
                split = s_pref[0][r] - (r > 0 ? s_pref[0][r - 1] : 0);   // its full splits
                ctx = s_ctx[r];
            }
        } else if (it.valid) {
            if (t_item < n_full) {
                locate(n_full_of, t_item, r, split);
            } else {
                locate(n_part_of, t_item - n_full, r, split);
                split = ctx_lens[__builtin_amdgcn_readfirstlane(r)] / split_tokens;
            }
            ctx = ctx_lens[__builtin_amdgcn_readfirstlane(r)];
        }
        it.r = __builtin_amdgcn_readfirstlane(r);
        it.split = __builtin_amdgcn_readfirstlane(split);
        ctx = __builtin_amdgcn_readfirstlane(ctx);
        it.tok0 = it.split * split_tokens;
        it.tok_end = min(ctx, it.tok0 + split_tokens);
        it.n_pages = (it.tok_end - it.tok0 + kPage - 1) / kPage;
        // pages of this wave: lp = wave + 4*i, i < cnt
        it.cnt = (it.valid && wave < it.n_pages)
                     ? (it.n_pages - wave + kDecWaves - 1) / kDecWaves : 0;
        it.bt = block_table + (int64_t)it.r * max_pages + it.tok0 / kPage;
        return it;
    };

    // query heads of the item's kv head as the B operand (column = head l16).  The
    // descriptor covers exactly the G heads of the group, so lanes past it read zeros; no
    // select on the loaded value means nothing waits for these loads before the first
    // product that uses them.
    u32x4 qreg[NKS];
    const int q_vofs = (l16 * D + g4 * 8) * 2;
    auto load_q = [&](const Item& it) {
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(q + ((int64_t)it.r * Hq + it.kvh * G) * D), (short)0, G * D * 2, 0x00020000);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            qreg[ks] = __builtin_amdgcn_raw_buffer_load_b128(rq, q_vofs + ks * 64, 0, 0);
    };

    struct Page { u32x4 k[IPP]; u32x4 v[IPP]; };
    // Page i of this wave's share of item it.  Past the share (a prefetch beyond the last
    // page, or an invalid item) the descriptors have length 0: nothing is read and the
    // registers receive zeros.  The loads are issued either way, so the wait counter sees
    // the same outstanding loads on every path.
    auto load_page = [&](const Item& it, Page& P, int i) {
        const bool inside = i < it.cnt;                       // wave-uniform
        const int lp = __builtin_amdgcn_readfirstlane(wave + kDecWaves * (inside ? i : 0));
        const int phys = inside ? it.bt[lp] : 0;
        const int64_t pofs = (int64_t)phys * kPage * row_stride + (int64_t)it.kvh * D;
        const int len = inside ? page_bytes : 0;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Kp + pofs), (short)0, len, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(Vp + pofs), (short)0, len, 0x00020000);
        // Every K/V byte is read exactly once: the loads are marked non-temporal (nt), so
        // they stream past the caches instead of displacing what is reused.
#pragma unroll
        for (int i = 0; i < IPP; ++i)
            P.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, vofs_ld + i * RPI * slot_bytes, 0, kLoadNT);
#pragma unroll
        for (int i = 0; i < IPP; ++i)
            P.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, vofs_ld + i * RPI * slot_bytes, 0, kLoadNT);
    };

    // The first item of a workgroup is its own index: the dispatcher spreads workgroups
    // round robin over the XCDs, so when there are fewer items than workgroups the busy ones
    // are spread evenly too (first-come tickets bunched them on a few XCDs).  Later items
    // come from the queue, numbered after the grid.
    int f = blockIdx.x;
    Item it = setup(f);
    Page b0, b1;
    load_q(it);
    load_page(it, b0, 0);
    load_page(it, b1, 1);
    while (f < n_items) {
        // The next item's ticket is drawn by thread 0 now, after this item's first two page
        // loads were issued (so waiting for those loads does not wait for the atomic), and
        // published at the cross-wave merge below.  It has no value on the other threads, so
        // nothing waits for the atomic before that point.
        int next_ticket;
        if (tid == 0) next_ticket = (int)(gridDim.x + atomicAdd(&queue[0], 1u));

        float m_run = -INFINITY, l_run = 0.f;
        f32x4 oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{};

        auto stage_page = [&](const Page& P, int i) {
            const int t_pg = it.tok0 + (wave + kDecWaves * i) * kPage;   // first token of the page
            const bool tail = t_pg + kPage > it.tok_end;                 // wave-uniform
            // the page's K and V rows into the slab; V rows at or past the context are zeros, so
            // poisoned slots never reach the sum
#pragma unroll
            for (int i = 0; i < IPP; ++i) {
                const int r = RPI * i + ld_row;
                const bool keep = !tail || t_pg + r < it.tok_end;
                const u32x4 vz = keep ? P.v[i] : zero4();
                *reinterpret_cast<u32x4*>(slab + kw_off(i)) = P.k[i];
                *reinterpret_cast<u32x4*>(slab + vw_off(i)) = vz;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };
        auto math_page = [&](int i) {
            const int t_pg = it.tok0 + (wave + kDecWaves * i) * kPage;   // first token of the page
            const bool tail = t_pg + kPage > it.tok_end;                 // wave-uniform
            // S^T: rows = slots 4*g4 + v, column = head l16
            f32x4 s = f32x4{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const u32x4 ka = *reinterpret_cast<const u32x4*>(slab + kr_off(ks));
                s = E::mfma16(ka, qreg[ks], s);
            }
            if (tail) {
#pragma unroll
                for (int v = 0; v < 4; ++v) s[v] = (t_pg + 4 * g4 + v < it.tok_end) ? s[v] : -INFINITY;
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
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                typedef short s16x4 __attribute__((ext_vector_type(4)));
                const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(slab + vr_off(db)));
                oacc[db] = E::mfma16k16(__builtin_bit_cast(u32x2, t), pb, oacc[db]);
            }
            // every lane has read the slab before the next page overwrites it
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };

        // Page sweep: two register sets; a page's set is reloaded (two pages ahead) as soon as
        // the page is in the slab, so two pages are in flight while one is computed.
        const int cnt = it.cnt;
        if (cnt > 0 && cnt <= kSweepUnroll) {
            // straight-line sweep (every wait on a load is counted exactly)
#pragma unroll
            for (int i = 0; i < kSweepUnroll; ++i) {
                // the loads are issued on every path (empty past the item), so the wait counts
                // below do not depend on cnt
                Page& P = (i & 1) ? b1 : b0;
                if (i < cnt) stage_page(P, i);
                load_page(it, P, i + 2);
                if (i < cnt) math_page(i);
                __builtin_amdgcn_sched_barrier(0);   // keep pages apart (register pressure)
            }
        } else if (cnt > 0) {
            for (int i = 0;;) {
                stage_page(b0, i);
                load_page(it, b0, i + 2);
                math_page(i);
                if (++i >= cnt) break;
                stage_page(b1, i);
                load_page(it, b1, i + 2);
                math_page(i);
                if (++i >= cnt) break;
            }
        }
        if (tid == 0) s_ticket = next_ticket;

        // per-head totals of this wave: l over the 4 lane groups
        float l_w = l_run + xor_lanes(l_run, 16);
        l_w += xor_lanes(l_w, 32);

        // cross-wave merge through LDS (slabs are dead now)
        __syncthreads();
        const int f_next = s_ticket;
        // The next item's Q and first two pages load while this item is merged (the page
        // registers and Q are free now), so HBM stays busy across the item boundary.
        const Item nx = setup(f_next);
        load_q(nx);
        load_page(nx, b0, 0);
        load_page(nx, b1, 1);
        float* mbuf = reinterpret_cast<float*>(lds);                 // [waves][16]
        float* lbuf = mbuf + kDecWaves * 16;                          // [waves][16]
        float* obuf = lbuf + kDecWaves * 16;                          // [waves][16][D]
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

        const int64_t part = ((int64_t)it.r * Hq + it.kvh * G) * S_max;   // (r, first head) partials
        for (int e = fresh_tid(); e < G * D; e += kDecThreads) {
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
            const int64_t pidx = part + (int64_t)hh * S_max + it.split;
            ws_o[pidx * D + d] = ot / lt;
            if (d == 0) ws_lse[pidx] = (m + fast_log2(lt)) * kLn2;
        }
        __syncthreads();   // merge buffers fully read before the next item reuses the LDS
        f = f_next;
        it = nx;
    }
    // the last workgroup to finish puts the counters back to zero for the next call on this
    // workspace
    if (tid == 0) {
        __threadfence();
        if (atomicAdd(&queue[1], 1u) == gridDim.x - 1) {
            atomicExch(&queue[0], 0u);
            atomicExch(&queue[1], 0u);
        }
    }
}

// a13: fixed-order merge of the partial states of one (sequence, head); one thread per dim.
// The states are the n_pre chunks of a shared prefix (at s_base.., cascade decode; none
// otherwise) and then the sequence's splits, in key order.  The loads are spread so that
// none waits for another: the LSEs are read by all threads at once (state u by thread
// u mod D) for the maximum, then the states go in chunks of D, thread d turning state
// c0 + d's LSE into its weight in LDS and every thread summing its dim over the chunk in
// ascending order with independent loads.
template <int D, bool IS_BF16>
__global__ __launch_bounds__(D) void decode_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    const int* __restrict__ ctx_lens, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int Hq, int split_tokens, int S_max, int n_pre, int s_base,
    const unsigned* __restrict__ queue) {
    using E = Elem<IS_BF16>;
    constexpr int NW = D / 64;                 // waves per workgroup
    __shared__ float s_w[D];
    __shared__ float s_red[NW];
    const int rh = blockIdx.x;                 // r * Hq + h
    const int r = rh / Hq;
    const int d = threadIdx.x;
    const int ctx = ctx_lens[r];
    // a split length chosen on the device was left in the call's control block
    if (split_tokens == 0) split_tokens = (int)queue[2];
    const int n_state = n_pre + (ctx + split_tokens - 1) / split_tokens;
    const float* lse_s = ws_lse + (int64_t)rh * S_max;
    const float* o_s = ws_o + (int64_t)rh * S_max * D;
    // state u: prefix chunk u (u < n_pre), else split u - n_pre
    auto slot = [&](int u) { return u < n_pre ? s_base + u : u - n_pre; };

    float M = -INFINITY;
    for (int u = d; u < n_state; u += D) M = fmaxf(M, lse_s[slot(u)]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    if ((d & 63) == 0) s_red[d >> 6] = M;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_red[w]);

    const float log2e = 1.4426950408889634f;
    float wsum = 0.f, acc = 0.f;
    for (int c0 = 0; c0 < n_state; c0 += D) {
        const int u = c0 + d;
        s_w[d] = u < n_state ? fast_exp2((lse_s[slot(u)] - M) * log2e) : 0.f;
        __syncthreads();
        const int cnt = min(D, n_state - c0);
        if (n_pre == 0) {
            const float* oc = o_s + (int64_t)c0 * D + d;
#pragma unroll 8
            for (int j = 0; j < cnt; ++j) {
                const float w = s_w[j];
                wsum += w;
                acc += w * oc[(int64_t)j * D];
            }
        } else {
#pragma unroll 8
            for (int j = 0; j < cnt; ++j) {
                const float w = s_w[j];
                wsum += w;
                acc += w * o_s[(int64_t)slot(c0 + j) * D + d];
            }
        }
        __syncthreads();
    }
    const float out = (n_state > 0) ? acc / wsum : 0.f;
    // store as 16 bits (RNE); pairs of threads cooperate through a packed write
    const float other = __shfl_xor(out, 1, 64);
    if ((d & 1) == 0)
        *reinterpret_cast<uint32_t*>(O + (int64_t)rh * D + d) = E::pack2(out, other);
    if (LSE && d == 0) LSE[rh] = (n_state > 0) ? M + __logf(wsum) : -INFINITY;
}

template <int D, bool IS_BF16>
hipError_t launch_decode_t(const DecodeArgs& a) {
    // partial states per (sequence, head): the splits, then the prefix chunks (if any)
    const long long S_split = decode_max_splits(a.page_size, a.max_pages, a.split_tokens);   // 0: shortest balanced split
    const long long n_pre = a.prefix_len > 0 ? cascade_chunks(a.prefix_len) : 0;
    const long long S = S_split + n_pre;
    unsigned* queue = (unsigned*)a.workspace;
    float* ws_o = (float*)((char*)a.workspace + kDecodeCtrlBytes);
    float* ws_lse = (float*)((char*)ws_o + (size_t)a.B * a.Hq * (size_t)S * D * sizeof(float));
    if (n_pre > 0) {
        const CascadePrefixArgs pa{a.q, a.Kprefix, a.Vprefix, ws_o, ws_lse, a.B, a.Hq, a.Hkv, D,
                                   a.prefix_len, kCascadeChunk, (int)n_pre, (int)S, (int)S_split,
                                   a.is_bf16, a.scale, a.stream};
        const hipError_t e = launch_cascade_prefix(pa);
        if (e != hipSuccess) return e;
    }
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    hipStream_t st = (hipStream_t)a.stream;
    const long long max_items = (long long)a.B * S_split * a.Hkv;
    const long long grid = std::min<long long>(max_items, (long long)device_cu_count());
    hipError_t e = launch_kernel(decode_split_kernel<D, IS_BF16>, dim3((unsigned)grid),
                                 dim3(kDecThreads), st, "decode_split_kernel", a.q, a.Kpages,
                                 a.Vpages, a.block_table, a.ctx_lens, ws_o, ws_lse, a.B, a.Hq,
                                 a.Hkv, a.max_pages, a.split_tokens, (int)S, scale_log2,
                                 queue, device_cu_count());
    if (e != hipSuccess) return e;
    return launch_kernel(decode_merge_kernel<D, IS_BF16>, dim3((unsigned)(a.B * a.Hq)), dim3(D),
                         st, "decode_merge_kernel", ws_o, ws_lse, a.ctx_lens, a.O, a.LSE, a.Hq,
                         a.split_tokens, (int)S, (int)n_pre, (int)S_split, queue);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a) {
    if (a.d == 128) return a.is_bf16 ? launch_decode_t<128, true>(a) : launch_decode_t<128, false>(a);
    return a.is_bf16 ? launch_decode_t<64, true>(a) : launch_decode_t<64, false>(a);
}

}  // namespace attn
