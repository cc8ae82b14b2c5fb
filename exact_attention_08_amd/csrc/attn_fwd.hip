// attn_fwd.hip -- fused exact attention forward (prefill) for gfx950.
//
// Method: FlashAttention-2 loop order [LLM Internals 10.3.2, tiled forward; 10.3.3]: one
// workgroup owns a block of BR query rows of one (batch, head); the K_j/V_j column blocks
// stream past it through LDS; for every block the running max m, the exp-sum l and the
// unnormalised output O~ are updated, one division by l happens at the end, and only O and
// LSE = m + ln l go back to HBM.  Fully masked causal blocks are never visited; diagonal
// and ragged-tail blocks are masked element by element before the max [zwjcode.cn
// FlashAttention blog, section 06; AI-infra handbook "FlashAttention and inference
// operators", causal masking and the teaching kernel's kv_end bound].
//
// Rescaling follows FlashAttention-4's conditional rescale [CS349D Lecture 4 notes, 3.5]
// in an exact form: the exponentials are taken relative to a reference max m_ref, which is
// only moved (and O~, l rescaled by e^(m_ref - m_new)) when a block's max exceeds it by
// more than 2^8 in the base-2 domain.  Until then the weights stay below 2^8, which bf16,
// fp16 and the fp32 accumulators hold without overflow; O = O~/l and LSE = m_ref + ln l
// are the same quantities as with the per-block rescale.
//
// MI355X mapping (not the pages' CUDA design):
//   * 4 waves per workgroup, one 32-row query block per wave (BR = 128 rows); 2 waves per
//     SIMD at d = 128, 3 at d = 64.  A wave computes S^T = K_j Q_i^T with
//     v_mfma_f32_32x32x16: keys are the MFMA rows and queries its columns, so one lane holds
//     16 scores of ONE query row per 32-key block.  Row max / row sum are in-lane reductions
//     plus one exchange with the lane 32 away; the exponentiated scores, rounded to 16 bits,
//     are already the B operand of O^T = V_j^T P^T, so P never leaves registers, and the
//     rescale factor is a per-lane scalar.
//   * The KV sweep is a software pipeline over 32-key blocks: the next block's S^T MFMAs are
//     issued in the same branch-free region as this block's exponentials and O^T MFMAs
//     (two alternating score buffers, so they carry no register dependence), and operands
//     are read from LDS one step ahead of their use.
//   * Q stays in registers for the whole KV sweep (B operand of the first product).
//   * K_j and V_j go from HBM straight into LDS with buffer loads that write LDS
//     (buffer_load ... lds): no register staging and no LDS store instructions.  Rows are
//     unpadded; each row's 16-byte chunks are permuted by an XOR of the row index, so that the
//     operand reads below are bank-conflict free.  K operands are 16-byte LDS reads; the
//     transposed V operand comes from the transposing LDS read (ds_read_b64_tr_b16), so
//     staging needs no shuffles.  LDS is double buffered: one barrier per 64-key tile, and
//     the next tile streams into the other stage during the math.
//   * All HBM reads are buffer loads whose range is the head's rows, so rows past N read as
//     zero without any branch.
//   * exp2 / log2 run on v_exp_f32 / v_log_f32 with log2(e) folded into the score scale.
//   * Work order: the query heads sharing one K/V head, and all their query tiles, run on
//     one XCD (one L2), heaviest causal tile first.  Short sequences use a persistent grid
//     (one workgroup per resident slot taking items in turn, each item at a pseudo-random
//     issue priority), long ones one workgroup per item (each block's MFMA/exp region at
//     raised issue priority).
//
// The same kernel serves three layouts (MODE: dense; the shared-prefix chunks of a cascade
// decode; paged / varlen prefill) and two variants of the dense layout (FEAT: sliding window,
// soft-cap); each is described where its geometry is defined below.
#include <type_traits>

#include "attn_common.h"
#include "attn_internal.h"
#include "attn_prefill_common.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Per head size: BC keys per KV tile, QB 32-row query blocks per wave (BR = 128 * QB rows
// per workgroup), OCC waves per SIMD (the register budget is 512 / OCC per wave).
template <int D> struct PrefillTile;
template <> struct PrefillTile<128> { static constexpr int BC = 64, QB = 1, OCC = 2; };
template <> struct PrefillTile<64> { static constexpr int BC = 64, QB = 1, OCC = 3; };

// Persistent grid: the order in which one XCD's workgroups take its n_x items (items are
// numbered head-major, heaviest causal tile first within a head group of `per` items).  The
// workgroups take the items in rounds of W, alternating direction, so in head-major order
// each pair of rounds gives every workgroup one heavy and one light tile of the same head
// groups.  The last round is partial, though, and in head-major order its items are heavy
// tiles for some workgroups and none for others.  So only the rounds before the last two
// full ones (an even number of them, keeping their pairs whole) stay head-major, and the
// head groups left for the tail are taken heaviest tile first across all of them: the
// lightest tiles then make up the partial round.  slot -> head-major item index, a bijection.
// (Modelled on the GPT-2-medium grid with each item costing its tiles plus ~3 tiles of fixed
// cost: the slowest workgroup's load falls from 1.085 to 1.024 times the mean.)
__device__ inline int persistent_order(int s, int n_x, int W, int per, int G) {
    const int R = (n_x + W - 1) / W;
    const int full = R - 1;
    const int hm = full < 2 ? 0 : full - (((full - 2) & 1) ? 3 : 2);
    const int S0 = (max(hm, 0) * W / per) * per;
    if (s < S0) return s;
    const int t = s - S0;
    const int hg0 = S0 / per;
    const int span = (n_x / per - hg0) * G;   // tail items of one tile rank
    const int rank = t / span, rem = t - rank * span;
    return (hg0 + rem / G) * per + rank * G + rem % G;
}

// Shared-prefix (cascade) mode [CS349D Lecture 4 notes, 4.4 and 5.3]: the query rows of a
// kv head are the single decode queries of all requests (request r, head kvh * G + g is row
// r * G + g), so the prefix keys are read once for all of them; an item sweeps one chunk of
// the prefix (non-causal) and writes its partial state -- O normalised, in fp32, and LSE --
// among the split partials that the decode merge combines.
struct ModeGeo {
    int n_rows;     // prefix mode: query rows per kv head (requests x G); paged: max q_len
    int chunk;      // prefix keys per item
    int n_chunks;
    int s_stride;   // partial states per (request, query head)
    int s_base;     // index of the first prefix chunk among them
    // variants (FEAT): sliding window length; soft-cap constants 2 log2(e) scale / c and
    // c / scale (a raw score s becomes (c / scale) tanh(s scale / c))
    int window;
    float cap_in, cap_out;
};

// Variants of dense attention [CS349D Lecture 4 notes 5.4]: kFeatWindow -- query i sees only
// keys i - window < j <= i (causal); kFeatCap -- each scaled score s becomes c tanh(s / c)
// before the softmax.  An item then starts at the tile holding its first visible key, each
// wave skips the blocks left of its rows' windows, and the capped scores replace the raw
// ones before the masks, the maximum and the exponentials.
enum { kFeatWindow = 1, kFeatCap = 2 };

// Paged / varlen prefill [LLM Internals 10.3.8, variable-length batching; 10.3.7, block
// table; CS349D Lecture 4 section 5.1, incremental prefill].  Request r's new queries are
// rows cu_q[r] .. cu_q[r+1]-1 of q [total_q, Hq, d]; its cache holds kv_lens[r] tokens in
// 16-token pages, the new ones last, so new query i sits at position kv_len - q_len + i and
// (causal) sees the keys up to it.  An item is (request, kv head, tile of 128 rows); as in
// the prefix mode the G query heads share the tile (row t = query t / G, head t % G), so
// each K/V byte is read once per tile, and wave w streams page w of each 64-key tile with a
// descriptor that ends at the page's last valid slot: slots past the cache read as zero.

enum { kModeDense = 0, kModePrefix = 1, kModePaged = 2 };

// MODE kModePrefix is the shared-prefix mode: Q is the decode query q [B, Hq, d], K/V the
// prefix [Hkv, N, d], O (as fp32) and LSE the partial-state buffers.  kModePaged: Q is q
// [total_q, Hq, d], K/V the page pools [pages, 16, Hkv, d], O [total_q, Hq, d], LSE
// [total_q, Hq] or null.
template <int D, bool IS_BF16, bool CAUSAL, bool PERSIST, int MODE, int FEAT = 0>
__global__ __launch_bounds__(kThreads, PrefillTile<D>::OCC) void prefill_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int B, int Hq, int Hkv, int N, float scale_log2, int n_qtiles, int n_items, int xcd_major,
    ModeGeo cg, const int* __restrict__ pg_table, const int* __restrict__ pg_cu_q,
    const int* __restrict__ pg_kv_lens, int pg_max_pages) {
    constexpr bool CASC = MODE == kModePrefix;
    constexpr bool PAGED = MODE == kModePaged;
    constexpr bool WIN = (FEAT & kFeatWindow) != 0;
    constexpr bool CAP = (FEAT & kFeatCap) != 0;
    static_assert(FEAT == 0 || MODE == kModeDense, "variants of dense attention");
    static_assert(!WIN || CAUSAL, "the sliding window is causal");
    static_assert(!CASC || (!CAUSAL && !PERSIST), "the prefix mode is non-causal, one item per workgroup");
    static_assert(!PAGED || !PERSIST, "the paged mode runs one item per workgroup");
    using E = Elem<IS_BF16>;
    constexpr int BC = PrefillTile<D>::BC;
    constexpr int kQB = PrefillTile<D>::QB;
    constexpr int kBR = 32 * kQB * kWaves;   // query rows per workgroup
    constexpr int NKB = BC / 32;         // 32-key blocks per KV tile
    constexpr int NKS = D / 16;          // k-steps of the first product
    constexpr int NDB = D / 32;          // 32-wide d blocks of the output
    constexpr int RB = 2 * D;            // bytes per K/V row in LDS
    constexpr int NSLOT = D / 8;         // 16-byte chunks per row
    constexpr int TILE_B = BC * RB;      // bytes of one K (or V) tile
    constexpr int STAGE_B = 2 * TILE_B;  // one LDS stage: the K tile, then the V tile
    constexpr int NDMA = TILE_B / 1024 / kWaves;   // 1 KiB wave loads per tile and wave
    static_assert(NDMA * 1024 * kWaves == TILE_B, "K/V tile must split into 1 KiB wave loads");
    static_assert(!PAGED || (BC == 16 * kWaves && NDMA * 1024 == 16 * RB),
                  "paged mode: each wave loads one 16-token page of a tile");

    __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGE_B];   // two stages of STAGE_B bytes

    const int G = Hq / Hkv;

    // Items per workgroup.  Without PERSIST there is one workgroup per item, this loop runs
    // once and the hardware dispatcher hands out the items.  With a smaller, persistent grid
    // (short items, where the gap between one workgroup ending and the next starting on a CU
    // costs more than the spread in workgroup speeds), workgroup b stays on XCD b % P
    // (P = 8 when items are XCD-interleaved, else 1; workgroups reach the XCDs round robin)
    // and takes that XCD's items in rounds of W, the workgroups of that XCD: forward on even
    // rounds and backward on odd ones, so heavy and light causal tiles pair up.
    const int P = xcd_major ? 8 : 1;
    const int x = blockIdx.x % P, w = blockIdx.x / P;
    const int W = ((int)gridDim.x - x + P - 1) / P;
    const int n_slots = (n_items - x + P - 1) / P;
    for (int round = 0;; ++round) {
        const int slot = round * W + ((round & 1) ? W - 1 - w : w);
        if (slot >= n_slots) break;
        // the previous item's last LDS reads must be done before this item's first store
        if (round > 0) __syncthreads();
        if (PERSIST) {
            // Co-resident persistent workgroups keep their dispatch order for the whole
            // kernel, and the instruction arbiter prefers the older waves, so the first
            // workgroup on a CU would always run fastest.  A pseudo-random issue priority per
            // item (three levels, from a hash of workgroup and round) spreads that advantage.
            const unsigned h = (unsigned)(blockIdx.x * 2654435761u + round * 40503u);
            switch ((h >> 16) % 3) {
                case 0: __builtin_amdgcn_s_setprio(0); break;
                case 1: __builtin_amdgcn_s_setprio(1); break;
                default: __builtin_amdgcn_s_setprio(2); break;
            }
        }
        // Lane indices are rederived per item (the empty asm hides that they are loop
        // invariant): kept live across the item loop they would cost registers.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int l32 = lane & 31;
        const int g = lane >> 5;
        // prefix mode: item = (kv head, chunk, query tile), query tiles fastest so that the
        // items sharing a chunk run together
        const int chunk_id = CASC ? ((int)blockIdx.x / n_qtiles) % cg.n_chunks : 0;
        const WorkItem wi = [&] {
            if constexpr (CASC) {
                WorkItem c;
                c.qt = (int)blockIdx.x % n_qtiles;
                c.kvh = (int)blockIdx.x / n_qtiles / cg.n_chunks;
                c.b = 0;
                c.h = 0;
                return c;
            } else if constexpr (PAGED) {
                WorkItem pw = prefill_work_item((int)blockIdx.x, n_qtiles, Hkv, 1, xcd_major);
                // Batches of at most 64 requests: position b of the launch order is the
                // request with the b-th longest cache (ties by index), so the heaviest items
                // start first.  Each wave ranks the requests with shuffles; all agree.
                if (B <= 64) {
                    const int key = lane < B ? pg_kv_lens[lane] : -1;
                    int rank = 0;
                    for (int j = 0; j < 64; ++j) {
                        const int kj = __shfl(key, j, 64);
                        rank += (j < B && (kj > key || (kj == key && j < lane))) ? 1 : 0;
                    }
                    const unsigned long long hit = __ballot(lane < B && rank == pw.b);
                    pw.b = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
                }
                return pw;
            } else {
                const int idx = PERSIST ? persistent_order(slot, n_slots, W, n_qtiles * G, G) : slot;
                return prefill_work_item(idx * P + x, n_qtiles, Hkv, G, xcd_major);
            }
        }();
        // paged mode: the request's packed query rows and cache length (clamped to what the
        // launch and the block table cover)
        int pq0 = 0, pq_len = 0, pkv_len = 0;
        if constexpr (PAGED) {
            pq0 = __builtin_amdgcn_readfirstlane(pg_cu_q[wi.b]);
            pq_len = min(max(__builtin_amdgcn_readfirstlane(pg_cu_q[wi.b + 1]) - pq0, 0), cg.n_rows);
            pkv_len = min(max(__builtin_amdgcn_readfirstlane(pg_kv_lens[wi.b]), 0), pg_max_pages * 16);
        }
        const int64_t qh_off = ((int64_t)wi.b * Hq + wi.h) * (int64_t)N;      // row offset of (b,h)
        const int64_t kh_off = ((int64_t)wi.b * Hkv + wi.kvh) * (int64_t)N;   // row offset of (b,kvh)
        const int head_bytes = N * D * 2;
        const int q_bytes = CASC ? B * Hq * D * 2 : PAGED ? pq_len * Hq * D * 2 : head_bytes;
        const __amdgpu_buffer_rsrc_t rq = head_rsrc(
            CASC ? Q : PAGED ? Q + (int64_t)pq0 * Hq * D : Q + qh_off * D, q_bytes);

        const int q_tile0 = wi.qt * kBR;
        const int q0w = q_tile0 + wave * (32 * kQB);   // first query row of this wave
        const int n_qrows = CASC ? cg.n_rows : PAGED ? pq_len * G : N;
        const bool wave_live = q0w < n_qrows;
        if (PAGED && q_tile0 >= n_qrows) break;        // a tile past this request's rows

        // Keys of the item: [kbase, kend) (a prefix chunk, the request's cache, or the whole
        // sequence).  KV tiles this workgroup visits: causal stops after the block holding
        // its last row.
        // window: the item starts at the tile holding the first key its first row sees
        const int kbase = CASC ? chunk_id * cg.chunk
                        : WIN ? (max(0, q_tile0 - cg.window + 1) / BC) * BC : 0;
        const int kend = CASC ? min(N, kbase + cg.chunk) : PAGED ? pkv_len : N;
        // paged: row t is query t / G at position pq_pos0 + t / G
        const int pq_pos0 = pkv_len - pq_len;
        int kv_last, n_kv;
        if constexpr (PAGED) {
            const int t_last = min(q_tile0 + kBR, n_qrows) - 1;
            kv_last = CAUSAL ? min(kend, pq_pos0 + t_last / G + 1) - 1 : kend - 1;
            n_kv = kv_last < 0 ? 1 : kv_last / BC + 1;
        } else {
            kv_last = CAUSAL ? min(N, q_tile0 + kBR) - 1 : kend - 1;
            n_kv = (kv_last - kbase) / BC + 1;
        }
        (void)pq_pos0;
        const int wave_last_q = min(q0w + 32 * kQB - 1, n_qrows - 1);

        // a2: this lane's Q rows (one per column block) as the B operand of S^T = K Q^T
        // (k-values d = 16ks + 8g..+7); rows past the last query read as zero (offset past
        // the buffer range)
        auto q_offset = [&](int t, int ks) {
            if constexpr (CASC || PAGED) {
                if (t >= n_qrows) return q_bytes;
                const int rr = t / G;
                return ((rr * Hq + wi.kvh * G + (t - rr * G)) * D + ks * 16 + g * 8) * 2;
            } else {
                return (t * D + ks * 16 + g * 8) * 2;
            }
        };
        u32x4 qreg[kQB][NKS];
    #pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
    #pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                qreg[qb][ks] = __builtin_amdgcn_raw_buffer_load_b128(
                    rq, q_offset(q0w + 32 * qb + l32, ks), 0, 0);

        // a3: K_j, V_j go from HBM straight into LDS stage st (buffer_load ... lds): wave load
        // i writes the 1 KiB block i * kWaves + wave of the tile, lane by lane in 16-byte
        // slots; each lane fetches the chunk that its slot holds under the swizzle.  Rows past
        // N read as zero (buffer range).
        const i32x4 rk4 = head_rsrc4(K + kh_off * D, head_bytes);
        const i32x4 rv4 = head_rsrc4(V + kh_off * D, head_bytes);
        const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)lds);
        auto dma_tile = [&](int j, int st) {
            const int key0 = kbase + j * BC;
            if constexpr (PAGED) {
                // this wave's page: tile rows 16 wave .. 16 wave + 15, LDS blocks
                // wave * NDMA + i; the descriptor ends at the page's last valid slot
                const int pkey = key0 + 16 * wave;
                const int valid = min(max(kend - pkey, 0), 16);
                const int phys = __builtin_amdgcn_readfirstlane(
                    valid > 0 ? pg_table[(int64_t)wi.b * pg_max_pages + pkey / 16] : 0);
                const int64_t pbase = ((int64_t)phys * 16 * Hkv + wi.kvh) * D;
                const int pbytes = valid > 0 ? ((valid - 1) * Hkv * D + D) * 2 : 0;
                const i32x4 rpk = head_rsrc4(K + pbase, pbytes);
                const i32x4 rpv = head_rsrc4(V + pbase, pbytes);
    #pragma unroll
                for (int i = 0; i < NDMA; ++i) {
                    const int blk = wave * NDMA + i;
                    const int p = blk * 64 + lane;
                    const int r = p / NSLOT, sl = p % NSLOT;
                    const int slot_ofs = (r - 16 * wave) * Hkv * D;
                    const int kofs = (slot_ofs + 8 * (sl ^ k_swz<D>(r))) * 2;
                    const int vofs = (slot_ofs + 8 * (sl ^ v_swz<D>(r))) * 2;
                    const uint32_t kdst = __builtin_amdgcn_readfirstlane(lds_base + st * STAGE_B + blk * 1024);
                    dma_b128(rpk, kdst, kofs);
                    dma_b128(rpv, kdst + TILE_B, vofs);
                }
                return;
            }
    #pragma unroll
            for (int i = 0; i < NDMA; ++i) {
                const int blk = i * kWaves + wave;
                const int p = blk * 64 + lane;
                const int r = p / NSLOT, sl = p % NSLOT;
                const int kofs = ((key0 + r) * D + 8 * (sl ^ k_swz<D>(r))) * 2;
                const int vofs = ((key0 + r) * D + 8 * (sl ^ v_swz<D>(r))) * 2;
                const uint32_t kdst = __builtin_amdgcn_readfirstlane(lds_base + st * STAGE_B + blk * 1024);
                dma_b128(rk4, kdst, kofs);
                dma_b128(rv4, kdst + TILE_B, vofs);
            }
        };
        // vmcnt(0): this wave's tile loads have landed in LDS
        auto wait_tile = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };

        // a6 state, per column block (fp32, per lane = per query row; l is this lane's half
        // of the keys)
        // m_thr = m_ref + slack and m_exp (m_ref, or 0 while it is -inf) change only with m_ref
        float m_ref[kQB], l_run[kQB], m_thr[kQB], m_exp[kQB];
        f32x16 oacc[kQB][NDB];
    #pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            m_ref[qb] = -INFINITY;
            m_thr[qb] = -INFINITY;
            m_exp[qb] = 0.f;
            l_run[qb] = 0.f;
    #pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[qb][db] = f32x16{};
        }

        // The KV sweep runs as a software pipeline over 32-key blocks.  Iteration b:
        //   1. read block b's V operands; read the next block's K operands (same tile)
        //      (at d = 128 these reads are issued one step earlier, at the end of step 4 of
        //      the previous block);
        //   2. statistics of block b's scores (mask, max, the rare rescale) -- branches here;
        //   3. at the last block of a tile: wait until this wave's loads of the next tile have
        //      landed in LDS, barrier, start the loads of the tile after it into the stage just
        //      freed, and read the next block's K operands from the new stage;
        //   4. one branch-free region: the next block's S^T MFMAs, block b's exponentials,
        //      sums and packing, and block b's O^T MFMAs -- independent matrix and vector work
        //      the scheduler interleaves, so the softmax runs under the matrix cores.
        // Blocks whose first key lies after the wave's last row (causal) are skipped by the
        // wave; it still takes part in the tile loads and barriers.  Near the end the "next"
        // S^T is computed on the current block and discarded, keeping step 4 branch free.
        const int nb = n_kv * NKB;
        int nb_live;
        // paged: positions of the wave's first row and of each of this lane's rows
        int pos_first = 0, qpos[kQB];
        if constexpr (PAGED) {
            const int pos_last = pq_pos0 + wave_last_q / G;
            nb_live = !wave_live ? 0 : !CAUSAL ? nb : pos_last < 0 ? 0 : min(nb, pos_last / 32 + 1);
            pos_first = pq_pos0 + q0w / G;
    #pragma unroll
            for (int qb = 0; qb < kQB; ++qb) qpos[qb] = pq_pos0 + (q0w + 32 * qb + l32) / G;
        } else {
            nb_live = !wave_live ? 0 : (CAUSAL ? min(nb, (wave_last_q - kbase) / 32 + 1) : nb);
        }
        // window: the wave's first block holding a key its first row sees, and the largest
        // left edge among its rows (blocks starting before it need the elementwise mask)
        const int nb_first = WIN ? max(0, q0w - cg.window + 1 - kbase) / 32 : 0;
        const int win_lo_max = WIN ? wave_last_q - cg.window + 1 : 0;

        // V^T operand of the second product from V (rows in key order) with the transposing LDS read
        // (ds_read_b64_tr_b16): within each 16-lane group G, destination lane i receives, as
        // element e, the (i % 4)-th 16-bit value of the 8 bytes addressed by lane 16G + 4e + i/4.
        // Lane 16G + 4e + a therefore addresses key 4(G >> 1) + e, dims 16(G & 1) + 4a..+3 of the
        // 16-key step, and lane l = 16G + i receives dim 16(G & 1) + i (= l % 32) for keys
        // 4(G >> 1) + 0..3; a second read 8 keys further gives keys 8 + 4(G >> 1) + 0..3.  These
        // are exactly the keys, in the same order, that the lane's P operand holds.
        //
        // Per-lane byte offsets (within a stage) of the V^T operand for each 32-wide d block,
        // and of the K operand for each k-step.  The swizzle depends only on the low row bits,
        // which the lane fixes (V: row mod 8, K: row mod 32), so the block's row offsets are
        // added as constants.
        int v_off[NDB], k_off[NKS];
        {
            const int vr = 4 * ((lane >> 5) & 1) + ((lane >> 2) & 3);
    #pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1) + 4 * db;
                v_off[db] = TILE_B + vr * RB + 16 * (c ^ v_swz<D>(vr)) + 8 * (lane & 1);
            }
    #pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                k_off[ks] = l32 * RB + 16 * ((2 * ks + g) ^ k_swz<D>(l32));
        }
        const char* lds_b = reinterpret_cast<const char*>(lds);
        auto read_tr = [&](const char* p) -> u32x2 {
            typedef short s16x4 __attribute__((ext_vector_type(4)));
            const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(p));
            return __builtin_bit_cast(u32x2, v);
        };
        auto read_k = [&](u32x4 (&ka)[NKS], int st, int kb) {
    #pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                ka[ks] = *reinterpret_cast<const u32x4*>(lds_b + k_off[ks] + st * STAGE_B + kb * 32 * RB);
        };
        auto read_v = [&](u32x4 (&va)[2][NDB], int st, int kb) {
    #pragma unroll
            for (int h = 0; h < 2; ++h)
    #pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const char* vp = lds_b + v_off[db] + st * STAGE_B + (kb * 32 + 16 * h) * RB;
                    const u32x2 lo = read_tr(vp);
                    const u32x2 hi = read_tr(vp + 8 * RB);
                    va[h][db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                }
        };
        // At d = 128 without a window the operands are read one block ahead: at the end of a
        // block's matrix region, into the registers its MFMAs have just consumed, the V^T
        // operands of the next block and (at a tile's last block, whose barrier has published
        // the next tile) the K operands of the block after it, so the reads have the next
        // block's statistics step to land (N = 8192: 2% faster, bitwise identical).  At
        // d = 64 it gained nothing.
        constexpr bool HOIST = !WIN && D == 128;
        u32x4 va_c[2][NDB];
        u32x4 ka_c[NKS];
        auto s_product = [&](const u32x4 (&ka)[NKS], f32x16 (&sacc)[kQB]) {
    #pragma unroll
            for (int qb = 0; qb < kQB; ++qb) {
                sacc[qb] = E::mfma32(ka[0], qreg[qb][0], f32x16{});
    #pragma unroll
                for (int ks = 1; ks < NKS; ++ks) sacc[qb] = E::mfma32(ka[ks], qreg[qb][ks], sacc[qb]);
            }
        };

        // One 32-key block.  sc holds this block's S^T, sn receives the next block's; the two
        // are distinct registers (the caller alternates them), so the next block's MFMAs carry
        // no register dependence on this block's exponentials and can overlap them.
        auto block = [&](int j, int kb, auto stage, f32x16 (&sc)[kQB], f32x16 (&sn)[kQB]) {
            constexpr int ST = decltype(stage)::value;   // == j & 1
            const int bi = j * NKB + kb;
            const int kfirst = kbase + bi * 32;
            // live: the wave computes this block; need_next: it computes the next block's S^T
            // here (with a window, also in the block just before its first live one)
            const bool live = WIN ? (bi >= nb_first && bi < nb_live) : bi < nb_live;   // wave-uniform
            const bool need_next = WIN ? (bi + 1 >= nb_first && bi < nb_live) : live;
            u32x4 va_l[2][NDB];
            u32x4 ka_l[NKS];
            u32x4 (&va)[2][NDB] = HOIST ? va_c : va_l;
            u32x4 (&ka)[NKS] = HOIST ? ka_c : ka_l;
            float m_use[kQB];
            if (live) {
                // 1. operands
                if constexpr (!HOIST) {
                    read_v(va, ST, kb);
                    if (!WIN && kb + 1 < NKB) read_k(ka, ST, kb + 1);
                }
                // 2. statistics
                if constexpr (CAP) {
                    // soft-cap: s -> (c / scale) tanh(s scale / c), tanh(y) = 1 - 2 / (1 + e^2y)
    #pragma unroll
                    for (int qb = 0; qb < kQB; ++qb)
    #pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const float e = fast_exp2(sc[qb][v] * cg.cap_in);
                            const float r = __builtin_amdgcn_rcpf(1.f + e);
                            sc[qb][v] = __builtin_fmaf(-2.f * cg.cap_out, r, cg.cap_out);
                        }
                }
                const bool mask_blk = (CAUSAL && kfirst + 31 > (PAGED ? pos_first : q0w)) ||
                                      kfirst + 32 > kend || (WIN && kfirst < win_lo_max);
    #pragma unroll
                for (int qb = 0; qb < kQB; ++qb) {
                    // a5: elementwise mask (select, never multiply)
                    if (mask_blk) {
                        const int q = PAGED ? qpos[qb] : q0w + 32 * qb + l32;
    #pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int key = kfirst + 8 * (v >> 2) + 4 * g + (v & 3);
                            const bool masked = key >= kend || (CAUSAL && key > q) ||
                                                (WIN && key < q - cg.window + 1);
                            sc[qb][v] = masked ? -INFINITY : sc[qb][v];
                        }
                    }
                    // a6: this lane sees half of the block's keys for its row; the half
                    // maximum decides whether the reference may stay.  Only when some lane's
                    // half exceeds it are the two halves combined (lanes l and l^32 hold the
                    // same row), so both halves always agree on m_ref.
                    float mloc = max3f(sc[qb][0], sc[qb][1], sc[qb][2]);
    #pragma unroll
                    for (int v = 3; v < 15; v += 2) mloc = max3f(mloc, sc[qb][v], sc[qb][v + 1]);
                    mloc = max3f(mloc, sc[qb][15], sc[qb][15]);
                    if (__ballot(mloc * scale_log2 > m_thr[qb])) {
                        const float m_blk = fmaxf(mloc, xor_lanes(mloc, 32)) * scale_log2;
                        const bool move = m_blk > m_thr[qb];
                        const float m_new = move ? m_blk : m_ref[qb];
                        // 0 on the first block; a row that has seen no key yet (paged, or
                        // left of a window; reference still -inf) keeps alpha = 1
                        const float alpha = ((PAGED || WIN) && m_new == -INFINITY)
                                                ? 1.f : fast_exp2(m_ref[qb] - m_new);
                        l_run[qb] *= alpha;
    #pragma unroll
                        for (int db = 0; db < NDB; ++db) oacc[qb][db] *= alpha;
                        m_ref[qb] = m_new;
                        m_thr[qb] = m_new + kRescaleSlack;
                        m_exp[qb] = (m_new == -INFINITY) ? 0.f : m_new;
                    }
                    m_use[qb] = m_exp[qb];
                }
            }
            // 3. tile boundary
            if (kb == NKB - 1) {
                // tile j+1 (this wave's part) is in LDS; the barrier makes the whole tile
                // visible and, with its wait on this wave's LDS reads, frees stage ST
                wait_tile();
                __syncthreads();
                if (j + 2 < n_kv) dma_tile(j + 2, ST);
                if (need_next) read_k(ka, 1 - ST, 0);
            }
            if constexpr (WIN) {
                if (need_next && kb + 1 < NKB) read_k(ka, ST, kb + 1);
            }
            // One workgroup per item: a wave issues step 4 at raised priority, so the SIMD's
            // other wave, in its statistics step, fills the gaps instead of competing for
            // the issue slots of the MFMA/exp stream (about 2% at N = 32768).  The persistent
            // grid sets a per-item priority instead.
            if constexpr (!PERSIST) __builtin_amdgcn_s_setprio(1);
            // 4. next S^T, this block's weights and O^T update (a live block always needs
            // the next S^T; with a window, so does the block just before the first live one)
            if constexpr (WIN) {
                if (!live && need_next) s_product(ka, sn);
            }
            if constexpr (HOIST) {
                if (live) {
                    // d = 128: the next block's S^T k-steps (one dependent chain) and this
                    // block's O^T d-blocks (independent of it) alternate, one MFMA per slot,
                    // with two of this block's weights in the slot after each MFMA:
                    //   S0 w01 | S1 w23 | S2 w45 | S3 w67 pack0 | O00 w89 | S4 | O01 w1011 |
                    //   S5 | O02 w1213 | S6 | O03 w1415 pack1 | S7 | O10 | O11 | O12 | O13
                    // so the matrix pipe always has an instruction it can take while the vector
                    // work issues behind it (the compiler's own order put up to eight vector
                    // instructions between dependent S^T steps and all O^T MFMAs at the end).
                    // The scheduling fences keep this order; N = 32768 ran 1.0% faster,
                    // N = 8192 0.7%, N = 2048 1.9% (interleaved trials).
                    static_assert(kQB == 1 && NKS == 8 && NDB == 4, "the slot order is for d = 128");
                    float p[16];
                    auto wgt = [&](int v) {
                        p[v] = fast_exp2(__builtin_fmaf(sc[0][v], scale_log2, -m_use[0]));
                    };
                    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
                    auto pack = [&](int h) {
                        return u32x4{E::pack2(p[8 * h + 0], p[8 * h + 1]), E::pack2(p[8 * h + 2], p[8 * h + 3]),
                                     E::pack2(p[8 * h + 4], p[8 * h + 5]), E::pack2(p[8 * h + 6], p[8 * h + 7])};
                    };
                    // (written out statement by statement: in a loop the optimiser sinks the
                    // S^T steps, whose result is used only at the end, past the O^T ones)
                    fence();
                    f32x16 sacc = E::mfma32(ka[0], qreg[0][0], f32x16{});
                    fence(); wgt(0); wgt(1); fence();
                    sacc = E::mfma32(ka[1], qreg[0][1], sacc);
                    fence(); wgt(2); wgt(3); fence();
                    sacc = E::mfma32(ka[2], qreg[0][2], sacc);
                    fence(); wgt(4); wgt(5); fence();
                    sacc = E::mfma32(ka[3], qreg[0][3], sacc);
                    fence(); wgt(6); wgt(7);
                    const u32x4 pk0 = pack(0);
                    fence();
                    oacc[0][0] = E::mfma32(va[0][0], pk0, oacc[0][0]);
                    fence(); wgt(8); wgt(9); fence();
                    sacc = E::mfma32(ka[4], qreg[0][4], sacc);
                    fence();
                    // the row sum in the order of the other paths (p0 + p1 + ... + p15), so
                    // that results are bitwise those of the window and soft-cap variants
                    float lsum = p[0];
                    lsum += p[1]; lsum += p[2]; lsum += p[3];
                    fence();
                    oacc[0][1] = E::mfma32(va[0][1], pk0, oacc[0][1]);
                    fence(); wgt(10); wgt(11); fence();
                    sacc = E::mfma32(ka[5], qreg[0][5], sacc);
                    fence();
                    lsum += p[4]; lsum += p[5]; lsum += p[6]; lsum += p[7];
                    fence();
                    oacc[0][2] = E::mfma32(va[0][2], pk0, oacc[0][2]);
                    fence(); wgt(12); wgt(13); fence();
                    sacc = E::mfma32(ka[6], qreg[0][6], sacc);
                    fence();
                    lsum += p[8]; lsum += p[9]; lsum += p[10]; lsum += p[11];
                    fence();
                    oacc[0][3] = E::mfma32(va[0][3], pk0, oacc[0][3]);
                    fence(); wgt(14); wgt(15);
                    const u32x4 pk1 = pack(1);
                    fence();
                    sacc = E::mfma32(ka[7], qreg[0][7], sacc);
                    fence();
                    lsum += p[12]; lsum += p[13]; lsum += p[14]; lsum += p[15];
                    fence();
                    oacc[0][0] = E::mfma32(va[1][0], pk1, oacc[0][0]);
                    fence();
                    oacc[0][1] = E::mfma32(va[1][1], pk1, oacc[0][1]);
                    fence();
                    oacc[0][2] = E::mfma32(va[1][2], pk1, oacc[0][2]);
                    fence();
                    oacc[0][3] = E::mfma32(va[1][3], pk1, oacc[0][3]);
                    fence();
                    l_run[0] += lsum;
                    sn[0] = sacc;
                }
            } else if (live) {
                s_product(ka, sn);
    #pragma unroll
                for (int qb = 0; qb < kQB; ++qb) {
                    float p[16];
    #pragma unroll
                    for (int v = 0; v < 16; ++v)
                        p[v] = fast_exp2(__builtin_fmaf(sc[qb][v], scale_log2, -m_use[qb]));
                    float lsum = p[0];   // the weights are >= +0, so 0 + p[0] == p[0]
    #pragma unroll
                    for (int v = 1; v < 16; ++v) lsum += p[v];
                    l_run[qb] += lsum;
                    // a7: O^T += V^T P^T over the block's two 16-key steps
    #pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const u32x4 pk = {E::pack2(p[8 * h + 0], p[8 * h + 1]),
                                          E::pack2(p[8 * h + 2], p[8 * h + 3]),
                                          E::pack2(p[8 * h + 4], p[8 * h + 5]),
                                          E::pack2(p[8 * h + 6], p[8 * h + 7])};
    #pragma unroll
                        for (int db = 0; db < NDB; ++db)
                            oacc[qb][db] = E::mfma32(va[h][db], pk, oacc[qb][db]);
                    }
                }
            }
            if constexpr (HOIST) {
                if (bi + 1 < nb_live) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (kb + 1 < NKB) {
                        read_v(va, ST, kb + 1);
                    } else {
                        read_v(va, 1 - ST, 0);
                        read_k(ka, 1 - ST, 1);
                    }
                }
            }
            if constexpr (!PERSIST) __builtin_amdgcn_s_setprio(0);
        };

        dma_tile(0, 0);
        wait_tile();
        __syncthreads();
        if (n_kv > 1) dma_tile(1, 1);

        static_assert(NKB == 2, "the block loop alternates two score buffers over two blocks per tile");
        f32x16 s_a[kQB], s_b[kQB];
        if (nb_live > 0 && nb_first == 0) {
            u32x4 ka[NKS];
            read_k(ka, 0, 0);
            s_product(ka, s_a);
            if constexpr (HOIST) {
                read_v(va_c, 0, 0);
                read_k(ka_c, 0, 1);
            }
        }
        // two tiles per trip, so that each block's LDS stage is a compile-time constant
        using st0 = std::integral_constant<int, 0>;
        using st1 = std::integral_constant<int, 1>;
        for (int j = 0; j < n_kv; j += 2) {
            block(j, 0, st0{}, s_a, s_b);
            block(j, 1, st0{}, s_b, s_a);
            if (j + 1 < n_kv) {
                block(j + 1, 0, st1{}, s_a, s_b);
                block(j + 1, 1, st1{}, s_b, s_a);
            }
        }

        // a8: epilogue -- O = O~ / l, LSE = (m_ref + log2 l) ln 2
    #pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            const int q = q0w + 32 * qb + l32;
            if (q >= n_qrows) continue;
            const float l_tot = l_run[qb] + xor_lanes(l_run[qb], 32);
            // v_rcp_f32 (about 1 ulp of fp32): far below the 16-bit rounding of the output
            const float inv_l = __builtin_amdgcn_rcpf(l_tot);
            if constexpr (CASC) {
                // partial state of (request, head) for this chunk: O~/l in fp32, and LSE
                const int rr = q / G;
                const int64_t pidx = ((int64_t)rr * Hq + wi.kvh * G + (q - rr * G)) * cg.s_stride +
                                     cg.s_base + chunk_id;
                float* prow = reinterpret_cast<float*>(O) + pidx * D;
    #pragma unroll
                for (int db = 0; db < NDB; ++db)
    #pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const f32x16& o = oacc[qb][db];
                        *reinterpret_cast<f32x4*>(prow + db * 32 + 8 * a + 4 * g) =
                            f32x4{o[4 * a + 0] * inv_l, o[4 * a + 1] * inv_l, o[4 * a + 2] * inv_l,
                                  o[4 * a + 3] * inv_l};
                    }
                if (g == 0) LSE[pidx] = (m_ref[qb] + fast_log2(l_tot)) * kLn2;
                continue;
            }
            if constexpr (PAGED) {
                // query q / G of the request, head kvh * G + q % G; a row that sees no key
                // (a cache shorter than its chunk) gets O = 0 and LSE = -inf
                const int qi = q / G;
                const int64_t row = (int64_t)(pq0 + qi) * Hq + wi.kvh * G + (q - qi * G);
                const float inv_p = l_tot > 0.f ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
                uint16_t* prow = O + row * D;
    #pragma unroll
                for (int db = 0; db < NDB; ++db)
    #pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const f32x16& o = oacc[qb][db];
                        const u32x2 w = {E::pack2(o[4 * a + 0] * inv_p, o[4 * a + 1] * inv_p),
                                         E::pack2(o[4 * a + 2] * inv_p, o[4 * a + 3] * inv_p)};
                        *reinterpret_cast<u32x2*>(prow + db * 32 + 8 * a + 4 * g) = w;
                    }
                if (g == 0 && LSE) LSE[row] = (m_ref[qb] + fast_log2(l_tot)) * kLn2;
                continue;
            }
            uint16_t* orow = O + (qh_off + q) * D;
    #pragma unroll
            for (int db = 0; db < NDB; ++db)
    #pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const f32x16& o = oacc[qb][db];
                    const u32x2 w = {E::pack2(o[4 * a + 0] * inv_l, o[4 * a + 1] * inv_l),
                                     E::pack2(o[4 * a + 2] * inv_l, o[4 * a + 3] * inv_l)};
                    *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * a + 4 * g) = w;
                }
            if (g == 0) LSE[qh_off + q] = (m_ref[qb] + fast_log2(l_tot)) * kLn2;
        }
        if (!PERSIST) break;
    }
}

template <int D, bool IS_BF16, bool CAUSAL, int FEAT = 0>
hipError_t launch_prefill_t(const PrefillArgs& a, const ModeGeo& cg = ModeGeo{}) {
    constexpr int kBR = 32 * PrefillTile<D>::QB * kWaves;
    const int n_qtiles = (a.N + kBR - 1) / kBR;
    const int n_hg = a.B * a.Hkv;
    const long long n_items = (long long)n_qtiles * a.B * a.Hq;
    const int xcd_major = (n_hg % 8 == 0) ? 1 : 0;
    // Short sequences: a persistent grid, one workgroup per resident slot (OCC per CU), so
    // CUs do not idle between short workgroups.  Long ones: one workgroup per item; there the
    // dispatcher's dynamic hand-out evens out the workgroups' different speeds.
    const bool persistent = a.N <= 2048;
    const long long slots = (long long)device_cu_count() * PrefillTile<D>::OCC;
    const long long grid = persistent && n_items > slots ? slots : n_items;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    if (grid < n_items)
        return launch_kernel(prefill_fwd_kernel<D, IS_BF16, CAUSAL, true, kModeDense, FEAT>,
                             dim3((unsigned)grid), dim3(kThreads), (hipStream_t)a.stream,
                             "prefill_fwd_kernel", a.Q, a.K, a.V, a.O, a.LSE, a.B, a.Hq, a.Hkv,
                             a.N, scale_log2, n_qtiles, (int)n_items, xcd_major, cg,
                             nullptr, nullptr, nullptr, 0);
    return launch_kernel(prefill_fwd_kernel<D, IS_BF16, CAUSAL, false, kModeDense, FEAT>,
                         dim3((unsigned)grid), dim3(kThreads), (hipStream_t)a.stream,
                         "prefill_fwd_kernel", a.Q, a.K, a.V, a.O, a.LSE, a.B, a.Hq, a.Hkv, a.N,
                         scale_log2, n_qtiles, (int)n_items, xcd_major, cg, nullptr,
                         nullptr, nullptr, 0);
}

// Variants share the dense launch (grid choice included); only the item geometry differs.
template <int D, bool IS_BF16, bool CAUSAL, int FEAT>
hipError_t launch_variant_t(const PrefillArgs& a, int window, float softcap) {
    ModeGeo cg{};
    cg.window = window;
    if (softcap > 0.f) {
        cg.cap_in = (float)(2.0 * 1.4426950408889634 * (double)a.scale / (double)softcap);
        cg.cap_out = (float)((double)softcap / (double)a.scale);
    }
    return launch_prefill_t<D, IS_BF16, CAUSAL, FEAT>(a, cg);
}

template <int D, bool IS_BF16>
hipError_t launch_variant_d(const PrefillArgs& a, int window, float softcap) {
    const bool cap = softcap > 0.f;
    if (!a.causal) return launch_variant_t<D, IS_BF16, false, kFeatCap>(a, 0, softcap);
    if (window > 0 && cap) return launch_variant_t<D, IS_BF16, true, kFeatWindow | kFeatCap>(a, window, softcap);
    if (window > 0) return launch_variant_t<D, IS_BF16, true, kFeatWindow>(a, window, 0.f);
    return launch_variant_t<D, IS_BF16, true, kFeatCap>(a, 0, softcap);
}

template <int D, bool IS_BF16>
hipError_t launch_cascade_prefix_t(const CascadePrefixArgs& a) {
    constexpr int kBR = 32 * PrefillTile<D>::QB * kWaves;
    const int n_rows = a.B * (a.Hq / a.Hkv);
    const int n_qtiles = (n_rows + kBR - 1) / kBR;
    const long long n_items = (long long)n_qtiles * a.Hkv * a.n_chunks;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const ModeGeo cg{n_rows, a.chunk, a.n_chunks, a.s_stride, a.s_base};
    return launch_kernel(prefill_fwd_kernel<D, IS_BF16, false, false, kModePrefix>,
                         dim3((unsigned)n_items), dim3(kThreads), (hipStream_t)a.stream,
                         "prefill_fwd_kernel(prefix)", a.q, a.Kprefix, a.Vprefix,
                         reinterpret_cast<uint16_t*>(a.ws_o), a.ws_lse, a.B, a.Hq, a.Hkv,
                         a.prefix_len, scale_log2, n_qtiles, (int)n_items, 0, cg, nullptr,
                         nullptr, nullptr, 0);
}

template <int D, bool IS_BF16, bool CAUSAL>
hipError_t launch_prefill_paged_t(const PagedPrefillArgs& a) {
    constexpr int kBR = 32 * PrefillTile<D>::QB * kWaves;
    const int G = a.Hq / a.Hkv;
    const long long n_qtiles = ((long long)a.max_q_len * G + kBR - 1) / kBR;
    const int n_hg = a.B * a.Hkv;
    const long long n_items = n_qtiles * n_hg;
    const int xcd_major = (n_hg % 8 == 0) ? 1 : 0;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    ModeGeo cg{};
    cg.n_rows = a.max_q_len;
    return launch_kernel(prefill_fwd_kernel<D, IS_BF16, CAUSAL, false, kModePaged>,
                         dim3((unsigned)n_items), dim3(kThreads), (hipStream_t)a.stream,
                         "prefill_fwd_kernel(paged)", a.q, a.Kpages, a.Vpages, a.O, a.LSE, a.B,
                         a.Hq, a.Hkv, 0, scale_log2, (int)n_qtiles, (int)n_items, xcd_major, cg,
                         a.block_table, a.cu_seqlens_q, a.kv_lens, a.max_pages);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a) {
    if (prefill_d128_applies(a)) return launch_prefill_d128(a);
    if (a.d == 128) {
        if (a.is_bf16) return a.causal ? launch_prefill_t<128, true, true>(a)
                                       : launch_prefill_t<128, true, false>(a);
        return a.causal ? launch_prefill_t<128, false, true>(a)
                        : launch_prefill_t<128, false, false>(a);
    }
    if (a.is_bf16) return a.causal ? launch_prefill_t<64, true, true>(a)
                                   : launch_prefill_t<64, true, false>(a);
    return a.causal ? launch_prefill_t<64, false, true>(a) : launch_prefill_t<64, false, false>(a);
}

hipError_t launch_prefill_variant(const PrefillArgs& a, int window, float softcap) {
    if (window <= 0 && !(softcap > 0.f)) return launch_prefill(a);   // plain attention
    if (a.d == 128) return a.is_bf16 ? launch_variant_d<128, true>(a, window, softcap)
                                     : launch_variant_d<128, false>(a, window, softcap);
    return a.is_bf16 ? launch_variant_d<64, true>(a, window, softcap)
                     : launch_variant_d<64, false>(a, window, softcap);
}

hipError_t launch_prefill_paged(const PagedPrefillArgs& a) {
    if (a.d == 128) {
        if (a.is_bf16) return a.causal ? launch_prefill_paged_t<128, true, true>(a)
                                       : launch_prefill_paged_t<128, true, false>(a);
        return a.causal ? launch_prefill_paged_t<128, false, true>(a)
                        : launch_prefill_paged_t<128, false, false>(a);
    }
    if (a.is_bf16) return a.causal ? launch_prefill_paged_t<64, true, true>(a)
                                   : launch_prefill_paged_t<64, true, false>(a);
    return a.causal ? launch_prefill_paged_t<64, false, true>(a)
                    : launch_prefill_paged_t<64, false, false>(a);
}

hipError_t launch_cascade_prefix(const CascadePrefixArgs& a) {
    if (a.d == 128) return a.is_bf16 ? launch_cascade_prefix_t<128, true>(a)
                                     : launch_cascade_prefix_t<128, false>(a);
    return a.is_bf16 ? launch_cascade_prefix_t<64, true>(a) : launch_cascade_prefix_t<64, false>(a);
}

}  // namespace attn
