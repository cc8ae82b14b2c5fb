// attn_fwd.hip -- fused exact attention forward (prefill) for gfx950.
//
// Method: FlashAttention-2 loop order [LLM Internals 10.3.2, tiled forward; 10.3.3]: one
// workgroup owns a block of BR = 128 query rows of one (batch, head); the K_j/V_j column
// blocks stream past it through LDS; for every block the running max m, the exp-sum l and
// the unnormalised output O~ are updated with the e^(m_old - m_new) correction, one
// division by l happens at the end, and only O and LSE = m + ln l go back to HBM.  Fully
// masked causal blocks are never visited; diagonal and ragged-tail blocks are masked
// element by element before the max [zwjcode.cn FlashAttention blog, section 06; AI-infra
// handbook "FlashAttention and inference operators", causal masking and the teaching
// kernel's kv_end bound].  The rescale of O~ is skipped when no row's max grew (an exact
// form of FlashAttention-4's conditional rescale) [CS349D Lecture 4 notes, 3.5].
//
// MI355X mapping (not the pages' CUDA design):
//   * 4 waves x 32 query rows.  Each wave computes S^T = K_j Q_i^T with
//     v_mfma_f32_32x32x16: the keys are the MFMA rows and the queries its columns, so one
//     lane holds 16 scores of ONE query row.  Row max / row sum are in-lane reductions plus
//     one exchange with the lane 32 away, and the fp32 scores, once exponentiated and
//     rounded, are already laid out as the B operand of O^T = V_j^T P^T -- P never leaves
//     registers.  The per-row rescale factor is a per-lane scalar.
//   * Q lives in registers for the whole KV sweep (B operand of the first product).
//   * K_j is staged row-major in LDS; V_j is staged transposed (d-major) with the key order
//     inside each 16-key chunk permuted so that every MFMA operand is one 16-byte LDS read.
//     Rows are padded by 16 bytes so the 16-byte reads are bank-conflict free.
//   * exp2 / log2 run on v_exp_f32 / v_log_f32 with log2(e) folded into the score scale.
//   * The next K/V block is fetched from HBM into registers while the current one is in
//     the matrix cores.
//   * Work items are ordered heaviest causal tile first, and the Hq/Hkv query heads that
//     share one K/V head are placed on the same XCD (same L2).
#include "attn_common.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kBR = 32 * kWaves;     // query rows per workgroup
constexpr int kThreads = 64 * kWaves;

template <int D> struct PrefillTile;
template <> struct PrefillTile<128> { static constexpr int BC = 64; };
template <> struct PrefillTile<64> { static constexpr int BC = 128; };

// a1: map the hardware workgroup id to (q tile, batch, head).  Group items (q tile,
// batch, kv head) are ordered heaviest first (largest q tile first when causal); the G
// query heads of a group item run on one XCD, consecutively, when the item count is a
// multiple of the XCD count (workgroups are handed to XCDs round robin).
struct WorkItem { int qt, b, h, kvh; };

__device__ inline WorkItem prefill_work_item(int bid, int n_qtiles, int B, int Hkv, int G,
                                             int xcd_remap) {
    int gi, hg;
    if (xcd_remap) {
        const int xcd = bid & 7, slot = bid >> 3;
        gi = (slot / G) * 8 + xcd;
        hg = slot % G;
    } else {
        gi = bid / G;
        hg = bid % G;
    }
    const int per_tile = B * Hkv;
    WorkItem w;
    w.qt = n_qtiles - 1 - gi / per_tile;
    const int bkv = gi % per_tile;
    w.b = bkv / Hkv;
    w.kvh = bkv % Hkv;
    w.h = w.kvh * G + hg;
    return w;
}

template <int D, bool IS_BF16, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void prefill_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int B, int Hq, int Hkv, int N, float scale_log2, int n_qtiles, int xcd_remap) {
    using E = Elem<IS_BF16>;
    constexpr int BC = PrefillTile<D>::BC;
    constexpr int NKB = BC / 32;         // 32-key blocks per KV tile (S accumulators)
    constexpr int NKS = D / 16;          // k-steps of the first product
    constexpr int NDB = D / 32;          // 32-wide d blocks of the output
    constexpr int NKK = BC / 16;         // k-steps of the second product
    constexpr int KSTR = D + 8;          // LDS row stride of K (elements)
    constexpr int VSTR = BC + 8;         // LDS row stride of V^T (elements)
    constexpr int KCH = D / 8;           // 16-byte chunks per K/V row
    constexpr int KLOADS = BC * KCH / kThreads;   // K chunks per thread
    static_assert(KLOADS * kThreads == BC * KCH, "K tile must split evenly");
    static_assert((BC / 4) * KCH == kThreads, "one V unit (4 keys x 8 dims) per thread");

    __shared__ __attribute__((aligned(16))) uint16_t Ks[BC * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VSTR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int G = Hq / Hkv;

    const WorkItem wi = prefill_work_item(blockIdx.x, n_qtiles, B, Hkv, G, xcd_remap);
    const int64_t qh_off = ((int64_t)wi.b * Hq + wi.h) * (int64_t)N;      // row offset of (b,h)
    const int64_t kh_off = ((int64_t)wi.b * Hkv + wi.kvh) * (int64_t)N;   // row offset of (b,kvh)
    const uint16_t* Kh = K + kh_off * D;
    const uint16_t* Vh = V + kh_off * D;

    const int q_tile0 = wi.qt * kBR;
    const int q0w = q_tile0 + wave * 32;      // first query row of this wave
    const int q = q0w + l32;                  // this lane's query row
    const bool wave_live = q0w < N;

    // KV tiles this workgroup visits: causal stops after the block holding its last row.
    const int kv_last = CAUSAL ? min(N, q_tile0 + kBR) - 1 : N - 1;
    const int n_kv = kv_last / BC + 1;
    const int wave_last_q = min(q0w + 31, N - 1);

    // a2: Q rows of this lane, as the B operand of S^T = K Q^T (k-values d = 16ks + 8g..+7)
    u32x4 qreg[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        qreg[ks] = (q < N) ? ldg16(Q + (qh_off + q) * D + ks * 16 + g * 8) : zero4();

    // a3: register staging of one K/V tile
    u32x4 kreg[KLOADS], vreg[4];
    const int v_kg = tid % (BC / 4);          // 4-key group of this thread's V unit
    const int v_dc = tid / (BC / 4);          // 8-dim chunk of this thread's V unit
    // transposed position of the 4-key group: swap bits 0 and 1 of the group index so that
    // MFMA k-values (8g + e) of a 16-key chunk are contiguous in LDS
    const int v_kgp = (v_kg & ~3) | ((v_kg & 1) << 1) | ((v_kg >> 1) & 1);

    auto load_tile = [&](int j) {
        const int key0 = j * BC;
#pragma unroll
        for (int r = 0; r < KLOADS; ++r) {
            const int c = tid + r * kThreads;
            const int row = c / KCH, col = (c % KCH) * 8;
            const int key = key0 + row;
            kreg[r] = key < N ? ldg16(Kh + (int64_t)key * D + col) : zero4();
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = key0 + v_kg * 4 + e;
            vreg[e] = key < N ? ldg16(Vh + (int64_t)key * D + v_dc * 8) : zero4();
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int r = 0; r < KLOADS; ++r) {
            const int c = tid + r * kThreads;
            const int row = c / KCH, col = (c % KCH) * 8;
            *reinterpret_cast<u32x4*>(&Ks[row * KSTR + col]) = kreg[r];
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int d = v_dc * 8 + 2 * p;
            *reinterpret_cast<u32x2*>(&Vt[d * VSTR + v_kgp * 4]) =
                pack_col_lo(vreg[0][p], vreg[1][p], vreg[2][p], vreg[3][p]);
            *reinterpret_cast<u32x2*>(&Vt[(d + 1) * VSTR + v_kgp * 4]) =
                pack_col_hi(vreg[0][p], vreg[1][p], vreg[2][p], vreg[3][p]);
        }
    };

    // a6 state (fp32, per lane = per query row; l is this lane's half of the keys)
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

    load_tile(0);
    for (int j = 0; j < n_kv; ++j) {
        __syncthreads();              // previous tile fully consumed
        store_tile();
        __syncthreads();              // tile j visible in LDS
        if (j + 1 < n_kv) load_tile(j + 1);   // next tile in flight during the math

        const int key0 = j * BC;
        if (!wave_live || (CAUSAL && key0 > wave_last_q)) continue;   // nothing visible

        // a4: S^T block by block: rows = keys key0 + 32kb + (row), columns = this wave's queries
        f32x16 sacc[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            sacc[kb] = f32x16{};
            const bool live = !CAUSAL || key0 + kb * 32 <= wave_last_q;
            if (live) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(
                        &Ks[(kb * 32 + l32) * KSTR + ks * 16 + g * 8]);
                    sacc[kb] = E::mfma32(a, qreg[ks], sacc[kb]);
                }
            }
        }

        // a5: elementwise mask on diagonal / tail tiles (select, never multiply)
        const bool need_mask = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q0w);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = key0 + kb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
                    const bool masked = key >= N || (CAUSAL && key > q);
                    sacc[kb][v] = masked ? -INFINITY : sacc[kb][v];
                }
        }

        // a6: online softmax statistics in the scaled base-2 domain
        float mloc = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, sacc[kb][v]);
        mloc = fmaxf(mloc, xor_lanes(mloc, 32));
        const float m_new = fmaxf(m_run, mloc * scale_log2);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);

        float lsum = 0.f;
        u32x4 pk[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int kb = kk >> 1, base = (kk & 1) * 8;
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = fast_exp2(__builtin_fmaf(sacc[kb][base + e], scale_log2, -m_use));
                lsum += p[e];
            }
            pk[kk] = u32x4{E::pack2(p[0], p[1]), E::pack2(p[2], p[3]), E::pack2(p[4], p[5]),
                           E::pack2(p[6], p[7])};
        }
        l_run = l_run * alpha + lsum;
        if (__ballot(alpha != 1.f)) {   // exact lazy rescale: skipped when no max grew
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        }
        m_run = m_new;

        // a7: O^T += V_j^T P^T
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const bool live = !CAUSAL || key0 + (kk >> 1) * 32 <= wave_last_q;
            if (live) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(
                        &Vt[(db * 32 + l32) * VSTR + kk * 16 + g * 8]);
                    oacc[db] = E::mfma32(a, pk[kk], oacc[db]);
                }
            }
        }
    }

    // a8: epilogue -- O = O~ / l, LSE = (m + log2 l) ln 2
    if (!wave_live || q >= N) return;
    const float l_tot = l_run + xor_lanes(l_run, 32);
    const float inv_l = 1.f / l_tot;
    uint16_t* orow = O + (qh_off + q) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const u32x2 w = {E::pack2(oacc[db][4 * a + 0] * inv_l, oacc[db][4 * a + 1] * inv_l),
                             E::pack2(oacc[db][4 * a + 2] * inv_l, oacc[db][4 * a + 3] * inv_l)};
            *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * a + 4 * g) = w;
        }
    if (g == 0) LSE[qh_off + q] = (m_run + fast_log2(l_tot)) * kLn2;
}

template <int D, bool IS_BF16, bool CAUSAL>
hipError_t launch_prefill_t(const PrefillArgs& a) {
    const int n_qtiles = (a.N + kBR - 1) / kBR;
    const int G = a.Hq / a.Hkv;
    const long long n_group_items = (long long)n_qtiles * a.B * a.Hkv;
    const long long grid = n_group_items * G;
    const int remap = (n_group_items % 8 == 0) ? 1 : 0;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    return launch_kernel(prefill_fwd_kernel<D, IS_BF16, CAUSAL>, dim3((unsigned)grid),
                         dim3(kThreads), (hipStream_t)a.stream, "prefill_fwd_kernel", a.Q, a.K,
                         a.V, a.O, a.LSE, a.B, a.Hq, a.Hkv, a.N, scale_log2, n_qtiles, remap);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a) {
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

long long prefill_grid_size(int B, int Hq, int N) {
    return (long long)((N + kBR - 1) / kBR) * B * Hq;
}

}  // namespace attn
