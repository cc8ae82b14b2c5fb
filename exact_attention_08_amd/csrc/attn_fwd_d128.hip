// attn_fwd_d128.hip -- exact attention forward (prefill) for head size 128 with 64 query
// rows per wave and one wave per SIMD (gfx950).
//
// Same method and arithmetic as prefill_fwd_kernel in attn_fwd.hip -- the FlashAttention-2
// loop order [LLM Internals 10.3.2 and 10.3.3], the exact conditional rescale [CS349D
// Lecture 4 notes, 3.5], S^T = K Q^T on 32x32x16 MFMA so a lane owns one query row -- with
// the results of that kernel bit for bit (same products in the same order, same reductions).
// What differs is the shape of the work:
//
//   * A wave owns 64 query rows, two 32-row blocks a and b, instead of 32.  Each K operand
//     and each V^T operand read from LDS then feeds two MFMAs instead of one, which halves
//     the LDS read traffic per FLOP.  A workgroup is 4 waves (256 rows), one per SIMD.
//   * The register file is placed by hand.  The O^T accumulators of both blocks (128
//     values per lane) live at the fixed accumulator registers a0..a127 and only inline asm
//     touches them: the O^T MFMAs, the rare rescale, the zeroing and the final read.  Every
//     such asm declares a0..a127 clobbered, so the compiler places nothing else there.  Q
//     sits in other accumulator registers (the B operand of the S^T MFMAs); scores, K and
//     V^T operands and weights are in arch registers.  Left to itself, the compiler routes
//     the accumulators through arch registers around the rescale branch on every block.
//   * One 32-key block is a fixed sequence of 32 MFMA slots: first the next block's S^T
//     (16 MFMAs, the two query blocks alternating) with this block's exponentials and packing
//     behind them, then this block's O^T update (16 MFMAs) with the row sums, the next
//     block's row maxima and the operand reads for later blocks behind it.  The compiler does
//     not model the hazards of inline-asm MFMAs: the order guarantees that no vector
//     instruction reads an MFMA result within 13 wait states of that MFMA, and every block
//     ends in 13 wait states.
//   * LDS holds three K/V tiles of 64 keys, so during tile t both tile t and tile t + 1 are
//     readable and the operand reads run one and two blocks ahead across tile edges.  The
//     first block of each tile issues the loads of the tile two on, spread over its first
//     MFMA slots, into the stage that the barrier ending the previous tile has freed.
#include <type_traits>

#include "attn_common.h"
#include "attn_internal.h"
#include "attn_prefill_common.h"

namespace attn {
namespace {

constexpr int kD = 128;
constexpr int kW = 4;                  // waves per workgroup, one per SIMD
constexpr int kBR = 64 * kW;           // query rows per workgroup
constexpr int kBC = 64;                // keys per KV tile: two 32-key blocks
constexpr int kNST = 3;                // LDS stages
constexpr int kRB = 2 * kD;            // bytes per K/V row
constexpr int kNSlot = kD / 8;         // 16-byte chunks per row
constexpr int kTileB = kBC * kRB;      // bytes of one K (or V) tile
// LDS: the K tiles of the three stages, then their V tiles, so that every operand read
// reaches its stage by a constant offset below 64 KiB from one base register
constexpr int kVBase = kNST * kTileB;
constexpr int kNDma = kTileB / 1024 / kW;   // 1 KiB loads per tile, wave and operand
constexpr int kNKS = kD / 16;          // k-steps of the first product
constexpr int kNDB = kD / 32;          // 32-wide d blocks of the output
static_assert(kNDma * 1024 * kW == kTileB, "a tile splits into 1 KiB wave loads");
static_assert(kVBase * 2 <= 160 * 1024, "the three stages fit the LDS");

// every asm that writes the fixed O^T accumulators declares all of them clobbered
#define D128_ACC_CLOBBERS                                                                         \
    "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13",       \
    "a14", "a15", "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26",    \
    "a27", "a28", "a29", "a30", "a31", "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39",    \
    "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47", "a48", "a49", "a50", "a51", "a52",    \
    "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63", "a64", "a65",    \
    "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78",    \
    "a79", "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91",    \
    "a92", "a93", "a94", "a95", "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103",       \
    "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111", "a112", "a113", "a114",       \
    "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125",       \
    "a126", "a127"

// S^T MFMAs: scores (D, C) in arch registers, K (A) in arch, Q (B) in accumulator registers
#define D128_S_MFMA(T)                                                                            \
    __device__ __forceinline__ void s_first_##T(f32x16& d, const u32x4& a, const u32x4& b) {      \
        asm volatile("v_mfma_f32_32x32x16_" #T " %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));    \
    }                                                                                             \
    __device__ __forceinline__ void s_next_##T(f32x16& d, const u32x4& a, const u32x4& b) {       \
        asm volatile("v_mfma_f32_32x32x16_" #T " %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));    \
    }                                                                                             \
    /* O^T tuple r (query block r / 4, d block r % 4) at a[16r : 16r + 15] += V^T P^T */        \
    template <int R>                                                                              \
    __device__ __forceinline__ void o_acc_##T(const u32x4& a, const u32x4& b) {                  \
        asm volatile("v_mfma_f32_32x32x16_" #T " a[%2:%3], %0, %1, a[%2:%3]"                     \
                     :: "v"(a), "v"(b), "i"(16 * R), "i"(16 * R + 15) : D128_ACC_CLOBBERS);       \
    }
D128_S_MFMA(bf16)
D128_S_MFMA(f16)
#undef D128_S_MFMA

template <bool BF16> struct Mma;
template <> struct Mma<true> {
    __device__ __forceinline__ static void s_first(f32x16& d, const u32x4& a, const u32x4& b) { s_first_bf16(d, a, b); }
    __device__ __forceinline__ static void s_next(f32x16& d, const u32x4& a, const u32x4& b) { s_next_bf16(d, a, b); }
    template <int R> __device__ __forceinline__ static void o_acc(const u32x4& a, const u32x4& b) { o_acc_bf16<R>(a, b); }
};
template <> struct Mma<false> {
    __device__ __forceinline__ static void s_first(f32x16& d, const u32x4& a, const u32x4& b) { s_first_f16(d, a, b); }
    __device__ __forceinline__ static void s_next(f32x16& d, const u32x4& a, const u32x4& b) { s_next_f16(d, a, b); }
    template <int R> __device__ __forceinline__ static void o_acc(const u32x4& a, const u32x4& b) { o_acc_f16<R>(a, b); }
};

// a0..a127 = 0; the trailing wait states cover an MFMA reading them next
__device__ __forceinline__ void oacc_zero() {
    asm volatile(".set d128_r, 0\n\t"
                 ".rept 128\n\t"
                 "v_accvgpr_write_b32 a[d128_r], 0\n\t"
                 ".set d128_r, d128_r + 1\n\t"
                 ".endr\n\t"
                 "s_nop 1" ::: D128_ACC_CLOBBERS);
}

// When some lane votes (need != 0, uniform): a0..a63 *= al_a, a64..a127 *= al_b, per lane
// (that is, per query row; lanes that did not vote pass 1).  The accumulators' last MFMA
// ended at least 13 wait states earlier.
__device__ __forceinline__ void oacc_rescale(unsigned long long need, float al_a, float al_b) {
    float t;
    asm volatile("s_cmp_eq_u64 %[need], 0\n\t"
                 "s_cbranch_scc1 .Ld128_rs%=\n\t"
                 ".set d128_r, 0\n\t"
                 ".rept 64\n\t"
                 "v_accvgpr_read_b32 %[t], a[d128_r]\n\t"
                 "v_mul_f32 %[t], %[t], %[A]\n\t"
                 "v_accvgpr_write_b32 a[d128_r], %[t]\n\t"
                 ".set d128_r, d128_r + 1\n\t"
                 ".endr\n\t"
                 ".rept 64\n\t"
                 "v_accvgpr_read_b32 %[t], a[d128_r]\n\t"
                 "v_mul_f32 %[t], %[t], %[B]\n\t"
                 "v_accvgpr_write_b32 a[d128_r], %[t]\n\t"
                 ".set d128_r, d128_r + 1\n\t"
                 ".endr\n\t"
                 "s_nop 1\n"
                 ".Ld128_rs%=:"
                 : [t] "=&v"(t)
                 : [need] "s"(need), [A] "v"(al_a), [B] "v"(al_b)
                 : "scc", D128_ACC_CLOBBERS);
}

// the 16 values of accumulator tuple R (after the final MFMA and its wait states)
template <int R> __device__ __forceinline__ void oacc_read(float (&o)[16]) {
#define D128_RD(i) "v_accvgpr_read_b32 %" #i ", a[%16 + " #i "]\n\t"
    asm volatile(D128_RD(0) D128_RD(1) D128_RD(2) D128_RD(3) D128_RD(4) D128_RD(5) D128_RD(6)
                 D128_RD(7) D128_RD(8) D128_RD(9) D128_RD(10) D128_RD(11) D128_RD(12)
                 D128_RD(13) D128_RD(14) D128_RD(15)
                 : "=v"(o[0]), "=v"(o[1]), "=v"(o[2]), "=v"(o[3]), "=v"(o[4]), "=v"(o[5]),
                   "=v"(o[6]), "=v"(o[7]), "=v"(o[8]), "=v"(o[9]), "=v"(o[10]), "=v"(o[11]),
                   "=v"(o[12]), "=v"(o[13]), "=v"(o[14]), "=v"(o[15])
                 : "i"(16 * R));
#undef D128_RD
}

// 13 wait states: a vector instruction may then read the result of any earlier MFMA
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 4"); }

template <bool IS_BF16, bool CAUSAL>
__global__ __launch_bounds__(64 * kW, 1) void prefill_d128_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int B, int Hq, int Hkv, int N, float scale_log2, int n_qtiles, int xcd_major) {
    using E = Elem<IS_BF16>;
    using M = Mma<IS_BF16>;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[kNST * kTileB];

    const int G = Hq / Hkv;
    const WorkItem wi = prefill_work_item((int)blockIdx.x, n_qtiles, Hkv, G, xcd_major);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int64_t qh_off = ((int64_t)wi.b * Hq + wi.h) * (int64_t)N;      // row offset of (b,h)
    const int64_t kh_off = ((int64_t)wi.b * Hkv + wi.kvh) * (int64_t)N;   // row offset of (b,kvh)
    const int head_bytes = N * kD * 2;
    const int q_tile0 = wi.qt * kBR;
    const int q0w = q_tile0 + wave * 64;   // first query row of this wave (block a; b is +32)
    // KV tiles of the item (causal: up to the one holding its last row); 32-key blocks the
    // wave computes (causal: up to the one holding its last row)
    const int kv_last = CAUSAL ? min(N, q_tile0 + kBR) - 1 : N - 1;
    const int n_kv = kv_last / kBC + 1;
    const int nb = 2 * n_kv;
    const int nb_live = q0w >= N ? 0 : CAUSAL ? min(nb, min(q0w + 63, N - 1) / 32 + 1) : nb;

    // a2: Q rows q0w + l32 (block a) and q0w + 32 + l32 (block b), the B operands of
    // S^T = K Q^T (k-values d = 16 ks + 8 g .. + 7); rows past N read as zero
    const __amdgpu_buffer_rsrc_t rq = head_rsrc(Q + qh_off * kD, head_bytes);
    u32x4 qa[kNKS], qb[kNKS];
#pragma unroll
    for (int ks = 0; ks < kNKS; ++ks) {
        qa[ks] = __builtin_amdgcn_raw_buffer_load_b128(rq, ((q0w + l32) * kD + ks * 16 + g * 8) * 2, 0, 0);
        qb[ks] = __builtin_amdgcn_raw_buffer_load_b128(rq, ((q0w + 32 + l32) * kD + ks * 16 + g * 8) * 2, 0, 0);
    }

    // a3: K_j, V_j from HBM straight into LDS (buffer_load ... lds), rows swizzled as in
    // prefill_fwd_kernel; wave load i writes the 1 KiB block i * kW + wave of each tile.
    // Rows past N read as zero (buffer range).
    const i32x4 rk4 = head_rsrc4(K + kh_off * kD, head_bytes);
    const i32x4 rv4 = head_rsrc4(V + kh_off * kD, head_bytes);
    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)lds);
    // this wave's i-th K and V loads of tile j into stage st
    auto load_pair = [&](int j, int st, int i) {
        const int key0 = j * kBC;
        const int blk = i * kW + wave;
        const int p = blk * 64 + lane;
        const int r = p / kNSlot, sl = p % kNSlot;
        const int kofs = ((key0 + r) * kD + 8 * (sl ^ k_swz<kD>(r))) * 2;
        const int vofs = ((key0 + r) * kD + 8 * (sl ^ v_swz<kD>(r))) * 2;
        const uint32_t kdst = __builtin_amdgcn_readfirstlane(lds_base + st * kTileB + blk * 1024);
        dma_b128(rk4, kdst, kofs);
        dma_b128(rv4, kdst + kVBase, vofs);
    };
    auto load_tile = [&](int j, int st) {
#pragma unroll
        for (int i = 0; i < kNDma; ++i) load_pair(j, st, i);
    };
    // this wave's tile loads have landed; then the workgroup barrier.  No wait on LDS reads
    // is needed: every read of the stage about to be refilled has been consumed already.
    auto publish = [] { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); };

    // Per-lane LDS byte offsets of the K operand of each k-step and of the V^T operand of
    // each d block within a stage (as in prefill_fwd_kernel; the V^T operand comes from the
    // transposing read, ds_read_b64_tr_b16)
    int v_off[kNDB], k_off[kNKS];
    {
        const int vr = 4 * ((lane >> 5) & 1) + ((lane >> 2) & 3);
#pragma unroll
        for (int db = 0; db < kNDB; ++db) {
            const int c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1) + 4 * db;
            v_off[db] = kVBase + vr * kRB + 16 * (c ^ v_swz<kD>(vr)) + 8 * (lane & 1);
        }
#pragma unroll
        for (int ks = 0; ks < kNKS; ++ks) k_off[ks] = l32 * kRB + 16 * ((2 * ks + g) ^ k_swz<kD>(l32));
    }
    const char* lds_b = reinterpret_cast<const char*>(lds);
    auto read_tr = [&](const char* p) -> u32x2 {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
        return __builtin_bit_cast(u32x2, v);
    };
    u32x4 ka[kNKS];     // K operands of the next S^T
    u32x4 va[2][kNDB];  // V^T operands of the current block's two 16-key steps
    auto rk = [&](int ks, int st, int kb) {
        ka[ks] = *reinterpret_cast<const u32x4*>(lds_b + k_off[ks] + st * kTileB + kb * 32 * kRB);
    };
    auto rv = [&](int h, int db, int st, int kb) {
        const char* vp = lds_b + v_off[db] + st * kTileB + (kb * 32 + 16 * h) * kRB;
        const u32x2 lo = read_tr(vp);
        const u32x2 hi = read_tr(vp + 8 * kRB);
        va[h][db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    };

    // a6 state per query block (fp32, per lane = per query row; l is this lane's half of
    // the keys); m_thr = m_ref + slack and m_exp (m_ref, or 0 while it is -inf)
    float m_ref[2], l_run[2], m_thr[2], m_exp[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        m_ref[x] = -INFINITY;
        m_thr[x] = -INFINITY;
        m_exp[x] = 0.f;
        l_run[x] = 0.f;
    }
    oacc_zero();

    // row maximum of a block's 16 scores in this lane (raw score units)
    auto rowmax = [](const f32x16& s) {
        float m = max3f(s[0], s[1], s[2]);
#pragma unroll
        for (int v = 3; v < 15; v += 2) m = max3f(m, s[v], s[v + 1]);
        return max3f(m, s[15], s[15]);
    };
    // a5: block bi needs the elementwise mask for query block x (causal diagonal, keys past
    // N); score v of a lane holds key 32 bi + 4g + c(v), c(v) = 8 (v / 4) + v % 4, and the
    // row sees the keys up to min(q, N - 1)
    auto needs_mask = [&](int bi, int x) {
        const int kfirst = bi * 32;
        return (CAUSAL && kfirst + 31 > q0w + 32 * x) || kfirst + 32 > N;
    };
    auto apply_mask = [&](int bi, int x, f32x16& s) {
        const int q = q0w + 32 * x + l32;
        const int lim = (CAUSAL ? min(q, N - 1) : N - 1) - bi * 32 - 4 * g;
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = (8 * (v >> 2) + (v & 3)) > lim ? -INFINITY : s[v];
    };

    // a6: statistics of block bi.  Its row maxima (ma, mb) come from the previous block's
    // region, over the unmasked scores; a block that needs the mask is masked here and its
    // maxima recomputed.  This lane's half maximum decides whether the reference may stay;
    // only when some lane's exceeds it are the halves combined (lanes l and l ^ 32 hold the
    // same row), the reference moved and O~, l rescaled.
    auto stats = [&](int bi, f32x16& sa, f32x16& sb, float ma, float mb, float& mu_a, float& mu_b) {
        float mloc[2] = {ma, mb};
        if (needs_mask(bi, 0)) {
            apply_mask(bi, 0, sa);
            mloc[0] = rowmax(sa);
        }
        if (needs_mask(bi, 1)) {
            apply_mask(bi, 1, sb);
            mloc[1] = rowmax(sb);
        }
        float alpha[2] = {1.f, 1.f};
        const unsigned long long vote =
            __ballot(mloc[0] * scale_log2 > m_thr[0] || mloc[1] * scale_log2 > m_thr[1]);
        if (vote) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const float m_blk = fmaxf(mloc[x], xor_lanes(mloc[x], 32)) * scale_log2;
                const bool move = m_blk > m_thr[x];
                const float m_new = move ? m_blk : m_ref[x];
                alpha[x] = fast_exp2(m_ref[x] - m_new);
                l_run[x] *= alpha[x];
                m_ref[x] = m_new;
                m_thr[x] = m_new + kRescaleSlack;
                m_exp[x] = (m_new == -INFINITY) ? 0.f : m_new;
            }
        }
        oacc_rescale(vote, alpha[0], alpha[1]);
        mu_a = m_exp[0];
        mu_b = m_exp[1];
    };

    // One 32-key block in 32 MFMA slots.  Slots 1-16: the next block's S^T (both query
    // blocks, into sna/snb, from the K operands read a block ago) with this block's weights
    // and their packing behind them.  Slots 17-32: this block's O^T update (a7) with the row
    // sums, the next block's row maxima, and the reads of the K operands two blocks on and of
    // the V^T operands one block on, each into registers an MFMA has just released.
    // (KST, KKB) and (VST, VKB): stage and block within the tile of those two reads.  In the
    // first block of a tile, dj >= 0 is the tile whose loads this block issues, into stage
    // dst, one K/V pair after each of four S^T MFMAs.
    auto region = [&](auto kst, auto kkb, auto vst, auto vkb, auto first, int dj, int dst,
                      const f32x16& sca, const f32x16& scb, f32x16& sna, f32x16& snb,
                      float mu_a, float mu_b, float& ma_n, float& mb_n) {
        constexpr int KST = decltype(kst)::value, KKB = decltype(kkb)::value;
        constexpr int VST = decltype(vst)::value, VKB = decltype(vkb)::value;
        constexpr bool FIRST = decltype(first)::value;
        auto dp = [&](int i) {
            if constexpr (FIRST) {
                if (dj >= 0) load_pair(dj, dst, i);
            }
        };
        // scheduling fence: nothing moves across a slot edge
        auto F = [] { __builtin_amdgcn_sched_barrier(0); };
        float pa[16], pb[16];
        auto wa = [&](int v) { pa[v] = fast_exp2(__builtin_fmaf(sca[v], scale_log2, -mu_a)); };
        auto wb = [&](int v) { pb[v] = fast_exp2(__builtin_fmaf(scb[v], scale_log2, -mu_b)); };
        // the weights of 8 keys, rounded to 16 bits: the B operand of one O^T k-step
        auto pk = [&](const float* p) {
            return u32x4{E::pack2(p[0], p[1]), E::pack2(p[2], p[3]), E::pack2(p[4], p[5]), E::pack2(p[6], p[7])};
        };
        u32x4 PA0, PA1, PB0, PB1;
        float la, lb, xa, xb;
        F();
        M::s_first(sna, ka[0], qa[0]); F(); wa(0); wa(1); F();
        M::s_first(snb, ka[0], qb[0]); F(); wa(2); wa(3); F();
        M::s_next(sna, ka[1], qa[1]); F(); wa(4); wa(5); dp(0); F();
        M::s_next(snb, ka[1], qb[1]); F(); wa(6); wa(7); PA0 = pk(pa); F();
        M::s_next(sna, ka[2], qa[2]); F(); wa(8); wa(9); dp(1); F();
        M::s_next(snb, ka[2], qb[2]); F(); wa(10); wa(11); F();
        M::s_next(sna, ka[3], qa[3]); F(); wa(12); wa(13); dp(2); F();
        M::s_next(snb, ka[3], qb[3]); F(); wa(14); wa(15); PA1 = pk(pa + 8); F();
        M::s_next(sna, ka[4], qa[4]); F(); wb(0); wb(1); dp(3); F();
        M::s_next(snb, ka[4], qb[4]); F(); wb(2); wb(3); F();
        M::s_next(sna, ka[5], qa[5]); F(); wb(4); wb(5); F();
        M::s_next(snb, ka[5], qb[5]); F(); wb(6); wb(7); PB0 = pk(pb); F();
        M::s_next(sna, ka[6], qa[6]); F(); wb(8); wb(9); F();
        M::s_next(snb, ka[6], qb[6]); F(); wb(10); wb(11); F();
        M::s_next(sna, ka[7], qa[7]); F(); wb(12); wb(13); F();
        M::s_next(snb, ka[7], qb[7]); F(); wb(14); wb(15); PB1 = pk(pb + 8); F();
        // row sums in the order p0 + p1 + ... + p15 of prefill_fwd_kernel
        M::template o_acc<0>(va[0][0], PA0); rk(0, KST, KKB); F(); la = pa[0]; la += pa[1]; la += pa[2]; la += pa[3]; F();
        M::template o_acc<4>(va[0][0], PB0); rk(1, KST, KKB); F(); lb = pb[0]; lb += pb[1]; lb += pb[2]; lb += pb[3]; rv(0, 0, VST, VKB); F();
        M::template o_acc<1>(va[0][1], PA0); rk(2, KST, KKB); F(); la += pa[4]; la += pa[5]; la += pa[6]; la += pa[7]; F();
        M::template o_acc<5>(va[0][1], PB0); rk(3, KST, KKB); F(); lb += pb[4]; lb += pb[5]; lb += pb[6]; lb += pb[7]; rv(0, 1, VST, VKB); F();
        M::template o_acc<2>(va[0][2], PA0); rk(4, KST, KKB); F(); la += pa[8]; la += pa[9]; la += pa[10]; la += pa[11]; F();
        M::template o_acc<6>(va[0][2], PB0); rk(5, KST, KKB); F(); lb += pb[8]; lb += pb[9]; lb += pb[10]; lb += pb[11]; rv(0, 2, VST, VKB); F();
        M::template o_acc<3>(va[0][3], PA0); rk(6, KST, KKB); F(); la += pa[12]; la += pa[13]; la += pa[14]; la += pa[15]; l_run[0] += la; F();
        M::template o_acc<7>(va[0][3], PB0); rk(7, KST, KKB); F(); lb += pb[12]; lb += pb[13]; lb += pb[14]; lb += pb[15]; l_run[1] += lb; rv(0, 3, VST, VKB); F();
        // the next block's row maxima: its S^T MFMAs ended eight MFMAs and more than
        // thirteen wait states ago
        M::template o_acc<0>(va[1][0], PA1); F();
        xa = max3f(sna[0], sna[1], sna[2]); xb = max3f(snb[0], snb[1], snb[2]);
        xa = max3f(xa, sna[3], sna[4]); xb = max3f(xb, snb[3], snb[4]); F();
        M::template o_acc<4>(va[1][0], PB1); F();
        xa = max3f(xa, sna[5], sna[6]); xb = max3f(xb, snb[5], snb[6]);
        xa = max3f(xa, sna[7], sna[8]); xb = max3f(xb, snb[7], snb[8]); rv(1, 0, VST, VKB); F();
        M::template o_acc<1>(va[1][1], PA1); F();
        xa = max3f(xa, sna[9], sna[10]); xb = max3f(xb, snb[9], snb[10]);
        xa = max3f(xa, sna[11], sna[12]); xb = max3f(xb, snb[11], snb[12]); F();
        M::template o_acc<5>(va[1][1], PB1); F();
        xa = max3f(xa, sna[13], sna[14]); xb = max3f(xb, snb[13], snb[14]);
        xa = max3f(xa, sna[15], sna[15]); xb = max3f(xb, snb[15], snb[15]); rv(1, 1, VST, VKB); F();
        M::template o_acc<2>(va[1][2], PA1); F();
        M::template o_acc<6>(va[1][2], PB1); F(); rv(1, 2, VST, VKB); F();
        M::template o_acc<3>(va[1][3], PA1); F();
        M::template o_acc<7>(va[1][3], PB1); F(); rv(1, 3, VST, VKB); F();
        mfma_drain();
        F();
        ma_n = xa;
        mb_n = xb;
    };

    // Prologue: tiles 0 and 1 in LDS; S^T of block 0 and its row maxima; K operands of
    // block 1 and V^T operands of block 0 in registers.
    load_tile(0, 0);
    if (n_kv > 1) load_tile(1, 1);
    publish();
    // Q has landed too (publish waited for every load); these uses make the compiler place
    // its own wait for Q here, not inside the loop where tile loads are in flight
#pragma unroll
    for (int ks = 0; ks < kNKS; ++ks) asm volatile("" : "+a"(qa[ks]), "+a"(qb[ks]));
    // likewise the scalar loads of the output pointers: while one is pending the compiler
    // can wait for LDS reads only with lgkmcnt(0) (scalar loads complete out of order)
    asm volatile("" :: "s"(O), "s"(LSE));
    f32x16 s0a, s0b, s1a, s1b;
    float ma = 0.f, mb = 0.f;
    if (nb_live > 0) {
#pragma unroll
        for (int ks = 0; ks < kNKS; ++ks) rk(ks, 0, 0);
        M::s_first(s0a, ka[0], qa[0]);
        M::s_first(s0b, ka[0], qb[0]);
#pragma unroll
        for (int ks = 1; ks < kNKS; ++ks) {
            M::s_next(s0a, ka[ks], qa[ks]);
            M::s_next(s0b, ka[ks], qb[ks]);
        }
#pragma unroll
        for (int ks = 0; ks < kNKS; ++ks) rk(ks, 0, 1);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int db = 0; db < kNDB; ++db) rv(h, db, 0, 0);
        mfma_drain();
        ma = rowmax(s0a);
        mb = rowmax(s0b);
    }

    // The block at position U (0..5) of a trip over three tiles (tile k of the trip in stage
    // k): K read-ahead at position U + 2, V^T read-ahead at U + 1.  Even positions are a
    // tile's first block and carry the loads of tile dj (stage: that of the previous tile).
    auto block = [&](int bi, auto u, int dj) {
        constexpr int U = decltype(u)::value;
        constexpr bool FIRST = U % 2 == 0;
        constexpr int DST = (U / 2 + kNST - 1) % kNST;
        if (bi >= nb_live) {
            // past the wave's rows (causal): it still loads its part of the tiles
            if constexpr (FIRST) {
                if (dj >= 0) load_tile(dj, DST);
            }
            return;
        }
        constexpr int KU = (U + 2) % (2 * kNST), VU = (U + 1) % (2 * kNST);
        using kst = std::integral_constant<int, KU / 2>;
        using kkb = std::integral_constant<int, KU % 2>;
        using vst = std::integral_constant<int, VU / 2>;
        using vkb = std::integral_constant<int, VU % 2>;
        using first = std::integral_constant<bool, FIRST>;
        float mu_a, mu_b;
        if constexpr (U % 2 == 0) {
            stats(bi, s0a, s0b, ma, mb, mu_a, mu_b);
            region(kst{}, kkb{}, vst{}, vkb{}, first{}, dj, DST, s0a, s0b, s1a, s1b, mu_a, mu_b, ma, mb);
        } else {
            stats(bi, s1a, s1b, ma, mb, mu_a, mu_b);
            region(kst{}, kkb{}, vst{}, vkb{}, first{}, dj, DST, s1a, s1b, s0a, s0b, mu_a, mu_b, ma, mb);
        }
        // past its last block a wave's read-ahead is never consumed: let it land before the
        // barriers that hand its stages to new loads
        if (bi == nb_live - 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };
    // end of tile t: tile t + 2 published, and tile t's stage free
    auto boundary = [&](int t) {
        if (t + 2 < n_kv) publish();
    };
    // the loads that tile t's first block issues: tile t + 2, into the stage of tile t - 1
    // (freed by the barrier at the end of tile t - 1; for t = 0 never used yet)
    auto loads_of = [&](int t) { return t + kNST - 1 < n_kv ? t + kNST - 1 : -1; };
    auto tile_step = [&](int t0, auto kc) {
        constexpr int k = decltype(kc)::value;
        const int t = t0 + k;
        if (t >= n_kv) return;
        block(2 * t, std::integral_constant<int, 2 * k>{}, loads_of(t));
        block(2 * t + 1, std::integral_constant<int, 2 * k + 1>{}, -1);
        boundary(t);
    };
    static_assert(kNST == 3, "a trip covers three tiles");
    for (int t0 = 0; t0 < n_kv; t0 += kNST) {
        tile_step(t0, std::integral_constant<int, 0>{});
        tile_step(t0, std::integral_constant<int, 1>{});
        tile_step(t0, std::integral_constant<int, 2>{});
    }

    // a8: epilogue -- O = O~ / l, LSE = (m_ref + log2 l) ln 2
    auto store = [&](auto r) {
        constexpr int R = decltype(r)::value, x = R / 4, db = R % 4;
        const int q = q0w + 32 * x + l32;
        float o[16];
        oacc_read<R>(o);
        if (q >= N) return;
        const float l_tot = l_run[x] + xor_lanes(l_run[x], 32);
        // v_rcp_f32 (about 1 ulp of fp32): far below the 16-bit rounding of the output
        const float inv_l = __builtin_amdgcn_rcpf(l_tot);
        uint16_t* orow = O + (qh_off + q) * kD;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const u32x2 w = {E::pack2(o[4 * a + 0] * inv_l, o[4 * a + 1] * inv_l),
                             E::pack2(o[4 * a + 2] * inv_l, o[4 * a + 3] * inv_l)};
            *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * a + 4 * g) = w;
        }
        if (db == 0 && g == 0) LSE[qh_off + q] = (m_ref[x] + fast_log2(l_tot)) * kLn2;
    };
    store(std::integral_constant<int, 0>{});
    store(std::integral_constant<int, 1>{});
    store(std::integral_constant<int, 2>{});
    store(std::integral_constant<int, 3>{});
    store(std::integral_constant<int, 4>{});
    store(std::integral_constant<int, 5>{});
    store(std::integral_constant<int, 6>{});
    store(std::integral_constant<int, 7>{});
}

template <bool IS_BF16, bool CAUSAL>
hipError_t launch_t(const PrefillArgs& a) {
    const int n_qtiles = (a.N + kBR - 1) / kBR;
    const int n_hg = a.B * a.Hkv;
    const long long n_items = (long long)n_qtiles * a.B * a.Hq;
    const int xcd_major = (n_hg % 8 == 0) ? 1 : 0;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    return launch_kernel(prefill_d128_kernel<IS_BF16, CAUSAL>, dim3((unsigned)n_items),
                         dim3(64 * kW), (hipStream_t)a.stream, "prefill_d128_kernel", a.Q, a.K,
                         a.V, a.O, a.LSE, a.B, a.Hq, a.Hkv, a.N, scale_log2, n_qtiles, xcd_major);
}

}  // namespace

bool prefill_d128_applies(const PrefillArgs& a) {
    if (a.d != 128 || a.N <= 2048) return false;
    // one workgroup per CU: below two 256-row items per CU the 128-row kernel, two
    // workgroups per CU, fills the chip better
    const long long n_items = (long long)((a.N + kBR - 1) / kBR) * a.B * a.Hq;
    return n_items >= 2LL * device_cu_count();
}

hipError_t launch_prefill_d128(const PrefillArgs& a) {
    if (a.is_bf16) return a.causal ? launch_t<true, true>(a) : launch_t<true, false>(a);
    return a.causal ? launch_t<false, true>(a) : launch_t<false, false>(a);
}

}  // namespace attn
