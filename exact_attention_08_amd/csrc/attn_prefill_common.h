// attn_prefill_common.h -- device helpers shared by the prefill kernels (gfx950 only): the
// work-item order, the K/V staging (buffer descriptors, loads that write LDS, the row
// swizzles) and small arithmetic helpers.
#pragma once

#include "attn_common.h"

namespace attn {

constexpr float kRescaleSlack = 8.0f;     // log2 headroom before the reference max moves

struct WorkItem { int qt, b, h, kvh; };

// a1: work item -> (q tile, batch, head).  A head group is a (batch, kv head) with its G
// query heads; its n_qtiles * G items are numbered heaviest tile first.  When the head
// groups divide evenly over the 8 XCDs (workgroups reach XCDs round robin), items are
// interleaved so that item i belongs to XCD i % 8 and head group hg lives entirely on XCD
// hg % 8, so its K/V stays in that XCD's L2.
__device__ inline WorkItem prefill_work_item(int bid, int n_qtiles, int Hkv, int G,
                                             int xcd_major) {
    const int per = n_qtiles * G;
    int hg, within;
    if (xcd_major) {
        const int xcd = bid & 7, slot = bid >> 3;
        hg = xcd + 8 * (slot / per);
        within = slot % per;
    } else {
        hg = bid / per;
        within = bid % per;
    }
    WorkItem w;
    w.qt = n_qtiles - 1 - within / G;
    w.b = hg / Hkv;
    w.kvh = hg % Hkv;
    w.h = w.kvh * G + within % G;
    return w;
}

__device__ inline __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
// buffer descriptor as four dwords (base, stride 0, byte range, flags) for inline asm
__device__ inline i32x4 head_rsrc4(const uint16_t* base, int bytes) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    return i32x4{(int)(uint32_t)b, (int)(uint32_t)(b >> 32) & 0xFFFF, bytes, 0x00020000};
}
// 16 bytes per lane from buffer offset voff into LDS at lds_addr + 16 * lane.  Issued as
// inline asm: the compiler then places no wait for it before later LDS reads (the kernel
// waits on vmcnt itself before the barrier that publishes a tile).
__device__ __forceinline__ void dma_b128(i32x4 rsrc, uint32_t lds_addr, int voff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}
// LDS layout of a K or V tile: rows of D elements, unpadded; the 16-byte chunk c of row r
// sits in slot c ^ swz(r) of that row.  K is read as 16 bytes of one row per lane, 16 rows
// at a time; V by the transposing read, 8 bytes per lane over 4 rows: with these XORs
// either read touches every LDS bank once per pass.
template <int D> __device__ __forceinline__ int k_swz(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D> __device__ __forceinline__ int v_swz(int r) {
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// max(a, b, c) in one instruction.  For finite inputs the scores are finite or -inf, so the
// NaN canonicalisation the compiler adds to fmaxf's inputs is not needed (two fewer vector
// instructions per block).
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

}  // namespace attn
