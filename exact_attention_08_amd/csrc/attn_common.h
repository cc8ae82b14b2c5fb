// attn_common.h -- device helpers shared by the prefill and decode kernels (gfx950 only).
//
// Operand conventions of the CDNA4 matrix instructions used here (wave64):
//   v_mfma_f32_32x32x16_{bf16,f16}: A lane l holds row l%32, 8 k-values of k-group l/32;
//     B lane l holds column l%32, the same 8 k-values; D lane l holds column l%32 and
//     rows 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
//   v_mfma_f32_16x16x32_{bf16,f16}: A lane l holds row l%16, 8 k-values of k-group l/16;
//     B lane l holds column l%16; D lane l holds column l%16 and rows 4*(l/16) + v, v = 0..3.
//   v_mfma_f32_16x16x16_{bf16,f16}: as above with 4 k-values per lane (k-group l/16).
// Only the pairing of A's and B's k-values matters for the product, so the kernels choose
// the k order freely as long as A and B use the same one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;

// Element traits: storage is always 16 bits; IS_BF16 picks the MFMA flavour and the
// fp32 -> 16-bit conversion (both round to nearest even).
template <bool IS_BF16> struct Elem;

template <> struct Elem<true> {
    __device__ static inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ static inline f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ static inline f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                         __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
    }
    // two fp32 -> packed pair of 16-bit values (x in the low half)
    __device__ static inline uint32_t pack2(float x, float y) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        bf16x2 r;
        r[0] = (__bf16)x;
        r[1] = (__bf16)y;
        return __builtin_bit_cast(uint32_t, r);
    }
};

template <> struct Elem<false> {
    __device__ static inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ static inline f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ static inline f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
    }
    __device__ static inline uint32_t pack2(float x, float y) {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        f16x2 r;
        r[0] = (_Float16)x;
        r[1] = (_Float16)y;
        return __builtin_bit_cast(uint32_t, r);
    }
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }   // v_log_f32

__device__ inline float xor_lanes(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ inline u32x4 ldg16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ inline u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

}  // namespace attn
