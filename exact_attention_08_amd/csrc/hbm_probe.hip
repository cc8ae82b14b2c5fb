// hbm_probe.hip -- a plain streaming read of one device buffer, used by the benchmark to show
// the HBM read bandwidth a simple kernel reaches on this GPU (the practical ceiling beside
// the nominal 8 TB/s).  Not part of the attention library.
//
// Each thread reads 16-byte pieces, 8 loads in flight, in a grid-stride loop; the loads are
// non-temporal (every byte is read once).  The XOR of the data is stored per thread so the
// loads cannot be dropped.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const u32x4* __restrict__ src,
                                                            size_t n16, uint32_t* __restrict__ out) {
    const size_t stride = (size_t)gridDim.x * kThreads * kUnroll;
    uint32_t acc = 0;
    for (size_t base = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n16;
         base += stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t i = base + (size_t)u * kThreads;
            v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from src with `blocks` workgroups of 256 threads; out
// must hold blocks * 256 uint32.  Returns 0, or -1 for bad arguments, -7 if the launch
// failed.
extern "C" int hbm_read_probe(const void* src, size_t bytes, uint32_t* out, int blocks,
                              void* stream) {
    if (!src || !out || blocks <= 0 || bytes % 16 != 0) return -1;
    hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, (const u32x4*)src, bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}
