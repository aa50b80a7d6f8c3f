// read_probe.hip - a streaming-read calibration kernel for the benchmark (not part of libmoe.so):
// the rate at which this GPU reads a cold buffer once, the ceiling the layer's HBM figures are
// set against next to the 8 TB/s specification.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Grid-stride over n16 16-byte pieces, four non-temporal loads in flight per lane. The XOR of
// the data goes to *sink only if it equals a fixed value, so the loads are not dropped and
// nothing is written in practice.
__global__ __launch_bounds__(512) void read_kernel(const u32x4_t *__restrict__ p, size_t n16,
                                                   unsigned *sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    unsigned acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4_t a = __builtin_nontemporal_load(p + i);
        const u32x4_t b = __builtin_nontemporal_load(p + i + stride);
        const u32x4_t c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4_t d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
               d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const u32x4_t a = __builtin_nontemporal_load(p + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9e3779b9u) *sink = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16; src 16-byte aligned) from device memory at `src` once, with
// `blocks` blocks of 512 threads on `stream` (a hipStream_t, or null for the default stream).
// `sink` is one device word the kernel may write. Returns 0, or the HIP error code.
extern "C" int moe_probe_read(const void *src, size_t bytes, int blocks, unsigned *sink,
                              void *stream) {
    if (!src || !sink || bytes % 16 || (uintptr_t)src % 16 || blocks < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                       reinterpret_cast<const u32x4_t *>(src), bytes / 16, sink);
    return (int)hipGetLastError();
}
