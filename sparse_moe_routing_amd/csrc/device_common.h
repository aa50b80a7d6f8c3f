// device_common.h - shared device helpers for the gfx950 kernels of libmoe.
//
// Element "ops": the kernels are written once over an element type. Each lane of a wave loads
// 16 bytes of a row at a time; the op turns a pair of such 16-byte fragments (A: a weight row,
// B: an activation row) into matrix-core instructions on a 16x16 output tile:
//   bf16: one v_mfma_f32_16x16x32_bf16 per fragment pair (8 elements per lane, 32 per tile step)
//   f32 : four v_mfma_f32_16x16x4_f32 per fragment pair (4 elements per lane, 16 per tile step)
// Lane l supplies row (l % 16) of A and column (l % 16) of B, and k-group q = l / 16. A and B use
// the same (q, element) -> k assignment, so every k of the step is summed exactly once whatever
// order the instruction uses inside a k-group. The accumulator tile: lane l holds rows
// 4 * (l / 16) + r, r = 0..3, of column l % 16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kTopK = 8;
constexpr int kTile = 16;  // MFMA tile edge (rows of A, columns of B)

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs; used only on finite intermediates).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

struct OpBF16 {
    using elem_t = uint16_t;
    static constexpr int kElemBytes = 2;
    static constexpr int kPerLane = 8;    // elements in one 16-byte fragment
    static constexpr int kStep = 32;      // k covered by one fragment pair across the 4 k-groups
    __device__ static __forceinline__ void mma(f32x4_t &acc, const uint4 &a, const uint4 &b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, b), acc, 0, 0,
                                                      0);
    }
};

struct OpF32 {
    using elem_t = float;
    static constexpr int kElemBytes = 4;
    static constexpr int kPerLane = 4;
    static constexpr int kStep = 16;
    __device__ static __forceinline__ void mma(f32x4_t &acc, const uint4 &a, const uint4 &b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc,
                                                   0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc,
                                                   0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc,
                                                   0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc,
                                                   0, 0, 0);
    }
};

__device__ __forceinline__ uint4 load16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// Weight streams are read once per call: a non-temporal load keeps them from evicting the
// activations and the routing tables other blocks reuse.
__device__ __forceinline__ uint4 load16_stream(const void *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return uint4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Device-coherent access for data that one wave writes and a wave on another XCD reads inside the
// same launch: relaxed agent-scope atomic loads and stores (on gfx950 these carry the device
// scope bit: stores write through the XCD's L2, loads do not hit a stale L2 line), so a producer
// publishes by waiting for its stores (vmcnt) before a counter update and the consumer needs no
// L2 invalidation. Element types of at most 8 bytes.
template <class T>
__device__ __forceinline__ T ld_dev(const T *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ void st_dev(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint4 ld_dev16(const void *p) {
    const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
    const uint64_t a = ld_dev(q), b = ld_dev(q + 1);
    return uint4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}
__device__ __forceinline__ void st_dev16(void *p, uint4 v) {
    uint64_t *q = reinterpret_cast<uint64_t *>(p);
    st_dev(q, (uint64_t)v.x | ((uint64_t)v.y << 32));
    st_dev(q + 1, (uint64_t)v.z | ((uint64_t)v.w << 32));
}
// Wait until every memory operation this wave issued has completed (its device-scope stores are
// then visible device-wide); a compiler barrier on both sides keeps them on their side.
__device__ __forceinline__ void wait_own_stores() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt not waited for
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace moe
