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

#include <type_traits>

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

// Buffer loads. A buffer resource (wave-uniform, four scalar registers) covers `bytes` bytes from
// `base`; a load whose offset lies past them returns zero and makes no memory access. A kernel that
// keeps a fixed number of loads in flight (so that the compiler's wait counts stay exact) issues
// its loads with nothing to read this way - with `bytes` = 0, or an offset past the range - instead
// of re-reading some cached address: thousands of waves re-reading one line all queue on the one
// L2 channel that holds it. The fourth descriptor word is the data-format field the gfx9-family
// parts take for untyped (raw) buffer access; offsets are 32-bit, so a resource covers < 4 GiB.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
constexpr int kBufNT = 2;  // cache-policy bit of a non-temporal (streamed) load
__device__ __forceinline__ uint4 bload16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kBufNT));
}
__device__ __forceinline__ u32x2_t bload8_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kBufNT));
}
__device__ __forceinline__ uint32_t bload4_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kBufNT);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t bload1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// Expert-weight storage formats. A weight "piece" is the Op::kPerLane elements one lane feeds to
// one matrix-core fragment (16 bytes of operand data). WeightFmt<Op, false> stores the operand
// type itself; WeightFmt<OpBF16, true> stores OCP FP8 E4M3 codes (8 bytes per piece) that are
// widened to bf16 exactly on load (every E4M3 value is a bf16 value; gfx950 converts two codes
// per instruction) and whose per-row scale is applied to the fp32 product afterwards:
// sum_k (code_k * s) x_k = s * sum_k code_k x_k.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Codes of bytes 2*kHi and 2*kHi + 1 of w as two bf16 (low half: the lower byte).
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    const bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    return uint4{e4m3x2_to_bf16x2<false>(lo), e4m3x2_to_bf16x2<true>(lo),
                 e4m3x2_to_bf16x2<false>(hi), e4m3x2_to_bf16x2<true>(hi)};
}

// MXFP4 (the Open Compute Project's Microscaling FP4): E2M1 codes two per byte (the even weight
// in the low nibble) and one E8M0 scale byte per 32 consecutive weights. The scale byte as the
// fp32 2^(b - 127) (b = 0: the subnormal 2^-127; b = 255: NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    return __uint_as_float(b == 0 ? 0x00400000u : b == 255 ? 0x7FC00000u : b << 23);
}

// The two codes of byte kByte of w times s as two bf16 (low half: the low nibble). gfx950
// converts and scales in one instruction, exactly while the product is a finite bf16.
template <int kByte>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t w, float s) {
    const bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, kByte);
    return __builtin_bit_cast(uint32_t, v);
}

// Eight codes (one 32-bit word, weights 8j .. 8j + 7 of a scale block) as one bf16 operand piece.
__device__ __forceinline__ uint4 e2m1x8_to_bf16x8(uint32_t w, float s) {
    return uint4{e2m1x2_to_bf16x2<0>(w, s), e2m1x2_to_bf16x2<1>(w, s),
                 e2m1x2_to_bf16x2<2>(w, s), e2m1x2_to_bf16x2<3>(w, s)};
}

// Wait states between the matrix instructions of one chunk and the scaled conversions (FP4, FP8)
// of the next: a matrix instruction still reads its A/B registers for several cycles after it
// issues, and the conversions may be allocated those registers; without this gap the last matrix
// steps before a conversion block read the new values (measured on gfx950 for the FP4 ones:
// exactly those steps' products were wrong). The FP8 conversions are the same instruction family
// and passed as built, but nothing but register allocation kept them clear, so they take the guard
// too (about 1 % of an FP8 round), except in the large-T gate/up kernel, where any such barrier
// makes the compiler spill; bitwise tests against bf16 contexts holding the decoded weights pin
// every path. The scheduling barriers keep every instruction on its side.
__device__ __forceinline__ void mfma_operand_guard() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);
}

// Stage position of operand piece p (0..15) of an MXFP4 chunk row, before the row swizzle: each
// group of four pieces (one lane's scale block) is rotated by its group index and by the stage
// buffer b, so that the eight lanes that write one row in one LDS instruction (one piece each)
// hit eight distinct 16-byte bank groups. Writer and operand reader use the same map.
__device__ __forceinline__ int mx_piece_pos(int p, int b) {
    return (p & 12) | (((p & 3) + (p >> 2) + b) & 3);
}

// The same for FP8 E4M3 chunks, where each of a row's 8 lanes writes pieces 2j and 2j + 1: the
// upper half of the row's pieces swaps pairs, so that one LDS instruction's 8 pieces are 8
// distinct bank groups.
__device__ __forceinline__ int fp8_piece_pos(int p) { return p ^ ((p >> 3) & 1); }

template <class Op, bool kFp8>
struct WeightFmt {
    static_assert(!kFp8 || Op::kElemBytes == 2, "FP8 weights feed bf16 matrix-core operands");
    using wt_t = typename std::conditional<kFp8, uint8_t, typename Op::elem_t>::type;
    // a piece as stored (8 bytes of FP8 codes, 16 bytes otherwise), kept in registers until it
    // is staged, so that FP8 holds twice the elements in flight in the same registers
    using raw_t = typename std::conditional<kFp8, u32x2_t, uint4>::type;
    static constexpr bool kScaled = kFp8;
    __device__ static __forceinline__ raw_t load_raw(const wt_t *p) {
        if constexpr (kFp8) return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
        else return load16_stream(p);
    }
    __device__ static __forceinline__ uint4 to_operand(const raw_t &r) {
        if constexpr (kFp8) return e4m3x8_to_bf16x8(r.x, r.y);
        else return r;
    }
    // one piece from p (element address), streamed (read once per call)
    __device__ static __forceinline__ uint4 piece(const wt_t *p) {
        if constexpr (kFp8) {
            const u32x2_t c = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
            return e4m3x8_to_bf16x8(c.x, c.y);
        } else {
            return load16_stream(p);
        }
    }
    // the same through the caches (weights other units re-read)
    __device__ static __forceinline__ uint4 piece_cached(const wt_t *p) {
        if constexpr (kFp8) {
            const uint2 c = *reinterpret_cast<const uint2 *>(p);
            return e4m3x8_to_bf16x8(c.x, c.y);
        } else {
            return load16(p);
        }
    }
};

// acc rows 4q + r (r = 0..3) of a tile times their row scales scale[0..3] (FP8 weights).
__device__ __forceinline__ void scale_rows(f32x4_t &acc, const float *scale) {
    const float4 s = *reinterpret_cast<const float4 *>(scale);
    acc[0] *= s.x;
    acc[1] *= s.y;
    acc[2] *= s.z;
    acc[3] *= s.w;
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
