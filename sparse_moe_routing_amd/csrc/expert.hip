// expert.hip - the expert stage: gate/up GEMM + SwiGLU + down GEMM over token groups, and the
// weighted combine with the shared expert.
//
// Decode rounds touch each selected expert with one or two tokens, so the stage is a stream of
// expert weights read once from HBM (the expert block dominates a MoE model's bytes and decode is
// bandwidth-bound: "RELEASE_NOTES_0.9.0" of the 16 GB ninfer fork, the expert-placement
// paragraphs). A unit of work is (group of up to 16 tokens routed to one expert, chunk of
// 16-wide slices of the intermediate dimension):
//   1. the group's x rows are staged in LDS (bf16 or fp32, row stride padded by 16 bytes so the
//      16 rows fall in different banks);
//   2. wave w (< s/16) computes the 16x16 gate tile and the 16x16 up tile of intermediate rows
//      j*s + 16w .. +16 with MFMA, streaming the weight rows straight from HBM into the A
//      operand (each weight fragment feeds exactly one instruction), then h = silu(gate) * up
//      in fp32 into LDS;
//   3. all four waves stream the matching [H x s] column block of the down weight and multiply
//      it by h. For bf16, h is split into hi = bf16(h) and lo = bf16(h - hi) and both terms go
//      through the bf16 MFMA, so the product keeps ~16 mantissa bits of h (a plain bf16 h would
//      lose ~5e-4 absolute accuracy on y);
//   4. the [tokens x H] result is written to the unit's slot rows of the partial buffer (token
//      slot = pair index t*8 + k, or T*8 + t for the shared expert); later slices of the same
//      unit accumulate into it in order.
// No atomics anywhere: every partial row has exactly one writer, and the combine kernel sums the
// partials of each token in a fixed order, so results are deterministic and independent of how
// the work was spread over the GPU.
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kExpertThreads = 256;
constexpr int kUnroll = 8;

__device__ __forceinline__ uint4 lds16(const void *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

template <class Op>
__global__ __launch_bounds__(kExpertThreads) void expert_kernel(ExpertParams p) {
    using elem_t = typename Op::elem_t;
    extern __shared__ __align__(16) unsigned char smem[];
    elem_t *xs = reinterpret_cast<elem_t *>(smem);
    const int hs_stride = p.s + 4;
    float *hs = reinterpret_cast<float *>(smem + (size_t)p.NG * p.x_stride * sizeof(elem_t));

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, q = lane >> 4;
    const int n_sc = p.S / p.SPU;
    const int nunits = p.num_groups[0] * n_sc;
    const int chunks_per_row = p.H / Op::kPerLane;
    const int n_row_tiles = p.H / kTile;
    const elem_t *x = reinterpret_cast<const elem_t *>(p.x);
    const uint4 zero = {0u, 0u, 0u, 0u};

    for (int u = blockIdx.x; u < nunits; u += gridDim.x) {
        const int gi = u / n_sc, sc = u - (u / n_sc) * n_sc;
        const int4 grp = p.groups[gi];
        const int e = grp.x, start = grp.y, n = grp.z;
        const bool shared = e == p.E;
        const int Ie = shared ? p.Is : p.I;
        const int j_begin = sc * p.SPU;
        if (j_begin * p.s >= Ie) continue;  // uniform over the block
        const int j_end = min(j_begin + p.SPU, Ie / p.s);

        __syncthreads();  // the previous unit's readers of xs / hs are done
        for (int idx = tid; idx < n * chunks_per_row; idx += kExpertThreads) {
            const int row = idx / chunks_per_row;
            const int c = idx - row * chunks_per_row;
            const int tok = shared ? start + row : (p.perm[start + row] >> 3);
            *reinterpret_cast<uint4 *>(xs + row * p.x_stride + c * Op::kPerLane) =
                load16(x + (size_t)tok * p.H + c * Op::kPerLane);
        }
        const bool col_ok = col < n;
        const int slot = !col_ok ? 0 : (shared ? p.T * kTopK + start + col : p.perm[start + col]);
        const elem_t *gu = reinterpret_cast<const elem_t *>(shared ? p.sgu : p.gate_up) +
                           (shared ? 0 : (size_t)e * 2 * Ie * p.H);
        const elem_t *dn = reinterpret_cast<const elem_t *>(shared ? p.sdn : p.down) +
                           (shared ? 0 : (size_t)e * p.H * Ie);
        float *yout = p.ypart + ((size_t)sc * p.slots + slot) * p.H;
        __syncthreads();

        for (int j = j_begin; j < j_end; ++j) {
            // ---- gate/up tiles + SwiGLU
            if (wave < p.s / kTile) {
                const int i0 = j * p.s + wave * kTile;
                const elem_t *grow = gu + (size_t)(i0 + col) * p.H + q * Op::kPerLane;
                const elem_t *urow = gu + (size_t)(Ie + i0 + col) * p.H + q * Op::kPerLane;
                const elem_t *xrow = xs + (col_ok ? col : 0) * p.x_stride + q * Op::kPerLane;
                f32x4_t ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
                for (int k0 = 0; k0 < p.H; k0 += kUnroll * Op::kStep) {
                    uint4 ga[kUnroll], ua[kUnroll], xb[kUnroll];
#pragma unroll
                    for (int v = 0; v < kUnroll; ++v) {
                        const int kk = k0 + v * Op::kStep;
                        if (kk < p.H) {
                            ga[v] = load16_stream(grow + kk);
                            ua[v] = load16_stream(urow + kk);
                        }
                    }
#pragma unroll
                    for (int v = 0; v < kUnroll; ++v) {
                        const int kk = k0 + v * Op::kStep;
                        if (kk < p.H) xb[v] = col_ok ? lds16(xrow + kk) : zero;
                    }
#pragma unroll
                    for (int v = 0; v < kUnroll; ++v) {
                        const int kk = k0 + v * Op::kStep;
                        if (kk < p.H) {
                            Op::mma(ag, ga[v], xb[v]);
                            Op::mma(au, ua[v], xb[v]);
                        }
                    }
                }
                f32x4_t hv;
#pragma unroll
                for (int r = 0; r < 4; ++r) hv[r] = ag[r] / (1.0f + expf(-ag[r])) * au[r];
                // lane holds intermediate rows 4q + r of this tile for token column `col`
                *reinterpret_cast<f32x4_t *>(hs + col * hs_stride + wave * kTile + 4 * q) = hv;
            }
            __syncthreads();

            // ---- B fragments of the down product: h^T for this slice
            constexpr int kMaxSteps = 64 / Op::kStep;  // s <= 64
            const int nsteps = p.s / Op::kStep;
            uint4 bhi[kMaxSteps], blo[kMaxSteps];
#pragma unroll
            for (int st = 0; st < kMaxSteps; ++st) {
                bhi[st] = zero;
                blo[st] = zero;
                if (st < nsteps && col_ok) {
                    const float *hp = hs + col * hs_stride + st * Op::kStep + q * Op::kPerLane;
                    if constexpr (Op::kElemBytes == 2) {
                        uint32_t hw[4], lw[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float h0 = hp[2 * i], h1 = hp[2 * i + 1];
                            const uint32_t a0 = f32_to_bf16_bits(h0), a1 = f32_to_bf16_bits(h1);
                            const uint32_t l0 = f32_to_bf16_bits(h0 - bf16_bits_to_f32(a0));
                            const uint32_t l1 = f32_to_bf16_bits(h1 - bf16_bits_to_f32(a1));
                            hw[i] = a0 | (a1 << 16);
                            lw[i] = l0 | (l1 << 16);
                        }
                        bhi[st] = uint4{hw[0], hw[1], hw[2], hw[3]};
                        blo[st] = uint4{lw[0], lw[1], lw[2], lw[3]};
                    } else {
                        bhi[st] = uint4{__float_as_uint(hp[0]), __float_as_uint(hp[1]),
                                        __float_as_uint(hp[2]), __float_as_uint(hp[3])};
                    }
                }
            }
            __syncthreads();  // hs may be overwritten by the next slice from here on

            // ---- down tiles: rows rt*16 .. +16 of the [H x s] column block
            const elem_t *dcol = dn + (size_t)col * Ie + j * p.s + q * Op::kPerLane;
            for (int rt0 = wave; rt0 < n_row_tiles; rt0 += 4 * kUnroll) {
                uint4 a[kUnroll][kMaxSteps];
#pragma unroll
                for (int v = 0; v < kUnroll; ++v) {
                    const int rt = rt0 + 4 * v;
#pragma unroll
                    for (int st = 0; st < kMaxSteps; ++st)
                        if (rt < n_row_tiles && st < nsteps)
                            a[v][st] = load16_stream(dcol + (size_t)rt * kTile * Ie + st * Op::kStep);
                }
#pragma unroll
                for (int v = 0; v < kUnroll; ++v) {
                    const int rt = rt0 + 4 * v;
                    if (rt >= n_row_tiles) break;
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < kMaxSteps; ++st) {
                        if (st < nsteps) {
                            Op::mma(acc, a[v][st], bhi[st]);
                            if constexpr (Op::kElemBytes == 2) Op::mma(acc, a[v][st], blo[st]);
                        }
                    }
                    if (col_ok) {
                        f32x4_t *dst = reinterpret_cast<f32x4_t *>(yout + rt * kTile + 4 * q);
                        if (j == j_begin) *dst = acc;
                        else *dst = *dst + acc;
                    }
                }
            }
        }
    }
}

// y[t] = sum_k w[t][k] * (sum of the routed partials of pair t*8+k) + g[t] * (shared partials)
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
    const int hchunks = (p.H / 4 + 255) / 256;
    const int t = blockIdx.x / hchunks;
    const int h = ((blockIdx.x - t * hchunks) * 256 + threadIdx.x) * 4;
    if (h >= p.H) return;
    const size_t chunk = (size_t)p.slots * p.H;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kTopK; ++k) {
        const float *src = p.ypart + (size_t)(t * kTopK + k) * p.H + h;
        float4 s = *reinterpret_cast<const float4 *>(src);
        for (int c = 1; c < p.n_sc_routed; ++c) {
            const float4 v = *reinterpret_cast<const float4 *>(src + c * chunk);
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        const float wk = p.w[t * kTopK + k];
        acc.x += wk * s.x; acc.y += wk * s.y; acc.z += wk * s.z; acc.w += wk * s.w;
    }
    if (p.has_shared) {
        const float *src = p.ypart + (size_t)(p.T * kTopK + t) * p.H + h;
        float4 s = *reinterpret_cast<const float4 *>(src);
        for (int c = 1; c < p.n_sc_shared; ++c) {
            const float4 v = *reinterpret_cast<const float4 *>(src + c * chunk);
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        const float gt = p.g[t];
        acc.x += gt * s.x; acc.y += gt * s.y; acc.z += gt * s.z; acc.w += gt * s.w;
    }
    *reinterpret_cast<float4 *>(p.y + (size_t)t * p.H + h) = acc;
}

hipError_t prepare_expert_kernels(size_t max_lds_bytes) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&expert_kernel<OpBF16>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)max_lds_bytes);
    if (err != hipSuccess) return err;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&expert_kernel<OpF32>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)max_lds_bytes);
}

hipError_t launch_expert(const ExpertParams &p, int dtype, int grid, size_t lds_bytes,
                         hipStream_t s) {
    if (dtype == 1) expert_kernel<OpBF16><<<grid, kExpertThreads, lds_bytes, s>>>(p);
    else expert_kernel<OpF32><<<grid, kExpertThreads, lds_bytes, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineParams &p, hipStream_t s) {
    const int hchunks = (p.H / 4 + 255) / 256;
    combine_kernel<<<hchunks * p.T, 256, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace moe
