// expert.hip - the expert stage: gate/up GEMM + SwiGLU + down GEMM over token groups, and the
// weighted combine with the shared expert.
//
// Decode rounds touch each selected expert with one or two tokens, so the stage is a stream of
// expert weights read once from HBM (the expert block dominates a MoE model's bytes and decode is
// bandwidth-bound: "RELEASE_NOTES_0.9.0" of the 16 GB ninfer fork, the expert-placement
// paragraphs). A unit of work is (group of up to 8 tokens routed to one expert, chunk of
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

__device__ __forceinline__ uint4 lds16(const void *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

// SW: slice width (intermediate rows per slice, 16 per gate/up wave); Op: element type.
template <class Op, int SW>
__global__ __launch_bounds__(kExpertThreads) void expert_kernel(ExpertParams p) {
    using elem_t = typename Op::elem_t;
    constexpr int kU = Op::kElemBytes == 2 ? 8 : 4;  // k steps / row tiles per load batch
    constexpr int kNst = SW / Op::kStep;             // k steps of the down product per slice
    constexpr int kGuWaves = SW / kTile;             // waves computing gate/up tiles
    static_assert(SW % Op::kStep == 0 && kGuWaves >= 1 && kGuWaves <= 4, "slice width");
    constexpr int kHs = SW + 4;                      // LDS row stride of h (floats)

    extern __shared__ __align__(16) unsigned char smem[];
    elem_t *xs = reinterpret_cast<elem_t *>(smem);
    float *hs = reinterpret_cast<float *>(smem + (size_t)p.NG * p.x_stride * sizeof(elem_t));

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, q = lane >> 4;
    const int n_sc = p.S / p.SPU;
    const int nunits = p.num_groups[0] * n_sc;
    const int chunks_per_row = p.H / Op::kPerLane;
    const int n_row_tiles = p.H / kTile;
    const int tiles_w = (n_row_tiles - wave + 3) / 4;  // down row tiles wave, wave+4, ...
    const int nfull3 = tiles_w / kU;
    const int nfull1 = p.H / (kU * Op::kStep);
    const int rem1 = nfull1 * kU * Op::kStep;
    const elem_t *x = reinterpret_cast<const elem_t *>(p.x);

    for (int u = blockIdx.x; u < nunits; u += gridDim.x) {
        const int gi = u / n_sc, sc = u - (u / n_sc) * n_sc;
        const int4 grp = p.groups[gi];
        const int e = grp.x, start = grp.y, n = grp.z;
        const bool shared = e == p.E;
        const int Ie = shared ? p.Is : p.I;
        const int j_begin = sc * p.SPU;
        if (j_begin * SW >= Ie) continue;  // uniform over the block
        const int j_end = min(j_begin + p.SPU, Ie / SW);

        __syncthreads();  // the previous unit's readers of xs / hs are done
        for (int idx = tid; idx < n * chunks_per_row; idx += kExpertThreads) {
            const int row = idx / chunks_per_row;
            const int c = idx - row * chunks_per_row;
            const int tok = shared ? start + row : (p.perm[start + row] >> 3);
            *reinterpret_cast<uint4 *>(xs + row * p.x_stride + c * Op::kPerLane) =
                load16(x + (size_t)tok * p.H + c * Op::kPerLane);
        }
        const bool col_ok = col < n;
        // Token columns >= n read row 0 of the tiles: matrix-core columns are independent, so
        // those columns only produce values that are never stored.
        const int crow = col_ok ? col : 0;
        const int slot = !col_ok ? 0 : (shared ? p.T * kTopK + start + col : p.perm[start + col]);
        const elem_t *gu = reinterpret_cast<const elem_t *>(shared ? p.sgu : p.gate_up) +
                           (shared ? 0 : (size_t)e * 2 * Ie * p.H);
        const elem_t *dn = reinterpret_cast<const elem_t *>(shared ? p.sdn : p.down) +
                           (shared ? 0 : (size_t)e * p.H * Ie);
        float *yout = p.ypart + ((size_t)sc * p.slots + slot) * p.H;
        __syncthreads();

        for (int j = j_begin; j < j_end; ++j) {
            const elem_t *dcol = dn + (size_t)col * Ie + j * SW + q * Op::kPerLane;
            uint4 dA[kU][kNst], dB[kU][kNst];
            // down weights of row-tile batch b: tiles wave + 4 * (b * kU + v)
            auto load_down = [&](uint4(&d)[kU][kNst], int b) {
#pragma unroll
                for (int v = 0; v < kU; ++v) {
                    const elem_t *src = dcol + (size_t)(wave + 4 * (b * kU + v)) * kTile * Ie;
#pragma unroll
                    for (int st = 0; st < kNst; ++st) d[v][st] = load16_stream(src + st * Op::kStep);
                }
            };

            // ---- gate/up tiles + SwiGLU: a double-buffered weight stream, then h into LDS
            if (wave < kGuWaves) {
                const int i0 = j * SW + wave * kTile;
                const elem_t *grow = gu + (size_t)(i0 + col) * p.H + q * Op::kPerLane;
                const elem_t *urow = gu + (size_t)(Ie + i0 + col) * p.H + q * Op::kPerLane;
                const elem_t *xrow = xs + crow * p.x_stride + q * Op::kPerLane;
                f32x4_t ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
                uint4 gA[kU], uA[kU], gB[kU], uB[kU];
                auto load_gu = [&](uint4(&g)[kU], uint4(&uu)[kU], int b) {
#pragma unroll
                    for (int v = 0; v < kU; ++v) {
                        const int kk = (b * kU + v) * Op::kStep;
                        g[v] = load16_stream(grow + kk);
                        uu[v] = load16_stream(urow + kk);
                    }
                };
                auto mma_gu = [&](const uint4(&g)[kU], const uint4(&uu)[kU], int b) {
#pragma unroll
                    for (int v = 0; v < kU; ++v) {
                        const uint4 xb = lds16(xrow + (b * kU + v) * Op::kStep);
                        Op::mma(ag, g[v], xb);
                        Op::mma(au, uu[v], xb);
                    }
                };
                if (nfull1 > 0) load_gu(gA, uA, 0);
                int b = 0;
                for (; b + 2 <= nfull1; b += 2) {
                    load_gu(gB, uB, b + 1);
                    mma_gu(gA, uA, b);
                    if (b + 2 < nfull1) load_gu(gA, uA, b + 2);
                    mma_gu(gB, uB, b + 1);
                }
                if (b < nfull1) mma_gu(gA, uA, b);
                for (int kk = rem1; kk < p.H; kk += Op::kStep) {  // only when H % (kU*step) != 0
                    const uint4 xb = lds16(xrow + kk);
                    Op::mma(ag, load16_stream(grow + kk), xb);
                    Op::mma(au, load16_stream(urow + kk), xb);
                }
                if (nfull3 > 0) load_down(dA, 0);  // the down stream does not depend on h
                f32x4_t hv;
#pragma unroll
                for (int r = 0; r < 4; ++r) hv[r] = ag[r] / (1.0f + expf(-ag[r])) * au[r];
                // lane holds intermediate rows 4q + r of this tile for token column `col`
                *reinterpret_cast<f32x4_t *>(hs + col * kHs + wave * kTile + 4 * q) = hv;
            } else if (nfull3 > 0) {
                load_down(dA, 0);
            }
            __syncthreads();

            // ---- B fragments of the down product: h^T of this slice
            uint4 bhi[kNst], blo[kNst];
#pragma unroll
            for (int st = 0; st < kNst; ++st) {
                const float *hp = hs + crow * kHs + st * Op::kStep + q * Op::kPerLane;
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
                    blo[st] = bhi[st];
                }
            }
            __syncthreads();  // hs may be overwritten by the next slice from here on

            // ---- down tiles: rows rt*16 .. +16 of the [H x SW] column block
            auto tile_out = [&](const uint4(&a)[kNst], int rt) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < kNst; ++st) {
                    Op::mma(acc, a[st], bhi[st]);
                    if constexpr (Op::kElemBytes == 2) Op::mma(acc, a[st], blo[st]);
                }
                if (col_ok) {
                    f32x4_t *dst = reinterpret_cast<f32x4_t *>(yout + rt * kTile + 4 * q);
                    if (j == j_begin) *dst = acc;
                    else *dst = *dst + acc;
                }
            };
            auto mma_down = [&](const uint4(&d)[kU][kNst], int b) {
#pragma unroll
                for (int v = 0; v < kU; ++v) tile_out(d[v], wave + 4 * (b * kU + v));
            };
            int b = 0;
            for (; b + 2 <= nfull3; b += 2) {
                load_down(dB, b + 1);
                mma_down(dA, b);
                if (b + 2 < nfull3) load_down(dA, b + 2);
                mma_down(dB, b + 1);
            }
            if (b < nfull3) mma_down(dA, b);
            for (int i = nfull3 * kU; i < tiles_w; ++i) {  // tiles past the last full batch
                const int rt = wave + 4 * i;
                uint4 a[kNst];
#pragma unroll
                for (int st = 0; st < kNst; ++st)
                    a[st] = load16_stream(dcol + (size_t)rt * kTile * Ie + st * Op::kStep);
                tile_out(a, rt);
            }
        }
    }
}

// y[t][h..h+4) = sum_k w[t][k] * (sum over slice chunks of the routed partials of pair t*8+k)
//               + g[t] * (sum over slice chunks of the shared partials of token t).
// One thread per 4 outputs, 64 threads per block, so even T = 4 spreads over 32 blocks.
__global__ __launch_bounds__(64) void combine_kernel(CombineParams p) {
    const int hblocks = (p.H + 255) / 256;
    const int t = blockIdx.x / hblocks;
    const int h = ((blockIdx.x - t * hblocks) * 64 + threadIdx.x) * 4;
    if (h >= p.H) return;
    const size_t chunk = (size_t)p.slots * p.H;
    constexpr int kMaxChunks = 8;
    // partial sums of one slot over its slice chunks: all loads issued before the adds, the
    // adds in chunk order (the same order an all-slices unit accumulates in)
    auto slot_sum = [&](int slot, int nch) {
        const float *src = p.ypart + (size_t)slot * p.H + h;
        float4 v[kMaxChunks];
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c)  // unconditional loads: chunks past nch re-read one
            v[c] = *reinterpret_cast<const float4 *>(src + (c < nch ? c : nch - 1) * chunk);
        float4 s = v[0];
#pragma unroll
        for (int c = 1; c < kMaxChunks; ++c) {
            const bool in = c < nch;
            s.x = in ? s.x + v[c].x : s.x;
            s.y = in ? s.y + v[c].y : s.y;
            s.z = in ? s.z + v[c].z : s.z;
            s.w = in ? s.w + v[c].w : s.w;
        }
        return s;
    };
    // a pair whose given id lies outside [0, E) was dropped by the bucketing: it adds zero
    auto valid = [&](int k) {
        const int e = p.ids[t * kTopK + k];
        return e >= 0 && e < p.E;
    };
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.w) {
#pragma unroll
        for (int k = 0; k < kTopK; ++k) {
            if (!valid(k)) continue;
            const float4 s = slot_sum(t * kTopK + k, p.n_sc_routed);
            const float wk = p.w[t * kTopK + k];
            acc.x += wk * s.x; acc.y += wk * s.y; acc.z += wk * s.z; acc.w += wk * s.w;
        }
        if (p.has_shared) {
            const float4 s = slot_sum(p.T * kTopK + t, p.n_sc_shared);
            const float gt = p.g[t];
            acc.x += gt * s.x; acc.y += gt * s.y; acc.z += gt * s.z; acc.w += gt * s.w;
        }
    } else {  // weighted partials, one chunk each: y = sum_k v_k + v_shared, in rank order
        // (each slot output is read exactly once: non-temporal loads keep it out of the caches)
        auto ld4 = [](const float *a) {
            const f32x4_t r = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(a));
            return make_float4(r[0], r[1], r[2], r[3]);
        };
        float4 v[kTopK + 1];
#pragma unroll
        for (int k = 0; k < kTopK; ++k)
            v[k] = valid(k) ? ld4(p.ypart + (size_t)(t * kTopK + k) * p.H + h)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        v[kTopK] = p.has_shared ? ld4(p.ypart + (size_t)(p.T * kTopK + t) * p.H + h)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < kTopK; ++k) {
            acc.x += v[k].x; acc.y += v[k].y; acc.z += v[k].z; acc.w += v[k].w;
        }
        if (p.has_shared) {
            acc.x += v[kTopK].x; acc.y += v[kTopK].y; acc.z += v[kTopK].z; acc.w += v[kTopK].w;
        }
    }
    *reinterpret_cast<float4 *>(p.y + (size_t)t * p.H + h) = acc;
}

template <class Op, int SW>
hipError_t set_lds_limit(size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&expert_kernel<Op, SW>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t prepare_expert_kernels(size_t max_lds_bytes) {
    hipError_t e;
    if ((e = set_lds_limit<OpBF16, 32>(max_lds_bytes)) != hipSuccess) return e;
    if ((e = set_lds_limit<OpBF16, 64>(max_lds_bytes)) != hipSuccess) return e;
    if ((e = set_lds_limit<OpF32, 16>(max_lds_bytes)) != hipSuccess) return e;
    if ((e = set_lds_limit<OpF32, 32>(max_lds_bytes)) != hipSuccess) return e;
    return set_lds_limit<OpF32, 64>(max_lds_bytes);
}

hipError_t launch_expert(const ExpertParams &p, int dtype, int grid, size_t lds_bytes,
                         hipStream_t s) {
    // dtype: 0 fp32, 1 bf16; the quantized weight formats have no variant of this kernel
    if (dtype != 0 && dtype != 1) return hipErrorInvalidValue;
    if (dtype == 1) {
        if (p.s == 64) launch_k(expert_kernel<OpBF16, 64>, grid, kExpertThreads, lds_bytes, s, p);
        else if (p.s == 32) launch_k(expert_kernel<OpBF16, 32>, grid, kExpertThreads, lds_bytes, s, p);
        else return hipErrorInvalidValue;
    } else {
        if (p.s == 64) launch_k(expert_kernel<OpF32, 64>, grid, kExpertThreads, lds_bytes, s, p);
        else if (p.s == 32) launch_k(expert_kernel<OpF32, 32>, grid, kExpertThreads, lds_bytes, s, p);
        else if (p.s == 16) launch_k(expert_kernel<OpF32, 16>, grid, kExpertThreads, lds_bytes, s, p);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_combine(const CombineParams &p, hipStream_t s) {
    launch_k(combine_kernel, ((p.H + 255) / 256) * p.T, 64, 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
