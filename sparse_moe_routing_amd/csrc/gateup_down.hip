// gateup_down.hip - the expert stage for decode and verify rounds (T <= 256) as two kernels.
//
// Decode rounds touch each selected expert with one or two tokens, so the stage is a stream of
// expert weights read once from HBM (the expert block dominates a MoE model's bytes and decode is
// bandwidth-bound: "RELEASE_NOTES_0.9.0" of the 16 GB ninfer fork, the expert-placement
// paragraphs). It is split so that each weight matrix is streamed in the order that suits it:
//
// gateup_kernel - one block per (expert group of <= 16 tokens, 64-row slice of the intermediate
//   dimension): the group's x rows are staged in LDS; wave w computes the 16x16 gate tile and
//   the 16x16 up tile of rows j*SW + 16w .. +16 with MFMA, the weight rows streaming from HBM
//   straight into the A operand; h = silu(gate) * up is written to the workspace, for bf16 as
//   two bf16 planes hi = bf16(h) and lo = bf16(h - hi) (so that the bf16 down product keeps ~16
//   mantissa bits of h), for fp32 as is. Row slot of a (token, rank) pair: t*8 + k; of the
//   shared expert for token t: T*8 + t.
//
// down_kernel - one block per (expert group, 64 rows of the output): the block reads that
//   expert's 64 down-weight rows (one contiguous block of 64 * I elements) and the group's h rows
//   (staged once in LDS) and writes w * (Wd h) for each of the group's (token, rank) pairs into
//   that pair's row of a [slots][H] buffer (w = the pair's routing weight, or the shared gate).
//   Every element of the buffer has exactly one writer; the combine kernel then sums a token's
//   eight ranks in rank order plus its shared slot. No atomics, and a token's bits do not depend
//   on the batch it came in.
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kThreads = 256;

__device__ __forceinline__ uint4 lds_load16(const void *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

template <class Op, int SW>
__global__ __launch_bounds__(kThreads) void gateup_kernel(GateUpParams p) {
    using elem_t = typename Op::elem_t;
    constexpr int kU = Op::kElemBytes == 2 ? 8 : 4;  // k steps per load batch
    constexpr int kGuWaves = SW / kTile;
    static_assert(kGuWaves >= 1 && kGuWaves <= 4, "slice width");

    extern __shared__ __align__(16) unsigned char smem[];
    elem_t *xs = reinterpret_cast<elem_t *>(smem);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, q = lane >> 4;
    const int nunits = p.num_groups[0] * p.S;
    const int chunks_per_row = p.H / Op::kPerLane;
    const int nfull = p.H / (kU * Op::kStep);
    const int rem = nfull * kU * Op::kStep;
    const elem_t *x = reinterpret_cast<const elem_t *>(p.x);

    for (int u = blockIdx.x; u < nunits; u += gridDim.x) {
        const int gi = u / p.S, j = u - (u / p.S) * p.S;
        const int4 grp = p.groups[gi];
        const int e = grp.x, start = grp.y, n = grp.z;
        const bool shared = e == p.E;
        const int Ie = shared ? p.Is : p.I;
        if (j * SW >= Ie) continue;  // uniform over the block

        __syncthreads();  // the previous unit's readers of xs are done
        for (int idx = tid; idx < n * chunks_per_row; idx += kThreads) {
            const int row = idx / chunks_per_row;
            const int c = idx - row * chunks_per_row;
            const int tok = shared ? start + row : (p.perm[start + row] >> 3);
            *reinterpret_cast<uint4 *>(xs + row * p.x_stride + c * Op::kPerLane) =
                load16(x + (size_t)tok * p.H + c * Op::kPerLane);
        }
        __syncthreads();
        if (wave >= kGuWaves) continue;

        const bool col_ok = col < n;
        // token columns >= n read row 0 of the x tile: matrix-core columns are independent, so
        // those columns only produce values that are never stored
        const int crow = col_ok ? col : 0;
        const int slot = !col_ok ? 0 : (shared ? p.T * kTopK + start + col : p.perm[start + col]);
        const elem_t *gu = reinterpret_cast<const elem_t *>(shared ? p.sgu : p.gate_up) +
                           (shared ? 0 : (size_t)e * 2 * Ie * p.H);
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
                const uint4 xb = lds_load16(xrow + (b * kU + v) * Op::kStep);
                Op::mma(ag, g[v], xb);
                Op::mma(au, uu[v], xb);
            }
        };
        if (nfull > 0) load_gu(gA, uA, 0);
        int b = 0;
        for (; b + 2 <= nfull; b += 2) {
            load_gu(gB, uB, b + 1);
            mma_gu(gA, uA, b);
            if (b + 2 < nfull) load_gu(gA, uA, b + 2);
            mma_gu(gB, uB, b + 1);
        }
        if (b < nfull) mma_gu(gA, uA, b);
        for (int kk = rem; kk < p.H; kk += Op::kStep) {  // only when H % (kU*step) != 0
            const uint4 xb = lds_load16(xrow + kk);
            Op::mma(ag, load16_stream(grow + kk), xb);
            Op::mma(au, load16_stream(urow + kk), xb);
        }
        if (!col_ok) continue;
        // lane holds intermediate rows i0 + 4q + r, r = 0..3, of token column `col`
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[r] = ag[r] / (1.0f + expf(-ag[r])) * au[r];
        const size_t off = (size_t)slot * p.Imax + i0 + 4 * q;
        if constexpr (Op::kElemBytes == 2) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hi[r] = f32_to_bf16_bits(hv[r]);
                lo[r] = f32_to_bf16_bits(hv[r] - bf16_bits_to_f32(hi[r]));
            }
            uint16_t *hp = reinterpret_cast<uint16_t *>(p.h);
            *reinterpret_cast<uint2 *>(hp + off) = uint2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
            *reinterpret_cast<uint2 *>(hp + p.plane + off) =
                uint2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
        } else {
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.h) + off) =
                make_float4(hv[0], hv[1], hv[2], hv[3]);
        }
    }
}

// One block per (expert group, 64 rows of y): wave w multiplies rows r0 + 16w .. +16 of the
// expert's down weight (Ie contiguous elements each, so the block reads one contiguous 64-row
// block) by the group's h, staged once per unit in LDS, and writes weight * (Wd h) to the row
// slot of each of the group's (token, rank) pairs.
template <class Op>
__global__ __launch_bounds__(kThreads) void down_kernel(DownParams p) {
    using elem_t = typename Op::elem_t;
    using h_t = typename Op::elem_t;                // h planes share the operand type
    constexpr int kRowsPerUnit = 64;
    constexpr int kMaxSteps = 32;                   // Ie / kStep <= 32 loads in flight
    extern __shared__ __align__(16) unsigned char smem[];
    const int hstride = p.Imax + 16 / Op::kElemBytes;  // padded row stride of the h tile
    h_t *hs_hi = reinterpret_cast<h_t *>(smem);                 // [16][hstride]
    h_t *hs_lo = hs_hi + (size_t)kTile * hstride;               // bf16 only

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, q = lane >> 4;
    const int n_rc = p.H / kRowsPerUnit;
    const int nunits = p.num_groups[0] * n_rc;
    const h_t *hg = reinterpret_cast<const h_t *>(p.h);

    for (int u = blockIdx.x; u < nunits; u += gridDim.x) {
        const int gi = u / n_rc, rc = u - (u / n_rc) * n_rc;
        const int4 grp = p.groups[gi];
        const int e = grp.x, start = grp.y, n = grp.z;
        const bool shared = e == p.E;
        const int Ie = shared ? p.Is : p.I;
        const int nsteps = Ie / Op::kStep;
        const elem_t *dn = reinterpret_cast<const elem_t *>(shared ? p.sdn : p.down) +
                           (shared ? 0 : (size_t)e * p.H * Ie);
        const int row = rc * kRowsPerUnit + wave * kTile + col;
        const elem_t *arp = dn + (size_t)row * Ie + q * Op::kPerLane;
        // the weight stream does not depend on h: issue its first chunk before staging h
        uint4 a[kMaxSteps];
        auto load_chunk = [&](int s0) {
#pragma unroll
            for (int st = 0; st < kMaxSteps; ++st)
                if (s0 + st < nsteps) a[st] = load16_stream(arp + (s0 + st) * Op::kStep);
        };
        load_chunk(0);

        __syncthreads();  // the previous unit's readers of the h tile are done
        const int cpr = Ie / Op::kPerLane;  // 16-byte chunks per h row
        for (int idx = tid; idx < n * cpr; idx += kThreads) {
            const int r = idx / cpr, c = idx - (idx / cpr) * cpr;
            const int slot = shared ? p.T * kTopK + start + r : p.perm[start + r];
            const size_t src = (size_t)slot * p.Imax + c * Op::kPerLane;
            *reinterpret_cast<uint4 *>(hs_hi + r * hstride + c * Op::kPerLane) = load16(hg + src);
            if constexpr (Op::kElemBytes == 2)
                *reinterpret_cast<uint4 *>(hs_lo + r * hstride + c * Op::kPerLane) =
                    load16(hg + p.plane + src);
        }
        __syncthreads();

        const bool col_ok = col < n;
        const int crow = col_ok ? col : 0;  // columns >= n repeat column 0 (dropped)
        const h_t *bhp = hs_hi + crow * hstride + q * Op::kPerLane;
        const h_t *blp = hs_lo + crow * hstride + q * Op::kPerLane;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < nsteps; s0 += kMaxSteps) {  // one pass unless Ie > kMaxSteps steps
            if (s0 > 0) load_chunk(s0);
#pragma unroll
            for (int st = 0; st < kMaxSteps; ++st) {
                const int kk = (s0 + st) * Op::kStep;
                if (s0 + st < nsteps) {  // uniform
                    Op::mma(acc, a[st], lds_load16(bhp + kk));
                    if constexpr (Op::kElemBytes == 2) Op::mma(acc, a[st], lds_load16(blp + kk));
                }
            }
        }
        if (col_ok) {
            const int slot = shared ? p.T * kTopK + start + col : p.perm[start + col];
            const float wt = shared ? p.g[start + col] : p.w[slot];
            // lane holds rows 4q + r of the wave's 16 rows for token column col
            *reinterpret_cast<float4 *>(p.ybuf + (size_t)slot * p.H + rc * kRowsPerUnit +
                                        wave * kTile + 4 * q) =
                make_float4(wt * acc[0], wt * acc[1], wt * acc[2], wt * acc[3]);
        }
    }
}

template <class Op, int SW>
static hipError_t set_gateup_lds(size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&gateup_kernel<Op, SW>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t prepare_split_kernels(size_t gateup_lds, size_t down_lds) {
    hipError_t err;
    if ((err = set_gateup_lds<OpBF16, 32>(gateup_lds)) != hipSuccess) return err;
    if ((err = set_gateup_lds<OpBF16, 64>(gateup_lds)) != hipSuccess) return err;
    if ((err = set_gateup_lds<OpF32, 16>(gateup_lds)) != hipSuccess) return err;
    if ((err = set_gateup_lds<OpF32, 32>(gateup_lds)) != hipSuccess) return err;
    if ((err = set_gateup_lds<OpF32, 64>(gateup_lds)) != hipSuccess) return err;
    if ((err = hipFuncSetAttribute(reinterpret_cast<const void *>(&down_kernel<OpBF16>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)down_lds)) !=
        hipSuccess)
        return err;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&down_kernel<OpF32>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)down_lds);
}

hipError_t launch_gateup(const GateUpParams &p, int dtype, int sw, int grid, size_t lds,
                         hipStream_t s) {
    if (dtype == 1) {
        if (sw == 64) gateup_kernel<OpBF16, 64><<<grid, kThreads, lds, s>>>(p);
        else if (sw == 32) gateup_kernel<OpBF16, 32><<<grid, kThreads, lds, s>>>(p);
        else return hipErrorInvalidValue;
    } else {
        if (sw == 64) gateup_kernel<OpF32, 64><<<grid, kThreads, lds, s>>>(p);
        else if (sw == 32) gateup_kernel<OpF32, 32><<<grid, kThreads, lds, s>>>(p);
        else if (sw == 16) gateup_kernel<OpF32, 16><<<grid, kThreads, lds, s>>>(p);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_down(const DownParams &p, int dtype, int grid, size_t lds, hipStream_t s) {
    if (dtype == 1) down_kernel<OpBF16><<<grid, kThreads, lds, s>>>(p);
    else down_kernel<OpF32><<<grid, kThreads, lds, s>>>(p);
    return hipGetLastError();
}

}  // namespace moe
