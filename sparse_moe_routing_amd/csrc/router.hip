// router.hip - router logits on the matrix cores.
//
// The router is a [R x H] weight times the [H x T] activations (R = E experts plus the shared
// gate row). Each wave owns one unit = (16-token tile, K range, group of up to MAXRT 16-row
// tiles) and accumulates fp32 16x16 tiles with MFMA; no LDS is needed because every weight
// fragment is used by exactly one instruction and the activation fragment is reused across the
// wave's row tiles from registers. At decode sizes the K dimension is split KS ways so that
// enough waves stream the 1 MiB router; the select kernel folds the KS partials in a fixed order.
// (The page "feat(windows): integrate upstream Qwen3.8 DFlash2 support - #8" describes the same
// split for its S1 kernel: four partial sums per score over 1028 blocks, folded by S2.)
#include "device_common.h"
#include "kernels.h"

namespace moe {

template <class Op, int MAXRT>
__global__ __launch_bounds__(256) void router_kernel(RouterParams p) {
    using elem_t = typename Op::elem_t;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int u = blockIdx.x * 4 + wave;
    const int total = p.n_tt * p.KS * p.n_rg;
    if (u >= total) return;  // whole wave leaves; the kernel has no block barrier
    const int rg = u % p.n_rg;
    const int ks = (u / p.n_rg) % p.KS;
    const int tt = u / (p.n_rg * p.KS);
    const int n_rt = (p.R + kTile - 1) / kTile;
    const int rt0 = rg * MAXRT;
    const int col = lane & 15;
    const int q = lane >> 4;
    const int tok = tt * kTile + col;
    const bool tok_ok = tok < p.T;
    const int Kc = p.H / p.KS;
    const int k_begin = ks * Kc;
    const elem_t *x = reinterpret_cast<const elem_t *>(p.x);
    const elem_t *w = reinterpret_cast<const elem_t *>(p.w);

    const elem_t *xrow = x + (size_t)(tok_ok ? tok : 0) * p.H;
    const elem_t *wrow[MAXRT];
    bool wok[MAXRT];
#pragma unroll
    for (int j = 0; j < MAXRT; ++j) {
        const int row = (rt0 + j) * kTile + col;
        wok[j] = (rt0 + j < n_rt) && row < p.R;
        wrow[j] = w + (size_t)(wok[j] ? row : 0) * p.H;
    }
    f32x4_t acc[MAXRT];
#pragma unroll
    for (int j = 0; j < MAXRT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const uint4 zero = {0u, 0u, 0u, 0u};
    constexpr int kBatch = 4;  // k steps whose loads are issued together
    const int k_end = k_begin + Kc;
    for (int k0 = k_begin; k0 < k_end; k0 += kBatch * Op::kStep) {
        uint4 b[kBatch], a[kBatch][MAXRT];
#pragma unroll
        for (int v = 0; v < kBatch; ++v) {
            const int kk = k0 + v * Op::kStep + q * Op::kPerLane;
            if (k0 + v * Op::kStep < k_end) {
                b[v] = tok_ok ? load16(xrow + kk) : zero;
#pragma unroll
                for (int j = 0; j < MAXRT; ++j) a[v][j] = wok[j] ? load16(wrow[j] + kk) : zero;
            }
        }
#pragma unroll
        for (int v = 0; v < kBatch; ++v) {
            if (k0 + v * Op::kStep < k_end) {
#pragma unroll
                for (int j = 0; j < MAXRT; ++j)
                    if (rt0 + j < n_rt) Op::mma(acc[j], a[v][j], b[v]);  // uniform condition
            }
        }
    }
    if (!tok_ok) return;
    float *out = p.zpart + ((size_t)ks * p.T + tok) * p.R;
#pragma unroll
    for (int j = 0; j < MAXRT; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = (rt0 + j) * kTile + 4 * q + r;
            if (rt0 + j < n_rt && row < p.R) out[row] = acc[j][r];
        }
    }
}

hipError_t launch_router(const RouterParams &p, int dtype, int maxrt, hipStream_t s) {
    const int units = p.n_tt * p.KS * p.n_rg;
    const dim3 grid((units + 3) / 4), block(256);
    if (dtype == 1) {
        if (maxrt == 1) router_kernel<OpBF16, 1><<<grid, block, 0, s>>>(p);
        else router_kernel<OpBF16, 4><<<grid, block, 0, s>>>(p);
    } else {
        if (maxrt == 1) router_kernel<OpF32, 1><<<grid, block, 0, s>>>(p);
        else router_kernel<OpF32, 4><<<grid, block, 0, s>>>(p);
    }
    return hipGetLastError();
}

}  // namespace moe
