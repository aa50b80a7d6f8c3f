// router.hip - the standalone router kernel (large T): one router unit per wave.
#include "router_core.h"

namespace moe {

template <class Op, int MAXRT>
__global__ __launch_bounds__(256) void router_kernel(RouterParams p) {
    router_unit<Op, MAXRT>(p, blockIdx.x * 4 + (threadIdx.x >> 6), threadIdx.x & 63);
}

// Large T: each wave covers 4 row tiles x 2 token tiles of a quarter (two waves per SIMD, four
// k steps of loads in flight per wave).
constexpr int kRouterTT = 2;
template <class Op>
__global__ __launch_bounds__(256) void router_tt_kernel(RouterParams p) {
    router_unit_tt<Op, 4, kRouterTT>(p, blockIdx.x * 4 + (threadIdx.x >> 6), threadIdx.x & 63);
}

// The same units with whole-line staging through LDS (an even number of steps per quarter).
template <class Op>
__global__ __launch_bounds__(256) void router_tt_lds_kernel(RouterParams p) {
    __shared__ __align__(16) unsigned char wst[4][(4 + kRouterTT) * kTile * 128];
    const int wave = threadIdx.x >> 6;
    router_unit_tt_lds<Op, 4, kRouterTT>(p, blockIdx.x * 4 + wave, threadIdx.x & 63, wst[wave]);
}

hipError_t launch_router(const RouterParams &p, int dtype, int maxrt, hipStream_t s) {
    const int units = p.n_tt * p.KS * p.n_rg;
    const dim3 grid((units + 3) / 4), block(256);
    if (maxrt == 4) {  // token-tile blocked form
        const int tunits = (p.n_tt + kRouterTT - 1) / kRouterTT * p.KS * p.n_rg;
        const dim3 tgrid((tunits + 3) / 4);
        const int kstep = dtype == 1 ? OpBF16::kStep : OpF32::kStep;
        const bool even = (p.H / kstep / p.KS) % 2 == 0;  // steps per quarter
        if (even) {
            if (dtype == 1) launch_k(router_tt_lds_kernel<OpBF16>, tgrid, block, 0, s, p);
            else launch_k(router_tt_lds_kernel<OpF32>, tgrid, block, 0, s, p);
        } else {
            if (dtype == 1) launch_k(router_tt_kernel<OpBF16>, tgrid, block, 0, s, p);
            else launch_k(router_tt_kernel<OpF32>, tgrid, block, 0, s, p);
        }
        return hipGetLastError();
    }
    if (dtype == 1) {
        if (maxrt == 1) launch_k(router_kernel<OpBF16, 1>, grid, block, 0, s, p);
        else launch_k(router_kernel<OpBF16, 4>, grid, block, 0, s, p);
    } else {
        if (maxrt == 1) launch_k(router_kernel<OpF32, 1>, grid, block, 0, s, p);
        else launch_k(router_kernel<OpF32, 4>, grid, block, 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace moe
