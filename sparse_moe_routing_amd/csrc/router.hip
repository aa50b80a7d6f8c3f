// router.hip - the standalone router kernels (T > 64): the per-wave form, its LDS-staged variant
// (an even number of k steps per quarter) and, for long bf16 rounds, the block form. All of them
// keep the summation order of router_core.h, so a token's logits do not depend on the kernel.
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

// Large T, bf16, R <= 320: block = (group of 128 tokens, quarter) with all the row tiles; eight
// waves, wave w takes row tiles [rg n_rt / 4, (rg + 1) n_rt / 4) (rg = w % 4; five tile slots, the
// slots past its range computed but never stored) against token tiles 4 (w / 4) .. + 4, so every
// weight fragment feeds four token tiles and every token fragment five row tiles (the per-wave
// form above reads each weight fragment for two token tiles only, and both operands for every
// wave). Both operands come straight into LDS (buffer loads with the LDS flag) in 64-element
// slabs, 128 bytes per row and 8 rows per load instruction, double-buffered; the two buffers are
// separate objects so that the compiler tells the loads into one from the reads of the other.
// Same runs, same order: a run is an MFMA chain from zero, the runs of a quarter add in order.
constexpr int kRBTok = 128;                           // tokens per block
constexpr int kRBMaxRT = 20;                          // row tiles the LDS holds (R <= 320)
constexpr int kRBSlots = 5;                           // row tile slots per wave
constexpr int kRBWaves = 8;
constexpr int kRBRowB = 128;                          // bytes of a staged row (64 bf16)
constexpr int kRBTileB = kTile * kRBRowB;
constexpr int kRBWBytes = kRBMaxRT * kRBTileB;        // 40 KB
constexpr int kRBXBytes = kRBTok * kRBRowB;           // 16 KB
__shared__ __align__(16) unsigned char g_rbw0[kRBWBytes], g_rbw1[kRBWBytes];
__shared__ __align__(16) unsigned char g_rbx0[kRBXBytes], g_rbx1[kRBXBytes];
template <int B>
__device__ __forceinline__ unsigned char *rbw() { return B ? g_rbw1 : g_rbw0; }
template <int B>
__device__ __forceinline__ unsigned char *rbx() { return B ? g_rbx1 : g_rbx0; }
// piece pc of staged row r: rows 2m, 2m + 1 rotate their pieces by m (16 rows of an operand read
// on 16 distinct bank groups; the rotation depends on r % 16 only)
__device__ __forceinline__ int rb_pos(int r, int pc) { return r * kRBRowB + ((pc ^ (r >> 1)) & 7) * 16; }
__device__ __forceinline__ uint4 rb_read16(const unsigned char *p) { return *reinterpret_cast<const uint4 *>(p); }
template <int kAux>
__device__ __forceinline__ void rb_load16(__amdgpu_buffer_rsrc_t r, unsigned char *seg, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)seg, 16, (int)off, 0, 0, kAux);
}

__global__ __launch_bounds__(kRBWaves * kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) void router_big_kernel(RouterParams p) {
    using Op = OpBF16;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, q = lane >> 4;
    const int rg = wave & 3, th = (wave >> 2) & 1;
    const int tg = blockIdx.x / kQuarters, kq = blockIdx.x % kQuarters;
    const int n_rt = (p.R + kTile - 1) / kTile;
    const int rt0 = rg * n_rt / 4, nrt = (rg + 1) * n_rt / 4 - rt0;
    const RouterGeom g(p.H, Op::kStep);
    const int nslab = g.Sq / 2;  // two k steps per slab
    const uint32_t kbase = (uint32_t)kq * g.Sq * Op::kStep * 2;  // byte offset of the quarter
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(p.w, (uint32_t)((size_t)p.R * p.H * 2));
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(p.x, (uint32_t)((size_t)p.T * p.H * 2));
    // loaders: weight segment sg (rows 8 sg .. + 8, row index clamped to R - 1) for sg = wave + 8 a
    // < 2 n_rt; x segment wave + 8 a (token rows, clamped to T - 1); lane l writes position l % 8 of
    // row l / 8 of its segment, i.e. it loads the piece the row's rotation puts there
    const int lrow = lane >> 3;
    uint32_t woff[kRBSlots], xoff[2];
#pragma unroll
    for (int a = 0; a < kRBSlots; ++a) {
        const int r = 8 * (wave + kRBWaves * a) + lrow;
        const int pc = ((lane & 7) ^ (r >> 1)) & 7;
        woff[a] = (uint32_t)(r < p.R ? r : p.R - 1) * (uint32_t)p.H * 2 + kbase + pc * 16;
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int r = 8 * (wave + kRBWaves * a) + lrow;
        const int pc = ((lane & 7) ^ (r >> 1)) & 7;
        const int tok = tg * kRBTok + r;
        xoff[a] = (uint32_t)(tok < p.T ? tok : p.T - 1) * (uint32_t)p.H * 2 + kbase + pc * 16;
    }
    auto issue = [&](unsigned char *wb, unsigned char *xb, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < kRBSlots; ++a)
            if (wave + kRBWaves * a < 2 * n_rt)  // uniform
                rb_load16<0>(rw, wb + (wave + kRBWaves * a) * 1024, woff[a] + st * kRBRowB);
#pragma unroll
        for (int a = 0; a < 2; ++a)
            rb_load16<0>(rx, xb + (wave + kRBWaves * a) * 1024, xoff[a] + st * kRBRowB);
    };
    f32x4_t s[kRBSlots][4], ch[kRBSlots][4];
#pragma unroll
    for (int j = 0; j < kRBSlots; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) ch[j][i] = s[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int rd_off[2] = {rb_pos(col, q), rb_pos(col, 4 + q)};
    auto compute = [&](const unsigned char *wb, const unsigned char *xb, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int step = 2 * st + h;
            uint4 a[kRBSlots], b[4];
#pragma unroll
            for (int j = 0; j < kRBSlots; ++j) a[j] = rb_read16(wb + (rt0 + j) * kRBTileB + rd_off[h]);
#pragma unroll
            for (int i = 0; i < 4; ++i) b[i] = rb_read16(xb + (4 * th + i) * kRBTileB + rd_off[h]);
#pragma unroll
            for (int j = 0; j < kRBSlots; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) Op::mma(ch[j][i], a[j], b[i]);
            if ((step + 1) % g.Sw == 0 || step + 1 == g.Sq) {  // run step / Sw ends here (uniform)
                const bool first = step < g.Sw;
#pragma unroll
                for (int j = 0; j < kRBSlots; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        s[j][i] = first ? ch[j][i] : s[j][i] + ch[j][i];
                        ch[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    }
            }
        }
    };
    auto slab = [&](auto bsel, int st) __attribute__((always_inline)) {
        constexpr int B = decltype(bsel)::value;
        if (st + 1 < nslab) issue(rbw<1 - B>(), rbx<1 - B>(), st + 1);
        compute(rbw<B>(), rbx<B>(), st);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's straight-to-LDS loads landed
        __syncthreads();
    };
    issue(rbw<0>(), rbx<0>(), 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (int st = 0; st < nslab; st += 2) {
        slab(std::integral_constant<int, 0>{}, st);
        if (st + 1 < nslab) slab(std::integral_constant<int, 1>{}, st + 1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = tg * kRBTok + (4 * th + i) * kTile + col;
        if (tok >= p.T) continue;
        float *out = p.zpart + ((size_t)kq * p.T + tok) * p.R;
#pragma unroll
        for (int j = 0; j < kRBSlots; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = (rt0 + j) * kTile + 4 * q + r;
                if (j < nrt && row < p.R) out[row] = s[j][i][r];
            }
        }
    }
}

hipError_t launch_router(const RouterParams &p, int dtype, int maxrt, hipStream_t s) {
    const int units = p.n_tt * p.KS * p.n_rg;
    const dim3 grid((units + 3) / 4), block(256);
    // each block of the block form is a chain of H / 256 slabs, ~25 us at H = 2048 whatever T is:
    // measured against the token-tile form, T = 2048 27.9 vs 22.3 us, 4096 30.2 vs 39.1, 8192 39.1
    // vs 63.5
    constexpr int kRouterBigMinTokens = 3072;
    if (maxrt == 4 && dtype == 1 && p.T >= kRouterBigMinTokens && p.KS == kQuarters &&
        (p.R + kTile - 1) / kTile <= kRBMaxRT &&
        p.H % (kQuarters * 2 * OpBF16::kStep) == 0 && (size_t)p.T * p.H * 2 < (1u << 31)) {
        launch_k(router_big_kernel, dim3((p.T + kRBTok - 1) / kRBTok * kQuarters), dim3(kRBWaves * kWave), 0, s, p);
        return hipGetLastError();
    }
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
