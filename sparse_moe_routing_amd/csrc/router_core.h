// router_core.h - one router unit (a wave's share of the router logits) on the matrix cores.
//
// The router is a [R x H] weight times the [H x T] activations (R = E experts plus the shared
// gate row). A wave owns one unit = (16-token tile, K range, group of up to MAXRT 16-row tiles)
// and accumulates fp32 16x16 tiles with MFMA; no LDS is needed because every weight fragment is
// used by exactly one instruction and the activation fragment is reused across the wave's row
// tiles from registers. The K dimension is split KS ways so that enough waves stream the 1 MiB
// router at decode sizes; the selection folds the KS partials in a fixed order. (The page
// "feat(windows): integrate upstream Qwen3.8 DFlash2 support - #8" describes the same split for
// its S1 kernel: four partial sums per score over 1028 blocks, folded by S2.)
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace moe {

// One router unit per wave: unit u = (16-token tile, K range, group of MAXRT 16-row tiles).
// Waves with u >= the unit count do nothing (callers may place a block barrier after this).
template <class Op, int MAXRT>
__device__ __forceinline__ void router_unit(const RouterParams &p, int u, int lane) {
    using elem_t = typename Op::elem_t;
    const int total = p.n_tt * p.KS * p.n_rg;
    if (u >= total) return;
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
    // Loads are unconditional (out-of-range steps, rows and tokens read clamped addresses) and
    // their values are zeroed by selects, so a batch's loads are all in flight together.
    constexpr int kBatch = 8;  // k steps whose loads are issued together
    const int k_end = k_begin + Kc;
    for (int k0 = k_begin; k0 < k_end; k0 += kBatch * Op::kStep) {
        uint4 b[kBatch], a[kBatch][MAXRT];
        bool ok[kBatch];
#pragma unroll
        for (int v = 0; v < kBatch; ++v) {
            ok[v] = k0 + v * Op::kStep < k_end;
            const int kk = (ok[v] ? k0 + v * Op::kStep : k_begin) + q * Op::kPerLane;
            b[v] = load16(xrow + kk);
#pragma unroll
            for (int j = 0; j < MAXRT; ++j) a[v][j] = load16(wrow[j] + kk);
        }
#pragma unroll
        for (int v = 0; v < kBatch; ++v) {
            const uint4 bv = (ok[v] && tok_ok) ? b[v] : zero;
#pragma unroll
            for (int j = 0; j < MAXRT; ++j) {
                const uint4 av = wok[j] ? a[v][j] : zero;
                if (rt0 + j < n_rt) Op::mma(acc[j], av, bv);  // uniform condition
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

}  // namespace moe
