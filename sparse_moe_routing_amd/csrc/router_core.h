// router_core.h - router logits on the matrix cores, in one fixed summation order.
//
// The router is a [R x H] weight times the [H x T] activations (R = E experts plus the shared
// gate row), computed on 16x16 (row, token) tiles with MFMA. The K dimension (H, in MFMA steps
// of 32 bf16 / 16 fp32 elements) is cut into kQuarters quarters of Sq steps, and each quarter
// into up to kChains contiguous runs of Sw = ceil(Sq / kChains) steps. A run is one MFMA
// accumulation chain; a quarter's partial logit is the sum of its runs' tiles in run order; the
// selection later adds the four partials in order and then the bias. Every kernel that produces
// logits uses exactly this order, so a token's logits - and therefore its routing - do not
// depend on the batch it is in or on which kernel computed them.
//
// Two ways to evaluate it:
//   router_quarter_block - 16 waves of a block compute the runs of one (token tile, row tile,
//     quarter) in parallel and add them through LDS (decode sizes: the 1 MiB router is spread
//     over many CUs).
//   router_unit - one wave computes a quarter for up to MAXRT row tiles, running the runs one
//     after the other (large T).
// (The page "feat(windows): integrate upstream Qwen3.8 DFlash2 support - #8" describes a K split
// for its S1 kernel as well: four partial sums per score, folded by S2.)
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kQuarters = 4;   // partial logits per score
constexpr int kChains = 16;    // accumulation runs per quarter

struct RouterGeom {
    int Sq, Sw, nchains;
    __device__ RouterGeom(int H, int kstep) {
        Sq = H / kstep / kQuarters;
        Sw = (Sq + kChains - 1) / kChains;
        nchains = (Sq + Sw - 1) / Sw;
    }
};

// One run: tile += sum over steps [s0, s1) of W[rows] . x[tokens] (MFMA chain), where `wrow` and
// `xrow` point at the lane's row / token with the lane's k-group offset already applied.
// Out-of-range rows and tokens read clamped addresses and are zeroed by `wok` / `tok_ok`.
template <class Op, int MAXRT>
__device__ __forceinline__ void router_run(f32x4_t (&ch)[MAXRT], const typename Op::elem_t *xrow,
                                           const typename Op::elem_t *const (&wrow)[MAXRT],
                                           const bool (&wok)[MAXRT], bool tok_ok, int nrt_here,
                                           int s0, int s1) {
    const uint4 zero = {0u, 0u, 0u, 0u};
    constexpr int kBatch = 8;  // steps whose loads are issued together
    for (int b0 = s0; b0 < s1; b0 += kBatch) {
        uint4 xb[kBatch], wa[kBatch][MAXRT];
#pragma unroll
        for (int v = 0; v < kBatch; ++v) {
            const int st = min(b0 + v, s1 - 1);  // past the end: re-read, unused
            xb[v] = load16(xrow + st * Op::kStep);
#pragma unroll
            for (int j = 0; j < MAXRT; ++j) wa[v][j] = load16(wrow[j] + st * Op::kStep);
        }
#pragma unroll
        for (int v = 0; v < kBatch; ++v) {
            if (b0 + v >= s1) break;  // uniform
            const uint4 bv = tok_ok ? xb[v] : zero;
#pragma unroll
            for (int j = 0; j < MAXRT; ++j)
                if (j < nrt_here) Op::mma(ch[j], wok[j] ? wa[v][j] : zero, bv);  // uniform j test
        }
    }
}

// Large-T form: wave unit u = (token tile, group of MAXRT row tiles, quarter); writes the
// quarter's partial logits zpart[quarter][t][r]. Waves with u >= the unit count do nothing.
// kDev: store them device-coherently (read by another wave of the same launch).
template <class Op, int MAXRT, bool kDev = false>
__device__ __forceinline__ void router_unit(const RouterParams &p, int u, int lane) {
    using elem_t = typename Op::elem_t;
    const int total = p.n_tt * p.KS * p.n_rg;
    if (u >= total) return;
    const int rg = u % p.n_rg;
    const int kq = (u / p.n_rg) % p.KS;
    const int tt = u / (p.n_rg * p.KS);
    const int n_rt = (p.R + kTile - 1) / kTile;
    const int rt0 = rg * MAXRT;
    const int nrt_here = min(MAXRT, n_rt - rt0);
    const int col = lane & 15, q = lane >> 4;
    const int tok = tt * kTile + col;
    const bool tok_ok = tok < p.T;
    const RouterGeom g(p.H, Op::kStep);
    const int kbase = kq * g.Sq * Op::kStep + q * Op::kPerLane;
    const elem_t *xrow = reinterpret_cast<const elem_t *>(p.x) + (size_t)(tok_ok ? tok : 0) * p.H + kbase;
    const elem_t *wrow[MAXRT];
    bool wok[MAXRT];
#pragma unroll
    for (int j = 0; j < MAXRT; ++j) {
        const int row = (rt0 + j) * kTile + col;
        wok[j] = j < nrt_here && row < p.R;
        wrow[j] = reinterpret_cast<const elem_t *>(p.w) + (size_t)(wok[j] ? row : 0) * p.H + kbase;
    }
    // The runs are evaluated one after the other, but the loads of kBatch consecutive steps are
    // issued together across run boundaries; a run's tile is added to the quarter sum when the
    // run ends (the first run initialises it), exactly as in router_quarter_block.
    const uint4 zero = {0u, 0u, 0u, 0u};
    constexpr int kBatch = 8;
    f32x4_t s[MAXRT], ch[MAXRT];
#pragma unroll
    for (int j = 0; j < MAXRT; ++j) ch[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int b0 = 0; b0 < g.Sq; b0 += kBatch) {
        uint4 xb[kBatch], wa[kBatch][MAXRT];
#pragma unroll
        for (int v = 0; v < kBatch; ++v) {
            const int st = min(b0 + v, g.Sq - 1);  // past the end: re-read, unused
            xb[v] = load16(xrow + st * Op::kStep);
#pragma unroll
            for (int j = 0; j < MAXRT; ++j) wa[v][j] = load16(wrow[j] + st * Op::kStep);
        }
#pragma unroll
        for (int v = 0; v < kBatch; ++v) {
            const int st = b0 + v;
            if (st >= g.Sq) break;  // uniform
            const uint4 bv = tok_ok ? xb[v] : zero;
#pragma unroll
            for (int j = 0; j < MAXRT; ++j)
                if (j < nrt_here) Op::mma(ch[j], wok[j] ? wa[v][j] : zero, bv);
            if ((st + 1) % g.Sw == 0 || st + 1 == g.Sq) {  // run st / Sw ends here (uniform)
                const bool first = st < g.Sw;
#pragma unroll
                for (int j = 0; j < MAXRT; ++j) {
                    s[j] = first ? ch[j] : s[j] + ch[j];
                    ch[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    }
    if (!tok_ok) return;
    float *out = p.zpart + ((size_t)kq * p.T + tok) * p.R;
#pragma unroll
    for (int j = 0; j < MAXRT; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = (rt0 + j) * kTile + 4 * q + r;
            if (j < nrt_here && row < p.R) {
                if constexpr (kDev) st_dev(out + row, s[j][r]);
                else out[row] = s[j][r];
            }
        }
    }
}

// Prefill form: wave unit u = (group of MAXTT token tiles, group of MAXRT row tiles, quarter):
// every weight fragment feeds MAXTT token tiles and every x fragment MAXRT row tiles, so the
// router weight is read from cache once per MAXTT token tiles. Per output element the steps,
// runs and their order are those of router_unit (the result is bitwise the same).
template <class Op, int MAXRT, int MAXTT>
__device__ __forceinline__ void router_unit_tt(const RouterParams &p, int u, int lane) {
    using elem_t = typename Op::elem_t;
    const int n_tg = (p.n_tt + MAXTT - 1) / MAXTT;
    const int total = n_tg * p.KS * p.n_rg;
    if (u >= total) return;
    const int rg = u % p.n_rg;
    const int kq = (u / p.n_rg) % p.KS;
    const int tg = u / (p.n_rg * p.KS);
    const int n_rt = (p.R + kTile - 1) / kTile;
    const int rt0 = rg * MAXRT, tt0 = tg * MAXTT;
    const int nrt_here = min(MAXRT, n_rt - rt0);
    const int ntt_here = min(MAXTT, p.n_tt - tt0);
    const int col = lane & 15, q = lane >> 4;
    const RouterGeom g(p.H, Op::kStep);
    const int kbase = kq * g.Sq * Op::kStep + q * Op::kPerLane;
    const elem_t *xrow[MAXTT];
    bool tok_ok[MAXTT];
#pragma unroll
    for (int i = 0; i < MAXTT; ++i) {
        const int tok = (tt0 + i) * kTile + col;
        tok_ok[i] = i < ntt_here && tok < p.T;
        xrow[i] = reinterpret_cast<const elem_t *>(p.x) + (size_t)(tok_ok[i] ? tok : 0) * p.H + kbase;
    }
    const elem_t *wrow[MAXRT];
    bool wok[MAXRT];
#pragma unroll
    for (int j = 0; j < MAXRT; ++j) {
        const int row = (rt0 + j) * kTile + col;
        wok[j] = j < nrt_here && row < p.R;
        wrow[j] = reinterpret_cast<const elem_t *>(p.w) + (size_t)(wok[j] ? row : 0) * p.H + kbase;
    }
    const uint4 zero = {0u, 0u, 0u, 0u};
    constexpr int kBatch = MAXTT >= 4 ? 2 : 4;  // k steps whose loads are issued together
    f32x4_t s[MAXRT][MAXTT], ch[MAXRT][MAXTT];
#pragma unroll
    for (int j = 0; j < MAXRT; ++j)
#pragma unroll
        for (int i = 0; i < MAXTT; ++i) ch[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int b0 = 0; b0 < g.Sq; b0 += kBatch) {
        uint4 xb[kBatch][MAXTT], wa[kBatch][MAXRT];
#pragma unroll
        for (int v = 0; v < kBatch; ++v) {
            const int st = min(b0 + v, g.Sq - 1);  // past the end: re-read, unused
#pragma unroll
            for (int i = 0; i < MAXTT; ++i) xb[v][i] = load16(xrow[i] + st * Op::kStep);
#pragma unroll
            for (int j = 0; j < MAXRT; ++j) wa[v][j] = load16(wrow[j] + st * Op::kStep);
        }
#pragma unroll
        for (int v = 0; v < kBatch; ++v) {
            const int st = b0 + v;
            if (st >= g.Sq) break;  // uniform
#pragma unroll
            for (int j = 0; j < MAXRT; ++j)
#pragma unroll
                for (int i = 0; i < MAXTT; ++i)
                    if (j < nrt_here && i < ntt_here)  // uniform
                        Op::mma(ch[j][i], wok[j] ? wa[v][j] : zero, tok_ok[i] ? xb[v][i] : zero);
            if ((st + 1) % g.Sw == 0 || st + 1 == g.Sq) {  // run st / Sw ends here (uniform)
                const bool first = st < g.Sw;
#pragma unroll
                for (int j = 0; j < MAXRT; ++j)
#pragma unroll
                    for (int i = 0; i < MAXTT; ++i) {
                        s[j][i] = first ? ch[j][i] : s[j][i] + ch[j][i];
                        ch[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < MAXTT; ++i) {
        if (!tok_ok[i]) continue;
        const int tok = (tt0 + i) * kTile + col;
        float *out = p.zpart + ((size_t)kq * p.T + tok) * p.R;
#pragma unroll
        for (int j = 0; j < MAXRT; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = (rt0 + j) * kTile + 4 * q + r;
                if (j < nrt_here && row < p.R) out[row] = s[j][i][r];
            }
        }
    }
}

// Prefill form with whole cache lines: as router_unit_tt, but every 16-row weight tile and
// 16-token x tile is read 128 contiguous bytes per row (8 rows x 128 B per load) for two k steps
// at a time and staged in the wave's own LDS area `wst` ((MAXRT + MAXTT) x 2 KiB; row rr, piece
// pc at rr * 128 + ((pc ^ (rr >> 1)) & 7) * 16), from which the operand fragments are read in
// matrix-core order. Per output element the steps, runs and their order are those of router_unit
// (the result is bitwise the same). Needs an even number of steps per quarter.
template <class Op, int MAXRT, int MAXTT>
__device__ __forceinline__ void router_unit_tt_lds(const RouterParams &p, int u, int lane,
                                                   unsigned char *wst) {
    using elem_t = typename Op::elem_t;
    constexpr int NTL = MAXRT + MAXTT;    // staged tiles: weights first, then x
    constexpr int kTileBytes = kTile * 128;
    constexpr int kHalf = 2 * Op::kStep;  // elements of a half chunk (128 bytes)
    const int n_tg = (p.n_tt + MAXTT - 1) / MAXTT;
    const int total = n_tg * p.KS * p.n_rg;
    if (u >= total) return;
    const int rg = u % p.n_rg;
    const int kq = (u / p.n_rg) % p.KS;
    const int tg = u / (p.n_rg * p.KS);
    const int n_rt = (p.R + kTile - 1) / kTile;
    const int rt0 = rg * MAXRT, tt0 = tg * MAXTT;
    const int nrt_here = min(MAXRT, n_rt - rt0);
    const int ntt_here = min(MAXTT, p.n_tt - tt0);
    const int col = lane & 15, q = lane >> 4;
    const int drow = lane >> 3, dpiece = lane & 7;
    const RouterGeom g(p.H, Op::kStep);
    const int nhalf = g.Sq / 2;
    const elem_t *x = reinterpret_cast<const elem_t *>(p.x);
    const elem_t *w = reinterpret_cast<const elem_t *>(p.w);
    // loader: element offsets (quarter start and piece included) of rows drow and drow + 8 of
    // every tile, clamped to a valid row (an out-of-range row is zeroed at its use)
    uint32_t off[NTL][2];
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = (t < MAXRT ? (rt0 + t) : (tt0 + t - MAXRT)) * kTile + 8 * i + drow;
            const int lim = t < MAXRT ? p.R : p.T;
            off[t][i] = (uint32_t)(r < lim ? r : lim - 1) * (uint32_t)p.H + kq * g.Sq * Op::kStep +
                        dpiece * Op::kPerLane;
        }
    bool wok[MAXRT], tok_ok[MAXTT];
#pragma unroll
    for (int j = 0; j < MAXRT; ++j) wok[j] = j < nrt_here && (rt0 + j) * kTile + col < p.R;
#pragma unroll
    for (int i = 0; i < MAXTT; ++i) tok_ok[i] = i < ntt_here && (tt0 + i) * kTile + col < p.T;
    uint4 rA[NTL][2], rB[NTL][2];
    auto load = [&](uint4 (&r)[NTL][2], int hc) {
        if (hc >= nhalf) return;  // uniform
#pragma unroll
        for (int t = 0; t < NTL; ++t)
#pragma unroll
            for (int i = 0; i < 2; ++i) r[t][i] = load16((t < MAXRT ? w : x) + off[t][i] + hc * kHalf);
    };
    const uint4 zero = {0u, 0u, 0u, 0u};
    f32x4_t s[MAXRT][MAXTT], ch[MAXRT][MAXTT];
#pragma unroll
    for (int j = 0; j < MAXRT; ++j)
#pragma unroll
        for (int i = 0; i < MAXTT; ++i) ch[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto half = [&](uint4 (&r)[NTL][2], int hc) {
#pragma unroll
        for (int t = 0; t < NTL; ++t)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int rr = 8 * i + drow;
                *reinterpret_cast<uint4 *>(wst + t * kTileBytes + rr * 128 + ((dpiece ^ ((rr >> 1) & 7)) * 16)) = r[t][i];
            }
        load(r, hc + 2);
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
            const int st = 2 * hc + sh;
            const int po = col * 128 + (((4 * sh + q) ^ ((col >> 1) & 7)) * 16);
            uint4 a[MAXRT], b[MAXTT];
#pragma unroll
            for (int j = 0; j < MAXRT; ++j) a[j] = *reinterpret_cast<const uint4 *>(wst + j * kTileBytes + po);
#pragma unroll
            for (int i = 0; i < MAXTT; ++i) b[i] = *reinterpret_cast<const uint4 *>(wst + (MAXRT + i) * kTileBytes + po);
#pragma unroll
            for (int j = 0; j < MAXRT; ++j)
#pragma unroll
                for (int i = 0; i < MAXTT; ++i)
                    if (j < nrt_here && i < ntt_here)  // uniform
                        Op::mma(ch[j][i], wok[j] ? a[j] : zero, tok_ok[i] ? b[i] : zero);
            if ((st + 1) % g.Sw == 0 || st + 1 == g.Sq) {  // run st / Sw ends here (uniform)
                const bool first = st < g.Sw;
#pragma unroll
                for (int j = 0; j < MAXRT; ++j)
#pragma unroll
                    for (int i = 0; i < MAXTT; ++i) {
                        s[j][i] = first ? ch[j][i] : s[j][i] + ch[j][i];
                        ch[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    }
            }
        }
    };
    load(rA, 0);
    load(rB, 1);
    for (int hc = 0; hc < nhalf; hc += 2) {
        half(rA, hc);
        if (hc + 1 < nhalf) half(rB, hc + 1);
    }
#pragma unroll
    for (int i = 0; i < MAXTT; ++i) {
        const int tok = (tt0 + i) * kTile + col;
        if (!(i < ntt_here && tok < p.T)) continue;
        float *out = p.zpart + ((size_t)kq * p.T + tok) * p.R;
#pragma unroll
        for (int j = 0; j < MAXRT; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = (rt0 + j) * kTile + 4 * q + r;
                if (j < nrt_here && row < p.R) out[row] = s[j][i][r];
            }
        }
    }
}

// Decode form: block b = (token tile, row tile, quarter) of 16 waves; wave w computes run w and
// the runs are added in order through LDS (red: 16 tiles of 256 floats). Every thread of the
// block calls it; it ends with the partial logits stored (no trailing barrier). kDev: stored
// device-coherently (read by another block of the same launch).
template <class Op, bool kDev = false>
__device__ __forceinline__ void router_quarter_block(const RouterParams &p, int b, float *red) {
    using elem_t = typename Op::elem_t;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n_rt = (p.R + kTile - 1) / kTile;
    const int rt = b % n_rt;
    const int kq = (b / n_rt) % kQuarters;
    const int tt = b / (n_rt * kQuarters);
    const int col = lane & 15, q = lane >> 4;
    const int tok = tt * kTile + col;
    const bool tok_ok = tok < p.T;
    const int row = rt * kTile + col;
    const bool wok[1] = {row < p.R};
    const RouterGeom g(p.H, Op::kStep);
    const int kbase = kq * g.Sq * Op::kStep + q * Op::kPerLane;
    const elem_t *xrow = reinterpret_cast<const elem_t *>(p.x) + (size_t)(tok_ok ? tok : 0) * p.H + kbase;
    const elem_t *const wrow[1] = {reinterpret_cast<const elem_t *>(p.w) +
                                   (size_t)(wok[0] ? row : 0) * p.H + kbase};
    f32x4_t ch[1] = {f32x4_t{0.f, 0.f, 0.f, 0.f}};
    if (wave < g.nchains)
        router_run<Op, 1>(ch, xrow, wrow, wok, tok_ok, 1, wave * g.Sw, min((wave + 1) * g.Sw, g.Sq));
    // tile element (row 4q + r, token col) of run `wave`
    *reinterpret_cast<f32x4_t *>(red + wave * 256 + col * 16 + 4 * q) = ch[0];
    __syncthreads();
    if (tid < 256) {
        const int c = tid >> 4, rr = tid & 15;  // token column, tile row
        float acc = red[c * 16 + rr];
        for (int w = 1; w < g.nchains; ++w) acc += red[w * 256 + c * 16 + rr];
        const int t = tt * kTile + c, r = rt * kTile + rr;
        if (t < p.T && r < p.R) {
            float *dst = p.zpart + ((size_t)kq * p.T + t) * p.R + r;
            if constexpr (kDev) st_dev(dst, acc);
            else *dst = acc;
        }
    }
}

}  // namespace moe
