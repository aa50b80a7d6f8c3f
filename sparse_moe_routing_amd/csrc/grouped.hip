// grouped.hip - expert-stationary gate/up and down for prefill-sized rounds.
//
// At T = 8192 tokens each of the 256 experts draws 256 +- 16 (token, rank) pairs. The
// 64-token-group kernels read an expert's weight slice once per group, about four times per call,
// and most of the repeats come from beyond L2. Here a unit is (tile of up to 320 tokens of one
// expert, 128 intermediate rows): the block holds the fp32 products of the 256 weight rows (gate
// and up of those 128 rows) with the tile's 320 token columns, so every weight line is read once
// per tile (once per call for almost every expert at T = 8192) and the tile's x rows once per 128
// intermediate rows. The units of one tile (its 128-row slices) are numbered next to each other
// and run side by side on one XCD, which then reads the tile's gathered x rows from its own L2.
// The time of a unit is mostly the streaming of its 1 MB of weights, whatever its token count,
// so the tile size is set by the number of units, not by the matrix work.
//
// Operands are staged in LDS in 64-element K slabs: one slab is 256 weight rows and 320 token
// rows of 128 bytes each (bf16), double-buffered. x rows and bf16 weights are loaded straight into
// LDS (buffer loads with the LDS flag: no registers held while in flight), whole 128-byte lines,
// 8 rows per load instruction; FP8 and MXFP4 codes come through registers to be widened (MXFP4
// with its block scale). The next slab's
// loads are in flight during the current slab's matrix instructions; one block barrier per slab.
// Eight waves, two per SIMD: wave w multiplies weight rows 128 (w % 2) .. + 128 (four 16-row gate
// tiles and the four matching up tiles, so h = silu(gate) * up is formed in its registers) by
// token columns 80 (w / 2) .. + 80 (five 16-token tiles); a wave whose columns hold no token of
// the tile skips its matrix instructions.
//
// Per output element the arithmetic is that of the 64-token-group kernels: the same matrix
// instruction, the same k order (k step kappa covers elements 32 kappa .. 32 kappa + 31, lane
// group q holding 32 kappa + 8 q .. + 7; the steps accumulate in increasing kappa), the same row
// scales for FP8 weights (after the K loop), the same SiLU and hi/lo split of h; a token's bits do
// not depend on which of them ran it.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kGWaves = 8;                      // two waves per SIMD
constexpr int kGThreads = kGWaves * kWave;
constexpr int kGTok = 320;                      // tokens per tile
constexpr int kGRows = 128;                     // intermediate rows per unit
constexpr int kGWRows = 2 * kGRows;             // weight rows per unit (gate, then up)
constexpr int kGRowB = 128;                     // bytes of one staged row (64 bf16)
constexpr int kGSlab = kGRowB / 2;              // K elements per slab
constexpr int kGWBytes = kGWRows * kGRowB;      // weight part of a slab buffer (32 KB)
constexpr int kGXBytes = kGTok * kGRowB;        // x part of a slab buffer (40 KB)
constexpr int kGSegs = kGWBytes / 1024 / kGWaves; // 1 KB weight segments per wave (4)
constexpr int kGXSegs = kGXBytes / 1024 / kGWaves; // 1 KB x segments per wave (5)
constexpr int kGTT = kGTok / 4 / kTile;         // token tiles per wave (5)
constexpr int kGRT = 8;                         // weight tiles per wave (4 gate, 4 up)
constexpr int kGXcds = 8;                       // XCDs of the chip, each with its own L2

__device__ __forceinline__ uint4 lds_read16(const unsigned char *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

// Byte position of 16-byte piece pc (0..7) of staged row r: rows 2m and 2m + 1 rotate their
// pieces by m, so that the 16 rows one operand read touches fall on 16 distinct bank groups. The
// rotation depends on r % 16 only, so rows 16 apart keep their pieces' order: a fragment of any
// 16-row tile sits at the lane's own offset plus a constant.
__device__ __forceinline__ int gpos(int r, int pc) { return r * kGRowB + ((pc ^ (r >> 1)) & 7) * 16; }
constexpr int kGTileB = kTile * kGRowB;  // bytes of 16 staged rows

// The two slab buffers (each a weight part and an x part) are separate objects, so that the
// compiler can tell loads straight into one (buffer loads with the LDS flag) from operand reads of
// the other; otherwise it waits for every such load before any LDS read.
__shared__ __align__(16) unsigned char g_wslab0[kGWBytes], g_wslab1[kGWBytes];
__shared__ __align__(16) unsigned char g_xslab0[kGXBytes], g_xslab1[kGXBytes];
template <int B>
__device__ __forceinline__ unsigned char *wslab() { return B ? g_wslab1 : g_wslab0; }
template <int B>
__device__ __forceinline__ unsigned char *xslab() { return B ? g_xslab1 : g_xslab0; }

// 16 bytes per lane from buffer offset off into LDS: lane l writes bytes 16 l .. 16 l + 15 of the
// 1 KB segment at seg (wave-uniform).
template <int kAux>
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, unsigned char *seg, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)seg, 16, (int)off, 0, 0, kAux);
}

// Weight formats of the kernel: bf16 (loaded straight into LDS); FP8 E4M3 codes with a scale per
// row (applied to the products); MXFP4 E2M1 codes with an E8M0 scale per 32 (applied while
// widening). Codes come through registers: a 128-byte code line per row feeds kLineSlabs slabs.
enum { kGBf16 = 0, kGFp8 = 1, kGMx = 2 };
template <int kFmt>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gateup_grp_kernel(GateUpParams p) {
    using Op = OpBF16;
    constexpr bool kCodes = kFmt != kGBf16;
    constexpr int kLineSlabs = kFmt == kGMx ? 4 : kFmt == kGFp8 ? 2 : 1;  // slabs per code line
    constexpr int kPeriod = kFmt == kGMx ? 8 : 4;  // slabs per unrolled loop step
    // code lines are requested kAhead slabs before their first slab is staged, into kSets
    // register sets (MXFP4: one set, a slab ahead - its lines cover four slabs)
    constexpr int kAhead = kFmt == kGMx ? 1 : 2, kSets = kFmt == kGMx ? 1 : 2;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, q = lane >> 4;
    const int rg = wave & 1, th = (wave >> 1) & 3;  // (the mask bounds the LDS offsets for the compiler)

    // unit of this block: blocks b, b + 8, ... run on one XCD and take one contiguous eighth of
    // the units, in order (a tile's slices next to each other)
    const int S = p.S;
    const int nunits = p.num_groups[0] * S;
    const int per = (nunits + kGXcds - 1) / kGXcds;
    const int idx = blockIdx.x / kGXcds;
    const int u = (blockIdx.x % kGXcds) * per + idx;
    if (idx >= per || u >= nunits) return;  // uniform over the block
    const int gi = u / S, j = u - gi * S;
    const int4 grp = p.groups[gi];
    const int e = grp.x, start = grp.y, n = grp.z;
    const bool shared = e == p.E;
    const int Ie = shared ? p.Is : p.I;
    if (j * kGRows >= Ie) return;  // uniform (Ie is a multiple of kGRows)
    const int i0 = j * kGRows + rg * (kGRows / 2);  // the wave's first intermediate row

    const size_t wrow = kFmt == kGMx ? (size_t)p.H / 2 : kFmt == kGFp8 ? (size_t)p.H : (size_t)p.H * 2;
    const unsigned char *wbase = reinterpret_cast<const unsigned char *>(shared ? p.sgu : p.gate_up) +
                                 (shared ? 0 : (size_t)e * 2 * Ie * wrow);
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(wbase, (uint32_t)(2 * Ie * wrow));
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(p.x, (uint32_t)((size_t)p.T * p.H * 2));
    // weight row of stage row R: tile t = R / 16 % 8 of wave group R / 128 (gate t < 4, up above)
    auto wrow_of = [&](int R) {
        const int t = (R >> 4) & 7;
        return (t < 4 ? 0 : Ie) + j * kGRows + (R >> 7) * (kGRows / 2) + (t & 3) * kTile + (R & 15);
    };
    // Straight-to-LDS loads (x rows; bf16 weights): wave w fills the 1 KB segments 5 w + a of the
    // x part (token rows 40 w + 8 a .. + 8) and 4 w + a of the weight part (stage rows
    // 32 w + 8 a .. + 8) of a slab buffer; lane l writes position l % 8 of row l / 8 of its
    // segment, i.e. it loads the piece the row's rotation puts there.
    uint32_t xoff[kGXSegs], woff[kCodes ? 1 : kGSegs];
#pragma unroll
    for (int a = 0; a < kGXSegs; ++a) {
        const int R = 8 * kGXSegs * wave + 8 * a + (lane >> 3);
        const int pc = ((lane & 7) ^ (R >> 1)) & 7;
        const int m = R < n ? R : 0;  // token rows past the tile repeat row 0 (columns dropped)
        const int tok = shared ? start + m : (p.perm[start + m] >> 3);
        xoff[a] = (uint32_t)((size_t)tok * p.H * 2) + pc * 16;
    }
    if constexpr (!kCodes) {
#pragma unroll
        for (int a = 0; a < kGSegs; ++a) {
            const int R = 8 * kGSegs * wave + 8 * a + (lane >> 3);
            woff[a] = (uint32_t)(wrow_of(R) * wrow) + (((lane & 7) ^ (R >> 1)) & 7) * 16;
        }
    }
    // (x segments wholly past the tile's tokens are not loaded: their columns are dropped; a
    // ragged tile then streams little more than its weights)
    auto issue = [&](unsigned char *wbuf, unsigned char *xbuf, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < kGXSegs; ++a)
            if (8 * (kGXSegs * wave + a) < n)  // uniform
                lds_load16<0>(rx, xbuf + (kGXSegs * wave + a) * 1024, xoff[a] + st * kGRowB);
        if constexpr (!kCodes) {
#pragma unroll
            for (int a = 0; a < kGSegs; ++a)
                lds_load16<kBufNT>(rw, wbuf + (kGSegs * wave + a) * 1024, woff[a] + st * kGRowB);
        }
    };
    // Codes go through registers (widened while staged): thread tid takes 16-byte piece lp of the
    // 128-byte code line of stage rows 64 a + lr (and, MXFP4, the scale byte of that piece's 32
    // codes), line L in register set L % kSets.
    constexpr int kW = kCodes ? kGWRows / (kGThreads / 8) : 1;  // line loads per thread (4)
    const int lr = tid >> 3, lp = tid & 7;
    const int srow = p.H / 32;  // MXFP4 scale bytes per row
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(kFmt == kGMx ? (shared ? p.sgu_mx : p.gu_mx + (size_t)e * 2 * Ie * srow) : nullptr,
                    kFmt == kGMx ? (uint32_t)(2 * Ie * srow) : 0u);
    uint32_t w8off[kW], soff[kW];
    if constexpr (kCodes) {
#pragma unroll
        for (int a = 0; a < kW; ++a) {
            const int row = wrow_of(kGThreads / 8 * a + lr);
            w8off[a] = (uint32_t)(row * wrow) + lp * 16;
            soff[a] = (uint32_t)(row * srow) + lp;
        }
    }
    struct Line {
        uint4 c[kW];
        uint32_t s[kFmt == kGMx ? kW : 1];
    };
    Line wa, wb;
    auto load_line = [&](Line &L, int line) __attribute__((always_inline)) {
        if constexpr (kCodes) {
#pragma unroll
            for (int a = 0; a < kW; ++a) L.c[a] = bload16_stream(rw, w8off[a] + line * kGRowB);
            if constexpr (kFmt == kGMx) {
#pragma unroll
                for (int a = 0; a < kW; ++a) L.s[a] = bload1(rs, soff[a] + line * 8);
            }
        }
    };
    // FP8: piece lp holds codes 16 lp .. + 15 of the line, i.e. bf16 pieces 2 (lp % 4) and
    // 2 (lp % 4) + 1 of slab lp / 4; MXFP4: codes 32 lp .. + 31, bf16 pieces 4 (lp % 2) .. + 3 of
    // slab lp / 2 (exact widening; the MXFP4 block scale multiplies as it widens)
    constexpr int kPcs = kFmt == kGMx ? 4 : 2;  // bf16 pieces per code piece
    const int pc0 = kFmt == kGMx ? 4 * (lp & 1) : 2 * (lp & 3);
    const int my_slab = kFmt == kGMx ? lp >> 1 : lp >> 2;  // slab (within the line) of the piece
    int st_off[kPcs];
#pragma unroll
    for (int k = 0; k < kPcs; ++k) st_off[k] = gpos(lr, pc0 + k);
    auto store_line = [&](unsigned char *b, const Line &L, int st) __attribute__((always_inline)) {
        if constexpr (kCodes) {
            if (my_slab == st % kLineSlabs) {
#pragma unroll
                for (int a = 0; a < kW; ++a) {
                    unsigned char *row = b + a * (kGThreads / 8) * kGRowB;
                    const uint32_t w4[4] = {L.c[a].x, L.c[a].y, L.c[a].z, L.c[a].w};
                    if constexpr (kFmt == kGMx) {
                        const float sf = e8m0_to_f32(L.s[a]);
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            *reinterpret_cast<uint4 *>(row + st_off[k]) = e2m1x8_to_bf16x8(w4[k], sf);
                    } else {
                        *reinterpret_cast<uint4 *>(row + st_off[0]) = e4m3x8_to_bf16x8(w4[0], w4[1]);
                        *reinterpret_cast<uint4 *>(row + st_off[1]) = e4m3x8_to_bf16x8(w4[2], w4[3]);
                    }
                }
            }
        }
    };

    f32x4_t acc[kGRT][kGTT];
#pragma unroll
    for (int t = 0; t < kGRT; ++t)
#pragma unroll
        for (int tt = 0; tt < kGTT; ++tt) acc[t][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // token tiles of this wave that hold tokens (uniform)
    int nt_w = (n - th * kGTT * kTile + kTile - 1) / kTile;
    nt_w = nt_w < 0 ? 0 : nt_w > kGTT ? kGTT : nt_w;

    // a k step: the wave's operand fragments (8 weight, 5 token) are read, then multiplied
    const int rd_off[2] = {gpos(col, q), gpos(col, 4 + q)};
    auto rd = [&](uint4 (&a)[kGRT], uint4 (&b)[kGTT], const unsigned char *wbuf, const unsigned char *xbuf,
                  int s) __attribute__((always_inline)) {
        const unsigned char *wb_ = wbuf + rg * kGRT * kGTileB;
        const unsigned char *xb_ = xbuf + th * kGTT * kGTileB;
#pragma unroll
        for (int t = 0; t < kGRT; ++t) a[t] = lds_read16(wb_ + t * kGTileB + rd_off[s]);
#pragma unroll
        for (int tt = 0; tt < kGTT; ++tt) b[tt] = lds_read16(xb_ + tt * kGTileB + rd_off[s]);
    };
    auto mm = [&](const uint4 (&a)[kGRT], const uint4 (&b)[kGTT]) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < kGTT; ++tt)
#pragma unroll
            for (int t = 0; t < kGRT; ++t) Op::mma(acc[t][tt], a[t], b[tt]);
    };
    uint4 a0[kGRT], b0[kGTT];

    const int nslab = p.H / kGSlab;  // a multiple of kPeriod
    // slab st0 + i (in buffer B = i % 2; st0 a multiple of kPeriod, so slab st0 + i's code line
    // is in set (i / kLineSlabs) % kSets): request slab st + 1 into the other buffer (read by slab
    // st - 1, a barrier ago) and, when slab st + kAhead starts a code line, that line; multiply
    // the slab's two k steps; widen slab st + 1's codes into the other buffer; wait for this
    // wave's loads (but a line requested two slabs ahead), barrier
    auto slab = [&](auto ic, int st0) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        constexpr int B = i & 1;
        constexpr bool kReq = kCodes && (i + kAhead) % kLineSlabs == 0;
        constexpr bool kNextInB = ((i + kAhead) / kLineSlabs) % kSets, kStageFromB = ((i + 1) / kLineSlabs) % kSets;
        const int st = st0 + i;
        if (st + 1 < nslab) issue(wslab<1 - B>(), xslab<1 - B>(), st + 1);
        const bool req = kReq && st + kAhead < nslab;  // a line requested after this slab's LDS loads
        if (req) load_line(kNextInB ? wb : wa, (st + kAhead) / kLineSlabs);
        if (nt_w > 0) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                rd(a0, b0, wslab<B>(), xslab<B>(), s2);
                mm(a0, b0);
            }
        }
        if constexpr (kCodes) {
            if (st + 1 < nslab) {
                mfma_operand_guard();  // the scaled conversions after the matrix steps
                store_line(wslab<1 - B>(), kStageFromB ? wb : wa, st + 1);
            }
        }
        constexpr int kLineLoads = kFmt == kGMx ? 2 * kW : kW;
        static_assert(!kCodes || kLineLoads == 4 || kLineLoads == 8, "vmcnt below");
        if (req && kAhead == 2) __builtin_amdgcn_s_waitcnt(kLineLoads == 8 ? 0x0F78 : 0x0F74);  // all but the line
        else __builtin_amdgcn_s_waitcnt(0x0F70);                                  // vmcnt(0)
        __syncthreads();
    };
    load_line(wa, 0);
    issue(wslab<0>(), xslab<0>(), 0);
    store_line(wslab<0>(), wa, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (int st0 = 0; st0 < nslab; st0 += kPeriod) {
        slab(std::integral_constant<int, 0>{}, st0);
        slab(std::integral_constant<int, 1>{}, st0);
        slab(std::integral_constant<int, 2>{}, st0);
        slab(std::integral_constant<int, 3>{}, st0);
        if constexpr (kPeriod == 8) {
            slab(std::integral_constant<int, 4>{}, st0);
            slab(std::integral_constant<int, 5>{}, st0);
            slab(std::integral_constant<int, 6>{}, st0);
            slab(std::integral_constant<int, 7>{}, st0);
        }
    }
    if (nt_w == 0) return;

    if constexpr (kFmt == kGFp8) {  // the rows' dequantization scales (gate rows, then up rows)
        const float *sc = shared ? p.sgu_scale : p.gu_scale + (size_t)e * 2 * Ie;
#pragma unroll
        for (int t = 0; t < kGRT; ++t)
#pragma unroll
            for (int tt = 0; tt < kGTT; ++tt)
                if (tt < nt_w)
                    scale_rows(acc[t][tt], sc + (t < 4 ? 0 : Ie) + i0 + kTile * (t & 3) + 4 * q);
    }
    uint16_t *hp = reinterpret_cast<uint16_t *>(p.h);
#pragma unroll
    for (int tt = 0; tt < kGTT; ++tt) {
        const int m = (th * kGTT + tt) * kTile + col;  // token row of this lane's column
        if (tt >= nt_w || m >= n) continue;
        const int slot = shared ? p.T * kTopK + start + m : p.perm[start + m];
#pragma unroll
        for (int g2 = 0; g2 < kGRT / 2; ++g2) {
            const f32x4_t ga = acc[g2][tt], up = acc[kGRT / 2 + g2][tt];
            float hv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) hv[r] = ga[r] / (1.0f + expf(-ga[r])) * up[r];
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hi[r] = f32_to_bf16_bits(hv[r]);
                lo[r] = f32_to_bf16_bits(hv[r] - bf16_bits_to_f32(hi[r]));
            }
            const size_t off = (size_t)slot * p.Imax + i0 + g2 * kTile + 4 * q;
            *reinterpret_cast<uint2 *>(hp + off) = uint2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
            *reinterpret_cast<uint2 *>(hp + p.plane + off) =
                uint2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
        }
    }
}

// down_grp_kernel - the down product of the same tiles: unit = (tile of up to 320 tokens of one
// expert, 256 rows of y), so an expert's down rows are read once per tile and a tile's h once per
// 256 rows of y. K (the expert's intermediate rows) goes in slabs of 32 elements: 256 down rows
// and the tile's 320 hi and 320 lo h rows of 64 bytes each, double-buffered, bf16 weights and h
// loaded straight into LDS (a slab of 128 bytes per row would not fit twice), FP8 codes through
// registers (FP8, MXFP4). Eight waves: wave w multiplies y rows 128 (w % 2) .. + 128 (eight 16-row tiles) by
// token columns 80 (w / 2) .. + 80 (five tiles). Per output element the steps, planes and their
// order are those of the 64-token-group down kernels: per k step the hi plane, then the lo plane,
// into one accumulator; FP8 row scales after the K loop; the routing weight (or the shared gate)
// times the product goes to the (token, rank) slot's row of the per-slot buffer.
constexpr int kDRows = 256;                    // rows of y per unit
constexpr int kDRowB = 64;                     // bytes of a staged row (32 bf16)
constexpr int kDSlab = kDRowB / 2;             // K elements per slab (one k step)
constexpr int kDWBytes = kDRows * kDRowB;      // weight part of a slab buffer (16 KB)
constexpr int kDHBytes = 2 * kGTok * kDRowB;   // h part: hi rows, then lo rows (40 KB)
constexpr int kDWSegs = kDWBytes / 1024 / kGWaves;  // 1 KB weight segments per wave (2)
constexpr int kDHSegs = kDHBytes / 1024 / kGWaves;  // 1 KB h segments per wave (5)
constexpr int kDRT = kDRows / 2 / kTile;       // row tiles per wave (8)
__shared__ __align__(16) unsigned char g_dw0[kDWBytes], g_dw1[kDWBytes];
__shared__ __align__(16) unsigned char g_dh0[kDHBytes], g_dh1[kDHBytes];
template <int B>
__device__ __forceinline__ unsigned char *dwslab() { return B ? g_dw1 : g_dw0; }
template <int B>
__device__ __forceinline__ unsigned char *dhslab() { return B ? g_dh1 : g_dh0; }

// Byte position of 16-byte piece pc (0..3) of staged 64-byte row r: rows 2m, 2m + 1 (one 128-byte
// line) rotate their pieces by m % 4, so that an operand read (16 rows x one piece per 16 lanes)
// has no bank conflicts; the rotation depends on r % 8 only. (Rotating rows 4m .. 4m + 3 by m
// instead costs 4 conflict cycles per read: a read probe gives 126 against 140 bytes per clock
// and CU, and the conflict counter 4 per read instruction, against 0.)
__device__ __forceinline__ int dpos(int r, int pc) { return r * kDRowB + ((pc ^ (r >> 1)) & 3) * 16; }
constexpr int kDTileB = kTile * kDRowB;  // bytes of 16 staged rows

template <int kFmt>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void down_grp_kernel(DownParams p) {
    using Op = OpBF16;
    constexpr bool kCodes = kFmt != kGBf16;
    constexpr int kLineSlabs = kFmt == kGMx ? 8 : 4;  // slabs per 128-byte code line
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, q = lane >> 4;
    const int rg = wave & 1, th = (wave >> 1) & 3;  // (the masks bound the LDS offsets for the compiler)

    // unit: blocks b, b + 8, ... run on one XCD and take one contiguous eighth of the units, in
    // order (a tile's row blocks next to each other: they read the same h rows)
    const int nrb = p.H / kDRows;
    const int nunits = p.num_groups[0] * nrb;
    const int per = (nunits + kGXcds - 1) / kGXcds;
    const int idx = blockIdx.x / kGXcds;
    const int u = (blockIdx.x % kGXcds) * per + idx;
    if (idx >= per || u >= nunits) return;  // uniform over the block
    const int gi = u / nrb, rb = u - gi * nrb;
    const int4 grp = p.groups[gi];
    const int e = grp.x, start = grp.y, n = grp.z;
    const bool shared = e == p.E;
    const int Ie = shared ? p.Is : p.I;
    const int row0 = rb * kDRows;  // the unit's first row of y

    const size_t wrow = kFmt == kGMx ? (size_t)Ie / 2 : kFmt == kGFp8 ? (size_t)Ie : (size_t)Ie * 2;
    const unsigned char *wbase = reinterpret_cast<const unsigned char *>(shared ? p.sdn : p.down) +
                                 (shared ? 0 : (size_t)e * p.H * wrow) + (size_t)row0 * wrow;
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(wbase, (uint32_t)(kDRows * wrow));
    const __amdgpu_buffer_rsrc_t rh = buffer_rsrc(p.h, (uint32_t)(2 * p.plane * 2));
    // Straight-to-LDS loads: wave w fills h segments 5 w + a (h stage rows 80 w + 16 a .. + 16:
    // rows < 320 the hi plane of token row r, rows >= 320 the lo plane of token row r - 320) and
    // bf16 weight segments 2 w + a (down rows 32 w + 16 a .. + 16); lane l writes position l % 4 of
    // row l / 4 of its segment, i.e. it loads the piece the row's rotation puts there.
    uint32_t hoff[kDHSegs], woff[kCodes ? 1 : kDWSegs];
#pragma unroll
    for (int a = 0; a < kDHSegs; ++a) {
        const int R = 16 * (kDHSegs * wave + a) + (lane >> 2);
        const int pc = ((lane & 3) ^ (R >> 1)) & 3;
        const int pl = R >= kGTok, r = R - pl * kGTok;
        const int m = r < n ? r : 0;  // token rows past the tile repeat row 0 (columns dropped)
        const int slot = shared ? p.T * kTopK + start + m : p.perm[start + m];
        hoff[a] = (uint32_t)(((size_t)pl * p.plane + (size_t)slot * p.Imax) * 2) + pc * 16;
    }
    if constexpr (!kCodes) {
#pragma unroll
        for (int a = 0; a < kDWSegs; ++a) {
            const int R = 16 * (kDWSegs * wave + a) + (lane >> 2);
            woff[a] = (uint32_t)(R * wrow) + (((lane & 3) ^ (R >> 1)) & 3) * 16;
        }
    }
    auto issue = [&](unsigned char *wbuf, unsigned char *hbuf, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < kDHSegs; ++a) {
            const int R0 = 16 * (kDHSegs * wave + a);
            if ((R0 >= kGTok ? R0 - kGTok : R0) < n)  // uniform: segments past the tile not loaded
                lds_load16<0>(rh, hbuf + (kDHSegs * wave + a) * 1024, hoff[a] + st * kDRowB);
        }
        if constexpr (!kCodes) {
#pragma unroll
            for (int a = 0; a < kDWSegs; ++a)
                lds_load16<kBufNT>(rw, wbuf + (kDWSegs * wave + a) * 1024, woff[a] + st * kDRowB);
        }
    };
    // Codes through registers: thread tid takes 16-byte piece lp of the 128-byte code line of down
    // rows 64 a + lr - FP8: codes 16 lp .. + 15, bf16 pieces 2 (lp % 2), 2 (lp % 2) + 1 of slab
    // lp / 2; MXFP4: codes 32 lp .. + 31 with their scale byte, the four bf16 pieces of slab lp -
    // one register set, a line requested a slab ahead of its first slab.
    constexpr int kW = kCodes ? kDRows / (kGThreads / 8) : 1;  // line loads per thread (4)
    const int lr = tid >> 3, lp = tid & 7;
    const int srow = Ie / 32;  // MXFP4 scale bytes per row
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(
        kFmt == kGMx ? (shared ? p.sdn_mx : p.dn_mx + (size_t)e * p.H * srow) + (size_t)row0 * srow : nullptr,
        kFmt == kGMx ? (uint32_t)(kDRows * srow) : 0u);
    uint32_t w8off[kW], soff[kW];
    if constexpr (kCodes) {
#pragma unroll
        for (int a = 0; a < kW; ++a) {
            w8off[a] = (uint32_t)((kGThreads / 8 * a + lr) * wrow) + lp * 16;
            soff[a] = (uint32_t)((kGThreads / 8 * a + lr) * srow) + lp;
        }
    }
    uint4 wl[kW];
    uint32_t wsc[kFmt == kGMx ? kW : 1];
    auto load_line = [&](int line) __attribute__((always_inline)) {
        if constexpr (kCodes) {
#pragma unroll
            for (int a = 0; a < kW; ++a) wl[a] = bload16_stream(rw, w8off[a] + line * 128);
            if constexpr (kFmt == kGMx) {
#pragma unroll
                for (int a = 0; a < kW; ++a) wsc[a] = bload1(rs, soff[a] + line * 8);
            }
        }
    };
    constexpr int kPcs = kFmt == kGMx ? 4 : 2;  // bf16 pieces per code piece
    const int pc0 = kFmt == kGMx ? 0 : 2 * (lp & 1);
    const int my_slab = kFmt == kGMx ? lp : lp >> 1;
    int st_off[kPcs];
#pragma unroll
    for (int k = 0; k < kPcs; ++k) st_off[k] = dpos(lr, pc0 + k);
    auto store_line = [&](unsigned char *b, int st) __attribute__((always_inline)) {
        if constexpr (kCodes) {
            if (my_slab == st % kLineSlabs) {
#pragma unroll
                for (int a = 0; a < kW; ++a) {
                    unsigned char *row = b + a * (kGThreads / 8) * kDRowB;
                    const uint32_t w4[4] = {wl[a].x, wl[a].y, wl[a].z, wl[a].w};
                    if constexpr (kFmt == kGMx) {
                        const float sf = e8m0_to_f32(wsc[a]);
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            *reinterpret_cast<uint4 *>(row + st_off[k]) = e2m1x8_to_bf16x8(w4[k], sf);
                    } else {
                        *reinterpret_cast<uint4 *>(row + st_off[0]) = e4m3x8_to_bf16x8(w4[0], w4[1]);
                        *reinterpret_cast<uint4 *>(row + st_off[1]) = e4m3x8_to_bf16x8(w4[2], w4[3]);
                    }
                }
            }
        }
    };

    f32x4_t acc[kDRT][kGTT];
#pragma unroll
    for (int t = 0; t < kDRT; ++t)
#pragma unroll
        for (int tt = 0; tt < kGTT; ++tt) acc[t][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int nt_w = (n - th * kGTT * kTile + kTile - 1) / kTile;
    nt_w = nt_w < 0 ? 0 : nt_w > kGTT ? kGTT : nt_w;

    // a slab (one k step): the wave's 8 weight and 5 + 5 h fragments are read, then multiplied,
    // hi plane then lo plane per accumulator
    const int rd_off = dpos(col, q);
    auto compute = [&](const unsigned char *wbuf, const unsigned char *hbuf) __attribute__((always_inline)) {
        const unsigned char *wb_ = wbuf + rg * kDRT * kDTileB;
        const unsigned char *hb_ = hbuf + th * kGTT * kDTileB;
        uint4 a[kDRT], bh[kGTT], bl[kGTT];
#pragma unroll
        for (int t = 0; t < kDRT; ++t) a[t] = lds_read16(wb_ + t * kDTileB + rd_off);
#pragma unroll
        for (int tt = 0; tt < kGTT; ++tt) {
            bh[tt] = lds_read16(hb_ + tt * kDTileB + rd_off);
            bl[tt] = lds_read16(hb_ + kGTok * kDRowB + tt * kDTileB + rd_off);
        }
#pragma unroll
        for (int tt = 0; tt < kGTT; ++tt) {
#pragma unroll
            for (int t = 0; t < kDRT; ++t) Op::mma(acc[t][tt], a[t], bh[tt]);
#pragma unroll
            for (int t = 0; t < kDRT; ++t) Op::mma(acc[t][tt], a[t], bl[tt]);
        }
    };

    const int nslab = Ie / kDSlab;  // a multiple of kLineSlabs
    // slab st (buffer B = st % 2): request slab st + 1 into the other buffer (read by slab st - 1,
    // a barrier ago) and, FP8, at the last slab of a code line the next line; multiply; FP8: widen
    // slab st + 1's codes into the other buffer; wait for this wave's loads, barrier
    auto slab = [&](auto ic, int st0) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        constexpr int B = i & 1;
        const int st = st0 + i;
        if (st + 1 < nslab) issue(dwslab<1 - B>(), dhslab<1 - B>(), st + 1);
        if constexpr (kCodes && (i + 1) % kLineSlabs == 0)
            if (st + 1 < nslab) load_line((st + 1) / kLineSlabs);
        if (nt_w > 0) compute(dwslab<B>(), dhslab<B>());
        if constexpr (kCodes) {
            if (st + 1 < nslab) {
                mfma_operand_guard();  // the scaled conversions after the matrix steps
                store_line(dwslab<1 - B>(), st + 1);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
    };
    load_line(0);
    issue(dwslab<0>(), dhslab<0>(), 0);
    store_line(dwslab<0>(), 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (int st0 = 0; st0 < nslab; st0 += kLineSlabs) {
        slab(std::integral_constant<int, 0>{}, st0);
        slab(std::integral_constant<int, 1>{}, st0);
        slab(std::integral_constant<int, 2>{}, st0);
        slab(std::integral_constant<int, 3>{}, st0);
        if constexpr (kLineSlabs == 8) {
            slab(std::integral_constant<int, 4>{}, st0);
            slab(std::integral_constant<int, 5>{}, st0);
            slab(std::integral_constant<int, 6>{}, st0);
            slab(std::integral_constant<int, 7>{}, st0);
        }
    }
    if (nt_w == 0) return;

    if constexpr (kFmt == kGFp8) {  // the output rows' dequantization scales
        const float *sc = (shared ? p.sdn_scale : p.dn_scale + (size_t)e * p.H) + row0 + rg * kDRT * kTile + 4 * q;
#pragma unroll
        for (int t = 0; t < kDRT; ++t)
#pragma unroll
            for (int tt = 0; tt < kGTT; ++tt) scale_rows(acc[t][tt], sc + t * kTile);
    }
#pragma unroll
    for (int tt = 0; tt < kGTT; ++tt) {
        const int m = (th * kGTT + tt) * kTile + col;
        if (tt >= nt_w || m >= n) continue;
        const int slot = shared ? p.T * kTopK + start + m : p.perm[start + m];
        const float wt = shared ? p.g[start + m] : p.w[slot];
        // lane holds rows 4q + r of each of the wave's 16-row tiles for its token column
#pragma unroll
        for (int t = 0; t < kDRT; ++t)
            *reinterpret_cast<float4 *>(p.ybuf + (size_t)slot * p.H + row0 + (rg * kDRT + t) * kTile + 4 * q) =
                make_float4(wt * acc[t][tt][0], wt * acc[t][tt][1], wt * acc[t][tt][2], wt * acc[t][tt][3]);
    }
}

}  // namespace

int grp_tile_tokens() { return kGTok; }
int grp_rows_per_gateup_unit() { return kGRows; }
size_t gateup_grp_lds() { return 0; }  // static LDS (two slab buffers)

// dtype: 1 bf16, 2 FP8 E4M3, 3 MXFP4 weights (bf16 activations)
bool gateup_grp_supported(int H, int I, int Is, int dtype, long x_bytes) {
    if (dtype < 1 || dtype > 3) return false;
    if (H % ((dtype == 3 ? 8 : 4) * kGSlab) || I % kGRows || Is % kGRows) return false;  // whole loop steps
    const long wbytes = 2L * (I > Is ? I : Is) * H * (dtype == 1 ? 2 : 1);
    return wbytes < (1L << 31) && x_bytes < (1L << 31);
}

// dtype: 1 bf16, 2 FP8 E4M3, 3 MXFP4 down weights
bool down_grp_supported(int H, int I, int Is, int dtype, size_t h_bytes) {
    if (dtype < 1 || dtype > 3) return false;
    const int m = dtype == 3 ? 256 : 128;  // whole loop steps (code lines)
    if (H % kDRows || I % m || Is % m) return false;
    return (size_t)kDRows * (I > Is ? I : Is) * 2 < (1u << 31) && h_bytes < (1u << 31);
}

hipError_t launch_down_grp(const DownParams &p, int dtype, int grid, hipStream_t s) {
    if (grid % kGXcds || p.NG != kGTok || p.H % kDRows) return hipErrorInvalidValue;  // a caller bug
    if (dtype == 3) launch_k(down_grp_kernel<kGMx>, grid, kGThreads, 0, s, p);
    else if (dtype == 2) launch_k(down_grp_kernel<kGFp8>, grid, kGThreads, 0, s, p);
    else launch_k(down_grp_kernel<kGBf16>, grid, kGThreads, 0, s, p);
    return hipGetLastError();
}
int grp_rows_per_down_unit() { return kDRows; }

hipError_t prepare_grouped_kernels() {
    hipError_t err;
    const void *k[] = {reinterpret_cast<const void *>(&gateup_grp_kernel<kGBf16>),
                       reinterpret_cast<const void *>(&gateup_grp_kernel<kGFp8>),
                       reinterpret_cast<const void *>(&gateup_grp_kernel<kGMx>)};
    for (const void *f : k)
        if ((err = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)gateup_grp_lds())) != hipSuccess)
            return err;
    return hipSuccess;
}

// dtype: 1 bf16, 2 FP8 E4M3, 3 MXFP4 weights (bf16 activations). p.groups: tiles of at most
// grp_tile_tokens() tokens; p.S: grp_rows_per_gateup_unit()-row slices of Imax; grid: a multiple
// of 8 holding every unit (8 * ceil(max tiles * S / 8)).
hipError_t launch_gateup_grp(const GateUpParams &p, int dtype, int grid, hipStream_t s) {
    if (grid % kGXcds || p.NG != kGTok) return hipErrorInvalidValue;  // a caller bug
    if (dtype == 3) launch_k(gateup_grp_kernel<kGMx>, grid, kGThreads, gateup_grp_lds(), s, p);
    else if (dtype == 2) launch_k(gateup_grp_kernel<kGFp8>, grid, kGThreads, gateup_grp_lds(), s, p);
    else launch_k(gateup_grp_kernel<kGBf16>, grid, kGThreads, gateup_grp_lds(), s, p);
    return hipGetLastError();
}

}  // namespace moe
