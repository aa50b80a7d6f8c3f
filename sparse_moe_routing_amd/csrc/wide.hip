// wide.hip - the expert stage for larger rounds (T > 64): expert groups of up to 64 tokens.
//
// With the decode path's 8-token groups an expert that draws 150 tokens (the skewed verify
// workload) would have its weights read nineteen times. Here a group holds up to 64 tokens, so every weight fragment that a wave
// stages feeds four 16-token matrix-core tiles and an expert's weights are read once per 64 of
// its tokens. The token operands no longer fit in LDS for the whole K range, so they are staged
// one 256-byte K chunk at a time, double-buffered, with one block barrier per chunk:
//
// gateup_wide_kernel - unit = (expert group, 64 intermediate rows), 8 waves: waves 0-3 stream
//   the 16-row gate tiles, waves 4-7 the matching up tiles (each load instruction reads 256
//   contiguous bytes of 4 rows, reordered into operands through a swizzled per-wave LDS buffer,
//   as in gateup_down.hip); the group's x chunk is staged cooperatively and shared by all eight
//   tiles; h = silu(gate) * up goes to the workspace (bf16: hi/lo planes).
// down_wide_kernel - unit = (expert group, 256 rows of y), 8 waves of two 16-row tiles each over
//   the contiguous 256-row block of the down weight, against the group's h (hi and lo planes
//   staged per chunk and shared by the sixteen tiles: h bytes per unit stay below weight bytes);
//   w * (Wd h) goes to the (token, rank) slot rows of the [slots][H] buffer, which the combine
//   kernel sums in rank order.
//
// Per output element the arithmetic is that of gateup_down.hip (the same matrix instruction, the
// same k order over chunks and steps, the same SiLU and split of h), so a token's bits do not
// depend on which of the two paths computed it.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kWWaves = 8;                    // waves per block
constexpr int kWThreads = kWWaves * kWave;
constexpr int kDownTiles = 2;                 // 16-row tiles of the down weight per wave
constexpr int kWPieces = 16;                  // 16-byte pieces per row per chunk (256 bytes)
constexpr int kWStage = kTile * kWPieces * 16;  // one wave's 16 x 256-byte weight chunk
// LDS row of a staged token chunk: 256 bytes plus 16. On gfx950 an operand read of 16 such rows
// still costs 4 bank-conflict cycles (conflict counter and a read probe); a conflict-free
// rotation of 256-byte rows measured no faster in these kernels and needs registers the wide
// gate/up kernel does not have at 4 waves per SIMD.
constexpr int kXRow = kWPieces * 16 + 16;

__device__ __forceinline__ uint4 lds_read16(const unsigned char *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

// Weight chunk of one wave (16 rows x 256 bytes of operands). bf16 / fp32: 4 loads of 4 rows x
// 256 bytes (lane: row lane / 16 + 4a, 16-byte piece lane % 16). FP8 codes (128 bytes per row):
// 2 loads of 8 rows x 128 bytes (lane: row lane / 8 + 8a, 16 codes at lane % 8), widened to bf16
// when staged.
// MXFP4 storage (packed E2M1 codes, an E8M0 scale byte per 32 weights) as a weight format of the
// wide kernels: a loaded piece carries its 32 codes and their scale byte.
struct MxFmt {
    using wt_t = uint8_t;
    struct raw_t {
        uint4 c;
        uint32_t s;
    };
    static constexpr bool kScaled = false;  // no row scales: the block scales act on load
};

template <class WF>
struct WChunk {
    static constexpr bool kMx = false;
    static constexpr bool k8 = WF::kScaled;
    static constexpr int kLoads = k8 ? 2 : 4;
    static constexpr int kRowStep = k8 ? 8 : 4;
    using raw_t = typename std::conditional<k8, uint4, typename WF::raw_t>::type;
    // the lane's first row and its element offset in a chunk
    __device__ static __forceinline__ int row(int lane) { return k8 ? lane >> 3 : lane >> 4; }
    __device__ static __forceinline__ int elem(int lane) {
        return k8 ? (lane & 7) * 16 : (lane & 15) * (int)(16 / sizeof(typename WF::wt_t));
    }
};

// MXFP4 chunk of one wave (16 rows x 64 bytes of codes): one load, lane: row lane / 4, the 32
// codes of scale block lane % 4 of the chunk, and that block's scale byte.
template <>
struct WChunk<MxFmt> {
    static constexpr bool kMx = true;
    static constexpr int kLoads = 1;
    using raw_t = MxFmt::raw_t;
    __device__ static __forceinline__ int row(int lane) { return lane >> 2; }
    __device__ static __forceinline__ int elem(int lane) { return (lane & 3) * 16; }  // bytes
};

// ssrc: the lane's scale byte of chunk 0 (MXFP4 only; the chunk's four blocks follow it)
template <class WF, int kCE>
__device__ __forceinline__ void load_wchunk(typename WChunk<WF>::raw_t (&r)[WChunk<WF>::kLoads],
                                            const typename WF::wt_t *src, size_t row_stride, int c,
                                            const uint8_t *ssrc = nullptr) {
    using W = WChunk<WF>;
    if constexpr (W::kMx) {
        r[0].c = load16_stream(src + c * (kCE / 2));
        r[0].s = ssrc[c * 4];
    } else {
#pragma unroll
        for (int a = 0; a < W::kLoads; ++a) {
            const typename WF::wt_t *ptr = src + (size_t)(W::kRowStep * a) * row_stride + c * kCE;
            if constexpr (W::k8) r[a] = load16_stream(ptr);
            else r[a] = WF::load_raw(ptr);
        }
    }
}

// Swizzled staging (row rr, piece p at rr * 256 + ((p ^ rr) & 15) * 16) and operand read of
// step s (piece 4s + q of row col).
template <class WF>
__device__ __forceinline__ void stage_w(unsigned char *buf,
                                        const typename WChunk<WF>::raw_t (&r)[WChunk<WF>::kLoads],
                                        int lane) {
    using W = WChunk<WF>;
    if constexpr (W::kMx) {  // 32 codes times their block scale as four bf16 pieces (exact)
        const int rr = W::row(lane), pb = 4 * (lane & 3);
        const float sf = e8m0_to_f32(r[0].s);
        const uint32_t w4[4] = {r[0].c.x, r[0].c.y, r[0].c.z, r[0].c.w};
        mfma_operand_guard();
#pragma unroll
        for (int k = 0; k < 4; ++k)
            *reinterpret_cast<uint4 *>(buf + rr * 256 + ((mx_piece_pos(pb + k, 0) ^ rr) & 15) * 16) =
                e2m1x8_to_bf16x8(w4[k], sf);
    } else {
        if constexpr (W::k8) mfma_operand_guard();  // the FP8 conversions as the MXFP4 ones
#pragma unroll
        for (int a = 0; a < W::kLoads; ++a) {
            const int rr = W::kRowStep * a + W::row(lane);
            if constexpr (W::k8) {  // 16 codes widened to two bf16 pieces (exact)
                const int p0 = 2 * (lane & 7);
                *reinterpret_cast<uint4 *>(buf + rr * 256 + ((fp8_piece_pos(p0) ^ rr) & 15) * 16) =
                    e4m3x8_to_bf16x8(r[a].x, r[a].y);
                *reinterpret_cast<uint4 *>(buf + rr * 256 + ((fp8_piece_pos(p0 + 1) ^ rr) & 15) * 16) =
                    e4m3x8_to_bf16x8(r[a].z, r[a].w);
            } else {
                const int lpiece = lane & 15;
                *reinterpret_cast<uint4 *>(buf + rr * 256 + ((lpiece ^ rr) & 15) * 16) =
                    WF::to_operand(r[a]);
            }
        }
    }
}
// kMap: 0 plain, 1 MXFP4, 2 FP8 piece positions (as staged by stage_w)
template <int kMap = 0>
__device__ __forceinline__ uint4 w_operand(const unsigned char *buf, int s, int col, int q) {
    const int pc = kMap == 1 ? mx_piece_pos(4 * s + q, 0) : kMap == 2 ? fp8_piece_pos(4 * s + q)
                                                                      : 4 * s + q;
    return lds_read16(buf + col * 256 + ((pc ^ col) & 15) * 16);
}

}  // namespace

template <class Op, int NT, bool kFp8, bool kMx = false>
__global__ __launch_bounds__(kWThreads) void gateup_wide_kernel(GateUpParams p) {
    using elem_t = typename Op::elem_t;
    using WF = typename std::conditional<kMx, MxFmt, WeightFmt<Op, kFp8>>::type;
    constexpr int kPack = kMx ? 2 : 1;  // weights per stored element
    using wt_t = typename WF::wt_t;
    constexpr int TG = NT * kTile;
    constexpr int kCE = kWPieces * Op::kPerLane;
    constexpr int kSteps = kWPieces / 4;
    constexpr int kGW = kWWaves / 2;   // gate waves (and up waves)
    constexpr int kSW = kGW * kTile;   // intermediate rows per unit
    constexpr int kXPasses = TG * kWPieces / kWThreads;  // x chunk loads per thread
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *xs = smem;                                       // [2][TG][kXRow]
    unsigned char *stage_all = smem + 2 * TG * kXRow;               // [waves][4 KB]
    // [kGW][NT][16][16] up tiles, in the stage area of the up waves once their K loop is done
    float *xchg = reinterpret_cast<float *>(stage_all + kGW * kWStage);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, q = lane >> 4;
    unsigned char *stage = stage_all + wave * kWStage;
    const int nunits = p.num_groups[0] * p.S;
    const int nchunks = p.H / kCE;
    const elem_t *x = reinterpret_cast<const elem_t *>(p.x);
    const int xp = tid & 15, xr0 = tid >> 4;  // x loader: piece xp of rows xr0 + (threads/16) i
    constexpr int kXRowsPerPass = kWThreads / kWPieces;

    for (int u = blockIdx.x; u < nunits; u += gridDim.x) {
        const int gi = u / p.S, j = u - (u / p.S) * p.S;
        const int4 grp = p.groups[gi];
        const int e = grp.x, start = grp.y, n = grp.z;
        const bool shared = e == p.E;
        const int Ie = shared ? p.Is : p.I;
        if (j * kSW >= Ie) continue;  // uniform over the block
        const int nt_used = (n + kTile - 1) / kTile;

        const wt_t *gu = reinterpret_cast<const wt_t *>(shared ? p.sgu : p.gate_up) +
                         (shared ? 0 : (size_t)e * 2 * Ie * (p.H / kPack));
        const int wrow0 = (wave < kGW ? 0 : Ie) + j * kSW + (wave % kGW) * kTile;
        using W = WChunk<WF>;
        const wt_t *src = gu + (size_t)(wrow0 + W::row(lane)) * (p.H / kPack) + W::elem(lane);
        const int srow = p.H / 32;  // MXFP4 scale bytes per row
        const uint8_t *ssrc = kMx ? (shared ? p.sgu_mx : p.gu_mx + (size_t)e * 2 * Ie * srow) +
                                        (size_t)(wrow0 + W::row(lane)) * srow + (lane & 3)
                                  : nullptr;
        const elem_t *xsrc[kXPasses];
#pragma unroll
        for (int i = 0; i < kXPasses; ++i) {
            const int r = xr0 + kXRowsPerPass * i;
            const int rr = r < n ? r : 0;  // rows >= n repeat row 0 (their columns are dropped)
            const int tok = shared ? start + rr : (p.perm[start + rr] >> 3);
            xsrc[i] = x + (size_t)tok * p.H + xp * Op::kPerLane;
        }
        // weight chunks in flight: a ring of kWD register buffers (FP8 codes are half the bytes,
        // so more chunks fill the same registers); bf16: 3 measured best (uniform T = 192 gate/up
        // 196.9 us against 202.9 with 2; 4 drops to three waves per SIMD: 206.8)
        constexpr int kWD = kMx ? 8 : kFp8 ? 4 : 3;
        typename W::raw_t wr[kWD][W::kLoads];
        uint4 xv[kXPasses];
        // a pass whose rows all lie past n is skipped (uniform): the columns those rows feed are
        // dropped, whatever the stale LDS holds
        auto load_x = [&](int c) {
#pragma unroll
            for (int i = 0; i < kXPasses; ++i)
                if (kXRowsPerPass * i < n) xv[i] = load16(xsrc[i] + c * kCE);
        };
        auto store_x = [&](int buf) {
#pragma unroll
            for (int i = 0; i < kXPasses; ++i)
                if (kXRowsPerPass * i < n)
                    *reinterpret_cast<uint4 *>(xs + (buf * TG + xr0 + kXRowsPerPass * i) * kXRow +
                                               xp * 16) = xv[i];
        };
        f32x4_t acc[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
        for (int d = 0; d < kWD; ++d)
            if (d < nchunks) load_wchunk<WF, kCE>(wr[d], src, p.H, d, ssrc);
        load_x(0);
        __syncthreads();  // the previous unit's readers of xs / xchg are done
        store_x(0);
        auto step = [&](typename W::raw_t (&wcur)[W::kLoads], int c) {
            if (c + 1 < nchunks) load_x(c + 1);
            __syncthreads();  // x chunk c is staged; chunk c - 1's readers are done
            stage_w<WF>(stage, wcur, lane);
            if (c + kWD < nchunks) load_wchunk<WF, kCE>(wcur, src, p.H, c + kWD, ssrc);
            const unsigned char *xb = xs + (c & 1) * TG * kXRow;
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
                const uint4 a = w_operand<kMx ? 1 : kFp8 ? 2 : 0>(stage, s, col, q);
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
                    if (tt < nt_used)  // uniform
                        Op::mma(acc[tt], a, lds_read16(xb + (tt * kTile + col) * kXRow + (4 * s + q) * 16));
            }
            if (c + 1 < nchunks) store_x((c + 1) & 1);
        };
        for (int c = 0; c < nchunks; c += kWD) {
#pragma unroll
            for (int d = 0; d < kWD; ++d)
                if (c + d < nchunks) step(wr[d], c + d);  // uniform
        }

        if constexpr (WF::kScaled) {  // the rows' dequantization scales (gate rows, then up rows)
            const float *sc = (shared ? p.sgu_scale : p.gu_scale + (size_t)e * 2 * Ie) + wrow0 + 4 * q;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) scale_rows(acc[tt], sc);
        }
        // up waves hand their tiles over (into their own stage buffers, free now); gate waves
        // form h
        static_assert(kGW * NT * kTile * kTile * 4 <= kGW * kWStage, "exchange exceeds the up stages");
        if (wave >= kGW) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
                *reinterpret_cast<f32x4_t *>(xchg + (((wave - kGW) * NT + tt) * kTile + col) * kTile + 4 * q) =
                    acc[tt];
        }
        __syncthreads();
        if (wave >= kGW) continue;
        const int i0 = j * kSW + wave * kTile + 4 * q;  // intermediate rows i0 + r of this lane
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int cc = tt * kTile + col;  // group row of this lane's token column
            if (cc >= n) continue;
            const f32x4_t up = *reinterpret_cast<const f32x4_t *>(
                xchg + ((wave * NT + tt) * kTile + col) * kTile + 4 * q);
            const int slot = shared ? p.T * kTopK + start + cc : p.perm[start + cc];
            float hv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) hv[r] = acc[tt][r] / (1.0f + expf(-acc[tt][r])) * up[r];
            const size_t off = (size_t)slot * p.Imax + i0;
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
}

template <class Op, int NT, bool kFp8, bool kMx = false>
__global__ __launch_bounds__(kWThreads) void down_wide_kernel(DownParams p) {
    using elem_t = typename Op::elem_t;
    using WF = typename std::conditional<kMx, MxFmt, WeightFmt<Op, kFp8>>::type;
    constexpr int kPack = kMx ? 2 : 1;  // weights per stored element
    using wt_t = typename WF::wt_t;
    constexpr int TG = NT * kTile;
    constexpr int kCE = kWPieces * Op::kPerLane;
    constexpr int kSteps = kWPieces / 4;
    constexpr int kRowsPerUnit = kWWaves * kDownTiles * kTile;  // 256
    constexpr int kPlanes = Op::kElemBytes == 2 ? 2 : 1;  // h as hi + lo bf16, or fp32
    constexpr int kHPasses = TG * kWPieces / kWThreads;
    constexpr int kHRowsPerPass = kWThreads / kWPieces;
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *hs = smem;                                      // [2][planes][TG][kXRow]
    unsigned char *stage_all = smem + 2 * kPlanes * TG * kXRow;    // [waves][tiles][4 KB]

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, q = lane >> 4;
    unsigned char *stage = stage_all + wave * kDownTiles * kWStage;
    const int n_rc = (p.H + kRowsPerUnit - 1) / kRowsPerUnit;  // the last block may be partial
    const int nunits = p.num_groups[0] * n_rc;
    const elem_t *hg = reinterpret_cast<const elem_t *>(p.h);
    const int hp = tid & 15, hr0 = tid >> 4;  // h loader: piece hp of rows hr0 + 16 i

    for (int u = blockIdx.x; u < nunits; u += gridDim.x) {
        const int gi = u / n_rc, rc = u - (u / n_rc) * n_rc;
        const int4 grp = p.groups[gi];
        const int e = grp.x, start = grp.y, n = grp.z;
        const bool shared = e == p.E;
        const int Ie = shared ? p.Is : p.I;
        const int nchunks = Ie / kCE;
        const int nt_used = (n + kTile - 1) / kTile;
        const int rowe = Ie / kPack;  // stored elements per weight row
        const wt_t *dn = reinterpret_cast<const wt_t *>(shared ? p.sdn : p.down) +
                         (shared ? 0 : (size_t)e * p.H * rowe);
        // rows rc * 256 + wave * 32 + tile * 16 + ...: one contiguous 32-row block per wave; a wave
        // past H (H is a multiple of 32) only joins the block barriers
        const int wrow = rc * kRowsPerUnit + wave * kDownTiles * kTile;
        const bool rows_ok = wrow < p.H;  // uniform over the wave
        using W = WChunk<WF>;
        const wt_t *src = dn + (size_t)((rows_ok ? wrow : 0) + W::row(lane)) * rowe + W::elem(lane);
        const int srow = Ie / 32;  // MXFP4 scale bytes per row
        const uint8_t *ssrc = kMx ? (shared ? p.sdn_mx : p.dn_mx + (size_t)e * p.H * srow) +
                                        (size_t)((rows_ok ? wrow : 0) + W::row(lane)) * srow + (lane & 3)
                                  : nullptr;
        const elem_t *hsrc[kHPasses];
#pragma unroll
        for (int i = 0; i < kHPasses; ++i) {
            const int r = hr0 + kHRowsPerPass * i;
            const int rr = r < n ? r : 0;
            const int slot = shared ? p.T * kTopK + start + rr : p.perm[start + rr];
            hsrc[i] = hg + (size_t)slot * p.Imax + hp * Op::kPerLane;
        }
        constexpr int kWD = kFp8 || kMx ? 4 : 2;  // weight chunks in flight (ring of register buffers)
        typename W::raw_t wr[kWD][kDownTiles][W::kLoads];
        uint4 hv[kPlanes][kHPasses];
        auto load_w = [&](typename W::raw_t (&w)[kDownTiles][W::kLoads], int c) {
#pragma unroll
            for (int t = 0; t < kDownTiles; ++t)
                load_wchunk<WF, kCE>(w[t], src + (size_t)(t * kTile) * rowe, rowe, c,
                                     kMx ? ssrc + (size_t)(t * kTile) * srow : nullptr);
        };
        // (unlike x, every pass is loaded: skipping passes here measured slower - the branches
        // break the load pipelining across chunks)
        auto load_h = [&](int c) {
#pragma unroll
            for (int pl = 0; pl < kPlanes; ++pl)
#pragma unroll
                for (int i = 0; i < kHPasses; ++i) hv[pl][i] = load16(hsrc[i] + pl * p.plane + c * kCE);
        };
        auto store_h = [&](int buf) {
#pragma unroll
            for (int pl = 0; pl < kPlanes; ++pl)
#pragma unroll
                for (int i = 0; i < kHPasses; ++i)
                    *reinterpret_cast<uint4 *>(hs + ((buf * kPlanes + pl) * TG + hr0 + kHRowsPerPass * i) *
                                                        kXRow + hp * 16) = hv[pl][i];
        };
        f32x4_t acc[kDownTiles][NT];
#pragma unroll
        for (int t = 0; t < kDownTiles; ++t)
#pragma unroll
            for (int i = 0; i < NT; ++i) acc[t][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        if (rows_ok) {
#pragma unroll
            for (int d = 0; d < kWD; ++d)
                if (d < nchunks) load_w(wr[d], d);
        }
        load_h(0);
        __syncthreads();  // the previous unit's readers of hs are done
        store_h(0);
        auto step = [&](typename W::raw_t (&wcur)[kDownTiles][W::kLoads], int c) {
            if (c + 1 < nchunks) load_h(c + 1);
            __syncthreads();  // h chunk c is staged; chunk c - 1's readers are done
            if (rows_ok) {
#pragma unroll
                for (int t = 0; t < kDownTiles; ++t) stage_w<WF>(stage + t * kWStage, wcur[t], lane);
                if (c + kWD < nchunks) load_w(wcur, c + kWD);
            }
#pragma unroll
            for (int s = 0; s < kSteps && rows_ok; ++s) {
                uint4 a[kDownTiles];
#pragma unroll
                for (int t = 0; t < kDownTiles; ++t)
                    a[t] = w_operand<kMx ? 1 : kFp8 ? 2 : 0>(stage + t * kWStage, s, col, q);
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    if (tt >= nt_used) continue;  // uniform
#pragma unroll
                    for (int pl = 0; pl < kPlanes; ++pl) {
                        const uint4 b = lds_read16(hs + (((c & 1) * kPlanes + pl) * TG + tt * kTile + col) *
                                                            kXRow + (4 * s + q) * 16);
#pragma unroll
                        for (int t = 0; t < kDownTiles; ++t) Op::mma(acc[t][tt], a[t], b);
                    }
                }
            }
            if (c + 1 < nchunks) store_h((c + 1) & 1);
        };
        for (int c = 0; c < nchunks; c += kWD) {
#pragma unroll
            for (int d = 0; d < kWD; ++d)
                if (c + d < nchunks) step(wr[d], c + d);  // uniform
        }

        if constexpr (WF::kScaled) {  // the output rows' dequantization scales
            if (rows_ok) {
                const float *sc = (shared ? p.sdn_scale : p.dn_scale + (size_t)e * p.H) + wrow + 4 * q;
#pragma unroll
                for (int t = 0; t < kDownTiles; ++t)
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) scale_rows(acc[t][tt], sc + t * kTile);
            }
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int cc = tt * kTile + col;
            if (cc >= n || !rows_ok) continue;
            const int slot = shared ? p.T * kTopK + start + cc : p.perm[start + cc];
            const float wt = shared ? p.g[start + cc] : p.w[slot];
            // lane holds rows 4q + r of each of the wave's 16-row tiles for its token column
#pragma unroll
            for (int t = 0; t < kDownTiles; ++t)
                *reinterpret_cast<float4 *>(p.ybuf + (size_t)slot * p.H + rc * kRowsPerUnit +
                                            (wave * kDownTiles + t) * kTile + 4 * q) =
                    make_float4(wt * acc[t][tt][0], wt * acc[t][tt][1], wt * acc[t][tt][2],
                                wt * acc[t][tt][3]);
        }
    }
}

// gateup_big_kernel (bf16, large T) - the same unit arithmetic as gateup_wide_kernel with the
// operand traffic cut for the matrix-core-bound regime. Unit = (expert group of <= 64 tokens,
// kBigRows * waves intermediate rows); wave w owns rows i0 .. i0 + kBigRows of BOTH the gate and
// the up matrix (kBigRows / 16 tiles each) against the group's four 16-token tiles, so h is formed
// in registers. Weight rows are read in whole 128-byte cache lines (8 rows x 128 bytes per load;
// an expert's other groups find them in the caches) into a ring of two half chunks of registers
// and staged per half chunk in the wave's own LDS area, from which each operand fragment feeds
// four token tiles; the group's x chunk is staged in LDS per 256-byte K chunk (double-buffered)
// and each of its fragments feeds every weight tile of the wave.
constexpr int kBigWaves = 4;
constexpr int kXcds = 8;      // accelerator complex dies of the chip, each with its own L2
constexpr int kBigThreads = kBigWaves * kWave;
constexpr int kBigRows = 32;  // intermediate rows per wave (two 16-row tiles of gate and of up)
constexpr int kBigTile = kTile * 128;  // LDS of one staged 16-row x 128-byte weight tile

template <int NT, bool kFp8>
__global__ __launch_bounds__(kBigThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gateup_big_kernel(GateUpParams p) {
    using Op = OpBF16;
    using elem_t = uint16_t;
    using wt_t = typename WeightFmt<Op, kFp8>::wt_t;  // bf16, or one-byte E4M3 codes
    constexpr int TG = NT * kTile;
    constexpr int kCE = kWPieces * Op::kPerLane;          // elements per chunk (128)
    constexpr int kRT = 2 * kBigRows / kTile;             // weight tiles per wave (gate, up)
    constexpr int kSW = kBigWaves * kBigRows;             // intermediate rows per unit
    constexpr int kXPasses = TG * kWPieces / kBigThreads;
    constexpr int kXRowsPerPass = kBigThreads / kWPieces;
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *xs = smem;  // [2][TG][kXRow]

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, q = lane >> 4;
    const int drow = lane >> 3, dpiece = lane & 7;  // weight loader: 8 rows x 128 B per load
    unsigned char *wst = smem + 2 * TG * kXRow + wave * kRT * kBigTile;  // the wave's weight tiles
    const int ngroups = p.num_groups[0];
    const int nunits = ngroups * p.S;
    const int nchunks = p.H / kCE;
    const elem_t *x = reinterpret_cast<const elem_t *>(p.x);
    const int xp = tid & 15, xr0 = tid >> 4;  // x loader: piece xp of rows xr0 + 16 i
    // XCD-aware schedule: units are numbered slice-major (u = j * groups + g), so the groups of
    // one expert that use the same weight slice are neighbours; blocks b, b + 8, ... share an XCD
    // (and its L2) and together take one contiguous eighth of the units, so those neighbours run
    // side by side on one XCD and read the slice from its L2 after the first miss.
    const bool xmap = gridDim.x % kXcds == 0;
    const int xcd = blockIdx.x % kXcds;
    const int per = xmap ? (nunits + kXcds - 1) / kXcds : nunits;
    const int u_end = xmap ? min(nunits, (xcd + 1) * per) : nunits;
    const int u_step = xmap ? gridDim.x / kXcds : gridDim.x;

    for (int u = xmap ? xcd * per + blockIdx.x / kXcds : blockIdx.x; u < u_end; u += u_step) {
        const int j = u / ngroups, gi = u - j * ngroups;
        const int4 grp = p.groups[gi];
        const int e = grp.x, start = grp.y, n = grp.z;
        const bool shared = e == p.E;
        const int Ie = shared ? p.Is : p.I;
        if (j * kSW >= Ie) continue;  // uniform over the block
        const int nt_used = (n + kTile - 1) / kTile;
        const int i0 = j * kSW + wave * kBigRows;
        const bool rows_ok = i0 < Ie;  // uniform over the wave (Ie is a multiple of 32)
        const wt_t *gu = reinterpret_cast<const wt_t *>(shared ? p.sgu : p.gate_up) +
                         (shared ? 0 : (size_t)e * 2 * Ie * p.H);
        // tile t: gate rows (t < kRT/2) or up rows i0 + 16 (t % (kRT/2)) .. + 16; the loader lane
        // takes row drow (+ 8) and 16-byte piece dpiece of each 128-byte line: of a half chunk
        // (bf16), of a whole chunk (FP8 codes, 16 per lane)
        constexpr int kLaneElems = kFp8 ? 16 : Op::kPerLane;
        const wt_t *arow[kRT];
#pragma unroll
        for (int t = 0; t < kRT; ++t) {
            const int row = (t < kRT / 2 ? 0 : Ie) + i0 + kTile * (t % (kRT / 2)) + drow;
            arow[t] = gu + (size_t)(rows_ok ? row : 0) * p.H + dpiece * kLaneElems;
        }
        const elem_t *xsrc[kXPasses];
#pragma unroll
        for (int i = 0; i < kXPasses; ++i) {
            const int r = xr0 + kXRowsPerPass * i;
            const int rr = r < n ? r : 0;  // rows >= n repeat row 0 (their columns are dropped)
            const int tok = shared ? start + rr : (p.perm[start + rr] >> 3);
            xsrc[i] = x + (size_t)tok * p.H + xp * Op::kPerLane;
        }
        uint4 xv[kXPasses];
        auto load_x = [&](int c) {
#pragma unroll
            for (int i = 0; i < kXPasses; ++i)
                if (kXRowsPerPass * i < n) xv[i] = load16(xsrc[i] + c * kCE);
        };
        auto store_x = [&](int buf) {
#pragma unroll
            for (int i = 0; i < kXPasses; ++i)
                if (kXRowsPerPass * i < n)
                    *reinterpret_cast<uint4 *>(xs + (buf * TG + xr0 + kXRowsPerPass * i) * kXRow +
                                               xp * 16) = xv[i];
        };
        // weight ring (two loads of 8 rows x 128 contiguous bytes per tile: whole cache lines).
        // bf16: rA / rB hold the first / second half of a chunk's rows, refilled with the same
        // half of the next chunk as soon as it is staged. FP8: rA / rB hold whole chunks (even /
        // odd), refilled two chunks later once both halves are staged.
        uint4 rA[kRT][2], rB[kRT][2];
        auto load_a = [&](uint4 (&r)[kRT][2], int hh, int c) {
            if (!rows_ok || c >= nchunks) return;  // uniform
#pragma unroll
            for (int t = 0; t < kRT; ++t)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    r[t][i] = load16(arow[t] + (size_t)(8 * i) * p.H + c * kCE + (kFp8 ? 0 : hh * (kCE / 2)));
        };
        f32x4_t acc[kRT][NT];
#pragma unroll
        for (int t = 0; t < kRT; ++t)
#pragma unroll
            for (int i = 0; i < NT; ++i) acc[t][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        load_a(rA, 0, 0);
        load_a(rB, 1, kFp8 ? 1 : 0);
        load_x(0);
        __syncthreads();  // the previous unit's readers of xs are done
        store_x(0);
        // one half chunk (two k steps) of the wave's tiles: stage the 16 rows x 128 bytes of each
        // tile in the wave's LDS area (row rr, piece pc at rr * 128 + ((pc ^ (rr >> 1)) & 7) * 16:
        // the 16 rows of an operand read fall on 16 distinct 16-byte bank groups), refill the ring,
        // then the two steps' operands in matrix-core order
        auto half = [&](uint4 (&r)[kRT][2], int hh, int c, const unsigned char *xb) {
            // (no operand guard before these FP8 conversions: any wait-state barrier here, even
            // the bare s_nop sequence, makes the compiler spill 176 bytes per lane and doubles the
            // kernel's time at T = 8192; the conversions' bits are pinned instead by the bitwise
            // test against a bf16 context holding the decoded weights, which runs this kernel)
            if (rows_ok) {
#pragma unroll
                for (int t = 0; t < kRT; ++t)
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int rr = 8 * i + drow;
                        unsigned char *row = wst + t * kBigTile + rr * 128;
                        if constexpr (kFp8) {
                            // lanes holding codes of this half widen their 16 codes to two
                            // 16-byte bf16 pieces (exact)
                            if ((dpiece >> 2) == hh) {
                                const int pc = 2 * (dpiece & 3);
                                *reinterpret_cast<uint4 *>(row + ((pc ^ ((rr >> 1) & 7)) * 16)) =
                                    e4m3x8_to_bf16x8(r[t][i].x, r[t][i].y);
                                *reinterpret_cast<uint4 *>(row + (((pc + 1) ^ ((rr >> 1) & 7)) * 16)) =
                                    e4m3x8_to_bf16x8(r[t][i].z, r[t][i].w);
                            }
                        } else {
                            *reinterpret_cast<uint4 *>(row + ((dpiece ^ ((rr >> 1) & 7)) * 16)) = r[t][i];
                        }
                    }
            }
            if constexpr (kFp8) {
                if (hh == 1) load_a(r, 0, c + 2);
            } else {
                load_a(r, hh, c + 1);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int s2 = 2 * hh + s;  // step within the chunk
                uint4 b[NT];
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
                    if (tt < nt_used)  // uniform
                        b[tt] = lds_read16(xb + (tt * kTile + col) * kXRow + (4 * s2 + q) * 16);
                if (rows_ok) {
                    uint4 a[kRT];
#pragma unroll
                    for (int t = 0; t < kRT; ++t)
                        a[t] = lds_read16(wst + t * kBigTile + col * 128 + (((4 * s + q) ^ ((col >> 1) & 7)) * 16));
#pragma unroll
                    for (int t = 0; t < kRT; ++t)
#pragma unroll
                        for (int tt = 0; tt < NT; ++tt)
                            if (tt < nt_used) Op::mma(acc[t][tt], a[t], b[tt]);
                }
            }
        };
        auto chunk = [&](uint4 (&r0)[kRT][2], uint4 (&r1)[kRT][2], int c) {
            if (c + 1 < nchunks) load_x(c + 1);
            __syncthreads();  // x chunk c is staged; chunk c - 1's readers are done
            const unsigned char *xb = xs + (c & 1) * TG * kXRow;
            half(r0, 0, c, xb);
            half(r1, 1, c, xb);
            if (c + 1 < nchunks) store_x((c + 1) & 1);
        };
        if constexpr (kFp8) {
            for (int c = 0; c < nchunks; c += 2) {
                chunk(rA, rA, c);
                if (c + 1 < nchunks) chunk(rB, rB, c + 1);
            }
        } else {
            for (int c = 0; c < nchunks; ++c) chunk(rA, rB, c);
        }
        if (!rows_ok) continue;
        if constexpr (kFp8) {  // the rows' dequantization scales (gate rows, then up rows)
            const float *sc = shared ? p.sgu_scale : p.gu_scale + (size_t)e * 2 * Ie;
#pragma unroll
            for (int t = 0; t < kRT; ++t)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
                    scale_rows(acc[t][tt], sc + (t < kRT / 2 ? 0 : Ie) + i0 + kTile * (t % (kRT / 2)) + 4 * q);
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int cc = tt * kTile + col;  // group row of this lane's token column
            if (cc >= n) continue;
            const int slot = shared ? p.T * kTopK + start + cc : p.perm[start + cc];
#pragma unroll
            for (int g2 = 0; g2 < kRT / 2; ++g2) {
                const f32x4_t ga = acc[g2][tt], up = acc[kRT / 2 + g2][tt];
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
                uint16_t *hp = reinterpret_cast<uint16_t *>(p.h);
                *reinterpret_cast<uint2 *>(hp + off) = uint2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
                *reinterpret_cast<uint2 *>(hp + p.plane + off) =
                    uint2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
            }
        }
    }
}

// down_big_kernel (bf16, large T) - the down product of the 64-token groups with the layout of
// gateup_big: unit = (expert group, kDBRows = 512 rows of y), so a group's h is staged 4 times
// per token instead of 8; wave w owns rows w * 64 .. + 64 of the unit (four 16-row tiles) against
// the group's four 16-token tiles. Weight rows are read in whole 128-byte lines (8 rows x 128 B
// per load; an expert's other groups find them in the caches) into a ring of two half chunks of
// registers and staged per half chunk in the wave's own LDS area; h (hi and lo planes) is staged
// per 256-byte chunk as in down_wide_kernel. Per
// output element the steps, planes and their order are those of down_wide_kernel (bitwise equal).
constexpr int kDBWaves = 8;
constexpr int kDBThreads = kDBWaves * kWave;
constexpr int kDBTiles = 4;                              // 16-row tiles per wave
constexpr int kDBRows = kDBWaves * kDBTiles * kTile;     // rows of y per unit (512)

template <int NT, bool kFp8>
__global__ __launch_bounds__(kDBThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void down_big_kernel(DownParams p) {
    using Op = OpBF16;
    using elem_t = uint16_t;
    using wt_t = typename WeightFmt<Op, kFp8>::wt_t;  // bf16, or one-byte E4M3 codes
    constexpr int TG = NT * kTile;
    constexpr int kCE = kWPieces * Op::kPerLane;     // 128 elements per chunk
    constexpr int kPlanes = 2;                       // h as hi + lo bf16
    constexpr int kHPasses = TG * kWPieces / kDBThreads;
    constexpr int kHRowsPerPass = kDBThreads / kWPieces;
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *hs = smem;                        // [2][planes][TG][kXRow]
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, q = lane >> 4;
    const int drow = lane >> 3, dpiece = lane & 7;   // weight loader: 8 rows x 128 B per load
    unsigned char *wst = smem + 2 * kPlanes * TG * kXRow + wave * kDBTiles * kBigTile;
    const int n_rc = p.H / kDBRows;
    const int ngroups = p.num_groups[0];
    const int nunits = ngroups * n_rc;
    const elem_t *hg = reinterpret_cast<const elem_t *>(p.h);
    const int hp = tid & 15, hr0 = tid >> 4;         // h loader: piece hp of rows hr0 + 32 i
    // XCD-aware schedule (as in gateup_big_kernel): units numbered row-block-major
    // (u = rc * groups + g), so an expert's groups, which read the same down rows, are neighbours;
    // blocks b, b + 8, ... share an XCD and take one contiguous eighth of the units
    const bool xmap = gridDim.x % kXcds == 0;
    const int xcd = blockIdx.x % kXcds;
    const int per = xmap ? (nunits + kXcds - 1) / kXcds : nunits;
    const int u_end = xmap ? min(nunits, (xcd + 1) * per) : nunits;
    const int u_step = xmap ? gridDim.x / kXcds : gridDim.x;

    for (int u = xmap ? xcd * per + blockIdx.x / kXcds : blockIdx.x; u < u_end; u += u_step) {
        const int rc = u / ngroups, gi = u - rc * ngroups;
        const int4 grp = p.groups[gi];
        const int e = grp.x, start = grp.y, n = grp.z;
        const bool shared = e == p.E;
        const int Ie = shared ? p.Is : p.I;
        const int nchunks = Ie / kCE;
        const int nt_used = (n + kTile - 1) / kTile;
        const wt_t *dn = reinterpret_cast<const wt_t *>(shared ? p.sdn : p.down) +
                         (shared ? 0 : (size_t)e * p.H * Ie);
        const int wrow = rc * kDBRows + wave * kDBTiles * kTile;  // the wave's first row
        const wt_t *src = dn + (size_t)(wrow + drow) * Ie + dpiece * (kFp8 ? 16 : Op::kPerLane);
        uint32_t hoff[kHPasses];  // element offsets of the h rows this thread stages
#pragma unroll
        for (int i = 0; i < kHPasses; ++i) {
            const int r = hr0 + kHRowsPerPass * i;
            const int rr = r < n ? r : 0;
            const int slot = shared ? p.T * kTopK + start + rr : p.perm[start + rr];
            hoff[i] = (uint32_t)slot * (uint32_t)p.Imax + hp * Op::kPerLane;
        }
        uint4 hv[kPlanes][kHPasses];
        auto load_h = [&](int c) {
#pragma unroll
            for (int pl = 0; pl < kPlanes; ++pl)
#pragma unroll
                for (int i = 0; i < kHPasses; ++i) hv[pl][i] = load16(hg + pl * p.plane + hoff[i] + c * kCE);
        };
        auto store_h = [&](int buf) {
#pragma unroll
            for (int pl = 0; pl < kPlanes; ++pl)
#pragma unroll
                for (int i = 0; i < kHPasses; ++i)
                    *reinterpret_cast<uint4 *>(hs + ((buf * kPlanes + pl) * TG + hr0 + kHRowsPerPass * i) *
                                                        kXRow + hp * 16) = hv[pl][i];
        };
        // weight ring (two loads of 8 rows x 128 bytes per tile): bf16 - rA / rB hold the first /
        // second half of a chunk's rows, refilled with the same half of the next chunk as soon as
        // it is staged; FP8 - whole chunks (even / odd), refilled two chunks later
        uint4 rA[kDBTiles][2], rB[kDBTiles][2];
        auto load_w = [&](uint4 (&r)[kDBTiles][2], int hh, int c) {
            if (c >= nchunks) return;  // uniform
#pragma unroll
            for (int t = 0; t < kDBTiles; ++t)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    r[t][i] = load16(src + (size_t)(t * kTile + 8 * i) * Ie + c * kCE + (kFp8 ? 0 : hh * (kCE / 2)));
        };
        f32x4_t acc[kDBTiles][NT];
#pragma unroll
        for (int t = 0; t < kDBTiles; ++t)
#pragma unroll
            for (int i = 0; i < NT; ++i) acc[t][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        load_w(rA, 0, 0);
        load_w(rB, 1, kFp8 ? 1 : 0);
        load_h(0);
        __syncthreads();  // the previous unit's readers of hs are done
        store_h(0);
        auto half = [&](uint4 (&r)[kDBTiles][2], int hh, int c, const unsigned char *hb) {
#pragma unroll
            for (int t = 0; t < kDBTiles; ++t)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int rr = 8 * i + drow;
                    *reinterpret_cast<uint4 *>(wst + t * kBigTile + rr * 128 + ((dpiece ^ ((rr >> 1) & 7)) * 16)) = r[t][i];
                }
            load_w(r, hh, c + 1);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int s2 = 2 * hh + s;  // step within the chunk
                uint4 a[kDBTiles];
#pragma unroll
                for (int t = 0; t < kDBTiles; ++t)
                    a[t] = lds_read16(wst + t * kBigTile + col * 128 + (((4 * s + q) ^ ((col >> 1) & 7)) * 16));
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    if (tt >= nt_used) continue;  // uniform
#pragma unroll
                    for (int pl = 0; pl < kPlanes; ++pl) {
                        const uint4 b = lds_read16(hb + (pl * TG + tt * kTile + col) * kXRow + (4 * s2 + q) * 16);
#pragma unroll
                        for (int t = 0; t < kDBTiles; ++t) Op::mma(acc[t][tt], a[t], b);
                    }
                }
            }
        };
        // FP8: a whole chunk of raw codes (16 rows x 128 bytes per tile) is staged at once, same
        // swizzle, and each operand fragment (8 codes) is widened to bf16 right before its use:
        // step s2, k-group q takes bytes 32 s2 + 8 q .. + 8 of the row
        auto chunk8 = [&](uint4 (&r)[kDBTiles][2], int c) {
            if (c + 1 < nchunks) load_h(c + 1);
            __syncthreads();  // h chunk c is staged; chunk c - 1's readers are done
            const unsigned char *hb = hs + (c & 1) * kPlanes * TG * kXRow;
#pragma unroll
            for (int t = 0; t < kDBTiles; ++t)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int rr = 8 * i + drow;
                    *reinterpret_cast<uint4 *>(wst + t * kBigTile + rr * 128 + ((dpiece ^ ((rr >> 1) & 7)) * 16)) = r[t][i];
                }
            load_w(r, 0, c + 2);
#pragma unroll
            for (int s2 = 0; s2 < kWPieces / 4; ++s2) {
                const int po = col * 128 + (((2 * s2 + (q >> 1)) ^ ((col >> 1) & 7)) * 16) + (q & 1) * 8;
                uint4 a[kDBTiles];
                mfma_operand_guard();  // these conversions write operand registers of the last step
#pragma unroll
                for (int t = 0; t < kDBTiles; ++t) {
                    const uint2 cd = *reinterpret_cast<const uint2 *>(wst + t * kBigTile + po);
                    a[t] = e4m3x8_to_bf16x8(cd.x, cd.y);
                }
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    if (tt >= nt_used) continue;  // uniform
#pragma unroll
                    for (int pl = 0; pl < kPlanes; ++pl) {
                        const uint4 b = lds_read16(hb + (pl * TG + tt * kTile + col) * kXRow + (4 * s2 + q) * 16);
#pragma unroll
                        for (int t = 0; t < kDBTiles; ++t) Op::mma(acc[t][tt], a[t], b);
                    }
                }
            }
            if (c + 1 < nchunks) store_h((c + 1) & 1);
        };
        if constexpr (kFp8) {
            for (int c = 0; c < nchunks; c += 2) {
                chunk8(rA, c);
                if (c + 1 < nchunks) chunk8(rB, c + 1);
            }
        } else {
            for (int c = 0; c < nchunks; ++c) {
                if (c + 1 < nchunks) load_h(c + 1);
                __syncthreads();  // h chunk c is staged; chunk c - 1's readers are done
                const unsigned char *hb = hs + (c & 1) * kPlanes * TG * kXRow;
                half(rA, 0, c, hb);
                half(rB, 1, c, hb);
                if (c + 1 < nchunks) store_h((c + 1) & 1);
            }
        }
        if constexpr (kFp8) {  // the output rows' dequantization scales
            const float *sc = (shared ? p.sdn_scale : p.dn_scale + (size_t)e * p.H) + wrow + 4 * q;
#pragma unroll
            for (int t = 0; t < kDBTiles; ++t)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) scale_rows(acc[t][tt], sc + t * kTile);
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int cc = tt * kTile + col;
            if (cc >= n) continue;
            const int slot = shared ? p.T * kTopK + start + cc : p.perm[start + cc];
            const float wt = shared ? p.g[start + cc] : p.w[slot];
            // lane holds rows 4q + r of each of the wave's 16-row tiles for its token column
#pragma unroll
            for (int t = 0; t < kDBTiles; ++t)
                *reinterpret_cast<float4 *>(p.ybuf + (size_t)slot * p.H + wrow + t * kTile + 4 * q) =
                    make_float4(wt * acc[t][tt][0], wt * acc[t][tt][1], wt * acc[t][tt][2],
                                wt * acc[t][tt][3]);
        }
    }
}

constexpr int kWideNT = 4;  // 64-token groups

size_t gateup_wide_lds() { return 2 * kWideNT * kTile * kXRow + kWWaves * kWStage; }
size_t down_wide_lds(int dtype) {
    return 2 * (dtype == 1 ? 2 : 1) * kWideNT * kTile * kXRow + kWWaves * kDownTiles * kWStage;
}
int wide_rows_per_down_unit() { return kWWaves * kDownTiles * kTile; }
int wide_rows_per_gateup_unit() { return kWWaves / 2 * kTile; }
int wide_group_tokens() { return kWideNT * kTile; }
int big_rows_per_gateup_unit() { return kBigWaves * kBigRows; }
size_t gateup_big_lds() {
    return 2 * kWideNT * kTile * kXRow + kBigWaves * (2 * kBigRows / kTile) * kBigTile;
}

// dtype: 1 bf16, 2 bf16 activations with FP8 E4M3 weights
hipError_t launch_gateup_big(const GateUpParams &p, int dtype, int grid, hipStream_t s) {
    if (dtype == 2) launch_k(gateup_big_kernel<kWideNT, true>, grid, kBigThreads, gateup_big_lds(), s, p);
    else launch_k(gateup_big_kernel<kWideNT, false>, grid, kBigThreads, gateup_big_lds(), s, p);
    return hipGetLastError();
}

size_t down_big_lds() { return 2 * 2 * kWideNT * kTile * kXRow + kDBWaves * kDBTiles * kBigTile; }
int big_rows_per_down_unit() { return kDBRows; }

// dtype: 1 bf16, 2 bf16 activations with FP8 E4M3 weights
hipError_t launch_down_big(const DownParams &p, int dtype, int grid, hipStream_t s) {
    if (p.NG != kWideNT * kTile || p.H % kDBRows) return hipErrorInvalidValue;  // a caller bug
    if (dtype == 2) launch_k(down_big_kernel<kWideNT, true>, grid, kDBThreads, down_big_lds(), s, p);
    else launch_k(down_big_kernel<kWideNT, false>, grid, kDBThreads, down_big_lds(), s, p);
    return hipGetLastError();
}

hipError_t prepare_wide_kernels() {
    hipError_t err;
    const void *big[] = {reinterpret_cast<const void *>(&down_big_kernel<kWideNT, false>),
                         reinterpret_cast<const void *>(&down_big_kernel<kWideNT, true>),
                         reinterpret_cast<const void *>(&gateup_big_kernel<kWideNT, false>),
                         reinterpret_cast<const void *>(&gateup_big_kernel<kWideNT, true>)};
    const size_t big_lds[] = {down_big_lds(), down_big_lds(), gateup_big_lds(), gateup_big_lds()};
    for (int i = 0; i < 4; ++i)
        if ((err = hipFuncSetAttribute(big[i], hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)big_lds[i])) != hipSuccess)
            return err;
    const void *gk[] = {reinterpret_cast<const void *>(&gateup_wide_kernel<OpBF16, kWideNT, false>),
                        reinterpret_cast<const void *>(&gateup_wide_kernel<OpF32, kWideNT, false>),
                        reinterpret_cast<const void *>(&gateup_wide_kernel<OpBF16, kWideNT, true>),
                        reinterpret_cast<const void *>(&gateup_wide_kernel<OpBF16, kWideNT, false, true>)};
    for (const void *k : gk)
        if ((err = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)gateup_wide_lds())) != hipSuccess)
            return err;
    const void *dk16[] = {reinterpret_cast<const void *>(&down_wide_kernel<OpBF16, kWideNT, false>),
                          reinterpret_cast<const void *>(&down_wide_kernel<OpBF16, kWideNT, true>),
                          reinterpret_cast<const void *>(&down_wide_kernel<OpBF16, kWideNT, false, true>)};
    for (const void *k : dk16)
        if ((err = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)down_wide_lds(1))) != hipSuccess)
            return err;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&down_wide_kernel<OpF32, kWideNT, false>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)down_wide_lds(0));
}

// dtype: 0 fp32, 1 bf16, 2 bf16 activations with FP8 E4M3 weights, 3 with MXFP4 weights
hipError_t launch_gateup_wide(const GateUpParams &p, int dtype, int grid, hipStream_t s) {
    if (dtype == 3) launch_k(gateup_wide_kernel<OpBF16, kWideNT, false, true>, grid, kWThreads, gateup_wide_lds(), s, p);
    else if (dtype == 2) launch_k(gateup_wide_kernel<OpBF16, kWideNT, true>, grid, kWThreads, gateup_wide_lds(), s, p);
    else if (dtype == 1) launch_k(gateup_wide_kernel<OpBF16, kWideNT, false>, grid, kWThreads, gateup_wide_lds(), s, p);
    else launch_k(gateup_wide_kernel<OpF32, kWideNT, false>, grid, kWThreads, gateup_wide_lds(), s, p);
    return hipGetLastError();
}

hipError_t launch_down_wide(const DownParams &p, int dtype, int grid, hipStream_t s) {
    if (dtype == 3) launch_k(down_wide_kernel<OpBF16, kWideNT, false, true>, grid, kWThreads, down_wide_lds(1), s, p);
    else if (dtype == 2) launch_k(down_wide_kernel<OpBF16, kWideNT, true>, grid, kWThreads, down_wide_lds(1), s, p);
    else if (dtype == 1) launch_k(down_wide_kernel<OpBF16, kWideNT, false>, grid, kWThreads, down_wide_lds(1), s, p);
    else launch_k(down_wide_kernel<OpF32, kWideNT, false>, grid, kWThreads, down_wide_lds(0), s, p);
    return hipGetLastError();
}

}  // namespace moe
