// gateup_down.hip - the expert stage for decode and verify rounds (T <= 256) as two kernels.
//
// Decode rounds touch each selected expert with one or two tokens, so the stage is a stream of
// expert weights read once from HBM (the expert block dominates a MoE model's bytes and decode is
// bandwidth-bound: "RELEASE_NOTES_0.9.0" of the 16 GB ninfer fork, the expert-placement
// paragraphs). It is split so that each weight matrix is streamed in the order that suits it:
//
// gateup_kernel - one block per (expert group of <= 8 tokens, 32-row slice of the intermediate
//   dimension): the group's x rows are staged in LDS; two waves compute the 16x16 gate tiles and
//   two the 16x16 up tiles of the slice with MFMA, each streaming its 16 weight rows from HBM in
//   long contiguous runs and reordering them through LDS into operand order;
//   h = silu(gate) * up is written to the workspace, for bf16 as
//   two bf16 planes hi = bf16(h) and lo = bf16(h - hi) (so that the bf16 down product keeps ~16
//   mantissa bits of h), for fp32 as is. Row slot of a (token, rank) pair: t*8 + k; of the
//   shared expert for token t: T*8 + t.
//
// down_kernel - one block per (expert group, 64 rows of the output): the block reads that
//   expert's 64 down-weight rows (one contiguous block of 64 * I elements) and the group's h rows
//   (staged once in LDS) and writes w * (Wd h) for each of the group's (token, rank) pairs into
//   that pair's row of a [slots][H] buffer (w = the pair's routing weight, or the shared gate).
//   Every element of the buffer has exactly one writer. The last unit to finish a 64-row block
//   (an arrival count per row block) then sums each token's eight ranks in rank order plus its
//   shared slot into y. No floating-point atomics, and a token's bits do not depend on the batch
//   it came in.
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kThreads = 256;

__device__ __forceinline__ uint4 lds_load16(const void *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

// Unit = (expert group, 32-row slice j of the intermediate dimension). Waves 0, 1 own the gate
// rows j*32 + 16w .. +16, waves 2, 3 the matching up rows. Each wave streams its 16 weight rows in
// chunks of 16 x 256 bytes: one load instruction reads 256 contiguous bytes of each of 4 rows (long
// runs per row are what keeps HBM near its streaming rate; the matrix-core operand order would
// read only 64 bytes per row per instruction). The chunk is written to the wave's own LDS buffer
// with an XOR swizzle of the 16-byte pieces (row r, piece p at r*256 + ((p ^ r) & 15)*16), so that
// the operand reads - lane (row i, k-group q) takes piece 4s + q of row i for step s - hit 16
// distinct bank groups. The up waves hand their 16x16 tiles to the gate waves through LDS, which
// write h = silu(gate) * up.
// MXFP4 weights (kMx): a ring slot is a pair of chunks, 16 rows x 128 bytes of packed codes read
// as 8 rows x 128 bytes per instruction like FP8; each lane's 16 bytes are one scale block of 32
// weights, widened with its E8M0 scale into four bf16 pieces of one of the two chunks. The two
// chunks go to the wave's two LDS buffers and feed the matrix instructions in chunk order, so
// every accumulator sees the k order of the other formats.
template <class Op, bool kFp8, bool kMx = false>
__global__ __launch_bounds__(kThreads) void gateup_kernel(GateUpParams p) {
    using elem_t = typename Op::elem_t;
    using WF = WeightFmt<Op, kFp8>;
    using wt_t = typename WF::wt_t;
    constexpr int kSW = 32;                           // intermediate rows per unit
    constexpr int kPieces = 16;                       // 16-byte pieces per row per chunk
    constexpr int kChunkElems = kPieces * Op::kPerLane;
    constexpr int kStepsPerChunk = kPieces / 4;       // 4 k-groups of one piece per step
    // chunks per load batch (two batches in flight); FP8 codes are half the bytes, so twice the
    // chunks fill the same registers
    // (MXFP4: chunk pairs per batch, a quarter of the bf16 bytes per chunk)
    constexpr int kDepth = kFp8 || kMx ? 4 : 2;
    constexpr bool k8 = kFp8 || kMx;                  // one-byte storage: 8 rows x 128 B loads
    constexpr int kStageBufs = 2;                     // LDS chunk buffers per wave
    constexpr int kStage = kTile * kPieces * 16;      // 4 KB of LDS per chunk per wave

    extern __shared__ __align__(16) unsigned char smem[];
    elem_t *xs = reinterpret_cast<elem_t *>(smem);
    unsigned char *stage_all = smem + (size_t)p.NG * p.x_stride * sizeof(elem_t);
    float *xchg = reinterpret_cast<float *>(stage_all + 4 * kStageBufs * kStage);  // [2][16][16] up tiles

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, q = lane >> 4;
    unsigned char *stage = stage_all + wave * kStageBufs * kStage;
    const int nunits = p.num_groups[0] * p.S;
    const int chunks_per_row = p.H / Op::kPerLane;
    const int nchunks = p.H / kChunkElems;
    const int nslots = kMx ? nchunks / 2 : nchunks;  // ring slots along K (H % 256 == 0 for MXFP4)
    const elem_t *x = reinterpret_cast<const elem_t *>(p.x);
    // loader lane -> (row, piece) of a chunk: 4 instructions of 4 rows x 256 contiguous bytes;
    // FP8 codes (128 bytes per row and chunk): 2 instructions of 8 rows x 128 bytes, 16 codes a lane
    const int lrow = lane >> 4, lpiece = lane & 15;
    const int lrow8 = lane >> 3, lpiece8 = lane & 7;
    constexpr int kLoads = k8 ? 2 : 4;  // load instructions per ring slot
    const int mx_row = p.H / 2, mx_srow = p.H / 32;  // MXFP4 bytes per row: codes, scales

    for (int u = blockIdx.x; u < nunits; u += gridDim.x) {
        const int gi = u / p.S, j = u - (u / p.S) * p.S;
        const int4 grp = p.groups[gi];
        const int e = grp.x, start = grp.y, n = grp.z;
        const bool shared = e == p.E;
        const int Ie = shared ? p.Is : p.I;
        if (j * kSW >= Ie) continue;  // uniform over the block

        const wt_t *gu = reinterpret_cast<const wt_t *>(shared ? p.sgu : p.gate_up) +
                         (shared ? 0 : (size_t)e * 2 * Ie * p.H);
        const int wrow0 = (wave < 2 ? 0 : Ie) + j * kSW + (wave & 1) * kTile;  // first weight row
        const wt_t *src = kFp8 ? gu + (size_t)(wrow0 + lrow8) * p.H + lpiece8 * 16
                               : gu + (size_t)(wrow0 + lrow) * p.H + lpiece * Op::kPerLane;
        // MXFP4: the lane's codes (16 bytes of a 128-byte pair of chunks) and their scale byte
        const unsigned char *msrc =
            reinterpret_cast<const unsigned char *>(shared ? p.sgu : p.gate_up) +
            (shared ? 0 : (size_t)e * 2 * Ie * mx_row) + (size_t)(wrow0 + lrow8) * mx_row + lpiece8 * 16;
        const uint8_t *ssrc = kMx ? (shared ? p.sgu_mx : p.gu_mx + (size_t)e * 2 * Ie * mx_srow) +
                                        (size_t)(wrow0 + lrow8) * mx_srow + lpiece8
                                  : nullptr;
        const bool col_ok = col < n;
        const int crow = col_ok ? col : 0;  // columns >= n repeat column 0 (dropped)
        const elem_t *xrow = xs + crow * p.x_stride + q * Op::kPerLane;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};

        using raw_t = typename std::conditional<k8, uint4, typename WF::raw_t>::type;
        raw_t rA[kDepth][kLoads], rB[kDepth][kLoads];
        uint32_t sA[kDepth][kLoads], sB[kDepth][kLoads];  // MXFP4 scale bytes (else unused)
        auto load = [&](raw_t(&r)[kDepth][kLoads], uint32_t(&sc)[kDepth][kLoads], int c0) {
#pragma unroll
            for (int d = 0; d < kDepth; ++d)
#pragma unroll
                for (int a = 0; a < kLoads; ++a) {
                    const int c = min(c0 + d, nslots - 1);  // past the end: re-read, unused
                    if constexpr (kMx) {
                        r[d][a] = load16_stream(msrc + (size_t)(8 * a) * mx_row + c * 128);
                        sc[d][a] = ssrc[(size_t)(8 * a) * mx_srow + c * 8];
                    } else if constexpr (kFp8) {
                        r[d][a] = load16_stream(src + (size_t)(8 * a) * p.H + c * kChunkElems);
                    } else {
                        r[d][a] = WF::load_raw(src + (size_t)(4 * a) * p.H + c * kChunkElems);
                    }
                }
        };
        auto mma_chunk = [&](const unsigned char *buf, int c, int mb) {  // mb: MXFP4 buffer
#pragma unroll
            for (int s2 = 0; s2 < kStepsPerChunk; ++s2) {
                const int pc = kMx ? mx_piece_pos(4 * s2 + q, mb) : kFp8 ? fp8_piece_pos(4 * s2 + q)
                                                                       : 4 * s2 + q;
                const uint4 av = lds_load16(buf + col * 256 + ((pc ^ col) & 15) * 16);
                const uint4 xb = lds_load16(xrow + c * kChunkElems + 4 * s2 * Op::kPerLane);
                Op::mma(acc, av, xb);
            }
        };
        auto consume = [&](const raw_t(&r)[kDepth][kLoads], const uint32_t(&sc)[kDepth][kLoads],
                           int c0) {
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                if (c0 + d >= nslots) break;  // uniform
                if constexpr (kMx) {
                    // lanes 0-3 of a row hold chunk 2(c0 + d), lanes 4-7 the next one; each lane's
                    // 32 weights are four consecutive pieces of its chunk
                    unsigned char *buf = stage + (lpiece8 >> 2) * kStage;
                    const int pb = 4 * (lpiece8 & 3);
                    mfma_operand_guard();
#pragma unroll
                    for (int a = 0; a < kLoads; ++a) {
                        const int rr = 8 * a + lrow8;
                        const float sf = e8m0_to_f32(sc[d][a]);
                        const uint32_t w4[4] = {r[d][a].x, r[d][a].y, r[d][a].z, r[d][a].w};
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            *reinterpret_cast<uint4 *>(
                                buf + rr * 256 + ((mx_piece_pos(pb + k, lpiece8 >> 2) ^ rr) & 15) * 16) =
                                e2m1x8_to_bf16x8(w4[k], sf);
                    }
                    mma_chunk(stage, 2 * (c0 + d), 0);  // a wave's LDS ops stay in order
                    mma_chunk(stage + kStage, 2 * (c0 + d) + 1, 1);
                    continue;
                }
                unsigned char *buf = stage + (d % kStageBufs) * kStage;  // a wave's LDS ops stay in order
                if constexpr (kFp8) mfma_operand_guard();  // the FP8 conversions as the MXFP4 ones
#pragma unroll
                for (int a = 0; a < kLoads; ++a) {
                    if constexpr (kFp8) {  // 16 codes widened to two bf16 pieces (exact)
                        const int rr = 8 * a + lrow8;
                        const int p0 = 2 * lpiece8;
                        *reinterpret_cast<uint4 *>(buf + rr * 256 + ((fp8_piece_pos(p0) ^ rr) & 15) * 16) =
                            e4m3x8_to_bf16x8(r[d][a].x, r[d][a].y);
                        *reinterpret_cast<uint4 *>(buf + rr * 256 + ((fp8_piece_pos(p0 + 1) ^ rr) & 15) * 16) =
                            e4m3x8_to_bf16x8(r[d][a].z, r[d][a].w);
                    } else {
                        const int rr = 4 * a + lrow;
                        *reinterpret_cast<uint4 *>(buf + rr * 256 + ((lpiece ^ rr) & 15) * 16) =
                            WF::to_operand(r[d][a]);
                    }
                }
                mma_chunk(buf, c0 + d, 0);
            }
        };
        // the weight stream does not depend on x: both buffers are requested before staging x
        load(rA, sA, 0);
        if (kDepth < nslots) load(rB, sB, kDepth);
        __syncthreads();  // the previous unit's readers of xs / xchg are done
        for (int idx = tid; idx < n * chunks_per_row; idx += kThreads) {
            const int row = idx / chunks_per_row;
            const int c = idx - row * chunks_per_row;
            const int tok = shared ? start + row : (p.perm[start + row] >> 3);
            *reinterpret_cast<uint4 *>(xs + row * p.x_stride + c * Op::kPerLane) =
                load16(x + (size_t)tok * p.H + c * Op::kPerLane);
        }
        __syncthreads();

        for (int c0 = 0; c0 < nslots; c0 += 2 * kDepth) {
            consume(rA, sA, c0);
            if (c0 + 2 * kDepth < nslots) load(rA, sA, c0 + 2 * kDepth);
            if (c0 + kDepth < nslots) {
                consume(rB, sB, c0 + kDepth);
                if (c0 + 3 * kDepth < nslots) load(rB, sB, c0 + 3 * kDepth);
            }
        }

        if constexpr (WF::kScaled)  // the rows' dequantization scales (gate rows, then up rows)
            scale_rows(acc, (shared ? p.sgu_scale : p.gu_scale + (size_t)e * 2 * Ie) + wrow0 + 4 * q);
        // up waves hand their tiles over; gate waves form h
        if (wave >= 2) {
            *reinterpret_cast<f32x4_t *>(xchg + ((wave - 2) * kTile + col) * kTile + 4 * q) = acc;
        }
        __syncthreads();
        if (wave >= 2 || !col_ok) continue;
        const f32x4_t up = *reinterpret_cast<const f32x4_t *>(xchg + (wave * kTile + col) * kTile + 4 * q);
        const int slot = shared ? p.T * kTopK + start + col : p.perm[start + col];
        const int i0 = j * kSW + wave * kTile;
        // lane holds intermediate rows i0 + 4q + r, r = 0..3, of token column `col`
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[r] = acc[r] / (1.0f + expf(-acc[r])) * up[r];
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

// y rows h0 .. h0 + 64 of every token from the weighted per-slot outputs: the eight ranks in
// rank order, then the shared slot (one float4 of one token per thread and step). A pair whose
// given id lies outside [0, E) was dropped by the bucketing, so its slot holds nothing of this
// call: it adds zero.
__device__ void combine_rows(const DownParams &p, int h0, int tid) {
    const bool has_shared = p.g != nullptr;
    for (int i = tid; i < p.T * 16; i += kThreads) {
        const int t = i >> 4;
        const int h = h0 + (i & 15) * 4;
        auto ld4 = [](const float *a) {
            const uint4 b = ld_dev16(a);
            return make_float4(__uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z),
                               __uint_as_float(b.w));
        };
        float4 v[kTopK + 1];
#pragma unroll
        for (int k = 0; k < kTopK; ++k) {
            const int e = p.ids[t * kTopK + k];
            v[k] = e >= 0 && e < p.E ? ld4(p.ybuf + (size_t)(t * kTopK + k) * p.H + h)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        v[kTopK] = has_shared ? ld4(p.ybuf + (size_t)(p.T * kTopK + t) * p.H + h)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < kTopK; ++k) {
            acc.x += v[k].x; acc.y += v[k].y; acc.z += v[k].z; acc.w += v[k].w;
        }
        if (has_shared) {
            acc.x += v[kTopK].x; acc.y += v[kTopK].y; acc.z += v[kTopK].z; acc.w += v[kTopK].w;
        }
        *reinterpret_cast<float4 *>(p.y + (size_t)t * p.H + h) = acc;
    }
}

// One block per (expert group, 64 rows of y): wave w multiplies rows r0 + 16w .. +16 of the
// expert's down weight (Ie contiguous elements each, so the block reads one contiguous 64-row
// block) by the group's h, staged once per unit in LDS, and writes weight * (Wd h) to the row
// slot of each of the group's (token, rank) pairs. Weight rows stream as in gateup_kernel: each
// load instruction reads 256 contiguous bytes of each of 4 rows, and a per-wave LDS buffer with
// the same XOR swizzle turns 16 x 256-byte chunks into matrix-core operands.
// MXFP4 weights (kMx): ring slots are chunk pairs as in gateup_kernel; the wave's one LDS buffer
// takes the pair's first chunk (written by the lanes that hold it), feeds its matrix
// instructions, then takes the second.
template <class Op, bool kFp8, bool kMx = false>
__global__ __launch_bounds__(kThreads) void down_kernel(DownParams p) {
    using WF = WeightFmt<Op, kFp8>;
    using wt_t = typename WF::wt_t;
    using h_t = typename Op::elem_t;                // h planes share the operand type
    constexpr int kRowsPerUnit = 64;
    constexpr int kPieces = 16;
    constexpr int kChunkElems = kPieces * Op::kPerLane;
    constexpr int kStepsPerChunk = kPieces / 4;
    constexpr int kBatch = 4;                       // chunks loaded together (16 KB per wave)
    constexpr int kStage = kTile * kPieces * 16;    // 4 KB of LDS per wave
    extern __shared__ __align__(16) unsigned char smem[];
    const int hstride = p.Imax + 16 / Op::kElemBytes;  // padded row stride of the h tile
    h_t *hs_hi = reinterpret_cast<h_t *>(smem);                 // [16][hstride]
    h_t *hs_lo = hs_hi + (size_t)p.NG * hstride;                // [NG][hstride], bf16 only
    unsigned char *stage_all = reinterpret_cast<unsigned char *>(
        hs_hi + (size_t)p.NG * hstride * (Op::kElemBytes == 2 ? 2 : 1));
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, q = lane >> 4;
    const int lrow = lane >> 4, lpiece = lane & 15;
    unsigned char *stage = stage_all + wave * kStage;
    const int n_rc = p.H / kRowsPerUnit;
    const int ngroups = p.num_groups[0];
    const int nunits = ngroups * n_rc;
    const h_t *hg = reinterpret_cast<const h_t *>(p.h);
    // With a grid that is a multiple of the row-block count every unit of this block has row
    // block blockIdx.x % n_rc: the block then waits for its stores and arrives once, after its
    // last unit, adding its unit count (one store-acknowledge wait per block, not per unit).
    const bool defer = gridDim.x % n_rc == 0;
    int my_units = 0;

    for (int u = blockIdx.x; u < nunits; u += gridDim.x) {
        const int gi = u / n_rc, rc = u - (u / n_rc) * n_rc;
        const int4 grp = p.groups[gi];
        const int e = grp.x, start = grp.y, n = grp.z;
        const bool shared = e == p.E;
        const int Ie = shared ? p.Is : p.I;
        const int nchunks = Ie / kChunkElems;
        const int nslots = kMx ? nchunks / 2 : nchunks;  // ring slots (MXFP4: chunk pairs)
        const wt_t *dn = reinterpret_cast<const wt_t *>(shared ? p.sdn : p.down) +
                         (shared ? 0 : (size_t)e * p.H * Ie);
        // FP8 codes: 2 loads of 8 rows x 128 bytes per chunk (16 codes a lane) in place of 4 of
        // 4 rows x 128 bytes; MXFP4: the same shape per chunk pair
        const int lrow8 = lane >> 3, lpiece8 = lane & 7;
        constexpr bool k8 = kFp8 || kMx;
        constexpr int kLoads = k8 ? 2 : 4;
        const int wr0 = rc * kRowsPerUnit + wave * kTile;  // the wave's first weight row
        const wt_t *src =
            kFp8 ? dn + (size_t)(wr0 + lrow8) * Ie + lpiece8 * 16
                 : dn + (size_t)(wr0 + lrow) * Ie + lpiece * Op::kPerLane;
        const int mx_row = Ie / 2, mx_srow = Ie / 32;  // MXFP4 bytes per row: codes, scales
        const unsigned char *msrc = reinterpret_cast<const unsigned char *>(shared ? p.sdn : p.down) +
                                    (shared ? 0 : (size_t)e * p.H * mx_row) +
                                    (size_t)(wr0 + lrow8) * mx_row + lpiece8 * 16;
        const uint8_t *ssrc = kMx ? (shared ? p.sdn_mx : p.dn_mx + (size_t)e * p.H * mx_srow) +
                                        (size_t)(wr0 + lrow8) * mx_srow + lpiece8
                                  : nullptr;
        using raw_t = typename std::conditional<k8, uint4, typename WF::raw_t>::type;
        raw_t a[kBatch][kLoads];
        uint32_t sc[kBatch][kLoads];  // MXFP4 scale bytes (else unused)
        auto load = [&](int c0) {
#pragma unroll
            for (int d = 0; d < kBatch; ++d)
#pragma unroll
                for (int r = 0; r < kLoads; ++r) {
                    const int c = min(c0 + d, nslots - 1);  // past the end: re-read, unused
                    if constexpr (kMx) {
                        a[d][r] = load16_stream(msrc + (size_t)(8 * r) * mx_row + c * 128);
                        sc[d][r] = ssrc[(size_t)(8 * r) * mx_srow + c * 8];
                    } else if constexpr (kFp8) {
                        a[d][r] = load16_stream(src + (size_t)(8 * r) * Ie + c * kChunkElems);
                    } else {
                        a[d][r] = WF::load_raw(src + (size_t)(4 * r) * Ie + c * kChunkElems);
                    }
                }
        };
        load(0);  // the weight stream does not depend on h: start it before staging h

        __syncthreads();  // the previous unit's readers of the h tile are done
        const int cpr = Ie / Op::kPerLane;  // 16-byte chunks per h row
        for (int idx = tid; idx < n * cpr; idx += kThreads) {
            const int r = idx / cpr, c = idx - (idx / cpr) * cpr;
            const int slot = shared ? p.T * kTopK + start + r : p.perm[start + r];
            const size_t hsrc = (size_t)slot * p.Imax + c * Op::kPerLane;
            *reinterpret_cast<uint4 *>(hs_hi + r * hstride + c * Op::kPerLane) = load16(hg + hsrc);
            if constexpr (Op::kElemBytes == 2)
                *reinterpret_cast<uint4 *>(hs_lo + r * hstride + c * Op::kPerLane) =
                    load16(hg + p.plane + hsrc);
        }
        __syncthreads();

        const bool col_ok = col < n;
        const int crow = col_ok ? col : 0;  // columns >= n repeat column 0 (dropped)
        const h_t *bhp = hs_hi + crow * hstride + q * Op::kPerLane;
        const h_t *blp = hs_lo + crow * hstride + q * Op::kPerLane;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        auto mma_chunk = [&](int c) {
#pragma unroll
            for (int s2 = 0; s2 < kStepsPerChunk; ++s2) {
                const int pc = kMx ? mx_piece_pos(4 * s2 + q, 0) : kFp8 ? fp8_piece_pos(4 * s2 + q)
                                                                      : 4 * s2 + q;
                const uint4 av = lds_load16(stage + col * 256 + ((pc ^ col) & 15) * 16);
                const int kk = c * kChunkElems + 4 * s2 * Op::kPerLane;
                Op::mma(acc, av, lds_load16(bhp + kk));
                if constexpr (Op::kElemBytes == 2) Op::mma(acc, av, lds_load16(blp + kk));
            }
        };
        for (int c0 = 0; c0 < nslots; c0 += kBatch) {
            if (c0 > 0) load(c0);
#pragma unroll
            for (int d = 0; d < kBatch; ++d) {
                if (c0 + d >= nslots) break;  // uniform
                if constexpr (kMx) {
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        mfma_operand_guard();
                        if ((lpiece8 >> 2) == half) {  // this lane's 32 weights are in chunk half
                            const int pb = 4 * (lpiece8 & 3);
#pragma unroll
                            for (int r = 0; r < kLoads; ++r) {
                                const int rr = 8 * r + lrow8;
                                const float sf = e8m0_to_f32(sc[d][r]);
                                const uint32_t w4[4] = {a[d][r].x, a[d][r].y, a[d][r].z, a[d][r].w};
#pragma unroll
                                for (int k = 0; k < 4; ++k)
                                    *reinterpret_cast<uint4 *>(
                                        stage + rr * 256 + ((mx_piece_pos(pb + k, 0) ^ rr) & 15) * 16) =
                                        e2m1x8_to_bf16x8(w4[k], sf);
                            }
                        }
                        mma_chunk(2 * (c0 + d) + half);  // a wave's LDS ops stay in order
                    }
                    continue;
                }
                if constexpr (kFp8) mfma_operand_guard();  // the FP8 conversions as the MXFP4 ones
#pragma unroll
                for (int r = 0; r < kLoads; ++r) {
                    if constexpr (kFp8) {  // 16 codes widened to two bf16 pieces (exact)
                        const int rr = 8 * r + lrow8;
                        const int p0 = 2 * lpiece8;
                        *reinterpret_cast<uint4 *>(stage + rr * 256 + ((fp8_piece_pos(p0) ^ rr) & 15) * 16) =
                            e4m3x8_to_bf16x8(a[d][r].x, a[d][r].y);
                        *reinterpret_cast<uint4 *>(stage + rr * 256 + ((fp8_piece_pos(p0 + 1) ^ rr) & 15) * 16) =
                            e4m3x8_to_bf16x8(a[d][r].z, a[d][r].w);
                    } else {
                        const int rr = 4 * r + lrow;
                        *reinterpret_cast<uint4 *>(stage + rr * 256 + ((lpiece ^ rr) & 15) * 16) =
                            WF::to_operand(a[d][r]);
                    }
                }
                mma_chunk(c0 + d);
            }
        }
        if constexpr (WF::kScaled)  // the output rows' dequantization scales
            scale_rows(acc, (shared ? p.sdn_scale : p.dn_scale + (size_t)e * p.H) + rc * kRowsPerUnit +
                                wave * kTile + 4 * q);
        if (col_ok) {
            const int slot = shared ? p.T * kTopK + start + col : p.perm[start + col];
            const float wt = shared ? p.g[start + col] : p.w[slot];
            // lane holds rows 4q + r of the wave's 16 rows for token column col; the combine of
            // this row block may run in another block of this launch: device-coherent store
            st_dev16(p.ybuf + (size_t)slot * p.H + rc * kRowsPerUnit + wave * kTile + 4 * q,
                     uint4{__float_as_uint(wt * acc[0]), __float_as_uint(wt * acc[1]),
                           __float_as_uint(wt * acc[2]), __float_as_uint(wt * acc[3])});
        }
        // The last unit to finish row block rc (of the num_groups units that write it) sums, for
        // every token, the eight weighted rank outputs in rank order and then the gated shared
        // output: the combine, without a kernel of its own.
        if (defer) {
            ++my_units;
            continue;
        }
        wait_own_stores();
        __syncthreads();
        if (tid == 0) {
            s_last = atomicAdd(p.rb_arrivals + rc, 1) == ngroups - 1;
            if (s_last) p.rb_arrivals[rc] = 0;  // all units of rc arrived: reset for the next call
        }
        __syncthreads();
        if (s_last) {
            int t2 = tid;
            asm volatile("" : "+v"(t2));  // keeps the combine's addressing out of the unit loop
            combine_rows(p, rc * kRowsPerUnit, t2);
        }
    }
    if (defer && my_units > 0) {  // uniform over the block
        const int rc = blockIdx.x % n_rc;
        wait_own_stores();
        __syncthreads();
        if (tid == 0) {
            s_last = atomicAdd(p.rb_arrivals + rc, my_units) + my_units == ngroups;
            if (s_last) p.rb_arrivals[rc] = 0;  // all units of rc arrived: reset for the next call
        }
        __syncthreads();
        if (s_last) combine_rows(p, rc * kRowsPerUnit, tid);
    }
}

hipError_t prepare_split_kernels(size_t gateup_lds, size_t down_lds) {
    const void *gk[] = {reinterpret_cast<const void *>(&gateup_kernel<OpBF16, false>),
                        reinterpret_cast<const void *>(&gateup_kernel<OpF32, false>),
                        reinterpret_cast<const void *>(&gateup_kernel<OpBF16, true>),
                        reinterpret_cast<const void *>(&gateup_kernel<OpBF16, false, true>)};
    const void *dk[] = {reinterpret_cast<const void *>(&down_kernel<OpBF16, false>),
                        reinterpret_cast<const void *>(&down_kernel<OpF32, false>),
                        reinterpret_cast<const void *>(&down_kernel<OpBF16, true>),
                        reinterpret_cast<const void *>(&down_kernel<OpBF16, false, true>)};
    hipError_t err;
    for (const void *k : gk)
        if ((err = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)gateup_lds)) != hipSuccess)
            return err;
    for (const void *k : dk)
        if ((err = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)down_lds)) != hipSuccess)
            return err;
    return hipSuccess;
}

// dtype: 0 fp32, 1 bf16, 2 bf16 activations with FP8 E4M3 weights
hipError_t launch_gateup(const GateUpParams &p, int dtype, int grid, size_t lds, hipStream_t s) {
    if (dtype == 3) launch_k(gateup_kernel<OpBF16, false, true>, grid, kThreads, lds, s, p);
    else if (dtype == 2) launch_k(gateup_kernel<OpBF16, true>, grid, kThreads, lds, s, p);
    else if (dtype == 1) launch_k(gateup_kernel<OpBF16, false>, grid, kThreads, lds, s, p);
    else launch_k(gateup_kernel<OpF32, false>, grid, kThreads, lds, s, p);
    return hipGetLastError();
}

size_t gateup_stage_bytes() { return 4 * 2 * 4096 + 2 * 16 * 16 * 4; }
size_t down_stage_bytes() { return 4 * 4096; }

hipError_t launch_down(const DownParams &p, int dtype, int grid, size_t lds, hipStream_t s) {
    if (dtype == 3) launch_k(down_kernel<OpBF16, false, true>, grid, kThreads, lds, s, p);
    else if (dtype == 2) launch_k(down_kernel<OpBF16, true>, grid, kThreads, lds, s, p);
    else if (dtype == 1) launch_k(down_kernel<OpBF16, false>, grid, kThreads, lds, s, p);
    else launch_k(down_kernel<OpF32, false>, grid, kThreads, lds, s, p);
    return hipGetLastError();
}

}  // namespace moe
