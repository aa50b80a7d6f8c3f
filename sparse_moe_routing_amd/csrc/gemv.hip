// gemv.hip - the decode expert stage on the vector ALUs (matrix-vector products).
//
// At decode sizes each selected expert serves one or two tokens, so its gate/up and down products
// are matrix-vector products and streaming the expert weights once from HBM is the whole cost
// (the expert block is most of a MoE model's bytes and decode at concurrency is bandwidth-bound:
// "RELEASE_NOTES_0.9.0" of the 16 GB ninfer fork, the expert-placement paragraphs; the lucebox
// pull request #652 log, on decode streaming every weight byte once). Here every weight load
// reads 1 KB of one row contiguously (lane l: bytes 16 l .. 16 l + 15 of the kilobyte), each
// lane multiplies its eight bf16 weights by the matching activations with v_dot2_f32_bf16 (bf16
// products, fp32 accumulation), and the 64 lane partials of a row are summed with lane moves. No
// matrix instruction and no LDS staging of the weights.
//
// gateup_gemv_kernel - a wave unit is (expert group, intermediate rows 2j and 2j + 1): it reads
//   gate rows 2j, 2j + 1 and up rows I + 2j, I + 2j + 1 (4 x H bf16, two units' rows in flight
//   per wave) and forms h = silu(gate) * up for each token of the group, written as the two bf16
//   planes hi = bf16(h), lo = bf16(h - hi) the down products read. The group's tokens are taken
//   kNB at a time with the weights kept in registers. The grid's waves split the group list:
//   with fewer groups than waves each group's units are cut into contiguous runs, one per wave
//   (a wave loads its group's activations once); otherwise each wave takes whole groups.
// down_rows_kernel - a block owns 8 consecutive rows of y for every token: its waves take the
//   groups in turn, read those 8 rows of each group's down weight (8 x I weights; the next group's
//   rows and h are requested before the current one is computed), multiply them by the group's
//   h and keep every (slot, row) product in LDS; the block then sums each token's eight ranks in
//   rank order, weighted, plus its gated shared slot into y. Every output element has one writer
//   and no step crosses blocks.
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kGemvWaves = 8;
constexpr int kGemvThreads = kGemvWaves * kWave;
// tokens per expert group on this path (the plan's group size): the gate/up kernel keeps
// their activations in registers, the down kernel their h rows
constexpr int kGuNB = 4;
constexpr int kDnNB = 4;      // members whose h rows a ring stage holds
constexpr int kDnMaxNB = 8;   // members a down_rows group may have (the rest load h when computed)
constexpr int kDownRows = 8;

__device__ __forceinline__ float dot8(const uint4 &w, const uint4 &x, float c) {
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x),
                                        __builtin_bit_cast(bf16x2_t, x.x), c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y),
                                        __builtin_bit_cast(bf16x2_t, x.y), c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z),
                                        __builtin_bit_cast(bf16x2_t, x.z), c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w),
                                        __builtin_bit_cast(bf16x2_t, x.w), c, false);
    return c;
}

// The value v of lane ^ 16 (kXor == 16) or lane ^ 32 (kXor == 32): a gfx950 permlane swap
// returns the lane's own value in one result and the partner's in the other.
template <int kXor>
__device__ __forceinline__ float lane_xor(float v) {
    const uint32_t u = __float_as_uint(v);
    if constexpr (kXor == 16) {
        const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return __uint_as_float(s[0] ^ s[1] ^ u);
    } else {
        const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return __uint_as_float(s[0] ^ s[1] ^ u);
    }
}

template <int kCtrl>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), kCtrl, 0xF, 0xF,
                                                           false));
}

// Sums over the 64 lanes of four per-lane values a0..a3: on return every lane of row group
// g = lane / 16 holds the total of a_g (the same bits in all 16 lanes). The halves of the wave
// first exchange the pairs they do not keep (lane ^ 32), then the rows of a pair (lane ^ 16), then
// each 16-lane row sums with DPP moves (xor 1, xor 2, mirror in 8, mirror in 16).
__device__ __forceinline__ float wave_sum4(float a0, float a1, float a2, float a3, int lane) {
    const bool upper = lane >= 32;
    float k0 = upper ? a2 : a0, k1 = upper ? a3 : a1;
    const float s0 = upper ? a0 : a2, s1 = upper ? a1 : a3;
    k0 += lane_xor<32>(s0);
    k1 += lane_xor<32>(s1);
    const bool odd = (lane & 16) != 0;
    float k = odd ? k1 : k0;
    k += lane_xor<16>(odd ? k0 : k1);
    k = dpp_add<0xB1>(k);   // quad_perm [1, 0, 3, 2]
    k = dpp_add<0x4E>(k);   // quad_perm [2, 3, 0, 1]
    k = dpp_add<0x141>(k);  // row_half_mirror
    k = dpp_add<0x140>(k);  // row_mirror
    return k;
}

// Wave unit split of the group list (see the file comment): the range of groups a wave takes and,
// for each, its range of units [j0, j1) out of S.
struct WaveShare {
    int g0, gstep, j0, j1;
    __device__ WaveShare(int gw, int W, int ng, int S) {
        if (ng <= W) {
            const int wpg = W / ng;      // waves per group (>= 1)
            const int gi = gw / wpg, k = gw - gi * wpg;
            g0 = gi < ng ? gi : ng;      // past the last group: no work
            gstep = ng;                  // one group only
            j0 = (int)((long)k * S / wpg);
            j1 = (int)((long)(k + 1) * S / wpg);
        } else {
            g0 = gw;
            gstep = W;
            j0 = 0;
            j1 = S;
        }
    }
};

// Weight formats of the vector-ALU kernels. A lane's piece of a row chunk is the 8 weights
// 512 c + 8 lane .. + 7 of the row (c: the chunk of 512 weights), held as stored until the
// compute step widens it to eight bf16 operands, exactly:
//   kBF16  - 16 bytes of bf16 (the operands themselves);
//   kFP8   - 8 bytes of OCP FP8 E4M3 codes (every E4M3 value is a bf16 value); the row's fp32
//            scale multiplies the row's reduced product (scale * sum(code * operand));
//   kMXFP4 - 4 bytes of E2M1 codes (two per byte, the even weight in the low nibble) with their
//            block's E8M0 scale byte (block (512 c + 8 lane) / 32 of the row), widened and scaled
//            in one gfx950 conversion (exact while the product is a finite bf16).
// Every format gives each lane the same weights, so the products and their order are the bf16
// kernel's: on weights a bf16 context holds exactly (every MXFP4 weight; FP8 under power-of-two
// row scales) the outputs are the same bits.
enum { kBF16 = 0, kFP8 = 1, kMXFP4 = 2 };

constexpr uint32_t kPast = 0x80000000u;  // an offset past every resource here (each < 2 GiB)

// The stored piece (chunk c, this lane) of row `row` of a matrix of rows of `cols` weights, read
// through the buffer resource rw (MXFP4: its scale bytes through rs). `in` false: nothing to read
// (a load past the resource: no memory access, the same count of loads in flight).
template <int FMT>
__device__ __forceinline__ uint4 load_piece(__amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rs,
                                            uint32_t row, int cols, int c, int lane, bool in) {
    if constexpr (FMT == kBF16) {
        return bload16_stream(rw, in ? (row * cols + 512 * c + 8 * lane) * 2 : kPast);
    } else if constexpr (FMT == kFP8) {
        const u32x2_t v = bload8_stream(rw, in ? row * cols + 512 * c + 8 * lane : kPast);
        return uint4{v.x, v.y, 0u, 0u};
    } else {
        const uint32_t v = bload4_stream(rw, in ? row * (cols / 2) + 256 * c + 4 * lane : kPast);
        const uint32_t sb = bload1(rs, in ? row * (cols / 32) + 16 * c + lane / 4 : kPast);
        return uint4{v, sb, 0u, 0u};
    }
}

// Bytes of a stored row of `cols` weights.
template <int FMT>
__host__ __device__ constexpr uint32_t row_bytes(int cols) {
    return FMT == kBF16 ? 2 * cols : FMT == kFP8 ? cols : cols / 2;
}

// The eight bf16 operands of a stored piece.
template <int FMT>
__device__ __forceinline__ uint4 widen(const uint4 &w) {
    if constexpr (FMT == kBF16) return w;
    else if constexpr (FMT == kFP8) return e4m3x8_to_bf16x8(w.x, w.y);
    else return e2m1x8_to_bf16x8(w.x, e8m0_to_f32(w.y));
}

// The gate/up units of wave gw of W.
template <int FMT, int KC>
__device__ __forceinline__ void gateup_gemv_waves(const GateUpParams &p, int gw, int W, int lane) {
    const int ng = p.num_groups[0];
    if (ng <= 0) return;       // no valid pair and no shared expert
    const int S = p.Imax / 2;  // units per group (two intermediate rows each)
    const WaveShare share(gw, W, ng, S);
    const uint16_t *x = reinterpret_cast<const uint16_t *>(p.x);
    uint16_t *hp = reinterpret_cast<uint16_t *>(p.h);

    for (int gi = share.g0; gi < ng; gi += share.gstep) {
        const int4 grp = p.groups[gi];
        const int e = grp.x, start = grp.y, n = grp.z;  // n <= kGuNB (the plan's group size)
        const bool shared = e == p.E;
        const int Ie = shared ? p.Is : p.I;
        const int j0 = share.j0, j1 = min(share.j1, Ie / 2);
        if (j0 >= j1) continue;  // uniform over the wave
        int slot[kGuNB], tok[kGuNB];
#pragma unroll
        for (int t = 0; t < kGuNB; ++t) {
            const int m = t < n ? t : 0;  // past the group: a repeat of member 0, unused
            slot[t] = shared ? p.T * kTopK + start + m : p.perm[start + m];
            tok[t] = shared ? slot[t] - p.T * kTopK : slot[t] >> 3;
        }
        // the expert's [2 Ie][H] matrix (rows: gate, then up) and its FP8 row scales or MXFP4
        // scale bytes; a unit past the wave's range issues its loads past the resources (no
        // memory access): every iteration issues the same loads, so the compiler's wait counts
        // stay exact and two units stay in flight
        const unsigned char *gu = static_cast<const unsigned char *>(shared ? p.sgu : p.gate_up) +
                                  (shared ? 0 : (size_t)e * 2 * Ie * row_bytes<FMT>(p.H));
        const auto rw = buffer_rsrc(gu, 2 * Ie * row_bytes<FMT>(p.H));
        const auto rs = FMT == kMXFP4 ? buffer_rsrc((shared ? p.sgu_mx : p.gu_mx + (size_t)e * 2 * Ie * (p.H / 32)),
                                                    2 * Ie * (p.H / 32))
                        : FMT == kFP8 ? buffer_rsrc(shared ? p.sgu_scale : p.gu_scale + (size_t)e * 2 * Ie, 8 * Ie)
                                      : rw;
        // the weights of unit j: gate rows 2j, 2j + 1, up rows Ie + 2j, Ie + 2j + 1; FP8: lane l
        // also reads the scale of row l & 3 of the unit, in the same queue as the weights
        // (scalar loads of the scales would each wait for every scalar load in flight)
        auto load_w = [&](uint4 (&w)[4][KC], float &sc, int j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t row = (r < 2 ? 0 : Ie) + 2 * j + (r & 1);
#pragma unroll
                for (int c = 0; c < KC; ++c) w[r][c] = load_piece<FMT>(rw, rs, row, p.H, c, lane, j < j1);
            }
            if constexpr (FMT == kFP8) {
                const int r = lane & 3;
                sc = __uint_as_float(bload4(rs, j < j1 ? ((r < 2 ? 0 : Ie) + 2 * j + (r & 1)) * 4 : kPast));
            }
        };
        uint4 xr[kGuNB][KC];
#pragma unroll
        for (int t = 0; t < kGuNB; ++t)
#pragma unroll
            for (int c = 0; c < KC; ++c) xr[t][c] = load16(x + (size_t)tok[t] * p.H + 8 * lane + 512 * c);
        auto compute = [&](const uint4 (&w)[4][KC], float scv, int j) {
#pragma unroll
            for (int t = 0; t < kGuNB; ++t) {
                if (t >= n) break;  // uniform
                float a[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float s = 0.f;
#pragma unroll
                    for (int c = 0; c < KC; ++c) s = dot8(widen<FMT>(w[r][c]), xr[t][c], s);
                    a[r] = s;
                }
                const float v = wave_sum4(a[0], a[1], a[2], a[3], lane);
                // row group 0: gate 2j, 1: gate 2j + 1, 2: up 2j, 3: up 2j + 1
                float ga = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
                float gb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
                float ua = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
                float ub = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
                if constexpr (FMT == kFP8) {  // the rows' scales, from lanes 0 .. 3
                    ga *= __int_as_float(__builtin_amdgcn_readlane(__float_as_int(scv), 0));
                    gb *= __int_as_float(__builtin_amdgcn_readlane(__float_as_int(scv), 1));
                    ua *= __int_as_float(__builtin_amdgcn_readlane(__float_as_int(scv), 2));
                    ub *= __int_as_float(__builtin_amdgcn_readlane(__float_as_int(scv), 3));
                }
                if (lane == 0) {
                    const float h0 = ga / (1.0f + expf(-ga)) * ua;
                    const float h1 = gb / (1.0f + expf(-gb)) * ub;
                    const uint32_t hi0 = f32_to_bf16_bits(h0), hi1 = f32_to_bf16_bits(h1);
                    const uint32_t lo0 = f32_to_bf16_bits(h0 - bf16_bits_to_f32(hi0));
                    const uint32_t lo1 = f32_to_bf16_bits(h1 - bf16_bits_to_f32(hi1));
                    const size_t off = (size_t)slot[t] * p.Imax + 2 * j;
                    *reinterpret_cast<uint32_t *>(hp + off) = hi0 | (hi1 << 16);
                    *reinterpret_cast<uint32_t *>(hp + p.plane + off) = lo0 | (lo1 << 16);
                }
            }
        };
        uint4 wA[4][KC], wB[4][KC];
        float sA = 1.f, sB = 1.f;
        load_w(wA, sA, j0);
        load_w(wB, sB, j0 + 1);
        for (int j = j0; j < j1; j += 2) {
            compute(wA, sA, j);
            load_w(wA, sA, j + 2);
            if (j + 1 < j1) compute(wB, sB, j + 1);  // uniform; no vector-memory loads inside
            load_w(wB, sB, j + 3);
        }
    }
}

template <int FMT, int KC>
__global__ __launch_bounds__(kGemvThreads) void gateup_gemv_kernel(GateUpParams p) {
    // wave-uniform indices live in scalar registers, so the group table and pair indices are
    // read through the scalar cache and never wait behind the weight stream
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    gateup_gemv_waves<FMT, KC>(p, blockIdx.x * kGemvWaves + wave, gridDim.x * kGemvWaves,
                               threadIdx.x & 63);
}


// The down rows of block blk (rows 8 blk .. 8 blk + 7 of y for every token) into LDS obuf, then
// y, with NW waves.
template <int FMT, int KD, int NW = kGemvWaves>
__device__ __forceinline__ void down_rows_block(const DownParams &p, int blk, float *obuf) {
    constexpr int kRing = KD == 1 ? 3 : 1;         // groups in flight per wave
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform indices live in scalar registers: the group table and pair indices are read
    // through the scalar cache, so the only vector-memory loads are the weights and h rows
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r0 = blk * kDownRows;
    const int ng = p.num_groups[0];
    const uint16_t *hg = reinterpret_cast<const uint16_t *>(p.h);

    // the weight (and scale) arrays as integers, chosen between as integers: a choice between two
    // parameter pointers otherwise becomes a two-entry table in scratch memory
    const uintptr_t w_rt = (uintptr_t)p.down, w_sh = (uintptr_t)p.sdn;
    const uintptr_t s_rt = FMT == kMXFP4 ? (uintptr_t)p.dn_mx : (uintptr_t)p.dn_scale;
    const uintptr_t s_sh = FMT == kMXFP4 ? (uintptr_t)p.sdn_mx : (uintptr_t)p.sdn_scale;
    struct Stage {
        uint4 w[kDownRows][KD];   // bf16: 4 words; FP8: words x, y; MXFP4: word x, scale byte y
        uint4 hh[kDnNB][KD], hl[kDnNB][KD];
        float s0, s1;             // FP8: the scales of rows lane / 16 and lane / 16 + 4
        int slot[kDnNB];          // the members' row slots (wave-uniform)
    };
    // Group gi's kDownRows rows of its down weight (with FP8 row scales), read through buffer
    // resources over just those rows. Every weight load is issued whatever the group, so that the
    // compiler's wait counts stay exact and kRing groups stay in flight: past the last group the
    // resources are empty and past a narrower expert's chunks the offsets lie beyond them, so
    // those loads make no memory access (the compute step never uses them).
    auto load_w = [&](Stage &st, int gi) {
        const bool ok = gi < ng;
        const int4 grp = p.groups[ok ? gi : 0];
        const int e = ok ? grp.x : p.E;
        const bool shared = e == p.E;
        const int Ie = shared ? p.Is : p.I;
        const int kd = ok ? Ie / 512 : 0;
        const size_t row0 = (shared ? 0 : (size_t)e * p.H) + r0;  // first row, of [E][H]
        const uintptr_t wbase = (shared ? w_sh : w_rt) + row0 * row_bytes<FMT>(Ie);
        const auto rw = buffer_rsrc(reinterpret_cast<const void *>(wbase), ok ? kDownRows * row_bytes<FMT>(Ie) : 0);
        // MXFP4: the rows' scale bytes; FP8: their fp32 scales
        const uint32_t srow = FMT == kMXFP4 ? Ie / 32 : 4;
        const auto rs = buffer_rsrc(reinterpret_cast<const void *>((shared ? s_sh : s_rt) + row0 * srow),
                                    ok && FMT != kBF16 ? kDownRows * srow : 0);
#pragma unroll
        for (int r = 0; r < kDownRows; ++r)
#pragma unroll
            for (int c = 0; c < KD; ++c) st.w[r][c] = load_piece<FMT>(rw, rs, r, Ie, c, lane, c < kd);
        if constexpr (FMT == kFP8) {
            st.s0 = __uint_as_float(bload4(rs, (lane >> 4) * 4));
            st.s1 = __uint_as_float(bload4(rs, ((lane >> 4) + 4) * 4));
        }
    };
    // The h rows of the group's members: only those the group has (a uniform condition; dummy
    // reads for the absent members measured 2.5 us of the T = 4 down pass). The members' slots
    // are read first, all at once and unconditionally (past the members: a repeat of the last
    // one), so that a group's scalar reads make one round trip, not one per member. A stage
    // issues these before its weight loads, which are unconditional, so the wait counts still
    // cover the ring.
    auto load_h = [&](Stage &st, int gi) {
        const bool ok = gi < ng;
        const int4 grp = p.groups[ok ? gi : 0];
        const int n = ok ? grp.z : 0;
        const int kd = ok ? (grp.x == p.E ? p.Is : p.I) / 512 : 0;
        const bool routed = ok && grp.x != p.E;
#pragma unroll
        for (int m = 0; m < kDnNB; ++m) {
            const int mm = min(m, n - 1);
            // one unconditional load per member (perm[0] where unused), so that the four reads
            // go out together
            const int pv = p.perm[routed ? grp.y + mm : 0];
            st.slot[m] = routed ? pv : p.T * kTopK + grp.y + mm;
        }
#pragma unroll
        for (int m = 0; m < kDnNB; ++m) {
            if (m >= n) break;  // uniform
            const uint16_t *hs = hg + (size_t)st.slot[m] * p.Imax + 8 * lane;
#pragma unroll
            for (int c = 0; c < KD; ++c) {
                if (c >= kd) break;  // uniform
                st.hh[m][c] = load16(hs + 512 * c);
                st.hl[m][c] = load16(hs + p.plane + 512 * c);
            }
        }
    };
    // the kDownRows row products of one member's h (hi and lo planes) over the expert's kd
    // chunks, summed over the wave: rows g and g + 4 land in row group g, which writes them
    // (times the rows' FP8 scales)
    auto emit = [&](const uint4 (&w)[kDownRows][KD], const uint4 (&hh)[KD], const uint4 (&hl)[KD],
                    int kd, float s0, float s1, int slot) {
        float a[kDownRows];
#pragma unroll
        for (int r = 0; r < kDownRows; ++r) {
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < KD; ++c) {
                if (c >= kd) break;  // uniform
                const uint4 wv = widen<FMT>(w[r][c]);
                s = dot8(wv, hh[c], s);
                s = dot8(wv, hl[c], s);
            }
            a[r] = s;
        }
        float v0 = wave_sum4(a[0], a[1], a[2], a[3], lane);
        float v1 = wave_sum4(a[4], a[5], a[6], a[7], lane);
        if ((lane & 15) == 0) {
            const int g = lane >> 4;
            if constexpr (FMT == kFP8) {  // the row scales, read with the stage
                v0 *= s0;
                v1 *= s1;
            }
            obuf[slot * kDownRows + g] = v0;
            obuf[slot * kDownRows + 4 + g] = v1;
        }
    };
    // The stage holds the first kDnNB members' h rows; a group with more members (up to
    // kDnMaxNB, the plan's group size: expert groups of 8 tokens keep a hot expert's weights
    // from being read once per 4 of its tokens) loads the others' h rows here, against the
    // weights already in registers.
    auto compute = [&](const Stage &st, int gi) {
        const int4 grp = p.groups[gi];
        const int n = grp.z;  // n <= kDnMaxNB
        const int kd = (grp.x == p.E ? p.Is : p.I) / 512;
#pragma unroll
        for (int m = 0; m < kDnNB; ++m)
            if (m < n) emit(st.w, st.hh[m], st.hl[m], kd, st.s0, st.s1, st.slot[m]);
        // members past the stage (uniform; rare in near-uniform routing): their h loads queue
        // behind the ring's, so each waits for the stages in flight
        for (int m = kDnNB; m < n; ++m) {
            const int slot = grp.x == p.E ? p.T * kTopK + grp.y + m : p.perm[grp.y + m];
            const uint16_t *hs = hg + (size_t)slot * p.Imax + 8 * lane;
            uint4 hh[KD], hl[KD];
#pragma unroll
            for (int c = 0; c < KD; ++c) {
                hh[c] = c < kd ? load16(hs + 512 * c) : uint4{0u, 0u, 0u, 0u};
                hl[c] = c < kd ? load16(hs + p.plane + 512 * c) : uint4{0u, 0u, 0u, 0u};
            }
            emit(st.w, hh, hl, kd, st.s0, st.s1, slot);
        }
    };
    // The combine's operands, requested before the weight stream so that they are in registers
    // when the products are: thread i < 8 T owns row r = i % 8 of token t = i / 8 (8 T <= the
    // block's threads; the launch checks it)
    const int ct = tid / kDownRows, cr = tid - ct * kDownRows;
    const bool cact = ct < p.T;
    int cid[kTopK];
    float cw[kTopK], cg = 0.f;
#pragma unroll
    for (int k = 0; k < kTopK; ++k) {
        cid[k] = cact ? p.ids[ct * kTopK + k] : -1;
        cw[k] = cact ? p.w[ct * kTopK + k] : 0.f;
    }
    if (cact && p.g) cg = p.g[ct];
    // a ring of kRing groups per wave: group k + kRing is requested right after group k is done
    Stage st[kRing];
#pragma unroll
    for (int d = 0; d < kRing; ++d) {
        load_h(st[d], wave + d * NW);
        load_w(st[d], wave + d * NW);
    }
    for (int k = 0; wave + k * NW < ng; k += kRing) {
#pragma unroll
        for (int d = 0; d < kRing; ++d) {
            const int gi = wave + (k + d) * NW;
            if (gi < ng) compute(st[d], gi);  // uniform
            load_h(st[d], gi + kRing * NW);
            load_w(st[d], gi + kRing * NW);
        }
    }
    __syncthreads();
    // y rows r0 .. r0 + kDownRows - 1: the eight ranks in rank order (weighted; a pair whose id
    // lies outside [0, E) was dropped by the bucketing and adds nothing), then the gated shared
    // slot
    if (cact) {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < kTopK; ++k)
            if (cid[k] >= 0 && cid[k] < p.E) acc += cw[k] * obuf[(ct * kTopK + k) * kDownRows + cr];
        if (p.g) acc += cg * obuf[(p.T * kTopK + ct) * kDownRows + cr];
        p.y[(size_t)ct * p.H + r0 + cr] = acc;
    }
}

template <int FMT, int KD>
__global__ __launch_bounds__(kGemvThreads) void down_rows_kernel(DownParams p) {
    extern __shared__ __align__(16) float obuf[];  // [slots][kDownRows]: (Wd h)[row] per slot
    down_rows_block<FMT, KD>(p, blockIdx.x, obuf);
}


int gemv_group_tokens() { return kGuNB; }
int down_rows_group_tokens() { return kDnMaxNB; }

// GEMV-path shapes: H a multiple of 512 up to 2048 (weight rows in chunks of 512 weights, at
// most four per row held per lane), I and I_s multiples of 512 up to 1024.
bool gemv_supported(int H, int I, int Is) {
    const int Imax = I > Is ? I : Is;
    return H % 512 == 0 && H <= 2048 && I % 512 == 0 && (Is == 0 || Is % 512 == 0) &&
           Imax <= 1024;
}

// down_rows shapes: rows of y in blocks of 8, intermediate rows of whole kilobytes (bf16), at
// most two of them per lane.
bool down_rows_supported(int H, int I, int Is) {
    const int Imax = I > Is ? I : Is;
    return H % kDownRows == 0 && I % 512 == 0 && (Is == 0 || Is % 512 == 0) && Imax <= 1024;
}

// LDS of down_rows_kernel: 32 bytes per slot (at most 64 tokens: 18 KB, under the default
// dynamic LDS limit)
size_t down_rows_lds(int slots) { return (size_t)slots * kDownRows * sizeof(float); }

template <int FMT>
hipError_t launch_gateup_gemv_fmt(const GateUpParams &p, int grid, hipStream_t s) {
    switch (p.H / 512) {
    case 1: launch_k(gateup_gemv_kernel<FMT, 1>, grid, kGemvThreads, 0, s, p); break;
    case 2: launch_k(gateup_gemv_kernel<FMT, 2>, grid, kGemvThreads, 0, s, p); break;
    case 3: launch_k(gateup_gemv_kernel<FMT, 3>, grid, kGemvThreads, 0, s, p); break;
    case 4: launch_k(gateup_gemv_kernel<FMT, 4>, grid, kGemvThreads, 0, s, p); break;
    default: return hipErrorInvalidValue;  // a caller bug: the plan checks gemv_supported
    }
    return hipGetLastError();
}

// dtype: 1 bf16, 2 FP8 E4M3, 3 MXFP4 weights (bf16 activations)
hipError_t launch_gateup_gemv(const GateUpParams &p, int dtype, int grid, hipStream_t s) {
    if (dtype == 1) return launch_gateup_gemv_fmt<kBF16>(p, grid, s);
    if (dtype == 2) return launch_gateup_gemv_fmt<kFP8>(p, grid, s);
    if (dtype == 3) return launch_gateup_gemv_fmt<kMXFP4>(p, grid, s);
    return hipErrorInvalidValue;
}

// dtype: 1 bf16, 2 FP8 E4M3, 3 MXFP4 weights (bf16 activations)
template <int FMT>
void launch_down_rows_fmt(const DownParams &p, int grid, size_t lds, hipStream_t s) {
    if (p.Imax <= 512) launch_k(down_rows_kernel<FMT, 1>, grid, kGemvThreads, lds, s, p);
    else launch_k(down_rows_kernel<FMT, 2>, grid, kGemvThreads, lds, s, p);
}

hipError_t launch_down_rows(const DownParams &p, int dtype, hipStream_t s) {
    // a caller bug: the plan checks down_rows_supported and T <= 64
    if (p.H % kDownRows || p.Imax > 1024 || p.T * kDownRows > kGemvThreads) return hipErrorInvalidValue;
    const size_t lds = down_rows_lds(p.T * kTopK + (p.g ? p.T : 0));
    const int grid = p.H / kDownRows;
    if (dtype == 1) launch_down_rows_fmt<kBF16>(p, grid, lds, s);
    else if (dtype == 2) launch_down_rows_fmt<kFP8>(p, grid, lds, s);
    else if (dtype == 3) launch_down_rows_fmt<kMXFP4>(p, grid, lds, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace moe
