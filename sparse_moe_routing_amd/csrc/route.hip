// route.hip - top-8 selection (one wave64 per token) and the atomic-free bucketing pass.
//
// Selection follows the router tail of the page "feat(windows): integrate upstream Qwen3.8
// DFlash2 support - #8" (commit message on the small-T MoE router): experts are ranked by a
// total order - the larger logit first, the lower expert id first on equal logits - so the
// eight winners and their order are unique and any exact method returns them. Here each lane
// holds its candidates as one 64-bit key per expert whose unsigned order IS that total order:
//   high 32 bits: the fp32 logit mapped monotonically to an unsigned integer, with -0 and +0
//                 sharing one key and every NaN mapped to 0 (below -inf);
//   low 32 bits : the complement of the expert id (a lower id gives a larger key).
// A lane sorts its (up to four) keys, then six exchange levels - each pairing the two halves of
// groups of 2, 4, 8, 16, 32, 64 lanes through register-to-register lane moves - merge sorted
// runs of eight: keep the larger of a[i] and partner[7-i] (a bitonic sequence that holds the top
// eight of the sixteen) and sort it with three compare-exchange stages. That is the page's
// pairwise merge of sorted per-lane runs, widened from its 32-lane warp (five levels) to the
// 64-lane wavefront (six levels). After the last level every lane holds the same sorted
// top eight; lanes 0..7 decode one winner each and form the softmax over the eight chosen logits
// (reference point: the top logit), and the shared-expert gate is the sigmoid of score E.
//
// Bucketing is a stable counting sort of the T*8 (token, rank) pairs by expert id, without
// atomics and without per-expert scans over all pairs. For a chunk of 64 consecutive pairs (one
// per lane), eight wave ballots of the expert-id bits (plus a validity ballot) describe the
// chunk completely: AND-ing, for each bit, the ballot or its complement gives the set of lanes
// holding a given expert. Expert e's count in the chunk is the popcount of that set; a pair's
// stable rank among the pairs of its expert is its rank inside the set (popcount of the lanes
// below it) plus the counts of e in the earlier chunks. Exclusive scans over experts give the
// offsets and the expert-group table that drives the expert kernel.
#include "select_core.h"

namespace moe {

// ----------------------------------------------------------------------------- bucketing
constexpr int kChunkTokens = 64;                       // most tokens one bucketing block takes
constexpr int kChunkPairs = kChunkTokens * kTopK;      // 512 pairs
constexpr int kSelBucketPairs = 256 * kTopK;           // select_bucket_kernel: T <= 256

// LDS of the bucketing of up to kPairs pairs (sub-chunks of 64 pairs, one wave ballot each).
template <int kPairs>
struct BucketSharedT {
    static constexpr int kSub = kPairs / kWave;
    alignas(16) int32_t ids[kPairs];  // expert id of each pair (any value outside [0,E): none)
    uint64_t bits[kSub][8];           // per sub-chunk: ballot of each expert-id bit
    uint64_t valid[kSub];             // per sub-chunk: ballot of the pairs with a valid id
    int pre[kSub][256];               // count of expert e in the sub-chunks before s
    int a[256], b[256];               // per-expert counts / group counts, then their scans
    int tot[2];
    uint64_t sel[16][kSelScratch];    // selection scratch of each of up to 16 waves
};
using BucketShared = BucketSharedT<kChunkPairs>;

// Lanes of sub-chunk sc whose pair holds expert e.
template <class S>
__device__ __forceinline__ uint64_t lanes_of(const S &s, int sc, int e) {
    uint64_t m = s.valid[sc];
#pragma unroll
    for (int b = 0; b < 8; ++b) m &= ((e >> b) & 1) ? s.bits[sc][b] : ~s.bits[sc][b];
    return m;
}

// Ballots of the n pairs in s.ids (wave w takes sub-chunks w, w + waves, ...), then per expert
// (threads 0..255): the counts of the sub-chunks before each sub-chunk (s.pre) and the total.
// Every thread calls it.
template <class S>
__device__ int chunk_counts(S &s, int n, int E) {
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int nw = blockDim.x / kWave;
    const int nsub = (n + kWave - 1) / kWave;
    for (int sc = wave; sc < nsub; sc += nw) {
        const int pidx = sc * kWave + lane;
        const int e = pidx < n ? s.ids[pidx] : -1;
        const bool ok = e >= 0 && e < E;
        const uint64_t vb = __ballot(ok);
        uint64_t bb[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) bb[b] = __ballot(ok && ((e >> b) & 1));
        if (lane == 0) {
            s.valid[sc] = vb;
#pragma unroll
            for (int b = 0; b < 8; ++b) s.bits[sc][b] = bb[b];
        }
    }
    __syncthreads();
    int cnt = 0;
    if (tid < E) {
        for (int sc = 0; sc < nsub; ++sc) {
            s.pre[sc][tid] = cnt;
            cnt += __popcll(lanes_of(s, sc, tid));
        }
    }
    return cnt;
}

// Writes perm[base_of(e) + stable rank] = p0 + pair index for every valid pair (sub-chunks as
// in chunk_counts). base_of(e) gives the destination of expert e's first pair of this chunk.
// Needs s.pre, i.e. a block barrier after chunk_counts.
template <class S, class Base>
__device__ void chunk_scatter(const S &s, int n, int E, int p0, int32_t *perm, Base base_of) {
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int nw = blockDim.x / kWave;
    const int nsub = (n + kWave - 1) / kWave;
    for (int sc = wave; sc < nsub; sc += nw) {
        const int pidx = sc * kWave + lane;
        const int e = pidx < n ? s.ids[pidx] : -1;
        if (e >= 0 && e < E) {
            const uint64_t m = lanes_of(s, sc, e);
            const int rank = __popcll(m & ((1ull << lane) - 1ull));
            perm[base_of(e) + s.pre[sc][e] + rank] = p0 + pidx;
        }
    }
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves (no LDS round trips):
// shifts by 1, 2, 4, 8 inside each 16-lane row, then each row adds the total of the row before
// (broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15 to rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31 to rows 2, 3
    return v;
}

// Exclusive scans over experts of s.a and s.b (256 entries each, by wave 0 of the block).
// Every thread of the block calls it.
template <class S>
__device__ void scan_experts(S &s) {
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < kWave) {
        const int l = tid;
        int a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = s.a[4 * l + i];
            b[i] = s.b[4 * l + i];
        }
        const int sa = a[0] + a[1] + a[2] + a[3];
        const int sb = b[0] + b[1] + b[2] + b[3];
        const int ia = wave_inclusive_sum(sa), ib = wave_inclusive_sum(sb);
        int ea = ia - sa, eb = ib - sb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s.a[4 * l + i] = ea;
            s.b[4 * l + i] = eb;
            ea += a[i];
            eb += b[i];
        }
        if (l == kWave - 1) {
            s.tot[0] = ia;
            s.tot[1] = ib;
        }
    }
    __syncthreads();
}

// Offsets, counts and the group table from per-expert totals (thread e < E owns expert e; its
// offset ends up in s.a[e]). Every thread calls it.
template <class S>
__device__ void write_tables(const BucketParams &bp, int cnt, S &s) {
    const int tid = threadIdx.x;
    const bool own = tid < bp.E;
    const int c = own ? cnt : 0;
    const int ng = (c + bp.NG - 1) / bp.NG;
    if (tid < 256) {
        s.a[tid] = c;
        s.b[tid] = ng;
    }
    scan_experts(s);
    const int off = tid < 256 ? s.a[tid] : 0;
    const int gbase = tid < 256 ? s.b[tid] : 0;
    const int nsh = bp.has_shared ? (bp.T + bp.NG - 1) / bp.NG : 0;
    if (own) {
        bp.counts[tid] = c;
        bp.offsets[tid] = off;
        for (int gg = 0; gg < ng; ++gg)
            bp.groups[nsh + gbase + gg] =
                make_int4(tid, off + gg * bp.NG, min(bp.NG, c - gg * bp.NG), 0);
    }
    if (tid < nsh) bp.groups[tid] = make_int4(bp.E, tid * bp.NG, min(bp.NG, bp.T - tid * bp.NG), 0);
    if (tid == 0) {
        bp.offsets[bp.E] = s.tot[0];
        bp.num_groups[0] = nsh + s.tot[1];
    }
    if (bp.NG2 > 0) {  // uniform: the second table, groups of up to NG2 tokens
        __syncthreads();  // every thread has read its scans
        const int ng2 = (c + bp.NG2 - 1) / bp.NG2;
        if (tid < 256) {
            s.a[tid] = 0;
            s.b[tid] = ng2;
        }
        scan_experts(s);
        const int gbase2 = tid < 256 ? s.b[tid] : 0;
        const int nsh2 = bp.has_shared ? (bp.T + bp.NG2 - 1) / bp.NG2 : 0;
        if (own)
            for (int gg = 0; gg < ng2; ++gg)
                bp.groups2[nsh2 + gbase2 + gg] =
                    make_int4(tid, off + gg * bp.NG2, min(bp.NG2, c - gg * bp.NG2), 0);
        if (tid < nsh2)
            bp.groups2[tid] = make_int4(bp.E, tid * bp.NG2, min(bp.NG2, bp.T - tid * bp.NG2), 0);
        if (tid == 0) bp.num_groups2[0] = nsh2 + s.tot[1];
        __syncthreads();  // every thread has read s.b
        if (tid < 256) s.a[tid] = off;  // as after the first table: the experts' offsets
        __syncthreads();
    }
}

// The whole bucketing of n <= 64 pairs by one wave (lane l holds pair l), with no block barrier
// and the tables of the block form. Lane l finds the pairs of its own id among the nine ballots
// of chunk_counts (its rank among them is its stable position); the first pair of each id enters
// the id's count and group count into a per-expert LDS histogram (the wave's LDS operations take
// effect in issue order, so no barrier is needed), and a wave scan over the experts (four per
// lane) turns both into exclusive offsets: the expert's first slot and first group.
template <class S>
__device__ void bucket_wave(const BucketParams &bp, int n, int lane, S &s) {
    const int e = lane < n ? s.ids[lane] : -1;
    const bool ok = e >= 0 && e < bp.E;
    uint64_t eq = __ballot(ok);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const uint64_t one = __ballot(ok && ((e >> b) & 1));
        eq &= ((e >> b) & 1) ? one : ~one;
    }
    const int rank = __popcll(eq & ((1ull << lane) - 1ull));
    const int cnt = __popcll(eq);
    const bool first = ok && rank == 0;
    const int ngrp = (cnt + bp.NG - 1) / bp.NG;
    // Lanes exchange values through LDS here: each exchange is fenced at wavefront scope around a
    // wave barrier, without which the compiler may forward a lane's own earlier store to its load.
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
#pragma unroll
    for (int k = 0; k < 4; ++k) s.a[4 * lane + k] = s.b[4 * lane + k] = 0;  // experts 4l .. 4l + 3
    wave_sync();
    if (first) {
        s.a[e] = cnt;
        s.b[e] = ngrp;
    }
    wave_sync();
    int c4[4], g4[4], cs = 0, gs = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        c4[k] = s.a[4 * lane + k];
        g4[k] = s.b[4 * lane + k];
        cs += c4[k];
        gs += g4[k];
    }
    const int ci = wave_inclusive_sum(cs), gi = wave_inclusive_sum(gs);
    int co[4], go[4];
    co[0] = ci - cs;
    go[0] = gi - gs;
#pragma unroll
    for (int k = 1; k < 4; ++k) {
        co[k] = co[k - 1] + c4[k - 1];
        go[k] = go[k - 1] + g4[k - 1];
    }
    wave_sync();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        s.a[4 * lane + k] = co[k];
        s.b[4 * lane + k] = go[k];
    }
    wave_sync();
    const int nsh = bp.has_shared ? (bp.T + bp.NG - 1) / bp.NG : 0;
    if (ok) {
        const int off = s.a[e];
        bp.perm[off + rank] = lane;
        if (first) {
            const int gb = nsh + s.b[e];
            for (int gg = 0; gg < ngrp; ++gg)
                bp.groups[gb + gg] = make_int4(e, off + gg * bp.NG, min(bp.NG, cnt - gg * bp.NG), 0);
        }
    }
    if (lane < nsh) bp.groups[lane] = make_int4(bp.E, lane * bp.NG, min(bp.NG, bp.T - lane * bp.NG), 0);
    const int ctot = __builtin_amdgcn_readlane(ci, kWave - 1), gtot = __builtin_amdgcn_readlane(gi, kWave - 1);
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (4 * lane + k < bp.E) {
            bp.counts[4 * lane + k] = c4[k];
            bp.offsets[4 * lane + k] = co[k];
        }
    if (lane == 0) {
        bp.offsets[bp.E] = ctot;
        bp.num_groups[0] = nsh + gtot;
    }
}

// Selection of T <= 64 tokens (one wave per token, 16 waves) and, optionally, the whole
// bucketing pass, by one block of 1024 threads (up to 64 pairs: by one wave).
template <bool kDev = false>
__device__ void select_bucket_block(const SelectParams &sp, const BucketParams &bp, bool do_select,
                                    bool do_bucket, BucketShared &s) {
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int T = do_select ? sp.T : bp.T;
    if (do_select) {
#pragma unroll 1
        for (int t = wave; t < T; t += 16)
            select_token<kDev>(sp, t, lane, s.ids + t * kTopK, s.sel[wave]);
    } else {
        for (int i = tid; i < T * kTopK; i += blockDim.x) s.ids[i] = bp.ids_in[i];
    }
    if (!do_bucket) return;  // uniform over the block
    __syncthreads();
    const int n = T * kTopK;
    if (n <= kWave) {  // uniform
        if (wave == 0) bucket_wave(bp, n, lane, s);
        return;
    }
    const int cnt = chunk_counts(s, n, bp.E);
    write_tables(bp, cnt, s);  // ends with a barrier; s.a[e] = offset of expert e
    chunk_scatter(s, n, bp.E, 0, bp.perm, [&](int e) { return s.a[e]; });
}

// T <= 64 with given ids (or selection from given logits): one block.
__global__ __launch_bounds__(1024) void route_small_kernel(SelectParams sp, BucketParams bp,
                                                          int do_select, int do_bucket) {
    __shared__ BucketShared s;
    select_bucket_block(sp, bp, do_select != 0, do_bucket != 0, s);
}

// T <= 64 from x: one block per (token tile, row tile, quarter) computes that quarter's partial
// logits; the last block to finish (an arrival counter in the workspace state, reset by that
// block) folds the partial logits and runs the selection and the bucketing. One launch for the
// whole routing step, with the 1 MiB router read spread over 4 * 17 blocks (T <= 16).
// The partial logits cross blocks inside the launch, so they are stored and loaded device-
// coherently: a block waits for its own stores before it arrives, and no L2 write-back or
// invalidation is needed (each would flush or drop an XCD's whole L2).
template <class Op>
__global__ __launch_bounds__(1024) void route_fused_kernel(RouterParams rp, SelectParams sp,
                                                          BucketParams bp, int do_bucket,
                                                          int *arrivals) {
    __shared__ BucketShared s;
    __shared__ float red[16 * 256];
    __shared__ int s_last;
    const int tid = threadIdx.x;
    router_quarter_block<Op, true>(rp, blockIdx.x, red);
    wait_own_stores();  // every wave: its partial-logit stores are complete
    __syncthreads();
    if (tid == 0) {
        s_last = atomicAdd(arrivals, 1) == (int)gridDim.x - 1;
        if (s_last) arrivals[0] = 0;  // every block has arrived: reset for the next call
    }
    __syncthreads();
    if (!s_last) return;  // uniform over the block
    select_bucket_block<true>(sp, bp, true, do_bucket != 0, s);
}

// 16 < T <= 64 from x: the blocks of route_fused_kernel for every token tile; the last block of
// a tile (one arrival counter per tile) selects that tile's tokens, one wave each; the last tile
// to finish (a second counter) runs the bucketing of all T*8 pairs. The selections of different
// tiles run on different CUs, and one launch replaces router, selection and three bucketing
// passes. The tile's ids reach the last block device-coherently.
template <class Op>
__global__ __launch_bounds__(1024) void route_tiles_kernel(RouterParams rp, SelectParams sp,
                                                          BucketParams bp, int do_bucket,
                                                          int *tile_arrivals, int *tiles_done) {
    __shared__ BucketShared s;
    __shared__ float red[16 * 256];
    __shared__ int s_last;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int per_tile = ((rp.R + kTile - 1) / kTile) * kQuarters;
    const int tt = blockIdx.x / per_tile;
    router_quarter_block<Op, true>(rp, blockIdx.x, red);
    wait_own_stores();
    __syncthreads();
    if (tid == 0) {
        s_last = atomicAdd(tile_arrivals + tt, 1) == per_tile - 1;
        if (s_last) tile_arrivals[tt] = 0;  // the tile's blocks have all arrived
    }
    __syncthreads();
    if (!s_last) return;  // uniform over the block
    const int t0 = tt * kTile, nt = min(kTile, sp.T - t0);
    if (wave < nt) select_token<true>(sp, t0 + wave, lane, s.ids + wave * kTopK, s.sel[wave]);
    if (!do_bucket) return;  // uniform
    __syncthreads();
    for (int i = tid; i < nt * kTopK; i += blockDim.x) st_dev(sp.ids + t0 * kTopK + i, s.ids[i]);
    wait_own_stores();
    __syncthreads();
    if (tid == 0) {
        s_last = atomicAdd(tiles_done, 1) == rp.n_tt - 1;
        if (s_last) tiles_done[0] = 0;  // every tile has arrived
    }
    __syncthreads();
    if (!s_last) return;
    const int n = sp.T * kTopK;
    for (int i = tid; i < n; i += blockDim.x) s.ids[i] = ld_dev(sp.ids + i);
    __syncthreads();
    const int cnt = chunk_counts(s, n, bp.E);
    write_tables(bp, cnt, s);  // ends with a barrier; s.a[e] = offset of expert e
    chunk_scatter(s, n, bp.E, 0, bp.perm, [&](int e) { return s.a[e]; });
}

// T > 64, pass 1: per chunk of chunk_tokens tokens (one wave each), selection (optional) and
// the per-expert histogram.
__global__ __launch_bounds__(1024) void select_hist_kernel(SelectParams sp, BucketParams bp,
                                                          int do_select, int do_hist) {
    __shared__ BucketShared s;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int T = do_select ? sp.T : bp.T;
    const int t0 = blockIdx.x * bp.chunk_tokens;
    const int nt = min(bp.chunk_tokens, T - t0);
    if (do_select) {
#pragma unroll 1
        for (int i = wave; i < nt; i += 16)
            select_token(sp, t0 + i, lane, s.ids + i * kTopK, s.sel[wave]);
    } else {
        for (int i = tid; i < nt * kTopK; i += blockDim.x)
            s.ids[i] = bp.ids_in[(size_t)t0 * kTopK + i];
    }
    if (!do_hist) return;
    __syncthreads();
    const int cnt = chunk_counts(s, nt * kTopK, bp.E);
    if (tid < bp.E) bp.hist[hist_at(bp, blockIdx.x, tid)] = cnt;
}

// 64 < T <= 256: per 16-token chunk (one wave per token) the selection (optional); the chunk's
// ids are published device-coherently and the last chunk block to finish (an arrival counter in
// the workspace state, reset by that block) buckets all T*8 pairs in one pass, as route_small
// does: one launch in place of the histogram, scan and scatter passes.
using BucketWide = BucketSharedT<kSelBucketPairs>;
__global__ __launch_bounds__(1024) void select_bucket_kernel(SelectParams sp, BucketParams bp,
                                                            int do_select, int *arrivals) {
    __shared__ BucketWide s;
    __shared__ int s_last;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int T = bp.T;
    const int t0 = blockIdx.x * bp.chunk_tokens;
    const int nt = min(bp.chunk_tokens, T - t0);
    if (do_select) {
#pragma unroll 1
        for (int i = wave; i < nt; i += 16)
            select_token(sp, t0 + i, lane, s.ids + i * kTopK, s.sel[wave]);
        __syncthreads();
        for (int i = tid; i < nt * kTopK; i += blockDim.x)
            st_dev(sp.ids + (size_t)t0 * kTopK + i, s.ids[i]);  // read by the last block below
        wait_own_stores();
    }
    __syncthreads();
    if (tid == 0) {
        s_last = atomicAdd(arrivals, 1) == (int)gridDim.x - 1;
        if (s_last) arrivals[0] = 0;  // every chunk has arrived: reset for the next call
    }
    __syncthreads();
    if (!s_last) return;  // uniform over the block
    const int n = T * kTopK;
    // both loads of a thread are issued before either is used (n <= 2 * 1024)
    const int i1 = tid + (int)blockDim.x;
    const int v0 = tid < n ? (do_select ? ld_dev(sp.ids + tid) : bp.ids_in[tid]) : 0;
    const int v1 = i1 < n ? (do_select ? ld_dev(sp.ids + i1) : bp.ids_in[i1]) : 0;
    if (tid < n) s.ids[tid] = v0;
    if (i1 < n) s.ids[i1] = v1;
    __syncthreads();
    const int cnt = chunk_counts(s, n, bp.E);
    write_tables(bp, cnt, s);  // ends with a barrier; s.a[e] = offset of expert e
    chunk_scatter(s, n, bp.E, 0, bp.perm, [&](int e) { return s.a[e]; });
}

// T > 256, pass 2 with up to kScanOneBlockChunks chunks (one block): per-expert running bases
// over the chunks, counts, offsets, groups.
__global__ __launch_bounds__(1024) void bucket_scan_one_kernel(BucketParams bp) {
    __shared__ int s_part[4][256];
    __shared__ BucketShared s;
    const int tid = threadIdx.x;
    const int e = tid & 255, quarter = tid >> 8;
    const int per = (bp.n_chunks + 3) / 4;
    const int c0 = quarter * per, c1 = min(bp.n_chunks, c0 + per);
    // loads in batches of 8 chunks issued together (clamped past the end, dropped)
    constexpr int kB = 8;
    int sum = 0;
    if (e < bp.E) {
        for (int c = c0; c < c1; c += kB) {
            int v[kB];
#pragma unroll
            for (int j = 0; j < kB; ++j) v[j] = bp.hist[(size_t)min(c + j, c1 - 1) * bp.E + e];
#pragma unroll
            for (int j = 0; j < kB; ++j) sum += c + j < c1 ? v[j] : 0;
        }
    }
    s_part[quarter][e] = sum;
    __syncthreads();
    int base = 0;
    for (int qq = 0; qq < quarter; ++qq) base += s_part[qq][e];
    if (e < bp.E) {
        for (int c = c0; c < c1; c += kB) {
            int v[kB];
#pragma unroll
            for (int j = 0; j < kB; ++j) v[j] = bp.hist[(size_t)min(c + j, c1 - 1) * bp.E + e];
#pragma unroll
            for (int j = 0; j < kB; ++j) {
                if (c + j < c1) {
                    bp.hist[(size_t)(c + j) * bp.E + e] = base;
                    base += v[j];
                }
            }
        }
    }
    const int cnt = (tid < 256) ? s_part[0][e] + s_part[1][e] + s_part[2][e] + s_part[3][e] : 0;
    write_tables(bp, cnt, s);
}

// T > 256, pass 2 with more chunks: per-expert running bases over the chunks, then counts, offsets and the group
// table. Wave w of block b owns expert e = 16 b + w: lane l takes a contiguous run of the
// expert's chunks, the lanes' run sums are scanned with lane moves, and each lane rewrites its
// chunks' histogram entries with their exclusive bases (chunk order). The expert's total goes to
// counts[e] device-coherently; the last block to finish (an arrival counter in the workspace
// state, reset by that block) builds the tables from all the totals, as the single-block form
// did - spread over E / 16 blocks, the histogram reads no longer queue behind one CU. The arrival
// chain costs a few microseconds, so below kScanOneBlockChunks chunks one block is faster.
constexpr int kScanWaves = 16;
__global__ __launch_bounds__(kScanWaves * kWave) void bucket_scan_kernel(BucketParams bp, int *arrivals) {
    __shared__ BucketShared s;
    __shared__ int s_last;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int e = blockIdx.x * kScanWaves + wave;
    if (e < bp.E) {  // uniform over the wave
        int32_t *col = bp.hist + (size_t)e * bp.n_chunks;  // the expert's counts, chunk order
        const int per = (bp.n_chunks + kWave - 1) / kWave;
        const int c0 = min(lane * per, bp.n_chunks), c1 = min(c0 + per, bp.n_chunks);
        constexpr int kB = 8;  // loads issued together (clamped past the end, dropped)
        int sum = 0;
        for (int c = c0; c < c1; c += kB) {
            int v[kB];
#pragma unroll
            for (int j = 0; j < kB; ++j) v[j] = col[min(c + j, c1 - 1)];
#pragma unroll
            for (int j = 0; j < kB; ++j) sum += c + j < c1 ? v[j] : 0;
        }
        const int incl = wave_inclusive_sum(sum);
        int base = incl - sum;
        for (int c = c0; c < c1; c += kB) {
            int v[kB];
#pragma unroll
            for (int j = 0; j < kB; ++j) v[j] = col[min(c + j, c1 - 1)];
#pragma unroll
            for (int j = 0; j < kB; ++j) {
                if (c + j < c1) {
                    col[c + j] = base;
                    base += v[j];
                }
            }
        }
        if (lane == kWave - 1) st_dev(bp.counts + e, incl);  // the expert's total
    }
    wait_own_stores();
    __syncthreads();
    if (tid == 0) {
        s_last = atomicAdd(arrivals, 1) == (int)gridDim.x - 1;
        if (s_last) arrivals[0] = 0;  // every block has arrived: reset for the next call
    }
    __syncthreads();
    if (!s_last) return;  // uniform over the block
    const int cnt = tid < bp.E ? ld_dev(bp.counts + tid) : 0;
    write_tables(bp, cnt, s);
}

// T > 64, pass 3: per chunk, every pair goes to offset + chunk base + its stable rank.
__global__ __launch_bounds__(512) void bucket_scatter_kernel(BucketParams bp) {
    __shared__ BucketShared s;
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * bp.chunk_tokens;
    const int nt = min(bp.chunk_tokens, bp.T - t0);
    for (int i = tid; i < nt * kTopK; i += blockDim.x) s.ids[i] = bp.ids_in[(size_t)t0 * kTopK + i];
    __syncthreads();
    chunk_counts(s, nt * kTopK, bp.E);
    __syncthreads();
    chunk_scatter(s, nt * kTopK, bp.E, t0 * kTopK, bp.perm,
                  [&](int e) { return bp.offsets[e] + bp.hist[hist_at(bp, blockIdx.x, e)]; });
}

hipError_t launch_route_small(const SelectParams &sp, const BucketParams &bp, bool do_select,
                              bool do_bucket, hipStream_t s) {
    launch_k(route_small_kernel, 1, 1024, 0, s, sp, bp, do_select ? 1 : 0, do_bucket ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_route_fused(const RouterParams &rp, const SelectParams &sp,
                              const BucketParams &bp, bool do_bucket, int *arrivals, int dtype,
                              hipStream_t s) {
    const int grid = rp.n_tt * ((rp.R + kTile - 1) / kTile) * kQuarters;
    if (dtype == 1)
        launch_k(route_fused_kernel<OpBF16>, grid, 1024, 0, s, rp, sp, bp, do_bucket ? 1 : 0, arrivals);
    else
        launch_k(route_fused_kernel<OpF32>, grid, 1024, 0, s, rp, sp, bp, do_bucket ? 1 : 0, arrivals);
    return hipGetLastError();
}

hipError_t launch_route_tiles(const RouterParams &rp, const SelectParams &sp,
                              const BucketParams &bp, bool do_bucket, int *tile_arrivals,
                              int *tiles_done, int dtype, hipStream_t s) {
    const int grid = rp.n_tt * ((rp.R + kTile - 1) / kTile) * kQuarters;
    if (dtype == 1)
        launch_k(route_tiles_kernel<OpBF16>, grid, 1024, 0, s, rp, sp, bp, do_bucket ? 1 : 0,
                 tile_arrivals, tiles_done);
    else
        launch_k(route_tiles_kernel<OpF32>, grid, 1024, 0, s, rp, sp, bp, do_bucket ? 1 : 0,
                 tile_arrivals, tiles_done);
    return hipGetLastError();
}

hipError_t launch_select_hist(const SelectParams &sp, const BucketParams &bp, bool do_select,
                              bool do_hist, hipStream_t s) {
    const int T = do_select ? sp.T : bp.T;
    launch_k(select_hist_kernel, (T + bp.chunk_tokens - 1) / bp.chunk_tokens, 1024, 0, s, 
        sp, bp, do_select ? 1 : 0, do_hist ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_select_bucket(const SelectParams &sp, const BucketParams &bp, bool do_select,
                                int *arrivals, hipStream_t s) {
    if (bp.T > kSelBucketPairs / kTopK) return hipErrorInvalidValue;  // a caller bug
    const int grid = (bp.T + bp.chunk_tokens - 1) / bp.chunk_tokens;
    launch_k(select_bucket_kernel, grid, 1024, 0, s, sp, bp, do_select ? 1 : 0, arrivals);
    return hipGetLastError();
}

hipError_t launch_bucket_scan(const BucketParams &bp, int *arrivals, hipStream_t s) {
    if (bp.n_chunks <= kScanOneBlockChunks)  // the boundary and its measurements: kernels.h
        launch_k(bucket_scan_one_kernel, 1, 1024, 0, s, bp);
    else
        launch_k(bucket_scan_kernel, (bp.E + kScanWaves - 1) / kScanWaves, kScanWaves * kWave, 0, s,
                 bp, arrivals);
    return hipGetLastError();
}

hipError_t launch_bucket_scatter(const BucketParams &bp, hipStream_t s) {
    launch_k(bucket_scatter_kernel, bp.n_chunks, 512, 0, s, bp);
    return hipGetLastError();
}

}  // namespace moe
