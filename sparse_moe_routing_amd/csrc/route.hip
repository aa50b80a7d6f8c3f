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
// A lane sorts its (up to four) keys, then six xor-exchange levels (partners 1, 2, 4, 8, 16, 32)
// merge sorted runs of eight: keep the larger of a[i] and partner[7-i] (a bitonic sequence that
// holds the top eight of the sixteen) and sort it with three compare-exchange stages. That is
// the page's pairwise merge of sorted per-lane runs, widened from its 32-lane warp (five levels)
// to the 64-lane wavefront (six levels). After the last level every lane holds the same sorted
// top eight; lanes 0..7 decode one winner each and form the softmax over the eight chosen logits
// (reference point: the top logit), and the shared-expert gate is the sigmoid of score E.
//
// Bucketing is a stable counting sort of the T*8 (token, rank) pairs by expert id without
// atomics: per expert, one thread counts and then writes its pairs in pair order; exclusive
// scans give the offsets and the expert-group table that drives the expert kernel.
#include "device_common.h"
#include "kernels.h"

namespace moe {

__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t b = __float_as_uint(v);
    const uint32_t mag = b & 0x7fffffffu;
    if (mag > 0x7f800000u) return 0u;      // NaN: below every number
    if (mag == 0u) return 0x80000000u;     // -0 and +0 compare equal
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
    if (k == 0u) return __uint_as_float(0x7fc00000u);
    return (k & 0x80000000u) ? __uint_as_float(k & 0x7fffffffu) : __uint_as_float(~k);
}

__device__ __forceinline__ void cex(uint64_t &a, uint64_t &b) {  // a gets the larger key
    const uint64_t hi = a > b ? a : b;
    const uint64_t lo = a > b ? b : a;
    a = hi;
    b = lo;
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
    const int lo = __shfl_xor((int)(uint32_t)v, m, kWave);
    const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m, kWave);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Folded logit of score e of token t: partials summed in ks order, then the bias.
__device__ __forceinline__ float fold_logit(const SelectParams &p, int t, int e) {
    const size_t pstride = (size_t)p.T * p.R;
    const float *zp = p.zpart + (size_t)t * p.R + e;
    float v = zp[0];
    for (int ks = 1; ks < p.KS; ++ks) v += zp[ks * pstride];
    if (p.bias) v += p.bias[e];
    return v;
}

// Select the top eight of token t with the calling wave; lanes 0..7 write rank `lane`.
// ids_lds (nullable) receives the eight ids as well.
__device__ void select_token(const SelectParams &p, int t, int lane, int32_t *ids_lds) {
    uint64_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + kWave * j;
        if (e < p.E) {
            const float v = fold_logit(p, t, e);
            if (p.logits_out) p.logits_out[(size_t)t * p.R + e] = v;
            c[j] = ((uint64_t)order_key(v) << 32) | (uint32_t)~(uint32_t)e;
        } else {
            c[j] = 0;  // padding ranks below every real expert, NaN included
        }
    }
    // sort the lane's four keys, largest first
    cex(c[0], c[1]);
    cex(c[2], c[3]);
    cex(c[0], c[2]);
    cex(c[1], c[3]);
    cex(c[1], c[2]);
    uint64_t r[8] = {c[0], c[1], c[2], c[3], 0, 0, 0, 0};
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        uint64_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = shfl_xor64(r[i], m);
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = r[i] > o[7 - i] ? r[i] : o[7 - i];
#pragma unroll
        for (int i = 0; i < 4; ++i) cex(r[i], r[i + 4]);
        cex(r[0], r[2]);
        cex(r[1], r[3]);
        cex(r[4], r[6]);
        cex(r[5], r[7]);
        cex(r[0], r[1]);
        cex(r[2], r[3]);
        cex(r[4], r[5]);
        cex(r[6], r[7]);
    }
    uint64_t mine = r[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
        if (lane == i) mine = r[i];
    const float top = key_value((uint32_t)(r[0] >> 32));
    const float v = key_value((uint32_t)(mine >> 32));
    const float ex = expf(v - top);
    float sum = ex;
    sum += __shfl_xor(sum, 1, kWave);
    sum += __shfl_xor(sum, 2, kWave);
    sum += __shfl_xor(sum, 4, kWave);
    if (lane < kTopK) {
        const int id = (int)~(uint32_t)mine;
        p.ids[(size_t)t * kTopK + lane] = id;
        p.w[(size_t)t * kTopK + lane] = ex / sum;
        if (ids_lds) ids_lds[lane] = id;
    }
    if (p.g && lane == kTopK) {
        const float zg = fold_logit(p, t, p.E);
        if (p.logits_out) p.logits_out[(size_t)t * p.R + p.E] = zg;
        p.g[t] = 1.0f / (1.0f + expf(-zg));
    }
}

// Exclusive scan of one int per expert over threads 0..255 (every thread of the block calls it).
__device__ void scan256(int v, int *buf, int &excl, int &total) {
    const int tid = threadIdx.x;
    if (tid < 256) buf[tid] = v;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
        const int add = (tid < 256 && tid >= d) ? buf[tid - d] : 0;
        __syncthreads();
        if (tid < 256) buf[tid] += add;
        __syncthreads();
    }
    excl = (tid < 256 ? buf[tid] : 0) - v;
    total = buf[255];
    __syncthreads();
}

// Offsets, counts and the group table from per-expert totals (threads 0..E-1 own an expert).
__device__ void write_tables(const BucketParams &bp, int cnt, int *buf, int &off_out) {
    const int tid = threadIdx.x;
    const int e = tid;
    const bool own = e < bp.E;
    const int c = own ? cnt : 0;
    int off, total;
    scan256(c, buf, off, total);
    const int ng = own ? (c + bp.NG - 1) / bp.NG : 0;
    int gbase, gtotal;
    scan256(ng, buf, gbase, gtotal);
    const int nsh = bp.has_shared ? (bp.T + bp.NG - 1) / bp.NG : 0;
    if (own) {
        bp.counts[e] = c;
        bp.offsets[e] = off;
        for (int gg = 0; gg < ng; ++gg)
            bp.groups[nsh + gbase + gg] = make_int4(e, off + gg * bp.NG, min(bp.NG, c - gg * bp.NG), 0);
    }
    if (tid < nsh) bp.groups[tid] = make_int4(bp.E, tid * bp.NG, min(bp.NG, bp.T - tid * bp.NG), 0);
    if (tid == 0) {
        bp.offsets[bp.E] = total;
        bp.num_groups[0] = nsh + gtotal;
    }
    off_out = off;
}

__device__ __forceinline__ int count_in(const int32_t *ids, int n, int e) {
    int cnt = 0;
    for (int p = 0; p < n; ++p) cnt += (ids[p] == e);
    return cnt;
}

// T <= 64: selection and the whole bucketing pass in one block of 1024 threads (16 waves).
__global__ __launch_bounds__(1024) void route_small_kernel(SelectParams sp, BucketParams bp,
                                                          int do_select, int do_bucket) {
    __shared__ int32_t s_ids[64 * kTopK];
    __shared__ int s_buf[256];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int T = do_select ? sp.T : bp.T;
    if (do_select) {
        for (int t = wave; t < T; t += 16) select_token(sp, t, lane, s_ids + t * kTopK);
    } else {
        for (int i = tid; i < T * kTopK; i += blockDim.x) s_ids[i] = bp.ids_in[i];
    }
    if (!do_bucket) return;  // uniform over the block
    __syncthreads();
    const int n = T * kTopK;
    const int e = tid;
    const int cnt = e < bp.E ? count_in(s_ids, n, e) : 0;
    int off;
    write_tables(bp, cnt, s_buf, off);
    if (e < bp.E && cnt > 0) {
        int c = 0;
        for (int p = 0; p < n; ++p)
            if (s_ids[p] == e) bp.perm[off + c++] = p;
    }
}

// T > 64, pass 1: per 64-token chunk, selection (optional) and the per-expert histogram.
__global__ __launch_bounds__(1024) void select_hist_kernel(SelectParams sp, BucketParams bp,
                                                          int do_select, int do_hist) {
    __shared__ int32_t s_ids[64 * kTopK];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int T = do_select ? sp.T : bp.T;
    const int t0 = blockIdx.x * 64;
    const int nt = min(64, T - t0);
    if (do_select) {
        for (int i = wave; i < nt; i += 16) select_token(sp, t0 + i, lane, s_ids + i * kTopK);
    } else {
        for (int i = tid; i < nt * kTopK; i += blockDim.x) s_ids[i] = bp.ids_in[(size_t)t0 * kTopK + i];
    }
    if (!do_hist) return;
    __syncthreads();
    if (tid < bp.E) bp.hist[(size_t)blockIdx.x * bp.E + tid] = count_in(s_ids, nt * kTopK, tid);
}

// T > 64, pass 2 (one block): per-expert running bases over chunks, counts, offsets, groups.
__global__ __launch_bounds__(1024) void bucket_scan_kernel(BucketParams bp) {
    __shared__ int s_part[4][256];
    __shared__ int s_buf[256];
    const int tid = threadIdx.x;
    const int e = tid & 255, quarter = tid >> 8;
    const int per = (bp.n_chunks + 3) / 4;
    const int c0 = quarter * per, c1 = min(bp.n_chunks, c0 + per);
    int sum = 0;
    if (e < bp.E)
        for (int c = c0; c < c1; ++c) sum += bp.hist[(size_t)c * bp.E + e];
    s_part[quarter][e] = sum;
    __syncthreads();
    int base = 0;
    for (int qq = 0; qq < quarter; ++qq) base += s_part[qq][e];
    if (e < bp.E) {
        for (int c = c0; c < c1; ++c) {
            const int v = bp.hist[(size_t)c * bp.E + e];
            bp.hist[(size_t)c * bp.E + e] = base;
            base += v;
        }
    }
    const int cnt = (tid < 256) ? s_part[0][e] + s_part[1][e] + s_part[2][e] + s_part[3][e] : 0;
    int off;
    write_tables(bp, cnt, s_buf, off);
}

// T > 64, pass 3: per chunk, every expert writes its pairs at offset + chunk base, in pair order.
__global__ __launch_bounds__(256) void bucket_scatter_kernel(BucketParams bp) {
    __shared__ int32_t s_ids[64 * kTopK];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * 64;
    const int nt = min(64, bp.T - t0);
    for (int i = tid; i < nt * kTopK; i += blockDim.x) s_ids[i] = bp.ids_in[(size_t)t0 * kTopK + i];
    __syncthreads();
    const int e = tid;
    if (e >= bp.E) return;
    int dst = bp.offsets[e] + bp.hist[(size_t)blockIdx.x * bp.E + e];
    const int p0 = t0 * kTopK;
    for (int p = 0; p < nt * kTopK; ++p)
        if (s_ids[p] == e) bp.perm[dst++] = p0 + p;
}

hipError_t launch_route_small(const SelectParams &sp, const BucketParams &bp, bool do_select,
                              bool do_bucket, hipStream_t s) {
    route_small_kernel<<<1, 1024, 0, s>>>(sp, bp, do_select ? 1 : 0, do_bucket ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_select_hist(const SelectParams &sp, const BucketParams &bp, bool do_select,
                              bool do_hist, hipStream_t s) {
    const int T = do_select ? sp.T : bp.T;
    select_hist_kernel<<<(T + 63) / 64, 1024, 0, s>>>(sp, bp, do_select ? 1 : 0, do_hist ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_bucket_scan(const BucketParams &bp, hipStream_t s) {
    bucket_scan_kernel<<<1, 1024, 0, s>>>(bp);
    return hipGetLastError();
}

hipError_t launch_bucket_scatter(const BucketParams &bp, hipStream_t s) {
    bucket_scatter_kernel<<<bp.n_chunks, 256, 0, s>>>(bp);
    return hipGetLastError();
}

}  // namespace moe
