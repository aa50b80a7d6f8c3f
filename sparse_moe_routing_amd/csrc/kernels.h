// kernels.h - parameter blocks and host-side launchers of the libmoe kernels (internal).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Events the next launch records its own start and end in (the timed entry point sets them
// around each kernel; null otherwise). Kernel-own timestamps: no launch gap inside the interval.
extern thread_local hipEvent_t g_launch_start, g_launch_stop;

template <typename... KArgs, typename... Args>
inline void launch_k(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                     Args &&...args) {
    hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)lds, s, g_launch_start, g_launch_stop,
                          0u, KArgs(args)...);
}

// Router partial logits: zpart[ks][t][r] = sum over the ks-th K range of W[r][h] * x[t][h].
struct RouterParams {
    const void *x;       // [T][H]
    const void *w;       // [R][H]
    float *zpart;        // [KS][T][R]
    int T, H, R;
    int KS;              // K split: H / KS is a multiple of the op's k step
    int n_tt;            // token tiles of 16
    int n_rg;            // row-tile groups (each covers up to MAXRT row tiles of 16)
};

// Fold of the router partials + top-8 + softmax + gate (one wave per token).
struct SelectParams {
    const float *zpart;  // [KS][T][R] (KS = 1 for given logits)
    const float *bias;   // [R] or nullptr
    float *logits_out;   // [T][R] or nullptr
    int32_t *ids;        // [T][8]
    float *w;            // [T][8]
    float *g;            // [T] or nullptr when there is no gate row
    int T, E, R, KS;
};

// Dispatch tables written by the bucketing pass.
struct BucketParams {
    int T, E;
    int NG;              // tokens per expert group (rows of the expert kernel's x tile)
    int has_shared;      // shared-expert groups come first in the group table
    int chunk_tokens;    // tokens per chunk of the multi-block path (16; at most 64)
    int n_chunks;
    const int32_t *ids_in;  // [T][8] when the selection is not run in the same kernel
    int32_t *counts;     // [E]
    int32_t *offsets;    // [E+1]
    int32_t *perm;       // [T*8]
    int32_t *hist;       // the chunks' expert histograms (multi-block path), then per-chunk
                         // bases: [n_chunks][E], or [E][n_chunks] above kScanOneBlockChunks
                         // chunks (hist_at)
    int4 *groups;        // [max_groups]: {expert (E = shared), start, n, 0}
    int32_t *num_groups; // [1]
    int NG2;             // > 0: a second table of groups of up to NG2 tokens (same order)
    int4 *groups2;       // [max_groups for NG2]
    int32_t *num_groups2;  // [1]
};

// Chunk histograms: the one-block scan (up to this many chunks) reads a chunk's row of E counts
// with consecutive threads, so they are stored chunk-major; the multi-block scan gives each expert
// a wave that reads the expert's counts over all chunks, so above it they are stored
// expert-major (one contiguous run per expert instead of one cache line per chunk). Measured
// (bucket_scan, us, one block against the multi-block form): 32 chunks (T = 512) 4.2 vs 4.3,
// 48 chunks 4.9 vs 4.3, 64 chunks 4.9 vs 4.1, 257 chunks 15.1 vs 6.6; 512 chunks 13.9 (20.7 with
// the chunk-major columns).
constexpr int kScanOneBlockChunks = 32;
__host__ __device__ inline size_t hist_at(const BucketParams &bp, int chunk, int e) {
    return bp.n_chunks > kScanOneBlockChunks ? (size_t)e * bp.n_chunks + chunk
                                             : (size_t)chunk * bp.E + e;
}

// Expert stage: gate/up + SwiGLU + down for (group, slice chunk) units.
struct ExpertParams {
    const void *x;
    const void *gate_up, *down, *sgu, *sdn;
    const int32_t *perm;
    const int4 *groups;
    const int32_t *num_groups;
    float *ypart;        // [n_sc][slots][H]
    int T, H, E, I, Is;
    int s;               // slice width of I per wave group (16 * gate/up waves)
    int S;               // slices of max(I, Is)
    int SPU;             // slices per unit (S % SPU == 0); n_sc = S / SPU
    int NG;              // x-tile rows
    int slots;           // T*8 (+ T with a shared expert)
    int x_stride;        // LDS row stride of the x tile in elements
};

// Split expert stage (T <= 256): gate/up + SwiGLU into h, then down + weighted sum into y.
struct GateUpParams {
    const void *x;
    const void *gate_up, *sgu;
    const int32_t *perm;
    const int4 *groups;
    const int32_t *num_groups;
    void *h;             // bf16: planes hi, lo of [slots][Imax]; fp32: [slots][Imax]
    size_t plane;        // elements from the hi plane to the lo plane
    int T, H, E, I, Is, Imax;
    int S;               // 32-row slices of Imax (units per group)
    int NG, x_stride;
    const float *gu_scale, *sgu_scale;  // FP8 weights: per-row scales [E][2I], [2Is]; else null
    const uint8_t *gu_mx, *sgu_mx;      // MXFP4 weights: E8M0 bytes [E][2I][H/32], [2Is][H/32]
};

struct DownParams {
    const void *down, *sdn;
    const void *h;
    size_t plane;
    const int32_t *perm;
    const int4 *groups;
    const int32_t *num_groups;
    const float *w;      // [T][8]
    const float *g;      // [T] or nullptr
    float *ybuf;         // [slots][H]: weighted expert outputs per (token, rank) / shared slot
    float *y;            // [T][H]
    const int32_t *ids;  // [T][8] routing ids: a pair whose id is outside [0, E) adds nothing
    int *rb_arrivals;    // [H / 64] zero at entry; left zero
    int T, H, E, I, Is, Imax, NG;
    const float *dn_scale, *sdn_scale;  // FP8 weights: per-row scales [E][H], [H]; else null
    const uint8_t *dn_mx, *sdn_mx;      // MXFP4 weights: E8M0 bytes [E][H][I/32], [H][Is/32]
};

struct CombineParams {
    const float *ypart;  // [n_sc][slots][H]
    const float *w;      // [T][8]; nullptr: the partials already carry their weights
    const float *g;      // [T] or nullptr
    const int32_t *ids;  // [T][8] routing ids: a pair whose id is outside [0, E) adds nothing
    float *y;            // [T][H]
    int T, H, E, slots, n_sc_routed, n_sc_shared, has_shared;
};

hipError_t launch_router(const RouterParams &p, int dtype, int maxrt, hipStream_t s);
hipError_t launch_route_small(const SelectParams &sp, const BucketParams &bp, bool do_select,
                              bool do_bucket, hipStream_t s);
hipError_t launch_route_fused(const RouterParams &rp, const SelectParams &sp,
                              const BucketParams &bp, bool do_bucket, int *arrivals, int dtype,
                              hipStream_t s);
hipError_t launch_route_tiles(const RouterParams &rp, const SelectParams &sp,
                              const BucketParams &bp, bool do_bucket, int *tile_arrivals,
                              int *tiles_done, int dtype, hipStream_t s);
hipError_t launch_select_hist(const SelectParams &sp, const BucketParams &bp, bool do_select,
                              bool do_hist, hipStream_t s);
// T > 256: per-expert chunk bases and the tables; arrivals: a zeroed workspace state word, left
// zero
hipError_t launch_bucket_scan(const BucketParams &bp, int *arrivals, hipStream_t s);
// 64 < T <= 256: selection (optional) and the whole bucketing in one launch; arrivals: a zeroed
// workspace state word, left zero
hipError_t launch_select_bucket(const SelectParams &sp, const BucketParams &bp, bool do_select,
                                int *arrivals, hipStream_t s);
hipError_t launch_bucket_scatter(const BucketParams &bp, hipStream_t s);
hipError_t launch_expert(const ExpertParams &p, int dtype, int grid, size_t lds_bytes,
                         hipStream_t s);
hipError_t prepare_expert_kernels(size_t max_lds_bytes);
hipError_t launch_combine(const CombineParams &p, hipStream_t s);
hipError_t prepare_split_kernels(size_t gateup_lds, size_t down_lds);
hipError_t launch_gateup(const GateUpParams &p, int dtype, int grid, size_t lds, hipStream_t s);
size_t gateup_stage_bytes();  // LDS of gateup_kernel beyond its x tile
size_t down_stage_bytes();    // LDS of down_kernel beyond its h tile
hipError_t launch_down(const DownParams &p, int dtype, int grid, size_t lds, hipStream_t s);
hipError_t prepare_wide_kernels();
hipError_t launch_gateup_wide(const GateUpParams &p, int dtype, int grid, hipStream_t s);
hipError_t launch_down_wide(const DownParams &p, int dtype, int grid, hipStream_t s);
int wide_group_tokens();          // tokens per expert group of the wide kernels
int big_rows_per_gateup_unit();   // intermediate rows per gateup_big unit
hipError_t launch_gateup_big(const GateUpParams &p, int dtype, int grid, hipStream_t s);  // bf16 / FP8
int big_rows_per_down_unit();     // rows of y per down_big unit
hipError_t launch_down_big(const DownParams &p, int dtype, int grid, hipStream_t s);  // bf16 / FP8
// Expert-stationary gate/up for prefill-sized rounds (grouped.hip): bf16 / FP8 weights, tiles of
// up to grp_tile_tokens() tokens of one expert (the second group table).
int grp_tile_tokens();
int grp_rows_per_gateup_unit();
bool gateup_grp_supported(int H, int I, int Is, int dtype, long x_bytes);
hipError_t prepare_grouped_kernels();
hipError_t launch_gateup_grp(const GateUpParams &p, int dtype, int grid, hipStream_t s);
// its down product over the same tiles (bf16 / FP8 / MXFP4 down weights), rows of y per unit
bool down_grp_supported(int H, int I, int Is, int dtype, size_t h_bytes);
int grp_rows_per_down_unit();
hipError_t launch_down_grp(const DownParams &p, int dtype, int grid, hipStream_t s);
// Decode expert stage on the vector ALUs (gemv.hip): bf16 shapes gemv_supported accepts.
bool gemv_supported(int H, int I, int Is);
bool down_rows_supported(int H, int I, int Is);
int gemv_group_tokens();       // tokens per expert group of the vector-ALU gate/up kernel
int down_rows_group_tokens();  // tokens per expert group down_rows takes

size_t down_rows_lds(int slots);
hipError_t launch_gateup_gemv(const GateUpParams &p, int dtype, int grid, hipStream_t s);
hipError_t launch_down_rows(const DownParams &p, int dtype, hipStream_t s);  // 1 bf16, 2 FP8, 3 MXFP4
int wide_rows_per_down_unit();    // rows of y per down_wide unit
int wide_rows_per_gateup_unit();  // intermediate rows per gateup_wide unit

}  // namespace moe
