// moe_api.hip - the C ABI of libmoe (include/moe.h): validation, workspace layout, kernel plans.
//
// Call sequence of moe_forward (all on the caller's stream, no host synchronisation); which
// kernels a T gets is the plan (make_plan), with the boundaries measured on MI355X:
//   route_fused    T <= 16 from x: router partials; the last block selects and buckets
//   route_tiles    16 < T <= 64 from x: as route_fused per 16-token tile; the last tile buckets
//   route_small    T <= 64, routing given: the whole bucketing pass, one block
//   router         T > 64: partial logits (matrix cores; router.hip picks the per-wave, the
//                  LDS-staged or, from 3072 bf16 tokens, the block form)
//   select_bucket  64 < T <= 256: per 16-token chunk fold + top-8 + softmax + gate; the last
//                  chunk block buckets all pairs
//   select_hist    T > 256: the same per chunk, plus the chunk's expert histogram
//   bucket_scan    per-expert chunk bases, counts, offsets, the 64-token group table (and the
//                  320-token tile table for the expert-stationary kernels)
//   bucket_scatter the stable scatter of pair indices
//   gateup         T <= 64: gate/up + SwiGLU into h per (<= 8-token expert group, 32 inter.
//                  rows), matrix cores (gateup_gemv: the vector-ALU form, opt-in)
//   down_rows      T <= 64: vector-ALU down product per 8 rows of y over every group, the
//                  eight ranks and the gated shared slot summed into y in the block
//   down           T <= 64 shapes down_rows does not take: matrix-core down per (group, 64 rows
//                  of y); the last unit of each 64-row block sums the slots into y
//   gateup_wide    T > 64: as gateup for 64-token expert groups (wide.hip)
//   gateup_big     bf16 / FP8, 1536 <= T < 3584: 64-token groups, whole-line weight staging
//   gateup_grp     T >= 3584: expert-stationary, tiles of <= 320 tokens (grouped.hip)
//   down_wide / down_big / down_grp  T > 64: the down product into per-slot rows, on the
//                  64-token groups (down_big: bf16 / FP8 at T <= 256 and 1536 <= T < 7680) or
//                  on the tiles (down_grp: bf16 / FP8 from 7680, MXFP4 from 4608 tokens)
//   combine        T > 64: the weighted slot outputs of each token summed in rank order into y
//   expert         shapes outside the chunked kernels: fused gate/up + SwiGLU + down per (group,
//                  intermediate slice chunk), then combine
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "../../include/moe.h"
#include "kernels.h"

using namespace moe;

namespace moe {
thread_local hipEvent_t g_launch_start = nullptr, g_launch_stop = nullptr;
}

struct moe_ctx {
    moe_config cfg;
    moe_weights w;
    int R;         // router rows
    int device;
    int num_cus;
    int s;         // intermediate slice width of the expert kernel
    int gemv_max_tokens;  // decode rounds up to this T run the vector-ALU expert kernels
    int grp_min_tokens;   // rounds from this T run the expert-stationary gate/up (0: never)
    int down_grp_min_tokens;  // ... and, from this T (and with that gate/up), its down (0: never)
    void *scratch; // device address of the static scratch array on this context's device
};

// Workspace of moe_forward_noalloc: a static device array, one copy per GPU the library runs on,
// held until the process ends. Its name is only a host-side stand-in for the symbol: host code
// uses the device address hipGetSymbolAddress returns for it (resolved once per device), never
// the name itself.
constexpr size_t kScratchBytes = (size_t)8 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kMaxXTileBytes = 144 * 1024;  // LDS for the expert kernel's x tile
constexpr size_t kMaxLds = 160 * 1024;         // LDS per workgroup on gfx950
constexpr int kRouterSplit = 4;  // the quarters of router_core.h
// workspace state words (32-bit): route_fused's arrival counter, route_tiles' counter of
// finished tiles and its per-tile arrival counters (up to 16 tiles), then (from word 64) the
// down kernel's per-64-row-block arrival counters
constexpr int kStateRouteArrival = 0;
constexpr int kStateSelectArrival = 1;  // select_bucket's arrival counter
constexpr int kStateScanArrival = 2;    // bucket_scan's arrival counter
constexpr int kStateTilesDone = 4;
constexpr int kStateTileArrivals = 8;
constexpr int kStateRowBlocks = 64;
// route_tiles: up to 4 token tiles (512 pairs). Above, its 68 blocks per tile no longer fit the
// chip in one round and the chained kernels are faster (measured at T = 192).
constexpr int kTileRouteMaxTokens = 64;
// T > 64: tokens per selection / histogram block (one wave per token in a 1024-thread block)
constexpr int kHistChunk = 16;
// 64 < T <= 256: selection and bucketing in one launch (select_bucket)
constexpr int kSelBucketMaxTokens = 256;
constexpr int kSplitMaxTokens = 64;   // 8-token groups up to here, 64-token groups above
constexpr int kBigMinTokens = 1536;     // bf16 from here: gateup_big in place of gateup_wide
// bf16 / FP8 from here: gateup_grp (320-token tiles) in place of gateup_big; measured, gateup_grp
// against gateup_big: bf16 T = 3072 296 vs 286 us, 4096 299 vs 332, 6144 327 vs 433, 8192 349 vs
// 538; FP8 3072 293 vs 274, 4096 303 vs 330, 8192 399 vs 592
constexpr int kGrpMinTokens = 3584;
// its down product (down_grp) from these T, with that gate/up (below them the gate/up's tiles
// are followed by down_big, or by down_wide for MXFP4, on the 64-token groups); measured on one
// box, step us with down_grp against without: bf16 T = 4097 754 vs 704, 6144 920 vs 905, 7168
// 984 vs 991, 8192 1053 vs 1078; FP8 6144 927 vs 889, 7168 985 vs 972, 8192 1034 vs 1051;
// MXFP4 (against down_wide) 4097 803 vs 787, 5120 904 vs 917, 8192 1083 vs 1241
constexpr int kDownGrpMinTokens = 7680;
constexpr int kDownGrpMinTokensMx = 4608;


size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Device address of `scratch` on each device, resolved with that device current (moe_create).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int resolve_scratch(int dev, void **out) {
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// Zero fill of the first n 32-bit words at p (the state region of the static scratch; a kernel
// rather than a memset so that the call can be captured into a graph).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t *p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

struct Plan {
    int T = 0;
    bool small = false;
    int KS = 1, n_tt = 1, n_rg = 1, maxrt = 1;
    int NG = 16, n_chunks = 0, max_groups = 0;
    int s = 64, S = 1, SPU = 1, n_sc = 1, n_sc_routed = 1, n_sc_shared = 0, slots = 0;
    int x_stride = 0, grid = 1;
    size_t lds = 0;
    bool split = false;          // T <= 64: gateup + down kernels, 8-token groups
    bool wide = false;           // T > 64: gateup_wide + down_wide + combine, 64-token groups
    bool big = false;            // wide, bf16 or FP8, T >= kBigMinTokens: gateup_big for gateup_wide
    bool down_big = false;       // wide, bf16 or FP8, H a multiple of 512, T <= 256 or big
    bool gemv = false;           // split, bf16 activations: gateup_gemv in place of gateup
    bool down_rows = false;      // split, bf16 activations: down_rows in place of down
    bool grp = false;            // wide, bf16 / FP8 / MXFP4: gateup_grp for the gate/up kernel
    bool down_grp = false;       // with grp: down_grp over the same tiles
    int NG2 = 0, max_groups2 = 0, grp_grid = 0, down_grp_grid = 0;
    int Imax = 0, gu_grid = 1, down_grid = 1, gu_S = 1;
    size_t gu_lds = 0, down_lds = 0;
    size_t o_state = 0, o_zpart = 0, o_ids = 0, o_w = 0, o_g = 0, o_counts = 0, o_offsets = 0, o_perm = 0,
           o_hist = 0, o_groups = 0, o_ngroups = 0, o_groups2 = 0, o_ngroups2 = 0, o_ypart = 0,
           o_h = 0, total = 0;
};

// Activation (x, router) element type of a config: bf16 for FP8 expert weights.
int act_dtype(int dtype) { return dtype == MOE_F32 ? MOE_F32 : MOE_BF16; }
// Bytes of one activation element.
int elem_bytes(int dtype) { return act_dtype(dtype) == MOE_BF16 ? 2 : 4; }
// Kernel variant of the router and routing kernels (0 fp32, 1 bf16) and of the expert kernels
// (2: bf16 operands with FP8 E4M3 weights, 3: with MXFP4 weights).
int route_kdt(const moe_ctx *c);
int expert_kdt(const moe_ctx *c);

int max_groups_for(const moe_ctx *c, int T, int NG) {
    const int nsh = c->cfg.shared_inter > 0 ? (T + NG - 1) / NG : 0;
    const int pairs = T * 8;
    return nsh + (pairs < c->cfg.num_experts ? pairs : c->cfg.num_experts) + pairs / NG + 1;
}

// Leading state region of every workspace of the context (the same size for every T, so that a
// workspace reused across token counts keeps it zero): the route kernel's arrival counter, then
// one arrival counter per 64-row block of y for the down kernel.
size_t state_bytes(const moe_ctx *c) {
    return align_up((size_t)(kStateRowBlocks + c->cfg.hidden / 64) * 4);
}

// Rows of an expert group: up to 8 tokens, fewer when the x tile would not fit in LDS. The x tile
// is sized for a full group, so the cap sets the gate/up kernel's blocks per CU: measured at the
// decode shapes, 8 rows against 16: T = 16 125.6 vs 134.5 us per step, T = 32 186.2 vs 200.0,
// T = 64 254.0 vs 270.8 (4 and 6 rows within 1 % of 8 below T = 64, worse at 64).
// Rows are also capped so that the split kernels' LDS (the gate/up x tile plus its weight
// stage, the down h tile plus its stage) fits the workgroup limit at every hidden size: the
// quantized formats run only the chunked kernels, so their plan must never fall through to the
// fused fallback kernel.
int group_rows(const moe_ctx *c, int T) {
    const int esz = elem_bytes(c->cfg.dtype);
    const int x_stride = c->cfg.hidden + 16 / esz;
    const size_t xrow = (size_t)x_stride * esz;
    const int Imax = c->cfg.inter > c->cfg.shared_inter ? c->cfg.inter : c->cfg.shared_inter;
    const size_t hrow = (size_t)(Imax + 16 / esz) * esz * (esz == 2 ? 2 : 1);
    int NG = T < 8 ? T : 8;
    const int ng_x = (int)(kMaxXTileBytes / xrow);
    const int ng_gu = (int)((kMaxLds - gateup_stage_bytes()) / xrow);
    const int ng_dn = (int)((kMaxLds - down_stage_bytes()) / hrow);
    if (NG > ng_x) NG = ng_x;
    if (NG > ng_gu) NG = ng_gu;
    if (NG > ng_dn) NG = ng_dn;
    return NG;
}

Plan make_plan(const moe_ctx *c, int T) {
    Plan p;
    const moe_config &cfg = c->cfg;
    const int H = cfg.hidden, E = cfg.num_experts, I = cfg.inter, Is = cfg.shared_inter;
    p.T = T;
    p.small = T <= 64;
    const int n_rt = (c->R + 15) / 16;
    p.n_tt = (T + 15) / 16;
    // Router: four partial sums per logit for every T (the summation order is fixed, so a
    // token's logits do not depend on the batch it comes in).
    p.KS = kRouterSplit;
    p.maxrt = T > 256 ? 4 : 1;
    p.n_rg = (n_rt + p.maxrt - 1) / p.maxrt;
    // bucketing and expert groups
    // x-tile rows: up to 8 tokens, fewer when a row of H elements would not leave room in LDS
    const int esz = elem_bytes(cfg.dtype);
    p.x_stride = H + 16 / esz;
    // the split and wide kernels stream weight rows in chunks of 16 x 16 bytes (128 bf16 / 64 fp32)
    const int chunk = act_dtype(cfg.dtype) == MOE_BF16 ? 128 : 64;
    const bool chunk_ok = I % chunk == 0 && Is % chunk == 0;
    p.wide = T > kSplitMaxTokens && chunk_ok;
    // bf16 / FP8 / MXFP4 decode rounds (T <= 64) end with down_rows (vector-ALU down products of
    // the rows a block owns, combined in the block: no per-slot buffer, no arrival counters;
    // measured faster than the matrix-core down kernel at every T from 1 to 32), whose groups
    // hold at most 8 tokens; the vector-ALU gate/up kernel (groups of at most 4: the tokens' x
    // rows stay in registers) is used up to gemv_max_tokens (0 unless MOE_GEMV_MAX_TOKENS sets
    // it: the matrix-core gate/up kernel is as fast or faster from 3 tokens up, and one gate/up
    // kernel for every decode T keeps a token's bits independent of its batch)
    p.gemv = cfg.dtype != MOE_F32 && T <= c->gemv_max_tokens && gemv_supported(H, I, Is);
    p.down_rows = cfg.dtype != MOE_F32 && T <= kSplitMaxTokens && down_rows_supported(H, I, Is);
    int ng_x = group_rows(c, T);  // x-tile rows of the split and fused expert kernels
    if (p.gemv && ng_x > gemv_group_tokens()) ng_x = gemv_group_tokens();
    // down_rows groups: at most 4 tokens up to 16 (an 8-token x tile halves the matrix-core
    // gate/up kernel's blocks per CU: 2-4 us slower at T = 5..11), at most 8 above (a hot
    // expert's weights are then read once per 8 of its tokens: skewed T = 64 162 -> 152 us,
    // near-uniform T = 64 260 -> 255 us)
    const int dr_group = T <= 16 ? gemv_group_tokens() : down_rows_group_tokens();
    if (p.down_rows && ng_x > dr_group) ng_x = dr_group;
    p.NG = p.wide ? wide_group_tokens() : ng_x;
    p.n_chunks = p.small ? 0 : (T + kHistChunk - 1) / kHistChunk;
    const int pairs = T * 8;
    p.max_groups = max_groups_for(c, T, p.NG);
    p.s = c->s;
    const int Imax = I > Is ? I : Is;
    p.S = Imax / p.s;
    // Slices per unit: 1 (many small units) or all of them (one unit per group). Both sum the
    // per-slice partials of a token in the same order, so y does not depend on the choice.
    p.SPU = T <= 256 ? 1 : p.S;
    p.n_sc = p.S / p.SPU;
    p.n_sc_routed = (I / p.s + p.SPU - 1) / p.SPU;
    p.n_sc_shared = Is > 0 ? (Is / p.s + p.SPU - 1) / p.SPU : 0;
    p.slots = pairs + (Is > 0 ? T : 0);
    p.lds = (size_t)ng_x * p.x_stride * esz + (size_t)16 * (p.s + 4) * 4;
    p.Imax = Imax;
    p.gu_lds = (size_t)ng_x * p.x_stride * esz + gateup_stage_bytes();
    p.gu_S = Imax / 32;
    p.down_lds = (size_t)ng_x * (Imax + 16 / esz) * esz * (esz == 2 ? 2 : 1) +
                 down_stage_bytes();
    p.split = T <= kSplitMaxTokens && p.gu_lds <= kMaxLds && p.down_lds <= kMaxLds && chunk_ok;
    if (p.gemv) p.split = true;
    if (!p.split) p.gemv = p.down_rows = false;
    if (p.wide) {
        const int dr = wide_rows_per_down_unit(), gr = wide_rows_per_gateup_unit();
        const long d_units = (long)p.max_groups * ((H + dr - 1) / dr);
        const long g_units = (long)p.max_groups * (Imax / gr);
        const long cap = (long)c->num_cus * 4;
        p.down_grid = (int)(d_units < cap ? d_units : cap);
        p.gu_grid = (int)(g_units < cap ? g_units : cap);
        p.gu_S = Imax / gr;
        const bool big_dtype = cfg.dtype == MOE_BF16 || cfg.dtype == MOE_FP8_E4M3;
        p.big = big_dtype && T >= kBigMinTokens && Imax % big_rows_per_gateup_unit() == 0;
        if (p.big) {
            p.gu_S = Imax / big_rows_per_gateup_unit();
            const long b_units = (long)p.max_groups * p.gu_S;
            const long b_cap = (long)c->num_cus * 8;
            p.gu_grid = (int)(b_units < b_cap ? b_units : b_cap);
            if (p.gu_grid >= 8) p.gu_grid -= p.gu_grid % 8;  // whole rounds over the 8 XCDs
        }
        // expert-stationary gate/up: tiles of up to 256 tokens of one expert (a second group
        // table), 8 * ceil(units / 8) blocks of one unit each
        p.grp = c->grp_min_tokens > 0 && T >= c->grp_min_tokens &&
                gateup_grp_supported(H, I, Is, expert_kdt(c), (long)T * H * esz);
        if (p.grp) {
            p.NG2 = grp_tile_tokens();
            p.max_groups2 = max_groups_for(c, T, p.NG2);
            const long units = (long)p.max_groups2 * (Imax / grp_rows_per_gateup_unit());
            p.grp_grid = (int)((units + 7) / 8 * 8);
            p.big = false;
            const size_t h_bytes = (size_t)2 * (T * 8 + (Is > 0 ? T : 0)) * Imax * 2;
            p.down_grp = c->down_grp_min_tokens > 0 && T >= c->down_grp_min_tokens &&
                         down_grp_supported(H, I, Is, expert_kdt(c), h_bytes);
            const long d_units = (long)p.max_groups2 * (H / grp_rows_per_down_unit());
            p.down_grp_grid = (int)((d_units + 7) / 8 * 8);
        }
        // down_big with gateup_big and up to 256 tokens (measured: skewed T = 192 51.1 against
        // 53.8 us; T = 768 140.1 against 137.1 us for down_wide). The big pair from 1536 tokens:
        // T = 2048 step 527 against 611 us, T = 1024 430 against 403 us.
        p.down_big = big_dtype && H % big_rows_per_down_unit() == 0 &&
                     (T >= kBigMinTokens || T <= kSelBucketMaxTokens);
        if (p.down_big) {
            const long db_units = (long)p.max_groups * (H / big_rows_per_down_unit());
            const long db_cap = (long)c->num_cus * 4;
            p.down_grid = (int)(db_units < db_cap ? db_units : db_cap);
            if (p.down_grid >= 8) p.down_grid -= p.down_grid % 8;  // whole rounds over the 8 XCDs
        }
    } else {
        const long d_units = (long)p.max_groups * (H / 64);
        const long d_cap = (long)c->num_cus * 8;
        p.down_grid = (int)(d_units < d_cap ? d_units : d_cap);
        if (p.down_grid < 1) p.down_grid = 1;
    }
    if (!p.wide) {
        const long gu_units = (long)p.max_groups * (Imax / 32);
        const long gu_cap = (long)c->num_cus * 8;
        p.gu_grid = (int)(gu_units < gu_cap ? gu_units : gu_cap);
        if (p.gu_grid < 1) p.gu_grid = 1;
    }
    const long units = (long)p.max_groups * p.n_sc;
    const long cap = (long)c->num_cus * 4;
    p.grid = (int)(units < cap ? units : cap);
    if (p.grid < 1) p.grid = 1;
    // workspace
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    p.o_state = take(state_bytes(c));  // zero before the first call, left zero by every call
    p.o_zpart = take((size_t)p.KS * T * c->R * 4);
    p.o_ids = take((size_t)pairs * 4);
    p.o_w = take((size_t)pairs * 4);
    p.o_g = take((size_t)T * 4);
    p.o_counts = take((size_t)E * 4);
    p.o_offsets = take((size_t)(E + 1) * 4);
    p.o_perm = take((size_t)pairs * 4);
    p.o_hist = take((size_t)p.n_chunks * E * 4);
    p.o_groups = take((size_t)p.max_groups * 16);
    p.o_ngroups = take(16);
    p.o_groups2 = take((size_t)p.max_groups2 * 16);
    p.o_ngroups2 = take(p.grp ? 16 : 0);
    const bool per_slot = p.split || p.wide;  // [slots][H] weighted outputs and an h buffer
    p.o_ypart = take(p.down_rows ? 0 : per_slot ? (size_t)p.slots * H * 4
                                                : (size_t)p.n_sc * p.slots * H * 4);
    p.o_h = take(per_slot ? (size_t)p.slots * Imax * 4 : 0);
    p.total = o;
    return p;
}

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

int check_call(const moe_ctx *c, int32_t T, void *ws, size_t ws_bytes, const Plan *plan) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (T < 0 || T > c->cfg.max_tokens) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!ws || !aligned(ws, kAlign) || ws_bytes < plan->total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Kernel sequence of one call; `run` false only lists the names.
struct Launcher {
    const moe_ctx *c;
    hipStream_t stream;
    hipEvent_t *events;
    int n_events;
    bool run;
    int count = 0;
    const char **names = nullptr;
    int max_names = 0;
    hipError_t err = hipSuccess;

    // With events, kernel i records its own start in events[2i] and its end in events[2i + 1]
    // (timestamps taken by the dispatch itself, so a launch gap is not counted).
    template <class F>
    void step(const char *name, F &&launch) {
        if (names && count < max_names) names[count] = name;
        if (run && err == hipSuccess) {
            const bool timed = events && 2 * count + 1 < n_events;
            g_launch_start = timed ? events[2 * count] : nullptr;
            g_launch_stop = timed ? events[2 * count + 1] : nullptr;
            err = launch();
            g_launch_start = g_launch_stop = nullptr;
        }
        ++count;
    }
    void finish() {}
};

SelectParams select_params(const moe_ctx *c, const Plan &p, const float *zpart, int KS,
                           const float *bias, float *logits_out, int32_t *ids, float *w, float *g) {
    SelectParams sp{};
    sp.zpart = zpart;
    sp.bias = bias;
    sp.logits_out = logits_out;
    sp.ids = ids;
    sp.w = w;
    sp.g = c->cfg.shared_inter > 0 ? g : nullptr;
    sp.T = p.T;
    sp.E = c->cfg.num_experts;
    sp.R = c->R;
    sp.KS = KS;
    return sp;
}

BucketParams bucket_params(const moe_ctx *c, const Plan &p, char *ws, const int32_t *ids_in,
                           int32_t *counts, int32_t *offsets, int32_t *perm) {
    BucketParams bp{};
    bp.T = p.T;
    bp.E = c->cfg.num_experts;
    bp.NG = p.NG;
    bp.has_shared = c->cfg.shared_inter > 0;
    bp.chunk_tokens = kHistChunk;
    bp.n_chunks = p.n_chunks;
    bp.ids_in = ids_in;
    bp.counts = counts;
    bp.offsets = offsets;
    bp.perm = perm;
    bp.hist = reinterpret_cast<int32_t *>(ws + p.o_hist);
    bp.groups = reinterpret_cast<int4 *>(ws + p.o_groups);
    bp.num_groups = reinterpret_cast<int32_t *>(ws + p.o_ngroups);
    bp.NG2 = p.NG2;
    bp.groups2 = p.grp ? reinterpret_cast<int4 *>(ws + p.o_groups2) : nullptr;
    bp.num_groups2 = p.grp ? reinterpret_cast<int32_t *>(ws + p.o_ngroups2) : nullptr;
    return bp;
}

RouterParams router_params(const moe_ctx *c, const Plan &p, const void *x, float *zpart);

void enqueue_router(Launcher &L, const moe_ctx *c, const Plan &p, const void *x, float *zpart) {
    const RouterParams rp = router_params(c, p, x, zpart);
    L.step("router", [&] { return launch_router(rp, route_kdt(c), p.maxrt, L.stream); });
}

RouterParams router_params(const moe_ctx *c, const Plan &p, const void *x, float *zpart) {
    RouterParams rp{};
    rp.x = x;
    rp.w = c->w.router_w;
    rp.zpart = zpart;
    rp.T = p.T;
    rp.H = c->cfg.hidden;
    rp.R = c->R;
    rp.KS = p.KS;
    rp.n_tt = p.n_tt;
    rp.n_rg = p.n_rg;
    return rp;
}

// T <= 64 from x: router, selection and (optionally) bucketing in one launch - one token tile:
// route_fused (its last block selects and buckets); several tiles: route_tiles (the last block of
// each tile selects the tile, the last tile buckets).
void enqueue_route_fused(Launcher &L, const moe_ctx *c, const Plan &p, const void *x,
                         float *zpart, const SelectParams &sp, const BucketParams &bp,
                         bool do_bucket, char *ws) {
    const RouterParams rp = router_params(c, p, x, zpart);
    int *state = reinterpret_cast<int *>(ws + p.o_state);
    if (p.n_tt == 1) {
        L.step("route_fused", [&] {
            return launch_route_fused(rp, sp, bp, do_bucket, state + kStateRouteArrival,
                                      route_kdt(c), L.stream);
        });
    } else {
        L.step("route_tiles", [&] {
            return launch_route_tiles(rp, sp, bp, do_bucket, state + kStateTileArrivals,
                                      state + kStateTilesDone, route_kdt(c), L.stream);
        });
    }
}

// Bucketing from ids already in memory (or selection + bucketing when sp is given).
void enqueue_dispatch(Launcher &L, const Plan &p, const SelectParams *sp, BucketParams bp,
                      char *ws) {
    if (!p.small && p.T <= kSelBucketMaxTokens) {
        SelectParams dummy{};
        const SelectParams &s = sp ? *sp : dummy;
        int *arrivals = reinterpret_cast<int *>(ws + p.o_state) + kStateSelectArrival;
        L.step("select_bucket", [&] {
            return launch_select_bucket(s, bp, sp != nullptr, arrivals, L.stream);
        });
        return;
    }
    if (p.small) {
        SelectParams dummy{};
        const SelectParams &s = sp ? *sp : dummy;
        L.step("route_small", [&] { return launch_route_small(s, bp, sp != nullptr, true, L.stream); });
        return;
    }
    {
        SelectParams dummy{};
        const SelectParams &s = sp ? *sp : dummy;
        L.step("select_hist", [&] { return launch_select_hist(s, bp, sp != nullptr, true, L.stream); });
    }
    if (sp) bp.ids_in = sp->ids;
    int *scan_arrivals = reinterpret_cast<int *>(ws + p.o_state) + kStateScanArrival;
    L.step("bucket_scan", [&] { return launch_bucket_scan(bp, scan_arrivals, L.stream); });
    L.step("bucket_scatter", [&] { return launch_bucket_scatter(bp, L.stream); });
}

int forward_impl(const moe_ctx *c, const void *x, int32_t T, const int32_t *ids_in,
                 const float *w_in, const float *gate_in, float *y, void *workspace,
                 size_t ws_bytes, hipStream_t stream, hipEvent_t *events, int32_t n_events,
                 const char **names, int32_t max_names, int32_t *n_kernels, bool run,
                 int routing_given_flag, bool clear_state = false) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (T < 0 || T > c->cfg.max_tokens) return MOE_ERR_INVALID_ARG;
    const bool has_shared = c->cfg.shared_inter > 0;
    const bool given = run ? (ids_in || w_in || gate_in) : routing_given_flag != 0;
    if (run) {
        if (T == 0) return MOE_OK;
        if (!x || !y) return MOE_ERR_INVALID_ARG;
        if (!aligned(x, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
        if (given && (!ids_in || !w_in || (has_shared && !gate_in))) return MOE_ERR_INVALID_ARG;
    }
    if (T == 0) {
        if (n_kernels) *n_kernels = 0;
        return MOE_OK;
    }
    const Plan p = make_plan(c, T);
    if (run) {
        const int st = check_call(c, T, workspace, ws_bytes, &p);
        if (st != MOE_OK) return st;
        if (clear_state) {  // the arguments are valid: the state region starts at zero
            const int words = (int)(state_bytes(c) / 4);
            zero_words_kernel<<<1, 256, 0, stream>>>(static_cast<uint32_t *>(workspace), words);
            if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
        }
    }
    char *ws = static_cast<char *>(workspace);
    Launcher L{c, stream, events, n_events, run};
    L.names = names;
    L.max_names = max_names;

    int32_t *ids = reinterpret_cast<int32_t *>(ws + p.o_ids);
    float *wts = reinterpret_cast<float *>(ws + p.o_w);
    float *g = reinterpret_cast<float *>(ws + p.o_g);
    int32_t *counts = reinterpret_cast<int32_t *>(ws + p.o_counts);
    int32_t *offsets = reinterpret_cast<int32_t *>(ws + p.o_offsets);
    int32_t *perm = reinterpret_cast<int32_t *>(ws + p.o_perm);
    const int32_t *ids_used = ids;
    const float *w_used = wts;
    const float *g_used = g;
    if (!given) {
        float *zpart = reinterpret_cast<float *>(ws + p.o_zpart);
        const SelectParams sp = select_params(c, p, zpart, p.KS, c->w.router_bias, nullptr, ids,
                                              wts, g);
        const BucketParams bp = bucket_params(c, p, ws, nullptr, counts, offsets, perm);
        if (T <= kTileRouteMaxTokens) {
            enqueue_route_fused(L, c, p, x, zpart, sp, bp, true, ws);
        } else {
            enqueue_router(L, c, p, x, zpart);
            enqueue_dispatch(L, p, &sp, bp, ws);
        }
    } else {
        ids_used = ids_in;
        w_used = w_in;
        g_used = gate_in;
        enqueue_dispatch(L, p, nullptr, bucket_params(c, p, ws, ids_in, counts, offsets, perm), ws);
    }
    if (p.split || p.wide) {
        GateUpParams gp{};
        gp.x = x;
        gp.gate_up = c->w.gate_up;
        gp.sgu = c->w.shared_gate_up;
        gp.perm = perm;
        gp.groups = reinterpret_cast<const int4 *>(ws + p.o_groups);
        gp.num_groups = reinterpret_cast<const int32_t *>(ws + p.o_ngroups);
        gp.h = ws + p.o_h;
        gp.plane = (size_t)p.slots * p.Imax;
        gp.T = T;
        gp.H = c->cfg.hidden;
        gp.E = c->cfg.num_experts;
        gp.I = c->cfg.inter;
        gp.Is = c->cfg.shared_inter;
        gp.Imax = p.Imax;
        gp.S = p.gu_S;
        gp.NG = p.NG;
        gp.x_stride = p.x_stride;
        const bool mx = c->cfg.dtype == MOE_MXFP4;
        gp.gu_scale = mx ? nullptr : static_cast<const float *>(c->w.gate_up_scale);
        gp.sgu_scale = mx ? nullptr : static_cast<const float *>(c->w.shared_gate_up_scale);
        gp.gu_mx = mx ? static_cast<const uint8_t *>(c->w.gate_up_scale) : nullptr;
        gp.sgu_mx = mx ? static_cast<const uint8_t *>(c->w.shared_gate_up_scale) : nullptr;
        if (p.gemv)
            L.step("gateup_gemv", [&] { return launch_gateup_gemv(gp, expert_kdt(c), c->num_cus, L.stream); });
        else if (p.grp)
            L.step("gateup_grp", [&] {
                GateUpParams g2 = gp;
                g2.groups = reinterpret_cast<const int4 *>(ws + p.o_groups2);
                g2.num_groups = reinterpret_cast<const int32_t *>(ws + p.o_ngroups2);
                g2.S = p.Imax / grp_rows_per_gateup_unit();
                g2.NG = p.NG2;
                return launch_gateup_grp(g2, expert_kdt(c), p.grp_grid, L.stream);
            });
        else if (p.big)
            L.step("gateup_big", [&] { return launch_gateup_big(gp, expert_kdt(c), p.gu_grid, L.stream); });
        else if (p.wide)
            L.step("gateup_wide", [&] {
                return launch_gateup_wide(gp, expert_kdt(c), p.gu_grid, L.stream);
            });
        else
            L.step("gateup", [&] {
                return launch_gateup(gp, expert_kdt(c), p.gu_grid, p.gu_lds, L.stream);
            });
        DownParams dp{};
        dp.down = c->w.down;
        dp.sdn = c->w.shared_down;
        dp.h = gp.h;
        dp.plane = gp.plane;
        dp.perm = perm;
        dp.groups = gp.groups;
        dp.num_groups = gp.num_groups;
        dp.w = w_used;
        dp.g = has_shared ? g_used : nullptr;
        dp.ybuf = reinterpret_cast<float *>(ws + p.o_ypart);
        dp.y = y;
        dp.ids = ids_used;
        dp.rb_arrivals = reinterpret_cast<int *>(ws + p.o_state) + kStateRowBlocks;
        dp.NG = p.NG;
        dp.T = T;
        dp.H = c->cfg.hidden;
        dp.E = c->cfg.num_experts;
        dp.I = c->cfg.inter;
        dp.Is = c->cfg.shared_inter;
        dp.Imax = p.Imax;
        dp.dn_scale = mx ? nullptr : static_cast<const float *>(c->w.down_scale);
        dp.sdn_scale = mx ? nullptr : static_cast<const float *>(c->w.shared_down_scale);
        dp.dn_mx = mx ? static_cast<const uint8_t *>(c->w.down_scale) : nullptr;
        dp.sdn_mx = mx ? static_cast<const uint8_t *>(c->w.shared_down_scale) : nullptr;
        if (p.down_rows) {
            L.step("down_rows", [&] { return launch_down_rows(dp, expert_kdt(c), L.stream); });
            L.finish();
            if (n_kernels) *n_kernels = L.count;
            return hip_status(L.err);
        }
        if (p.down_grp) {
            L.step("down_grp", [&] {
                DownParams d2 = dp;
                d2.groups = reinterpret_cast<const int4 *>(ws + p.o_groups2);
                d2.num_groups = reinterpret_cast<const int32_t *>(ws + p.o_ngroups2);
                d2.NG = p.NG2;
                return launch_down_grp(d2, expert_kdt(c), p.down_grp_grid, L.stream);
            });
        } else if (p.down_big) {
            L.step("down_big", [&] { return launch_down_big(dp, expert_kdt(c), p.down_grid, L.stream); });
        } else if (p.wide) {
            L.step("down_wide", [&] {
                return launch_down_wide(dp, expert_kdt(c), p.down_grid, L.stream);
            });
        }
        if (p.wide) {
            CombineParams cp{};
            cp.ypart = dp.ybuf;
            cp.w = nullptr;  // the slot outputs already carry their routing weight / gate
            cp.g = nullptr;
            cp.ids = ids_used;
            cp.y = y;
            cp.T = T;
            cp.H = c->cfg.hidden;
            cp.E = c->cfg.num_experts;
            cp.slots = p.slots;
            cp.n_sc_routed = 1;
            cp.n_sc_shared = has_shared ? 1 : 0;
            cp.has_shared = has_shared ? 1 : 0;
            L.step("combine", [&] { return launch_combine(cp, L.stream); });
        } else {
            L.step("down", [&] {
                return launch_down(dp, expert_kdt(c), p.down_grid, p.down_lds, L.stream);
            });
        }
        L.finish();
        if (n_kernels) *n_kernels = L.count;
        return hip_status(L.err);
    }
    ExpertParams ep{};
    ep.x = x;
    ep.gate_up = c->w.gate_up;
    ep.down = c->w.down;
    ep.sgu = c->w.shared_gate_up;
    ep.sdn = c->w.shared_down;
    ep.perm = perm;
    ep.groups = reinterpret_cast<const int4 *>(ws + p.o_groups);
    ep.num_groups = reinterpret_cast<const int32_t *>(ws + p.o_ngroups);
    ep.ypart = reinterpret_cast<float *>(ws + p.o_ypart);
    ep.T = T;
    ep.H = c->cfg.hidden;
    ep.E = c->cfg.num_experts;
    ep.I = c->cfg.inter;
    ep.Is = c->cfg.shared_inter;
    ep.s = p.s;
    ep.S = p.S;
    ep.SPU = p.SPU;
    ep.NG = p.NG;
    ep.slots = p.slots;
    ep.x_stride = p.x_stride;
    L.step("expert", [&] { return launch_expert(ep, c->cfg.dtype, p.grid, p.lds, L.stream); });
    CombineParams cp{};
    cp.ypart = ep.ypart;
    cp.w = w_used;
    cp.g = has_shared ? g_used : nullptr;
    cp.ids = ids_used;
    cp.y = y;
    cp.T = T;
    cp.H = c->cfg.hidden;
    cp.E = c->cfg.num_experts;
    cp.slots = p.slots;
    cp.n_sc_routed = p.n_sc_routed;
    cp.n_sc_shared = p.n_sc_shared;
    cp.has_shared = has_shared ? 1 : 0;
    L.step("combine", [&] { return launch_combine(cp, L.stream); });
    L.finish();
    if (n_kernels) *n_kernels = L.count;
    return hip_status(L.err);
}

bool valid_inter(int v, int dtype) {
    // FP8 weights run only the chunked expert kernels: 128-element weight-row chunks; MXFP4
    // weights stream chunk pairs (256 weights, 128 bytes of codes per row)
    const int m = dtype == MOE_MXFP4 ? 256 : dtype == MOE_FP8_E4M3 ? 128 : dtype == MOE_BF16 ? 32 : 16;
    return v >= m && v <= 4096 && v % m == 0;
}

int route_kdt(const moe_ctx *c) { return act_dtype(c->cfg.dtype) == MOE_BF16 ? 1 : 0; }
int expert_kdt(const moe_ctx *c) {
    return c->cfg.dtype == MOE_MXFP4 ? 3 : c->cfg.dtype == MOE_FP8_E4M3 ? 2
                                         : c->cfg.dtype == MOE_BF16 ? 1 : 0;
}

// The kernels' dynamic-LDS caps (hipFuncAttributeMaxDynamicSharedMemorySize) are process-wide:
// they only ever grow, to the largest any context has needed, so that creating a context never
// lowers a cap another context's launches rely on.
std::mutex g_lds_mu;
size_t g_split_gu_lds, g_split_down_lds, g_expert_lds;
bool g_wide_ready;

hipError_t raise_lds_caps(const moe_ctx *c, const Plan &p_max) {
    std::lock_guard<std::mutex> lock(g_lds_mu);
    hipError_t err = hipSuccess;
    size_t gu = 0, dn = 0;
    const int tmax = c->cfg.max_tokens < kSplitMaxTokens ? c->cfg.max_tokens : kSplitMaxTokens;
    for (int T : {1, 4, 8, tmax}) {  // the decode plans' LDS needs grow with T up to 8 tokens
        if (T > tmax) continue;
        const Plan q = make_plan(c, T);
        if (q.split) {
            gu = q.gu_lds > gu ? q.gu_lds : gu;
            dn = q.down_lds > dn ? q.down_lds : dn;
        }
    }
    if (gu > g_split_gu_lds || dn > g_split_down_lds) {
        const size_t ngu = gu > g_split_gu_lds ? gu : g_split_gu_lds;
        const size_t ndn = dn > g_split_down_lds ? dn : g_split_down_lds;
        if ((err = prepare_split_kernels(ngu, ndn)) != hipSuccess) return err;
        g_split_gu_lds = ngu;
        g_split_down_lds = ndn;
    }
    if (p_max.lds > g_expert_lds) {
        if ((err = prepare_expert_kernels(p_max.lds)) != hipSuccess) return err;
        g_expert_lds = p_max.lds;
    }
    if (!g_wide_ready) {
        if ((err = prepare_wide_kernels()) != hipSuccess) return err;
        if ((err = prepare_grouped_kernels()) != hipSuccess) return err;
        g_wide_ready = true;
    }
    return hipSuccess;
}

}  // namespace

extern "C" {

const char *moe_status_str(int status) {
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or parameter";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int moe_create(const moe_config *cfg, const moe_weights *weights, moe_ctx **out) {
    if (!out) return MOE_ERR_INVALID_ARG;
    *out = nullptr;
    if (!cfg || !weights) return MOE_ERR_INVALID_ARG;
    if (cfg->dtype != MOE_F32 && cfg->dtype != MOE_BF16 && cfg->dtype != MOE_FP8_E4M3 &&
        cfg->dtype != MOE_MXFP4)
        return MOE_ERR_INVALID_ARG;
    if (cfg->top_k != 8) return MOE_ERR_UNSUPPORTED;
    if (cfg->num_experts < 8 || cfg->num_experts > 256) return MOE_ERR_UNSUPPORTED;
    if (cfg->hidden < 64 || cfg->hidden > 16384 || cfg->hidden % 64) return MOE_ERR_UNSUPPORTED;
    if (cfg->dtype != MOE_F32 && cfg->hidden % 128) return MOE_ERR_UNSUPPORTED;
    if (cfg->dtype == MOE_MXFP4 && cfg->hidden % 256) return MOE_ERR_UNSUPPORTED;
    if (!valid_inter(cfg->inter, cfg->dtype)) return MOE_ERR_UNSUPPORTED;
    if (cfg->shared_inter != 0 && !valid_inter(cfg->shared_inter, cfg->dtype))
        return MOE_ERR_UNSUPPORTED;
    if (cfg->max_tokens < 1) return MOE_ERR_INVALID_ARG;
    if (cfg->max_tokens > 65536) return MOE_ERR_UNSUPPORTED;
    if (!weights->router_w || !weights->gate_up || !weights->down) return MOE_ERR_INVALID_ARG;
    const bool has_shared = cfg->shared_inter > 0;
    if (has_shared != (weights->shared_gate_up != nullptr) ||
        has_shared != (weights->shared_down != nullptr))
        return MOE_ERR_INVALID_ARG;
    const void *ptrs[] = {weights->router_w, weights->gate_up, weights->down,
                          weights->shared_gate_up, weights->shared_down};
    for (const void *ptr : ptrs)
        if (ptr && !aligned(ptr, 16)) return MOE_ERR_INVALID_ARG;
    if (weights->router_bias && !aligned(weights->router_bias, 4)) return MOE_ERR_INVALID_ARG;
    // scales: all present with quantized weights (FP8 row scales 16-byte aligned; MXFP4 scale
    // bytes at any address), all absent otherwise
    const void *scales[] = {weights->gate_up_scale, weights->down_scale,
                            weights->shared_gate_up_scale, weights->shared_down_scale};
    const bool fp8 = cfg->dtype == MOE_FP8_E4M3;
    const bool quant = fp8 || cfg->dtype == MOE_MXFP4;
    for (int i = 0; i < 4; ++i) {
        const bool need = quant && (i < 2 || has_shared);
        if (need != (scales[i] != nullptr)) return MOE_ERR_INVALID_ARG;
        if (fp8 && scales[i] && !aligned(scales[i], 16)) return MOE_ERR_INVALID_ARG;
    }

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_ERR_UNSUPPORTED;

    moe_ctx *c = new (std::nothrow) moe_ctx;
    if (!c) return MOE_ERR_HIP;
    c->cfg = *cfg;
    c->w = *weights;
    c->R = cfg->num_experts + (has_shared ? 1 : 0);
    c->device = dev;
    c->num_cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
    c->gemv_max_tokens = 0;
    if (const char *env = getenv("MOE_GEMV_MAX_TOKENS")) {
        char *end = nullptr;
        const long v = strtol(env, &end, 10);
        if (end == env || *end != '\0' || v < 0 || v > kSplitMaxTokens) {
            delete c;
            return MOE_ERR_INVALID_ARG;
        }
        c->gemv_max_tokens = (int)v;
    }
    c->grp_min_tokens = kGrpMinTokens;
    if (const char *env = getenv("MOE_GRP_MIN_TOKENS")) {  // 0: never
        char *end = nullptr;
        const long v = strtol(env, &end, 10);
        if (end == env || *end != '\0' || v < 0 || (v > 0 && v <= kSplitMaxTokens) || v > (1L << 30)) {
            delete c;
            return MOE_ERR_INVALID_ARG;
        }
        c->grp_min_tokens = (int)v;
    }
    c->down_grp_min_tokens = cfg->dtype == MOE_MXFP4 ? kDownGrpMinTokensMx : kDownGrpMinTokens;
    if (const char *env = getenv("MOE_DOWN_GRP_MIN_TOKENS")) {  // 0: never
        char *end = nullptr;
        const long v = strtol(env, &end, 10);
        if (end == env || *end != '\0' || v < 0 || (v > 0 && v <= kSplitMaxTokens) || v > (1L << 30)) {
            delete c;
            return MOE_ERR_INVALID_ARG;
        }
        c->down_grp_min_tokens = (int)v;
    }
    const int Is = cfg->shared_inter;
    c->s = (cfg->inter % 64 == 0 && Is % 64 == 0) ? 64 : (cfg->inter % 32 == 0 && Is % 32 == 0) ? 32 : 16;
    // largest LDS any plan of this context asks for (x tile of up to 16 rows + h tile)
    const Plan p = make_plan(c, cfg->max_tokens);
    if (p.NG < 1 || p.lds > kMaxLds) {
        delete c;
        return MOE_ERR_UNSUPPORTED;
    }
    // The quantized formats have no fused fallback kernel: every token count the context takes
    // must plan the chunked kernels (8-token groups up to 64 tokens, 64-token groups above).
    if (quant) {
        const int t_small = cfg->max_tokens < kSplitMaxTokens ? cfg->max_tokens : kSplitMaxTokens;
        const bool small_ok = make_plan(c, t_small).split && make_plan(c, 1).split;
        const bool wide_ok = cfg->max_tokens <= kSplitMaxTokens || p.wide;
        if (!small_ok || !wide_ok) {
            delete c;
            return MOE_ERR_UNSUPPORTED;
        }
    }
    if (resolve_scratch(dev, &c->scratch) != MOE_OK) {
        delete c;
        return MOE_ERR_HIP;
    }
    if (raise_lds_caps(c, p) != hipSuccess) {
        delete c;
        return MOE_ERR_HIP;
    }
    *out = c;
    return MOE_OK;
}

void moe_destroy(moe_ctx *ctx) { delete ctx; }

size_t moe_workspace_bytes(const moe_ctx *ctx, int32_t T) {
    if (!ctx || T <= 0 || T > ctx->cfg.max_tokens) return 0;
    // the plans' needs grow with T inside each regime; should the decode regime's largest ever
    // exceed the next regime's smallest, the larger of the two keeps the size monotone in T
    const size_t need = make_plan(ctx, T).total;
    const size_t decode = make_plan(ctx, T < kSplitMaxTokens ? T : kSplitMaxTokens).total;
    return need > decode ? need : decode;
}

size_t moe_workspace_state_bytes(const moe_ctx *ctx) { return ctx ? state_bytes(ctx) : 0; }

int moe_route(const moe_ctx *c, const void *x, const float *logits_in, int32_t T,
              float *logits_out, int32_t *topk_ids, float *topk_w, float *shared_gate,
              void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (T < 0 || T > c->cfg.max_tokens) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if ((x == nullptr) == (logits_in == nullptr)) return MOE_ERR_INVALID_ARG;
    if (!topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
    if (c->cfg.shared_inter > 0 && !shared_gate) return MOE_ERR_INVALID_ARG;
    if (x && !aligned(x, 16)) return MOE_ERR_INVALID_ARG;
    const Plan p = make_plan(c, T);
    const int st = check_call(c, T, workspace, ws_bytes, &p);
    if (st != MOE_OK) return st;
    char *ws = static_cast<char *>(workspace);
    Launcher L{c, stream, nullptr, 0, true};
    const float *zpart = logits_in;
    int KS = 1;
    const float *bias = nullptr;
    float *zp = reinterpret_cast<float *>(ws + p.o_zpart);
    if (x) {
        zpart = zp;
        KS = p.KS;
        bias = c->w.router_bias;
    }
    const SelectParams sp = select_params(c, p, zpart, KS, bias, logits_out, topk_ids, topk_w,
                                          shared_gate);
    BucketParams bp = bucket_params(c, p, ws, nullptr, nullptr, nullptr, nullptr);
    if (x && T <= kTileRouteMaxTokens) {
        enqueue_route_fused(L, c, p, x, zp, sp, bp, false, ws);
    } else {
        if (x) enqueue_router(L, c, p, x, zp);
        if (p.small)
            L.step("route_small", [&] { return launch_route_small(sp, bp, true, false, stream); });
        else
            L.step("select_hist", [&] { return launch_select_hist(sp, bp, true, false, stream); });
    }
    return hip_status(L.err);
}

int moe_bucket(const moe_ctx *c, const int32_t *ids_in, int32_t T, int32_t *counts,
               int32_t *offsets, int32_t *perm, void *workspace, size_t ws_bytes,
               hipStream_t stream) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (T < 0 || T > c->cfg.max_tokens) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!ids_in || !counts || !offsets || !perm) return MOE_ERR_INVALID_ARG;
    const Plan p = make_plan(c, T);
    const int st = check_call(c, T, workspace, ws_bytes, &p);
    if (st != MOE_OK) return st;
    Launcher L{c, stream, nullptr, 0, true};
    char *ws = static_cast<char *>(workspace);
    enqueue_dispatch(L, p, nullptr, bucket_params(c, p, ws, ids_in, counts, offsets, perm), ws);
    return hip_status(L.err);
}

int moe_forward(const moe_ctx *c, const void *x, int32_t T, const int32_t *ids_in,
                const float *w_in, const float *gate_in, float *y, void *workspace,
                size_t ws_bytes, hipStream_t stream) {
    return forward_impl(c, x, T, ids_in, w_in, gate_in, y, workspace, ws_bytes, stream, nullptr,
                        0, nullptr, 0, nullptr, true, 0);
}

int moe_forward_noalloc(const moe_ctx *c, const void *x, int32_t T, const int32_t *ids_in,
                        const float *w_in, const float *gate_in, float *y, hipStream_t stream) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (T < 0 || T > c->cfg.max_tokens) return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!c->scratch) return MOE_ERR_HIP;
    // the scratch must hold this call's workspace (forward_impl checks the call's own plan too)
    if (moe_workspace_bytes(c, T) > kScratchBytes) return MOE_ERR_WORKSPACE;
    return forward_impl(c, x, T, ids_in, w_in, gate_in, y, c->scratch, kScratchBytes, stream,
                        nullptr, 0, nullptr, 0, nullptr, true, 0, true);
}

int moe_forward_timed(const moe_ctx *c, const void *x, int32_t T, const int32_t *ids_in,
                      const float *w_in, const float *gate_in, float *y, void *workspace,
                      size_t ws_bytes, hipStream_t stream, hipEvent_t *events,
                      int32_t n_events) {
    if (!events || n_events < 2) return MOE_ERR_INVALID_ARG;
    int32_t n = 0;
    const int given = (ids_in || w_in || gate_in) ? 1 : 0;
    int st = forward_impl(c, x, T, ids_in, w_in, gate_in, y, workspace, ws_bytes, stream, nullptr,
                          0, nullptr, 0, &n, false, given);
    if (st != MOE_OK) return st;
    if (n_events != 2 * n) return MOE_ERR_INVALID_ARG;
    return forward_impl(c, x, T, ids_in, w_in, gate_in, y, workspace, ws_bytes, stream, events,
                        n_events, nullptr, 0, nullptr, true, 0);
}

int moe_forward_plan(const moe_ctx *c, int32_t T, int32_t routing_given, int32_t *n_kernels,
                     const char **names, int32_t max_names) {
    if (!c || !n_kernels) return MOE_ERR_INVALID_ARG;
    if (T < 0 || T > c->cfg.max_tokens) return MOE_ERR_INVALID_ARG;
    return forward_impl(c, nullptr, T, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr,
                        nullptr, 0, names, max_names, n_kernels, false, routing_given);
}

}  // extern "C"
