// select_core.h - per-token top-8 selection on one wave64 (device code shared by the kernels
// that select). The method and the key encoding are described in route.hip.
#pragma once

#include "router_core.h"

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

// The value of v held by this lane's partner at merge level L (0..5). The partners pair the two
// halves of every group of 2^(L+1) lanes: lane ^ 1 and lane ^ 2 (DPP quad permutations), the
// mirror lane within 8 and within 16 lanes (DPP half-row / row mirror), then the other row of a
// row pair and the other half of the wave (gfx950 permlane swaps). All of them are register-to-
// register moves: no LDS round trip. A permlane swap returns the lane's own value in one of its
// two results and the partner's in the other, so their xor with the own value is the partner's.
template <int L>
__device__ __forceinline__ uint32_t partner32(uint32_t v) {
    if constexpr (L == 0) return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);
    else if constexpr (L == 1) return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);
    else if constexpr (L == 2) return __builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false);
    else if constexpr (L == 3) return __builtin_amdgcn_update_dpp(0u, v, 0x140, 0xF, 0xF, false);
    else if constexpr (L == 4) {
        const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return s[0] ^ s[1] ^ v;
    } else {
        const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return s[0] ^ s[1] ^ v;
    }
}

template <int L>
__device__ __forceinline__ uint64_t partner64(uint64_t v) {
    const uint32_t lo = partner32<L>((uint32_t)v), hi = partner32<L>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// One merge level: r (sorted, largest first) becomes the sorted top eight of r and the partner's
// list: max(r[i], partner[7 - i]) is a bitonic sequence holding them, sorted by three stages.
template <int L>
__device__ __forceinline__ void merge_level(uint64_t (&r)[8]) {
    uint64_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = partner64<L>(r[i]);
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

// Select the top eight of token t with the calling wave; lanes 0..7 write rank `lane`.
// ids_lds (nullable) receives the eight ids as well.
// Folding: logit = (((p_0 + p_1) + ...) + p_{KS-1}) + bias, the partials in ks order. All
// partial loads are issued before the first add; loads past KS re-read partial KS-1 (in bounds)
// and are dropped by a select (KS <= 4). Offsets are 32-bit from a wave-uniform base.
// kDev: the partial logits are read device-coherently (written by other blocks of the same
// launch). The outputs are plain stores: they are read by later launches.
// Per-wave LDS scratch of select_token: up to 64 candidate keys, then the eight winners.
constexpr int kSelScratch = kWave + kTopK;

// Lower bound of the wave's 8th largest lane maximum (value halves): the smallest of the maxima
// of the eight groups of 8 lanes. Those are eight keys of distinct lanes, all >= the bound, so
// the 8th largest key is >= it too. Register-to-register lane moves only: maxima within 8 lanes
// (quad permutations, half-row mirror), then minima across the groups (row mirror, then the
// row-pair and half-wave swaps).
__device__ __forceinline__ uint32_t eighth_bound(uint32_t h) {
    h = max(h, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0xB1, 0xF, 0xF, false));
    h = max(h, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0x4E, 0xF, 0xF, false));
    h = max(h, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0x141, 0xF, 0xF, false));
    h = min(h, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0x140, 0xF, 0xF, false));
    h = min(h, partner32<4>(h));
    return min(h, partner32<5>(h));
}

// The eight largest keys of the wave (each lane holds four, sorted), largest first: lane i < 8
// gets the i-th in `mine`; `top` is the largest on every lane.
//
// Most keys cannot be among the eight, so the exact answer is taken from a short candidate list:
// let v8 be a lower bound of the 8th largest key's value half (eighth_bound); every one of the
// eight winners has a value half >= v8, so the keys reaching v8 - about twenty for untied logits -
// are candidates. They are packed into LDS; each one's rank is the number of candidates above it,
// and a candidate's rank among them is its rank among all keys (every key above a winner is a
// winner). With more than 64 candidates (heavy ties) the merge network runs instead.
__device__ __forceinline__ void top8_of_wave(const uint64_t (&c)[4], int lane, uint64_t *scr,
                                             uint64_t &mine, uint64_t &top) {
    const uint32_t v8 = eighth_bound((uint32_t)(c[0] >> 32));
    int n = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) n += (uint32_t)(c[j] >> 32) >= v8 ? 1 : 0;
    const uint64_t b0 = __ballot(n & 1), b1 = __ballot(n & 2), b2 = __ballot(n & 4);
    const int total = __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
    if (total <= kWave) {  // uniform
        const uint64_t below = (1ull << lane) - 1ull;
        const int off = __popcll(b0 & below) + 2 * __popcll(b1 & below) + 4 * __popcll(b2 & below);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j < n) scr[off + j] = c[j];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < total) {
            const uint64_t key = scr[lane];
            int rank = 0;
            for (int k = 0; k < total; ++k) rank += scr[k] > key ? 1 : 0;
            if (rank < kTopK) scr[kWave + rank] = key;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        mine = scr[kWave + (lane < kTopK ? lane : 0)];
        top = scr[kWave];
        return;
    }
    uint64_t r[8] = {c[0], c[1], c[2], c[3], 0, 0, 0, 0};
    merge_level<0>(r);
    merge_level<1>(r);
    merge_level<2>(r);
    merge_level<3>(r);
    merge_level<4>(r);
    merge_level<5>(r);
    mine = r[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
        if (lane == i) mine = r[i];
    top = r[0];
}

template <bool kDev = false>
__device__ inline void select_token(const SelectParams &p, int t, int lane, int32_t *ids_lds,
                                    uint64_t *scr) {
    constexpr int kMaxKS = kQuarters;
    const float *zt = p.zpart + (size_t)t * p.R;
    const int pstride = p.T * p.R;
    int eo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) eo[j] = min(lane + kWave * j, p.E - 1);
    float part[kMaxKS][4];
    float gpart[kMaxKS];
#pragma unroll
    for (int ks = 0; ks < kMaxKS; ++ks) {
        const int ko = (ks < p.KS ? ks : p.KS - 1) * pstride;
#pragma unroll
        for (int j = 0; j < 4; ++j) part[ks][j] = kDev ? ld_dev(zt + ko + eo[j]) : zt[ko + eo[j]];
        const int gi = ko + (p.g ? p.E : 0);
        gpart[ks] = kDev ? ld_dev(zt + gi) : zt[gi];
    }
    float bj[4] = {0.f, 0.f, 0.f, 0.f}, bg = 0.f;
    if (p.bias) {
#pragma unroll
        for (int j = 0; j < 4; ++j) bj[j] = p.bias[eo[j]];
        bg = p.g ? p.bias[p.E] : 0.f;
    }
    float zv[4], zg = gpart[0];
#pragma unroll
    for (int j = 0; j < 4; ++j) zv[j] = part[0][j];
#pragma unroll
    for (int ks = 1; ks < kMaxKS; ++ks) {
        const bool in = ks < p.KS;
#pragma unroll
        for (int j = 0; j < 4; ++j) zv[j] = in ? zv[j] + part[ks][j] : zv[j];
        zg = in ? zg + gpart[ks] : zg;
    }
    if (p.bias) {
#pragma unroll
        for (int j = 0; j < 4; ++j) zv[j] += bj[j];
        zg += bg;
    }

    uint64_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + kWave * j;
        if (e < p.E) {
            if (p.logits_out) p.logits_out[(size_t)t * p.R + e] = zv[j];
            c[j] = ((uint64_t)order_key(zv[j]) << 32) | (uint32_t)~(uint32_t)e;
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
    uint64_t mine, topkey;
    top8_of_wave(c, lane, scr, mine, topkey);
    const float top = key_value((uint32_t)(topkey >> 32));
    const float v = key_value((uint32_t)(mine >> 32));
    const float ex = expf(v - top);
    // the sum over lanes 0..7 (pairs, then quads, then the two quads of the half row): every
    // lane of the eight gets the same bits
    float sum = ex;
    sum += __uint_as_float(__builtin_amdgcn_update_dpp(0, __float_as_uint(sum), 0xB1, 0xF, 0xF, false));
    sum += __uint_as_float(__builtin_amdgcn_update_dpp(0, __float_as_uint(sum), 0x4E, 0xF, 0xF, false));
    sum += __uint_as_float(__builtin_amdgcn_update_dpp(0, __float_as_uint(sum), 0x141, 0xF, 0xF, false));
    if (lane < kTopK) {
        const int id = (int)~(uint32_t)mine;
        p.ids[(size_t)t * kTopK + lane] = id;
        p.w[(size_t)t * kTopK + lane] = ex / sum;
        if (ids_lds) ids_lds[lane] = id;
    }
    if (p.g && lane == kTopK) {
        if (p.logits_out) p.logits_out[(size_t)t * p.R + p.E] = zg;
        p.g[t] = 1.0f / (1.0f + expf(-zg));
    }
}

}  // namespace moe
