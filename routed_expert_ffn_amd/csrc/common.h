// common.h -- device helpers shared by the gfx950 kernels of libmoe.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;

// ------------------------------------------------------------------ bf16 / fp16 bits
MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
MOE_DEV float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
MOE_DEV float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
MOE_DEV uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

// IEEE binary16 bits -> fp32 (exact).
MOE_DEV float fp16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// A block barrier that orders LDS accesses only: the waves' outstanding global
// loads stay in flight across it (__syncthreads' workgroup release would wait
// for them, e.g. for a weight prefetch issued just before).  Use it where
// only LDS data is exchanged between the waves of a block.
MOE_DEV void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------------ wave helpers
MOE_DEV int lane_id() { return __lane_id(); }

template <typename T>
MOE_DEV T wave_xor(T v, int m) { return __shfl_xor(v, m, WAVE); }

// inclusive prefix sum over the 64 lanes
MOE_DEV int wave_incl_scan(int v) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
        int o = __shfl_up(v, d, WAVE);
        if (l >= d) v += o;
    }
    return v;
}
MOE_DEV int wave_sum(int v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, WAVE);
    return v;
}

// (value, index) key order used for routing: larger value first, then lower index.
MOE_DEV bool key_better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Wave-wide best (value, index) under key_better.  Invalid entries carry ia = INT_MAX.
MOE_DEV void wave_best(float& v, int& i) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        float ov = __shfl_xor(v, d, WAVE);
        int oi = __shfl_xor(i, d, WAVE);
        if (key_better(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

// Routing order as one 64-bit key: larger value first, then lower index.
// The float maps to an order-preserving unsigned (-0 and +0 compare equal, as
// in IEEE comparison); the low word is the complemented index.
MOE_DEV uint32_t f32_order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
MOE_DEV unsigned long long route_key(float v, int idx) {
    return ((unsigned long long)f32_order_key(v) << 32) | (uint32_t)(~(uint32_t)idx);
}
MOE_DEV int route_key_index(unsigned long long k) { return (int)(~(uint32_t)k); }
MOE_DEV float route_key_value(unsigned long long k) {
    const uint32_t h = (uint32_t)(k >> 32);
    return __uint_as_float((h & 0x80000000u) ? (h & 0x7FFFFFFFu) : ~h);
}
MOE_DEV unsigned long long wave_max_u64(unsigned long long k) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const unsigned long long o = __shfl_xor(k, d, WAVE);
        k = o > k ? o : k;
    }
    return k;
}

// Wave-wide maximum of a u32, returned wave-uniform: DPP maxima within each
// row of 16 lanes (quad swaps, half-row and row mirrors), then row 0 into row
// 1 and row 2 into row 3 (row_bcast:15), then rows 0-1 into rows 2-3
// (row_bcast:31), so lane 63 holds the maximum; 0 (the identity) is the value
// of lanes a step does not write, so each step is one DPP max.
MOE_DEV uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));   // row_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));   // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));   // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Softmax weights of a wave's selection (lane k < K holds the k-th largest
// value v): exp(v - v_0) / sum_k exp(v_k - v_0), the sum taken in rank order
// (k = 0, 1, ...) from register reads, the same value in every lane.
MOE_DEV float selection_weight(float v, int K) {
    const int l = lane_id();
    const float v0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float ex = l < K ? expf(v - v0) : 0.0f;
    float sum = 0.0f;
    for (int k = 0; k < K; k++) sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), k));
    return ex / sum;
}

MOE_DEV float order_key_value(uint32_t h) { return __uint_as_float((h & 0x80000000u) ? (h & 0x7FFFFFFFu) : ~h); }

// The order keys of a row of E logits, kv[j] for expert lane + 64 j (0 past
// E).  Every load is unconditional (past E they re-read the last logit) so
// all VPL are in flight together: a guarded load would wait for each in turn.
template <int VPL>
MOE_DEV void load_order_keys(const float* __restrict__ row, int E, uint32_t (&kv)[VPL]) {
    const int l = lane_id();
    float v[VPL];
#pragma unroll
    for (int j = 0; j < VPL; j++) v[j] = row[min(l + j * WAVE, E - 1)];
#pragma unroll
    for (int j = 0; j < VPL; j++) kv[j] = l + j * WAVE < E ? f32_order_key(v[j]) : 0u;
}

// Top-`rounds` under (value desc, expert asc) of the order keys kv[j] of expert
// e = lane + 64 j (0 = absent; every finite or infinite logit has a key > 0):
// lane r < rounds receives round r's key and expert.  Per round: the lane
// maxima, their wave maximum M, and the lowest expert holding M (lowest j,
// then lowest lane, by ballot), which is then cleared.
template <int VPL>
MOE_DEV void select_top(uint32_t (&kv)[VPL], int rounds, uint32_t& my_key, int& my_e) {
    const int l = lane_id();
    my_key = 0;
    my_e = 0;
    for (int r = 0; r < rounds; r++) {
        uint32_t m = kv[0];
#pragma unroll
        for (int j = 1; j < VPL; j++) m = max(m, kv[j]);
        const uint32_t M = wave_max_u32(m);
        // the lowest expert holding M: the lowest j whose ballot is not empty,
        // its lowest lane (scalar selects, no branches)
        int win = 0x7fffffff;
#pragma unroll
        for (int j = VPL - 1; j >= 0; j--) {
            const unsigned long long bm = __ballot(kv[j] == M);
            win = bm ? (__ffsll((long long)bm) - 1) + j * WAVE : win;
        }
#pragma unroll
        for (int j = 0; j < VPL; j++) kv[j] = (l + j * WAVE == win) ? 0u : kv[j];
        if (l == r) {
            my_key = M;
            my_e = win;
        }
    }
}

// select_top's result (lane r < K: rank r's key and expert) by a cut, for
// latency: tau = the K-th largest of the 64 lane maxima (one lane per round,
// single values), then every key >= tau is a candidate -- the K lanes with
// the largest maxima hold K keys >= tau, so the K-th largest key is >= tau
// and the whole top K is among the candidates -- and each candidate's rank is
// the number of candidates ahead of it under (key desc, expert asc).  cand
// (64 entries) and outb (K entries) are the wave's LDS scratch.  Returns
// false, touching nothing the caller uses, when more than 64 keys reach tau
// (ties at the cut); then select_top gives the answer.  K <= 64.
template <int VPL>
MOE_DEV bool select_top_cut(const uint32_t (&kv)[VPL], int K, uint2* __restrict__ cand, uint2* __restrict__ outb,
                            uint32_t& my_key, int& my_e) {
    const int l = lane_id();
    uint32_t mm = kv[0];
#pragma unroll
    for (int j = 1; j < VPL; j++) mm = max(mm, kv[j]);
    uint32_t tau = 0;
    for (int r = 0; r < K; r++) {
        const uint32_t M = wave_max_u32(mm);
        tau = M;
        const unsigned long long bm = __ballot(mm == M);
        mm = l == (__ffsll((long long)bm) - 1) ? 0u : mm;
    }
    unsigned long long bj[VPL];
    int c = 0;
#pragma unroll
    for (int j = 0; j < VPL; j++) {
        bj[j] = __ballot(kv[j] >= tau && kv[j] != 0u);
        c += __popcll(bj[j]);
    }
    if (c > WAVE) return false;
    int base = 0;
#pragma unroll
    for (int j = 0; j < VPL; j++) {
        if (kv[j] >= tau && kv[j] != 0u)
            cand[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bj[j] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bj[j], 0))] =
                make_uint2(kv[j], (uint32_t)(l + j * WAVE));
        base += __popcll(bj[j]);
    }
    // candidate i in lane i; its rank = the candidates ahead of it in (key
    // descending, expert ascending) order: one 64-bit compare of packed
    // (key, ~expert) per candidate, each read from its lane's registers
    const uint2 me = cand[min(l, c - 1)];
    const uint64_t pm = ((uint64_t)me.x << 32) | (uint32_t)~me.y;
    int rank = 0;
    for (int i = 0; i < c; i++) {
        const uint64_t po = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)me.x, i) << 32) |
                            (uint32_t)~(uint32_t)__builtin_amdgcn_readlane((int)me.y, i);
        rank += po > pm;
    }
    if (l < c && rank < K) outb[rank] = me;
    const uint2 mine = outb[min(l, K - 1)];
    my_key = l < K ? mine.x : 0u;
    my_e = l < K ? (int)mine.y : 0;
    return true;
}

MOE_DEV int ceil_div(int a, int b) { return (a + b - 1) / b; }

// The tile that block `bid` of a grouped launch works on: experts own
// ceil(count/bm) consecutive row tiles each.  Returns the expert (or -1 if bid
// is past the last tile) and the tile's first permuted row.  Every lane of the
// calling wave gets the result.
MOE_DEV int find_group_tile(const int32_t* __restrict__ offsets, int E, int bm, int bid, int& row0, int& rows) {
    const int l = lane_id();
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += WAVE) {
        int e = e0 + l;
        int n = 0, off = 0;
        if (e < E) { off = offsets[e]; n = offsets[e + 1] - off; }
        int t = ceil_div(n, bm);
        int incl = wave_incl_scan(t);
        int excl = incl - t;
        bool hit = (bid >= base + excl) && (bid < base + incl);
        unsigned long long m = __ballot(hit);
        if (m) {
            int src = __ffsll((long long)m) - 1;
            int he = __shfl(e, src, WAVE);
            int hoff = __shfl(off, src, WAVE);
            int hn = __shfl(n, src, WAVE);
            int hex = __shfl(excl, src, WAVE);
            int j = bid - base - hex;
            row0 = hoff + j * bm;
            rows = min(bm, hn - j * bm);
            return he;
        }
        base += __shfl(incl, WAVE - 1, WAVE);
    }
    return -1;
}
