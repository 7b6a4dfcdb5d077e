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

// Wave-wide maximum of a u32, returned wave-uniform: DPP within each row of
// 16 lanes (quad swaps, half-row and row mirrors), then the four row maxima.
MOE_DEV uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));   // row_mirror
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return max(max(a, b), max(c, d));
}

MOE_DEV float order_key_value(uint32_t h) { return __uint_as_float((h & 0x80000000u) ? (h & 0x7FFFFFFFu) : ~h); }

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
        int win = -1;
#pragma unroll
        for (int j = 0; j < VPL; j++) {
            if (win < 0) {
                const unsigned long long bm = __ballot(kv[j] == M);
                if (bm) win = (__ffsll((long long)bm) - 1) + j * WAVE;
            }
        }
#pragma unroll
        for (int j = 0; j < VPL; j++) kv[j] = (l + j * WAVE == win) ? 0u : kv[j];
        if (l == r) {
            my_key = M;
            my_e = win;
        }
    }
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
