// stream.h -- device helpers of the weight-streaming kernels (few tokens):
// non-temporal 16-byte loads, bf16 dot products, the transposing wave
// reduction, the per-wave prefetch ring over work items, the touched-expert
// list, and the block-quantised (int4 / int3 / int2) weight decoding.
#pragma once
#include <type_traits>

#include "common.h"

namespace {

typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

MOE_DEV uint4 ldnt16(const void* p) {
    const u32x4_v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_v*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
MOE_DEV float dot2bf(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a), __builtin_bit_cast(bf16x2_v, b), c, false);
}
MOE_DEV float dot8bf(uint4 w, uint4 x, float c) {
    c = dot2bf(w.x, x.x, c);
    c = dot2bf(w.y, x.y, c);
    c = dot2bf(w.z, x.z, c);
    return dot2bf(w.w, x.w, c);
}
MOE_DEV float silu_ref(float g) { return g / (1.0f + expf(-g)); }

// The partner's value at distance D of the transposing reduction below.
// Within a row of 16 lanes it is a DPP move, whose partner pairs lanes across
// bit D as xor D does (D = 8: lane 15 - i, the row mirror; D = 4: 7 - i within
// each half row; D = 2, 1: the quad swaps), so every lane keeps the same
// entries; only which lanes' partial sums meet differs.  Across rows it is the
// lane i ^ D exactly: v_permlane16_swap / v_permlane32_swap with both operands
// x leave row r ^ 1 (half h ^ 1) of x in the first result on odd rows (upper
// half) and in the second on even rows (lower half).
template <int D>
MOE_DEV float tr_partner(float x) {
    if constexpr (D >= 16) {
        const unsigned u = __builtin_bit_cast(unsigned, x);
        const bool hi = (lane_id() & D) != 0;
        if constexpr (D == 32) {
            const auto q = __builtin_amdgcn_permlane32_swap(u, u, false, false);
            return __builtin_bit_cast(float, hi ? q[0] : q[1]);
        } else {
            const auto q = __builtin_amdgcn_permlane16_swap(u, u, false, false);
            return __builtin_bit_cast(float, hi ? q[0] : q[1]);
        }
    } else {
        constexpr int ctrl = D == 8 ? 0x140 : D == 4 ? 0x141 : D == 2 ? 0x4E : 0xB1;
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, 0xF, 0xF,
                                                                     false));
    }
}

template <int CNT, int D, int V>
MOE_DEV void tr_step(float (&v)[V], int l) {
    if constexpr (D >= 1) {
        if constexpr (CNT > 1) {
            constexpr int half = CNT / 2;
            const bool bit = (l & D) != 0;
#pragma unroll
            for (int i = 0; i < half; i++) {
                const float keep = bit ? v[i + half] : v[i];
                const float send = bit ? v[i] : v[i + half];
                v[i] = keep + tr_partner<D>(send);
            }
            tr_step<half, D / 2, V>(v, l);
        } else {
            v[0] += tr_partner<D>(v[0]);
            tr_step<1, D / 2, V>(v, l);
        }
    }
}
// in-place transposing reduction of v[V] (V a power of two <= 64) over the
// wave; returns the sum of entry lane >> (6 - log2 V)
template <int V>
MOE_DEV float wave_tr_reduce(float (&v)[V]) {
    tr_step<V, 32, V>(v, lane_id());
    return v[0];
}
template <int V>
constexpr int tr_shift() { return V == 64 ? 0 : V == 32 ? 1 : V == 16 ? 2 : V == 8 ? 3 : V == 4 ? 4 : V == 2 ? 5 : 6; }

// Calls f(std::integral_constant<int, R>) with R = the expert's row count n
// rounded up to 1, 2, 4 or NT: the accumulators and the cross-lane reduction
// are sized for the rows an item really has (at T = 5 almost every expert
// has one), not for the largest T the kernel accepts.  n is wave-uniform.
template <int NT, typename Fn>
MOE_DEV void by_rows(int n, Fn&& f) {
    if (n <= 1) f(std::integral_constant<int, 1>{});
    else if (n <= 2) f(std::integral_constant<int, (NT < 2 ? NT : 2)>{});
    else if (n <= 4) f(std::integral_constant<int, (NT < 4 ? NT : 4)>{});
    else f(std::integral_constant<int, NT>{});
}

// The touched experts (count > 0) in expert order as (expert, first row,
// rows), built by the whole block from the grouping offsets; returns their
// number.  Needs 256 threads and E <= 256 * EPT.
constexpr int EPT = 16;
MOE_DEV int block_touched_list(const int32_t* __restrict__ offsets, int E, int4* __restrict__ list, int* scan) {
    const int tid = threadIdx.x;
    int off[EPT + 1];
    const int e0 = tid * EPT;
#pragma unroll
    for (int i = 0; i <= EPT; i++) off[i] = e0 + i <= E ? offsets[min(e0 + i, E)] : 0;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < EPT; i++) cnt += (e0 + i < E && off[i + 1] > off[i]) ? 1 : 0;
    // block exclusive scan of cnt
    const int incl = wave_incl_scan(cnt);
    const int w = tid / WAVE;
    if (lane_id() == WAVE - 1) scan[w] = incl;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < w; i++) base += scan[i];
    const int total = scan[0] + scan[1] + scan[2] + scan[3];
    int pos = base + incl - cnt;
#pragma unroll
    for (int i = 0; i < EPT; i++)
        if (e0 + i < E && off[i + 1] > off[i]) list[pos++] = make_int4(e0 + i, off[i], off[i + 1] - off[i], 0);
    return total;
}

// Copy n_kb KB from global memory to the start of LDS, 16 bytes per thread
// and step, four loads in flight per thread.  Plain loads, not the LDS DMA:
// the compiler makes every later LDS access in a loop wait for an LDS DMA,
// which would also wait for the weight prefetch of the streaming loops.
MOE_DEV void stage_lds(const void* src, int n_kb, unsigned char* lds, int wave, int l) {
    (void)wave; (void)l;
    const uint4* g = reinterpret_cast<const uint4*>(src);
    uint4* d = reinterpret_cast<uint4*>(lds);
    const int n16 = n_kb * 64;
    int i = threadIdx.x;
    for (; i + 3 * 256 < n16; i += 4 * 256) {
        const uint4 a = g[i], b = g[i + 256], c = g[i + 512], e = g[i + 768];
        d[i] = a; d[i + 256] = b; d[i + 512] = c; d[i + 768] = e;
    }
    for (; i < n16; i += 256) d[i] = g[i];
}

// A wave's walk over items it, it + W, it + 2W, ... < n: RING weight buffers,
// the load of the item RING-1 steps ahead is issued before each multiply, so
// RING-1 items' weights are always in flight.  Loads past the end repeat the
// last item (never predicated); all have landed when the walk returns.
template <int RING, typename Buf, typename LoadF>
MOE_DEV void ring_start(int it, int W, int n, Buf (&buf)[RING], LoadF&& load) {
#pragma unroll
    for (int b = 0; b < RING - 1; b++) load(min(it + b * W, n - 1), buf[b]);
}
template <int RING, typename Buf, typename LoadF, typename ComputeF>
MOE_DEV void ring_run(int it, int W, int n, Buf (&buf)[RING], LoadF&& load, ComputeF&& compute) {
    bool more = true;
    while (more) {
#pragma unroll
        for (int b = 0; b < RING; b++) {
            if (more) {
                load(min(it + (RING - 1) * W, n - 1), buf[(b + RING - 1) % RING]);
                compute(it, buf[b]);
                it += W;
                more = it < n;
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the repeated tail loads land before the wave ends
}
template <int RING, typename Buf, typename LoadF, typename ComputeF>
MOE_DEV void ring_walk(int it, int W, int n, Buf (&buf)[RING], LoadF&& load, ComputeF&& compute) {
    ring_start<RING>(it, W, n, buf, load);
    ring_run<RING>(it, W, n, buf, load, compute);
}


// ---------------------------------------------------------------------------- block-quantised weights
// 8 nibbles -> 8 bf16 values 128 + u (dword i holds elements 2i, 2i+1)
MOE_DEV uint4 nib8_bf16(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    uint4 o;
    o.x = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x43004300u;
    o.y = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x43004300u;
    o.z = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x43004300u;
    o.w = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x43004300u;
    return o;
}
// D = sum over one 32-element block of x * (128 + u)
MOE_DEV float dot_block_q4(uint4 q, const uint16_t* __restrict__ xl) {
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
    float d = 0.f;
#pragma unroll
    for (int k = 0; k < 4; k++) d = dot8bf(nib8_bf16(w4[k]), *reinterpret_cast<const uint4*>(xl + k * 8), d);
    return d;
}
MOE_DEV uint16_t ldnt_u16(const uint16_t* p) { return __builtin_nontemporal_load(p); }
MOE_DEV uint32_t ldnt_u32(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)); }
typedef unsigned int u32x2_v __attribute__((ext_vector_type(2)));
MOE_DEV u32x2_v ldnt8(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x2_v*>(p)); }

// Lower-bit blocks (int2: value d (u - 2); int3: d (u - 4)).  A block's 32
// levels: two 32-bit words of the low two bits (16 elements each, element
// 4k + j of a word in byte j, bits 2k..2k+1) and, for int3, one word of third
// bits (element 16g + 4k + j in byte j, bit 4g + k).  Shifting a low word by
// 2k and masking 0x03030303 leaves elements 4k..4k+3 one per byte (the third
// bits join them the same way), and a byte permute spreads two of them into
// the bf16 pair 128 + u, so the dot product takes the activations in their
// natural order:  sum_k x w = d (D - (128 + 2^(bits-1)) S).
template <int QB>
MOE_DEV float dot_block_low(const uint32_t (&q)[QB], const uint16_t* __restrict__ xl) {
    float d = 0.f;
#pragma unroll
    for (int g = 0; g < 2; g++) {
        const uint4 xa = *reinterpret_cast<const uint4*>(xl + g * 16);
        const uint4 xb = *reinterpret_cast<const uint4*>(xl + g * 16 + 8);
        const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            uint32_t m = (q[g] >> (2 * k)) & 0x03030303u;
            if constexpr (QB == 3) m |= ((q[2] >> (4 * g + k)) & 0x01010101u) << 2;
            d = dot2bf(__builtin_amdgcn_perm(m, m, 0x0C010C00u) | 0x43004300u, xw[2 * k], d);
            d = dot2bf(__builtin_amdgcn_perm(m, m, 0x0C030C02u) | 0x43004300u, xw[2 * k + 1], d);
        }
    }
    return d;
}
// Pair order: the same blocks decoded with one v_and_or per bf16 pair.  Masking
// a packed word, shifted by s, with 0x000F000F (int4) or 0x00030003 (int2)
// leaves one level in each 16-bit half, and or-ing 0x4300 into both halves
// makes the pair 128 + u directly (no byte permute).  The two levels of a pair
// lie 4 elements apart (int4: e_i, e_{i+4} of every 8; int2: e_{4k}, e_{4k+2}
// and e_{4k+1}, e_{4k+3}), so the activations are kept in LDS in that pair
// order (pair_order below, applied as they are staged): each dword of an
// 8-element chunk holds the two activations of one weight pair.  The products
// and the block sums are the same; only which products share a dot2 differs.
template <int QB>
MOE_DEV uint4 pair_order(uint4 v) {
    if constexpr (QB == 4) {
        return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                          __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
    } else if constexpr (QB == 2) {
        return make_uint4(__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.y, v.x, 0x07060302u),
                          __builtin_amdgcn_perm(v.w, v.z, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u));
    } else {
        return v;   // int3 and bf16 rows keep the natural order
    }
}
// 0x43004300 in a VGPR that the compiler cannot see through: with the or
// constant in a register, (w & mask) | c can be one v_and_or_b32 (the mask
// from an SGPR; one instruction may read only one scalar operand), where with
// two constants it is always an and and an or.  Where the weights serve
// several token rows the compiler still hoists the and out of the per-row
// code and keeps a separate or per row.
MOE_DEV uint32_t exp_pair() {
    uint32_t c;
    asm("v_mov_b32 %0, 0x43004300" : "=v"(c));
    return c;
}
MOE_DEV uint32_t lev_pair(uint32_t w, uint32_t mask, uint32_t c) { return (w & mask) | c; }
MOE_DEV float dot_block_q4p(uint4 q, const uint16_t* __restrict__ xl) {
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
    const uint32_t c = exp_pair();
    float d = 0.f;
#pragma unroll
    for (int k = 0; k < 4; k++) {   // elements 8k .. 8k+7
        const uint4 xv = *reinterpret_cast<const uint4*>(xl + k * 8);
        const uint32_t w = w4[k];
        d = dot2bf(lev_pair(w, 0x000F000Fu, c), xv.x, d);
        d = dot2bf(lev_pair(w >> 4, 0x000F000Fu, c), xv.y, d);
        d = dot2bf(lev_pair(w >> 8, 0x000F000Fu, c), xv.z, d);
        d = dot2bf(lev_pair(w >> 12, 0x000F000Fu, c), xv.w, d);
    }
    return d;
}
MOE_DEV float dot_block_q2p(const uint32_t (&q)[2], const uint16_t* __restrict__ xl) {
    const uint32_t c = exp_pair();
    float d = 0.f;
#pragma unroll
    for (int g = 0; g < 2; g++) {   // elements 16g .. 16g+15; element 4k + j in byte j, bits 2k, 2k+1
        const uint4 xa = *reinterpret_cast<const uint4*>(xl + g * 16);
        const uint4 xb = *reinterpret_cast<const uint4*>(xl + g * 16 + 8);
        const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            d = dot2bf(lev_pair(q[g] >> (2 * k), 0x00030003u, c), xw[2 * k], d);
            d = dot2bf(lev_pair(q[g] >> (2 * k + 8), 0x00030003u, c), xw[2 * k + 1], d);
        }
    }
    return d;
}
// one lane's block: 4 dwords (int4), 2 (int2) or 3 (int3)
template <int QB> struct QWords { static constexpr int n = QB == 4 ? 4 : QB; };
template <int QB>
MOE_DEV float dot_block(const uint32_t (&q)[QWords<QB>::n], const uint16_t* __restrict__ xl) {
    if constexpr (QB == 4) return dot_block_q4(make_uint4(q[0], q[1], q[2], q[3]), xl);
    else return dot_block_low<QB>(q, xl);
}
// the same with the activations in pair order (pair_order<QB>)
template <int QB>
MOE_DEV float dot_block_p(const uint32_t (&q)[QWords<QB>::n], const uint16_t* __restrict__ xl) {
    if constexpr (QB == 4) return dot_block_q4p(make_uint4(q[0], q[1], q[2], q[3]), xl);
    else if constexpr (QB == 2) return dot_block_q2p(q, xl);
    else return dot_block_low<QB>(q, xl);
}
// the lane's block of a row of n inputs at `row` (bytes n*QB/8), block b
template <int QB>
MOE_DEV void load_block(uint32_t (&q)[QWords<QB>::n], const uint8_t* __restrict__ row, int n, int b) {
    if constexpr (QB == 4) {
        const uint4 v = ldnt16(row + b * 16);
        q[0] = v.x; q[1] = v.y; q[2] = v.z; q[3] = v.w;
    } else {
        const u32x2_v v = ldnt8(row + b * 8);
        q[0] = v.x; q[1] = v.y;
        if constexpr (QB == 3) q[2] = ldnt_u32(row + n / 4 + b * 4);
    }
}
template <int QB> constexpr float zero_level() { return 128.0f + (float)(1 << (QB - 1)); }

// sums of every 32-element block of `rows` LDS rows of `cols` bf16 into sums[row][cols/32]
MOE_DEV void block_sums(const uint16_t* __restrict__ rowsp, int rows, int cols, float* __restrict__ sums) {
    const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
    const int nb = cols / 32;
    for (int i = threadIdx.x; i < rows * nb; i += blockDim.x) {
        const uint16_t* p = rowsp + (i / nb) * cols + (i % nb) * 32;
        float sacc = 0.f;
#pragma unroll
        for (int k = 0; k < 4; k++) sacc = dot8bf(ones, *reinterpret_cast<const uint4*>(p + k * 8), sacc);
        sums[i] = sacc;
    }
}

// transposing reduction within each 16-lane group (xor 8, 4, 2, 1): lane l
// returns the group's full sum of entry (l & 15) >> (4 - log2 V)
template <int V>
MOE_DEV float group16_tr_reduce(float (&v)[V]) {
    tr_step<V, 8, V>(v, lane_id());
    return v[0];
}
}  // namespace
