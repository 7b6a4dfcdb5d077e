// verify.hip -- one whole MoE layer for a handful of tokens (T <= 8: the
// speculative verify step of 4 drafted tokens plus one, and decode) in three
// launches instead of five.
//
// The layer ("Strata Coder 编程模型深度剖析", §1: 10 experts per token; §3:
// gate, up and down matrices per expert): route every token to its K experts,
// run each touched expert's SwiGLU on its tokens, and combine the K outputs
// of every token with its routing weights (+ the residual stream).
//
//   1. exact router logits [T][E] (the small-token logits kernel of route.hip);
//   2. k_vgateup: every block selects each token's top K from the logits and
//      groups the T*K slots by expert itself, so no separate selection or
//      grouping launch runs; block 0 also writes the routing and grouping
//      outputs and the touched-expert list.  Then the gate/up weight stream of
//      the touched experts (as in ffn_stream.hip) writes a = bf16(silu(g) u);
//   3. k_vdown / k_vdown_q: one wave per hidden row (bf16) or per four rows
//      and an eighth of the touched experts (block-quantised weights) walks the
//      touched experts' down rows, keeps each grouped row's output in LDS and
//      then combines each token's K outputs in k order with the residual, one
//      rounding: y_perm never goes to memory and no combine launch runs.
// A steered layer (a unit direction removed from the stream after the layer)
// stores the unrounded rows and a fourth small kernel projects and rounds.
//
// Results: routing and grouping are identical to moe_route_group's; the layer
// output differs from the separate calls only in that the expert outputs are
// combined from fp32 rather than from a bf16 y_perm.
#include "../../include/moe.h"
#include "common.h"
#include "device.h"
#include "launch.h"
#include "stream.h"

namespace {

constexpr int VF = 512;              // expert width of the fused path
constexpr int VH = 2048;             // hidden size of the fused path
constexpr int VMAX_SLOTS = 128;      // T * K

struct VerifyOut {
    int32_t* idx;
    float* w;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    int32_t* inv;
    int4* list;     // touched experts (expert, first grouped row, rows), expert order
    int32_t* nlist;
};

// Top K of one token's logits (their order keys kv, as load_order_keys
// gives them) by one wave, with the routing weights computed as moe_route
// computes them; lane r < K ends with rank r's expert and weight.
template <int VPL>
MOE_DEV void select_weights(uint32_t (&kv)[VPL], int K, uint2* __restrict__ scratch, bool want_w, int& e_out,
                            float& w_out) {
    uint32_t key;
    int sel;
    if (!select_top_cut<VPL>(kv, K, scratch, scratch + WAVE, key, sel)) select_top<VPL>(kv, K, key, sel);
    e_out = sel;
    w_out = want_w ? selection_weight(order_key_value(key), K) : 0.f;
}

// Calls f(u, v[u]) for u < n rounded up to 16, over an LDS array v of
// VMAX_SLOTS ints (16-byte aligned) whose entries past n hold a padding value
// that f must count for nothing: 16 entries per step, the four 16-byte reads
// of a step in flight together, no per-entry branch.
template <typename Fn>
MOE_DEV void for_slots(const int* __restrict__ v, int n, Fn&& f) {
    const int4* v4 = reinterpret_cast<const int4*>(__builtin_assume_aligned(v, 16));
    for (int u0 = 0; u0 < n; u0 += 16) {
        int4 q[4];
#pragma unroll
        for (int i = 0; i < 4; i++) q[i] = v4[(u0 >> 2) + i];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int u = u0 + 4 * i;
            f(u, q[i].x);
            f(u + 1, q[i].y);
            f(u + 2, q[i].z);
            f(u + 3, q[i].w);
        }
    }
}

// Routing and grouping of T <= 8 tokens inside one block of 8 waves (every
// block of the gate/up launch runs it), in two phases so that the weight loads
// of a wave's first items can go out between them.
//
// route_select_block: wave t selects token t from the order keys it loaded
// (kv, see the kernels), stores the slot keys e * VMAX_SLOTS + s and sets the
// selected experts' bits in `touched` (E bits, cleared beforehand; the j-th
// touched expert in ascending order is touched_nth(j)).  The writer block also
// stores ids and weights.
//
// route_group_rest: the T*K slots grouped by expert, stable by slot: the
// grouped row of slot s is its rank in (expert, slot) order, counted by the
// waves that hold slots only (one compare of packed keys per slot).  Group
// starts over the sorted rows become two 64-bit ballots, from which every
// touched expert's list index and row count follow by population counts.  The
// writer block also stores the grouping outputs (counts and offsets by a
// binary search of each expert in the touched list).  Returns the number of
// touched experts.
//
// Needs T <= 8 and T*K <= VMAX_SLOTS <= blockDim.x.  LDS: sel, srt
// [VMAX_SLOTS] int (16-byte aligned; slot keys, sorted keys); list [T*K] int4
// (expert, first grouped row, rows), expert order; prow [T*K] int (token of
// every grouped row); sscratch [8 waves][128] uint2 (the selection's scratch);
// touched [VTOUCH_WORDS] uint64.
constexpr int VTOUCH_WORDS = 16;     // E <= 1024

template <int VPL>
MOE_DEV void route_select_block(uint32_t (&kv)[VPL], int T, int K, int* __restrict__ sel,
                                uint64_t* __restrict__ touched, uint2* __restrict__ sscratch, bool writer,
                                const VerifyOut& o) {
    const int tid = threadIdx.x, wave = tid / WAVE, l = lane_id();
    const int n = T * K;
    if (wave < T) {
        int e;
        float w;
        select_weights<VPL>(kv, K, sscratch + wave * 2 * WAVE, writer, e, w);
        if (l < K) {
            sel[wave * K + l] = e * VMAX_SLOTS + wave * K + l;
            __hip_atomic_fetch_or(touched + (e >> 6), 1ull << (e & 63), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (writer) {
                o.idx[wave * K + l] = e;
                o.w[wave * K + l] = w;
            }
        }
    }
    if (tid < VMAX_SLOTS - n) sel[n + tid] = 0x7fffffff;   // padding read by for_slots, never counted
    lds_barrier();
}

// Number of touched experts (wave-uniform).
MOE_DEV int touched_count(const uint64_t* __restrict__ touched, int E) {
    int c = 0;
    for (int w = 0; w < (E + 63) / 64; w++) c += __popcll(touched[w]);
    return c;
}

// The j-th touched expert in ascending order, j < touched_count (wave-uniform):
// the word holding it by running population counts, then the bit whose count
// of set bits below it is j's remainder (one ballot).
MOE_DEV int touched_nth(const uint64_t* __restrict__ touched, int E, int j) {
    int base = 0, wsel = 0, bsel = 0;
    uint64_t msel = 0;
    for (int w = 0; w < (E + 63) / 64; w++) {
        const uint64_t m = touched[w];
        const int c = __popcll(m);
        if (j >= base && j < base + c) {
            wsel = w;
            msel = m;
            bsel = base;
        }
        base += c;
    }
    const int l = lane_id();
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(msel >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)msel, 0));
    const uint64_t b = __ballot(((msel >> l) & 1ull) && below == j - bsel);
    return wsel * 64 + (__ffsll((long long)b) - 1);
}

MOE_DEV int route_group_rest(int T, int E, int K, const int* __restrict__ sel, int* __restrict__ srt,
                             int4* __restrict__ list, int* __restrict__ prow, bool writer, const VerifyOut& o) {
    const int tid = threadIdx.x, wave = tid / WAVE, l = lane_id();
    const int n = T * K;
    if (tid < n) {
        const int me = sel[tid];
        int pos = 0;
        for_slots(sel, n, [&](int, int ku) __attribute__((always_inline)) { pos += ku < me; });
        srt[pos] = me;
        prow[pos] = tid / K;
        if (writer) {
            o.perm[pos] = tid;
            o.inv[tid] = pos;
        }
    }
    if (tid < VMAX_SLOTS - n) srt[n + tid] = 0x7fffffff;
    lds_barrier();
    // a sorted row starts a group when its expert differs from the row before
    auto starts = [&](int p) __attribute__((always_inline)) -> bool {
        return p < n && (p == 0 || (srt[p - 1] / VMAX_SLOTS) != (srt[p] / VMAX_SLOTS));
    };
    const uint64_t m0 = __ballot(starts(l)), m1 = __ballot(starts(l + WAVE));
    const int c0 = __popcll(m0), nlist = c0 + __popcll(m1);
    if (wave < 2) {
        const int p = wave * WAVE + l;
        const uint64_t m = wave ? m1 : m0;
        if ((m >> l) & 1ull) {
            const int j = (wave ? c0 : 0) +
                          (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            const uint64_t above = l == WAVE - 1 ? 0ull : m >> (l + 1);
            const int next = above ? p + 1 + __builtin_ctzll(above) : (wave == 0 && m1) ? WAVE + __builtin_ctzll(m1) : n;
            const int4 ent = make_int4(srt[p] / VMAX_SLOTS, p, next - p, 0);
            list[j] = ent;
            if (writer) o.list[j] = ent;
        }
    }
    lds_barrier();
    if (writer) {
        if (tid == 0) {
            *o.nlist = nlist;
            o.offsets[E] = n;
        }
        for (int x = tid; x < E; x += blockDim.x) {   // the first touched expert >= x
            int lo = 0, hi = nlist;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (list[mid].x < x) lo = mid + 1;
                else hi = mid;
            }
            const bool hit = lo < nlist && list[lo].x == x;
            o.counts[x] = hit ? list[lo].z : 0;
            o.offsets[x] = lo < nlist ? list[lo].y : n;
        }
    }
    return nlist;
}

// x [T][H] bf16 (T <= NT) into LDS, every chunk's load in flight before the
// first store.
template <int NT, int H, int THREADS>
struct XStage {
    static constexpr int MAXC = NT * H * 2 / 16 / THREADS;   // 16-byte chunks per thread
    uint4 r[MAXC];
    MOE_DEV void load_x(const uint16_t* __restrict__ x, int T) {
        const int n16 = T * H * 2 / 16;
        const uint4* g = reinterpret_cast<const uint4*>(x);
#pragma unroll
        for (int c = 0; c < MAXC; c++) r[c] = g[min((int)threadIdx.x + c * THREADS, n16 - 1)];
    }
    // QB: the rows go to LDS in the pair order of QB-bit weights (pair_order)
    template <int QB>
    MOE_DEV void store_x(uint16_t* __restrict__ xs, int T) {
        const int n16 = T * H * 2 / 16;
#pragma unroll
        for (int c = 0; c < MAXC; c++)   // past the end: the last chunk again, same value
            reinterpret_cast<uint4*>(xs)[min((int)threadIdx.x + c * THREADS, n16 - 1)] = pair_order<QB>(r[c]);
    }
};

// Copy n16 16-byte chunks from global memory to LDS with THREADS threads,
// CH chunks per thread in flight at a time (past the end the last chunk is
// loaded and stored again, the same value).
template <int THREADS, int CH>
MOE_DEV void copy_to_lds(const void* __restrict__ src, void* __restrict__ dst, int n16) {
    const uint4* g = reinterpret_cast<const uint4*>(src);
    uint4* d = reinterpret_cast<uint4*>(dst);
    const int tid = threadIdx.x;
    for (int c0 = 0; c0 * THREADS < n16; c0 += CH) {
        uint4 a[CH];
#pragma unroll
        for (int c = 0; c < CH; c++) a[c] = g[min(tid + (c0 + c) * THREADS, n16 - 1)];
#pragma unroll
        for (int c = 0; c < CH; c++) d[min(tid + (c0 + c) * THREADS, n16 - 1)] = a[c];
    }
}

constexpr int VG_THREADS = 512;   // gate/up blocks: 8 waves, one token's selection each
constexpr int VB_THREADS = 1024;  // bf16 gate/up: 16 waves (the first T select), items of one gate and one up row
constexpr int VQ_ROWS = 2;        // token rows per pass of the quantised gate/up and down

}  // namespace

// ---------------------------------------------------------------------------- gate/up

// bf16 weights.  Item = (touched expert j, FR feature rows of gate and the
// same FR of up) over all of H; lane l owns 8 consecutive inputs per 512.
template <int NT, int FR, int RING, int VPL>
__global__ __launch_bounds__(VB_THREADS) void k_vgateup(const float* __restrict__ lg, const uint16_t* __restrict__ x,
                                                 const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                                                 int T, int K, int E, VerifyOut o, uint16_t* __restrict__ abuf) {
    constexpr int H = VH, CH = H / 512, F = VF;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int n = T * K;
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                 // [T][H]
    int4* list = reinterpret_cast<int4*>(smem + (size_t)T * H * 2);   // [n]
    int* sel = reinterpret_cast<int*>(list + n);                      // [VMAX_SLOTS]
    int* srt = sel + VMAX_SLOTS;                                      // [VMAX_SLOTS]
    uint2* sscr = reinterpret_cast<uint2*>(srt + VMAX_SLOTS);       // [8][128]
    uint64_t* touched = reinterpret_cast<uint64_t*>(sscr + 8 * 2 * WAVE);   // [VTOUCH_WORDS]
    int* prow = reinterpret_cast<int*>(touched + VTOUCH_WORDS);       // [n]
    const int tid = threadIdx.x, wave = tid / WAVE, l = lane_id();
    const bool writer = blockIdx.x == 0;
    // the token rows' loads go out first, then wave t's loads of token t's
    // logits; x goes to LDS while the selection waits for the logits
    XStage<NT, H, VB_THREADS> xst;
    xst.load_x(x, T);
    uint32_t kv[VPL];
    load_order_keys<VPL>(lg + (long)min(wave, T - 1) * E, E, kv);
    if (tid < VTOUCH_WORDS) touched[tid] = 0ull;
    xst.template store_x<16>(xs, T);
    lds_barrier();
    route_select_block<VPL>(kv, T, K, sel, touched, sscr, writer, o);

    const int tpe = F / FR;
    const int n_items = touched_count(touched, E) * tpe;
    const int W = gridDim.x * (VB_THREADS / WAVE);
    const int it = blockIdx.x * (VB_THREADS / WAVE) + wave;
    const bool active = it < n_items;

    uint4 wbuf[RING][2 * FR][CH];
    auto load_e = [&](int e, int f0, uint4 (&w)[2 * FR][CH]) __attribute__((always_inline)) {
        const uint16_t* g0 = wg + ((long)e * F + f0) * H + l * 8;
        const uint16_t* u0 = wu + ((long)e * F + f0) * H + l * 8;
#pragma unroll
        for (int c = 0; c < CH; c++)
#pragma unroll
            for (int r = 0; r < FR; r++) {
                w[r][c] = ldnt16(g0 + (long)r * H + c * 512);
                w[FR + r][c] = ldnt16(u0 + (long)r * H + c * 512);
            }
    };
    auto load = [&](int item, uint4 (&w)[2 * FR][CH]) __attribute__((always_inline)) {
        load_e(list[item / tpe].x, (item % tpe) * FR, w);
    };
    auto compute = [&](int item, const uint4 (&w)[2 * FR][CH]) __attribute__((always_inline)) {
        const int4 ent = list[item / tpe];
        const int off = ent.y, nj = __builtin_amdgcn_readfirstlane(ent.z), f0 = (item % tpe) * FR;
        auto rows = [&](auto ntn) __attribute__((always_inline)) {
            constexpr int NTN = decltype(ntn)::value;
            constexpr int V = 2 * FR * NTN;
            float acc[V];
#pragma unroll
            for (int i = 0; i < V; i++) acc[i] = 0.f;
#pragma unroll
            for (int t = 0; t < NTN; t++) {
                if (t < nj) {
                    const uint16_t* xr = xs + prow[off + t] * H + l * 8;
#pragma unroll
                    for (int c = 0; c < CH; c++) {
                        const uint4 a = *reinterpret_cast<const uint4*>(xr + c * 512);
#pragma unroll
                        for (int r = 0; r < 2 * FR; r++) acc[r * NTN + t] = dot8bf(w[r][c], a, acc[r * NTN + t]);
                    }
                }
            }
            const float v = wave_tr_reduce<V>(acc);
            constexpr int shift = tr_shift<V>();
            const float up = __shfl_down(v, (FR * NTN) << shift, WAVE);
            const int j = l >> shift, r = j / NTN, t = j % NTN;
            if ((l & ((1 << shift) - 1)) == 0 && r < FR && t < nj)
                abuf[(long)(off + t) * F + f0 + r] = f32_to_bf16_rne(silu_ref(v) * up);
        };
        by_rows<NT>(nj, rows);
    };
    // the first items' weights (as ring_start would load them, their experts
    // from the bitmap) go out before the grouping
    if (active) {
#pragma unroll
        for (int b = 0; b < RING - 1; b++) {
            const int item = min(it + b * W, n_items - 1);
            load_e(touched_nth(touched, E, item / tpe), (item % tpe) * FR, wbuf[b]);
        }
    }
    route_group_rest(T, E, K, sel, srt, list, prow, writer, o);
    if (!active) return;
    ring_run<RING>(it, W, n_items, wbuf, load, compute);
}

// Block-quantised weights (QB = 4, 3 or 2 bits), H = 2048: item = FR gate rows
// and the same FR up rows, a lane owning one 32-input quant block of each.
template <int NT, int FR, int RING, int QB, int VPL>
__global__ __launch_bounds__(VG_THREADS) void k_vgateup_q(
    const float* __restrict__ lg, const uint16_t* __restrict__ x, const uint8_t* __restrict__ wg,
    const uint8_t* __restrict__ wu, const uint16_t* __restrict__ sg, const uint16_t* __restrict__ su, int T, int K,
    int E, VerifyOut o, uint16_t* __restrict__ abuf) {
    constexpr int H = VH, F = VF;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int n = T * K;
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                      // [T][H]
    float* xsum = reinterpret_cast<float*>(smem + (size_t)T * H * 2);      // [T][H/32]
    int4* list = reinterpret_cast<int4*>(xsum + T * (H / 32));             // [n]
    int* sel = reinterpret_cast<int*>(list + n);                           // [VMAX_SLOTS]
    int* srt = sel + VMAX_SLOTS;                                           // [VMAX_SLOTS]
    uint2* sscr = reinterpret_cast<uint2*>(srt + VMAX_SLOTS);            // [8][128]
    uint64_t* touched = reinterpret_cast<uint64_t*>(sscr + 8 * 2 * WAVE);  // [VTOUCH_WORDS]
    int* prow = reinterpret_cast<int*>(touched + VTOUCH_WORDS);            // [n]
    const int tid = threadIdx.x, wave = tid / WAVE, l = lane_id();
    const bool writer = blockIdx.x == 0;
    // the token rows' loads go out first, then wave t's loads of token t's
    // logits; x goes to LDS while the selection waits for the logits
    XStage<NT, H, VG_THREADS> xst;
    xst.load_x(x, T);
    uint32_t kv[VPL];
    load_order_keys<VPL>(lg + (long)min(wave, T - 1) * E, E, kv);
    if (tid < VTOUCH_WORDS) touched[tid] = 0ull;
    xst.template store_x<QB>(xs, T);
    lds_barrier();
    route_select_block<VPL>(kv, T, K, sel, touched, sscr, writer, o);

    const int tpe = F / FR;
    const int n_items = touched_count(touched, E) * tpe;
    const int W = gridDim.x * (VG_THREADS / WAVE);
    const int it = blockIdx.x * (VG_THREADS / WAVE) + wave;
    const bool active = it < n_items;

    constexpr int QW = QWords<QB>::n;
    struct Buf { uint32_t q[2 * FR][QW]; uint16_t d[2 * FR]; };
    Buf wbuf[RING];
    auto load_e = [&](int e, int f0, Buf& b) __attribute__((always_inline)) {
        const long row0 = (long)e * F + f0;
#pragma unroll
        for (int r = 0; r < FR; r++) {
            load_block<QB>(b.q[r], wg + (row0 + r) * (H * QB / 8), H, l);
            load_block<QB>(b.q[FR + r], wu + (row0 + r) * (H * QB / 8), H, l);
            b.d[r] = ldnt_u16(sg + (row0 + r) * (H / 32) + l);
            b.d[FR + r] = ldnt_u16(su + (row0 + r) * (H / 32) + l);
        }
    };
    auto load = [&](int item, Buf& b) __attribute__((always_inline)) {
        load_e(list[item / tpe].x, (item % tpe) * FR, b);
    };
    auto compute = [&](int item, const Buf& b) __attribute__((always_inline)) {
        const int4 ent = list[item / tpe];
        const int off = ent.y, nj = __builtin_amdgcn_readfirstlane(ent.z), f0 = (item % tpe) * FR;
        // rows t0 .. t0 + NTN - 1 of the item's expert
        auto rows = [&](auto ntn, int t0) __attribute__((always_inline)) {
            constexpr int NTN = decltype(ntn)::value;
            constexpr int V = 2 * FR * NTN;
            const int nr = nj - t0;
            float acc[V];
#pragma unroll
            for (int i = 0; i < V; i++) acc[i] = 0.f;
#pragma unroll
            for (int t = 0; t < NTN; t++) {
                if (t < nr) {
                    const int tok = prow[off + t0 + t];
                    const uint16_t* xl = xs + tok * H + l * 32;
                    const float S = xsum[tok * (H / 32) + l];
#pragma unroll
                    for (int r = 0; r < 2 * FR; r++) {
                        const float D = dot_block_p<QB>(b.q[r], xl);
                        acc[r * NTN + t] = fmaf(fp16_to_f32(b.d[r]), fmaf(-zero_level<QB>(), S, D), acc[r * NTN + t]);
                    }
                }
            }
            const float v = wave_tr_reduce<V>(acc);
            constexpr int shift = tr_shift<V>();
            const float up = __shfl_down(v, (FR * NTN) << shift, WAVE);
            const int j = l >> shift, r = j / NTN, t = j % NTN;
            if ((l & ((1 << shift) - 1)) == 0 && r < FR && t < nr)
                abuf[(long)(off + t0 + t) * F + f0 + r] = f32_to_bf16_rne(silu_ref(v) * up);
        };
        // at most VQ_ROWS rows per pass (more rows: further passes over the
        // same weights), which bounds the accumulators and the reduction
        if (nj <= VQ_ROWS) {
            by_rows<(NT < VQ_ROWS ? NT : VQ_ROWS)>(nj, [&](auto ntn) __attribute__((always_inline)) { rows(ntn, 0); });
        } else {
            for (int t0 = 0; t0 < nj; t0 += VQ_ROWS) rows(std::integral_constant<int, VQ_ROWS>{}, t0);
        }
    };
    // the first items' weights (as ring_start would load them, their experts
    // from the bitmap) go out before the grouping
    if (active) {
#pragma unroll
        for (int b = 0; b < RING - 1; b++) {
            const int item = min(it + b * W, n_items - 1);
            load_e(touched_nth(touched, E, item / tpe), (item % tpe) * FR, wbuf[b]);
        }
    }
    route_group_rest(T, E, K, sel, srt, list, prow, writer, o);
    block_sums(xs, T, H, xsum);
    lds_barrier();
    if (!active) return;
    ring_run<RING>(it, W, n_items, wbuf, load, compute);
}

// ---------------------------------------------------------------------------- down + combine

namespace {
// The touched list held in registers by every wave: lane j keeps entries j
// and j + 64, read back wave-uniformly.  The loads are clamped to the list's
// capacity (T*K entries), not to its length, so they need not wait for the
// length; entries past the length are never read back.
struct WaveList {
    int4 a, b;
    MOE_DEV void load(const int4* __restrict__ g_list, int cap) {
        const int l = lane_id();
        a = g_list[min(l, cap - 1)];
        b = g_list[min(l + WAVE, cap - 1)];
    }
    MOE_DEV int x(int j) const {
        return j < WAVE ? __builtin_amdgcn_readlane(a.x, j) : __builtin_amdgcn_readlane(b.x, j - WAVE);
    }
    MOE_DEV int y(int j) const {
        return j < WAVE ? __builtin_amdgcn_readlane(a.y, j) : __builtin_amdgcn_readlane(b.y, j - WAVE);
    }
    MOE_DEV int z(int j) const {
        return j < WAVE ? __builtin_amdgcn_readlane(a.z, j) : __builtin_amdgcn_readlane(b.z, j - WAVE);
    }
    // the same for an index that differs between lanes (a cross-lane read)
    MOE_DEV int y_any(int j) const {
        const int u = __shfl(a.y, j & (WAVE - 1), WAVE), v = __shfl(b.y, j & (WAVE - 1), WAVE);
        return j < WAVE ? u : v;
    }
    MOE_DEV int z_any(int j) const {
        const int u = __shfl(a.z, j & (WAVE - 1), WAVE), v = __shfl(b.z, j & (WAVE - 1), WAVE);
        return j < WAVE ? u : v;
    }
};

// The grouped intermediate rows [n][F] and every slot's routing weight and
// grouped row, for LDS (THREADS threads, n * 64 <= THREADS * MS): load() issues every load,
// store() writes LDS once they have landed, so weight loads issued between the
// two do not hold up the staging.  Past the end the last chunk is loaded and
// stored again (the same value).
template <int MS, int THREADS = 512>
struct DownStage {
    uint4 c[MS];
    float w;
    int p;
    MOE_DEV void load(const uint16_t* __restrict__ abuf, int n, const float* __restrict__ topk_w,
                      const int32_t* __restrict__ inv) {
        const int n16 = n * VF * 2 / 16, tid = threadIdx.x;
        const uint4* g = reinterpret_cast<const uint4*>(abuf);
#pragma unroll
        for (int i = 0; i < MS; i++) c[i] = g[min(tid + i * THREADS, n16 - 1)];
        w = topk_w[min(tid, n - 1)];
        p = inv[min(tid, n - 1)];
    }
    template <int QB>   // the rows in the pair order of QB-bit weights (pair_order)
    MOE_DEV void store(uint16_t* __restrict__ as, float* __restrict__ tw, int* __restrict__ tinv, int n) const {
        const int n16 = n * VF * 2 / 16, tid = threadIdx.x;
        uint4* d = reinterpret_cast<uint4*>(as);
#pragma unroll
        for (int i = 0; i < MS; i++) d[min(tid + i * THREADS, n16 - 1)] = pair_order<QB>(c[i]);
        if (tid < n) {
            tw[tid] = w;
            tinv[tid] = p;
        }
    }
};

// out[t][h] (or the unrounded row for a steered layer) from the grouped rows'
// outputs ys[p] of hidden row h: the K outputs of token t in k order, fp32,
// then the residual, one rounding (the combine of combine.hip, per element).
template <int STEER>
MOE_DEV void combine_one(const float* __restrict__ ys, const float* __restrict__ tw, const int* __restrict__ tinv,
                         int t, int K, int H, int h, const uint16_t* __restrict__ residual, uint16_t* __restrict__ out,
                         float* __restrict__ hbuf) {
    float acc = 0.f;
    for (int k = 0; k < K; k++) acc = fmaf(tw[t * K + k], ys[tinv[t * K + k]], acc);
    const long o = (long)t * H + h;
    if (residual) acc += bf16_to_f32(residual[o]);
    if constexpr (STEER) hbuf[o] = acc;
    else out[o] = f32_to_bf16_rne(acc);
}
}  // namespace

// bf16 weights: wave w of block b owns hidden row h = 8 b + w and walks the
// touched experts' rows Wd[e][h] (1 KB each, a lane 8 inputs) in batches of
// VB experts, the next batch's loads in flight while one is multiplied; a
// batch's partial sums are reduced across the wave together (one transposing
// reduction of VB x rows values instead of one per expert).  The first loads
// go out before the block stages the intermediate rows.  512 threads; LDS:
// the grouped rows, the slots' weights and grouped rows, per-wave outputs.
constexpr int VB = 8;
template <int NT, int MS, int STEER>
__global__ __launch_bounds__(512) void k_vdown(const uint16_t* __restrict__ abuf, const uint16_t* __restrict__ wd,
                                               const int4* __restrict__ g_list, const int32_t* __restrict__ g_nlist,
                                               const float* __restrict__ topk_w, const int32_t* __restrict__ inv,
                                               int T, int K, int H, const uint16_t* __restrict__ residual,
                                               uint16_t* __restrict__ out, float* __restrict__ hbuf) {
    constexpr int F = VF;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int n = T * K;
    uint16_t* as = reinterpret_cast<uint16_t*>(smem);                  // [n][F]
    float* ys = reinterpret_cast<float*>(smem + (size_t)n * F * 2);    // [8][n]
    float* tw = ys + 8 * n;                                            // [n]
    int* tinv = reinterpret_cast<int*>(tw + n);                        // [n]
    const int tid = threadIdx.x, wave = tid / WAVE, l = lane_id();
    const int nlist = __builtin_amdgcn_readfirstlane(*g_nlist);
    const int h = blockIdx.x * 8 + wave;          // grid = H / 8: every row exists
    WaveList lst;
    lst.load(g_list, n);
    DownStage<MS> stg;
    stg.load(abuf, n, topk_w, inv);
    float* yw = ys + wave * n;
    // batch jb: experts jb .. jb + VB - 1 (past the list: the last again, not used)
    auto load = [&](int jb, uint4 (&w)[VB]) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < VB; b++) w[b] = ldnt16(wd + ((long)lst.x(min(jb + b, nlist - 1)) * H + h) * F + l * 8);
    };
    auto compute = [&](int jb, const uint4 (&w)[VB]) __attribute__((always_inline)) {
        int nmax = 1;
#pragma unroll
        for (int b = 0; b < VB; b++)
            if (jb + b < nlist) nmax = max(nmax, lst.z(jb + b));
        auto rows = [&](auto ntn) __attribute__((always_inline)) {
            constexpr int NTN = decltype(ntn)::value;
            constexpr int V = VB * NTN;
            float acc[V];
#pragma unroll
            for (int b = 0; b < VB; b++) {
                const int j = min(jb + b, nlist - 1);
                const int off = lst.y(j), nj = jb + b < nlist ? lst.z(j) : 0;
#pragma unroll
                for (int t = 0; t < NTN; t++)
                    acc[b * NTN + t] =
                        t < nj ? dot8bf(w[b], *reinterpret_cast<const uint4*>(as + (off + t) * F + l * 8), 0.f) : 0.f;
            }
            const float v = wave_tr_reduce<V>(acc);
            constexpr int shift = tr_shift<V>();
            const int e = l >> shift, b = e / NTN, t = e % NTN;
            const int j = min(jb + b, nlist - 1);
            const int off = lst.y_any(j), nj = jb + b < nlist ? lst.z_any(j) : 0;
            if ((l & ((1 << shift) - 1)) == 0 && t < nj) yw[off + t] = v;
        };
        by_rows<NT>(nmax, rows);
    };
    uint4 w0[VB], w1[VB];
    load(0, w0);
    stg.template store<16>(as, tw, tinv, n);
    lds_barrier();
    for (int jb = 0; jb < nlist; jb += 2 * VB) {
        load(jb + VB, w1);
        compute(jb, w0);
        if (jb + VB >= nlist) break;
        load(jb + 2 * VB, w0);
        compute(jb + VB, w1);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the loads past the end land before the wave ends
    if (l < T) combine_one<STEER>(yw, tw, tinv, l, K, H, h, residual, out, hbuf);
}

// Block-quantised weights, F = 512: a wave covers four hidden rows (16 lanes
// per row, a lane one quant block) and an eighth of the touched experts
// (j = q, q + 8, ...); the block's 16 waves are 2 row groups x 8 eighths, so
// a block owns 8 rows and combines them once all eighths are done.  The
// level decoding keeps this launch on the vector ALU, so it runs more waves
// per CU (16, within 128 registers: at most two token rows per pass) with
// one item's loads in flight each, rather than fewer waves with deep rings
// of loads; the deeper rings also grow the unrolled code.
template <int NT, int RING, int QB, int MS, int STEER>
__global__ __launch_bounds__(1024) void k_vdown_q(const uint16_t* __restrict__ abuf, const uint8_t* __restrict__ wd,
                                                 const uint16_t* __restrict__ sd, const int4* __restrict__ g_list,
                                                 const int32_t* __restrict__ g_nlist, const float* __restrict__ topk_w,
                                                 const int32_t* __restrict__ inv, int T, int K, int H,
                                                 const uint16_t* __restrict__ residual, uint16_t* __restrict__ out,
                                                 float* __restrict__ hbuf) {
    constexpr int F = VF, NB = F / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int n = T * K;
    uint16_t* as = reinterpret_cast<uint16_t*>(smem);                  // [n][F]
    float* asum = reinterpret_cast<float*>(smem + (size_t)n * F * 2);  // [n][F/32]
    float* ys = asum + n * NB;                                         // [8 rows][n]
    float* tw = ys + 8 * n;                                            // [n]
    int* tinv = reinterpret_cast<int*>(tw + n);                        // [n]
    const int tid = threadIdx.x, wave = tid / WAVE, l = lane_id();
    const int nlist = __builtin_amdgcn_readfirstlane(*g_nlist);
    const int rg = wave >> 3, q = wave & 7, g = l >> 4, b = l & 15;
    const int rloc = rg * 4 + g;                  // the lane's row within the block
    const int h = blockIdx.x * 8 + rloc;          // grid = H / 8: every row exists
    float* yr = ys + rloc * n;
    const int n_items = nlist > q ? (nlist - q + 7) / 8 : 0;
    WaveList lst;
    lst.load(g_list, n);
    DownStage<MS, 1024> stg;
    stg.load(abuf, n, topk_w, inv);
    constexpr int QW = QWords<QB>::n;
    struct Buf { uint32_t q[QW]; uint16_t d; };
    Buf wb[RING];
    auto load = [&](int i, Buf& bf) __attribute__((always_inline)) {
        const long row = (long)lst.x(q + 8 * i) * H + h;
        load_block<QB>(bf.q, wd + row * (F * QB / 8), F, b);
        bf.d = ldnt_u16(sd + row * NB + b);
    };
    auto compute = [&](int i, const Buf& bf) __attribute__((always_inline)) {
        const int j = q + 8 * i;
        const int off = lst.y(j), nj = lst.z(j);
        const float d = fp16_to_f32(bf.d);
        auto rows = [&](auto ntn, int t0) __attribute__((always_inline)) {
            constexpr int NTN = decltype(ntn)::value;
            const int nr = nj - t0;
            float acc[NTN];
#pragma unroll
            for (int t = 0; t < NTN; t++) {
                acc[t] = 0.f;
                if (t < nr) {
                    const float S = asum[(off + t0 + t) * NB + b];
                    const float D = dot_block_p<QB>(bf.q, as + (off + t0 + t) * F + b * 32);
                    acc[t] = d * fmaf(-zero_level<QB>(), S, D);
                }
            }
            const float v = group16_tr_reduce<NTN>(acc);
            constexpr int shift = NTN == 16 ? 0 : NTN == 8 ? 1 : NTN == 4 ? 2 : NTN == 2 ? 3 : 4;
            const int t = b >> shift;
            if ((b & ((1 << shift) - 1)) == 0 && t < nr) yr[off + t0 + t] = v;
        };
        if (nj <= VQ_ROWS) {
            by_rows<(NT < VQ_ROWS ? NT : VQ_ROWS)>(nj, [&](auto ntn) __attribute__((always_inline)) { rows(ntn, 0); });
        } else {
            for (int t0 = 0; t0 < nj; t0 += VQ_ROWS) rows(std::integral_constant<int, VQ_ROWS>{}, t0);
        }
    };
    if (n_items > 0) ring_start<RING>(0, 1, n_items, wb, load);
    stg.template store<QB>(as, tw, tinv, n);
    lds_barrier();
    block_sums(as, n, F, asum);
    lds_barrier();
    if (n_items > 0) ring_run<RING>(0, 1, n_items, wb, load, compute);
    lds_barrier();
    if (tid < 8 * T) {
        const int r = tid / T, t = tid % T;
        combine_one<STEER>(ys + r * n, tw, tinv, t, K, H, blockIdx.x * 8 + r, residual, out, hbuf);
    }
}

// Steered layer: out[t] = bf16(h[t] - (h[t] . v) v) from the unrounded rows
// h [T][H] fp32; one block per token, the dot product summed in a fixed order
// (each thread's elements in order, the wave butterfly, the four waves in
// order), so every run gives the same bits.
__global__ __launch_bounds__(256) void k_vsteer(const float* __restrict__ hbuf, const float* __restrict__ v, int H,
                                                uint16_t* __restrict__ out) {
    __shared__ float part[4];
    const int t = blockIdx.x, tid = threadIdx.x;
    const float* hr = hbuf + (long)t * H;
    float d = 0.f;
    for (int i = tid; i < H; i += 256) d = fmaf(hr[i], v[i], d);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) d += __shfl_xor(d, m, WAVE);
    if (lane_id() == 0) part[tid / WAVE] = d;
    lds_barrier();
    d = ((part[0] + part[1]) + part[2]) + part[3];
    for (int i = tid; i < H; i += 256) out[(long)t * H + i] = f32_to_bf16_rne(fmaf(-d, v[i], hr[i]));
}

// ---------------------------------------------------------------------------- host

namespace {
constexpr int VG_FR = 1, VG_RING = 2;      // bf16 gate/up: 8 KB items, one in flight per wave, 16 waves per CU
constexpr int VQ_FR = 2, VQ_RING = 2;      // quantised gate/up: 4 rows per item, one item in flight
constexpr int VDQ_RING = 2;                // quantised down: one item in flight per wave, 16 waves per CU

size_t gateup_lds(int T, int K, int quant) {
    const size_t n = (size_t)T * K;
    return (size_t)T * VH * 2 + (quant ? (size_t)T * (VH / 32) * 4 : 0) + n * 16 + 2 * VMAX_SLOTS * 4 +
           8 * 2 * WAVE * 8 + VTOUCH_WORDS * 8 + n * 4;
}
size_t down_lds(int T, int K, int quant) {
    const size_t n = (size_t)T * K;
    return n * VF * 2 + (quant ? n * (VF / 32) * 4 : 0) + n * 8 * 4 + n * 8;
}
constexpr size_t VLDS_MAX = 160 * 1024;

template <int NT, int VPL>
hipError_t gateup_bf16_v(int grid, hipStream_t st, const float* lg, const void* x, const void* wg, const void* wu,
                         int T, int K, int E, const VerifyOut& o, uint16_t* abuf) {
    auto kern = k_vgateup<NT, VG_FR, VG_RING, VPL>;
    static LdsLimit lim;
    hipError_t e = lim.ensure((const void*)kern, (int)VLDS_MAX);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(VB_THREADS), gateup_lds(T, K, 0), st, lg, (const uint16_t*)x,
                       (const uint16_t*)wg, (const uint16_t*)wu, T, K, E, o, abuf);
    return hipSuccess;
}
template <int NT, int QB, int VPL>
hipError_t gateup_q_v(int grid, hipStream_t st, const float* lg, const void* x, const void* wg, const void* wu,
                      const void* sg, const void* su, int T, int K, int E, const VerifyOut& o, uint16_t* abuf) {
    auto kern = k_vgateup_q<NT, VQ_FR, VQ_RING, QB, VPL>;
    static LdsLimit lim;
    hipError_t e = lim.ensure((const void*)kern, (int)VLDS_MAX);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(VG_THREADS), gateup_lds(T, K, 1), st, lg, (const uint16_t*)x,
                       (const uint8_t*)wg, (const uint8_t*)wu, (const uint16_t*)sg, (const uint16_t*)su, T, K, E, o,
                       abuf);
    return hipSuccess;
}
// the selection's logits per lane: E <= 256, 512 or 1024
template <int NT>
hipError_t gateup_bf16(int grid, hipStream_t st, const float* lg, const void* x, const void* wg, const void* wu, int T,
                       int K, int E, const VerifyOut& o, uint16_t* abuf) {
    if (E <= 256) return gateup_bf16_v<NT, 4>(grid, st, lg, x, wg, wu, T, K, E, o, abuf);
    if (E <= 512) return gateup_bf16_v<NT, 8>(grid, st, lg, x, wg, wu, T, K, E, o, abuf);
    return gateup_bf16_v<NT, 16>(grid, st, lg, x, wg, wu, T, K, E, o, abuf);
}
template <int NT, int QB>
hipError_t gateup_q(int grid, hipStream_t st, const float* lg, const void* x, const void* wg, const void* wu,
                    const void* sg, const void* su, int T, int K, int E, const VerifyOut& o, uint16_t* abuf) {
    if (E <= 256) return gateup_q_v<NT, QB, 4>(grid, st, lg, x, wg, wu, sg, su, T, K, E, o, abuf);
    if (E <= 512) return gateup_q_v<NT, QB, 8>(grid, st, lg, x, wg, wu, sg, su, T, K, E, o, abuf);
    return gateup_q_v<NT, QB, 16>(grid, st, lg, x, wg, wu, sg, su, T, K, E, o, abuf);
}

template <int NT, int MS, int STEER>
hipError_t down_bf16_ms(hipStream_t st, const uint16_t* abuf, const void* wd, const VerifyOut& o, int T, int K,
                        int H, const void* residual, void* out, float* hbuf) {
    auto kern = k_vdown<NT, MS, STEER>;
    static LdsLimit lim;
    hipError_t e = lim.ensure((const void*)kern, (int)VLDS_MAX);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(H / 8), dim3(512), down_lds(T, K, 0), st, abuf, (const uint16_t*)wd, o.list,
                       o.nlist, o.w, o.inv, T, K, H, (const uint16_t*)residual, (uint16_t*)out, hbuf);
    return hipSuccess;
}
template <int NT, int STEER>
hipError_t down_bf16(hipStream_t st, const uint16_t* abuf, const void* wd, const VerifyOut& o, int T, int K, int H,
                     const void* residual, void* out, float* hbuf) {
    // staging chunks per thread: n * 64 16-byte chunks over 512 threads
    return T * K <= 64 ? down_bf16_ms<NT, 8, STEER>(st, abuf, wd, o, T, K, H, residual, out, hbuf)
                       : down_bf16_ms<NT, 16, STEER>(st, abuf, wd, o, T, K, H, residual, out, hbuf);
}
template <int NT, int QB, int MS, int STEER>
hipError_t down_q_ms(hipStream_t st, const uint16_t* abuf, const void* wd, const void* sd, const VerifyOut& o, int T,
                     int K, int H, const void* residual, void* out, float* hbuf) {
    auto kern = k_vdown_q<NT, VDQ_RING, QB, MS, STEER>;
    static LdsLimit lim;
    hipError_t e = lim.ensure((const void*)kern, (int)VLDS_MAX);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(H / 8), dim3(1024), down_lds(T, K, 1), st, abuf, (const uint8_t*)wd,
                       (const uint16_t*)sd, o.list, o.nlist, o.w, o.inv, T, K, H, (const uint16_t*)residual,
                       (uint16_t*)out, hbuf);
    return hipSuccess;
}
template <int NT, int QB, int STEER>
hipError_t down_q(hipStream_t st, const uint16_t* abuf, const void* wd, const void* sd, const VerifyOut& o, int T,
                  int K, int H, const void* residual, void* out, float* hbuf) {
    return T * K <= 64 ? down_q_ms<NT, QB, 4, STEER>(st, abuf, wd, sd, o, T, K, H, residual, out, hbuf)
                       : down_q_ms<NT, QB, 8, STEER>(st, abuf, wd, sd, o, T, K, H, residual, out, hbuf);
}

template <int NT, int STEER>
hipError_t run_nt(int grid, hipStream_t st, int w_dtype, const float* lg, const void* x, const void* wg,
                  const void* wu, const void* wd, const void* sg, const void* su, const void* sd, int T, int K, int E,
                  int H, const VerifyOut& o, uint16_t* abuf, const void* residual, void* out, float* hbuf) {
    hipError_t e;
    switch (w_dtype) {
        case MOE_BF16:
            e = gateup_bf16<NT>(grid, st, lg, x, wg, wu, T, K, E, o, abuf);
            if (e == hipSuccess) e = down_bf16<NT, STEER>(st, abuf, wd, o, T, K, H, residual, out, hbuf);
            return e;
        case MOE_INT4_B32:
            e = gateup_q<NT, 4>(grid, st, lg, x, wg, wu, sg, su, T, K, E, o, abuf);
            if (e == hipSuccess) e = down_q<NT, 4, STEER>(st, abuf, wd, sd, o, T, K, H, residual, out, hbuf);
            return e;
        case MOE_INT3_B32:
            e = gateup_q<NT, 3>(grid, st, lg, x, wg, wu, sg, su, T, K, E, o, abuf);
            if (e == hipSuccess) e = down_q<NT, 3, STEER>(st, abuf, wd, sd, o, T, K, H, residual, out, hbuf);
            return e;
        case MOE_INT2_B32:
            e = gateup_q<NT, 2>(grid, st, lg, x, wg, wu, sg, su, T, K, E, o, abuf);
            if (e == hipSuccess) e = down_q<NT, 2, STEER>(st, abuf, wd, sd, o, T, K, H, residual, out, hbuf);
            return e;
    }
    return hipErrorInvalidValue;
}
}  // namespace

bool verify_layer_eligible(int T, int H, int E, int K, int F, int x_dtype, int w_dtype) {
    const bool wt = w_dtype == MOE_BF16 || w_dtype == MOE_INT4_B32 || w_dtype == MOE_INT3_B32 || w_dtype == MOE_INT2_B32;
    return x_dtype == MOE_BF16 && wt && T >= 1 && T <= 8 && K >= 1 && T * K <= VMAX_SLOTS && H == VH && F == VF &&
           E >= K && E <= 1024 && gateup_lds(T, K, 1) <= VLDS_MAX && down_lds(T, K, 1) <= VLDS_MAX;
}

size_t verify_layer_workspace_bytes(int T, int H, int E, int K, int F) {
    auto r = [](size_t b) { return (b + 255) / 256 * 256; };
    return r((size_t)T * E * 4) + r((size_t)T * K * F * 2) + r((size_t)T * K * 16) + 256 + r((size_t)T * H * 4);
}

hipError_t launch_verify_layer(const void* x, const float* wr, const float* bias, int w_dtype, const void* wg,
                               const void* wu, const void* wd, const void* sg, const void* su, const void* sd, int T,
                               int H, int E, int K, int F, const void* residual, const float* steer_v, void* out,
                               int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                               void* ws, hipStream_t st) {
    auto r = [](size_t b) { return (b + 255) / 256 * 256; };
    char* p = (char*)ws;
    float* lg = (float*)p;
    p += r((size_t)T * E * 4);
    uint16_t* abuf = (uint16_t*)p;
    p += r((size_t)T * K * F * 2);
    int4* list = (int4*)p;
    p += r((size_t)T * K * 16);
    int32_t* nlist = (int32_t*)p;
    p += 256;
    float* hbuf = (float*)p;
    hipError_t e = launch_logits_exact(x, 1, wr, bias, T, H, E, lg, st);
    if (e != hipSuccess) return e;
    int ncu = 0;
    e = current_device_cus(&ncu);
    if (e != hipSuccess) return e;
    const int grid = ncu;           // gate/up: one 8-wave block per CU
    const VerifyOut o{idx, w, counts, offsets, perm, inv, list, nlist};
    if (steer_v) {
        e = T <= 4 ? run_nt<4, 1>(grid, st, w_dtype, lg, x, wg, wu, wd, sg, su, sd, T, K, E, H, o, abuf, residual, out,
                                  hbuf)
                   : run_nt<8, 1>(grid, st, w_dtype, lg, x, wg, wu, wd, sg, su, sd, T, K, E, H, o, abuf, residual, out,
                                  hbuf);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_vsteer, dim3(T), dim3(256), 0, st, (const float*)hbuf, steer_v, H, (uint16_t*)out);
    } else {
        e = T <= 4 ? run_nt<4, 0>(grid, st, w_dtype, lg, x, wg, wu, wd, sg, su, sd, T, K, E, H, o, abuf, residual, out,
                                  nullptr)
                   : run_nt<8, 0>(grid, st, w_dtype, lg, x, wg, wu, wd, sg, su, sd, T, K, E, H, o, abuf, residual, out,
                                  nullptr);
        if (e != hipSuccess) return e;
    }
    return hipGetLastError();
}
