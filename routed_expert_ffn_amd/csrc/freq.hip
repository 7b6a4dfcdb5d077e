// freq.hip -- the expert-pruning statistic (gfx950).
//
// Pruning counts, on calibration data, which experts each token's routing
// selects, and keeps the most-selected experts of every layer, with one keep
// decision for gate, up and down and the kept experts listed in their
// original order ("Strata Coder 编程模型深度剖析", §3 "RCO 专家剪枝是怎么砍一半
// 而不伤脑的"; the per-(layer, expert) ranking of the kwkr.cn Coder write-up,
// "专家配置文件：48 x 256 的全量排名").
//
//   k_freq_count      top-K of every logit row (routing's rule: larger first,
//                     ties to the lower id), per-block LDS histogram, int64
//                     totals via integer atomics (exact and order-independent).
//   k_freq_count_thr  the same counts for wide rows (E > 128): a threshold cut
//                     settles almost every row (below); the rest use routing's
//                     wave selection, as k_freq_count does for every row.
//   k_freq_rank   per layer: rank_of[e] = number of experts ahead of e in
//                 (count desc, id asc) order; keep_map = ids of rank < keep in
//                 ascending id order.
#include "common.h"
#include "launch.h"

// One wave per logit row, rows walked with a stride so every block sees many;
// the next row's logits are loaded while the current one is selected.  The
// selection is routing's (select_top: order keys, ties to the lower id); each
// of the K winners adds one to its expert's LDS bin, and the block's bins go
// to the int64 totals with one atomic per expert at the end.
template <int VPL>
__global__ __launch_bounds__(256) void k_freq_count(const float* __restrict__ logits, int64_t T, int E, int K,
                                                    int64_t rows_per_layer_blocks, unsigned long long* __restrict__ counts) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int* hist = reinterpret_cast<int*>(smem);
    const int layer = blockIdx.y;
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const int wave = threadIdx.x / WAVE, l = lane_id();
    const float* base = logits + (long)layer * T * E;
    const int64_t step = rows_per_layer_blocks * 4;
    int64_t t = (int64_t)blockIdx.x * 4 + wave;
    float cur[VPL], nxt[VPL];
    auto load = [&](int64_t row, float (&v)[VPL]) __attribute__((always_inline)) {
        const float* r = base + (row < T ? row : T - 1) * E;   // past the end: re-read the last row (unused)
#pragma unroll
        for (int j = 0; j < VPL; j++) {
            const int e = l + j * WAVE;
            v[j] = __builtin_nontemporal_load(r + (e < E ? e : E - 1));
        }
    };
    if (t < T) load(t, cur);
    for (; t < T; t += step) {
        load(t + step, nxt);
        uint32_t kv[VPL];
#pragma unroll
        for (int j = 0; j < VPL; j++) kv[j] = l + j * WAVE < E ? f32_order_key(cur[j]) : 0u;
        uint32_t key;
        int e;
        select_top<VPL>(kv, K, key, e);
        if (l < K && e >= 0) atomicAdd(&hist[e], 1);   // e < 0 only if keys ran out (NaN rows)
#pragma unroll
        for (int j = 0; j < VPL; j++) cur[j] = nxt[j];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        if (hist[e]) atomicAdd(&counts[(long)layer * E + e], (unsigned long long)hist[e]);
}

// Wide rows (E > 128): only the SET of the K winners matters for the counts,
// so a row is first cut at a threshold value th carried over from the rows
// before it (all rows of a wave belong to one layer).  If c, the number of
// values >= th, lies in [K, 64], every winner is among those c candidates
// (the K-th largest value is >= th), so they are packed into one slot per
// lane in expert order (the count and the packing share one ballot per
// compare), and each candidate's rank is the number of others with a larger
// (order key, lower slot) pair -- one 64-bit compare per candidate, four per
// LDS read, no branches.  The K candidates of rank < K are the winners.  The
// row work is vector-ALU bound, so FULL (E = 64 * VPL) drops the per-slot
// bounds checks and three rows are in flight per wave.
// Any other row takes routing's selection, whose K-th and first values then
// reset th (the K-th value minus 3/4 of their spread) and its adjustment
// step; after a cut row th moves by the step to keep c within [K + 3, 28].  The
// threshold only decides which exact method runs, never the result (a NaN
// is never a candidate; NaN rows are unspecified, as in routing).
constexpr int THR_MAX = 64;
constexpr int FR_RING = 3;
template <int VPL, bool FULL>
__global__ __launch_bounds__(256) void k_freq_count_thr(const float* __restrict__ logits, int64_t T, int E, int K,
                                                        int64_t rows_per_layer_blocks,
                                                        unsigned long long* __restrict__ counts) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned long long* comp_all = reinterpret_cast<unsigned long long*>(smem);   // [4][64] candidate ranks keys
    float* cval_all = reinterpret_cast<float*>(comp_all + 4 * THR_MAX);          // [4][64] candidate values
    int* cid_all = reinterpret_cast<int*>(cval_all + 4 * THR_MAX);               // [4][64] candidate experts
    int* hist = cid_all + 4 * THR_MAX;                                           // [E]
    const int layer = blockIdx.y;
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const int wave = threadIdx.x / WAVE, l = lane_id();
    unsigned long long* comp = comp_all + wave * THR_MAX;
    float* cval = cval_all + wave * THR_MAX;
    int* cid = cid_all + wave * THR_MAX;
    const float* base = logits + (long)layer * T * E;
    const int64_t step_rows = rows_per_layer_blocks * 4;
    int64_t t = (int64_t)blockIdx.x * 4 + wave;
    auto load = [&](int64_t row, float (&v)[VPL]) __attribute__((always_inline)) {
        const float* r = base + (row < T ? row : T - 1) * E;   // past the end: re-read the last row (unused)
#pragma unroll
        for (int j = 0; j < VPL; j++) {
            const int e = l + j * WAVE;
            v[j] = __builtin_nontemporal_load(r + (FULL || e < E ? e : E - 1));
        }
    };
    bool have = false;        // wave-uniform threshold state
    float th = 0.f, th_step = 0.f;
    auto process = [&](const float (&cur)[VPL]) __attribute__((always_inline)) {
        auto valid = [&](int j) __attribute__((always_inline)) { return FULL || l + j * WAVE < E; };
        // one pass: count the values at or above th and compact the first
        // THR_MAX of them (used only when the count lands in [K, THR_MAX])
        int c = 0;
        if (have) {
#pragma unroll
            for (int j = 0; j < VPL; j++) {
                const bool in = valid(j) && cur[j] >= th;
                const unsigned long long m = __ballot(in);
                const int p = c + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                if (in && p < THR_MAX) {
                    cval[p] = cur[j];
                    cid[p] = l + j * WAVE;
                }
                c += __popcll(m);
            }
        }
        c = __builtin_amdgcn_readfirstlane(c);
        if (have && c >= K && c <= THR_MAX) {
            __builtin_amdgcn_wave_barrier();
            // slot l's composite: order key (the float order of non-NaN values,
            // -0 == +0), then the lower slot (= lower expert); 0 past c
            const int me = cid[l];
            const unsigned long long mine =
                l < c ? ((unsigned long long)f32_order_key(cval[l]) << 32) | (uint32_t)(WAVE - 1 - l) : 0ull;
            comp[l] = mine;
            __builtin_amdgcn_wave_barrier();
            int rank = 0;
            for (int j = 0; j < c; j += 4) {
                const ulonglong2 q = *reinterpret_cast<const ulonglong2*>(comp + j);   // the same 16 B for every lane
                const ulonglong2 r = *reinterpret_cast<const ulonglong2*>(comp + j + 2);
                rank += q.x > mine ? 1 : 0;
                rank += q.y > mine ? 1 : 0;
                rank += r.x > mine ? 1 : 0;
                rank += r.y > mine ? 1 : 0;
            }
            if (l < c && rank < K) atomicAdd(&hist[me], 1);
            if (c < K + 3) th -= th_step;
            else if (c > 28) th += th_step;
            __builtin_amdgcn_wave_barrier();
        } else {
            uint32_t kv[VPL];
#pragma unroll
            for (int j = 0; j < VPL; j++) kv[j] = valid(j) ? f32_order_key(cur[j]) : 0u;
            uint32_t key;
            int e;
            select_top<VPL>(kv, K, key, e);
            if (l < K && e >= 0) atomicAdd(&hist[e], 1);   // e < 0 only if keys ran out (NaN rows)
            const float v1 = order_key_value(__shfl(key, 0, WAVE));
            const float vk = order_key_value(__shfl(key, K - 1, WAVE));
            const float sp = v1 - vk;
            have = __builtin_isfinite(vk) && __builtin_isfinite(sp) && sp > 0.f && __builtin_isfinite(vk - sp);
            th = vk - 0.75f * sp;
            th_step = 0.125f * sp;
        }
    };
    // ring of FR_RING row buffers: FR_RING - 1 rows in flight while one is selected
    float rb[FR_RING][VPL];
#pragma unroll
    for (int b = 0; b < FR_RING - 1; b++) load(t + b * step_rows, rb[b]);
    bool more = t < T;
    while (more) {
#pragma unroll
        for (int b = 0; b < FR_RING; b++) {
            if (more) {
                load(t + (FR_RING - 1) * step_rows, rb[(b + FR_RING - 1) % FR_RING]);
                process(rb[b]);
                t += step_rows;
                more = t < T;
            }
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        if (hist[e]) atomicAdd(&counts[(long)layer * E + e], (unsigned long long)hist[e]);
}

__global__ __launch_bounds__(256) void k_freq_zero(unsigned long long* __restrict__ counts, long n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) counts[i] = 0ull;
}

__global__ __launch_bounds__(256) void k_freq_rank(const unsigned long long* __restrict__ counts, int E, int keep,
                                                   int32_t* __restrict__ rank_of, int32_t* __restrict__ keep_map) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    long long* c = reinterpret_cast<long long*>(smem);
    int* rk = reinterpret_cast<int*>(c + E);
    const int layer = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x) c[e] = (long long)counts[(long)layer * E + e];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const long long ce = c[e];
        int ahead = 0;
        for (int f = 0; f < E; f++) ahead += (c[f] > ce) || (c[f] == ce && f < e);
        rk[e] = ahead;
        rank_of[(long)layer * E + e] = ahead;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        if (rk[e] < keep) {
            int pos = 0;
            for (int f = 0; f < e; f++) pos += rk[f] < keep;
            keep_map[(long)layer * keep + pos] = e;
        }
    }
}

template <int VPL>
static void count_dispatch(const float* logits, int L, int64_t T, int E, int K, unsigned long long* counts,
                           hipStream_t st) {
    // grid-stride over rows, histogram flushed once per block: about 12288
    // blocks in all (a few rounds of the CUs), at least one per layer
    int64_t blocks = (T + 3) / 4;
    const int64_t cap = (12288 + L - 1) / L;
    if (blocks > cap) blocks = cap;
    dim3 grid((unsigned)blocks, L);
    if constexpr (VPL >= 4 && VPL <= 16) {
        if (K <= THR_MAX) {
            const size_t lds = (size_t)4 * THR_MAX * 16 + (size_t)E * sizeof(int);
            if (E == VPL * WAVE)
                hipLaunchKernelGGL((k_freq_count_thr<VPL, true>), grid, dim3(256), lds, st, logits, T, E, K, blocks,
                                   counts);
            else
                hipLaunchKernelGGL((k_freq_count_thr<VPL, false>), grid, dim3(256), lds, st, logits, T, E, K, blocks,
                                   counts);
            return;
        }
    }
    hipLaunchKernelGGL(k_freq_count<VPL>, grid, dim3(256), (size_t)E * sizeof(int), st, logits, T, E, K, blocks,
                       counts);
}

hipError_t launch_freq(const float* logits, int L, int64_t T, int E, int K, unsigned long long* counts,
                       int accumulate, int keep, int32_t* rank_of, int32_t* keep_map, hipStream_t st) {
    if (!accumulate) {
        const long n = (long)L * E;
        hipLaunchKernelGGL(k_freq_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, counts, n);
    }
    if (T > 0) {
        const int vpl = (E + WAVE - 1) / WAVE;
        if (vpl <= 1) count_dispatch<1>(logits, L, T, E, K, counts, st);
        else if (vpl <= 2) count_dispatch<2>(logits, L, T, E, K, counts, st);
        else if (vpl <= 4) count_dispatch<4>(logits, L, T, E, K, counts, st);
        else if (vpl <= 8) count_dispatch<8>(logits, L, T, E, K, counts, st);
        else if (vpl <= 16) count_dispatch<16>(logits, L, T, E, K, counts, st);
        else if (vpl <= 32) count_dispatch<32>(logits, L, T, E, K, counts, st);
        else count_dispatch<64>(logits, L, T, E, K, counts, st);
    }
    if (keep > 0)
        hipLaunchKernelGGL(k_freq_rank, dim3(L), dim3(256), (size_t)E * (sizeof(long long) + sizeof(int)), st, counts, E,
                           keep, rank_of, keep_map);
    return hipGetLastError();
}
