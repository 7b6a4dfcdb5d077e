// freq.hip -- the expert-pruning statistic (gfx950).
//
// Pruning counts, on calibration data, which experts each token's routing
// selects, and keeps the most-selected experts of every layer, with one keep
// decision for gate, up and down and the kept experts listed in their
// original order ("Strata Coder 编程模型深度剖析", §3 "RCO 专家剪枝是怎么砍一半
// 而不伤脑的"; the per-(layer, expert) ranking of the kwkr.cn Coder write-up,
// "专家配置文件：48 x 256 的全量排名").
//
//   k_freq_count  top-K of every logit row (routing's rule: larger first, ties
//                 to the lower id; the same wave selection as routing's),
//                 per-block LDS histogram, int64 totals via integer atomics
//                 (exact and order-independent).
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
    int64_t blocks = (T + 3) / 4;
    if (blocks > 1024) blocks = 1024;      // grid-stride over rows; histogram flushed once per block
    dim3 grid((unsigned)blocks, L);
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
