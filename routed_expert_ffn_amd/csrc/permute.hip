// permute.hip -- token->expert grouping (gfx950): per-expert histogram,
// exclusive scan and a stable scatter of the flat slots s = t*K + k.
//
// Grouping the routed rows by expert lets every expert run as one GEMM over
// its rows (each expert's matrices are read once per step; cf. the pages'
// per-expert execution, kwkr.cn Coder write-up, "为什么 Coder 快" part 2).
//
// Determinism: positions inside an expert's segment never come from atomic
// return values; the stable scatter and the block scan are in group.h.
#include "common.h"
#include "group.h"
#include "launch.h"

// Whole grouping in one block (n <= PERM_CHUNK).
__global__ __launch_bounds__(256) void k_perm_small(const int32_t* __restrict__ idx, int n, int E,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);
    int* cur = reinterpret_cast<int*>(mask + E);
    __shared__ int wave_tot[4];
    for (int e = threadIdx.x; e < E; e += blockDim.x) { cur[e] = 0; mask[e] = 0ull; }
    __syncthreads();
    for (int s = threadIdx.x; s < n; s += blockDim.x) {
        const int e = idx[s];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cur[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] = cur[e];
    __syncthreads();
    const int total = block_exclusive_scan(cur, E, wave_tot);
    for (int e = threadIdx.x; e < E; e += blockDim.x) offsets[e] = cur[e];
    if (threadIdx.x == 0) offsets[E] = total;
    __syncthreads();
    if (threadIdx.x < WAVE) wave_stable_scatter(idx, 0, n, E, cur, mask, perm, inv);
}

// Chunked grouping, pass 1: per-chunk histograms chunk_counts[c][e].
__global__ __launch_bounds__(256) void k_perm_hist(const int32_t* __restrict__ idx, int n, int E,
                                                   int32_t* __restrict__ chunk_counts) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int* cnt = reinterpret_cast<int*>(smem);
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int s0 = blockIdx.x * PERM_CHUNK, s1 = min(n, s0 + PERM_CHUNK);
    for (int s = s0 + threadIdx.x; s < s1; s += blockDim.x) {
        const int e = idx[s];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_counts[(long)blockIdx.x * E + e] = cnt[e];
}

// Pass 2 (one block): counts, offsets, and each chunk's first position within
// each expert's segment.
__global__ __launch_bounds__(1024) void k_perm_scan(int32_t* __restrict__ chunk_counts, int nchunks, int E,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int* tot = reinterpret_cast<int*>(smem);
    __shared__ int wave_tot[16];
    // per expert: exclusive prefix over the chunks (16 chunk counts in flight
    // per thread at a time); the scatter adds the expert's offset
    constexpr int B = 16;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int run = 0;
        for (int c0 = 0; c0 < nchunks; c0 += B) {
            int v[B];
#pragma unroll
            for (int u = 0; u < B; u++) v[u] = chunk_counts[(long)min(c0 + u, nchunks - 1) * E + e];
#pragma unroll
            for (int u = 0; u < B; u++)
                if (c0 + u < nchunks) {
                    chunk_counts[(long)(c0 + u) * E + e] = run;
                    run += v[u];
                }
        }
        counts[e] = run;
        tot[e] = run;
    }
    __syncthreads();
    const int total = block_exclusive_scan(tot, E, wave_tot);
    for (int e = threadIdx.x; e < E; e += blockDim.x) offsets[e] = tot[e];
    if (threadIdx.x == 0) offsets[E] = total;
}

// Pass 3: stable scatter, one wave per chunk.  The chunk's expert ids (16
// per lane) and the cursor inputs (8 experts per lane at a time) are loaded
// with all their loads in flight before the scatter's sequential steps.
__global__ __launch_bounds__(64) void k_perm_scatter(const int32_t* __restrict__ idx, int n, int E,
                                                     const int32_t* __restrict__ chunk_base,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);
    int* cur = reinterpret_cast<int*>(mask + E);
    const int l = threadIdx.x;
    constexpr int G = PERM_CHUNK / WAVE;
    const int s0 = blockIdx.x * PERM_CHUNK, s1 = min(n, s0 + PERM_CHUNK);
    int ev[G];
#pragma unroll
    for (int g = 0; g < G; g++) {
        const int s = s0 + g * WAVE + l;
        ev[g] = s < s1 ? idx[s] : -1;
    }
    const int32_t* cb = chunk_base + (long)blockIdx.x * E;
    for (int e0 = 0; e0 < E; e0 += 8 * WAVE) {
        int a[8], b[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int e = e0 + u * WAVE + l;
            a[u] = e < E ? offsets[e] : 0;
            b[u] = e < E ? cb[e] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int e = e0 + u * WAVE + l;
            if (e < E) {
                cur[e] = a[u] + b[u];
                mask[e] = 0ull;
            }
        }
    }
    __syncthreads();
    wave_stable_scatter_regs<G>(ev, s0, s1, E, cur, mask, perm, inv);
}

hipError_t launch_permute(const int32_t* idx, int n, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                          int32_t* inv, int32_t* chunk_buf, hipStream_t st) {
    const size_t lds_ms = (size_t)E * (sizeof(unsigned long long) + sizeof(int));
    if (n <= PERM_CHUNK) {
        hipLaunchKernelGGL(k_perm_small, dim3(1), dim3(256), lds_ms, st, idx, n, E, counts, offsets, perm, inv);
        return hipGetLastError();
    }
    const int nchunks = (n + PERM_CHUNK - 1) / PERM_CHUNK;
    hipLaunchKernelGGL(k_perm_hist, dim3(nchunks), dim3(256), (size_t)E * sizeof(int), st, idx, n, E, chunk_buf);
    hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), (size_t)E * sizeof(int), st, chunk_buf, nchunks, E, counts,
                       offsets);
    hipLaunchKernelGGL(k_perm_scatter, dim3(nchunks), dim3(64), lds_ms, st, idx, n, E, chunk_buf, offsets, perm,
                       inv);
    return hipGetLastError();
}
