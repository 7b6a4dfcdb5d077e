// permute.hip -- token->expert grouping (gfx950): per-expert histogram,
// exclusive scan and a stable scatter of the flat slots s = t*K + k.
//
// Grouping the routed rows by expert lets every expert run as one GEMM over
// its rows (each expert's matrices are read once per step; cf. the pages'
// per-expert execution, kwkr.cn Coder write-up, "为什么 Coder 快" part 2).
//
// Determinism: counts commute, but the order in which LDS atomics return does
// not, so positions inside an expert's segment never come from atomic return
// values.  A single wave walks each chunk of slots in ascending order, 64 at a
// time; the lanes holding the same expert set their bits in a per-expert
// 64-bit LDS mask, and a lane's rank is the popcount of the bits below it.
// The result is the stable order (slots ascending within an expert).
#include "common.h"
#include "launch.h"

// Stable scatter of slots [s_begin, s_end) by one wave.  cursor[e] holds the
// next free position of expert e; mask[e] must be zero on entry (and is on exit).
MOE_DEV void wave_stable_scatter(const int32_t* __restrict__ idx, int s_begin, int s_end, int E, int* cursor,
                                 unsigned long long* mask, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    const int l = lane_id();
    const unsigned long long below = (1ull << l) - 1ull;
    for (int g = s_begin; g < s_end; g += WAVE) {
        const int s = g + l;
        int e = s < s_end ? idx[s] : -1;
        const bool valid = (unsigned)e < (unsigned)E;   // out-of-range ids are skipped, never written
        if (!valid) e = 0;
        if (valid) atomicOr(&mask[e], 1ull << l);
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS atomics are done
        __builtin_amdgcn_wave_barrier();
        unsigned long long m = valid ? mask[e] : 0ull;
        int base = valid ? cursor[e] : 0;
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            const int p = base + __popcll(m & below);
            perm[p] = s;
            inv[s] = p;
            if (63 - __clzll(m) == l) {        // the highest lane of this expert advances it
                cursor[e] = base + __popcll(m);
                mask[e] = 0ull;
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
    }
}

// Block-wide exclusive scan of counts[0..E) held in LDS (in place -> offsets).
// Returns the total.  nthreads threads, E <= 4096.
MOE_DEV int block_exclusive_scan(int* v, int E, int* wave_tot) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int per = (E + nthr - 1) / nthr;
    const int b = tid * per;
    int local = 0;
    for (int i = 0; i < per; i++)
        if (b + i < E) local += v[b + i];
    int incl = wave_incl_scan(local);
    const int w = tid / WAVE, nw = nthr / WAVE;
    if (lane_id() == WAVE - 1) wave_tot[w] = incl;
    __syncthreads();
    int wbase = 0, total = 0;
    for (int i = 0; i < nw; i++) {
        if (i < w) wbase += wave_tot[i];
        total += wave_tot[i];
    }
    int run = wbase + incl - local;
    for (int i = 0; i < per; i++)
        if (b + i < E) {
            int c = v[b + i];
            v[b + i] = run;
            run += c;
        }
    __syncthreads();
    return total;
}

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

// Pass 3: stable scatter, one wave per chunk.
__global__ __launch_bounds__(64) void k_perm_scatter(const int32_t* __restrict__ idx, int n, int E,
                                                     const int32_t* __restrict__ chunk_base,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);
    int* cur = reinterpret_cast<int*>(mask + E);
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        cur[e] = offsets[e] + chunk_base[(long)blockIdx.x * E + e];
        mask[e] = 0ull;
    }
    __syncthreads();
    const int s0 = blockIdx.x * PERM_CHUNK, s1 = min(n, s0 + PERM_CHUNK);
    wave_stable_scatter(idx, s0, s1, E, cur, mask, perm, inv);
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
