// profile.hip -- the expert profile (gfx950 kernels + host file helpers).
//
// An engine fills its fast-memory expert slots in the order of a global
// ranking of every (layer, expert) pair by selection count; a pruned model's
// profile is the full one mapped through its list of kept experts, and the
// share of routed reads that land on the first S ranked pairs checks that the
// mapping is right ("Strata Coder 编程模型深度剖析", §3; kwkr.cn Coder write-up,
// "专家配置文件：48 x 256 的全量排名": its file format, construction and
// hit-rate check).
//
//   k_prof_layer_sort  per layer: each expert's position in (count desc, id
//                      asc) order, and the counts in that order;
//   k_prof_global      per pair: its global rank = its layer position + for
//                      every other layer the number of pairs ahead of it
//                      (count >= c in earlier layers, count > c in later
//                      ones: ties go to the lower flat index), found by binary
//                      search in that layer's sorted counts;
//   k_prof_hits        routed reads whose pair ranks below S, one atomic per
//                      block.
// STRP v1 (little-endian): "STRP", five uint32 (version 1, layers, experts,
// ranked pairs, layers * experts), the pairs as (uint16 layer, uint16 expert)
// in rank order, then per layer an int16 table of each expert's rank, -1 if
// unranked.
#include <string.h>

#include "../../include/moe.h"
#include "common.h"
#include "launch.h"

namespace {

constexpr int PROF_MAX_E = 4096;

// one block per layer; the layer's counts in LDS, each thread ranks E/256 experts
__global__ __launch_bounds__(256) void k_prof_layer_sort(const int64_t* __restrict__ counts, int E,
                                                         int64_t* __restrict__ sorted, int32_t* __restrict__ lrank) {
    __shared__ int64_t c[PROF_MAX_E];
    const int layer = blockIdx.x;
    const int64_t* row = counts + (long)layer * E;
    for (int e = threadIdx.x; e < E; e += blockDim.x) c[e] = row[e];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int64_t ce = c[e];
        int ahead = 0;
        for (int f = 0; f < E; f++) ahead += (c[f] > ce) || (c[f] == ce && f < e);
        lrank[(long)layer * E + e] = ahead;
        sorted[(long)layer * E + ahead] = ce;
    }
}

// entries of a descending array s[0..n) that are >= v (ge) or > v
MOE_DEV int count_ahead(const int64_t* __restrict__ s, int n, int64_t v, bool ge) {
    int lo = 0, hi = n;                    // first index whose entry is < v (ge) or <= v
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const bool ahead = ge ? s[mid] >= v : s[mid] > v;
        if (ahead) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(256) void k_prof_global(const int64_t* __restrict__ counts,
                                                     const int64_t* __restrict__ sorted,
                                                     const int32_t* __restrict__ lrank, int L, int E,
                                                     int32_t* __restrict__ rank, uint32_t* __restrict__ pairs) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)L * E) return;
    const int l = (int)(i / E), e = (int)(i % E);
    const int64_t c = counts[i];
    long g = lrank[i];
    for (int m = 0; m < L; m++)
        if (m != l) g += count_ahead(sorted + (long)m * E, E, c, m < l);
    rank[i] = (int32_t)g;
    pairs[g] = (uint32_t)l | ((uint32_t)e << 16);       // (uint16 layer, uint16 expert)
}

__global__ __launch_bounds__(256) void k_prof_zero(unsigned long long* __restrict__ v) { *v = 0ull; }

__global__ __launch_bounds__(256) void k_prof_hits(const int32_t* __restrict__ trace, int L, long n_per_layer,
                                                   const int32_t* __restrict__ rank, int E, long S,
                                                   unsigned long long* __restrict__ hits) {
    __shared__ unsigned long long part[4];
    const long total = (long)L * n_per_layer;
    unsigned long long h = 0;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
        const int l = (int)(i / n_per_layer);
        const int e = trace[i];
        const bool hit = e >= 0 && e < E && rank[(long)l * E + e] < S;
        h += (unsigned long long)__popcll(__ballot(hit));
    }
    if (lane_id() == 0) part[threadIdx.x / WAVE] = h;
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned long long b = part[0] + part[1] + part[2] + part[3];
        if (b) atomicAdd(hits, b);
    }
}

size_t r256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

extern "C" {

size_t moe_profile_workspace_size(int32_t L, int32_t E) {
    if (L <= 0 || E <= 0) return 0;
    return r256((size_t)L * E * sizeof(int64_t)) + r256((size_t)L * E * sizeof(int32_t));
}

moe_status moe_profile_rank(const int64_t* counts, int32_t L, int32_t E, int32_t* rank, uint16_t* pairs,
                            void* workspace, size_t ws_bytes, moe_stream stream) {
    if (!counts || !rank || !pairs || L <= 0 || E <= 0 || L > 65535) return MOE_ERR_INVALID_ARG;
    if (E > PROF_MAX_E || ((uintptr_t)pairs & 3u)) return MOE_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < moe_profile_workspace_size(L, E)) return MOE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    int64_t* sorted = (int64_t*)workspace;
    int32_t* lrank = (int32_t*)((char*)workspace + r256((size_t)L * E * sizeof(int64_t)));
    hipLaunchKernelGGL(k_prof_layer_sort, dim3(L), dim3(256), 0, st, counts, E, sorted, lrank);
    const long n = (long)L * E;
    hipLaunchKernelGGL(k_prof_global, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, counts, sorted, lrank, L, E,
                       rank, (uint32_t*)pairs);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_profile_hits(const int32_t* trace, int32_t L, int64_t T, int32_t K, const int32_t* rank, int32_t E,
                            int64_t S, uint64_t* hits, moe_stream stream) {
    if (!hits || !rank || L <= 0 || T < 0 || K <= 0 || E <= 0 || S < 0) return MOE_ERR_INVALID_ARG;
    if (T > 0 && !trace) return MOE_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(k_prof_zero, dim3(1), dim3(1), 0, st, (unsigned long long*)hits);
    const long total = (long)L * T * K;
    if (total > 0) {
        long blocks = (total + 255) / 256;
        if (blocks > 2048) blocks = 2048;
        hipLaunchKernelGGL(k_prof_hits, dim3((unsigned)blocks), dim3(256), 0, st, trace, L, (long)T * K, rank, E, S,
                           (unsigned long long*)hits);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ------------------------------------------------------------------ host: STRP file and remap

size_t moe_strp_size(int32_t L, int32_t E, int32_t n_ranked) {
    if (L <= 0 || E <= 0 || n_ranked < 0) return 0;
    return 24 + 4 * (size_t)n_ranked + 2 * (size_t)L * E;
}

static void put_u32(unsigned char* p, uint32_t v) {
    p[0] = (unsigned char)v; p[1] = (unsigned char)(v >> 8); p[2] = (unsigned char)(v >> 16); p[3] = (unsigned char)(v >> 24);
}
static void put_u16(unsigned char* p, uint16_t v) { p[0] = (unsigned char)v; p[1] = (unsigned char)(v >> 8); }
static uint32_t get_u32(const unsigned char* p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
static uint16_t get_u16(const unsigned char* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

moe_status moe_strp_write(const uint16_t* pairs, int32_t n_ranked, int32_t L, int32_t E, void* out,
                          size_t out_bytes) {
    if (!out || L <= 0 || E <= 0 || L > 65535 || E > 65535 || n_ranked < 0 || (n_ranked > 0 && !pairs))
        return MOE_ERR_INVALID_ARG;
    if (n_ranked > 32767 || (long)n_ranked > (long)L * E) return MOE_ERR_UNSUPPORTED;   // int16 ranks
    const size_t need = moe_strp_size(L, E, n_ranked);
    if (out_bytes < need) return MOE_ERR_WORKSPACE;
    unsigned char* p = (unsigned char*)out;
    unsigned char* tail = p + 24 + 4 * (size_t)n_ranked;      // the inverse table, built in place
    for (long i = 0; i < (long)L * E; i++) put_u16(tail + 2 * i, 0xFFFFu);
    for (int r = 0; r < n_ranked; r++) {               // every pair in range and ranked once
        const int l = pairs[2 * r], e = pairs[2 * r + 1];
        if (l >= L || e >= E || get_u16(tail + 2 * ((long)l * E + e)) != 0xFFFFu) return MOE_ERR_INVALID_ARG;
        put_u16(tail + 2 * ((long)l * E + e), (uint16_t)r);
    }
    memcpy(p, "STRP", 4);
    put_u32(p + 4, 1u);
    put_u32(p + 8, (uint32_t)L);
    put_u32(p + 12, (uint32_t)E);
    put_u32(p + 16, (uint32_t)n_ranked);
    put_u32(p + 20, (uint32_t)((long)L * E));
    unsigned char* q = p + 24;
    for (int r = 0; r < n_ranked; r++, q += 4) {
        put_u16(q, pairs[2 * r]);
        put_u16(q + 2, pairs[2 * r + 1]);
    }
    return MOE_OK;
}

moe_status moe_strp_read(const void* buf, size_t bytes, int32_t* L, int32_t* E, int32_t* n_ranked,
                         uint16_t* pairs, int32_t pairs_capacity, int16_t* inverse, int64_t inverse_capacity) {
    if (!buf || !L || !E || !n_ranked) return MOE_ERR_INVALID_ARG;
    const unsigned char* p = (const unsigned char*)buf;
    if (bytes < 24 || memcmp(p, "STRP", 4) != 0) return MOE_ERR_INVALID_ARG;
    const uint32_t version = get_u32(p + 4), l = get_u32(p + 8), e = get_u32(p + 12), n = get_u32(p + 16),
                   entries = get_u32(p + 20);
    if (version != 1u || l == 0 || e == 0 || l > 65535u || e > 65535u || (uint64_t)entries != (uint64_t)l * e ||
        n > entries || bytes != 24 + 4 * (size_t)n + 2 * (size_t)entries)
        return MOE_ERR_INVALID_ARG;
    *L = (int32_t)l;
    *E = (int32_t)e;
    *n_ranked = (int32_t)n;
    if (pairs) {
        if ((uint32_t)pairs_capacity < n) return MOE_ERR_WORKSPACE;
        for (uint32_t r = 0; r < n; r++) {
            pairs[2 * r] = get_u16(p + 24 + 4 * (size_t)r);
            pairs[2 * r + 1] = get_u16(p + 26 + 4 * (size_t)r);
        }
    }
    if (inverse) {
        if ((uint64_t)inverse_capacity < entries) return MOE_ERR_WORKSPACE;
        const unsigned char* q = p + 24 + 4 * (size_t)n;
        for (uint32_t i = 0; i < entries; i++) inverse[i] = (int16_t)get_u16(q + 2 * (size_t)i);
    }
    return MOE_OK;
}

moe_status moe_profile_remap(const uint16_t* pairs, int32_t n, int32_t L, int32_t E_old, const int32_t* keep_map,
                             int32_t keep, uint16_t* out, int32_t* n_out) {
    if (!n_out || n < 0 || L <= 0 || E_old <= 0 || keep < 0 || keep > E_old || (n > 0 && (!pairs || !out)) ||
        (keep > 0 && !keep_map))
        return MOE_ERR_INVALID_ARG;
    for (int l = 0; l < L; l++)                         // each keep list: ascending ids in [0, E_old)
        for (int j = 0; j < keep; j++) {
            const int e = keep_map[(long)l * keep + j];
            if (e < 0 || e >= E_old || (j > 0 && keep_map[(long)l * keep + j - 1] >= e)) return MOE_ERR_INVALID_ARG;
        }
    for (int r = 0; r < n; r++)
        if (pairs[2 * r] >= L || pairs[2 * r + 1] >= E_old) return MOE_ERR_INVALID_ARG;
    int m = 0;
    for (int r = 0; r < n; r++) {
        const int l = pairs[2 * r], e = pairs[2 * r + 1];
        const int32_t* row = keep_map + (long)l * keep;
        int lo = 0, hi = keep;                          // the expert's position in the keep list, if kept
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (row[mid] < e) lo = mid + 1;
            else hi = mid;
        }
        if (lo < keep && row[lo] == e) {
            out[2 * m] = (uint16_t)l;
            out[2 * m + 1] = (uint16_t)lo;
            m++;
        }
    }
    *n_out = m;
    return MOE_OK;
}

}  // extern "C"
