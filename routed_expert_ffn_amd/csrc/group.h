// group.h -- device helpers of the token->expert grouping, shared by the
// grouping kernels (permute.hip) and the router's one-block select-and-group
// kernel for a few tokens (route.hip).
//
// Determinism: counts commute, but the order in which LDS atomics return does
// not, so positions inside an expert's segment never come from atomic return
// values.  A single wave walks the slots in ascending order, 64 at a time; the
// lanes holding the same expert set their bits in a per-expert 64-bit LDS
// mask, and a lane's rank is the popcount of the bits below it.  The result is
// the stable order (slots ascending within an expert).
#pragma once
#include "common.h"

// One step of the stable scatter: lane l holds slot s and its expert id e
// (out of range: skipped, never written).  cursor[e] holds the next free
// position of expert e; mask[e] is zero on entry and on exit.
MOE_DEV void scatter_group(int e, int s, int E, int* cursor, unsigned long long* mask, int32_t* __restrict__ perm,
                           int32_t* __restrict__ inv) {
    const int l = lane_id();
    const unsigned long long below = (1ull << l) - 1ull;
    const bool valid = (unsigned)e < (unsigned)E;
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

// Stable scatter of slots [s_begin, s_end) by one wave, 64 slots a step.
MOE_DEV void wave_stable_scatter(const int32_t* __restrict__ idx, int s_begin, int s_end, int E, int* cursor,
                                 unsigned long long* mask, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    const int l = lane_id();
    for (int g = s_begin; g < s_end; g += WAVE) {
        const int s = g + l;
        scatter_group(s < s_end ? idx[s] : -1, s, E, cursor, mask, perm, inv);
    }
}

// The same with the slots' expert ids already in registers: ev[g] holds the
// id of slot s_begin + 64 g + lane (-1 past s_end), s_end - s_begin <= 64 G.
template <int G>
MOE_DEV void wave_stable_scatter_regs(const int (&ev)[G], int s_begin, int s_end, int E, int* cursor,
                                      unsigned long long* mask, int32_t* __restrict__ perm,
                                      int32_t* __restrict__ inv) {
    const int l = lane_id();
#pragma unroll
    for (int g = 0; g < G; g++) {
        if (s_begin + g * WAVE >= s_end) break;   // uniform
        scatter_group(ev[g], s_begin + g * WAVE + l, E, cursor, mask, perm, inv);
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
