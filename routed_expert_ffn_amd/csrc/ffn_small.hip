// ffn_small.hip -- the expert FFN when every expert has at most 16 rows
// (T <= 16: the speculative verify step of 4 drafts + 1, and decode).
//
// Here the layer is a pure stream of expert weights (each touched expert's
// gate, up and down matrices are read once, ~1 flop per byte), so the kernels
// are built for HBM bandwidth, not MFMA throughput:
//   * no LDS staging: every lane streams its part of a 16-row weight tile
//     straight from HBM into registers (non-temporal 16-byte loads) through a
//     ring of up to 8 steps; loads are never predicated, so the compiler
//     waits for the oldest load only;
//   * the MFMA 16x16x32 does the dot products: the expert's <= 16 token rows
//     are the A operand (rows past the expert's count read a valid row and
//     are zeroed), the weight tile is the B operand, no cross-lane reductions;
//   * gate/up splits K over the 4 waves of a block (each wave a quarter of
//     H, partial sums added through LDS in a fixed order), so a block is 16
//     feature rows of gate AND up and the grid has enough blocks to fill all
//     CUs; down gives each wave 16 hidden rows over the full (short) K = F.
//   * a small preparation kernel lists the touched experts and gathers the
//     token rows in grouped order, so every FFN block starts streaming after
//     one dependent load; the grid only depends on T*K, and blockIdx.x runs
//     over the tiles of one expert (blocks dispatched together read one
//     expert's matrix contiguously).
// int4 weights: each 32-element block along K is one MFMA K step.  The
// nibbles u become the bf16 values 128 + u (bit pattern 0x4300 | u, exact);
// with the weight d (u - 8):
//     sum_k x w = d (D - 136 S),  D = MFMA(x, 128 + u),  S = MFMA(x, 1)
// so the row sums S come out of the same MFMA layout, and the weights enter
// exactly (no rounding of d * q).
#include "common.h"
#include "launch.h"

enum { SDT_BF16 = 1, SDT_INT4 = 2 };
constexpr int SM_ROWS = 16;     // rows per expert handled (T <= 16)
constexpr int GU_SPLIT = 4;     // gate/up: waves per block sharing one 16-row tile, each a quarter of K

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

MOE_DEV float silu_s(float g) { return g / (1.0f + expf(-g)); }

MOE_DEV uint4 ld_nt(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
MOE_DEV uint32_t ld_nt32(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)); }
MOE_DEV uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
MOE_DEV uint4 zero_unless(bool keep, uint4 v) {
    return keep ? v : make_uint4(0, 0, 0, 0);
}

// Preparation (one small kernel ahead of the FFN kernels, so their blocks
// start streaming weights after a single dependent load):
//   * list[j] = (expert, first row, rows) of the j-th expert with rows, in
//     expert order; entries past the last touched expert hold expert -1;
//   * xp[p] = x[perm[p] / K]: the token rows gathered in grouped order.
__global__ __launch_bounds__(256) void k_small_prep(const uint16_t* __restrict__ x,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ perm, int K, int H, int E, int n,
                                                    int slots, int4* __restrict__ list, uint16_t* __restrict__ xp) {
    const int row_chunks = H / 8;
    const long total = (long)n * row_chunks;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
        const int r = (int)(i / row_chunks), c = (int)(i % row_chunks) * 8;
        const long t = perm[r] / K;
        *reinterpret_cast<uint4*>(xp + (long)r * H + c) = *reinterpret_cast<const uint4*>(x + t * H + c);
    }
    if (blockIdx.x != 0 || threadIdx.x >= WAVE) return;
    const int l = lane_id();
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += WAVE) {
        const int e = e0 + l;
        int o = 0, c = 0;
        if (e < E) { o = offsets[e]; c = offsets[e + 1] - o; }
        const int t = c > 0 ? 1 : 0;
        const int incl = wave_incl_scan(t);
        if (t) list[base + incl - 1] = make_int4(e, o, c, 0);
        base += __shfl(incl, WAVE - 1, WAVE);
    }
    for (int j = base + l; j < slots; j += WAVE) list[j] = make_int4(-1, 0, 0, 0);
}

MOE_DEV bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 8 nibbles (one lane's 8 consecutive int4 weights) -> bf16 values 128 + u.
MOE_DEV uint4 nib8_to_bf16_128(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu;          // elements 0,2,4,6
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // elements 1,3,5,7
    uint4 o;
    // dword i holds elements (2i, 2i+1): bytes (lo.byte i, 0, hi.byte i, 0)
    o.x = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x43004300u;
    o.y = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x43004300u;
    o.z = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x43004300u;
    o.w = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x43004300u;
    return o;
}

MOE_DEV uint4 bf16_ones() { return make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u); }

MOE_DEV f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------- gate/up

template <int WT, int RING>
__global__ __launch_bounds__(256) void k_gateup_small(const uint16_t* __restrict__ xp, const void* __restrict__ wg_,
                                                      const void* __restrict__ wu_, const uint16_t* __restrict__ sg,
                                                      const uint16_t* __restrict__ su, const int4* __restrict__ list,
                                                      int H, int F, uint16_t* __restrict__ abuf) {
    __shared__ f32x4_t s_part[GU_SPLIT - 1][2][WAVE];
    const int tid = threadIdx.x;
    const int4 ent = list[blockIdx.y];
    const int e = ent.x, off = ent.y, n = ent.z;
    if (e < 0) return;
    const int wave = tid / WAVE, l = lane_id();
    const int f0 = blockIdx.x * 16;
    const int row = l & 15, grp = l >> 4;
    const bool arow = row < n;
    const int steps = H / 32 / GU_SPLIT;            // K steps of this wave
    const int k0 = wave * steps * 32;               // this wave's quarter of H
    const uint16_t* xa = xp + (long)(off + (arow ? row : 0)) * H + k0 + grp * 8;

    f32x4_t ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
    if constexpr (WT == SDT_BF16) {
        const uint16_t* pg = (const uint16_t*)wg_ + ((long)e * F + f0 + row) * H + k0 + grp * 8;
        const uint16_t* pu = (const uint16_t*)wu_ + ((long)e * F + f0 + row) * H + k0 + grp * 8;
        uint4 rg[RING], ru[RING], rx[RING];
#pragma unroll
        for (int i = 0; i < RING; i++) {
            rg[i] = ld_nt(pg + i * 32);
            ru[i] = ld_nt(pu + i * 32);
            rx[i] = ld16(xa + i * 32);
        }
        for (int s0 = 0; s0 < steps - RING; s0 += RING) {
#pragma unroll
            for (int i = 0; i < RING; i++) {
                const int s = s0 + i;
                const uint4 av = zero_unless(arow, rx[i]);
                ag = mfma(av, rg[i], ag);
                au = mfma(av, ru[i], au);
                rg[i] = ld_nt(pg + (s + RING) * 32);
                ru[i] = ld_nt(pu + (s + RING) * 32);
                rx[i] = ld16(xa + (s + RING) * 32);
            }
        }
#pragma unroll
        for (int i = 0; i < RING; i++) {
            const uint4 av = zero_unless(arow, rx[i]);
            ag = mfma(av, rg[i], ag);
            au = mfma(av, ru[i], au);
        }
    } else {
        // lane: 4 bytes (8 nibbles) of its row per step, plus the row's block scale
        const long rowg = (long)e * F + f0 + row;
        const uint8_t* pg = (const uint8_t*)wg_ + rowg * (H / 2) + k0 / 2 + grp * 4;
        const uint8_t* pu = (const uint8_t*)wu_ + rowg * (H / 2) + k0 / 2 + grp * 4;
        const uint16_t* qg = sg + rowg * (H / 32) + k0 / 32;
        const uint16_t* qu = su + rowg * (H / 32) + k0 / 32;
        uint32_t rg[RING], ru[RING];
        uint16_t dg[RING], du[RING];
        uint4 rx[RING];
#pragma unroll
        for (int i = 0; i < RING; i++) {
            rg[i] = ld_nt32(pg + i * 16);
            ru[i] = ld_nt32(pu + i * 16);
            dg[i] = qg[i];
            du[i] = qu[i];
            rx[i] = ld16(xa + i * 32);
        }
        auto step = [&](uint4 xv, uint32_t wgq, uint32_t wuq, uint16_t dgs, uint16_t dus) __attribute__((always_inline)) {
            const uint4 av = zero_unless(arow, xv);
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            const f32x4_t S = mfma(av, bf16_ones(), z);
            const f32x4_t Dg = mfma(av, nib8_to_bf16_128(wgq), z);
            const f32x4_t Du = mfma(av, nib8_to_bf16_128(wuq), z);
            // the scale of this lane's weight row is the scale of its output column (lane & 15)
            const float dgc = fp16_to_f32(dgs), duc = fp16_to_f32(dus);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                ag[r] = fmaf(dgc, fmaf(-136.0f, S[r], Dg[r]), ag[r]);
                au[r] = fmaf(duc, fmaf(-136.0f, S[r], Du[r]), au[r]);
            }
        };
        for (int s0 = 0; s0 < steps - RING; s0 += RING) {
#pragma unroll
            for (int i = 0; i < RING; i++) {
                const int s = s0 + i;
                step(rx[i], rg[i], ru[i], dg[i], du[i]);
                rg[i] = ld_nt32(pg + (s + RING) * 16);
                ru[i] = ld_nt32(pu + (s + RING) * 16);
                dg[i] = qg[s + RING];
                du[i] = qu[s + RING];
                rx[i] = ld16(xa + (s + RING) * 32);
            }
        }
#pragma unroll
        for (int i = 0; i < RING; i++) step(rx[i], rg[i], ru[i], dg[i], du[i]);
    }
    // split-K: waves 1..3 hand their partial sums to wave 0, which adds them in wave order
    if (wave > 0) {
        s_part[wave - 1][0][l] = ag;
        s_part[wave - 1][1][l] = au;
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < GU_SPLIT - 1; w++) {
        ag += s_part[w][0][l];
        au += s_part[w][1][l];
    }
    // D[m][c]: lane holds rows m = grp*4 + r, column c = l & 15 (feature f0 + c)
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int m = grp * 4 + r;
        if (m < n) abuf[(long)(off + m) * F + f0 + (l & 15)] = f32_to_bf16_rne(silu_s(ag[r]) * au[r]);
    }
}

// ---------------------------------------------------------------------------- down

template <int WT, int YBF16, int RING>
__global__ __launch_bounds__(256) void k_down_small(const uint16_t* __restrict__ abuf, const void* __restrict__ wd_,
                                                    const uint16_t* __restrict__ sd, const int4* __restrict__ list,
                                                    int H, int F, void* __restrict__ y) {
    const int tid = threadIdx.x;
    const int4 ent = list[blockIdx.y];
    const int e = ent.x, off = ent.y, n = ent.z;
    if (e < 0) return;
    const int wave = tid / WAVE, l = lane_id();
    const int h0 = (blockIdx.x * 4 + wave) * 16;
    const int row = l & 15, grp = l >> 4;
    const bool arow = row < n;
    const uint16_t* ap = abuf + (long)(off + (arow ? row : 0)) * F + grp * 8;
    const int steps = F / 32;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (WT == SDT_BF16) {
        const uint16_t* pw = (const uint16_t*)wd_ + ((long)e * H + h0 + row) * F + grp * 8;
        uint4 rw[RING], ra[RING];
#pragma unroll
        for (int i = 0; i < RING; i++) {
            rw[i] = ld_nt(pw + i * 32);
            ra[i] = ld16(ap + i * 32);
        }
        for (int s0 = 0; s0 < steps - RING; s0 += RING) {
#pragma unroll
            for (int i = 0; i < RING; i++) {
                const int s = s0 + i;
                acc = mfma(zero_unless(arow, ra[i]), rw[i], acc);
                rw[i] = ld_nt(pw + (s + RING) * 32);
                ra[i] = ld16(ap + (s + RING) * 32);
            }
        }
#pragma unroll
        for (int i = 0; i < RING; i++) acc = mfma(zero_unless(arow, ra[i]), rw[i], acc);
    } else {
        const long rowg = (long)e * H + h0 + row;
        const uint8_t* pw = (const uint8_t*)wd_ + rowg * (F / 2) + grp * 4;
        const uint16_t* qd = sd + rowg * (F / 32);
        uint32_t rw[RING];
        uint16_t dw[RING];
        uint4 ra[RING];
#pragma unroll
        for (int i = 0; i < RING; i++) {
            rw[i] = ld_nt32(pw + i * 16);
            dw[i] = qd[i];
            ra[i] = ld16(ap + i * 32);
        }
        auto step = [&](uint4 a, uint32_t wq, uint16_t ds) __attribute__((always_inline)) {
            const uint4 av = zero_unless(arow, a);
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            const f32x4_t S = mfma(av, bf16_ones(), z);
            const f32x4_t D = mfma(av, nib8_to_bf16_128(wq), z);
            const float dc = fp16_to_f32(ds);
#pragma unroll
            for (int r = 0; r < 4; r++) acc[r] = fmaf(dc, fmaf(-136.0f, S[r], D[r]), acc[r]);
        };
        for (int s0 = 0; s0 < steps - RING; s0 += RING) {
#pragma unroll
            for (int i = 0; i < RING; i++) {
                const int s = s0 + i;
                step(ra[i], rw[i], dw[i]);
                rw[i] = ld_nt32(pw + (s + RING) * 16);
                dw[i] = qd[s + RING];
                ra[i] = ld16(ap + (s + RING) * 32);
            }
        }
#pragma unroll
        for (int i = 0; i < RING; i++) step(ra[i], rw[i], dw[i]);
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int m = grp * 4 + r;
        if (m < n) {
            const long o = (long)(off + m) * H + h0 + (l & 15);
            if constexpr (YBF16) ((uint16_t*)y)[o] = f32_to_bf16_rne(acc[r]);
            else ((float*)y)[o] = acc[r];
        }
    }
}

// ---------------------------------------------------------------------------- host

static int ring_for(int steps) {
    return steps % 8 == 0 ? 8 : steps % 4 == 0 ? 4 : steps % 2 == 0 ? 2 : 1;
}

bool ffn_small_eligible(int T, int H, int F) {
    return T <= SM_ROWS && H % (32 * GU_SPLIT) == 0 && F % 64 == 0 && H % 64 == 0;
}

static size_t al256(size_t b) { return (b + 255) / 256 * 256; }

// Workspace of the small path: [A: n x F bf16][list: slots x int4][xp: n x H bf16].
size_t ffn_small_workspace_bytes(int T, int K, int E, int H, int F) {
    const size_t n = (size_t)T * K, slots = (size_t)(E < (int)n ? E : (int)n);
    return al256(n * F * 2) + al256(slots * 16) + al256(n * H * 2);
}

template <int WT, int RG>
static void gateup_small(dim3 g, hipStream_t st, const uint16_t* xp, const void* wg, const void* wu, const void* sg,
                         const void* su, const int4* list, int H, int F, uint16_t* abuf) {
    hipLaunchKernelGGL((k_gateup_small<WT, RG>), g, dim3(256), 0, st, xp, wg, wu, (const uint16_t*)sg,
                       (const uint16_t*)su, list, H, F, abuf);
}

template <int WT, int YB, int RG>
static void down_small(dim3 g, hipStream_t st, const uint16_t* abuf, const void* wd, const void* sd, const int4* list,
                       int H, int F, void* y) {
    hipLaunchKernelGGL((k_down_small<WT, YB, RG>), g, dim3(256), 0, st, abuf, wd, (const uint16_t*)sd, list, H, F, y);
}

template <int WT>
static void launch_wt(const uint16_t* xp, const void* wg, const void* wu, const void* wd, const void* sg,
                      const void* su, const void* sd, const int4* list, int slots, int H, int F, void* y,
                      int y_bf16, uint16_t* abuf, hipStream_t st) {
    dim3 gg(F / 16, slots), gd(H / 64, slots);
    switch (ring_for(H / 32 / GU_SPLIT)) {
        case 8: gateup_small<WT, 8>(gg, st, xp, wg, wu, sg, su, list, H, F, abuf); break;
        case 4: gateup_small<WT, 4>(gg, st, xp, wg, wu, sg, su, list, H, F, abuf); break;
        case 2: gateup_small<WT, 2>(gg, st, xp, wg, wu, sg, su, list, H, F, abuf); break;
        default: gateup_small<WT, 1>(gg, st, xp, wg, wu, sg, su, list, H, F, abuf); break;
    }
    const int rd = ring_for(F / 32);
    if (y_bf16) {
        if (rd == 8) down_small<WT, 1, 8>(gd, st, abuf, wd, sd, list, H, F, y);
        else if (rd == 4) down_small<WT, 1, 4>(gd, st, abuf, wd, sd, list, H, F, y);
        else down_small<WT, 1, 2>(gd, st, abuf, wd, sd, list, H, F, y);
    } else {
        if (rd == 8) down_small<WT, 0, 8>(gd, st, abuf, wd, sd, list, H, F, y);
        else if (rd == 4) down_small<WT, 0, 4>(gd, st, abuf, wd, sd, list, H, F, y);
        else down_small<WT, 0, 2>(gd, st, abuf, wd, sd, list, H, F, y);
    }
}

hipError_t launch_ffn_small(const void* x, int w_dtype, const void* wg, const void* wu, const void* wd,
                            const void* sg, const void* su, const void* sd, const int32_t* offsets,
                            const int32_t* perm, int T, int K, int H, int F, int E, void* y, int y_bf16, void* ws,
                            hipStream_t st) {
    // bf16, T <= 8: the persistent streaming kernels (no preparation pass)
    if (w_dtype == SDT_BF16 && ffn_stream_eligible(T, K, E, H, F))
        return launch_ffn_stream(x, wg, wu, wd, offsets, perm, T, K, H, F, E, y, y_bf16, ws, st);
    if (w_dtype == SDT_INT4 && ffn_stream_q4_eligible(T, K, E, H, F))
        return launch_ffn_stream_q4(x, wg, wu, wd, sg, su, sd, offsets, perm, T, K, H, F, E, y, y_bf16, ws, st);
    const int n = T * K;
    const int slots = E < n ? E : n;          // at most this many experts are touched
    char* base = (char*)ws;
    uint16_t* abuf = (uint16_t*)base;
    int4* list = (int4*)(base + al256((size_t)n * F * 2));
    uint16_t* xp = (uint16_t*)(base + al256((size_t)n * F * 2) + al256((size_t)slots * 16));
    const long chunks = (long)n * H / 8;
    const int prep_blocks = (int)((chunks + 255) / 256);
    hipLaunchKernelGGL(k_small_prep, dim3(prep_blocks > 0 ? prep_blocks : 1), dim3(256), 0, st, (const uint16_t*)x,
                       offsets, perm, K, H, E, n, slots, list, xp);
    if (w_dtype == SDT_BF16)
        launch_wt<SDT_BF16>(xp, wg, wu, wd, sg, su, sd, list, slots, H, F, y, y_bf16, abuf, st);
    else
        launch_wt<SDT_INT4>(xp, wg, wu, wd, sg, su, sd, list, slots, H, F, y, y_bf16, abuf, st);
    return hipGetLastError();
}
