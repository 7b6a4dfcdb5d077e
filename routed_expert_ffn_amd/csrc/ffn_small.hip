// ffn_small.hip -- the expert FFN when every expert has at most 16 rows
// (T <= 16: the speculative verify step of 4 drafts + 1 and decode).
//
// Here the layer is a pure stream of expert weights (each touched expert's
// gate, up and down matrices are read once, ~1 flop per byte), so the
// kernels are built for HBM bandwidth, not for MFMA throughput:
//   * no LDS staging of weights: every lane streams its part of a 16-row
//     weight tile straight from HBM into registers through a ring of up to 8
//     16-byte loads, which keeps enough bytes in flight per CU;
//   * the MFMA 16x16x32 does the dot products (the expert's <= 16 token rows
//     are the A operand, zero-padded), so no cross-lane reductions are needed;
//   * one block covers one touched expert and 64 output rows (4 waves x 16);
//     a block finds its expert by a wave-wide scan of the expert offsets, so
//     the grid only depends on T*K.
//
//   k_gateup_small  a = silu(Wg x) * (Wu x) for 16 feature rows per wave, both
//                   gate and up streamed together (their epilogue meets in
//                   registers); x rows staged in LDS; a -> bf16 workspace.
//   k_down_small    y = Wd a for 16 hidden rows per wave (K = F is short, the
//                   whole A tile is held in registers).
// int4 weights: each 32-element block along K is exactly one MFMA K step.  The
// nibbles become the bf16 values 128 + u (bit pattern 0x4300 | u, exact), so
// the MFMA gives D = sum x (128 + u); since the weight is d (u - 8),
//     sum x w = d (D - 136 sum x)
// with sum x over the block precomputed per row.  The weights enter exactly
// (no rounding of d*q).
#include "common.h"
#include "launch.h"

enum { SDT_BF16 = 1, SDT_INT4 = 2 };
constexpr int SM_ROWS = 16;     // rows per expert handled (T <= 16)

MOE_DEV float silu_s(float g) { return g / (1.0f + expf(-g)); }

// The j-th expert with a non-empty segment (-1 if none); result in every lane.
MOE_DEV int find_touched(const int32_t* __restrict__ offsets, int E, int j, int& off, int& n) {
    const int l = lane_id();
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += WAVE) {
        const int e = e0 + l;
        int o = 0, c = 0;
        if (e < E) { o = offsets[e]; c = offsets[e + 1] - o; }
        const int t = c > 0 ? 1 : 0;
        const int incl = wave_incl_scan(t);
        const bool hit = t && (base + incl - 1 == j);
        const unsigned long long m = __ballot(hit);
        if (m) {
            const int src = __ffsll((long long)m) - 1;
            off = __shfl(o, src, WAVE);
            n = __shfl(c, src, WAVE);
            return e0 + src;
        }
        base += __shfl(incl, WAVE - 1, WAVE);
    }
    return -1;
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

// ---------------------------------------------------------------------------- gate/up

template <int WT, int RING>
__global__ __launch_bounds__(256) void k_gateup_small(const uint16_t* __restrict__ x, const void* __restrict__ wg_,
                                                      const void* __restrict__ wu_, const uint16_t* __restrict__ sg,
                                                      const uint16_t* __restrict__ su,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ perm, int K, int H, int F, int E,
                                                      int rows_cap, uint16_t* __restrict__ abuf) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ int s_info[3];
    const int tid = threadIdx.x;
    if (tid < WAVE) {
        int off = 0, n = 0;
        const int e = find_touched(offsets, E, blockIdx.x, off, n);
        if (tid == 0) { s_info[0] = e; s_info[1] = off; s_info[2] = n; }
    }
    __syncthreads();
    const int e = s_info[0], off = s_info[1], n = s_info[2];
    if (e < 0) return;
    const int LDX = H + 8;                       // padded row (bank spread)
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
    float* xsum = reinterpret_cast<float*>(smem + (size_t)rows_cap * LDX * 2);   // [rows][H/32] (int4 only)
    // stage the expert's token rows
    const int chunks = H / 8;
    for (int i = tid; i < n * chunks; i += blockDim.x) {
        const int r = i / chunks, c = (i % chunks) * 8;
        const long t = perm[off + r] / K;
        *reinterpret_cast<uint4*>(&xs[r * LDX + c]) = *reinterpret_cast<const uint4*>(x + t * H + c);
    }
    __syncthreads();
    if constexpr (WT == SDT_INT4) {
        const int nb = H / 32;
        for (int i = tid; i < n * nb; i += blockDim.x) {
            const int r = i / nb, b = i % nb;
            float s = 0.f;
            for (int k = 0; k < 32; k++) s += bf16_to_f32(xs[r * LDX + b * 32 + k]);
            xsum[r * nb + b] = s;
        }
        __syncthreads();
    }
    const int wave = tid / WAVE, l = lane_id();
    const int f0 = (blockIdx.y * 4 + wave) * 16;
    if (f0 >= F) return;
    const int row = l & 15, grp = l >> 4;
    const bool arow = row < n;
    const uint16_t* xa = xs + row * LDX + grp * 8;
    const int steps = H / 32;

    f32x4_t ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
    if constexpr (WT == SDT_BF16) {
        const uint16_t* pg = (const uint16_t*)wg_ + ((long)e * F + f0 + row) * H + grp * 8;
        const uint16_t* pu = (const uint16_t*)wu_ + ((long)e * F + f0 + row) * H + grp * 8;
        uint4 rg[RING], ru[RING];
#pragma unroll
        for (int i = 0; i < RING; i++) {
            rg[i] = *reinterpret_cast<const uint4*>(pg + i * 32);
            ru[i] = *reinterpret_cast<const uint4*>(pu + i * 32);
        }
        // steady state: consume step s, refill its slot with step s + RING (no conditional loads,
        // so the compiler can wait for the oldest load only)
        for (int s0 = 0; s0 < steps - RING; s0 += RING) {
#pragma unroll
            for (int i = 0; i < RING; i++) {
                const int s = s0 + i;
                const uint4 av = arow ? *reinterpret_cast<const uint4*>(xa + s * 32) : make_uint4(0, 0, 0, 0);
                ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(rg[i]), ag, 0, 0, 0);
                au = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(ru[i]), au, 0, 0, 0);
                rg[i] = *reinterpret_cast<const uint4*>(pg + (s + RING) * 32);
                ru[i] = *reinterpret_cast<const uint4*>(pu + (s + RING) * 32);
            }
        }
#pragma unroll
        for (int i = 0; i < RING; i++) {
            const int s = steps - RING + i;
            const uint4 av = arow ? *reinterpret_cast<const uint4*>(xa + s * 32) : make_uint4(0, 0, 0, 0);
            ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(rg[i]), ag, 0, 0, 0);
            au = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(ru[i]), au, 0, 0, 0);
        }
    } else {
        // lane: 4 bytes (8 nibbles) of its row per step, plus the row's block scale
        const long rowg = (long)e * F + f0 + row;
        const uint32_t* pg = reinterpret_cast<const uint32_t*>((const uint8_t*)wg_ + rowg * (H / 2) + grp * 4);
        const uint32_t* pu = reinterpret_cast<const uint32_t*>((const uint8_t*)wu_ + rowg * (H / 2) + grp * 4);
        const uint16_t* qg = sg + rowg * (H / 32);
        const uint16_t* qu = su + rowg * (H / 32);
        const int nb = H / 32;
        // correction rows: this lane's output rows are (grp*4 + r)
        const float* xs_r[4];
#pragma unroll
        for (int r = 0; r < 4; r++) xs_r[r] = xsum + (grp * 4 + r < n ? grp * 4 + r : 0) * nb;
        uint32_t rg[RING], ru[RING];
        uint16_t dg[RING], du[RING];
#pragma unroll
        for (int i = 0; i < RING; i++) {
            rg[i] = pg[i * 4];
            ru[i] = pu[i * 4];
            dg[i] = qg[i];
            du[i] = qu[i];
        }
        auto step = [&](int s, uint32_t wgq, uint32_t wuq, uint16_t dgs, uint16_t dus) __attribute__((always_inline)) {
            const uint4 av = arow ? *reinterpret_cast<const uint4*>(xa + s * 32) : make_uint4(0, 0, 0, 0);
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            const f32x4_t Dg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(nib8_to_bf16_128(wgq)), z, 0, 0, 0);
            const f32x4_t Du = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(nib8_to_bf16_128(wuq)), z, 0, 0, 0);
            // the scale of this lane's weight row is the scale of its output column (lane & 15)
            const float dgc = fp16_to_f32(dgs), duc = fp16_to_f32(dus);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float c = 136.0f * xs_r[r][s];
                ag[r] = fmaf(dgc, Dg[r] - c, ag[r]);
                au[r] = fmaf(duc, Du[r] - c, au[r]);
            }
        };
        for (int s0 = 0; s0 < steps - RING; s0 += RING) {
#pragma unroll
            for (int i = 0; i < RING; i++) {
                const int s = s0 + i;
                step(s, rg[i], ru[i], dg[i], du[i]);
                rg[i] = pg[(s + RING) * 4];
                ru[i] = pu[(s + RING) * 4];
                dg[i] = qg[s + RING];
                du[i] = qu[s + RING];
            }
        }
#pragma unroll
        for (int i = 0; i < RING; i++) step(steps - RING + i, rg[i], ru[i], dg[i], du[i]);
        (void)nb;
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
                                                    const uint16_t* __restrict__ sd,
                                                    const int32_t* __restrict__ offsets, int H, int F, int E,
                                                    void* __restrict__ y) {
    __shared__ int s_info[3];
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float* asum = reinterpret_cast<float*>(smem);     // [16][F/32] (int4 only)
    const int tid = threadIdx.x;
    if (tid < WAVE) {
        int off = 0, n = 0;
        const int e = find_touched(offsets, E, blockIdx.x, off, n);
        if (tid == 0) { s_info[0] = e; s_info[1] = off; s_info[2] = n; }
    }
    __syncthreads();
    const int e = s_info[0], off = s_info[1], n = s_info[2];
    if (e < 0) return;
    const int nb = F / 32;
    if constexpr (WT == SDT_INT4) {
        for (int i = tid; i < n * nb; i += blockDim.x) {
            const int r = i / nb, b = i % nb;
            const uint16_t* a = abuf + (long)(off + r) * F + b * 32;
            float s = 0.f;
            for (int k = 0; k < 32; k++) s += bf16_to_f32(a[k]);
            asum[r * nb + b] = s;
        }
        __syncthreads();
    }
    const int wave = tid / WAVE, l = lane_id();
    const int h0 = (blockIdx.y * 4 + wave) * 16;
    if (h0 >= H) return;
    const int row = l & 15, grp = l >> 4;
    const bool arow = row < n;
    const uint16_t* ap = abuf + (long)(off + (arow ? row : 0)) * F + grp * 8;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int steps = nb;
    if constexpr (WT == SDT_BF16) {
        const uint16_t* pw = (const uint16_t*)wd_ + ((long)e * H + h0 + row) * F + grp * 8;
        uint4 rw[RING];
#pragma unroll
        for (int i = 0; i < RING; i++) rw[i] = *reinterpret_cast<const uint4*>(pw + i * 32);
        for (int s0 = 0; s0 < steps - RING; s0 += RING) {
#pragma unroll
            for (int i = 0; i < RING; i++) {
                const int s = s0 + i;
                const uint4 av = arow ? *reinterpret_cast<const uint4*>(ap + s * 32) : make_uint4(0, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(rw[i]), acc, 0, 0, 0);
                rw[i] = *reinterpret_cast<const uint4*>(pw + (s + RING) * 32);
            }
        }
#pragma unroll
        for (int i = 0; i < RING; i++) {
            const int s = steps - RING + i;
            const uint4 av = arow ? *reinterpret_cast<const uint4*>(ap + s * 32) : make_uint4(0, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(rw[i]), acc, 0, 0, 0);
        }
    } else {
        const long rowg = (long)e * H + h0 + row;
        const uint32_t* pw = reinterpret_cast<const uint32_t*>((const uint8_t*)wd_ + rowg * (F / 2) + grp * 4);
        const uint16_t* qd = sd + rowg * nb;
        const float* as_r[4];
#pragma unroll
        for (int r = 0; r < 4; r++) as_r[r] = asum + (grp * 4 + r < n ? grp * 4 + r : 0) * nb;
        uint32_t rw[RING];
        uint16_t dw[RING];
#pragma unroll
        for (int i = 0; i < RING; i++) { rw[i] = pw[i * 4]; dw[i] = qd[i]; }
        auto step = [&](int s, uint32_t wq, uint16_t ds) __attribute__((always_inline)) {
            const uint4 av = arow ? *reinterpret_cast<const uint4*>(ap + s * 32) : make_uint4(0, 0, 0, 0);
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            const f32x4_t D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(nib8_to_bf16_128(wq)), z, 0, 0, 0);
            const float dc = fp16_to_f32(ds);
#pragma unroll
            for (int r = 0; r < 4; r++) acc[r] = fmaf(dc, D[r] - 136.0f * as_r[r][s], acc[r]);
        };
        for (int s0 = 0; s0 < steps - RING; s0 += RING) {
#pragma unroll
            for (int i = 0; i < RING; i++) {
                const int s = s0 + i;
                step(s, rw[i], dw[i]);
                rw[i] = pw[(s + RING) * 4];
                dw[i] = qd[s + RING];
            }
        }
#pragma unroll
        for (int i = 0; i < RING; i++) step(steps - RING + i, rw[i], dw[i]);
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
    return T <= SM_ROWS && H % 64 == 0 && F % 64 == 0;
}

template <int WT, int RG>
static void gateup_small(dim3 g, size_t lds, hipStream_t st, const void* x, const void* wg, const void* wu,
                         const void* sg, const void* su, const int32_t* offsets, const int32_t* perm, int K, int H,
                         int F, int E, int rows_cap, uint16_t* abuf) {
    hipLaunchKernelGGL((k_gateup_small<WT, RG>), g, dim3(256), lds, st, (const uint16_t*)x, wg, wu,
                       (const uint16_t*)sg, (const uint16_t*)su, offsets, perm, K, H, F, E, rows_cap, abuf);
}

template <int WT, int YB, int RG>
static void down_small(dim3 g, size_t lds, hipStream_t st, const uint16_t* abuf, const void* wd, const void* sd,
                       const int32_t* offsets, int H, int F, int E, void* y) {
    hipLaunchKernelGGL((k_down_small<WT, YB, RG>), g, dim3(256), lds, st, abuf, wd, (const uint16_t*)sd, offsets, H,
                       F, E, y);
}

template <int WT>
static void launch_wt(const void* x, const void* wg, const void* wu, const void* wd, const void* sg, const void* su,
                      const void* sd, const int32_t* offsets, const int32_t* perm, int T, int K, int H, int F, int E,
                      void* y, int y_bf16, uint16_t* abuf, hipStream_t st) {
    const int n = T * K;
    const int slots = E < n ? E : n;          // at most this many experts are touched
    const int rows_cap = T < SM_ROWS ? T : SM_ROWS;   // an expert has at most T rows
    const size_t lds_g = (size_t)rows_cap * (H + 8) * 2 + (WT == SDT_INT4 ? (size_t)rows_cap * (H / 32) * 4 : 0);
    const size_t lds_d = WT == SDT_INT4 ? (size_t)SM_ROWS * (F / 32) * 4 : 0;
    dim3 gg(slots, F / 64), gd(slots, H / 64);
    switch (ring_for(H / 32)) {
        case 8: gateup_small<WT, 8>(gg, lds_g, st, x, wg, wu, sg, su, offsets, perm, K, H, F, E, rows_cap, abuf); break;
        case 4: gateup_small<WT, 4>(gg, lds_g, st, x, wg, wu, sg, su, offsets, perm, K, H, F, E, rows_cap, abuf); break;
        default: gateup_small<WT, 2>(gg, lds_g, st, x, wg, wu, sg, su, offsets, perm, K, H, F, E, rows_cap, abuf); break;
    }
    const int rd = ring_for(F / 32);
    if (y_bf16) {
        if (rd == 8) down_small<WT, 1, 8>(gd, lds_d, st, abuf, wd, sd, offsets, H, F, E, y);
        else if (rd == 4) down_small<WT, 1, 4>(gd, lds_d, st, abuf, wd, sd, offsets, H, F, E, y);
        else down_small<WT, 1, 2>(gd, lds_d, st, abuf, wd, sd, offsets, H, F, E, y);
    } else {
        if (rd == 8) down_small<WT, 0, 8>(gd, lds_d, st, abuf, wd, sd, offsets, H, F, E, y);
        else if (rd == 4) down_small<WT, 0, 4>(gd, lds_d, st, abuf, wd, sd, offsets, H, F, E, y);
        else down_small<WT, 0, 2>(gd, lds_d, st, abuf, wd, sd, offsets, H, F, E, y);
    }
}

hipError_t launch_ffn_small(const void* x, int w_dtype, const void* wg, const void* wu, const void* wd,
                            const void* sg, const void* su, const void* sd, const int32_t* offsets,
                            const int32_t* perm, int T, int K, int H, int F, int E, void* y, int y_bf16, void* ws,
                            hipStream_t st) {
    uint16_t* abuf = (uint16_t*)ws;
    if (w_dtype == SDT_BF16)
        launch_wt<SDT_BF16>(x, wg, wu, wd, sg, su, sd, offsets, perm, T, K, H, F, E, y, y_bf16, abuf, st);
    else
        launch_wt<SDT_INT4>(x, wg, wu, wd, sg, su, sd, offsets, perm, T, K, H, F, E, y, y_bf16, abuf, st);
    return hipGetLastError();
}
