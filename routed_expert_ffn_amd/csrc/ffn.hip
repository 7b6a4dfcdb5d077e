// ffn.hip -- grouped SwiGLU expert FFN (gfx950).
//
// Every expert has gate, up and down matrices ("Strata Coder 编程模型深度剖析",
// §3 "RCO 专家剪枝是怎么砍一半而不伤脑的"); the expert is
//     a = silu(Wg x) * (Wu x),   y = Wd a
// run over the rows that the grouping step assigned to it.  Rows are the
// permuted slots p of the expert's segment; row p reads token perm[p] / K.
//
// bf16 activations (bf16 or int4 weights): two MFMA kernels.
//   k_gateup_mfma  one block = 64 rows x 64 columns of BOTH gate and up
//                  (128 weight rows), K = H; epilogue silu(g)*u -> bf16 into
//                  the workspace A[p][f].
//   k_down_mfma    one block = 64 rows x 128 output columns, K = F; writes
//                  y_perm[p][h].
//   The activation rows are gathered straight from x (no permuted copy).
//   int4 weights (symmetric, blocks of 32 along K, fp16 scale) are decoded
//   while staging the tile into LDS: d*q is exact in fp32 and is rounded to
//   bf16 for the MFMA (relative weight error <= 2^-9).
// fp32 activations and weights: plain per-element kernels (fp32 FMA).
//
// launch_ffn picks the path: int3 / int2 weights go to the few-token streaming
// kernels (ffn_stream.hip); T <= 16 to the small-T paths (ffn_small.hip, which
// hands T <= 8 bf16 and int4 shapes on to the streaming kernels); bf16 and
// int4 at larger T to the grouped GEMM (ffn_gemm.hip) where its shapes allow;
// anything else to the two MFMA kernels here.
#include "common.h"
#include "launch.h"

enum { DT_F32 = 0, DT_BF16 = 1, DT_INT4 = 2, DT_INT2 = 3, DT_INT3 = 4 };

constexpr int G_BM = 64, G_BNF = 64, G_BK = 64, G_LD = G_BK + 8;   // gate/up tile
constexpr int D_BM = 64, D_BN = 128, D_BK = 64, D_LD = D_BK + 8;   // down tile

MOE_DEV float silu_f(float g) { return g / (1.0f + expf(-g)); }

// ---- staging helpers ---------------------------------------------------------

// Decode 32 int4 weights (16 bytes) with scale d to 32 bf16 (4 x uint4).
MOE_DEV void int4x32_to_bf16(const uint4 q, float d, uint4 out[4]) {
    const uint32_t words[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int w = 0; w < 4; w++) {
        uint32_t v = words[w];
        uint32_t o[4];
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const uint32_t byte = (v >> (8 * b)) & 0xFFu;
            const float lo = d * (float)((int)(byte & 15u) - 8);
            const float hi = d * (float)((int)(byte >> 4) - 8);
            o[b] = pack_bf16x2(lo, hi);
        }
        out[w] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// ---- gate/up -------------------------------------------------------------------

template <int WT>
__global__ __launch_bounds__(256) void k_gateup_mfma(const uint16_t* __restrict__ x,
                                                     const void* __restrict__ wg_, const void* __restrict__ wu_,
                                                     const uint16_t* __restrict__ sg, const uint16_t* __restrict__ su,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ perm, int K, int H, int F, int E,
                                                     uint16_t* __restrict__ abuf) {
    __shared__ __attribute__((aligned(16))) uint16_t As[G_BM * G_LD];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2 * G_BNF * G_LD];
    __shared__ int s_tile[3];
    const int tid = threadIdx.x;
    if (tid < WAVE) {
        int row0 = 0, rows = 0;
        const int e = find_group_tile(offsets, E, G_BM, blockIdx.x, row0, rows);
        if (tid == 0) { s_tile[0] = e; s_tile[1] = row0; s_tile[2] = rows; }
    }
    __syncthreads();
    const int e = s_tile[0], row0 = s_tile[1], rows = s_tile[2];
    if (e < 0) return;
    const int f0 = blockIdx.y * G_BNF;
    const int wave = tid / WAVE, l = lane_id();
    const int wm = wave >> 1, wn = wave & 1;

    // A staging: 64 rows x 64 bf16 -> 2 x 16B per thread
    const uint16_t* a_src[2];
    int a_dst[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const int idx = tid + q * 256;
        const int r = idx >> 3, c = (idx & 7) * 8;
        a_dst[q] = r * G_LD + c;
        a_src[q] = nullptr;
        if (r < rows) a_src[q] = x + (long)(perm[row0 + r] / K) * H + c;
    }
    uint4 a0, a1, b0, b1, b2, b3;   // staged tile (named, so they stay in registers)
    float b_scale = 0.f;
    const int b_r = tid >> 3, b_c = (tid & 7) * 8;     // bf16 B: rows b_r + 32q, 16B column b_c
    const int q_r = tid >> 1, q_blk = tid & 1;          // int4 B: (row, block of 32) per thread
    auto bsrc = [&](int r) -> const uint16_t* {
        return (r < G_BNF ? (const uint16_t*)wg_ : (const uint16_t*)wu_) + ((long)e * F + f0 + (r & (G_BNF - 1))) * H +
               b_c;
    };
    const uint16_t* bp0 = bsrc(b_r);
    const uint16_t* bp1 = bsrc(b_r + 32);
    const uint16_t* bp2 = bsrc(b_r + 64);
    const uint16_t* bp3 = bsrc(b_r + 96);
    const long q_row = (long)e * F + f0 + (q_r & (G_BNF - 1));
    const uint8_t* qp = (q_r < G_BNF ? (const uint8_t*)wg_ : (const uint8_t*)wu_) + q_row * (H / 2) + q_blk * 16;
    const uint16_t* sp = (q_r < G_BNF ? sg : su) + q_row * (H / 32) + q_blk;
    auto load = [&](int k0) __attribute__((always_inline)) {
        a0 = a_src[0] ? *reinterpret_cast<const uint4*>(a_src[0] + k0) : make_uint4(0, 0, 0, 0);
        a1 = a_src[1] ? *reinterpret_cast<const uint4*>(a_src[1] + k0) : make_uint4(0, 0, 0, 0);
        if constexpr (WT == DT_BF16) {
            b0 = *reinterpret_cast<const uint4*>(bp0 + k0);
            b1 = *reinterpret_cast<const uint4*>(bp1 + k0);
            b2 = *reinterpret_cast<const uint4*>(bp2 + k0);
            b3 = *reinterpret_cast<const uint4*>(bp3 + k0);
        } else {
            b0 = *reinterpret_cast<const uint4*>(qp + k0 / 2);
            b_scale = fp16_to_f32(sp[k0 / 32]);
        }
    };
    auto store = [&]() __attribute__((always_inline)) {
        *reinterpret_cast<uint4*>(&As[a_dst[0]]) = a0;
        *reinterpret_cast<uint4*>(&As[a_dst[1]]) = a1;
        if constexpr (WT == DT_BF16) {
            *reinterpret_cast<uint4*>(&Bs[(b_r) * G_LD + b_c]) = b0;
            *reinterpret_cast<uint4*>(&Bs[(b_r + 32) * G_LD + b_c]) = b1;
            *reinterpret_cast<uint4*>(&Bs[(b_r + 64) * G_LD + b_c]) = b2;
            *reinterpret_cast<uint4*>(&Bs[(b_r + 96) * G_LD + b_c]) = b3;
        } else {
            uint4 o[4];
            int4x32_to_bf16(b0, b_scale, o);
#pragma unroll
            for (int q = 0; q < 4; q++) *reinterpret_cast<uint4*>(&Bs[q_r * G_LD + q_blk * 32 + q * 8]) = o[q];
        }
    };

    f32x4_t acc[2][2][2];   // [gate/up][m sub-tile][n sub-tile]
#pragma unroll
    for (int g = 0; g < 2; g++)
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) acc[g][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load(0);
    for (int k0 = 0; k0 < H; k0 += G_BK) {
        store();
        __syncthreads();
        if (k0 + G_BK < H) load(k0 + G_BK);
#pragma unroll
        for (int kk = 0; kk < G_BK; kk += 32) {
            bf16x8_t af[2], bfr[2][2];
#pragma unroll
            for (int i = 0; i < 2; i++)
                af[i] = *reinterpret_cast<const bf16x8_t*>(
                    &As[(wm * 32 + i * 16 + (l & 15)) * G_LD + kk + (l >> 4) * 8]);
#pragma unroll
            for (int g = 0; g < 2; g++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    bfr[g][j] = *reinterpret_cast<const bf16x8_t*>(
                        &Bs[(g * G_BNF + wn * 32 + j * 16 + (l & 15)) * G_LD + kk + (l >> 4) * 8]);
#pragma unroll
            for (int g = 0; g < 2; g++)
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < 2; j++)
                        acc[g][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[g][j], acc[g][i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    // epilogue: a = bf16(silu(g) * u)
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int f = f0 + wn * 32 + j * 16 + (l & 15);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int rr = wm * 32 + i * 16 + (l >> 4) * 4 + r;
                if (rr < rows) {
                    const float a = silu_f(acc[0][i][j][r]) * acc[1][i][j][r];
                    abuf[(long)(row0 + rr) * F + f] = f32_to_bf16_rne(a);
                }
            }
        }
}

// ---- down ----------------------------------------------------------------------

template <int WT, int YBF16>
__global__ __launch_bounds__(256) void k_down_mfma(const uint16_t* __restrict__ abuf, const void* __restrict__ wd_,
                                                   const uint16_t* __restrict__ sd, const int32_t* __restrict__ offsets,
                                                   int H, int F, int E, void* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) uint16_t As[D_BM * D_LD];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[D_BN * D_LD];
    __shared__ int s_tile[3];
    const int tid = threadIdx.x;
    if (tid < WAVE) {
        int row0 = 0, rows = 0;
        const int e = find_group_tile(offsets, E, D_BM, blockIdx.x, row0, rows);
        if (tid == 0) { s_tile[0] = e; s_tile[1] = row0; s_tile[2] = rows; }
    }
    __syncthreads();
    const int e = s_tile[0], row0 = s_tile[1], rows = s_tile[2];
    if (e < 0) return;
    const int h0 = blockIdx.y * D_BN;
    const int wave = tid / WAVE, l = lane_id();
    const int wm = wave >> 1, wn = wave & 1;

    uint4 a0, a1, b0, b1, b2, b3;
    float b_scale = 0.f;
    const int a_r = tid >> 3, a_c = (tid & 7) * 8;      // A rows a_r and a_r + 32
    const uint16_t* ap0 = a_r < rows ? abuf + (long)(row0 + a_r) * F + a_c : nullptr;
    const uint16_t* ap1 = a_r + 32 < rows ? abuf + (long)(row0 + a_r + 32) * F + a_c : nullptr;
    const uint16_t* bp = (const uint16_t*)wd_ + ((long)e * H + h0 + a_r) * F + a_c;   // rows a_r + 32q
    const int q_r = tid >> 1, q_blk = tid & 1;
    const long q_row = (long)e * H + h0 + q_r;
    const uint8_t* qp = (const uint8_t*)wd_ + q_row * (F / 2) + q_blk * 16;
    const uint16_t* sp = (WT == DT_INT4) ? sd + q_row * (F / 32) + q_blk : nullptr;
    auto load = [&](int k0) __attribute__((always_inline)) {
        a0 = ap0 ? *reinterpret_cast<const uint4*>(ap0 + k0) : make_uint4(0, 0, 0, 0);
        a1 = ap1 ? *reinterpret_cast<const uint4*>(ap1 + k0) : make_uint4(0, 0, 0, 0);
        if constexpr (WT == DT_BF16) {
            b0 = *reinterpret_cast<const uint4*>(bp + k0);
            b1 = *reinterpret_cast<const uint4*>(bp + 32L * F + k0);
            b2 = *reinterpret_cast<const uint4*>(bp + 64L * F + k0);
            b3 = *reinterpret_cast<const uint4*>(bp + 96L * F + k0);
        } else {
            b0 = *reinterpret_cast<const uint4*>(qp + k0 / 2);
            b_scale = fp16_to_f32(sp[k0 / 32]);
        }
    };
    auto store = [&]() __attribute__((always_inline)) {
        *reinterpret_cast<uint4*>(&As[a_r * D_LD + a_c]) = a0;
        *reinterpret_cast<uint4*>(&As[(a_r + 32) * D_LD + a_c]) = a1;
        if constexpr (WT == DT_BF16) {
            *reinterpret_cast<uint4*>(&Bs[a_r * D_LD + a_c]) = b0;
            *reinterpret_cast<uint4*>(&Bs[(a_r + 32) * D_LD + a_c]) = b1;
            *reinterpret_cast<uint4*>(&Bs[(a_r + 64) * D_LD + a_c]) = b2;
            *reinterpret_cast<uint4*>(&Bs[(a_r + 96) * D_LD + a_c]) = b3;
        } else {
            uint4 o[4];
            int4x32_to_bf16(b0, b_scale, o);
#pragma unroll
            for (int q = 0; q < 4; q++) *reinterpret_cast<uint4*>(&Bs[q_r * D_LD + q_blk * 32 + q * 8]) = o[q];
        }
    };

    f32x4_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load(0);
    for (int k0 = 0; k0 < F; k0 += D_BK) {
        store();
        __syncthreads();
        if (k0 + D_BK < F) load(k0 + D_BK);
#pragma unroll
        for (int kk = 0; kk < D_BK; kk += 32) {
            bf16x8_t af[2], bfr[4];
#pragma unroll
            for (int i = 0; i < 2; i++)
                af[i] = *reinterpret_cast<const bf16x8_t*>(
                    &As[(wm * 32 + i * 16 + (l & 15)) * D_LD + kk + (l >> 4) * 8]);
#pragma unroll
            for (int j = 0; j < 4; j++)
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(
                    &Bs[(wn * 64 + j * 16 + (l & 15)) * D_LD + kk + (l >> 4) * 8]);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int h = h0 + wn * 64 + j * 16 + (l & 15);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int rr = wm * 32 + i * 16 + (l >> 4) * 4 + r;
                if (rr < rows) {
                    const long o = (long)(row0 + rr) * H + h;
                    if constexpr (YBF16) ((uint16_t*)y)[o] = f32_to_bf16_rne(acc[i][j][r]);
                    else ((float*)y)[o] = acc[i][j][r];
                }
            }
        }
}

// ---- fp32 path ---------------------------------------------------------------

MOE_DEV int expert_of_row(const int32_t* __restrict__ offsets, int E, int p) {
    int lo = 0, hi = E - 1;          // largest e with offsets[e] <= p
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= p) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(256) void k_gateup_f32(const float* __restrict__ x, const float* __restrict__ wg,
                                                    const float* __restrict__ wu, const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ perm, int n, int K, int H, int F,
                                                    int E, float* __restrict__ abuf) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)n * F) return;
    const int p = (int)(i / F), f = (int)(i % F);
    const int e = expert_of_row(offsets, E, p);
    const float* xr = x + (long)(perm[p] / K) * H;
    const float* g = wg + ((long)e * F + f) * H;
    const float* u = wu + ((long)e * F + f) * H;
    float sg = 0.f, su = 0.f;
    for (int h = 0; h < H; h++) {
        sg = fmaf(xr[h], g[h], sg);
        su = fmaf(xr[h], u[h], su);
    }
    abuf[i] = silu_f(sg) * su;
}

__global__ __launch_bounds__(256) void k_down_f32(const float* __restrict__ abuf, const float* __restrict__ wd,
                                                  const int32_t* __restrict__ offsets, int n, int H, int F, int E,
                                                  float* __restrict__ y) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)n * H) return;
    const int p = (int)(i / H), h = (int)(i % H);
    const int e = expert_of_row(offsets, E, p);
    const float* ar = abuf + (long)p * F;
    const float* d = wd + ((long)e * H + h) * F;
    float s = 0.f;
    for (int f = 0; f < F; f++) s = fmaf(ar[f], d[f], s);
    y[i] = s;
}

// ---- host ------------------------------------------------------------------------

size_t ffn_workspace_bytes(int T, int K, int E, int H, int F, int x_dtype, int w_dtype) {
    const size_t n = (size_t)T * K;
    const size_t elt = x_dtype == DT_F32 ? 4 : 2;
    size_t b = ((n * F * elt) + 255) / 256 * 256;
    if (x_dtype != DT_F32 && ffn_small_eligible(T, H, F)) {
        const size_t s = ffn_small_workspace_bytes(T, K, E, H, F);
        b = s > b ? s : b;
    }
    if (x_dtype != DT_F32 && ffn_gemm_eligible(T, K, H, F)) {
        const size_t s = ffn_gemm_workspace_bytes(T, K, E, H, F);
        b = s > b ? s : b;
    }
    if (x_dtype != DT_F32 && w_dtype == DT_INT4 && !ffn_small_eligible(T, H, F) && ffn_gemm_q4_eligible(T, K, E, H, F)) {
        const size_t s = ffn_gemm_q4_workspace_bytes(T, K, E, H, F);
        b = s > b ? s : b;
    }
    return b;
}

hipError_t launch_ffn(const void* x, int x_dtype, int w_dtype, const void* wg, const void* wu, const void* wd,
                      const void* sg, const void* su, const void* sd, const int32_t* offsets, const int32_t* perm,
                      int T, int K, int H, int F, int E, void* y, int y_dtype, void* ws, hipStream_t st) {
    const int n = T * K;
    if (n == 0) return hipSuccess;
    if (x_dtype == DT_F32) {
        float* abuf = (float*)ws;
        const long ng = (long)n * F, nd = (long)n * H;
        hipLaunchKernelGGL(k_gateup_f32, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0, st, (const float*)x,
                           (const float*)wg, (const float*)wu, offsets, perm, n, K, H, F, E, abuf);
        hipLaunchKernelGGL(k_down_f32, dim3((unsigned)((nd + 255) / 256)), dim3(256), 0, st, abuf, (const float*)wd,
                           offsets, n, H, F, E, (float*)y);
        return hipGetLastError();
    }
    // int3 / int2 experts: the verify-step streaming kernels only (checked by the caller)
    if (w_dtype == DT_INT2 || w_dtype == DT_INT3)
        return launch_ffn_stream_q4(x, wg, wu, wd, sg, su, sd, offsets, perm, T, K, H, F, E, y, y_dtype == DT_BF16, ws,
                                    st, w_dtype == DT_INT2 ? 2 : 3);
    if (ffn_small_eligible(T, H, F))
        return launch_ffn_small(x, w_dtype, wg, wu, wd, sg, su, sd, offsets, perm, T, K, H, F, E, y,
                                y_dtype == DT_BF16, ws, st);
    if (w_dtype == DT_BF16 && ffn_gemm_eligible(T, K, H, F))
        return launch_ffn_gemm(x, wg, wu, wd, offsets, perm, T, K, H, F, E, y, y_dtype == DT_BF16, ws, st);
    if (w_dtype == DT_INT4 && ffn_gemm_q4_eligible(T, K, E, H, F))
        return launch_ffn_gemm_q4(x, wg, wu, wd, sg, su, sd, offsets, perm, T, K, H, F, E, y, y_dtype == DT_BF16, ws,
                                  st);
    uint16_t* abuf = (uint16_t*)ws;
    const int tiles_g = (n + G_BM - 1) / G_BM + (E < n ? E : n);
    const int tiles_d = (n + D_BM - 1) / D_BM + (E < n ? E : n);
    dim3 gg(tiles_g, F / G_BNF), gd(tiles_d, H / D_BN);
    if (w_dtype == DT_BF16) {
        hipLaunchKernelGGL(k_gateup_mfma<DT_BF16>, gg, dim3(256), 0, st, (const uint16_t*)x, wg, wu, nullptr, nullptr,
                           offsets, perm, K, H, F, E, abuf);
        if (y_dtype == DT_BF16)
            hipLaunchKernelGGL((k_down_mfma<DT_BF16, 1>), gd, dim3(256), 0, st, abuf, wd, nullptr, offsets, H, F, E, y);
        else
            hipLaunchKernelGGL((k_down_mfma<DT_BF16, 0>), gd, dim3(256), 0, st, abuf, wd, nullptr, offsets, H, F, E, y);
    } else {
        hipLaunchKernelGGL(k_gateup_mfma<DT_INT4>, gg, dim3(256), 0, st, (const uint16_t*)x, wg, wu,
                           (const uint16_t*)sg, (const uint16_t*)su, offsets, perm, K, H, F, E, abuf);
        if (y_dtype == DT_BF16)
            hipLaunchKernelGGL((k_down_mfma<DT_INT4, 1>), gd, dim3(256), 0, st, abuf, wd, (const uint16_t*)sd, offsets, H,
                               F, E, y);
        else
            hipLaunchKernelGGL((k_down_mfma<DT_INT4, 0>), gd, dim3(256), 0, st, abuf, wd, (const uint16_t*)sd, offsets, H,
                               F, E, y);
    }
    return hipGetLastError();
}
