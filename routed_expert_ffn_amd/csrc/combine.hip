// combine.hip -- weighted combine of the K expert outputs of each token (gfx950).
//
//   out[t] = cast( sum_k w[t][k] * y_perm[inv[t*K + k]] + residual[t] )
//
// A gather in k order with fp32 accumulation: no atomics, so the result is
// deterministic.  Each thread owns 8 consecutive hidden elements (16-byte
// bf16 loads/stores); the residual add (between stacked MoE layers) is fused
// before the single rounding.
//
// The steered variant also removes the row's component along a unit
// direction v, h - (h . v) v, before that rounding: the per-layer steering
// projection of the kwkr.cn Coder write-up ("实验加速投影在 Coder 上的表现"),
// applied to the stream right after the layer adds its expert outputs.
#include "common.h"
#include "launch.h"

// acc = sum_k w[t][k] * y[inv[t*K+k]][h .. h+7] (+ res[t][h .. h+7]), fp32, k order
template <int YB, int OB>
MOE_DEV void combine_acc8(const void* __restrict__ y, const int32_t* __restrict__ inv, const float* __restrict__ w,
                          const void* __restrict__ res, int t, int h, int K, int H, float (&acc)[8]) {
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = 0.f;
    const long o = (long)t * H + h;
    // the residual chunk's load goes out with the first group's row loads
    float rv[8];
    auto load_res = [&]() __attribute__((always_inline)) {
        if constexpr (OB) {
            const uint4 q = *reinterpret_cast<const uint4*>((const uint16_t*)res + o);
            const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; i++) { rv[2 * i] = bf16lo_to_f32(u[i]); rv[2 * i + 1] = bf16hi_to_f32(u[i]); }
        } else {
            const float4 a = *reinterpret_cast<const float4*>((const float*)res + o);
            const float4 b = *reinterpret_cast<const float4*>((const float*)res + o + 4);
            rv[0] = a.x; rv[1] = a.y; rv[2] = a.z; rv[3] = a.w;
            rv[4] = b.x; rv[5] = b.y; rv[6] = b.z; rv[7] = b.w;
        }
    };
    // K routed rows in groups of KB (K <= KB: one group): the group's row
    // loads are all in flight before its multiply-adds, which run in k order
    constexpr int KB = 16;
    for (int k0 = 0; k0 < K; k0 += KB) {
        uint4 q[KB][YB ? 1 : 2];                        // the rows as loaded, widened at their multiply-adds
        float wk[KB];
#pragma unroll
        for (int u = 0; u < KB; u++) {
            if (k0 + u < K) {                           // uniform
                const long row = inv[(long)t * K + k0 + u];
                wk[u] = w[(long)t * K + k0 + u];
                if constexpr (YB) {
                    q[u][0] = *reinterpret_cast<const uint4*>((const uint16_t*)y + row * H + h);
                } else {
                    q[u][0] = *reinterpret_cast<const uint4*>((const float*)y + row * H + h);
                    q[u][YB ? 0 : 1] = *reinterpret_cast<const uint4*>((const float*)y + row * H + h + 4);
                }
            }
        }
        if (k0 == 0 && res) load_res();
#pragma unroll
        for (int u = 0; u < KB; u++) {
            if (k0 + u < K) {                           // uniform
                float v[8];
                if constexpr (YB) {
                    const uint32_t uu[4] = {q[u][0].x, q[u][0].y, q[u][0].z, q[u][0].w};
#pragma unroll
                    for (int i = 0; i < 4; i++) { v[2 * i] = bf16lo_to_f32(uu[i]); v[2 * i + 1] = bf16hi_to_f32(uu[i]); }
                } else {
                    const uint4 a = q[u][0], b = q[u][YB ? 0 : 1];
                    const uint32_t uu[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                    for (int i = 0; i < 8; i++) v[i] = __uint_as_float(uu[i]);
                }
#pragma unroll
                for (int i = 0; i < 8; i++) acc[i] = fmaf(wk[u], v[i], acc[i]);
            }
        }
    }
    if (res) {
#pragma unroll
        for (int i = 0; i < 8; i++) acc[i] += rv[i];
    }
}

template <int OB>
MOE_DEV void store8(void* __restrict__ out, long o, const float (&acc)[8]) {
    if constexpr (OB) {
        uint4 q;
        q.x = pack_bf16x2(acc[0], acc[1]);
        q.y = pack_bf16x2(acc[2], acc[3]);
        q.z = pack_bf16x2(acc[4], acc[5]);
        q.w = pack_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<uint4*>((uint16_t*)out + o) = q;
    } else {
        *reinterpret_cast<float4*>((float*)out + o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        *reinterpret_cast<float4*>((float*)out + o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

template <int YB, int OB>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ y, const int32_t* __restrict__ inv,
                                                 const float* __restrict__ w, const void* __restrict__ res, int K,
                                                 int H, void* __restrict__ out) {
    const int t = blockIdx.y;
    const int h = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (h >= H) return;
    float acc[8];
    combine_acc8<YB, OB>(y, inv, w, res, t, h, K, H, acc);
    store8<OB>(out, (long)t * H + h, acc);
}

// Steered combine: one block per token holds the whole row h = combine(...)
// in registers (NCH chunks of 2048 elements, 8 per thread), forms d = h . v
// in fp32 (per-thread products in element order, then the 64 lanes, then the
// 4 waves in wave order: the same d in every thread, the same on every run),
// and stores round(h - d v).  The projection costs one block reduction; the
// row is read and written once, as in the plain combine.
template <int YB, int OB, int NCH>
__global__ __launch_bounds__(256) void k_combine_steer(const void* __restrict__ y, const int32_t* __restrict__ inv,
                                                       const float* __restrict__ w, const void* __restrict__ res,
                                                       const float* __restrict__ sv, int K, int H,
                                                       void* __restrict__ out) {
    __shared__ float part[4];
    const int t = blockIdx.x;
    float acc[NCH][8], v[NCH][8];
    float d = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
        const int h = (c * 256 + threadIdx.x) * 8;
        if (h < H) {
            combine_acc8<YB, OB>(y, inv, w, res, t, h, K, H, acc[c]);
            const float4 a = *reinterpret_cast<const float4*>(sv + h);
            const float4 b = *reinterpret_cast<const float4*>(sv + h + 4);
            v[c][0] = a.x; v[c][1] = a.y; v[c][2] = a.z; v[c][3] = a.w;
            v[c][4] = b.x; v[c][5] = b.y; v[c][6] = b.z; v[c][7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++) { acc[c][i] = 0.f; v[c][i] = 0.f; }
        }
#pragma unroll
        for (int i = 0; i < 8; i++) d = fmaf(acc[c][i], v[c][i], d);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) d += wave_xor(d, m);
    if (lane_id() == 0) part[threadIdx.x / WAVE] = d;
    __syncthreads();
    d = ((part[0] + part[1]) + part[2]) + part[3];
#pragma unroll
    for (int c = 0; c < NCH; c++) {
        const int h = (c * 256 + threadIdx.x) * 8;
        if (h < H) {
#pragma unroll
            for (int i = 0; i < 8; i++) acc[c][i] = fmaf(-d, v[c][i], acc[c][i]);
            store8<OB>(out, (long)t * H + h, acc[c]);
        }
    }
}

hipError_t launch_combine(const void* y, int y_bf16, const int32_t* inv, const float* w, const void* res, int T,
                          int K, int H, void* out, int out_bf16, hipStream_t st) {
    if (T == 0) return hipSuccess;
    dim3 grid((H + 2047) / 2048, T);
    if (y_bf16 && out_bf16) hipLaunchKernelGGL((k_combine<1, 1>), grid, dim3(256), 0, st, y, inv, w, res, K, H, out);
    else if (y_bf16) hipLaunchKernelGGL((k_combine<1, 0>), grid, dim3(256), 0, st, y, inv, w, res, K, H, out);
    else if (out_bf16) hipLaunchKernelGGL((k_combine<0, 1>), grid, dim3(256), 0, st, y, inv, w, res, K, H, out);
    else hipLaunchKernelGGL((k_combine<0, 0>), grid, dim3(256), 0, st, y, inv, w, res, K, H, out);
    return hipGetLastError();
}

template <int NCH>
static hipError_t launch_steer_n(const void* y, int y_bf16, const int32_t* inv, const float* w, const void* res,
                                 const float* sv, int T, int K, int H, void* out, int out_bf16, hipStream_t st) {
    const dim3 grid(T), block(256);
    if (y_bf16 && out_bf16) hipLaunchKernelGGL((k_combine_steer<1, 1, NCH>), grid, block, 0, st, y, inv, w, res, sv, K, H, out);
    else if (y_bf16) hipLaunchKernelGGL((k_combine_steer<1, 0, NCH>), grid, block, 0, st, y, inv, w, res, sv, K, H, out);
    else if (out_bf16) hipLaunchKernelGGL((k_combine_steer<0, 1, NCH>), grid, block, 0, st, y, inv, w, res, sv, K, H, out);
    else hipLaunchKernelGGL((k_combine_steer<0, 0, NCH>), grid, block, 0, st, y, inv, w, res, sv, K, H, out);
    return hipGetLastError();
}

hipError_t launch_combine_steer(const void* y, int y_bf16, const int32_t* inv, const float* w, const void* res,
                                const float* sv, int T, int K, int H, void* out, int out_bf16, hipStream_t st) {
    if (T == 0) return hipSuccess;
    switch ((H + 2047) / 2048) {
        case 1: return launch_steer_n<1>(y, y_bf16, inv, w, res, sv, T, K, H, out, out_bf16, st);
        case 2: return launch_steer_n<2>(y, y_bf16, inv, w, res, sv, T, K, H, out, out_bf16, st);
        case 3: return launch_steer_n<3>(y, y_bf16, inv, w, res, sv, T, K, H, out, out_bf16, st);
        case 4: return launch_steer_n<4>(y, y_bf16, inv, w, res, sv, T, K, H, out, out_bf16, st);
    }
    return hipErrorInvalidValue;
}
