// route.hip -- router projection, top-K selection and routing weights (gfx950).
//
// The operation: each token is routed to K of the E experts of its layer
// ("Strata Coder 编程模型深度剖析", §1 "先搞懂 Strata": 10 of 512 per token).
// The routing weights are the softmax renormalised over the K selected logits;
// ties go to the lower expert id.
//
// Exactness.  The logit is defined as fp32(S) (+ bias in fp32) where S is the
// fp64 sum of the exact products x[h]*w[h] taken in wave-64 order: lane j of a
// wave sums h = j, j+64, j+128, ... in ascending order, then the 64 partial
// sums are combined by the butterfly 32,16,8,4,2,1 (lane 0 ends with
// P_0 + P_32, then + P_16 + P_48, ...: the pairwise tree).  A bf16 or fp32
// activation times an fp32 weight is exact in fp64, so fma and mul+add agree
// and the value is reproducible bit for bit.
//
// Two ways to get the logits:
//   k_logits_exact   the definition itself, one wave per (expert, token group);
//   k_logits_fast    an fp32 estimate on bf16 MFMA: the fp32 router weight is
//                    split exactly into three bf16 terms (8+8+8 significand
//                    bits), so every product is exact and only the fp32
//                    accumulation differs from the definition.
// k_route_select takes the top-(K+1) of a token's logits.  With exact logits it
// is final.  With estimates, a token whose K+1 leading values are all separated
// by at least tau is final too (an estimate error below tau/2 cannot reorder
// them or let an outside expert in); any other token recomputes the exact
// logits of every expert within tau of its K-th value and selects among those.
#include "common.h"
#include "launch.h"

// ------------------------------------------------------------------ exact logits

template <typename XT>
MOE_DEV double xval(const XT* p, long i);
template <>
MOE_DEV double xval<float>(const float* p, long i) { return (double)p[i]; }
template <>
MOE_DEV double xval<uint16_t>(const uint16_t* p, long i) { return (double)bf16_to_f32(p[i]); }

// One exact logit dot product by a whole wave; every lane returns the result.
template <typename XT>
MOE_DEV double wave_dot_exact(const XT* __restrict__ xrow, const float* __restrict__ wrow, int H) {
    const int l = lane_id();
    double p = 0.0;
    for (int h = l; h < H; h += WAVE) p = __fma_rn(xval(xrow, h), (double)wrow[h], p);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) p += __shfl_xor(p, d, WAVE);
    return p;
}

constexpr int EXACT_TPG = 4;   // tokens per register group

template <typename XT>
__global__ __launch_bounds__(256) void k_logits_exact(const XT* __restrict__ x, const float* __restrict__ wr,
                                                      const float* __restrict__ bias, int T, int H, int E,
                                                      int tokens_per_wave, float* __restrict__ logits) {
    const int wave = threadIdx.x / WAVE;
    const int e = blockIdx.x * 4 + wave;
    if (e >= E) return;
    const int l = lane_id();
    const float* wrow = wr + (long)e * H;
    const int t_begin = blockIdx.y * tokens_per_wave;
    const int t_end = min(T, t_begin + tokens_per_wave);
    const float b = bias ? bias[e] : 0.0f;
    for (int t0 = t_begin; t0 < t_end; t0 += EXACT_TPG) {
        double p[EXACT_TPG];
#pragma unroll
        for (int i = 0; i < EXACT_TPG; i++) p[i] = 0.0;
        for (int h = l; h < H; h += WAVE) {
            const double w = (double)wrow[h];
#pragma unroll
            for (int i = 0; i < EXACT_TPG; i++)
                if (t0 + i < t_end) p[i] = __fma_rn(xval(x + (long)(t0 + i) * H, h), w, p[i]);
        }
#pragma unroll
        for (int i = 0; i < EXACT_TPG; i++) {
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) p[i] += __shfl_xor(p[i], d, WAVE);
        }
        if (l == 0) {
#pragma unroll
            for (int i = 0; i < EXACT_TPG; i++)
                if (t0 + i < t_end) {
                    float v = (float)p[i];
                    if (bias) v = __fadd_rn(v, b);
                    logits[(long)(t0 + i) * E + e] = v;
                }
        }
    }
}

// ------------------------------------------------------------------ fast logits (bf16 x, 3-term split MFMA)

// Block tile 64 tokens x 64 experts, K step 32; 4 waves as 2x2 of 32x32.
constexpr int FL_BM = 64, FL_BN = 64, FL_BK = 32, FL_LD = FL_BK + 8;

__global__ __launch_bounds__(256) void k_logits_fast(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                     const float* __restrict__ bias, int T, int H, int E,
                                                     float* __restrict__ logits) {
    __shared__ __attribute__((aligned(16))) uint16_t As[FL_BM * FL_LD];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[3][FL_BN * FL_LD];
    const int tid = threadIdx.x;
    const int wave = tid / WAVE, l = lane_id();
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.x * FL_BM, n0 = blockIdx.y * FL_BN;

    f32x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // loaders: A 64 rows x 32 bf16 = 256 x 16B (one per thread);
    //          B 64 rows x 32 fp32 = 512 x 16B (two per thread)
    const int a_r = tid >> 2, a_c = (tid & 3) * 8;
    const int a_t = m0 + a_r;
    for (int k0 = 0; k0 < H; k0 += FL_BK) {
        uint4 av = make_uint4(0, 0, 0, 0);
        if (a_t < T) av = *reinterpret_cast<const uint4*>(x + (long)a_t * H + k0 + a_c);
        *reinterpret_cast<uint4*>(&As[a_r * FL_LD + a_c]) = av;
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int idx = tid + q * 256;
            const int b_r = idx >> 3, b_c = (idx & 7) * 4;
            const int e = n0 + b_r;
            float4 wv = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < E) wv = *reinterpret_cast<const float4*>(wr + (long)e * H + k0 + b_c);
            float w4[4] = {wv.x, wv.y, wv.z, wv.w};
            uint16_t hi[4], mi[4], lo[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                // exact split: w = hi + mid + lo, each a bf16 (8 significant bits)
                float w = w4[i];
                uint16_t h16 = f32_to_bf16_rne(w);
                float r1 = w - bf16_to_f32(h16);
                uint16_t m16 = f32_to_bf16_rne(r1);
                float r2 = r1 - bf16_to_f32(m16);
                hi[i] = h16; mi[i] = m16; lo[i] = f32_to_bf16_rne(r2);
            }
            uint2 hv = make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
            uint2 mv = make_uint2(mi[0] | ((uint32_t)mi[1] << 16), mi[2] | ((uint32_t)mi[3] << 16));
            uint2 lv = make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
            *reinterpret_cast<uint2*>(&Bs[0][b_r * FL_LD + b_c]) = hv;
            *reinterpret_cast<uint2*>(&Bs[1][b_r * FL_LD + b_c]) = mv;
            *reinterpret_cast<uint2*>(&Bs[2][b_r * FL_LD + b_c]) = lv;
        }
        __syncthreads();
        bf16x8_t af[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int r = wm * 32 + i * 16 + (l & 15);
            af[i] = *reinterpret_cast<const bf16x8_t*>(&As[r * FL_LD + (l >> 4) * 8]);
        }
#pragma unroll
        for (int s = 0; s < 3; s++) {
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int c = wn * 32 + j * 16 + (l & 15);
                bf16x8_t bfv = *reinterpret_cast<const bf16x8_t*>(&Bs[s][c * FL_LD + (l >> 4) * 8]);
#pragma unroll
                for (int i = 0; i < 2; i++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfv, acc[i][j], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    // D layout (16x16 tile): lane l holds column l%16, rows (l/16)*4 + 0..3
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int e = n0 + wn * 32 + j * 16 + (l & 15);
            if (e >= E) continue;
            const float b = bias ? bias[e] : 0.0f;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int t = m0 + wm * 32 + i * 16 + (l >> 4) * 4 + r;
                if (t < T) logits[(long)t * E + e] = bias ? __fadd_rn(acc[i][j][r], b) : acc[i][j][r];
            }
        }
}

// ------------------------------------------------------------------ selection

constexpr int SEL_CAP = 64;   // candidates re-decided on exact logits (one per lane)

// Top-`rounds` of the keys held by the wave (any layout); lane r receives
// round r's key.  Selected entries are cleared from k[].
template <int VPL>
MOE_DEV unsigned long long select_rounds(unsigned long long (&k)[VPL], int rounds) {
    const int l = lane_id();
    unsigned long long mine = 0;
    for (int r = 0; r < rounds; r++) {
        unsigned long long b = 0;
#pragma unroll
        for (int j = 0; j < VPL; j++) b = k[j] > b ? k[j] : b;
        b = wave_max_u64(b);
#pragma unroll
        for (int j = 0; j < VPL; j++) k[j] = k[j] == b ? 0ull : k[j];   // keys are unique (id embedded)
        if (l == r) mine = b;
    }
    return mine;
}

template <int VPL, typename XT>
__global__ __launch_bounds__(256) void k_route_select(const float* __restrict__ logits, int T, int E, int K,
                                                      float tau, int exact,
                                                      const XT* __restrict__ x, const float* __restrict__ wr,
                                                      const float* __restrict__ bias, int H,
                                                      int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                                      int32_t* __restrict__ rechecked) {
    const int wave = threadIdx.x / WAVE;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int l = lane_id();
    const float* row = logits + (long)t * E;

    float v[VPL];
    unsigned long long k[VPL];
#pragma unroll
    for (int j = 0; j < VPL; j++) {
        const int e = l + j * WAVE;
        v[j] = e < E ? row[e] : 0.f;
        k[j] = e < E ? route_key(v[j], e) : 0ull;
    }
    const int rounds = (exact || K == E) ? K : K + 1;
    unsigned long long sel = select_rounds<VPL>(k, rounds);
    float sel_v = route_key_value(sel);
    int sel_i = route_key_index(sel);

    bool flagged = false;
    if (!exact) {
        // every gap between consecutive selected values, down to the (K+1)-th, must clear tau
        const float nxt = __shfl_down(sel_v, 1, WAVE);
        const bool check = l < K && l + 1 < rounds;
        flagged = __ballot(check && !(sel_v - nxt >= tau)) != 0;
    }

    if (flagged) {
        // Candidates: every expert whose estimate exceeds the K-th estimate - tau.
        const float cut = __shfl(sel_v, K - 1, WAVE) - tau;
        int ncand = 0;
#pragma unroll
        for (int j = 0; j < VPL; j++) {
            const int e = l + j * WAVE;
            ncand += wave_sum((e < E && v[j] > cut) ? 1 : 0);
        }
        const XT* xrow = x + (long)t * H;
        if (ncand <= SEL_CAP) {
            unsigned long long ck = 0;      // lane c holds candidate c's exact key
            int slot = 0;
#pragma unroll
            for (int j = 0; j < VPL; j++) {
                const int e = l + j * WAVE;
                unsigned long long m = __ballot(e < E && v[j] > cut);
                while (m) {
                    const int src = __ffsll((long long)m) - 1;
                    m &= m - 1;
                    const int ce = src + j * WAVE;
                    float lv = (float)wave_dot_exact(xrow, wr + (long)ce * H, H);
                    if (bias) lv = __fadd_rn(lv, bias[ce]);
                    if (l == slot) ck = route_key(lv, ce);
                    slot++;
                }
            }
            unsigned long long c1[1] = {ck};
            sel = select_rounds<1>(c1, K);
        } else {
            // too many near-equal estimates: decide on exact logits of all experts
            unsigned long long ek[VPL];
#pragma unroll
            for (int j = 0; j < VPL; j++) {
                ek[j] = 0;
                for (int src = 0; src < WAVE; src++) {
                    const int ce = src + j * WAVE;
                    if (ce >= E) break;
                    float lv = (float)wave_dot_exact(xrow, wr + (long)ce * H, H);
                    if (bias) lv = __fadd_rn(lv, bias[ce]);
                    if (l == src) ek[j] = route_key(lv, ce);
                }
            }
            sel = select_rounds<VPL>(ek, K);
        }
        sel_v = route_key_value(sel);
        sel_i = route_key_index(sel);
    }
    if (rechecked && l == 0) rechecked[t] = flagged ? 1 : 0;

    // weights: softmax over the K selected values
    const float v0 = __shfl(sel_v, 0, WAVE);
    const float ex = (l < K) ? expf(sel_v - v0) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, WAVE);
    if (l < K) {
        idx_out[(long)t * K + l] = sel_i;
        w_out[(long)t * K + l] = ex / sum;
    }
}

// ------------------------------------------------------------------ exact logits, few tokens

// One wave per expert, every token: the router row (H fp32) is loaded once into
// registers (H/64 independent loads per lane in flight); token rows are staged
// in LDS.  Two experts per block.
constexpr int XS_MAX_T = 16;

template <typename XT, int HL>
__global__ __launch_bounds__(128) void k_logits_exact_small(const XT* __restrict__ x, const float* __restrict__ wr,
                                                            const float* __restrict__ bias, int T, int H, int E,
                                                            float* __restrict__ logits) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    XT* xs = reinterpret_cast<XT*>(smem);
    const int tid = threadIdx.x;
    // stage x [T][H] (16-byte copies)
    const int per = 16 / (int)sizeof(XT);
    const int nchunk = T * H / per;
    for (int i = tid; i < nchunk; i += blockDim.x)
        reinterpret_cast<uint4*>(xs)[i] = reinterpret_cast<const uint4*>(x)[i];
    __syncthreads();
    const int e = blockIdx.x * 2 + tid / WAVE;
    if (e >= E) return;
    const int l = lane_id();
    double w[HL];
#pragma unroll
    for (int i = 0; i < HL; i++) w[i] = (double)wr[(long)e * H + l + i * WAVE];   // H == 64 * HL
    const float b = bias ? bias[e] : 0.f;
    for (int t = 0; t < T; t++) {
        double p = 0.0;
#pragma unroll
        for (int i = 0; i < HL; i++) p = __fma_rn(xval(xs + t * H, l + i * WAVE), w[i], p);
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) p += __shfl_xor(p, d, WAVE);
        if (l == 0) {
            float v = (float)p;
            if (bias) v = __fadd_rn(v, b);
            logits[(long)t * E + e] = v;
        }
    }
}

// ------------------------------------------------------------------ launchers

template <int HL>
static bool small_exact(const void* x, int x_bf16, const float* wr, const float* bias, int T, int H, int E,
                        float* logits, hipStream_t st) {
    const size_t lds = (size_t)T * H * (x_bf16 ? 2 : 4);
    if (x_bf16)
        hipLaunchKernelGGL((k_logits_exact_small<uint16_t, HL>), dim3((E + 1) / 2), dim3(128), lds, st,
                           (const uint16_t*)x, wr, bias, T, H, E, logits);
    else
        hipLaunchKernelGGL((k_logits_exact_small<float, HL>), dim3((E + 1) / 2), dim3(128), lds, st, (const float*)x,
                           wr, bias, T, H, E, logits);
    return true;
}

hipError_t launch_logits_exact(const void* x, int x_bf16, const float* wr, const float* bias, int T, int H, int E,
                               float* logits, hipStream_t st) {
    // few tokens, H = 64 * {4,8,16,32,64} and 16-byte rows: router rows held in registers
    const int hl = H / 64;
    if (T <= XS_MAX_T && H % 64 == 0 && (hl == 4 || hl == 8 || hl == 16 || hl == 32 || hl == 64) &&
        ((uintptr_t)x & 15) == 0 && (size_t)T * H * (x_bf16 ? 2 : 4) <= 64 * 1024) {
        if (hl == 4) small_exact<4>(x, x_bf16, wr, bias, T, H, E, logits, st);
        else if (hl == 8) small_exact<8>(x, x_bf16, wr, bias, T, H, E, logits, st);
        else if (hl == 16) small_exact<16>(x, x_bf16, wr, bias, T, H, E, logits, st);
        else if (hl == 32) small_exact<32>(x, x_bf16, wr, bias, T, H, E, logits, st);
        else small_exact<64>(x, x_bf16, wr, bias, T, H, E, logits, st);
        return hipGetLastError();
    }
    const int tpw = T <= 64 ? T : 32;
    dim3 grid((E + 3) / 4, (T + tpw - 1) / tpw);
    if (x_bf16)
        hipLaunchKernelGGL(k_logits_exact<uint16_t>, grid, dim3(256), 0, st, (const uint16_t*)x, wr, bias, T, H, E,
                           tpw, logits);
    else
        hipLaunchKernelGGL(k_logits_exact<float>, grid, dim3(256), 0, st, (const float*)x, wr, bias, T, H, E, tpw,
                           logits);
    return hipGetLastError();
}

hipError_t launch_logits_fast(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                              float* logits, hipStream_t st) {
    dim3 grid((T + FL_BM - 1) / FL_BM, (E + FL_BN - 1) / FL_BN);
    hipLaunchKernelGGL(k_logits_fast, grid, dim3(256), 0, st, x, wr, bias, T, H, E, logits);
    return hipGetLastError();
}

template <int VPL>
static hipError_t sel_dispatch_x(const float* logits, int T, int E, int K, float tau, int exact, const void* x,
                                 int x_bf16, const float* wr, const float* bias, int H, int32_t* idx, float* w,
                                 int32_t* nre, hipStream_t st) {
    dim3 grid((T + 3) / 4);
    if (x_bf16)
        hipLaunchKernelGGL((k_route_select<VPL, uint16_t>), grid, dim3(256), 0, st, logits, T, E, K, tau, exact,
                           (const uint16_t*)x, wr, bias, H, idx, w, nre);
    else
        hipLaunchKernelGGL((k_route_select<VPL, float>), grid, dim3(256), 0, st, logits, T, E, K, tau, exact,
                           (const float*)x, wr, bias, H, idx, w, nre);
    return hipGetLastError();
}

hipError_t launch_route_select(const float* logits, int T, int E, int K, float tau, int exact, const void* x,
                               int x_bf16, const float* wr, const float* bias, int H, int32_t* idx, float* w,
                               int32_t* rechecked, hipStream_t st) {
    const int vpl = (E + WAVE - 1) / WAVE;
    if (vpl <= 1) return sel_dispatch_x<1>(logits, T, E, K, tau, exact, x, x_bf16, wr, bias, H, idx, w, rechecked, st);
    if (vpl <= 2) return sel_dispatch_x<2>(logits, T, E, K, tau, exact, x, x_bf16, wr, bias, H, idx, w, rechecked, st);
    if (vpl <= 4) return sel_dispatch_x<4>(logits, T, E, K, tau, exact, x, x_bf16, wr, bias, H, idx, w, rechecked, st);
    if (vpl <= 8) return sel_dispatch_x<8>(logits, T, E, K, tau, exact, x, x_bf16, wr, bias, H, idx, w, rechecked, st);
    if (vpl <= 16) return sel_dispatch_x<16>(logits, T, E, K, tau, exact, x, x_bf16, wr, bias, H, idx, w, rechecked, st);
    if (vpl <= 32) return sel_dispatch_x<32>(logits, T, E, K, tau, exact, x, x_bf16, wr, bias, H, idx, w, rechecked, st);
    return sel_dispatch_x<64>(logits, T, E, K, tau, exact, x, x_bf16, wr, bias, H, idx, w, rechecked, st);
}
