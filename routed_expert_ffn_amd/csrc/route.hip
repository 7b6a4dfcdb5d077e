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
#include "device.h"
#include "group.h"
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

// Up to four exact logit dot products of one token row by a whole wave, with
// the same per-lane order and butterfly as wave_dot_exact; the loads of an
// 8-term slice of every candidate are issued together (the recheck of a
// near-tie is latency-bound otherwise).  Results for c >= nc are meaningless.
template <typename XT>
MOE_DEV void wave_dot_exact4(const XT* __restrict__ xrow, const float* __restrict__ wr, const int (&ce)[4], int nc,
                             int H, double (&out)[4]) {
    constexpr int U = 8;
    const int l = lane_id();
    // every load is unconditional (a predicated load would serialise on its
    // wait): past-the-end terms re-read element H-1 and are not accumulated,
    // absent candidates re-read the first
    const float* wrow[4];
#pragma unroll
    for (int c = 0; c < 4; c++) wrow[c] = wr + (long)(c < nc ? ce[c] : ce[0]) * H;
    double p[4] = {0.0, 0.0, 0.0, 0.0};
    for (int h0 = 0; h0 < H; h0 += WAVE * U) {
        double xv[U];
        float wv[4][U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int h = min(h0 + u * WAVE + l, H - 1);
            xv[u] = xval(xrow, h);
#pragma unroll
            for (int c = 0; c < 4; c++) wv[c][u] = wrow[c][h];
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (h0 + u * WAVE + l < H) {
#pragma unroll
                for (int c = 0; c < 4; c++) p[c] = __fma_rn(xv[u], (double)wv[c][u], p[c]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 4; c++) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) p[c] += __shfl_xor(p[c], d, WAVE);
        out[c] = p[c];
    }
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

// The router weight split once per call: w = hi + mid + lo exactly, each a
// bf16 (8 significant bits each cover fp32's 24), stored as three planes
// [3][E][H] so the estimate is a plain bf16 GEMM of x against all three.
// One block per router row; the block also stores the row's squared norm
// (summed in a fixed order) for the selection's error margin, and thread 0 of
// block 0 clears the recheck queue's counter for the selection that follows.
__global__ __launch_bounds__(256) void k_router_split(const float* __restrict__ wr, int H,
                                                      uint16_t* __restrict__ planes, long plane_elems,
                                                      float* __restrict__ wnorm2, int32_t* __restrict__ rc_count) {
    __shared__ float part[4];
    const int e = blockIdx.x;
    if (e == 0 && threadIdx.x == 0) rc_count[0] = 0;
    const int h4 = H / 4;
    float sq = 0.f;
#pragma unroll 4
    for (int j = threadIdx.x; j < h4; j += 256) {
        const long i = (long)e * h4 + j;
        const float4 wv = reinterpret_cast<const float4*>(wr)[i];
        const float w4[4] = {wv.x, wv.y, wv.z, wv.w};
        uint32_t hi[2], mi[2], lo[2];
#pragma unroll
        for (int q = 0; q < 2; q++) {
            uint16_t h16[2], m16[2], l16[2];
#pragma unroll
            for (int u = 0; u < 2; u++) {
                const float w = w4[q * 2 + u];
                sq = fmaf(w, w, sq);
                h16[u] = f32_to_bf16_rne(w);
                const float r1 = w - bf16_to_f32(h16[u]);
                m16[u] = f32_to_bf16_rne(r1);
                const float r2 = r1 - bf16_to_f32(m16[u]);
                l16[u] = f32_to_bf16_rne(r2);
            }
            hi[q] = h16[0] | ((uint32_t)h16[1] << 16);
            mi[q] = m16[0] | ((uint32_t)m16[1] << 16);
            lo[q] = l16[0] | ((uint32_t)l16[1] << 16);
        }
        reinterpret_cast<uint2*>(planes)[i] = make_uint2(hi[0], hi[1]);
        reinterpret_cast<uint2*>(planes + plane_elems)[i] = make_uint2(mi[0], mi[1]);
        reinterpret_cast<uint2*>(planes + 2 * plane_elems)[i] = make_uint2(lo[0], lo[1]);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) sq += __shfl_xor(sq, d, WAVE);
    if (lane_id() == 0) part[threadIdx.x / WAVE] = sq;
    __syncthreads();
    if (threadIdx.x == 0) wnorm2[e] = (part[0] + part[1]) + (part[2] + part[3]);
}

// Estimate GEMM: block tile 128 tokens x 128 experts, K step 64, two LDS stages
// filled by the LDS DMA (rows of 128 B, 16-byte chunks XOR-swizzled by row & 7);
// 4 waves as 2 x 2 of 64 x 64 on the 32x32x16 MFMA, the three weight planes
// multiplied against the same activation fragments into one accumulator.
namespace {
constexpr int LM_BM = 128, LM_BN = 128, LM_BK = 64;
constexpr int LM_A = LM_BM * LM_BK * 2;                  // 16 KB
constexpr int LM_B = LM_BN * LM_BK * 2;                  // 16 KB per plane
constexpr int LM_STAGE = LM_A + 3 * LM_B;                // 64 KB
constexpr int LM_DMA_A = LM_A / 1024 / 4, LM_DMA_B = 3 * LM_B / 1024 / 4;   // 4 + 12 per wave
typedef __attribute__((address_space(3))) void lds_void_t;
template <int N>
MOE_DEV void lm_wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
MOE_DEV void lm_wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
}  // namespace

__global__ __launch_bounds__(256) void k_logits_mfma(const uint16_t* __restrict__ x, const uint16_t* __restrict__ planes,
                                                     const float* __restrict__ bias, int T, int H, int E,
                                                     float* __restrict__ logits) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int mt = (T + LM_BM - 1) / LM_BM, ntl = (E + LM_BN - 1) / LM_BN;
    const int items = mt * ntl;
    // consecutive items (the n-tiles of one token tile) stay on one XCD
    const int per_xcd = (items + 7) / 8;
    const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if ((int)(blockIdx.x >> 3) >= per_xcd || item >= items) return;
    const int m0 = (item / ntl) * LM_BM, n0 = (item % ntl) * LM_BN;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), l = lane_id();
    const int wm = wave >> 1, wn = wave & 1;
    const int dma_row = l >> 3, dma_slot = l & 7;
    const unsigned char* xb = (const unsigned char*)x;
    const unsigned char* pb = (const unsigned char*)planes;
    uint32_t a_off[LM_DMA_A];
#pragma unroll
    for (int i = 0; i < LM_DMA_A; i++) {
        const int r = (wave * LM_DMA_A + i) * 8 + dma_row;
        const int t = m0 + r < T ? m0 + r : m0;          // rows past T re-read the first (discarded)
        a_off[i] = (uint32_t)t * (uint32_t)(H * 2) + (uint32_t)((dma_slot ^ (r & 7)) * 16);
    }
    uint32_t b_off[LM_DMA_B];
#pragma unroll
    for (int i = 0; i < LM_DMA_B; i++) {
        const int q = wave * LM_DMA_B + i;               // 0..47: plane q/16, rows (q%16)*8 ..
        const int plane = q >> 4, n = (q & 15) * 8 + dma_row;
        const int e = n0 + n < E ? n0 + n : n0;
        b_off[i] = ((uint32_t)plane * (uint32_t)E + (uint32_t)e) * (uint32_t)(H * 2) +
                   (uint32_t)((dma_slot ^ (n & 7)) * 16);
    }
    auto issue = [&](int k) __attribute__((always_inline)) {
        unsigned char* st = smem + (k & 1) * LM_STAGE;
#pragma unroll
        for (int i = 0; i < LM_DMA_A; i++)
            __builtin_amdgcn_global_load_lds(xb + k * LM_BK * 2 + a_off[i], (lds_void_t*)(st + (wave * LM_DMA_A + i) * 1024), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < LM_DMA_B; i++)
            __builtin_amdgcn_global_load_lds(pb + k * LM_BK * 2 + b_off[i],
                                             (lds_void_t*)(st + LM_A + (wave * LM_DMA_B + i) * 1024), 16, 0, 0);
    };
    const int fr = l & 31, fh = l >> 5;
    struct Frag { bf16x8_t a[2][2], b[3][2][2]; };
    auto load_frag = [&](Frag& f, int stage, int kk) __attribute__((always_inline)) {
        const unsigned char* st = smem + stage * LM_STAGE;
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int c = kk * 4 + q * 2 + fh;
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int r = wm * 64 + i * 32 + fr;
                f.a[i][q] = *reinterpret_cast<const bf16x8_t*>(st + r * 128 + ((c ^ (r & 7)) * 16));
            }
#pragma unroll
            for (int p = 0; p < 3; p++)
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const int n = wn * 64 + j * 32 + fr;
                    f.b[p][j][q] = *reinterpret_cast<const bf16x8_t*>(st + LM_A + p * LM_B + n * 128 + ((c ^ (n & 7)) * 16));
                }
        }
    };
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;
    auto mma = [&](const Frag& f) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 2; q++)
#pragma unroll
            for (int p = 0; p < 3; p++)
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < 2; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[p][j][q], f.a[i][q], acc[i][j], 0, 0, 0);
    };
    auto interleave = [&]() __attribute__((always_inline)) {   // 16 LDS reads over 24 MFMAs
#pragma unroll
        for (int q = 0; q < 8; q++) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < 8; q++) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
    };

    const int nk = H / LM_BK;
    issue(0);
    if (nk > 1) {
        issue(1);
        lm_wait_vmcnt<LM_DMA_A + LM_DMA_B>();
    } else {
        lm_wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    Frag f0, f1;
    load_frag(f0, 0, 0);
    auto step = [&](int k, bool more) __attribute__((always_inline)) {
        const int s = k & 1;
        load_frag(f1, s, 1);
        mma(f0);
        interleave();
        lm_wait_vmcnt<0>();
        lm_wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        if (more) issue(k + 2);
        load_frag(f0, s ^ 1, 0);
        mma(f1);
        interleave();
    };
    int k = 0;
    for (; k + 2 < nk; k++) step(k, true);
    if (k + 1 < nk) { step(k, false); k++; }
    load_frag(f1, k & 1, 1);
    mma(f0);
    mma(f1);

    // acc[i][j][v]: token m0 + wm*64 + i*32 + (l & 31), expert n0 + wn*64 + j*32 + (v/4)*8 + (l>>5)*4 + v%4
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int t = m0 + wm * 64 + i * 32 + fr;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int e = n0 + wn * 64 + j * 32 + g * 8 + fh * 4;
                float v4[4];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const float a = acc[i][j][g * 4 + u];
                    v4[u] = bias ? __fadd_rn(a, bias[min(e + u, E - 1)]) : a;
                }
                if (e + 3 < E) {
                    *reinterpret_cast<float4*>(logits + (long)t * E + e) = make_float4(v4[0], v4[1], v4[2], v4[3]);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; u++)
                        if (e + u < E) logits[(long)t * E + e + u] = v4[u];
                }
            }
    }
}

// ------------------------------------------------------------------ selection

constexpr int SEL_CAP = 64;   // candidates re-decided on exact logits (one per lane)

// Top-`rounds` of the 64-bit keys held by the wave (any layout); lane r
// receives round r's key.  Selected entries are cleared from k[].
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

// Routing weights of a wave's selection (lane k < K holds the k-th value and
// id): softmax over the K selected values, written to row t.
MOE_DEV void write_selection(float sel_v, int sel_i, int K, long t, int32_t* __restrict__ idx_out,
                             float* __restrict__ w_out) {
    const int l = lane_id();
    const float w = selection_weight(sel_v, K);
    if (l < K) {
        idx_out[t * K + l] = sel_i;
        w_out[t * K + l] = w;
    }
}

// One wave per token; the leading values come from the threshold cut (the
// K-th largest lane maximum bounds the candidates, which are then ranked),
// with the round-by-round selection when more than 64 candidates pass it.
// With exact logits the top K is final.  With estimates,
// a token whose K+1 leading values are all separated by at least tau is final
// too; any other token is queued, with its cut (K-th estimate - tau), for
// k_route_recheck and written there.
//
// The margin of a token is tau_t = max(tau, tau_scale * |x_t| * max_e |w_e|)
// (Euclidean norms; tau_scale = 2^-24 sqrt(H)): the estimate's accumulation
// error grows in proportion to the magnitudes of x and of the router rows,
// so the margin keeps its headroom over that error when either is scaled.
template <int VPL>
__global__ __launch_bounds__(256) void k_route_select(const float* __restrict__ logits, int T, int E, int K,
                                                      float tau, int exact, const uint16_t* __restrict__ xb, int H,
                                                      const float* __restrict__ wnorm2, float tau_scale,
                                                      int32_t* __restrict__ idx_out,
                                                      float* __restrict__ w_out, int32_t* __restrict__ rechecked,
                                                      int2* __restrict__ rc_list, int32_t* __restrict__ rc_count) {
    const int wave = threadIdx.x / WAVE;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int l = lane_id();
    const float* row = logits + (long)t * E;
    uint32_t kv[VPL];
    load_order_keys<VPL>(row, E, kv);
    if (!exact) {
        float xs = 0.f, wm = 0.f;
        const uint4* xr = reinterpret_cast<const uint4*>(xb + (long)t * H);
        for (int c = l; c < H / 8; c += WAVE) {
            const uint4 v = xr[c];
            const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const float a = bf16lo_to_f32(q[u]), b = bf16hi_to_f32(q[u]);
                xs = fmaf(a, a, xs);
                xs = fmaf(b, b, xs);
            }
        }
        for (int e = l; e < E; e += WAVE) wm = fmaxf(wm, wnorm2[e]);
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            xs += __shfl_xor(xs, d, WAVE);
            wm = fmaxf(wm, __shfl_xor(wm, d, WAVE));
        }
        tau = fmaxf(tau, tau_scale * sqrtf(xs * wm));
    }
    const int rounds = (exact || K == E) ? K : K + 1;
    uint32_t key;
    int sel_i;
    __shared__ uint2 cut_scratch[4][2 * WAVE];
    if (!select_top_cut<VPL>(kv, rounds, cut_scratch[wave], cut_scratch[wave] + WAVE, key, sel_i))
        select_top<VPL>(kv, rounds, key, sel_i);
    const float sel_v = order_key_value(key);
    bool flagged = false;
    if (!exact) {
        // every gap between consecutive selected values, down to the (K+1)-th, must clear tau
        const float nxt = __shfl_down(sel_v, 1, WAVE);
        const bool check = l < K && l + 1 < rounds;
        flagged = __ballot(check && !(sel_v - nxt >= tau)) != 0;
    }
    if (rechecked && l == 0) rechecked[t] = flagged ? 1 : 0;
    if (flagged) {
        const float cut = __shfl(sel_v, K - 1, WAVE) - tau;
        if (l == 0) {
            const int slot = atomicAdd(rc_count, 1);
            rc_list[slot] = make_int2(t, __float_as_int(cut));
        }
        return;
    }
    write_selection(sel_v, sel_i, K, t, idx_out, w_out);
}

// A few tokens on exact logits (T <= 16, T*K <= PERM_CHUNK): one block
// selects every token's top K (one wave per token, as k_route_select) and then
// groups the T*K slots by expert in the same block -- counts, offsets, the
// stable permutation and its inverse, exactly as the grouping kernels do -- so
// selection and grouping take one launch.
template <int VPL>
__global__ __launch_bounds__(1024) void k_route_select_group(const float* __restrict__ logits, int T, int E, int K,
                                                             int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);   // [E]
    int* cur = reinterpret_cast<int*>(mask + E);                              // [E]
    int* sidx = cur + E;                                                      // [T*K] selected experts
    __shared__ int wave_tot[16];
    __shared__ uint2 cut_scratch[16][2 * WAVE];
    const int wave = threadIdx.x / WAVE, l = lane_id();
    for (int e = threadIdx.x; e < E; e += blockDim.x) { cur[e] = 0; mask[e] = 0ull; }
    if (wave < T) {
        const int t = wave;
        const float* row = logits + (long)t * E;
        uint32_t kv[VPL];
        load_order_keys<VPL>(row, E, kv);
        uint32_t key;
        int sel_i;
        if (!select_top_cut<VPL>(kv, K, cut_scratch[wave], cut_scratch[wave] + WAVE, key, sel_i))
            select_top<VPL>(kv, K, key, sel_i);
        write_selection(order_key_value(key), sel_i, K, t, idx_out, w_out);
        if (l < K) sidx[t * K + l] = sel_i;
    }
    __syncthreads();
    const int n = T * K;
    for (int s = threadIdx.x; s < n; s += blockDim.x) {
        const int e = sidx[s];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cur[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] = cur[e];
    __syncthreads();
    const int total = block_exclusive_scan(cur, E, wave_tot);
    for (int e = threadIdx.x; e < E; e += blockDim.x) offsets[e] = cur[e];
    if (threadIdx.x == 0) offsets[E] = total;
    __syncthreads();
    if (wave == 0) wave_stable_scatter(sidx, 0, n, E, cur, mask, perm, inv);
}

// Re-decision of the queued tokens on exact logits, one block per token at a
// time: the candidates are every expert whose estimate exceeds the cut (all E
// if more than 64 do), their exact keys are computed four per wave pass, and
// the first wave selects the top K among them.
template <int VPL, typename XT>
__global__ __launch_bounds__(256) void k_route_recheck(const float* __restrict__ est, int T, int E, int K,
                                                       const int2* __restrict__ rc_list,
                                                       const int32_t* __restrict__ rc_count,
                                                       const XT* __restrict__ x, const float* __restrict__ wr,
                                                       const float* __restrict__ bias, int H,
                                                       int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
    __shared__ unsigned long long keys[VPL * WAVE];
    __shared__ int cids[VPL * WAVE];
    __shared__ int s_n;
    const int tid = threadIdx.x, wave = tid / WAVE, l = lane_id();
    const int n = rc_count[0];
    for (int it = blockIdx.x; it < n; it += gridDim.x) {
        const int2 ent = rc_list[it];
        const int t = ent.x;
        const float cut = __int_as_float(ent.y);
        if (tid == 0) s_n = 0;
        __syncthreads();
        for (int e = tid; e < E; e += 256)
            if (est[(long)t * E + e] > cut) cids[atomicAdd(&s_n, 1)] = e;
        __syncthreads();
        const bool all = s_n > SEL_CAP;
        const int nc = all ? E : s_n;
        const XT* xrow = x + (long)t * H;
        for (int g = wave * 4; g < nc; g += 16) {
            int ce[4];
#pragma unroll
            for (int c = 0; c < 4; c++) ce[c] = g + c < nc ? (all ? g + c : cids[g + c]) : 0;
            const int m = min(4, nc - g);
            double d[4];
            wave_dot_exact4(xrow, wr, ce, m, H, d);
            if (l == 0) {
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    if (c < m) {
                        float lv = (float)d[c];
                        if (bias) lv = __fadd_rn(lv, bias[ce[c]]);
                        keys[g + c] = route_key(lv, ce[c]);
                    }
                }
            }
        }
        __syncthreads();
        if (wave == 0) {
            unsigned long long k[VPL];
#pragma unroll
            for (int j = 0; j < VPL; j++) k[j] = l + j * WAVE < nc ? keys[l + j * WAVE] : 0ull;
            const unsigned long long sel = select_rounds<VPL>(k, K);
            write_selection(route_key_value(sel), route_key_index(sel), K, t, idx_out, w_out);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ exact logits, few tokens

// G = 2 or 4 waves per expert, wave h taking tokens h, h + G, ...: the router
// row (H fp32) is held in registers (H/64 independent loads per lane in
// flight), the token rows are staged in LDS.  4 / G experts per block, so a
// block's four waves fill a CU's four SIMDs; G = 4 when two experts per block
// would leave CUs without a block.
constexpr int XS_MAX_T = 16;
constexpr int XS_GROUP = 4;          // tokens whose partial sums a wave builds together

// Lane j < D receives lane j + D's value (the other lanes' results are not
// used): the pairings of the exact logit's summation tree, on 64-bit values.
// D = 32 and 16 cross rows of 16 lanes with the permlane swaps, D = 8 and 4
// shift within a row (row_shl), D = 2 and 1 are quad permutations.
template <int D>
MOE_DEV double lane_down(double v) {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    unsigned lo = (unsigned)u, hi = (unsigned)(u >> 32);
    if constexpr (D == 32) {
        lo = __builtin_amdgcn_permlane32_swap(lo, lo, false, false)[1];
        hi = __builtin_amdgcn_permlane32_swap(hi, hi, false, false)[1];
    } else if constexpr (D == 16) {
        lo = __builtin_amdgcn_permlane16_swap(lo, lo, false, false)[1];
        hi = __builtin_amdgcn_permlane16_swap(hi, hi, false, false)[1];
    } else {
        constexpr int ctrl = D == 8 ? 0x108 : D == 4 ? 0x104 : D == 2 ? 0x4E : 0xB1;
        lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)lo, ctrl, 0xF, 0xF, false);
        hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)hi, ctrl, 0xF, 0xF, false);
    }
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// Logits of NT tokens t0, t0 + G, ... for this wave's expert: the strided
// partial sums of all NT tokens are built in one pass over the row (each in
// ascending i), then every step of the tree runs on all of them.
template <typename XT, int HL, int NT, int G>
MOE_DEV void logits_group(const XT* xs, const float (&wf)[HL], int H, int t0, int l, float b, bool has_bias, int E,
                          int e, float* __restrict__ logits) {
    double p[NT];
#pragma unroll
    for (int k = 0; k < NT; k++) p[k] = 0.0;
#pragma unroll
    for (int i = 0; i < HL; i++) {
        const double wd = (double)wf[i];
#pragma unroll
        for (int k = 0; k < NT; k++) p[k] = __fma_rn(xval(xs + (long)(t0 + G * k) * H, l + i * WAVE), wd, p[k]);
    }
#pragma unroll
    for (int k = 0; k < NT; k++) p[k] += lane_down<32>(p[k]);
#pragma unroll
    for (int k = 0; k < NT; k++) p[k] += lane_down<16>(p[k]);
#pragma unroll
    for (int k = 0; k < NT; k++) p[k] += lane_down<8>(p[k]);
#pragma unroll
    for (int k = 0; k < NT; k++) p[k] += lane_down<4>(p[k]);
#pragma unroll
    for (int k = 0; k < NT; k++) p[k] += lane_down<2>(p[k]);
#pragma unroll
    for (int k = 0; k < NT; k++) p[k] += lane_down<1>(p[k]);
    if (l == 0) {
#pragma unroll
        for (int k = 0; k < NT; k++) {
            float v = (float)p[k];
            if (has_bias) v = __fadd_rn(v, b);
            logits[(long)(t0 + G * k) * E + e] = v;
        }
    }
}

template <typename XT, int HL, int G>
__global__ __launch_bounds__(256) void k_logits_exact_small(const XT* __restrict__ x, const float* __restrict__ wr,
                                                            const float* __restrict__ bias, int T, int H, int E,
                                                            float* __restrict__ logits) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    XT* xs = reinterpret_cast<XT*>(smem);
    const int tid = threadIdx.x;
    const int l = lane_id();
    const int wave = tid / WAVE;
    const int e = blockIdx.x * (4 / G) + wave / G;
    const int h = wave % G;
    const int er = e < E ? e : E - 1;              // a wave past E re-reads row E-1
    // x [T][H] goes to LDS by the LDS DMA (1 KB of 16-byte chunks per wave
    // instruction; the LDS is sized to whole 1 KB pieces and past the end the
    // last chunk is loaded again into the padding), issued before the router
    // row's loads so that it lands while the router row still streams in
    const int per = 16 / (int)sizeof(XT);
    const int nchunk = T * H / per;
    const unsigned char* xg = reinterpret_cast<const unsigned char*>(x);
    for (int c = wave * WAVE; c < nchunk; c += 4 * WAVE)
        __builtin_amdgcn_global_load_lds(xg + (long)min(c + l, nchunk - 1) * 16, (lds_void_t*)(smem + (long)c * 16), 16,
                                         0, 0);
    float wf[HL];
#pragma unroll
    for (int i = 0; i < HL; i++) wf[i] = wr[(long)er * H + l + i * WAVE];   // H == 64 * HL
    const float b = bias ? bias[er] : 0.f;
    lm_wait_vmcnt<0>();
    __syncthreads();
    if (e >= E) return;
    const int nt = (T - h + G - 1) / G;            // tokens h, h + G, ... below T
    for (int k0 = 0; k0 < nt; k0 += XS_GROUP) {
        const int t0 = h + G * k0;
        const int m = nt - k0;
        if (m >= 4) logits_group<XT, HL, 4, G>(xs, wf, H, t0, l, b, bias != nullptr, E, e, logits);
        else if (m == 3) logits_group<XT, HL, 3, G>(xs, wf, H, t0, l, b, bias != nullptr, E, e, logits);
        else if (m == 2) logits_group<XT, HL, 2, G>(xs, wf, H, t0, l, b, bias != nullptr, E, e, logits);
        else logits_group<XT, HL, 1, G>(xs, wf, H, t0, l, b, bias != nullptr, E, e, logits);
    }
}

// ------------------------------------------------------------------ launchers

template <int HL, int G>
static void small_exact_g(const void* x, int x_bf16, const float* wr, const float* bias, int T, int H, int E,
                          float* logits, hipStream_t st) {
    const size_t lds = ((size_t)T * H * (x_bf16 ? 2 : 4) + 1023) / 1024 * 1024;   // whole 1 KB DMA pieces
    const dim3 grid((E + 4 / G - 1) / (4 / G));
    if (x_bf16)
        hipLaunchKernelGGL((k_logits_exact_small<uint16_t, HL, G>), grid, dim3(256), lds, st, (const uint16_t*)x, wr,
                           bias, T, H, E, logits);
    else
        hipLaunchKernelGGL((k_logits_exact_small<float, HL, G>), grid, dim3(256), lds, st, (const float*)x, wr, bias,
                           T, H, E, logits);
}
template <int HL>
static bool small_exact(const void* x, int x_bf16, const float* wr, const float* bias, int T, int H, int E,
                        float* logits, hipStream_t st) {
    int ncu = 0;
    if (current_device_cus(&ncu) != hipSuccess || ncu <= 0) ncu = 256;
    if ((E + 1) / 2 < ncu) small_exact_g<HL, 4>(x, x_bf16, wr, bias, T, H, E, logits, st);
    else small_exact_g<HL, 2>(x, x_bf16, wr, bias, T, H, E, logits, st);
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

bool logits_fast_eligible(int T, int H, int E) {
    return H % LM_BK == 0 && E % 4 == 0 && (size_t)T * H * 2 < ((size_t)1 << 32) &&
           (size_t)3 * E * H * 2 < ((size_t)1 << 32);
}

size_t logits_fast_planes_bytes(int H, int E) { return (size_t)3 * E * H * 2; }

hipError_t launch_logits_fast(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                              float* logits, uint16_t* planes, float* wnorm2, int32_t* rc_count, hipStream_t st) {
    hipLaunchKernelGGL(k_router_split, dim3(E), dim3(256), 0, st, wr, H, planes, (long)E * H, wnorm2, rc_count);
    static LdsLimit lim;          // the estimate GEMM's LDS limit, raised once per device
    hipError_t e = lim.ensure((const void*)k_logits_mfma, 2 * LM_STAGE);
    if (e != hipSuccess) return e;
    const int items = ((T + LM_BM - 1) / LM_BM) * ((E + LM_BN - 1) / LM_BN);
    hipLaunchKernelGGL(k_logits_mfma, dim3((items + 7) / 8 * 8), dim3(256), 2 * LM_STAGE, st, x, planes, bias, T, H, E,
                       logits);
    return hipGetLastError();
}

template <int VPL>
static hipError_t sel_dispatch(const float* logits, int T, int E, int K, float tau, int exact, const void* x,
                               int x_bf16, const float* wr, const float* bias, int H, const float* wnorm2,
                               int32_t* idx, float* w, int32_t* flags, int2* rc_list, int32_t* rc_count,
                               hipStream_t st) {
    const float tau_scale = ldexpf(sqrtf((float)H), -24);
    hipLaunchKernelGGL((k_route_select<VPL>), dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E, K, tau, exact,
                       (const uint16_t*)x, H, wnorm2, tau_scale, idx, w, flags, rc_list, rc_count);
    if (exact) return hipGetLastError();
    const int grid = T < 256 ? T : 256;
    if (x_bf16)
        hipLaunchKernelGGL((k_route_recheck<VPL, uint16_t>), dim3(grid), dim3(256), 0, st, logits, T, E, K, rc_list,
                           rc_count, (const uint16_t*)x, wr, bias, H, idx, w);
    else
        hipLaunchKernelGGL((k_route_recheck<VPL, float>), dim3(grid), dim3(256), 0, st, logits, T, E, K, rc_list,
                           rc_count, (const float*)x, wr, bias, H, idx, w);
    return hipGetLastError();
}

hipError_t launch_route_select(const float* logits, int T, int E, int K, float tau, int exact, const void* x,
                               int x_bf16, const float* wr, const float* bias, int H, const float* wnorm2,
                               int32_t* idx, float* w, int32_t* flags, int2* rc_list, int32_t* rc_count,
                               hipStream_t st) {
    if (!exact && (!x_bf16 || !wnorm2 || H % 8 != 0)) return hipErrorInvalidValue;
    const int vpl = (E + WAVE - 1) / WAVE;
#define MOE_SEL(V) return sel_dispatch<V>(logits, T, E, K, tau, exact, x, x_bf16, wr, bias, H, wnorm2, idx, w, flags, rc_list, rc_count, st)
    if (vpl <= 1) MOE_SEL(1);
    if (vpl <= 2) MOE_SEL(2);
    if (vpl <= 4) MOE_SEL(4);
    if (vpl <= 8) MOE_SEL(8);
    if (vpl <= 16) MOE_SEL(16);
    if (vpl <= 32) MOE_SEL(32);
    MOE_SEL(64);
#undef MOE_SEL
}

bool route_group_fused_eligible(int T, int K, int E) {
    return T >= 1 && T <= 16 && (long)T * K <= PERM_CHUNK && E <= 4096;
}

hipError_t launch_route_select_group(const float* logits, int T, int E, int K, int32_t* idx, float* w,
                                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, hipStream_t st) {
    const size_t lds = (size_t)E * (sizeof(unsigned long long) + sizeof(int)) + (size_t)T * K * sizeof(int);
    const dim3 block(WAVE * (T > 4 ? T : 4));
    const int vpl = (E + WAVE - 1) / WAVE;
#define MOE_SELG(V)                                                                                              \
    hipLaunchKernelGGL((k_route_select_group<V>), dim3(1), block, lds, st, logits, T, E, K, idx, w, counts, offsets, \
                       perm, inv);                                                                               \
    return hipGetLastError()
    if (vpl <= 1) { MOE_SELG(1); }
    if (vpl <= 2) { MOE_SELG(2); }
    if (vpl <= 4) { MOE_SELG(4); }
    if (vpl <= 8) { MOE_SELG(8); }
    if (vpl <= 16) { MOE_SELG(16); }
    if (vpl <= 32) { MOE_SELG(32); }
    MOE_SELG(64);
#undef MOE_SELG
}
