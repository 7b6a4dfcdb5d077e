// ffn_stream.hip -- the expert FFN for a handful of tokens (T <= 8: the
// speculative verify step of 4 drafts + 1, and decode); bf16 weights, and
// int4 / int3 / int2 blocks of 32 with an fp16 scale.
//
// Per touched expert e with rows p in [off_e, off_e + n_e) (token perm[p] / K):
//   a[p] = bf16(silu(x Wg_e^T) * (x Wu_e^T)),   y_perm[p] = a[p] Wd_e^T
// (expert = gate/up/down matrices, "Strata Coder 编程模型深度剖析" §3).
//
// At this size the layer is one stream of expert weights (each touched
// expert's matrices are read once, ~1 flop per byte), so the kernels are built
// to keep HBM busy:
//   * persistent blocks (two per CU); every wave walks its own sequence of
//     equal-sized work items (FR feature rows of gate and up, or DR hidden rows
//     of down), consecutive items going to concurrently running waves so the
//     weight rows in flight at any moment are contiguous;
//   * the next item's weight rows are loaded (non-temporal 16-byte loads, one
//     contiguous 1 KB chunk of a row per wave instruction, never predicated)
//     while the current item is multiplied, so the loads of a wave never stop;
//   * the operands that are reused, the token rows (gate/up) or all the
//     intermediate rows (down), sit in LDS, loaded once per block, together
//     with the touched-expert list, which every block derives from the
//     grouping offsets itself (no preparation kernel);
//   * each lane multiplies its 8 weights by the matching 8 activations of every
//     row of the expert with v_dot2_f32_bf16; the per-lane partial sums are
//     combined across the wave by a transposing butterfly (with V sums per
//     lane, each xor step keeps half of them and adds the partner's copy of
//     that half, so lane l ends with the full sum of entry l >> (6 - log2 V)).
#include <type_traits>

#include "common.h"
#include "device.h"
#include "launch.h"
#include "stream.h"


// gate/up.  Item = (touched expert j, feature tile): FR gate rows and the same
// FR up rows over the whole of H = CH x 512.  LDS: the T token rows, the
// touched list, the token of every grouped row.
template <int NT, int CH, int FR, int RING>
__global__ __launch_bounds__(256) void k_gateup_stream(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
                                                       const uint16_t* __restrict__ wu,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ perm, int T, int K, int E, int F,
                                                       uint16_t* __restrict__ abuf) {
    constexpr int H = CH * 512;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                          // [T][H]
    int4* list = reinterpret_cast<int4*>(smem + (size_t)T * H * 2);            // [<= T*K]
    int* prow = reinterpret_cast<int*>(list + T * K);                          // [T*K] token of grouped row
    __shared__ int scan[4];
    const int tid = threadIdx.x, wave = tid / WAVE, l = lane_id();
    // the grouped rows' tokens and the touched list (from the offsets) come
    // first; then the first items' weight loads and all of the token rows'
    // loads go out together, so the block waits for memory twice before it
    // multiplies
    const int pv = tid < T * K ? perm[tid] : 0;
    const int nlist = block_touched_list(offsets, E, list, scan);
    if (tid < T * K) prow[tid] = pv / K;
    for (int i = tid + 256; i < T * K; i += 256) prow[i] = perm[i] / K;
    __syncthreads();

    const int tpe = F / FR;                     // items per expert
    const int n_items = nlist * tpe;
    const int W = gridDim.x * 4;
    const int it = blockIdx.x * 4 + wave;
    const bool active = it < n_items;

    uint4 wbuf[RING][2 * FR][CH];
    auto load = [&](int item, uint4 (&w)[2 * FR][CH]) __attribute__((always_inline)) {
        const int e = list[item / tpe].x, f0 = (item % tpe) * FR;
        const uint16_t* g0 = wg + ((long)e * F + f0) * H + l * 8;
        const uint16_t* u0 = wu + ((long)e * F + f0) * H + l * 8;
#pragma unroll
        for (int c = 0; c < CH; c++)
#pragma unroll
            for (int r = 0; r < FR; r++) {
                w[r][c] = ldnt16(g0 + (long)r * H + c * 512);
                w[FR + r][c] = ldnt16(u0 + (long)r * H + c * 512);
            }
    };
    auto compute = [&](int item, const uint4 (&w)[2 * FR][CH]) __attribute__((always_inline)) {
        const int4 ent = list[item / tpe];
        const int off = ent.y, n = __builtin_amdgcn_readfirstlane(ent.z), f0 = (item % tpe) * FR;
        auto rows = [&](auto ntn) __attribute__((always_inline)) {
            constexpr int NTN = decltype(ntn)::value;
            constexpr int V = 2 * FR * NTN;
            float acc[V];
#pragma unroll
            for (int i = 0; i < V; i++) acc[i] = 0.f;
#pragma unroll
            for (int t = 0; t < NTN; t++) {
                if (t < n) {
                    const uint16_t* xr = xs + prow[off + t] * H + l * 8;
#pragma unroll
                    for (int c = 0; c < CH; c++) {
                        const uint4 a = *reinterpret_cast<const uint4*>(xr + c * 512);
#pragma unroll
                        for (int r = 0; r < 2 * FR; r++) acc[r * NTN + t] = dot8bf(w[r][c], a, acc[r * NTN + t]);
                    }
                }
            }
            // lane l owns entry j = l >> shift: row r = j / NTN (< FR gate, else up), token t = j % NTN
            const float v = wave_tr_reduce<V>(acc);
            constexpr int shift = tr_shift<V>();
            const float up = __shfl_down(v, (FR * NTN) << shift, WAVE);
            const int j = l >> shift, r = j / NTN, t = j % NTN;
            if ((l & ((1 << shift) - 1)) == 0 && r < FR && t < n)
                abuf[(long)(off + t) * F + f0 + r] = f32_to_bf16_rne(silu_ref(v) * up);
        };
        by_rows<NT>(n, rows);
    };
    // (for H > 2048 the first item's buffers are too large to hold across
    // the staging: the loads go out after it)
    constexpr bool early = CH <= 4;
    if (early && active) ring_start<RING>(it, W, n_items, wbuf, load);
    {
        constexpr int MAXC = NT * H * 2 / 16 / 256;   // 16-byte chunks per thread for T = NT
        constexpr int BATCH = MAXC < 8 ? MAXC : 8;
        const int n16 = T * H * 2 / 16;
        const uint4* g = reinterpret_cast<const uint4*>(x);
#pragma unroll
        for (int c0 = 0; c0 < MAXC; c0 += BATCH) {
            uint4 r[BATCH];
#pragma unroll
            for (int c = 0; c < BATCH; c++) r[c] = g[min(tid + (c0 + c) * 256, n16 - 1)];
#pragma unroll
            for (int c = 0; c < BATCH; c++)   // past the end: the last chunk again, same value
                reinterpret_cast<uint4*>(xs)[min(tid + (c0 + c) * 256, n16 - 1)] = r[c];
        }
    }
    if (!early && active) ring_start<RING>(it, W, n_items, wbuf, load);
    __syncthreads();
    if (!active) return;
    ring_run<RING>(it, W, n_items, wbuf, load, compute);
}

// down.  Item = (touched expert j, hidden tile): DR rows of Wd over the whole
// of F = FCH x 512.  The expert's intermediate rows (n <= NT, a few KB, L2
// resident) are loaded with the weights of the item, so nothing is staged.
template <int NT, int FCH, int DR, int YBF16, int RING>
__global__ __launch_bounds__(256) void k_down_stream(const uint16_t* __restrict__ abuf, const uint16_t* __restrict__ wd,
                                                     const int32_t* __restrict__ offsets, int nrows, int E, int H,
                                                     void* __restrict__ y) {
    constexpr int F = FCH * 512;
    __shared__ int4 list[256];                   // touched experts (<= nrows <= 256)
    __shared__ int scan[4];
    (void)nrows;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / WAVE), l = lane_id();
    const int nlist = block_touched_list(offsets, E, list, scan);
    __syncthreads();

    const int tpe = H / DR;
    const int n_items = nlist * tpe;
    const int W = gridDim.x * 4;
    int it = blockIdx.x * 4 + wave;
    if (it >= n_items) return;

    struct Buf { uint4 w[DR][FCH]; uint4 a[NT][FCH]; };
    Buf wbuf[RING];
    auto load = [&](int item, Buf& b) __attribute__((always_inline)) {
        const int4 ent = list[item / tpe];
        const int e = __builtin_amdgcn_readfirstlane(ent.x), off = __builtin_amdgcn_readfirstlane(ent.y);
        const int n = __builtin_amdgcn_readfirstlane(ent.z);
        const int h0 = (item % tpe) * DR;
        const uint16_t* d0 = wd + ((long)e * H + h0) * F + l * 8;
#pragma unroll
        for (int c = 0; c < FCH; c++)
#pragma unroll
            for (int r = 0; r < DR; r++) b.w[r][c] = ldnt16(d0 + (long)r * F + c * 512);
#pragma unroll
        for (int t = 0; t < NT; t++)
            if (t < n) {                         // wave-uniform
#pragma unroll
                for (int c = 0; c < FCH; c++)
                    b.a[t][c] = *reinterpret_cast<const uint4*>(abuf + (long)(off + t) * F + c * 512 + l * 8);
            }
    };
    auto compute = [&](int item, const Buf& b) __attribute__((always_inline)) {
        const int4 ent = list[item / tpe];
        const int off = ent.y, n = __builtin_amdgcn_readfirstlane(ent.z), h0 = (item % tpe) * DR;
        auto rows = [&](auto ntn) __attribute__((always_inline)) {
            constexpr int NTN = decltype(ntn)::value;
            constexpr int V = DR * NTN;
            float acc[V];
#pragma unroll
            for (int i = 0; i < V; i++) acc[i] = 0.f;
#pragma unroll
            for (int t = 0; t < NTN; t++) {
                if (t < n) {
#pragma unroll
                    for (int c = 0; c < FCH; c++)
#pragma unroll
                        for (int r = 0; r < DR; r++) acc[r * NTN + t] = dot8bf(b.w[r][c], b.a[t][c], acc[r * NTN + t]);
                }
            }
            const float v = wave_tr_reduce<V>(acc);
            constexpr int shift = tr_shift<V>();
            const int j = l >> shift, r = j / NTN, t = j % NTN;
            if ((l & ((1 << shift) - 1)) == 0 && t < n) {
                const long o = (long)(off + t) * H + h0 + r;
                if constexpr (YBF16) ((uint16_t*)y)[o] = f32_to_bf16_rne(v);
                else ((float*)y)[o] = v;
            }
        };
        by_rows<NT>(n, rows);
    };
    ring_walk<RING>(it, W, n_items, wbuf, load, compute);
}

// ---------------------------------------------------------------------------- int4 weights
//
// Block int4 (32 consecutive inputs share an fp16 scale d; value d (u - 8), u
// the stored nibble, element 2j in the low nibble of byte j).  One lane's 16
// bytes are exactly one quant block, so a 1 KB wave instruction reads 64
// whole blocks.  The nibbles become the exact bf16 values 128 + u (bit pattern
// 0x4300 | u), so with the block's activation sum S = sum x:
//     sum_k x w = d (D - 136 S),  D = sum_k x (128 + u)   (v_dot2_f32_bf16)
// and S comes from LDS, summed once per block of activations.


// gate/up, int4 / int3 / int2 (QB bits).  Item = FR gate rows and the same FR
// up rows over all of H = CH x 2048 (a lane: one quant block per row and chunk).
template <int NT, int CH, int FR, int RING, int QB>
__global__ __launch_bounds__(256, (QB == 4 ? 1 : 2)) void k_gateup_stream_q4(const uint16_t* __restrict__ x, const uint8_t* __restrict__ wg,
                                                          const uint8_t* __restrict__ wu, const uint16_t* __restrict__ sg,
                                                          const uint16_t* __restrict__ su,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ perm, int T, int K, int E, int F,
                                                          uint16_t* __restrict__ abuf) {
    constexpr int H = CH * 2048;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                           // [T][H]
    float* xsum = reinterpret_cast<float*>(smem + (size_t)T * H * 2);           // [T][H/32]
    int4* list = reinterpret_cast<int4*>(xsum + T * (H / 32));                  // [<= T*K]
    int* prow = reinterpret_cast<int*>(list + T * K);                           // [T*K]
    __shared__ int scan[4];
    const int tid = threadIdx.x, wave = tid / WAVE, l = lane_id();
    stage_lds(x, T * H * 2 / 1024, smem, wave, l);
    for (int i = tid; i < T * K; i += 256) prow[i] = perm[i] / K;
    const int nlist = block_touched_list(offsets, E, list, scan);
    __syncthreads();
    block_sums(xs, T, H, xsum);
    __syncthreads();

    const int tpe = F / FR;
    const int n_items = nlist * tpe;
    const int W = gridDim.x * 4;
    const int it = blockIdx.x * 4 + wave;
    if (it >= n_items) return;

    constexpr int QW = QWords<QB>::n;
    struct Buf { uint32_t q[2 * FR][CH][QW]; uint16_t d[2 * FR][CH]; };
    Buf wbuf[RING];
    auto load = [&](int item, Buf& b) __attribute__((always_inline)) {
        const long row0 = (long)list[item / tpe].x * F + (item % tpe) * FR;
#pragma unroll
        for (int r = 0; r < FR; r++)
#pragma unroll
            for (int c = 0; c < CH; c++) {
                load_block<QB>(b.q[r][c], wg + (row0 + r) * (H * QB / 8), H, c * 64 + l);
                load_block<QB>(b.q[FR + r][c], wu + (row0 + r) * (H * QB / 8), H, c * 64 + l);
                b.d[r][c] = ldnt_u16(sg + (row0 + r) * (H / 32) + c * 64 + l);
                b.d[FR + r][c] = ldnt_u16(su + (row0 + r) * (H / 32) + c * 64 + l);
            }
    };
    auto compute = [&](int item, const Buf& b) __attribute__((always_inline)) {
        const int4 ent = list[item / tpe];
        const int off = ent.y, n = __builtin_amdgcn_readfirstlane(ent.z), f0 = (item % tpe) * FR;
        auto rows = [&](auto ntn) __attribute__((always_inline)) {
            constexpr int NTN = decltype(ntn)::value;
            constexpr int V = 2 * FR * NTN;
            float acc[V];
#pragma unroll
            for (int i = 0; i < V; i++) acc[i] = 0.f;
#pragma unroll
            for (int t = 0; t < NTN; t++) {
                if (t < n) {
                    const int tok = prow[off + t];
#pragma unroll
                    for (int c = 0; c < CH; c++) {
                        const uint16_t* xl = xs + tok * H + c * 2048 + l * 32;
                        const float S = xsum[tok * (H / 32) + c * 64 + l];
#pragma unroll
                        for (int r = 0; r < 2 * FR; r++) {
                            const float D = dot_block<QB>(b.q[r][c], xl);
                            acc[r * NTN + t] =
                                fmaf(fp16_to_f32(b.d[r][c]), fmaf(-zero_level<QB>(), S, D), acc[r * NTN + t]);
                        }
                    }
                }
            }
            const float v = wave_tr_reduce<V>(acc);
            constexpr int shift = tr_shift<V>();
            const float up = __shfl_down(v, (FR * NTN) << shift, WAVE);
            const int j = l >> shift, r = j / NTN, t = j % NTN;
            if ((l & ((1 << shift) - 1)) == 0 && r < FR && t < n)
                abuf[(long)(off + t) * F + f0 + r] = f32_to_bf16_rne(silu_ref(v) * up);
        };
        by_rows<NT>(n, rows);
    };
    ring_walk<RING>(it, W, n_items, wbuf, load, compute);
}

// down, int4 / int3 / int2 (QB bits), F = 512: a wave instruction covers 4
// rows of Wd (16 lanes x one quant block each).  Item = I instructions = 4I
// hidden rows.
template <int NT, int I, int YBF16, int RING, int QB>
__global__ __launch_bounds__(256) void k_down_stream_q4(const uint16_t* __restrict__ abuf, const uint8_t* __restrict__ wd,
                                                        const uint16_t* __restrict__ sd,
                                                        const int32_t* __restrict__ offsets, int nrows, int E, int H,
                                                        void* __restrict__ y) {
    constexpr int F = 512, NB = F / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t* as = reinterpret_cast<uint16_t*>(smem);                            // [nrows][F]
    float* asum = reinterpret_cast<float*>(smem + (size_t)nrows * F * 2);        // [nrows][F/32]
    int4* list = reinterpret_cast<int4*>(asum + nrows * NB);                     // [<= nrows]
    __shared__ int scan[4];
    const int tid = threadIdx.x, wave = tid / WAVE, l = lane_id();
    stage_lds(abuf, nrows * F * 2 / 1024, smem, wave, l);
    const int nlist = block_touched_list(offsets, E, list, scan);
    __syncthreads();
    block_sums(as, nrows, F, asum);
    __syncthreads();

    const int tpe = H / (4 * I);
    const int n_items = nlist * tpe;
    const int W = gridDim.x * 4;
    const int it = blockIdx.x * 4 + wave;
    if (it >= n_items) return;
    const int g = l >> 4, b = l & 15;            // row within an instruction, quant block within the row

    constexpr int QW = QWords<QB>::n;
    struct Buf { uint32_t q[I][QW]; uint16_t d[I]; };
    Buf wbuf[RING];
    auto load = [&](int item, Buf& bf) __attribute__((always_inline)) {
        const long row0 = (long)list[item / tpe].x * H + (item % tpe) * (4 * I) + g;
#pragma unroll
        for (int i = 0; i < I; i++) {
            load_block<QB>(bf.q[i], wd + (row0 + 4 * i) * (F * QB / 8), F, b);
            bf.d[i] = ldnt_u16(sd + (row0 + 4 * i) * NB + b);
        }
    };
    auto compute = [&](int item, const Buf& bf) __attribute__((always_inline)) {
        const int4 ent = list[item / tpe];
        const int off = ent.y, n = __builtin_amdgcn_readfirstlane(ent.z), h0 = (item % tpe) * (4 * I);
        auto rows = [&](auto ntn) __attribute__((always_inline)) {
            constexpr int NTN = decltype(ntn)::value;
            constexpr int V = I * NTN;
            static_assert(V <= 16, "one entry per lane after the 16-lane reduction");
            float acc[V];
#pragma unroll
            for (int i = 0; i < V; i++) acc[i] = 0.f;
#pragma unroll
            for (int t = 0; t < NTN; t++) {
                if (t < n) {
                    const uint16_t* al = as + (off + t) * F + b * 32;
                    const float S = asum[(off + t) * NB + b];
#pragma unroll
                    for (int i = 0; i < I; i++) {
                        const float D = dot_block<QB>(bf.q[i], al);
                        acc[i * NTN + t] = fmaf(fp16_to_f32(bf.d[i]), fmaf(-zero_level<QB>(), S, D), acc[i * NTN + t]);
                    }
                }
            }
            const float v = group16_tr_reduce<V>(acc);
            constexpr int shift = V == 16 ? 0 : V == 8 ? 1 : V == 4 ? 2 : V == 2 ? 3 : 4;
            const int j = b >> shift, i = j / NTN, t = j % NTN;
            if ((b & ((1 << shift) - 1)) == 0 && t < n) {
                const long o = (long)(off + t) * H + h0 + 4 * i + g;
                if constexpr (YBF16) ((uint16_t*)y)[o] = f32_to_bf16_rne(v);
                else ((float*)y)[o] = v;
            }
        };
        by_rows<NT>(n, rows);
    };
    ring_walk<RING>(it, W, n_items, wbuf, load, compute);
}

// ---------------------------------------------------------------------------- host

namespace {
constexpr int GU_FR = 2, DN_DR = 8;
constexpr int GU_RING = 2, DN_RING = 2;      // weight buffers per wave (16 KB / 8 KB items)
constexpr size_t STREAM_LDS_MAX = 64 * 1024;    // two blocks per CU

size_t gu_lds(int T, int K, int H) { return (size_t)T * H * 2 + (size_t)T * K * 16 + (size_t)T * K * 4; }
size_t dn_lds(int T, int K, int F) { (void)T; (void)K; (void)F; return 0; }   // rows are loaded per item

int stream_grid(hipError_t& err) {
    int ncu = 0;
    err = current_device_cus(&ncu);
    return 2 * (ncu > 0 ? ncu : 1);
}

template <int NT, int CH>
hipError_t gu_launch(int grid, hipStream_t st, const uint16_t* x, const void* wg, const void* wu,
                     const int32_t* offsets, const int32_t* perm, int T, int K, int E, int F, uint16_t* abuf) {
    auto kern = k_gateup_stream<NT, CH, GU_FR, GU_RING>;
    const size_t lds = gu_lds(T, K, CH * 512);
    static LdsLimit lim;   // this launcher's kernel: raise its LDS limit once per device
    hipError_t e = lim.ensure((const void*)kern, (int)STREAM_LDS_MAX);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, x, (const uint16_t*)wg, (const uint16_t*)wu, offsets,
                       perm, T, K, E, F, abuf);
    return hipSuccess;
}

template <int NT, int FCH, int YB>
hipError_t dn_launch(int grid, hipStream_t st, const uint16_t* abuf, const void* wd, const int32_t* offsets,
                     int nrows, int T, int K, int E, int H, void* y) {
    auto kern = k_down_stream<NT, FCH, DN_DR, YB, DN_RING>;
    const size_t lds = dn_lds(T, K, FCH * 512);
    static LdsLimit lim;   // this launcher's kernel: raise its LDS limit once per device
    hipError_t e = lim.ensure((const void*)kern, (int)STREAM_LDS_MAX);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, abuf, (const uint16_t*)wd, offsets, nrows, E, H, y);
    return hipSuccess;
}

template <int NT>
hipError_t stream_nt(int grid, hipStream_t st, const uint16_t* x, const void* wg, const void* wu, const void* wd,
                     const int32_t* offsets, const int32_t* perm, int T, int K, int E, int H, int F, void* y,
                     int y_bf16, uint16_t* abuf) {
    hipError_t e;
    switch (H / 512) {
        case 1: e = gu_launch<NT, 1>(grid, st, x, wg, wu, offsets, perm, T, K, E, F, abuf); break;
        case 2: e = gu_launch<NT, 2>(grid, st, x, wg, wu, offsets, perm, T, K, E, F, abuf); break;
        case 4: e = gu_launch<NT, 4>(grid, st, x, wg, wu, offsets, perm, T, K, E, F, abuf); break;
        default: e = gu_launch<NT, 8>(grid, st, x, wg, wu, offsets, perm, T, K, E, F, abuf); break;
    }
    if (e != hipSuccess) return e;
    const int nrows = T * K;
    if (F == 512)
        return y_bf16 ? dn_launch<NT, 1, 1>(grid, st, abuf, wd, offsets, nrows, T, K, E, H, y)
                      : dn_launch<NT, 1, 0>(grid, st, abuf, wd, offsets, nrows, T, K, E, H, y);
    return y_bf16 ? dn_launch<NT, 2, 1>(grid, st, abuf, wd, offsets, nrows, T, K, E, H, y)
                  : dn_launch<NT, 2, 0>(grid, st, abuf, wd, offsets, nrows, T, K, E, H, y);
}
}  // namespace

namespace {
constexpr int Q4_FR = 4, Q4_I = 2;
// weight items in flight per wave: int4 items are the largest
constexpr int Q_RING = 2;   // weight items per wave: one in flight while one multiplies
size_t gu_lds_q4(int T, int K, int H) { return (size_t)T * H * 2 + (size_t)T * (H / 32) * 4 + (size_t)T * K * 20; }
size_t dn_lds_q4(int T, int K) { return (size_t)T * K * 512 * 2 + (size_t)T * K * 16 * 4 + (size_t)T * K * 16; }

template <int NT, int CH, int QB>
hipError_t gu_launch_q4(int grid, hipStream_t st, const uint16_t* x, const void* wg, const void* wu, const void* sg,
                        const void* su, const int32_t* offsets, const int32_t* perm, int T, int K, int E, int F,
                        uint16_t* abuf) {
    auto kern = k_gateup_stream_q4<NT, CH, Q4_FR, Q_RING, QB>;
    const size_t lds = gu_lds_q4(T, K, CH * 2048);
    static LdsLimit lim;   // this launcher's kernel: raise its LDS limit once per device
    hipError_t e = lim.ensure((const void*)kern, (int)STREAM_LDS_MAX);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, x, (const uint8_t*)wg, (const uint8_t*)wu,
                       (const uint16_t*)sg, (const uint16_t*)su, offsets, perm, T, K, E, F, abuf);
    return hipSuccess;
}
template <int NT, int YB, int QB>
hipError_t dn_launch_q4(int grid, hipStream_t st, const uint16_t* abuf, const void* wd, const void* sd,
                        const int32_t* offsets, int T, int K, int E, int H, void* y) {
    auto kern = k_down_stream_q4<NT, Q4_I, YB, Q_RING, QB>;
    const size_t lds = dn_lds_q4(T, K);
    static LdsLimit lim;   // this launcher's kernel: raise its LDS limit once per device
    hipError_t e = lim.ensure((const void*)kern, (int)STREAM_LDS_MAX);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, abuf, (const uint8_t*)wd, (const uint16_t*)sd, offsets,
                       T * K, E, H, y);
    return hipSuccess;
}
template <int NT, int QB>
hipError_t stream_q4_nt(int grid, hipStream_t st, const uint16_t* x, const void* wg, const void* wu, const void* wd,
                        const void* sg, const void* su, const void* sd, const int32_t* offsets, const int32_t* perm,
                        int T, int K, int E, int H, int F, void* y, int y_bf16, uint16_t* abuf) {
    hipError_t e = gu_launch_q4<NT, 1, QB>(grid, st, x, wg, wu, sg, su, offsets, perm, T, K, E, F, abuf);   // H = 2048
    if (e != hipSuccess) return e;
    return y_bf16 ? dn_launch_q4<NT, 1, QB>(grid, st, abuf, wd, sd, offsets, T, K, E, H, y)
                  : dn_launch_q4<NT, 0, QB>(grid, st, abuf, wd, sd, offsets, T, K, E, H, y);
}
template <int QB>
hipError_t stream_q_bits(int grid, hipStream_t st, const void* x, const void* wg, const void* wu, const void* wd,
                         const void* sg, const void* su, const void* sd, const int32_t* offsets, const int32_t* perm,
                         int T, int K, int E, int H, int F, void* y, int y_bf16, uint16_t* abuf) {
    return T <= 4 ? stream_q4_nt<4, QB>(grid, st, (const uint16_t*)x, wg, wu, wd, sg, su, sd, offsets, perm, T, K, E, H,
                                        F, y, y_bf16, abuf)
                  : stream_q4_nt<8, QB>(grid, st, (const uint16_t*)x, wg, wu, wd, sg, su, sd, offsets, perm, T, K, E, H,
                                        F, y, y_bf16, abuf);
}
}  // namespace

bool ffn_stream_q4_eligible(int T, int K, int E, int H, int F) {
    return T >= 1 && T <= 8 && H == 2048 && F == 512 && E <= 256 * EPT &&
           gu_lds_q4(T, K, H) <= STREAM_LDS_MAX && dn_lds_q4(T, K) <= STREAM_LDS_MAX;
}

hipError_t launch_ffn_stream_q4(const void* x, const void* wg, const void* wu, const void* wd, const void* sg,
                                const void* su, const void* sd, const int32_t* offsets, const int32_t* perm, int T,
                                int K, int H, int F, int E, void* y, int y_bf16, void* ws, hipStream_t st, int bits) {
    hipError_t err;
    const int grid = stream_grid(err);
    if (err != hipSuccess) return err;
    uint16_t* abuf = (uint16_t*)ws;
    if (bits == 4) err = stream_q_bits<4>(grid, st, x, wg, wu, wd, sg, su, sd, offsets, perm, T, K, E, H, F, y, y_bf16, abuf);
    else if (bits == 3) err = stream_q_bits<3>(grid, st, x, wg, wu, wd, sg, su, sd, offsets, perm, T, K, E, H, F, y, y_bf16, abuf);
    else if (bits == 2) err = stream_q_bits<2>(grid, st, x, wg, wu, wd, sg, su, sd, offsets, perm, T, K, E, H, F, y, y_bf16, abuf);
    else return hipErrorInvalidValue;
    if (err != hipSuccess) return err;
    return hipGetLastError();
}

bool ffn_stream_eligible(int T, int K, int E, int H, int F) {
    const int hc = H / 512;
    return T >= 1 && T <= 8 && H % 512 == 0 && (hc == 1 || hc == 2 || hc == 4 || hc == 8) && (F == 512 || F == 1024) &&
           E <= 256 * EPT && gu_lds(T, K, H) <= STREAM_LDS_MAX && dn_lds(T, K, F) <= STREAM_LDS_MAX;
}

size_t ffn_stream_workspace_bytes(int T, int K, int F) { return ((size_t)T * K * F * 2 + 255) / 256 * 256; }

hipError_t launch_ffn_stream(const void* x, const void* wg, const void* wu, const void* wd, const int32_t* offsets,
                             const int32_t* perm, int T, int K, int H, int F, int E, void* y, int y_bf16, void* ws,
                             hipStream_t st) {
    hipError_t err;
    const int grid = stream_grid(err);
    if (err != hipSuccess) return err;
    uint16_t* abuf = (uint16_t*)ws;
    err = T <= 4 ? stream_nt<4>(grid, st, (const uint16_t*)x, wg, wu, wd, offsets, perm, T, K, E, H, F, y, y_bf16, abuf)
                 : stream_nt<8>(grid, st, (const uint16_t*)x, wg, wu, wd, offsets, perm, T, K, E, H, F, y, y_bf16, abuf);
    if (err != hipSuccess) return err;
    return hipGetLastError();
}
