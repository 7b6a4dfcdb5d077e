// ffn_gemm.hip -- the grouped expert GEMMs for many rows per expert (prefill).
//
// Per touched expert e with rows p in [off_e, off_e + n_e) (token perm[p] / K):
//   gate/up:  C = X_e [Wg_e; Wu_e]^T  (K = H),  a = bf16(silu(C_g) * C_u)  -> A[p][f]
//   down:     Y = A_e Wd_e^T         (K = F)                              -> y_perm[p][h]
// (expert = gate/up/down matrices, "Strata Coder 编程模型深度剖析" §3).
//
// MFMA-bound at prefill (an 8192-token chunk is ~465 flop per weight byte),
// so the kernel is built around the bf16 MFMA 16x16x32:
//   * block tile 128 rows x 256 columns, K step 64; 4 waves, each 64 x 128 (32
//     MFMA tiles, 128 fp32 accumulators), which keeps LDS reads at ~75% of the
//     MFMA time;
//   * global -> LDS with the gfx950 LDS DMA (global_load_lds_dwordx4): no VGPR
//     staging, three LDS stages (3 x 48 KB) so two K steps of loads are in
//     flight while one is multiplied;
//   * LDS rows are 128 B with the 16-byte chunks XOR-swizzled by (row & 7), so
//     the MFMA operand reads (16 rows x 16 B per lane group) hit distinct
//     banks; the swizzle is applied on the global side of the DMA;
//   * gate/up: the 256 B-rows of a block are, per wave half, 64 gate rows then
//     the same 64 up rows, so silu(g)*u meets in one lane's accumulators;
//   * the activation rows are gathered through perm in the DMA addresses;
//   * a plan kernel lists every (expert, 128-row tile); blocks map to
//     (m-tile, n-tile) with n fastest, and consecutive work items are kept on
//     one XCD (blocks are dealt round-robin over the 8 XCDs) so the tiles that
//     share weights and activation rows share an L2.
#include "common.h"
#include "launch.h"

namespace {

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int STAGES = 3;
constexpr int A_BYTES = BM * BK * 2;          // 16 KB
constexpr int B_BYTES = BN * BK * 2;          // 32 KB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int DMA_A = A_BYTES / 1024 / 4;     // 1 KB DMA instructions per wave per stage (A)
constexpr int DMA_B = B_BYTES / 1024 / 4;     // (B)
constexpr int DMA_PER_STAGE = DMA_A + DMA_B;  // 12

typedef __attribute__((address_space(3))) void lds_void;

MOE_DEV void dma16(const void* g, lds_void* l) {
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
MOE_DEV void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

MOE_DEV float silu_g(float g) { return g / (1.0f + expf(-g)); }

}  // namespace

// Plan: tiles[i] = (expert, first row, rows) for every 128-row tile of every
// touched expert, in expert order; tiles_count[0] = their number.
__global__ __launch_bounds__(256) void k_gemm_plan(const int32_t* __restrict__ offsets, int E,
                                                   int4* __restrict__ tiles, int32_t* __restrict__ count) {
    __shared__ int wave_tot[4];
    __shared__ int s_base;
    if (threadIdx.x == 0) s_base = 0;
    __syncthreads();
    for (int e0 = 0; e0 < E; e0 += 256) {
        const int e = e0 + threadIdx.x;
        int off = 0, n = 0;
        if (e < E) { off = offsets[e]; n = offsets[e + 1] - off; }
        const int t = (n + BM - 1) / BM;
        const int incl = wave_incl_scan(t);
        const int w = threadIdx.x / WAVE;
        if (lane_id() == WAVE - 1) wave_tot[w] = incl;
        __syncthreads();
        int before = s_base;
        for (int i = 0; i < w; i++) before += wave_tot[i];
        const int start = before + incl - t;
        for (int j = 0; j < t; j++) tiles[start + j] = make_int4(e, off + j * BM, min(BM, n - j * BM), 0);
        __syncthreads();
        if (threadIdx.x == 255) s_base = start + t;
        __syncthreads();
    }
    if (threadIdx.x == 0) count[0] = s_base;
}

template <int PHASE, int YBF16>   // PHASE 0: gate/up (K = H), 1: down (K = F)
__global__ __launch_bounds__(256) void k_gemm(const uint16_t* __restrict__ src, const uint16_t* __restrict__ w0,
                                              const uint16_t* __restrict__ w1, const int4* __restrict__ tiles,
                                              const int32_t* __restrict__ tile_count, const int32_t* __restrict__ perm,
                                              int topk, int H, int F, void* __restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int KD = PHASE == 0 ? H : F;            // reduction length
    const int NT = PHASE == 0 ? (2 * F) / BN : H / BN;   // n-tiles per m-tile
    const int items = tile_count[0] * NT;
    // XCD-aware work mapping: blocks b = x (mod 8) take a contiguous range of items
    const int per_xcd = (items + 7) / 8;
    const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if ((blockIdx.x >> 3) >= per_xcd || item >= items) return;
    const int4 tl = tiles[item / NT];
    const int e = tl.x, row0 = tl.y, rows = tl.z;
    const int nt = item % NT;

    const int tid = threadIdx.x, wave = tid / WAVE, l = lane_id();
    const int wm = wave >> 1, wn = wave & 1;

    // ---- DMA source rows (per lane: one row for each of this wave's instructions)
    // an instruction covers 8 rows x 128 B: lane j -> row r0 + j/8, slot j%8 holding chunk (j%8) ^ (row & 7)
    const int dma_row = l >> 3, dma_slot = l & 7;
    const uint16_t* a_src[DMA_A];
#pragma unroll
    for (int i = 0; i < DMA_A; i++) {
        const int r = (wave * DMA_A + i) * 8 + dma_row;
        const int rr = r < rows ? r : 0;              // rows past the expert's count re-read row 0 (discarded)
        long base;
        if constexpr (PHASE == 0) base = (long)(perm[row0 + rr] / topk) * H;
        else base = (long)(row0 + rr) * F;
        a_src[i] = src + base + ((dma_slot ^ (r & 7)) * 8);
    }
    const uint16_t* b_src[DMA_B];
#pragma unroll
    for (int i = 0; i < DMA_B; i++) {
        const int n = (wave * DMA_B + i) * 8 + dma_row;     // B tile row 0..255
        long wrow;
        const uint16_t* wsrc;
        if constexpr (PHASE == 0) {
            const int half = n >> 7, q = n & 127;            // wave half, then 64 gate rows + 64 up rows
            const int f = nt * 128 + half * 64 + (q & 63);
            wsrc = q < 64 ? w0 : w1;
            wrow = (long)e * F + f;
        } else {
            wsrc = w0;
            wrow = (long)e * H + nt * BN + n;
        }
        b_src[i] = wsrc + wrow * KD + ((dma_slot ^ (n & 7)) * 8);
    }
    auto issue = [&](int k) __attribute__((always_inline)) {
        unsigned char* st = smem + (k % STAGES) * STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < DMA_A; i++)
            dma16(a_src[i] + k * BK, (lds_void*)(st + (wave * DMA_A + i) * 1024));
#pragma unroll
        for (int i = 0; i < DMA_B; i++)
            dma16(b_src[i] + k * BK, (lds_void*)(st + A_BYTES + (wave * DMA_B + i) * 1024));
    };

    f32x4_t acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = KD / BK;
    issue(0);
    if (nk > 1) issue(1);
    // operand read offsets: row within the stage region, swizzled chunk
    const int fr = l & 15, fg = l >> 4;
    for (int k = 0; k < nk; k++) {
        if (k + 1 < nk) wait_vmcnt<DMA_PER_STAGE>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        if (k + 2 < nk) issue(k + 2);
        const unsigned char* st = smem + (k % STAGES) * STAGE_BYTES;
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
            const int c = kk * 4 + fg;
            bf16x8_t af[4], bfr[8];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = wm * 64 + i * 16 + fr;
                af[i] = *reinterpret_cast<const bf16x8_t*>(st + r * 128 + ((c ^ (r & 7)) * 16));
            }
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const int n = wn * 128 + j * 16 + fr;
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(st + A_BYTES + n * 128 + ((c ^ (n & 7)) * 16));
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 8; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }

    // ---- epilogue.  acc[i][j]: rows wm*64 + i*16 + fg*4 + r, column (l & 15) of n-subtile j
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int m = wm * 64 + i * 16 + fg * 4 + r;
            if (m >= rows) continue;
            const long prow = row0 + m;
            if constexpr (PHASE == 0) {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int f = nt * 128 + wn * 64 + j * 16 + fr;
                    const float a = silu_g(acc[i][j][r]) * acc[i][j + 4][r];
                    ((uint16_t*)out)[prow * F + f] = f32_to_bf16_rne(a);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const int h = nt * BN + wn * 128 + j * 16 + fr;
                    if constexpr (YBF16) ((uint16_t*)out)[prow * H + h] = f32_to_bf16_rne(acc[i][j][r]);
                    else ((float*)out)[prow * H + h] = acc[i][j][r];
                }
            }
        }
    }
}

bool ffn_gemm_eligible(int H, int F) { return H % BN == 0 && H % BK == 0 && (2 * F) % BN == 0 && F % BK == 0; }

// Workspace: [A n x F bf16][tiles: (n/BM + min(E,n)) x int4][count]
size_t ffn_gemm_workspace_bytes(int T, int K, int E, int H, int F) {
    (void)H;
    const size_t n = (size_t)T * K;
    const size_t mt = n / BM + (size_t)(E < (int)n ? E : (int)n) + 1;
    return (n * F * 2 + 255) / 256 * 256 + (mt * 16 + 255) / 256 * 256 + 256;
}

hipError_t launch_ffn_gemm(const void* x, const void* wg, const void* wu, const void* wd, const int32_t* offsets,
                           const int32_t* perm, int T, int K, int H, int F, int E, void* y, int y_bf16, void* ws,
                           hipStream_t st) {
    const size_t n = (size_t)T * K;
    const size_t mt = n / BM + (size_t)(E < (int)n ? E : (int)n) + 1;
    char* base = (char*)ws;
    uint16_t* abuf = (uint16_t*)base;
    int4* tiles = (int4*)(base + (n * F * 2 + 255) / 256 * 256);
    int32_t* count = (int32_t*)((char*)tiles + (mt * 16 + 255) / 256 * 256);
    hipLaunchKernelGGL(k_gemm_plan, dim3(1), dim3(256), 0, st, offsets, E, tiles, count);
    const size_t lds = (size_t)STAGES * STAGE_BYTES;
    const int items_g = (int)mt * ((2 * F) / BN), items_d = (int)mt * (H / BN);
    const int grid_g = (items_g + 7) / 8 * 8, grid_d = (items_d + 7) / 8 * 8;
    hipLaunchKernelGGL((k_gemm<0, 1>), dim3(grid_g), dim3(256), lds, st, (const uint16_t*)x, (const uint16_t*)wg,
                       (const uint16_t*)wu, tiles, count, perm, K, H, F, (void*)abuf);
    if (y_bf16)
        hipLaunchKernelGGL((k_gemm<1, 1>), dim3(grid_d), dim3(256), lds, st, (const uint16_t*)abuf,
                           (const uint16_t*)wd, nullptr, tiles, count, perm, K, H, F, y);
    else
        hipLaunchKernelGGL((k_gemm<1, 0>), dim3(grid_d), dim3(256), lds, st, (const uint16_t*)abuf,
                           (const uint16_t*)wd, nullptr, tiles, count, perm, K, H, F, y);
    return hipGetLastError();
}
