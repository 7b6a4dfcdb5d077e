// ffn_gemm.hip -- the grouped expert GEMMs for many rows per expert (prefill).
//
// Per touched expert e with rows p in [off_e, off_e + n_e) (token perm[p] / K):
//   gate/up:  C = X_e [Wg_e; Wu_e]^T  (K = H),  a = bf16(silu(C_g) * C_u)  -> A[p][f]
//   down:     Y = A_e Wd_e^T         (K = F)                              -> y_perm[p][h]
// (expert = gate/up/down matrices, "Strata Coder 编程模型深度剖析" §3).
//
// At prefill an 8192-token chunk is ~465 flop per weight byte, so the kernel
// is built around the bf16 MFMA 32x32x16 with one wave per SIMD:
//   * block tile BM x BN = 128 x 512, K step 64; each of the 4 waves owns a
//     128 x 128 sub-tile (4 x 4 MFMA tiles, 256 fp32 accumulators), the
//     largest a wave holds, which minimises LDS operand traffic per MFMA;
//   * global -> LDS with the gfx950 LDS DMA (global_load_lds_dwordx4), two LDS
//     stages of 80 KB; the operand fragments are prefetched from LDS into
//     registers one half-step ahead, so LDS reads and the next stage's DMA
//     both run under the MFMAs and one barrier per K step suffices;
//   * LDS rows are 128 B with the 16-byte chunks XOR-swizzled by (row & 7), so
//     the MFMA operand reads hit distinct banks; the swizzle is applied on the
//     global side of the DMA;
//   * the MFMA is issued with the weight fragment as its first operand, so a
//     lane's accumulators are 4 consecutive output columns of one row: the
//     epilogue packs them to bf16 and stages each wave's tile through LDS for
//     16-byte row-contiguous global stores;
//   * gate/up: the 128 B-rows of a wave are 64 gate rows then the same 64 up
//     rows, so silu(g)*u meets in one lane's accumulators;
//   * the activation rows are gathered through perm in the DMA addresses;
//   * a plan kernel lists every (expert, BM-row tile); blocks map to
//     (m-tile, n-tile) with n fastest, and consecutive work items are kept on
//     one XCD (blocks are dealt round-robin over the 8 XCDs) so the tiles that
//     share weights and activation rows share an L2.
// The kernel is bound by filling LDS (L2 misses and the per-step barrier
// that the shared A rows need), not by MFMA issue.
#include <type_traits>

#include "common.h"
#include "device.h"
#include "launch.h"

namespace {

constexpr int BK = 64;
constexpr int NWAVE = 4;

template <int BM, int BN, int WQ>
struct Geo {
    static constexpr int WM = BM / 128, WN = NWAVE / WM;     // waves along rows / columns
    static_assert(BM == 128 && WM * WN == NWAVE, "4 waves side by side over 128 rows");
    static constexpr int WCOLS = BN / WN;                    // columns of a wave's tile: 128 or 64
    static constexpr int JT = WCOLS / 32;                    // its 32-column MFMA tiles
    static_assert(WCOLS == 128 || WCOLS == 64, "wave tile 128 x 128 or 128 x 64");
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int BQ_BYTES = WQ ? BN * BK / 2 : BN * BK * 2;   // B rows: bf16, or int4 nibbles
    static constexpr int BS_BYTES = WQ ? BN * 4 : 0;                  // int4: a row's two fp16 scales per K step
    static constexpr int STAGE = A_BYTES + BQ_BYTES + BS_BYTES;
    static constexpr int DMA_A = A_BYTES / 1024 / NWAVE;     // 1 KB DMA instructions per wave per stage
    static constexpr int DMA_B = BQ_BYTES / 1024 / NWAVE;
    static constexpr int DMA_S = BS_BYTES / 256 / NWAVE;     // 4-byte DMA: 256 B per instruction
    static constexpr int DMA = DMA_A + DMA_B + DMA_S;
    static_assert(DMA_A * 1024 * NWAVE == A_BYTES && DMA_B * 1024 * NWAVE == BQ_BYTES &&
                  DMA_S * 256 * NWAVE == BS_BYTES, "whole DMA instructions per wave");
    // epilogue staging per wave, after stage 0: the activation (128 rows x
    // WCOLS/2 bf16), y in bf16 (two passes of 64 rows) or fp32 (four of 32);
    // each row padded by 16 B
    static constexpr int AST = WCOLS + 16, YST = WCOLS * 2 + 16, FST = WCOLS * 4 + 16;
    static constexpr int EPI_A = 128 * AST, EPI_Y = 64 * YST, EPI_F = 32 * FST;
    static constexpr int EPI_WAVE = EPI_A > EPI_Y ? (EPI_A > EPI_F ? EPI_A : EPI_F) : (EPI_Y > EPI_F ? EPI_Y : EPI_F);
    static constexpr int LDS = 2 * STAGE > STAGE + NWAVE * EPI_WAVE ? 2 * STAGE : STAGE + NWAVE * EPI_WAVE;
    static constexpr int BLOCKS_PER_CU = LDS <= 80 * 1024 ? 2 : 1;   // two blocks share a CU when their LDS fits
};

typedef __attribute__((address_space(3))) void lds_void;

MOE_DEV void dma16(const void* g, lds_void* l) {
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}
MOE_DEV void dma4(const void* g, lds_void* l) {
    __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
}

// s_waitcnt vmcnt(N) / lgkmcnt(0), the other counters left alone (gfx9 encoding)
template <int N>
MOE_DEV void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
MOE_DEV void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// silu(g) = g / (1 + e^-g) with the hardware exp and reciprocal (~1 ulp each;
// the product is rounded to bf16 right after)
MOE_DEV float silu_fast(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16 pair (round to nearest even, one v_cvt_pk_bf16_f32)
MOE_DEV uint32_t cvt_bf16x2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 8 int4 weights of one quant block (element 2b in the low nibble of byte b)
// -> bf16 RNE of d (u - 8): fma(u, d, -8d) rounds the exact product once
// (u d and 8 d are exact in fp32), the same value as the fp32 product.
MOE_DEV bf16x8_t q4x8_bf16(uint32_t w, float d) {
    const float m8 = -8.0f * d;
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    u32x4_t o;
#pragma unroll
    for (int b = 0; b < 4; b++)
        o[b] = cvt_bf16x2(fmaf((float)((lo >> (8 * b)) & 0xFFu), d, m8), fmaf((float)((hi >> (8 * b)) & 0xFFu), d, m8));
    return __builtin_bit_cast(bf16x8_t, o);
}

}  // namespace

// Plan: tiles[i] = (expert, first row, rows) for every bm-row tile of every
// touched expert, in expert order; tiles_count[0] = their number.  One block:
// each thread owns 16 consecutive experts (E <= 4096) and loads their offsets
// at once; the experts' first tile indices go to LDS, and then all threads
// write the tiles, each finding its tile's expert by binary search.
__global__ __launch_bounds__(256) void k_gemm_plan(const int32_t* __restrict__ offsets, int E, int bm,
                                                   int4* __restrict__ tiles, int32_t* __restrict__ count) {
    constexpr int EPT = 16;
    __shared__ int wave_tot[4];
    __shared__ int tstart[256 * EPT + 1];         // first tile of expert e; tstart[E] = total
    __shared__ int eoff[256 * EPT + 1];           // offsets[e]
    const int e0 = threadIdx.x * EPT;
    int off[EPT + 1];
#pragma unroll
    for (int i = 0; i <= EPT; i++) off[i] = offsets[min(e0 + i, E)];
    int t = 0;
#pragma unroll
    for (int i = 0; i < EPT; i++)
        if (e0 + i < E) t += (off[i + 1] - off[i] + bm - 1) / bm;
    const int incl = wave_incl_scan(t);
    const int w = threadIdx.x / WAVE;
    if (lane_id() == WAVE - 1) wave_tot[w] = incl;
    __syncthreads();
    int pos = incl - t;
    for (int i = 0; i < w; i++) pos += wave_tot[i];
    const int total = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
#pragma unroll
    for (int i = 0; i < EPT; i++) {
        if (e0 + i < E) {
            tstart[e0 + i] = pos;
            eoff[e0 + i] = off[i];
            pos += (off[i + 1] - off[i] + bm - 1) / bm;
        }
    }
    if (threadIdx.x == 0) {
        tstart[E] = total;
        eoff[E] = offsets[E];
        count[0] = total;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < total; i += 256) {
        int lo = 0, hi = E;                        // largest e with tstart[e] <= i (experts with no tiles share it)
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tstart[mid] <= i) lo = mid; else hi = mid;
        }
        const int j = i - tstart[lo];
        const int n = eoff[lo + 1] - eoff[lo];
        tiles[i] = make_int4(lo, eoff[lo] + j * bm, min(bm, n - j * bm), 0);
    }
}

// WQ 1: int4 weights (nibbles + fp16 scale per 32 along K), staged in LDS as
// they are and turned into the bf16 MFMA operand in registers as the
// fragments are read; the values are the bf16 RNE of d (u - 8).
template <int BM, int BN, int PHASE, int YBF16, int WQ>   // PHASE 0: gate/up (K = H), 1: down (K = F)
__global__ __launch_bounds__(256, (Geo<BM, BN, WQ>::BLOCKS_PER_CU)) void k_gemm(const uint16_t* __restrict__ src, const void* __restrict__ w0,
                                              const void* __restrict__ w1, const uint16_t* __restrict__ s0,
                                              const uint16_t* __restrict__ s1, const int4* __restrict__ tiles,
                                              const int32_t* __restrict__ tile_count, const int32_t* __restrict__ perm,
                                              int topk, int H, int F, void* __restrict__ out) {
    using G = Geo<BM, BN, WQ>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int KD = PHASE == 0 ? H : F;                       // reduction length
    const int NT = PHASE == 0 ? (2 * F) / BN : H / BN;       // n-tiles per m-tile
    const int nk = KD / BK;
    const int items = tile_count[0] * NT;
    // persistent blocks, XCD-aware: the blocks of XCD x (= blockIdx mod 8) own
    // the contiguous item range [x*per_xcd, (x+1)*per_xcd) and walk it with a
    // stride of their number, so the blocks running together on one XCD work on
    // neighbouring items (same expert weights, same activation rows) in its L2
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslot = gridDim.x >> 3;
    const int per_xcd = (items + 7) / 8;
    const int item_end = min(items, (xcd + 1) * per_xcd);
    int item = xcd * per_xcd + slot;
    if (item >= item_end) return;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), l = lane_id();
    const int wm = wave / G::WN, wn = wave % G::WN;

    // ---- DMA source rows: an instruction covers 8 rows x 128 B; lane j -> row
    // r0 + j/8, LDS slot j%8 holding global chunk (j%8) ^ (row & 7).  Addresses
    // are a wave-uniform base plus a 32-bit per-lane byte offset.
    const int dma_row = l >> 3, dma_slot = l & 7;
    const unsigned char* src_b = (const unsigned char*)src;
    // B: the rows of one instruction are consecutive weight rows (and all gate
    // or all up), so one lane offset serves every instruction.  bf16: 8 rows x
    // 128 B; int4: 32 rows x 32 B of nibbles (lane -> row l/2, 16-B chunk l&1,
    // swizzled by bit 3 of the row), and the scales 64 rows x 4 B.
    const uint32_t b_off = WQ ? (uint32_t)(l >> 1) * (uint32_t)(KD / 2) + (uint32_t)((((l & 1) ^ ((l >> 4) & 1))) * 16)
                              : (uint32_t)dma_row * (uint32_t)(KD * 2) + (uint32_t)((dma_slot ^ dma_row) * 16);
    struct Item { int e, row0, rows, nt; };
    auto item_of = [&](int it) __attribute__((always_inline)) -> Item {
        const int4 tl = tiles[it / NT];
        return Item{tl.x, tl.y, tl.z, it % NT};
    };
    uint32_t a_off[G::DMA_A];
    auto set_a = [&](const Item& c) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < G::DMA_A; i++) {
            const int r = (wave * G::DMA_A + i) * 8 + dma_row;
            const int rr = r < c.rows ? r : 0;        // rows past the tile's count re-read row 0 (discarded)
            uint32_t row;
            if constexpr (PHASE == 0) row = (uint32_t)(perm[c.row0 + rr] / topk);
            else row = (uint32_t)(c.row0 + rr);
            a_off[i] = row * (uint32_t)(KD * 2) + (uint32_t)((dma_slot ^ (r & 7)) * 16);
        }
    };
    // weight row of B tile row n: its index in matrix `mat`.  Gate/up: per
    // wave tile of WCOLS rows, WCOLS/2 gate rows then the same WCOLS/2 up rows.
    auto b_row = [&](const Item& c, int n, int& mat) __attribute__((always_inline)) -> long {
        if constexpr (PHASE == 0) {
            constexpr int HW = G::WCOLS / 2;
            const int q = n & (G::WCOLS - 1);
            mat = q < HW ? 0 : 1;
            return (long)c.e * F + c.nt * (BN / 2) + (n / G::WCOLS) * HW + (q & (HW - 1));
        } else {
            mat = 0;
            return (long)c.e * H + c.nt * BN + n;
        }
    };
    // B DMA groups (8 bf16 rows, 32 int4 rows) never straddle a gate/up half
    static_assert(G::WCOLS / 2 >= 32, "DMA row groups within one matrix");
    auto b_base = [&](const Item& c, int i) __attribute__((always_inline)) -> const unsigned char* {
        int mat;
        const long r = b_row(c, (wave * G::DMA_B + i) * (WQ ? 32 : 8), mat);
        return (const unsigned char*)(mat ? w1 : w0) + r * (WQ ? KD / 2 : KD * 2);
    };
    // int4 scales: 64 rows per instruction, lane l -> row l (per-lane matrix)
    auto s_lane = [&](const Item& c, int i) __attribute__((always_inline)) -> const unsigned char* {
        int mat;
        const long r = b_row(c, (wave * G::DMA_S + i) * 64 + l, mat);
        return (const unsigned char*)(mat ? s1 : s0) + r * (KD / 16);
    };
    auto issue = [&](const Item& c, int k) __attribute__((always_inline)) {
        unsigned char* st = smem + (k & 1) * G::STAGE;
#pragma unroll
        for (int i = 0; i < G::DMA_A; i++)
            dma16(src_b + k * BK * 2 + a_off[i], (lds_void*)(st + (wave * G::DMA_A + i) * 1024));
#pragma unroll
        for (int i = 0; i < G::DMA_B; i++)
            dma16(b_base(c, i) + k * (WQ ? BK / 2 : BK * 2) + b_off,
                  (lds_void*)(st + G::A_BYTES + (wave * G::DMA_B + i) * 1024));
#pragma unroll
        for (int i = 0; i < G::DMA_S; i++)
            dma4(s_lane(c, i) + k * 4,
                 (lds_void*)(st + G::A_BYTES + G::BQ_BYTES + (wave * G::DMA_S + i) * 256));
    };

    // ---- operand fragments of one K half (32) for the 32x32x16 MFMA: 4 row
    // tiles of A and 4 column tiles of B, each as two K=16 slices.  Slice q of
    // lane half fh holds the 8 k values at chunk kk*4 + q*2 + fh (bf16), or at
    // chunk kk*4 + fh*2 + q (int4: a lane's 16 consecutive nibbles then feed
    // both slices); A and B use the same order, so the sum is over the same k.
    const int fr = l & 31, fh = l >> 5;
    constexpr int JT = G::JT;
    struct Frag { bf16x8_t a[4][2], b[JT][2]; };
    auto load_frag = [&](Frag& fragm, int stage, int kk) __attribute__((always_inline)) {
        const unsigned char* st = smem + stage * G::STAGE;
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int c = WQ ? kk * 4 + fh * 2 + q : kk * 4 + q * 2 + fh;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = wm * 128 + i * 32 + fr;
                fragm.a[i][q] = *reinterpret_cast<const bf16x8_t*>(st + r * 128 + ((c ^ (r & 7)) * 16));
            }
            if constexpr (!WQ) {
#pragma unroll
                for (int j = 0; j < JT; j++) {
                    const int n = wn * G::WCOLS + j * 32 + fr;
                    fragm.b[j][q] =
                        *reinterpret_cast<const bf16x8_t*>(st + G::A_BYTES + n * 128 + ((c ^ (n & 7)) * 16));
                }
            }
        }
        if constexpr (WQ) {
            // a lane's 16 nibbles of column n (one quant block) and its scale
#pragma unroll
            for (int j = 0; j < JT; j++) {
                const int n = wn * G::WCOLS + j * 32 + fr;
                const u32x2_t nb = *reinterpret_cast<const u32x2_t*>(st + G::A_BYTES + n * 32 +
                                                                     ((kk ^ ((n >> 3) & 1)) * 16) + fh * 8);
                const float d =
                    fp16_to_f32(*reinterpret_cast<const uint16_t*>(st + G::A_BYTES + G::BQ_BYTES + n * 4 + kk * 2));
                fragm.b[j][0] = q4x8_bf16(nb[0], d);
                fragm.b[j][1] = q4x8_bf16(nb[1], d);
            }
        }
    };
    // acc[i][j][v]: output row i*32 + (l & 31), column j*32 + (v/4)*8 + (l >> 5)*4 + v%4 of the wave tile
    f32x16_t acc[4][JT];
    auto mma = [&](const Frag& fragm) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 2; q++)
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < JT; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fragm.b[j][q], fragm.a[i][q], acc[i][j], 0, 0, 0);
    };
    // The LDS reads of a K half (8 for A, 2 per B column tile) and, after the
    // barrier, this wave's DMA instructions for the stage two steps ahead,
    // spread over the 8 x JT MFMAs of the K half.
    auto interleave = [&]() __attribute__((always_inline)) {
        if constexpr (JT == 4) {
#pragma unroll
            for (int q = 0; q < 16; q++) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 DS read
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMA
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
#pragma unroll
            for (int q = 4; q < 12; q++) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
        }
    };
    auto interleave_dma = [&]() __attribute__((always_inline)) {
        if constexpr (JT == 4 && G::DMA >= 16) {
            static_assert(G::DMA <= 32, "1 or 2 DMA instructions per group");
#pragma unroll
            for (int q = 0; q < G::DMA - 16; q++) {
                __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);   // 2 VMEM (LDS DMA)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 DS read
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMA
            }
#pragma unroll
            for (int q = G::DMA - 16; q < 16; q++) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // 1 VMEM (LDS DMA)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 DS read
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMA
            }
        } else if constexpr (JT == 4) {
#pragma unroll
            for (int q = 0; q < G::DMA; q++) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
#pragma unroll
            for (int q = G::DMA; q < 16; q++) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
        } else {
            static_assert(G::DMA >= 4 && G::DMA <= 12, "one DMA instruction per group");
#pragma unroll
            for (int q = 0; q < 4; q++) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
#pragma unroll
            for (int q = 4; q < G::DMA; q++) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
#pragma unroll
            for (int q = G::DMA; q < 12; q++) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
        }
    };

    // ---- epilogue of one item, staged per wave through the LDS after stage 0
    // while the next item's first stage loads into stage 0; rows go out as
    // 16-byte row-contiguous stores
    auto epilogue = [&](const Item& c) __attribute__((always_inline)) {
        unsigned char* ep = smem + G::STAGE + wave * G::EPI_WAVE;
        const int orow0 = wm * 128;                  // wave tile's first row within the block tile
        if constexpr (PHASE == 0) {
            // activation: 128 rows x WCOLS/2 columns bf16 (gate tile j meets up tile j + JT/2)
            constexpr int JH = JT / 2, LPR = G::WCOLS / 16, RPI = WAVE / LPR;
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < JH; j++)
#pragma unroll
                    for (int g = 0; g < 4; g++) {
                        u32x2_t v;
                        const f32x16_t& ga = acc[i][j];
                        const f32x16_t& ua = acc[i][j + JH];
                        v[0] = cvt_bf16x2(silu_fast(ga[g * 4 + 0]) * ua[g * 4 + 0], silu_fast(ga[g * 4 + 1]) * ua[g * 4 + 1]);
                        v[1] = cvt_bf16x2(silu_fast(ga[g * 4 + 2]) * ua[g * 4 + 2], silu_fast(ga[g * 4 + 3]) * ua[g * 4 + 3]);
                        *reinterpret_cast<u32x2_t*>(ep + (i * 32 + fr) * G::AST + (j * 32 + g * 8 + fh * 4) * 2) = v;
                    }
            wait_lgkm0();
            __builtin_amdgcn_wave_barrier();
            uint16_t* A = (uint16_t*)out;
            const int fc0 = c.nt * (BN / 2) + wn * (G::WCOLS / 2);
#pragma unroll
            for (int it = 0; it < 128 / RPI; it++) {   // LPR lanes x 16 B per row
                const int r = it * RPI + l / LPR, cc = l % LPR;
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ep + r * G::AST + cc * 16);
                const int m = orow0 + r;
                if (m < c.rows) *reinterpret_cast<u32x4_t*>(A + (long)(c.row0 + m) * F + fc0 + cc * 8) = v;
            }
        } else if constexpr (YBF16) {
            // two passes of 64 rows x WCOLS columns bf16
            constexpr int LPR = G::WCOLS / 8, RPI = WAVE / LPR;
            uint16_t* Y = (uint16_t*)out;
            const int h0 = c.nt * BN + wn * G::WCOLS;
#pragma unroll
            for (int half = 0; half < 2; half++) {
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < JT; j++)
#pragma unroll
                        for (int g = 0; g < 4; g++) {
                            const f32x16_t& a = acc[half * 2 + i][j];
                            u32x2_t v;
                            v[0] = cvt_bf16x2(a[g * 4 + 0], a[g * 4 + 1]);
                            v[1] = cvt_bf16x2(a[g * 4 + 2], a[g * 4 + 3]);
                            *reinterpret_cast<u32x2_t*>(ep + (i * 32 + fr) * G::YST + (j * 32 + g * 8 + fh * 4) * 2) = v;
                        }
                wait_lgkm0();
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int it = 0; it < 64 / RPI; it++) {    // LPR lanes x 16 B per row
                    const int r = it * RPI + l / LPR, cc = l % LPR;
                    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ep + r * G::YST + cc * 16);
                    const int m = orow0 + half * 64 + r;
                    if (m < c.rows) *reinterpret_cast<u32x4_t*>(Y + (long)(c.row0 + m) * H + h0 + cc * 8) = v;
                }
                wait_lgkm0();
                __builtin_amdgcn_wave_barrier();
            }
        } else {
            // four passes of 32 rows x WCOLS columns fp32
            constexpr int LPR = G::WCOLS / 4, RPI = WAVE / LPR;
            float* Y = (float*)out;
            const int h0 = c.nt * BN + wn * G::WCOLS;
#pragma unroll
            for (int i = 0; i < 4; i++) {
#pragma unroll
                for (int j = 0; j < JT; j++)
#pragma unroll
                    for (int g = 0; g < 4; g++) {
                        const f32x16_t& a = acc[i][j];
                        *reinterpret_cast<f32x4_t*>(ep + fr * G::FST + (j * 32 + g * 8 + fh * 4) * 4) =
                            f32x4_t{a[g * 4 + 0], a[g * 4 + 1], a[g * 4 + 2], a[g * 4 + 3]};
                    }
                wait_lgkm0();
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int it = 0; it < 32 / RPI; it++) {    // LPR lanes x 16 B per row
                    const int r = it * RPI + l / LPR, cc = l % LPR;
                    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(ep + r * G::FST + cc * 16);
                    const int m = orow0 + i * 32 + r;
                    if (m < c.rows) *reinterpret_cast<f32x4_t*>(Y + (long)(c.row0 + m) * H + h0 + cc * 4) = v;
                }
                wait_lgkm0();
                __builtin_amdgcn_wave_barrier();
            }
        }
    };

    Item cur = item_of(item);
    set_a(cur);
    issue(cur, 0);
    if (nk > 1) issue(cur, 1);
    Frag f0, f1;
    // Two blocks per CU (SB): one fragment set, read just before its MFMAs --
    // the other block's waves cover the LDS latency -- and one barrier per K
    // step, after which the drained stage takes the DMA of step k + 2.
    constexpr bool SB = G::BLOCKS_PER_CU == 2;
    auto step_sb = [&](int k, bool more) __attribute__((always_inline)) {
        const int s = k & 1;
        load_frag(f0, s, 0);
        mma(f0);
        load_frag(f0, s, 1);
        mma(f0);
        wait_vmcnt<0>();           // this wave's DMA of stage k+1 has landed
        wait_lgkm0();              // and its reads of stage k are done
        __builtin_amdgcn_s_barrier();
        if (more) issue(cur, k + 2);
    };
    // One block per CU: the first K half multiplies f0 while the second half
    // of this stage is read into f1; then, once stage k+1 has landed
    // everywhere, the DMA of k+2 goes into the drained stage and f0 is refilled
    // from k+1 under the second half's MFMAs.  The last two steps are peeled so
    // the loop body has no branches.
    auto step = [&](int k, bool more) __attribute__((always_inline)) {
        const int s = k & 1;
        load_frag(f1, s, 1);
        mma(f0);
        interleave();
        wait_vmcnt<0>();           // this wave's DMA of stage k+1 has landed
        wait_lgkm0();              // and its reads of stage k are done
        __builtin_amdgcn_s_barrier();
        if (more) issue(cur, k + 2);   // into the stage just drained
        load_frag(f0, s ^ 1, 0);
        mma(f1);
        if (more) interleave_dma();
        else interleave();
    };
    for (;;) {
        if (nk > 1) wait_vmcnt<G::DMA>();   // this wave's stage 0 has landed (stage 1 may be in flight)
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < JT; j++)
#pragma unroll
                for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;
        if constexpr (SB) {
            int k = 0;
            for (; k + 2 < nk; k++) step_sb(k, true);
            for (; k < nk; k++) step_sb(k, false);
            // the last step's barrier: every wave is done with the LDS
        } else {
            load_frag(f0, 0, 0);
            int k = 0;
            for (; k + 2 < nk; k++) step(k, true);
            if (k + 1 < nk) { step(k, false); k++; }
            load_frag(f1, k & 1, 1);
            mma(f0);
            interleave();
            // every operand of this item is in registers once f1 has arrived: the
            // LDS is free for the next item's first stage and this item's epilogue
            wait_lgkm0();
            __builtin_amdgcn_s_barrier();
        }
        const Item done = cur;
        item += nslot;
        const bool more = item < item_end;
        if (more) {
            cur = item_of(item);
            set_a(cur);
            issue(cur, 0);
        }
        if constexpr (!SB) mma(f1);
        epilogue(done);
        if (!more) break;
        __builtin_amdgcn_s_barrier();       // every wave is done with its staging area (stage 1)
        if (nk > 1) issue(cur, 1);
    }
}

namespace {
// tile shape: 128 rows keep the row padding of small experts at most 127 rows
// per expert.  bf16 weights: 128 x 512 (one block per CU, 160 KB of LDS, the
// fewest LDS fill bytes per flop); int4 weights: 128 x 256 (57 KB of LDS, two
// blocks per CU, so one block's operand conversion runs beside the other's
// MFMAs).
constexpr int GU_BM = 128, GU_BN = 512;
constexpr int DN_BM = 128, DN_BN = 512;
constexpr int Q4_BN = 256;
constexpr int PLAN_BM = 128;
static_assert(GU_BM == PLAN_BM && DN_BM == PLAN_BM, "one tile plan serves both phases");
}  // namespace

// Shapes the tiles cover exactly; the DMA addresses are 32-bit byte offsets
// into the activation rows (T x H) and the intermediate (T*K x F).
bool ffn_gemm_eligible(int T, int K, int H, int F) {
    return H % DN_BN == 0 && H % BK == 0 && (2 * F) % GU_BN == 0 && F % BK == 0 &&
           (size_t)T * H * 2 < ((size_t)1 << 32) && (size_t)T * K * F * 2 < ((size_t)1 << 32);
}

// int4 weights at prefill: the same GEMMs with the nibbles and scales staged in
// LDS (K steps of 64 = two quant blocks); worth it once most experts are
// touched by several rows, below that the streaming kernels win.
bool ffn_gemm_q4_eligible(int T, int K, int E, int H, int F) {
    return ffn_gemm_eligible(T, K, H, F) && (long)T * K >= 4L * E && H % BK == 0 && F % BK == 0;
}

size_t ffn_gemm_q4_workspace_bytes(int T, int K, int E, int H, int F) { return ffn_gemm_workspace_bytes(T, K, E, H, F); }

// Workspace: [A n x F bf16][tiles: (n/BM + min(E,n) + 1) x int4][count]
size_t ffn_gemm_workspace_bytes(int T, int K, int E, int H, int F) {
    (void)H;
    const size_t n = (size_t)T * K;
    const size_t mt = n / PLAN_BM + (size_t)(E < (int)n ? E : (int)n) + 1;
    return (n * F * 2 + 255) / 256 * 256 + (mt * 16 + 255) / 256 * 256 + 256;
}

template <int BM, int BN, int PHASE, int YBF16, int WQ>
static hipError_t launch_one(int items, hipStream_t st, const uint16_t* src, const void* w0, const void* w1,
                             const uint16_t* s0, const uint16_t* s1, const int4* tiles, const int32_t* count,
                             const int32_t* perm, int K, int H, int F, void* out) {
    auto kern = k_gemm<BM, BN, PHASE, YBF16, WQ>;
    const int lds = Geo<BM, BN, WQ>::LDS;
    static LdsLimit lim;          // this instantiation's LDS limit, raised once per device
    hipError_t e = lim.ensure((const void*)kern, lds);
    if (e != hipSuccess) return e;
    // persistent: as many blocks as the CUs hold at once (one or two per CU,
    // by LDS), a multiple of the 8 XCDs
    int ncu = 0;
    e = current_device_cus(&ncu);
    if (e != hipSuccess) return e;
    const int slots = ncu * Geo<BM, BN, WQ>::BLOCKS_PER_CU;
    const int cap = slots / 8 * 8 > 8 ? slots / 8 * 8 : 8;
    const int grid = (items + 7) / 8 * 8 < cap ? (items + 7) / 8 * 8 : cap;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, src, w0, w1, s0, s1, tiles, count, perm, K, H, F, out);
    return hipSuccess;
}

// plan + gate/up + down; WQ 1: int4 weights with their scales
template <int WQ>
static hipError_t gemm_phases(const void* x, const void* wg, const void* wu, const void* wd, const void* sg,
                              const void* su, const void* sd, const int32_t* offsets, const int32_t* perm, int T,
                              int K, int H, int F, int E, void* y, int y_bf16, void* ws, hipStream_t st) {
    const size_t n = (size_t)T * K;
    const size_t mt = n / PLAN_BM + (size_t)(E < (int)n ? E : (int)n) + 1;
    char* base = (char*)ws;
    uint16_t* abuf = (uint16_t*)base;
    int4* tiles = (int4*)(base + (n * F * 2 + 255) / 256 * 256);
    int32_t* count = (int32_t*)((char*)tiles + (mt * 16 + 255) / 256 * 256);
    hipLaunchKernelGGL(k_gemm_plan, dim3(1), dim3(256), 0, st, offsets, E, PLAN_BM, tiles, count);
    constexpr int BNG = WQ ? Q4_BN : GU_BN, BND = WQ ? Q4_BN : DN_BN;
    const int items_g = (int)mt * ((2 * F) / BNG), items_d = (int)mt * (H / BND);
    const uint16_t *s_g = (const uint16_t*)sg, *s_u = (const uint16_t*)su, *s_d = (const uint16_t*)sd;
    hipError_t e = launch_one<GU_BM, BNG, 0, 1, WQ>(items_g, st, (const uint16_t*)x, wg, wu, s_g, s_u, tiles, count,
                                                    perm, K, H, F, abuf);
    if (e != hipSuccess) return e;
    if (y_bf16)
        e = launch_one<DN_BM, BND, 1, 1, WQ>(items_d, st, abuf, wd, nullptr, s_d, nullptr, tiles, count, perm, K, H, F, y);
    else
        e = launch_one<DN_BM, BND, 1, 0, WQ>(items_d, st, abuf, wd, nullptr, s_d, nullptr, tiles, count, perm, K, H, F, y);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

hipError_t launch_ffn_gemm(const void* x, const void* wg, const void* wu, const void* wd, const int32_t* offsets,
                           const int32_t* perm, int T, int K, int H, int F, int E, void* y, int y_bf16, void* ws,
                           hipStream_t st) {
    return gemm_phases<0>(x, wg, wu, wd, nullptr, nullptr, nullptr, offsets, perm, T, K, H, F, E, y, y_bf16, ws, st);
}

hipError_t launch_ffn_gemm_q4(const void* x, const void* wg, const void* wu, const void* wd, const void* sg,
                              const void* su, const void* sd, const int32_t* offsets, const int32_t* perm, int T,
                              int K, int H, int F, int E, void* y, int y_bf16, void* ws, hipStream_t st) {
    return gemm_phases<1>(x, wg, wu, wd, sg, su, sd, offsets, perm, T, K, H, F, E, y, y_bf16, ws, st);
}
