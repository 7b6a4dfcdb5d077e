/*
 * moe.h -- C ABI of the routed-expert (sparse mixture-of-experts) layer for
 * AMD MI355X (gfx950).  Library: routed_expert_ffn_amd/_lib/libmoe.so.
 *
 * The operation, per the pages this library follows:
 *   "Strata Coder 编程模型深度剖析：RCO 专家剪枝砍掉一半专家却保留 91% 编程能力",
 *     §1 "先搞懂 Strata": a 48-layer model of 512 experts per layer in which the
 *        router picks 10 experts for every token;
 *     §3 "RCO 专家剪枝是怎么砍一半而不伤脑的": every expert has gate, up and down
 *        matrices; pruning counts which experts the routing selects on
 *        calibration data and keeps the 256 most-selected of each layer, with one
 *        keep decision for all three matrices, the kept experts listed in their
 *        original order.
 *   Coder benchmark write-up (kwkr.cn), "测试环境与运行配置": still 10 active
 *     experts per token after pruning; prefill in chunks of up to 8,192 tokens;
 *     speculative verify of 4 drafted tokens plus one.
 * The expert is the SwiGLU y = Wd (silu(Wg x) * (Wu x)); routing weights are the
 * softmax over the K selected logits; ties go to the lower expert id.
 *
 * Conventions for every call:
 *   - All tensors are row-major and contiguous.  Every pointer argument is a
 *     DEVICE pointer owned by the caller (the library allocates nothing and
 *     keeps no per-call state); only sizes and enums are host values.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work on it: no host synchronisation, no device->host copies.
 *   - Arguments are checked on the host before anything is enqueued; on any
 *     error the outputs are untouched and nothing is launched.
 *       MOE_ERR_INVALID_ARG  null required pointer, non-positive size, K > E,
 *                            counts that overflow int32, unknown dtype;
 *       MOE_ERR_UNSUPPORTED  a valid request the library does not implement
 *                            (listed per call), or a pointer not aligned to 16 B;
 *       MOE_ERR_WORKSPACE    workspace smaller than the matching *_workspace_size;
 *       MOE_ERR_HIP          a kernel launch reported an error.
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - Calls are re-entrant; calls on different streams may run concurrently
 *     if their buffers do not overlap.
 *   - bf16 tensors are passed as 16-bit bit patterns; int4 weights as packed
 *     bytes (see MOE_INT4_B32).
 */
#ifndef ROUTED_EXPERT_FFN_MOE_H
#define ROUTED_EXPERT_FFN_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE = 3,
    MOE_ERR_HIP = 4
} moe_status;

typedef enum {
    MOE_F32 = 0,
    MOE_BF16 = 1,
    /* Symmetric int4 in blocks of 32 consecutive elements along the input
     * (reduction) dimension of each out x in weight row: the element is
     * d * (nibble - 8), d the block's IEEE fp16 scale; byte j of a row holds
     * element 2j in its low nibble and 2j+1 in its high nibble. */
    MOE_INT4_B32 = 2,
    /* Lower-bit variants of the same block scheme (32 consecutive elements
     * along the input dimension share an fp16 scale d): the element is
     * d * (u - 2) (int2) or d * (u - 4) (int3), u its stored level.  A row
     * of n elements is n/4 bytes of the low two bits of every level, as
     * 32-bit little-endian words of 16 elements (element 4k + j of a word in
     * byte j, bits 2k and 2k+1); an int3 row continues with n/8 bytes of the
     * third bits, as words of 32 elements (element 16g + 4k + j of a word in
     * byte j, bit 4g + k). */
    MOE_INT2_B32 = 3,
    MOE_INT3_B32 = 4
} moe_dtype;

typedef void* moe_stream; /* hipStream_t */

/* One layer's expert weights, E experts of width F over hidden size H.
 *   F32 / BF16:  w_gate, w_up [E][F][H];  w_down [E][H][F];  s_* must be NULL.
 *   INT4_B32:    w_gate, w_up [E][F][H/2] bytes, s_gate, s_up [E][F][H/32] fp16;
 *                w_down [E][H][F/2] bytes, s_down [E][H][F/32] fp16.
 *   INT3_B32 / INT2_B32: as INT4_B32 with rows of 3n/8 / n/4 bytes. */
typedef struct {
    int32_t dtype; /* moe_dtype */
    const void* w_gate;
    const void* w_up;
    const void* w_down;
    const void* s_gate;
    const void* s_up;
    const void* s_down;
} moe_expert_weights;

int moe_abi_version(void);
const char* moe_status_string(moe_status s);

/* ---------------------------------------------------------------- routing
 * Router projection, selection and weights (page 1 §1: each token is routed
 * to K of the E experts).
 *   x          [T][H] activations, x_dtype MOE_F32 or MOE_BF16.
 *   w_router   [E][H] fp32.
 *   bias       [E] fp32 added to every logit (a router offset), or NULL.
 *   topk_idx   [T][K] int32 out: the K largest logits, in descending order,
 *              ties to the lower expert id.
 *   topk_w     [T][K] fp32 out: exp(l_k - l_0) / sum_j exp(l_j - l_0) over the
 *              K selected, fp32, the sum taken in rank order j = 0, 1, ...
 *   logits_out [T][E] fp32 out, or NULL.
 * Logits are fp32(S + 0) then + bias in fp32, S the fp64 sum of the exact
 * products x*w taken in wave-64 order (64 strided partial sums, then a pairwise
 * tree 32,16,...,1); the selection is exact with respect to these values.  A
 * faster fp32 estimate is used where every gap among the leading K+1 logits
 * clears a safety margin; other tokens are re-decided on the exact values.
 * The estimate (bf16 activations, T >= 64, logits_out NULL) is exact in every
 * product and rounds only in its fp32 accumulation, so the selection stays
 * exact while that error stays below half the margin.  The error grows in
 * proportion to |x_t| and the router rows' norms, and so does the margin:
 * token t's is max(2^-12, 2^-24 sqrt(H) |x_t|_2 max_e |w_e|_2).  For
 * activations ~N(0,1) and router weights ~N(0,0.02) at H = 2048 the margin is
 * 2^-12 and the measured error below 1e-6, over 100 times smaller than half
 * the margin, and scaling x or w_router keeps that ratio.  This is a measured
 * margin, not a proven bound: passing logits_out selects the exact logits for
 * every token.
 * Unsupported: K > 32, E > 4096, H % 8 != 0.  NaN logits give unspecified
 * selections. */
size_t moe_route_workspace_size(int32_t T, int32_t H, int32_t E, int32_t K, int32_t x_dtype);
moe_status moe_route(const void* x, int32_t x_dtype, const float* w_router, const float* bias,
                     int32_t T, int32_t H, int32_t E, int32_t K,
                     int32_t* topk_idx, float* topk_w, float* logits_out,
                     void* workspace, size_t ws_bytes, moe_stream stream);

/* ---------------------------------------------------------------- grouping
 * Token->expert grouping (the kwkr.cn Coder write-up, "为什么 Coder 快" part 2:
 * work is done per expert, for the experts a batch of tokens actually hits;
 * grouping the routed slots by expert lets each touched expert's weights be
 * read once for all of its rows): a stable counting sort of the flat slots
 * s = t*K + k by expert id.
 *   counts   [E]     int32 out: slots per expert.
 *   offsets  [E+1]   int32 out: exclusive scan of counts (offsets[E] = T*K).
 *   perm     [T*K]   int32 out: perm[p] = slot at permuted position p; within an
 *                    expert's segment slots ascend.
 *   inv_perm [T*K]   int32 out: inv_perm[perm[p]] = p.
 * Unsupported: E > 4096. */
size_t moe_permute_workspace_size(int32_t T, int32_t K, int32_t E);
moe_status moe_permute(const int32_t* topk_idx, int32_t T, int32_t K, int32_t E,
                       int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                       void* workspace, size_t ws_bytes, moe_stream stream);

/* ---------------------------------------------------------------- routing + grouping
 * moe_route followed by moe_permute on its topk_idx, with the same results
 * (no logits_out).  For a few tokens on the exact path (T <= 16, T*K <= 1024,
 * T < 64 or fp32 activations) the selection and the grouping run in one
 * launch after the logits; otherwise the two calls run as they are.
 * Workspace: moe_route_group_workspace_size(T, H, E, K, x_dtype) bytes. */
size_t moe_route_group_workspace_size(int32_t T, int32_t H, int32_t E, int32_t K, int32_t x_dtype);
moe_status moe_route_group(const void* x, int32_t x_dtype, const float* w_router, const float* bias,
                           int32_t T, int32_t H, int32_t E, int32_t K,
                           int32_t* topk_idx, float* topk_w,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                           void* workspace, size_t ws_bytes, moe_stream stream);

/* ---------------------------------------------------------------- routing + grouping, no allocation
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_route_group with the same arguments and results, minus the workspace.
 * Its scratch is a fixed 32 MiB device array inside the library, one copy per
 * GPU, made when the library is loaded on that GPU and held until the process
 * ends; its address is looked up once per device, on the first call made with
 * that device current (the stream must belong to the current device).  This
 * call allocates nothing and calls no allocating routine.
 * Returns MOE_ERR_WORKSPACE, with nothing launched, when
 * moe_route_group_workspace_size(T, H, E, K, x_dtype) exceeds 32 MiB (e.g.
 * E = 512, H = 2048, K = 10: up to 13,106 tokens); MOE_ERR_HIP if the device
 * array cannot be found.  Every call on one GPU uses that GPU's one array, so
 * calls that overlap in time on one GPU (different streams, or host threads
 * without ordering) race and give undefined results; calls on one stream are
 * ordered and safe.  The array keeps the last call's contents; everything a
 * call needs cleared is cleared by its own kernels. */
moe_status moe_route_group_noalloc(const void* x, int32_t x_dtype, const float* w_router, const float* bias,
                                   int32_t T, int32_t H, int32_t E, int32_t K,
                                   int32_t* topk_idx, float* topk_w,
                                   int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                   moe_stream stream);

/* ---------------------------------------------------------------- experts
 * Grouped SwiGLU expert FFN (page 1 §3: gate, up and down per expert).  For
 * every permuted row p in expert e's segment [offsets[e], offsets[e+1]), with
 * token t = perm[p] / K:
 *     a = silu(Wg[e] x[t]) * (Wu[e] x[t])      (rounded to bf16 if x is bf16)
 *     y_perm[p] = Wd[e] a                      (fp32 accumulation)
 *   x        [T][H] activations, MOE_F32 or MOE_BF16.
 *   y_perm   [T*K][H] out, y_dtype MOE_F32 or MOE_BF16.
 * Built combinations: (x F32, weights F32, y F32), (x BF16, weights BF16,
 * y BF16 or F32), (x BF16, weights INT4_B32, y BF16 or F32), and for the
 * verify and decode steps (x BF16, weights INT3_B32 or INT2_B32, y BF16 or
 * F32) with T <= 8, T*K <= 59, H = 2048, F = 512 (the lower-bit expert
 * variant; other shapes return MOE_ERR_UNSUPPORTED; moe_layer takes these
 * weights up to T*K = 128).
 * Unsupported: H or F not a multiple of 64. */
size_t moe_ffn_workspace_size(int32_t T, int32_t K, int32_t E, int32_t H, int32_t F, int32_t x_dtype,
                              int32_t w_dtype);
moe_status moe_ffn(const void* x, int32_t x_dtype, const moe_expert_weights* w,
                   const int32_t* offsets, const int32_t* perm,
                   int32_t T, int32_t K, int32_t H, int32_t F, int32_t E,
                   void* y_perm, int32_t y_dtype,
                   void* workspace, size_t ws_bytes, moe_stream stream);

/* ---------------------------------------------------------------- combine
 * The layer's output (page 1 §1: 10 experts work on every token, so a token's
 * output is its selected experts' outputs weighted by the routing weights;
 * the stacked layers add it to the residual stream):
 *   out[t] = cast( sum_k topk_w[t][k] * y_perm[inv_perm[t*K+k]] + residual[t] )
 * accumulated in fp32 in k order (a gather: deterministic), one final
 * rounding to out_dtype (bf16: nearest-even).  residual [T][H] in out_dtype, or
 * NULL.  out may alias residual (in-place residual update). */
moe_status moe_combine(const void* y_perm, int32_t y_dtype, const int32_t* inv_perm,
                       const float* topk_w, const void* residual,
                       int32_t T, int32_t K, int32_t H, void* out, int32_t out_dtype,
                       moe_stream stream);

/* ---------------------------------------------------------------- steered combine
 * moe_combine followed by the steering projection of a steered layer (the
 * kwkr.cn Coder write-up, "实验加速投影在 Coder 上的表现": one unit direction
 * per steered layer, whose component is removed from the stream after it):
 *     h[t]   = sum_k topk_w[t][k] * y_perm[inv_perm[t*K+k]] + residual[t]
 *     out[t] = cast( h[t] - (h[t] . v) v )
 * h, the dot product and the subtraction in fp32 (the dot summed in a fixed
 * order: the result does not vary from run to run), one rounding at the end.
 *   steer_v  [H] fp32, device, 16-byte aligned; used as given (the caller
 *            passes a unit vector; it is not renormalised here).
 * Other arguments, aliasing and dtypes as for moe_combine; layers that are
 * not steered call moe_combine.  Unsupported: H > 8192 or not a multiple of 8. */
moe_status moe_combine_steer(const void* y_perm, int32_t y_dtype, const int32_t* inv_perm,
                             const float* topk_w, const void* residual, const float* steer_v,
                             int32_t T, int32_t K, int32_t H, void* out, int32_t out_dtype,
                             moe_stream stream);

/* ---------------------------------------------------------------- one whole layer
 * The MoE layer in one call (page 1 §1: every token routed to K experts whose
 * outputs are combined with the routing weights; §3: gate, up and down per
 * expert): moe_route_group, moe_ffn and moe_combine (moe_combine_steer when
 * steer_v is given) with the same arguments and meanings, and
 *     out[t] = cast( sum_k topk_w[t][k] * FFN_{topk_idx[t][k]}(x[t]) + residual[t] )
 * in x's dtype.  The routing and grouping outputs are produced as those calls
 * produce them.  residual [T][H] (x's dtype) or NULL; out [T][H] may alias x
 * and residual (an in-place residual stream).  steer_v [H] fp32 or NULL.
 * For a few tokens (T <= 8, T*K <= 128, H = 2048, F = 512, E <= 1024, bf16
 * activations, bf16 or block-quantised weights, 16-byte aligned tensors) the
 * layer runs as three launches: the exact logits; the selection and grouping
 * (redone by every block of the gate/up launch) with the gate/up projections;
 * the down projections with the combine, the expert outputs kept in fp32
 * (no y_perm).  Other shapes run the three calls as they are (y_perm in x's
 * dtype).  Errors as for those calls; workspace:
 * moe_layer_workspace_size(T, H, E, K, F, x_dtype, w_dtype) bytes. */
size_t moe_layer_workspace_size(int32_t T, int32_t H, int32_t E, int32_t K, int32_t F, int32_t x_dtype,
                                int32_t w_dtype);
moe_status moe_layer(const void* x, int32_t x_dtype, const float* w_router, const float* bias,
                     const moe_expert_weights* w, int32_t T, int32_t H, int32_t E, int32_t K, int32_t F,
                     const void* residual, const float* steer_v, void* out,
                     int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                     int32_t* perm, int32_t* inv_perm, void* workspace, size_t ws_bytes, moe_stream stream);

/* ---------------------------------------------------------------- pruning statistic
 * Per-(layer, expert) selection counts over given router logits (page 1 §3:
 * routing counted on calibration data, the most-selected kept per layer, kept
 * experts listed in original order).
 *   logits   [L][T][E] fp32; each row's top-K follows moe_route's rule.
 *   counts   [L][E] int64: overwritten (accumulate = 0) or added to
 *            (accumulate = 1, chunked calibration).
 *   keep     0: counts only.  Else rank_of [L][E] int32 = position of e in
 *            (count descending, id ascending) order, and keep_map [L][keep]
 *            int32 = the ids with rank_of < keep, ascending.
 * Unsupported: K > 32, E > 4096. */
moe_status moe_expert_freq(const float* logits, int32_t L, int64_t T, int32_t E, int32_t K,
                           int64_t* counts, int32_t accumulate, int32_t keep,
                           int32_t* rank_of, int32_t* keep_map, moe_stream stream);

/* ---------------------------------------------------------------- expert profile
 * The global ranking an engine uses to choose which experts stay in its fast
 * memory (page 1 §3; the kwkr.cn Coder write-up, "专家配置文件：48 x 256 的全量
 * 排名": a ranking of every (layer, expert) pair, written as an STRP file,
 * mapped to the pruned model through its keep list, and checked by the share
 * of routed reads that hit the first S ranked pairs).
 *
 * moe_profile_rank (device): counts [L][E] int64 (e.g. moe_expert_freq's) ->
 *   rank  [L][E] int32: each pair's position in (count descending, flat index
 *         layer*E + expert ascending) order;
 *   pairs [L*E][2] uint16 (4-byte aligned): (layer, expert) in rank order.
 *   Workspace: moe_profile_workspace_size(L, E) bytes.  Unsupported: E > 4096.
 * moe_profile_hits (device): trace [L][T][K] int32 expert ids (one routing per
 *   layer, e.g. moe_route's topk_idx), rank as above -> *hits (uint64, device)
 *   = the number of trace entries whose pair has rank < S (ids outside [0, E)
 *   never hit).  The hit rate is *hits / (L*T*K).
 * STRP v1, host memory, little-endian: "STRP", uint32 version (1), layers,
 *   experts, ranked pairs n, entries (= layers*experts); n pairs of uint16
 *   (layer, expert) in rank order; an int16 [layers][experts] table of each
 *   pair's rank, -1 if unranked.  n <= 32767 (int16 ranks).
 *   moe_strp_write fills out[moe_strp_size(L, E, n)] from host pairs [n][2]
 *   (each pair in range and ranked once, else MOE_ERR_INVALID_ARG);
 *   moe_strp_read checks the header and sizes, sets *L, *E, *n_ranked and, when
 *   given room (pairs_capacity >= n pairs, inverse_capacity >= L*E entries),
 *   copies the pairs and the table (NULL skips either).
 * moe_profile_remap (host): ranked pairs of an E_old-expert profile -> the
 *   pruned model's: expert e of layer l becomes its position in keep_map[l]
 *   ([L][keep] int32, ascending ids, e.g. moe_expert_freq's keep_map); pairs
 *   of pruned experts are dropped and the order is kept; *n_out = survivors.
 *   out holds up to n pairs. */
size_t moe_profile_workspace_size(int32_t L, int32_t E);
moe_status moe_profile_rank(const int64_t* counts, int32_t L, int32_t E, int32_t* rank, uint16_t* pairs,
                            void* workspace, size_t ws_bytes, moe_stream stream);
moe_status moe_profile_hits(const int32_t* trace, int32_t L, int64_t T, int32_t K, const int32_t* rank,
                            int32_t E, int64_t S, uint64_t* hits, moe_stream stream);
size_t moe_strp_size(int32_t L, int32_t E, int32_t n_ranked);
moe_status moe_strp_write(const uint16_t* pairs, int32_t n_ranked, int32_t L, int32_t E, void* out,
                          size_t out_bytes);
moe_status moe_strp_read(const void* buf, size_t bytes, int32_t* L, int32_t* E, int32_t* n_ranked,
                         uint16_t* pairs, int32_t pairs_capacity, int16_t* inverse, int64_t inverse_capacity);
moe_status moe_profile_remap(const uint16_t* pairs, int32_t n, int32_t L, int32_t E_old, const int32_t* keep_map,
                             int32_t keep, uint16_t* out, int32_t* n_out);

#ifdef __cplusplus
}
#endif
#endif /* ROUTED_EXPERT_FFN_MOE_H */
