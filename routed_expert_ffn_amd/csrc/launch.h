// launch.h -- internal host-side launchers of libmoe's kernels (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// route.hip
hipError_t launch_logits_exact(const void* x, int x_bf16, const float* wr, const float* bias, int T, int H, int E,
                               float* logits, hipStream_t st);
bool logits_fast_eligible(int T, int H, int E);
size_t logits_fast_planes_bytes(int H, int E);
// the estimate (three-plane bf16 split of the router, then the MFMA GEMM); the
// split kernel also stores each router row's squared norm in wnorm2 [E] and
// clears *rc_count, the recheck queue's counter
hipError_t launch_logits_fast(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                              float* logits, uint16_t* planes, float* wnorm2, int32_t* rc_count, hipStream_t st);
// selection; with estimates (exact == 0, bf16 x, wnorm2 from the split) tokens
// whose leading gaps fall within their margin (tau, scaled up with |x_t| and
// the largest router row norm) are queued in rc_list / rc_count and re-decided
// on exact logits by a second kernel
hipError_t launch_route_select(const float* logits, int T, int E, int K, float tau, int exact, const void* x,
                               int x_bf16, const float* wr, const float* bias, int H, const float* wnorm2,
                               int32_t* idx, float* w, int32_t* flags, int2* rc_list, int32_t* rc_count,
                               hipStream_t st);
// A few tokens on exact logits: selection and grouping in one launch (route.hip)
bool route_group_fused_eligible(int T, int K, int E);
hipError_t launch_route_select_group(const float* logits, int T, int E, int K, int32_t* idx, float* w,
                                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, hipStream_t st);

// permute.hip
constexpr int PERM_CHUNK = 1024;   // slots per grouping block
hipError_t launch_permute(const int32_t* idx, int n, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                          int32_t* inv, int32_t* chunk_buf, hipStream_t st);

// ffn.hip
size_t ffn_workspace_bytes(int T, int K, int E, int H, int F, int x_dtype, int w_dtype);
hipError_t launch_ffn(const void* x, int x_dtype, int w_dtype, const void* wg, const void* wu, const void* wd,
                      const void* sg, const void* su, const void* sd, const int32_t* offsets, const int32_t* perm,
                      int T, int K, int H, int F, int E, void* y, int y_dtype, void* ws, hipStream_t st);

// ffn_small.hip (every expert has <= 16 rows)
bool ffn_small_eligible(int T, int H, int F);
size_t ffn_small_workspace_bytes(int T, int K, int E, int H, int F);
hipError_t launch_ffn_small(const void* x, int w_dtype, const void* wg, const void* wu, const void* wd,
                            const void* sg, const void* su, const void* sd, const int32_t* offsets,
                            const int32_t* perm, int T, int K, int H, int F, int E, void* y, int y_bf16, void* ws,
                            hipStream_t st);

// ffn_stream.hip (bf16, T <= 8; uses the first T*K*F*2 bytes of the small-path workspace)
bool ffn_stream_eligible(int T, int K, int E, int H, int F);
size_t ffn_stream_workspace_bytes(int T, int K, int F);
bool ffn_stream_q4_eligible(int T, int K, int E, int H, int F);
hipError_t launch_ffn_stream_q4(const void* x, const void* wg, const void* wu, const void* wd, const void* sg,
                                const void* su, const void* sd, const int32_t* offsets, const int32_t* perm, int T,
                                int K, int H, int F, int E, void* y, int y_bf16, void* ws, hipStream_t st,
                                int bits = 4);   // int4, int3 or int2 blocks
hipError_t launch_ffn_stream(const void* x, const void* wg, const void* wu, const void* wd, const int32_t* offsets,
                             const int32_t* perm, int T, int K, int H, int F, int E, void* y, int y_bf16, void* ws,
                             hipStream_t st);

// ffn_gemm.hip (many rows per expert; bf16 weights)
bool ffn_gemm_eligible(int T, int K, int H, int F);
size_t ffn_gemm_workspace_bytes(int T, int K, int E, int H, int F);
bool ffn_gemm_q4_eligible(int T, int K, int E, int H, int F);
size_t ffn_gemm_q4_workspace_bytes(int T, int K, int E, int H, int F);
hipError_t launch_ffn_gemm_q4(const void* x, const void* wg, const void* wu, const void* wd, const void* sg,
                              const void* su, const void* sd, const int32_t* offsets, const int32_t* perm, int T,
                              int K, int H, int F, int E, void* y, int y_bf16, void* ws, hipStream_t st);
hipError_t launch_ffn_gemm(const void* x, const void* wg, const void* wu, const void* wd, const int32_t* offsets,
                           const int32_t* perm, int T, int K, int H, int F, int E, void* y, int y_bf16, void* ws,
                           hipStream_t st);

// combine.hip
hipError_t launch_combine(const void* y, int y_bf16, const int32_t* inv, const float* w, const void* res, int T,
                          int K, int H, void* out, int out_bf16, hipStream_t st);
constexpr int STEER_MAX_H = 8192;   // the steered combine keeps one token row per block in registers
hipError_t launch_combine_steer(const void* y, int y_bf16, const int32_t* inv, const float* w, const void* res,
                                const float* sv, int T, int K, int H, void* out, int out_bf16, hipStream_t st);

// freq.hip
hipError_t launch_freq(const float* logits, int L, int64_t T, int E, int K, unsigned long long* counts,
                       int accumulate, int keep, int32_t* rank_of, int32_t* keep_map, hipStream_t st);

// verify.hip: one whole layer for a few tokens (logits, routing + grouping +
// gate/up, down + combine; + the projection of a steered layer)
bool verify_layer_eligible(int T, int H, int E, int K, int F, int x_dtype, int w_dtype);
size_t verify_layer_workspace_bytes(int T, int H, int E, int K, int F);
hipError_t launch_verify_layer(const void* x, const float* wr, const float* bias, int w_dtype, const void* wg,
                               const void* wu, const void* wd, const void* sg, const void* su, const void* sd, int T,
                               int H, int E, int K, int F, const void* residual, const float* steer_v, void* out,
                               int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                               void* ws, hipStream_t st);
