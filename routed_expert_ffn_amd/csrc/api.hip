// api.hip -- the C ABI of libmoe (declared in include/moe.h): argument
// checks, workspace sizing, path selection and kernel launches.  Nothing here
// allocates memory or synchronises; every call only enqueues on `stream`.
#include "../../include/moe.h"
#include "common.h"
#include "launch.h"

#include <mutex>

namespace {

constexpr int MAX_E = 4096;
constexpr int MAX_K = 32;
constexpr int FAST_ROUTE_MIN_T = 64;      // below this the exact logits are cheap enough
constexpr float ROUTE_TAU = 1.0f / 4096;  // safety margin of the fp32 logit estimate

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }
size_t round256(size_t b) { return (b + 255) / 256 * 256; }
hipStream_t S(moe_stream s) { return (hipStream_t)s; }
moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool fast_route_eligible(int T, int H, int E, int x_dtype, const void* x, const float* w_router,
                         const float* logits_out) {
    return x_dtype == MOE_BF16 && T >= FAST_ROUTE_MIN_T && logits_fast_eligible(T, H, E) && logits_out == nullptr &&
           aligned16(x) && aligned16(w_router);
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported request";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

// Workspace: [T][E] fp32 logits, [T] int32 flags (1 = token re-decided on
// exact logits), the recheck queue (a counter, then [T] (token, cut) pairs),
// and (bf16 activations, many tokens) the router weight split into three
// bf16 planes for the estimate.
namespace {
struct RouteWs {
    size_t flags, count, list, planes, wnorm, total;
};
RouteWs route_ws_layout(int T, int H, int E, int x_dtype) {
    RouteWs w;
    w.flags = round256((size_t)T * E * sizeof(float));
    w.count = w.flags + round256((size_t)T * sizeof(int32_t));
    w.list = w.count + 256;
    w.planes = w.list + round256((size_t)T * 8);
    w.wnorm = w.planes;
    w.total = w.planes;
    if (x_dtype == MOE_BF16 && T >= FAST_ROUTE_MIN_T && logits_fast_eligible(T, H, E)) {
        w.wnorm = w.planes + round256(logits_fast_planes_bytes(H, E));
        w.total = w.wnorm + round256((size_t)E * sizeof(float));
    }
    return w;
}
}  // namespace

size_t moe_route_workspace_size(int32_t T, int32_t H, int32_t E, int32_t K, int32_t x_dtype) {
    (void)K;
    if (T < 0 || E <= 0 || H <= 0) return 0;
    return route_ws_layout(T, H, E, x_dtype).total;
}

}  // extern "C"

namespace {
moe_status route_check(const void* x, int32_t x_dtype, const float* w_router, int32_t T, int32_t H, int32_t E,
                       int32_t K, const int32_t* topk_idx, const float* topk_w) {
    if (T < 0 || H <= 0 || E <= 0 || K <= 0 || K > E) return MOE_ERR_INVALID_ARG;
    if (!w_router || (T > 0 && (!x || !topk_idx || !topk_w))) return MOE_ERR_INVALID_ARG;
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if ((int64_t)T * K > INT32_MAX || (int64_t)T * E > ((int64_t)1 << 40)) return MOE_ERR_INVALID_ARG;
    if (K > MAX_K || E > MAX_E || H % 8 != 0) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_route(const void* x, int32_t x_dtype, const float* w_router, const float* bias, int32_t T, int32_t H,
                     int32_t E, int32_t K, int32_t* topk_idx, float* topk_w, float* logits_out, void* workspace,
                     size_t ws_bytes, moe_stream stream) {
    const moe_status chk = route_check(x, x_dtype, w_router, T, H, E, K, topk_idx, topk_w);
    if (chk != MOE_OK) return chk;
    const size_t need = moe_route_workspace_size(T, H, E, K, x_dtype);
    if (!workspace || ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (T == 0) return MOE_OK;
    hipStream_t st = S(stream);
    const RouteWs L = route_ws_layout(T, H, E, x_dtype);
    char* wb = (char*)workspace;
    float* lg = (float*)wb;
    int32_t* flags = (int32_t*)(wb + L.flags);
    int32_t* rc_count = (int32_t*)(wb + L.count);
    int2* rc_list = (int2*)(wb + L.list);
    const int xb = x_dtype == MOE_BF16;
    hipError_t err;
    if (fast_route_eligible(T, H, E, x_dtype, x, w_router, logits_out)) {
        float* wnorm2 = (float*)(wb + L.wnorm);
        err = launch_logits_fast((const uint16_t*)x, w_router, bias, T, H, E, lg, (uint16_t*)(wb + L.planes), wnorm2,
                                 rc_count, st);
        if (err != hipSuccess) return MOE_ERR_HIP;
        err = launch_route_select(lg, T, E, K, ROUTE_TAU, 0, x, xb, w_router, bias, H, wnorm2, topk_idx, topk_w,
                                  flags, rc_list, rc_count, st);
    } else {
        float* dst = logits_out ? logits_out : lg;
        err = launch_logits_exact(x, xb, w_router, bias, T, H, E, dst, st);
        if (err != hipSuccess) return MOE_ERR_HIP;
        err = launch_route_select(dst, T, E, K, 0.f, 1, x, xb, w_router, bias, H, nullptr, topk_idx, topk_w, flags, rc_list,
                                  rc_count, st);
    }
    return hip_status(err);
}

size_t moe_permute_workspace_size(int32_t T, int32_t K, int32_t E) {
    if (T < 0 || K <= 0 || E <= 0) return 0;
    const int64_t n = (int64_t)T * K;
    if (n <= PERM_CHUNK) return 256;
    const int64_t chunks = (n + PERM_CHUNK - 1) / PERM_CHUNK;
    return round256((size_t)chunks * E * sizeof(int32_t));
}

moe_status moe_permute(const int32_t* topk_idx, int32_t T, int32_t K, int32_t E, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* inv_perm, void* workspace, size_t ws_bytes, moe_stream stream) {
    if (T < 0 || K <= 0 || E <= 0 || (int64_t)T * K > INT32_MAX) return MOE_ERR_INVALID_ARG;
    if (!counts || !offsets || (T > 0 && (!topk_idx || !perm || !inv_perm))) return MOE_ERR_INVALID_ARG;
    if (E > MAX_E) return MOE_ERR_UNSUPPORTED;
    const size_t need = moe_permute_workspace_size(T, K, E);
    if (!workspace || ws_bytes < need) return MOE_ERR_WORKSPACE;
    return hip_status(launch_permute(topk_idx, T * K, E, counts, offsets, perm, inv_perm, (int32_t*)workspace,
                                     S(stream)));
}

size_t moe_route_group_workspace_size(int32_t T, int32_t H, int32_t E, int32_t K, int32_t x_dtype) {
    if (T < 0 || E <= 0 || H <= 0 || K <= 0) return 0;
    return round256(moe_route_workspace_size(T, H, E, K, x_dtype)) + moe_permute_workspace_size(T, K, E);
}

}  // extern "C"

namespace {
// moe_route_group's body on a given workspace (the caller's, or the per-GPU
// scratch of moe_route_group_noalloc).
moe_status route_group_on(const void* x, int32_t x_dtype, const float* w_router, const float* bias, int32_t T,
                          int32_t H, int32_t E, int32_t K, int32_t* topk_idx, float* topk_w, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* workspace, size_t ws_bytes,
                          moe_stream stream) {
    const moe_status chk = route_check(x, x_dtype, w_router, T, H, E, K, topk_idx, topk_w);
    if (chk != MOE_OK) return chk;
    if (!counts || !offsets || (T > 0 && (!perm || !inv_perm))) return MOE_ERR_INVALID_ARG;
    const size_t rws = round256(moe_route_workspace_size(T, H, E, K, x_dtype));
    if (!workspace || ws_bytes < moe_route_group_workspace_size(T, H, E, K, x_dtype)) return MOE_ERR_WORKSPACE;
    if (T > 0 && !fast_route_eligible(T, H, E, x_dtype, x, w_router, nullptr) && route_group_fused_eligible(T, K, E)) {
        hipStream_t st = S(stream);
        float* lg = (float*)workspace;
        hipError_t err = launch_logits_exact(x, x_dtype == MOE_BF16, w_router, bias, T, H, E, lg, st);
        if (err != hipSuccess) return MOE_ERR_HIP;
        return hip_status(launch_route_select_group(lg, T, E, K, topk_idx, topk_w, counts, offsets, perm, inv_perm, st));
    }
    const moe_status r = moe_route(x, x_dtype, w_router, bias, T, H, E, K, topk_idx, topk_w, nullptr, workspace, rws,
                                   stream);
    if (r != MOE_OK) return r;
    return moe_permute(topk_idx, T, K, E, counts, offsets, perm, inv_perm, (char*)workspace + rws, ws_bytes - rws,
                       stream);
}

}  // namespace

// The scratch of moe_route_group_noalloc: a fixed device array, one copy per
// GPU (made when the library's code object is loaded on that GPU, held until
// the process ends).  Host code must not use the array's name as an address:
// its device address is looked up once per device and kept in scratch_ptr.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::once_flag scratch_once[NOALLOC_MAX_DEVICES];
void* scratch_ptr[NOALLOC_MAX_DEVICES];
hipError_t scratch_err[NOALLOC_MAX_DEVICES];

// The current device's copy of `scratch` (its address looked up on the first
// call made with that device current), or nullptr.
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return nullptr;
    std::call_once(scratch_once[dev], [dev] {
        void* p = nullptr;
        scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    return scratch_ptr[dev];
}
}  // namespace

extern "C" {

moe_status moe_route_group(const void* x, int32_t x_dtype, const float* w_router, const float* bias, int32_t T,
                           int32_t H, int32_t E, int32_t K, int32_t* topk_idx, float* topk_w, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* workspace, size_t ws_bytes,
                           moe_stream stream) {
    return route_group_on(x, x_dtype, w_router, bias, T, H, E, K, topk_idx, topk_w, counts, offsets, perm, inv_perm,
                          workspace, ws_bytes, stream);
}

moe_status moe_route_group_noalloc(const void* x, int32_t x_dtype, const float* w_router, const float* bias,
                                   int32_t T, int32_t H, int32_t E, int32_t K, int32_t* topk_idx, float* topk_w,
                                   int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                   moe_stream stream) {
    const moe_status chk = route_check(x, x_dtype, w_router, T, H, E, K, topk_idx, topk_w);
    if (chk != MOE_OK) return chk;
    if (moe_route_group_workspace_size(T, H, E, K, x_dtype) > NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    void* ws = device_scratch();
    if (!ws) return MOE_ERR_HIP;
    return route_group_on(x, x_dtype, w_router, bias, T, H, E, K, topk_idx, topk_w, counts, offsets, perm, inv_perm,
                          ws, NOALLOC_SCRATCH_BYTES, stream);
}

size_t moe_ffn_workspace_size(int32_t T, int32_t K, int32_t E, int32_t H, int32_t F, int32_t x_dtype,
                              int32_t w_dtype) {
    if (T < 0 || K <= 0 || E <= 0 || H <= 0 || F <= 0) return 0;
    return ffn_workspace_bytes(T, K, E, H, F, x_dtype, w_dtype) + 256;
}

}  // extern "C"

namespace {
// moe_ffn's argument checks (everything but the workspace)
moe_status ffn_check(const void* x, int32_t x_dtype, const moe_expert_weights* w, const int32_t* offsets,
                     const int32_t* perm, int32_t T, int32_t K, int32_t H, int32_t F, int32_t E, const void* y_perm,
                     int32_t y_dtype) {
    if (T < 0 || K <= 0 || E <= 0 || H <= 0 || F <= 0 || K > E || (int64_t)T * K > INT32_MAX)
        return MOE_ERR_INVALID_ARG;
    if (!w || !offsets || (T > 0 && (!x || !perm || !y_perm))) return MOE_ERR_INVALID_ARG;
    if (!w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_INVALID_ARG;
    const bool quant = w->dtype == MOE_INT4_B32 || w->dtype == MOE_INT3_B32 || w->dtype == MOE_INT2_B32;
    if ((x_dtype != MOE_F32 && x_dtype != MOE_BF16) || (y_dtype != MOE_F32 && y_dtype != MOE_BF16) ||
        (w->dtype != MOE_F32 && w->dtype != MOE_BF16 && !quant))
        return MOE_ERR_INVALID_ARG;
    if (quant && (!w->s_gate || !w->s_up || !w->s_down)) return MOE_ERR_INVALID_ARG;
    // int3 / int2: the few-token (verify, decode) streaming kernels
    if ((w->dtype == MOE_INT3_B32 || w->dtype == MOE_INT2_B32) &&
        (x_dtype != MOE_BF16 || !ffn_stream_q4_eligible(T, K, E, H, F)))
        return MOE_ERR_UNSUPPORTED;
    if ((int64_t)T * K * H > ((int64_t)1 << 40)) return MOE_ERR_INVALID_ARG;
    // built combinations
    if (x_dtype == MOE_F32) {
        if (w->dtype != MOE_F32 || y_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
    } else {
        if (w->dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
        if (H % 128 != 0 || F % 64 != 0) return MOE_ERR_UNSUPPORTED;
        if (!aligned16(x) || !aligned16(w->w_gate) || !aligned16(w->w_up) || !aligned16(w->w_down) ||
            !aligned16(y_perm))
            return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_ffn(const void* x, int32_t x_dtype, const moe_expert_weights* w, const int32_t* offsets,
                   const int32_t* perm, int32_t T, int32_t K, int32_t H, int32_t F, int32_t E, void* y_perm,
                   int32_t y_dtype, void* workspace, size_t ws_bytes, moe_stream stream) {
    const moe_status chk = ffn_check(x, x_dtype, w, offsets, perm, T, K, H, F, E, y_perm, y_dtype);
    if (chk != MOE_OK) return chk;
    const size_t need = moe_ffn_workspace_size(T, K, E, H, F, x_dtype, w->dtype);
    if (!workspace || ws_bytes < need || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
    return hip_status(launch_ffn(x, x_dtype, w->dtype, w->w_gate, w->w_up, w->w_down, w->s_gate, w->s_up, w->s_down,
                                 offsets, perm, T, K, H, F, E, y_perm, y_dtype, workspace, S(stream)));
}

moe_status moe_combine(const void* y_perm, int32_t y_dtype, const int32_t* inv_perm, const float* topk_w,
                       const void* residual, int32_t T, int32_t K, int32_t H, void* out, int32_t out_dtype,
                       moe_stream stream) {
    if (T < 0 || K <= 0 || H <= 0 || (int64_t)T * K > INT32_MAX) return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!y_perm || !inv_perm || !topk_w || !out)) return MOE_ERR_INVALID_ARG;
    if ((y_dtype != MOE_F32 && y_dtype != MOE_BF16) || (out_dtype != MOE_F32 && out_dtype != MOE_BF16))
        return MOE_ERR_INVALID_ARG;
    if (H % 8 != 0 || !aligned16(y_perm) || !aligned16(residual) || !aligned16(out)) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_combine(y_perm, y_dtype == MOE_BF16, inv_perm, topk_w, residual, T, K, H, out,
                                     out_dtype == MOE_BF16, S(stream)));
}

moe_status moe_combine_steer(const void* y_perm, int32_t y_dtype, const int32_t* inv_perm, const float* topk_w,
                             const void* residual, const float* steer_v, int32_t T, int32_t K, int32_t H, void* out,
                             int32_t out_dtype, moe_stream stream) {
    if (T < 0 || K <= 0 || H <= 0 || (int64_t)T * K > INT32_MAX) return MOE_ERR_INVALID_ARG;
    if (!steer_v || (T > 0 && (!y_perm || !inv_perm || !topk_w || !out))) return MOE_ERR_INVALID_ARG;
    if ((y_dtype != MOE_F32 && y_dtype != MOE_BF16) || (out_dtype != MOE_F32 && out_dtype != MOE_BF16))
        return MOE_ERR_INVALID_ARG;
    if (H % 8 != 0 || H > STEER_MAX_H || !aligned16(y_perm) || !aligned16(residual) || !aligned16(out) ||
        !aligned16(steer_v))
        return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_combine_steer(y_perm, y_dtype == MOE_BF16, inv_perm, topk_w, residual, steer_v, T, K, H,
                                           out, out_dtype == MOE_BF16, S(stream)));
}

size_t moe_layer_workspace_size(int32_t T, int32_t H, int32_t E, int32_t K, int32_t F, int32_t x_dtype,
                                int32_t w_dtype) {
    if (T < 0 || H <= 0 || E <= 0 || K <= 0 || F <= 0) return 0;
    const size_t separate = round256(moe_route_group_workspace_size(T, H, E, K, x_dtype)) +
                            round256(moe_ffn_workspace_size(T, K, E, H, F, x_dtype, w_dtype)) +
                            round256((size_t)T * K * H * (x_dtype == MOE_F32 ? 4 : 2));
    const size_t fused = verify_layer_eligible(T, H, E, K, F, x_dtype, w_dtype)
                             ? round256(verify_layer_workspace_bytes(T, H, E, K, F))
                             : 0;
    return separate > fused ? separate : fused;
}

moe_status moe_layer(const void* x, int32_t x_dtype, const float* w_router, const float* bias,
                     const moe_expert_weights* w, int32_t T, int32_t H, int32_t E, int32_t K, int32_t F,
                     const void* residual, const float* steer_v, void* out, int32_t* topk_idx, float* topk_w,
                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* workspace,
                     size_t ws_bytes, moe_stream stream) {
    moe_status chk = route_check(x, x_dtype, w_router, T, H, E, K, topk_idx, topk_w);
    if (chk != MOE_OK) return chk;
    if (!counts || !offsets || (T > 0 && (!perm || !inv_perm || !out))) return MOE_ERR_INVALID_ARG;
    if (!w || !w->w_gate || !w->w_up || !w->w_down || F <= 0) return MOE_ERR_INVALID_ARG;
    const bool quant = w->dtype == MOE_INT4_B32 || w->dtype == MOE_INT3_B32 || w->dtype == MOE_INT2_B32;
    if (quant && (!w->s_gate || !w->s_up || !w->s_down)) return MOE_ERR_INVALID_ARG;
    const int32_t ydt = x_dtype == MOE_F32 ? MOE_F32 : MOE_BF16;
    const bool fused = T > 0 && verify_layer_eligible(T, H, E, K, F, x_dtype, w->dtype) && aligned16(x) &&
                       aligned16(w->w_gate) && aligned16(w->w_up) && aligned16(w->w_down) &&
                       (!quant || (aligned16(w->s_gate) && aligned16(w->s_up) && aligned16(w->s_down)));
    // otherwise the separate path's checks (the expert call's, on a stand-in y_perm)
    if (!fused) {
        chk = ffn_check(x, x_dtype, w, offsets, perm, T, K, H, F, E, workspace, ydt);
        if (chk != MOE_OK) return chk;
    }
    if (H % 8 != 0 || !aligned16(residual) || !aligned16(out)) return MOE_ERR_UNSUPPORTED;
    if (steer_v && (H > STEER_MAX_H || !aligned16(steer_v))) return MOE_ERR_UNSUPPORTED;
    const size_t need = moe_layer_workspace_size(T, H, E, K, F, x_dtype, w->dtype);
    if (!workspace || ws_bytes < need || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
    if (T == 0) return MOE_OK;
    hipStream_t st = S(stream);
    if (fused)
        return hip_status(launch_verify_layer(x, w_router, bias, w->dtype, w->w_gate, w->w_up, w->w_down, w->s_gate,
                                              w->s_up, w->s_down, T, H, E, K, F, residual, steer_v, out, topk_idx,
                                              topk_w, counts, offsets, perm, inv_perm, workspace, st));
    // the separate calls: routing + grouping, experts into y_perm, combine
    const size_t rg = round256(moe_route_group_workspace_size(T, H, E, K, x_dtype));
    const size_t fw = round256(moe_ffn_workspace_size(T, K, E, H, F, x_dtype, w->dtype));
    char* wb = (char*)workspace;
    void* y = wb + rg + fw;
    moe_status s = route_group_on(x, x_dtype, w_router, bias, T, H, E, K, topk_idx, topk_w, counts, offsets, perm,
                                  inv_perm, wb, rg, stream);
    if (s != MOE_OK) return s;
    s = moe_ffn(x, x_dtype, w, offsets, perm, T, K, H, F, E, y, ydt, wb + rg, fw, stream);
    if (s != MOE_OK) return s;
    if (steer_v) return moe_combine_steer(y, ydt, inv_perm, topk_w, residual, steer_v, T, K, H, out, x_dtype, stream);
    return moe_combine(y, ydt, inv_perm, topk_w, residual, T, K, H, out, x_dtype, stream);
}

moe_status moe_expert_freq(const float* logits, int32_t L, int64_t T, int32_t E, int32_t K, int64_t* counts,
                           int32_t accumulate, int32_t keep, int32_t* rank_of, int32_t* keep_map,
                           moe_stream stream) {
    if (!counts || L <= 0 || T < 0 || E <= 0 || K <= 0 || K > E || keep < 0 || keep > E) return MOE_ERR_INVALID_ARG;
    if (T > 0 && !logits) return MOE_ERR_INVALID_ARG;
    if (keep > 0 && (!rank_of || !keep_map)) return MOE_ERR_INVALID_ARG;
    if (L > 65535) return MOE_ERR_INVALID_ARG;
    if (K > MAX_K || E > MAX_E) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_freq(logits, L, T, E, K, (unsigned long long*)counts, accumulate != 0, keep, rank_of,
                                  keep_map, S(stream)));
}

}  // extern "C"
