"""Thin Python binding of libmoe (include/moe.h) over torch device tensors.

Argument marshalling only: every step runs in the library's HIP kernels.
torch provides device memory and the current stream.  If the library has not
been built, loading fails with an error (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
F32, BF16, INT4_B32, INT2_B32, INT3_B32 = 0, 1, 2, 3, 4
_QUANT_BY_BITS = {4: INT4_B32, 3: INT3_B32, 2: INT2_B32}

EXPORTS = ["moe_abi_version", "moe_status_string", "moe_route_workspace_size", "moe_route",
           "moe_permute_workspace_size", "moe_permute", "moe_ffn_workspace_size", "moe_ffn",
           "moe_route_group_workspace_size", "moe_route_group", "moe_route_group_noalloc", "moe_combine", "moe_combine_steer", "moe_layer_workspace_size", "moe_layer", "moe_expert_freq", "moe_profile_workspace_size", "moe_profile_rank",
           "moe_profile_hits", "moe_strp_size", "moe_strp_write", "moe_strp_read", "moe_profile_remap"]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class ExpertWeights(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p),
                ("s_down", ctypes.c_void_p)]


_lib = None


def lib_path() -> str:
    return _build.LIB


def load():
    """Load libmoe.so (raises if it is missing: build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m routed_expert_ffn_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.moe_abi_version.restype = ctypes.c_int
    L.moe_abi_version.argtypes = []
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_route_workspace_size.restype = sz
    L.moe_route_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.moe_route.restype = ctypes.c_int
    L.moe_route.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.moe_permute_workspace_size.restype = sz
    L.moe_permute_workspace_size.argtypes = [i32, i32, i32]
    L.moe_permute.restype = ctypes.c_int
    L.moe_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.moe_ffn_workspace_size.restype = sz
    L.moe_ffn_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.moe_ffn.restype = ctypes.c_int
    L.moe_ffn.argtypes = [vp, i32, ctypes.POINTER(ExpertWeights), vp, vp, i32, i32, i32, i32, i32, vp, i32, vp, sz,
                          vp]
    L.moe_combine.restype = ctypes.c_int
    L.moe_combine.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, vp, i32, vp]
    L.moe_route_group_workspace_size.restype = sz
    L.moe_route_group_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.moe_route_group.restype = ctypes.c_int
    L.moe_route_group.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_route_group_noalloc.restype = ctypes.c_int
    L.moe_route_group_noalloc.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.moe_combine_steer.restype = ctypes.c_int
    L.moe_combine_steer.argtypes = [vp, i32, vp, vp, vp, vp, i32, i32, i32, vp, i32, vp]
    L.moe_layer_workspace_size.restype = sz
    L.moe_layer_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.moe_layer.restype = ctypes.c_int
    L.moe_layer.argtypes = [vp, i32, vp, vp, ctypes.POINTER(ExpertWeights), i32, i32, i32, i32, i32, vp, vp, vp,
                            vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_freq.restype = ctypes.c_int
    L.moe_expert_freq.argtypes = [vp, i32, i64, i32, i32, vp, i32, i32, vp, vp, vp]
    L.moe_profile_workspace_size.restype = sz
    L.moe_profile_workspace_size.argtypes = [i32, i32]
    L.moe_profile_rank.restype = ctypes.c_int
    L.moe_profile_rank.argtypes = [vp, i32, i32, vp, vp, vp, sz, vp]
    L.moe_profile_hits.restype = ctypes.c_int
    L.moe_profile_hits.argtypes = [vp, i32, i64, i32, vp, i32, i64, vp, vp]
    L.moe_strp_size.restype = sz
    L.moe_strp_size.argtypes = [i32, i32, i32]
    L.moe_strp_write.restype = ctypes.c_int
    L.moe_strp_write.argtypes = [vp, i32, i32, i32, vp, sz]
    L.moe_strp_read.restype = ctypes.c_int
    L.moe_strp_read.argtypes = [vp, sz, vp, vp, vp, vp, i32, vp, i64]
    L.moe_profile_remap.restype = ctypes.c_int
    L.moe_profile_remap.argtypes = [vp, i32, i32, i32, vp, i32, vp, vp]
    _lib = L
    return L


def status_string(s: int) -> str:
    return load().moe_status_string(int(s)).decode()


def abi_version() -> int:
    return int(load().moe_abi_version())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _chk(rc, what):
    if rc != MOE_OK:
        raise MoeError(rc, what)


def _act_dtype(t) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"activations must be float32 or bfloat16, not {t.dtype}")


def _need(t, name, dtype=None, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _workspace(nbytes: int, device, ws=None):
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ moe_route
def route_workspace_size(T, H, E, K, x_dtype=BF16) -> int:
    return int(load().moe_route_workspace_size(T, H, E, K, x_dtype))


def route(x, w_router, K: int, bias=None, logits_out=None, workspace=None, stream=None, out=None):
    """Top-K expert ids [T][K] int32 and weights [T][K] fp32 (out: optional (idx, w) to fill)."""
    _need(x, "x")
    T, H = x.shape
    E = w_router.shape[0]
    _need(w_router, "w_router", torch.float32, (E, H))
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    if logits_out is not None:
        _need(logits_out, "logits_out", torch.float32, (T, E))
    if out is not None:
        idx, w = out
        _need(idx, "topk_idx", torch.int32, (T, K))
        _need(w, "topk_w", torch.float32, (T, K))
    else:
        idx = torch.empty((T, K), dtype=torch.int32, device=x.device)
        w = torch.empty((T, K), dtype=torch.float32, device=x.device)
    nb = route_workspace_size(T, H, E, K, _act_dtype(x))
    ws = _workspace(nb, x.device, workspace)
    _chk(load().moe_route(_ptr(x), _act_dtype(x), _ptr(w_router), _ptr(bias), T, H, E, K, _ptr(idx), _ptr(w),
                          _ptr(logits_out), _ptr(ws), nb, _stream(stream)), "moe_route")
    return idx, w


# ------------------------------------------------------------------ moe_permute
def permute_workspace_size(T, K, E) -> int:
    return int(load().moe_permute_workspace_size(T, K, E))


def permute(topk_idx, E: int, workspace=None, stream=None, out=None):
    """(counts [E], offsets [E+1], perm [T*K], inv_perm [T*K]), all int32 (out: optional tuple to fill)."""
    _need(topk_idx, "topk_idx", torch.int32)
    T, K = topk_idx.shape
    dev = topk_idx.device
    if out is not None:
        counts, offsets, perm, inv = out
        for n, t, shp in (("counts", counts, (E,)), ("offsets", offsets, (E + 1,)), ("perm", perm, (T * K,)),
                          ("inv_perm", inv, (T * K,))):
            _need(t, n, torch.int32, shp)
    else:
        counts = torch.empty(E, dtype=torch.int32, device=dev)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        perm = torch.empty(T * K, dtype=torch.int32, device=dev)
        inv = torch.empty(T * K, dtype=torch.int32, device=dev)
    nb = permute_workspace_size(T, K, E)
    ws = _workspace(nb, dev, workspace)
    _chk(load().moe_permute(_ptr(topk_idx), T, K, E, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv), _ptr(ws),
                            nb, _stream(stream)), "moe_permute")
    return counts, offsets, perm, inv


# ------------------------------------------------------------------ moe_route_group
def route_group_workspace_size(T, H, E, K, x_dtype=BF16) -> int:
    return int(load().moe_route_group_workspace_size(T, H, E, K, x_dtype))


def route_group(x, w_router, K: int, bias=None, workspace=None, stream=None, out=None):
    """moe_route then moe_permute in one call (one launch for selection and
    grouping when few tokens are routed).  Returns (idx, w, counts, offsets,
    perm, inv); out: optional 6-tuple to fill."""
    _need(x, "x")
    T, H = x.shape
    E = w_router.shape[0]
    _need(w_router, "w_router", torch.float32, (E, H))
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    dev = x.device
    if out is not None:
        idx, w, counts, offsets, perm, inv = out
        for n, t, dt, shp in (("topk_idx", idx, torch.int32, (T, K)), ("topk_w", w, torch.float32, (T, K)),
                              ("counts", counts, torch.int32, (E,)), ("offsets", offsets, torch.int32, (E + 1,)),
                              ("perm", perm, torch.int32, (T * K,)), ("inv_perm", inv, torch.int32, (T * K,))):
            _need(t, n, dt, shp)
    else:
        i32 = dict(dtype=torch.int32, device=dev)
        idx, w = torch.empty((T, K), **i32), torch.empty((T, K), dtype=torch.float32, device=dev)
        counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
        perm, inv = torch.empty(T * K, **i32), torch.empty(T * K, **i32)
    nb = route_group_workspace_size(T, H, E, K, _act_dtype(x))
    ws = _workspace(nb, dev, workspace)
    _chk(load().moe_route_group(_ptr(x), _act_dtype(x), _ptr(w_router), _ptr(bias), T, H, E, K, _ptr(idx), _ptr(w),
                                _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv), _ptr(ws), nb, _stream(stream)),
         "moe_route_group")
    return idx, w, counts, offsets, perm, inv


def route_group_noalloc(x, w_router, K: int, bias=None, stream=None, out=None):
    """moe_route_group_noalloc: route_group on the library's own per-GPU
    scratch (no workspace argument, nothing allocated by the library).
    Returns (idx, w, counts, offsets, perm, inv); out: optional 6-tuple to fill."""
    _need(x, "x")
    T, H = x.shape
    E = w_router.shape[0]
    _need(w_router, "w_router", torch.float32, (E, H))
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    dev = x.device
    if out is not None:
        idx, w, counts, offsets, perm, inv = out
        for n, t, dt, shp in (("topk_idx", idx, torch.int32, (T, K)), ("topk_w", w, torch.float32, (T, K)),
                              ("counts", counts, torch.int32, (E,)), ("offsets", offsets, torch.int32, (E + 1,)),
                              ("perm", perm, torch.int32, (T * K,)), ("inv_perm", inv, torch.int32, (T * K,))):
            _need(t, n, dt, shp)
    else:
        i32 = dict(dtype=torch.int32, device=dev)
        idx, w = torch.empty((T, K), **i32), torch.empty((T, K), dtype=torch.float32, device=dev)
        counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
        perm, inv = torch.empty(T * K, **i32), torch.empty(T * K, **i32)
    _chk(load().moe_route_group_noalloc(_ptr(x), _act_dtype(x), _ptr(w_router), _ptr(bias), T, H, E, K, _ptr(idx),
                                        _ptr(w), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv),
                                        _stream(stream)), "moe_route_group_noalloc")
    return idx, w, counts, offsets, perm, inv


# ------------------------------------------------------------------ moe_ffn
def weights_struct(wg, wu, wd, sg=None, su=None, sd=None) -> ExpertWeights:
    if wg.dtype == torch.uint8:
        # block-quantised: the bits per weight follow from the row lengths
        # (gate/up rows hold H inputs, H = the down matrix's row count)
        H, F = wd.shape[1], wg.shape[1]
        bits = wg.shape[2] * 8 // H
        if bits not in _QUANT_BY_BITS or wg.shape[2] * 8 != bits * H or wd.shape[2] * 8 != bits * F:
            raise ValueError(f"packed weights of shapes {tuple(wg.shape)} / {tuple(wd.shape)} are not int4, int3 or int2")
        dt = _QUANT_BY_BITS[bits]
        for n, s in (("s_gate", sg), ("s_up", su), ("s_down", sd)):
            _need(s, n, torch.float16)
    elif wg.dtype == torch.bfloat16:
        dt = BF16
    elif wg.dtype == torch.float32:
        dt = F32
    else:
        raise TypeError(f"expert weights must be float32, bfloat16 or uint8 (int4/int3/int2), not {wg.dtype}")
    for n, t in (("w_gate", wg), ("w_up", wu), ("w_down", wd)):
        _need(t, n, wg.dtype)
    return ExpertWeights(dt, wg.data_ptr(), wu.data_ptr(), wd.data_ptr(),
                         sg.data_ptr() if sg is not None else None, su.data_ptr() if su is not None else None,
                         sd.data_ptr() if sd is not None else None)


def ffn_workspace_size(T, K, E, H, F, x_dtype, w_dtype) -> int:
    return int(load().moe_ffn_workspace_size(T, K, E, H, F, x_dtype, w_dtype))


def ffn(x, wg, wu, wd, offsets, perm, K: int, sg=None, su=None, sd=None, y_dtype=None, out=None, workspace=None,
        stream=None):
    """y_perm [T*K][H] for the grouped rows."""
    _need(x, "x")
    T, H = x.shape
    E = wg.shape[0]
    F = wg.shape[1]
    _need(offsets, "offsets", torch.int32, (E + 1,))
    _need(perm, "perm", torch.int32, (T * K,))
    ws_struct = weights_struct(wg, wu, wd, sg, su, sd)
    if y_dtype is None:
        y_dtype = x.dtype
    y = out if out is not None else torch.empty((T * K, H), dtype=y_dtype, device=x.device)
    _need(y, "y_perm", y_dtype, (T * K, H))
    nb = ffn_workspace_size(T, K, E, H, F, _act_dtype(x), ws_struct.dtype)
    ws = _workspace(nb, x.device, workspace)
    _chk(load().moe_ffn(_ptr(x), _act_dtype(x), ctypes.byref(ws_struct), _ptr(offsets), _ptr(perm), T, K, H, F, E,
                        _ptr(y), _act_dtype(y), _ptr(ws), nb, _stream(stream)), "moe_ffn")
    return y


# ------------------------------------------------------------------ moe_combine
def combine(y_perm, inv_perm, topk_w, residual=None, out_dtype=None, out=None, stream=None, steer_v=None):
    """out [T][H] = sum_k w * y_perm[inv] (+ residual); with steer_v ([H] fp32
    unit vector) the row's component along it is removed before rounding
    (moe_combine_steer)."""
    _need(y_perm, "y_perm")
    _need(topk_w, "topk_w", torch.float32)
    T, K = topk_w.shape
    H = y_perm.shape[1]
    _need(inv_perm, "inv_perm", torch.int32, (T * K,))
    if out_dtype is None:
        out_dtype = residual.dtype if residual is not None else y_perm.dtype
    if residual is not None:
        _need(residual, "residual", out_dtype, (T, H))
    o = out if out is not None else torch.empty((T, H), dtype=out_dtype, device=y_perm.device)
    _need(o, "out", out_dtype, (T, H))
    if steer_v is not None:
        _need(steer_v, "steer_v", torch.float32, (H,))
        _chk(load().moe_combine_steer(_ptr(y_perm), _act_dtype(y_perm), _ptr(inv_perm), _ptr(topk_w), _ptr(residual),
                                      _ptr(steer_v), T, K, H, _ptr(o), _act_dtype(o), _stream(stream)),
             "moe_combine_steer")
        return o
    _chk(load().moe_combine(_ptr(y_perm), _act_dtype(y_perm), _ptr(inv_perm), _ptr(topk_w), _ptr(residual), T, K, H,
                            _ptr(o), _act_dtype(o), _stream(stream)), "moe_combine")
    return o


# ------------------------------------------------------------------ moe_expert_freq
def expert_freq(logits, K: int, keep: int = 0, counts=None, accumulate: bool = False, stream=None):
    """(counts [L][E] int64, rank_of [L][E] int32 | None, keep_map [L][keep] int32 | None)."""
    _need(logits, "logits", torch.float32)
    if logits.dim() == 2:
        logits = logits.unsqueeze(0)
    L, T, E = logits.shape
    dev = logits.device
    if counts is None:
        counts = torch.zeros((L, E), dtype=torch.int64, device=dev)
    _need(counts, "counts", torch.int64, (L, E))
    rank_of = torch.empty((L, E), dtype=torch.int32, device=dev) if keep else None
    keep_map = torch.empty((L, keep), dtype=torch.int32, device=dev) if keep else None
    _chk(load().moe_expert_freq(_ptr(logits), L, T, E, K, _ptr(counts), 1 if accumulate else 0, keep, _ptr(rank_of),
                                _ptr(keep_map), _stream(stream)), "moe_expert_freq")
    return counts, rank_of, keep_map


# ------------------------------------------------------------------ expert profile
def profile_rank(counts, workspace=None, stream=None):
    """counts [L][E] int64 (device) -> (rank [L][E] int32, pairs [L*E][2] int16 holding uint16 (layer, expert))."""
    _need(counts, "counts", torch.int64)
    L, E = counts.shape
    dev = counts.device
    rank = torch.empty((L, E), dtype=torch.int32, device=dev)
    pairs = torch.empty((L * E, 2), dtype=torch.int16, device=dev)
    nb = int(load().moe_profile_workspace_size(L, E))
    ws = _workspace(nb, dev, workspace)
    _chk(load().moe_profile_rank(_ptr(counts), L, E, _ptr(rank), _ptr(pairs), _ptr(ws), nb, _stream(stream)),
         "moe_profile_rank")
    return rank, pairs


def profile_hits(trace, rank, S: int, stream=None):
    """trace [L][T][K] int32, rank [L][E] int32 (device) -> hits (a 1-element int64 tensor, device)."""
    _need(trace, "trace", torch.int32)
    _need(rank, "rank", torch.int32)
    L, T, K = trace.shape
    E = rank.shape[1]
    hits = torch.empty(1, dtype=torch.int64, device=trace.device)   # the uint64 count, < 2^63
    _chk(load().moe_profile_hits(_ptr(trace), L, T, K, _ptr(rank), E, int(S), _ptr(hits), _stream(stream)),
         "moe_profile_hits")
    return hits


def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def strp_write(pairs, L: int, E: int) -> bytes:
    """Host pairs [n][2] (uint16 (layer, expert) in rank order) -> the STRP v1 file's bytes."""
    import numpy as np
    p = np.ascontiguousarray(np.asarray(pairs, dtype=np.uint16).reshape(-1, 2))
    n = p.shape[0]
    nb = int(load().moe_strp_size(L, E, n))
    out = np.empty(nb, dtype=np.uint8)
    _chk(load().moe_strp_write(_np_ptr(p), n, L, E, _np_ptr(out), nb), "moe_strp_write")
    return out.tobytes()


def strp_read(buf: bytes):
    """STRP v1 bytes -> (L, E, pairs [n][2] uint16, inverse [L][E] int16)."""
    import numpy as np
    b = np.frombuffer(buf, dtype=np.uint8).copy()
    L, E, n = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _chk(load().moe_strp_read(_np_ptr(b), b.size, ctypes.byref(L), ctypes.byref(E), ctypes.byref(n), None, 0, None,
                              0), "moe_strp_read")
    pairs = np.empty((n.value, 2), dtype=np.uint16)
    inv = np.empty((L.value, E.value), dtype=np.int16)
    _chk(load().moe_strp_read(_np_ptr(b), b.size, ctypes.byref(L), ctypes.byref(E), ctypes.byref(n), _np_ptr(pairs),
                              n.value, _np_ptr(inv), inv.size), "moe_strp_read")
    return L.value, E.value, pairs, inv


def profile_remap(pairs, keep_map, E_old: int):
    """Host ranked pairs of an E_old-expert profile + keep_map [L][keep] -> the pruned model's ranked pairs."""
    import numpy as np
    p = np.ascontiguousarray(np.asarray(pairs, dtype=np.uint16).reshape(-1, 2))
    km = np.ascontiguousarray(np.asarray(keep_map, dtype=np.int32))
    L, keep = km.shape
    out = np.empty((max(p.shape[0], 1), 2), dtype=np.uint16)
    m = ctypes.c_int32()
    _chk(load().moe_profile_remap(_np_ptr(p), p.shape[0], L, E_old, _np_ptr(km), keep, _np_ptr(out),
                                  ctypes.byref(m)), "moe_profile_remap")
    return out[:m.value].copy()


# ------------------------------------------------------------------ one whole layer
def layer_workspace_size(T, H, E, K, F, x_dtype=BF16, w_dtype=BF16) -> int:
    return int(load().moe_layer_workspace_size(T, H, E, K, F, x_dtype, w_dtype))


class LayerWorkspace:
    """Preallocated workspaces and outputs for repeated calls of `layer` at one shape
    (and of the separate calls at that shape)."""

    def __init__(self, T, H, E, K, F, x_dtype=torch.bfloat16, w_dtype=BF16, y_dtype=None, device="cuda"):
        xd = F32 if x_dtype == torch.float32 else BF16
        self.y_dtype = y_dtype or x_dtype
        self.layer_ws = torch.empty(layer_workspace_size(T, H, E, K, F, xd, w_dtype), dtype=torch.uint8,
                                    device=device)
        self.route_ws = torch.empty(route_workspace_size(T, H, E, K, xd), dtype=torch.uint8, device=device)
        self.group_ws = torch.empty(route_group_workspace_size(T, H, E, K, xd), dtype=torch.uint8, device=device)
        self.perm_ws = torch.empty(permute_workspace_size(T, K, E), dtype=torch.uint8, device=device)
        self.ffn_ws = torch.empty(ffn_workspace_size(T, K, E, H, F, xd, w_dtype), dtype=torch.uint8, device=device)
        self.y = torch.empty((T * K, H), dtype=self.y_dtype, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        self.route_out = (torch.empty((T, K), **i32), torch.empty((T, K), dtype=torch.float32, device=device))
        self.perm_out = (torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(T * K, **i32),
                         torch.empty(T * K, **i32))
        self.out = torch.empty((T, H), dtype=x_dtype, device=device)


def layer(x, w_router, wg, wu, wd, K: int, bias=None, sg=None, su=None, sd=None, residual=None, lw=None,
          stream=None, out=None, steer_v=None):
    """One MoE layer in one library call (moe_layer): routing + grouping, the
    experts and the combine (steered if steer_v is given).  Returns (out,
    routing dict)."""
    _need(x, "x")
    T, H = x.shape
    E, F = wg.shape[0], wg.shape[1]
    _need(w_router, "w_router", torch.float32, (E, H))
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    if residual is not None:
        _need(residual, "residual", x.dtype, (T, H))
    if steer_v is not None:
        _need(steer_v, "steer_v", torch.float32, (H,))
    ws_struct = weights_struct(wg, wu, wd, sg, su, sd)
    dev = x.device
    if lw is not None:
        idx, w = lw.route_out
        counts, offsets, perm, inv = lw.perm_out
        if out is None:
            out = lw.out
    else:
        i32 = dict(dtype=torch.int32, device=dev)
        idx, w = torch.empty((T, K), **i32), torch.empty((T, K), dtype=torch.float32, device=dev)
        counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
        perm, inv = torch.empty(T * K, **i32), torch.empty(T * K, **i32)
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=dev)
    _need(out, "out", x.dtype, (T, H))
    nb = layer_workspace_size(T, H, E, K, F, _act_dtype(x), ws_struct.dtype)
    ws = _workspace(nb, dev, lw.layer_ws if lw is not None else None)
    _chk(load().moe_layer(_ptr(x), _act_dtype(x), _ptr(w_router), _ptr(bias), ctypes.byref(ws_struct), T, H, E, K, F,
                          _ptr(residual), _ptr(steer_v), _ptr(out), _ptr(idx), _ptr(w), _ptr(counts), _ptr(offsets),
                          _ptr(perm), _ptr(inv), _ptr(ws), nb, _stream(stream)), "moe_layer")
    return out, dict(idx=idx, w=w, counts=counts, offsets=offsets, perm=perm, inv=inv)
