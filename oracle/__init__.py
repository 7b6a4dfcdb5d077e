"""CPU oracle for the routed-expert MoE layer (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps `moe_oracle.c` (plain single-threaded C, fp64)
through ctypes and shares no code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(BUILD_DIR, "liboracle.so")
# a deliberately mutated oracle build (planted-mistake tests) may be loaded instead
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB_OVERRIDE")

F32, BF16, INT4, INT2, INT3 = 0, 1, 2, 3, 4
_DT = {"f32": F32, "bf16": BF16, "int4": INT4, "int2": INT2, "int3": INT3}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (single-threaded, no fp contraction)."""
    if not force and os.path.exists(LIB):
        return LIB
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O3", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(LIB):
                build()
            L = ctypes.CDLL(LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_bf16_value.restype = ctypes.c_double
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_round_bf16.restype = ctypes.c_uint16
        L.oracle_round_bf16.argtypes = [ctypes.c_double]
        L.oracle_fp16_value.restype = ctypes.c_double
        L.oracle_fp16_value.argtypes = [ctypes.c_uint16]
        L.oracle_int4_dequant.argtypes = [vp, vp, i64, i64, vp]
        L.oracle_lowbit_dequant.argtypes = [vp, vp, i64, i64, i32, vp]
        L.oracle_router_logits.argtypes = [vp, i32, vp, vp, i64, i32, i32, vp]
        L.oracle_topk.argtypes = [vp, i64, i32, i32, vp, vp]
        L.oracle_permute.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp]
        L.oracle_expert_ffn.argtypes = [vp, i32, i64, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
        L.oracle_layer_rows.argtypes = [vp, i32, vp, vp, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                        vp, vp, i64, i32, vp, vp]
        L.oracle_expert_freq.argtypes = [vp, i32, i64, i32, i32, vp, i32, i32, vp, vp]
        L.oracle_rank_keep.argtypes = [vp, i32, i32, i32, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def _act(x):
    """(array, dtype code) for an activation array: float32 values or uint16 bf16 bits."""
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), BF16
    return np.ascontiguousarray(x, dtype=np.float32), F32


# ---------------------------------------------------------------- formats
def bf16_value(bits: int) -> float:
    return lib().oracle_bf16_value(int(bits))


def round_bf16(v: float) -> int:
    return int(lib().oracle_round_bf16(float(v)))


def fp16_value(bits: int) -> float:
    return lib().oracle_fp16_value(int(bits))


def int4_dequant(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Dequantise a 2-D int4 matrix [rows][cols/2] with fp16 scales [rows][cols/32]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    sc = np.ascontiguousarray(scales).view(np.uint16)
    rows, cols = packed.shape[0], packed.shape[1] * 2
    out = np.empty((rows, cols), dtype=np.float64)
    _check(lib().oracle_int4_dequant(_p(packed), _p(sc), rows, cols, _p(out)), "int4_dequant")
    return out


def lowbit_dequant(packed: np.ndarray, scales: np.ndarray, bits: int) -> np.ndarray:
    """Dequantise a 2-D int2 (bits 2) or int3 (bits 3) matrix [rows][cols*bits/8]
    with fp16 scales [rows][cols/32] (R16)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    sc = np.ascontiguousarray(scales).view(np.uint16)
    rows, cols = packed.shape[0], packed.shape[1] * 8 // bits
    out = np.empty((rows, cols), dtype=np.float64)
    _check(lib().oracle_lowbit_dequant(_p(packed), _p(sc), rows, cols, bits, _p(out)), "lowbit_dequant")
    return out


# ---------------------------------------------------------------- a1 / a2
def router_logits(x, wr, bias=None) -> np.ndarray:
    x, xdt = _act(x)
    wr = _c(wr, np.float32)
    bias = _c(bias, np.float32)
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    _check(lib().oracle_router_logits(_p(x), xdt, _p(wr), _p(bias), T, H, E, _p(out)), "router_logits")
    return out


def topk(logits, K: int, weights: bool = True):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, K), dtype=np.int32)
    w = np.empty((T, K), dtype=np.float32) if weights else None
    _check(lib().oracle_topk(_p(logits), T, E, K, _p(idx), _p(w)), "topk")
    return (idx, w) if weights else idx


def route(x, wr, K: int, bias=None):
    """(idx, w, logits) for all tokens."""
    logits = router_logits(x, wr, bias)
    idx, w = topk(logits, K)
    return idx, w, logits


# ---------------------------------------------------------------- a3
def permute(idx, E: int):
    idx = _c(idx, np.int32)
    T, K = idx.shape
    n = T * K
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(n, np.int32)
    inv = np.empty(n, np.int32)
    _check(lib().oracle_permute(_p(idx), T, K, E, _p(counts), _p(offsets), _p(perm), _p(inv)), "permute")
    return counts, offsets, perm, inv


# ---------------------------------------------------------------- a4 / a5
class Weights:
    """Expert weights as host arrays: f32, bf16 bits (uint16) or int4 / int3 / int2 (packed + fp16 scales)."""

    def __init__(self, wdt, wg, wu, wd, sg=None, su=None, sd=None):
        self.dt = _DT[wdt]
        if self.dt == F32:
            conv = lambda a: _c(a, np.float32)  # noqa: E731
        elif self.dt == BF16:
            conv = lambda a: _c(a, np.uint16)  # noqa: E731
        else:
            conv = lambda a: _c(a, np.uint8)  # noqa: E731
        self.wg, self.wu, self.wd = conv(wg), conv(wu), conv(wd)
        sc = lambda a: None if a is None else np.ascontiguousarray(a).view(np.uint16)  # noqa: E731
        self.sg, self.su, self.sd = sc(sg), sc(su), sc(sd)
        self.E, self.F = self.wg.shape[0], self.wg.shape[1]
        self.H = self.wd.shape[1]


def expert_ffn(x_row, w: Weights, e: int) -> np.ndarray:
    x, xdt = _act(np.asarray(x_row)[None, :])
    y = np.empty(w.H, dtype=np.float64)
    _check(lib().oracle_expert_ffn(_p(x), xdt, 0, _p(w.wg), _p(w.wu), _p(w.wd), _p(w.sg), _p(w.su), _p(w.sd),
                                   w.dt, e, w.H, w.F, 1 if xdt == BF16 else 0, _p(y)), "expert_ffn")
    return y


def layer_rows(x, idx, wts, w: Weights, rows=None, residual=None, out_bf16=None, want_y=False):
    """Layer output rows (after combine and optional residual) for the listed tokens.

    Returns float32 rows, or uint16 bf16 bits when out_bf16 (default: same as x)."""
    x, xdt = _act(x)
    T, H = x.shape
    idx = _c(idx, np.int32)
    wts = _c(wts, np.float32)
    K = idx.shape[1]
    rows = np.arange(T, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    if out_bf16 is None:
        out_bf16 = xdt == BF16
    res = None
    if residual is not None:
        res = np.ascontiguousarray(residual, dtype=np.uint16 if xdt == BF16 else np.float32)
    n = len(rows)
    out = np.empty((n, H), dtype=np.uint16 if out_bf16 else np.float32)
    y = np.empty((n, K, H), dtype=np.float64) if want_y else None
    _check(lib().oracle_layer_rows(_p(x), xdt, _p(idx), _p(wts), K, _p(w.wg), _p(w.wu), _p(w.wd),
                                   _p(w.sg), _p(w.su), _p(w.sd), w.dt, H, w.F, _p(res), _p(rows), n,
                                   BF16 if out_bf16 else F32, _p(out), _p(y)), "layer_rows")
    return (out, y) if want_y else out


# ---------------------------------------------------------------- a6
def expert_freq(logits, K: int, keep: int = 0, counts=None, accumulate=False):
    logits = _c(logits, np.float32)
    L, T, E = logits.shape
    if counts is None:
        counts = np.zeros((L, E), dtype=np.int64)
    rank_of = np.empty((L, E), np.int32) if keep else None
    keep_map = np.empty((L, keep), np.int32) if keep else None
    _check(lib().oracle_expert_freq(_p(logits), L, T, E, K, _p(counts), 1 if accumulate else 0, keep,
                                    _p(rank_of), _p(keep_map)), "expert_freq")
    return counts, rank_of, keep_map


def rank_keep(counts, keep: int):
    counts = _c(counts, np.int64)
    L, E = counts.shape
    rank_of = np.empty((L, E), np.int32)
    keep_map = np.empty((L, keep), np.int32)
    _check(lib().oracle_rank_keep(_p(counts), L, E, keep, _p(rank_of), _p(keep_map)), "rank_keep")
    return rank_of, keep_map
