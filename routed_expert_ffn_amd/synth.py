"""Seeded synthetic inputs for the routed-expert MoE layer.

This module only *makes inputs*: activations, router weights and bias, expert
weights (fp32, bf16 or block-int4) and given router logits.  It holds none of
the layer's arithmetic (no routing, no FFN, no combine, no counting), so both
the CPU oracle's tests and the GPU path may draw from it.

Workload shapes follow the pages: 48 MoE layers of 512 experts with 10 routed
per token, pruned to 256 per layer ("Strata Coder 编程模型深度剖析", §1 and
§3), prefill chunks of at most 8,192 tokens and a 4-deep speculative verify
(kwkr.cn Coder benchmark write-up, "测试环境与运行配置").  Dimensions the pages
do not print (hidden 2048, expert width 512, the N(0,1)/N(0,0.02) value
distributions, the Zipf(1.1) router offset and the int4 block format) are
the workload definitions this library is built for.

Two generator back-ends produce the same distributions:
  * numpy PCG64 on the host for small cases (tests the oracle can finish);
  * torch's device generator for GB-sized tensors (parity at full size and
    the benchmark); the same bytes are then handed to both sides.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

# tensor ids for seed derivation
TID_X, TID_WR, TID_PERM, TID_WG, TID_WU, TID_WD, TID_Z, TID_V = 0, 1, 2, 3, 4, 5, 6, 7

ZIPF_S = 1.1
INT4_BLOCK = 32


@dataclasses.dataclass(frozen=True)
class LayerShape:
    T: int          # tokens
    H: int          # hidden
    E: int          # experts
    K: int          # routed per token
    F: int          # expert FFN width
    act: str        # "f32" | "bf16"
    wdt: str        # "f32" | "bf16" | "int4" | "int3" | "int2"
    zipf: bool = False   # Zipf(1.1) per-expert router offset


# The five workloads.  Names say what each one is.
TINY_FP32 = LayerShape(T=32, H=256, E=64, K=4, F=128, act="f32", wdt="f32")
VERIFY_BF16 = LayerShape(T=5, H=2048, E=512, K=10, F=512, act="bf16", wdt="bf16")
PREFILL_BF16 = LayerShape(T=8192, H=2048, E=512, K=10, F=512, act="bf16", wdt="bf16", zipf=True)
STACK_INT4_LAYERS = 48
STACK_INT4_PREFILL = LayerShape(T=8192, H=2048, E=256, K=10, F=512, act="bf16", wdt="int4")
STACK_INT4_VERIFY = LayerShape(T=5, H=2048, E=256, K=10, F=512, act="bf16", wdt="int4")
# the same verify step with lower-bit experts
STACK_INT3_VERIFY = LayerShape(T=5, H=2048, E=256, K=10, F=512, act="bf16", wdt="int3")
STACK_INT2_VERIFY = LayerShape(T=5, H=2048, E=256, K=10, F=512, act="bf16", wdt="int2")
LOWBIT = {"int2": 2, "int3": 3}
FREQ_L, FREQ_T, FREQ_E, FREQ_K, FREQ_KEEP = 48, 262144, 512, 10, 256


def seed_words(seed: int, cfg: int, layer: int, tid: int) -> list[int]:
    return [int(seed), int(cfg), int(layer), int(tid)]


def np_rng(seed: int, cfg: int, layer: int, tid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed_words(seed, cfg, layer, tid))))


def torch_seed(seed: int, cfg: int, layer: int, tid: int) -> int:
    """63-bit seed for torch's generator derived from the same four words."""
    h = hashlib.sha256(np.asarray(seed_words(seed, cfg, layer, tid), dtype=np.int64).tobytes()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


# ---------------------------------------------------------------- casts
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def int4_quantize(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric int4 in blocks of 32 along the last axis, fp16 scale per block.

    d = fp16(max|w| / 7) (0 for an all-zero block); q = clamp(rne(w / d), -8, 7);
    stored as the unsigned nibble q + 8, element 2j in the low nibble of byte j.
    Returns (packed uint8 [..., cols/2], scales float16 [..., cols/32]).
    """
    w = np.asarray(w, dtype=np.float32)
    cols = w.shape[-1]
    assert cols % INT4_BLOCK == 0
    blk = w.reshape(*w.shape[:-1], cols // INT4_BLOCK, INT4_BLOCK)
    amax = np.abs(blk).max(axis=-1)
    d16 = (amax / np.float32(7.0)).astype(np.float16)
    d32 = d16.astype(np.float32)
    safe = np.where(d32 == 0, np.float32(1.0), d32)
    q = np.rint(blk / safe[..., None]).astype(np.int32)
    q = np.where(d32[..., None] == 0, 0, q)
    q = np.clip(q, -8, 7) + 8
    q = q.reshape(*w.shape[:-1], cols).astype(np.uint8)
    packed = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
    return packed, d16


def lowbit_levels_np(w: np.ndarray, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric `bits`-bit quantisation in blocks of 32 along the last axis:
    d = fp16(max|w| / (2^(bits-1) - 1)), q = clamp(rne(w / d), -2^(bits-1),
    2^(bits-1) - 1), level u = q + 2^(bits-1).  Returns (u uint8 [..., cols],
    scales float16 [..., cols/32])."""
    w = np.asarray(w, dtype=np.float32)
    cols = w.shape[-1]
    assert cols % INT4_BLOCK == 0
    half = 1 << (bits - 1)
    blk = w.reshape(*w.shape[:-1], cols // INT4_BLOCK, INT4_BLOCK)
    amax = np.abs(blk).max(axis=-1)
    d16 = (amax / np.float32(half - 1)).astype(np.float16)
    d32 = d16.astype(np.float32)
    safe = np.where(d32 == 0, np.float32(1.0), d32)
    q = np.rint(blk / safe[..., None]).astype(np.int32)
    q = np.where(d32[..., None] == 0, 0, q)
    u = (np.clip(q, -half, half - 1) + half).reshape(*w.shape[:-1], cols).astype(np.uint8)
    return u, d16


def lowbit_pack_np(u: np.ndarray, bits: int) -> np.ndarray:
    """Pack levels u [..., cols] (0 <= u < 2^bits) into rows of cols*bits/8
    bytes: the low two bits as little-endian 32-bit words of 16 elements
    (element 4k + j of a word in byte j, bits 2k..2k+1), then for int3 the third
    bit as words of 32 elements (element 16g + 4k + j in byte j, bit 4g + k)."""
    u = np.asarray(u, dtype=np.uint8)
    lead, cols = u.shape[:-1], u.shape[-1]
    lo = (u & 3).reshape(*lead, cols // 16, 4, 4)                 # [word][k][j]
    plane2 = np.zeros((*lead, cols // 16, 4), dtype=np.uint8)
    for k in range(4):
        plane2 |= lo[..., k, :] << (2 * k)
    out = plane2.reshape(*lead, cols // 4)
    if bits == 3:
        hi = (u >> 2).reshape(*lead, cols // 32, 2, 4, 4)         # [word][g][k][j]
        plane3 = np.zeros((*lead, cols // 32, 4), dtype=np.uint8)
        for g in range(2):
            for k in range(4):
                plane3 |= hi[..., g, k, :] << (4 * g + k)
        out = np.concatenate([out, plane3.reshape(*lead, cols // 8)], axis=-1)
    return out


def lowbit_quantize(w: np.ndarray, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """(packed uint8 [..., cols*bits/8], scales float16 [..., cols/32])."""
    u, d = lowbit_levels_np(w, bits)
    return lowbit_pack_np(u, bits), d


# ---------------------------------------------------------------- host generators
def zipf_bias_np(E: int, seed: int, cfg: int, layer: int) -> np.ndarray:
    """Per-expert router offset b[e] = -s * ln(1 + pi(e)) (log of a Zipf(s) pmf,
    normaliser dropped), pi a seeded permutation so hot experts are spread over ids."""
    pi = np_rng(seed, cfg, layer, TID_PERM).permutation(E)
    return (-ZIPF_S * np.log1p(pi.astype(np.float64))).astype(np.float32)


@dataclasses.dataclass
class HostLayer:
    shape: LayerShape
    x: np.ndarray            # [T][H] float32 or uint16 (bf16 bits)
    wr: np.ndarray           # [E][H] float32
    bias: Optional[np.ndarray]
    wg: np.ndarray           # f32 [E][F][H] | bf16 bits | int4 packed [E][F][H/2]
    wu: np.ndarray
    wd: np.ndarray           # [E][H][F] (int4: [E][H][F/2])
    sg: Optional[np.ndarray] = None   # int4 scales fp16 [E][F][H/32]
    su: Optional[np.ndarray] = None
    sd: Optional[np.ndarray] = None   # [E][H][F/32]


def make_host_layer(s: LayerShape, seed: int = 0, cfg: int = 0, layer: int = 0,
                    sigma_x: float = 1.0, sigma_w: float = 0.02) -> HostLayer:
    """Numpy-generated layer inputs (C-order standard normals, scaled, fp32)."""
    x = (np_rng(seed, cfg, layer, TID_X).standard_normal((s.T, s.H), dtype=np.float32) * np.float32(sigma_x))
    wr = np_rng(seed, cfg, layer, TID_WR).standard_normal((s.E, s.H), dtype=np.float32) * np.float32(sigma_w)
    wg = np_rng(seed, cfg, layer, TID_WG).standard_normal((s.E, s.F, s.H), dtype=np.float32) * np.float32(sigma_w)
    wu = np_rng(seed, cfg, layer, TID_WU).standard_normal((s.E, s.F, s.H), dtype=np.float32) * np.float32(sigma_w)
    wd = np_rng(seed, cfg, layer, TID_WD).standard_normal((s.E, s.H, s.F), dtype=np.float32) * np.float32(sigma_w)
    bias = zipf_bias_np(s.E, seed, cfg, layer) if s.zipf else None
    if s.act == "bf16":
        x = f32_to_bf16_bits(x)
    out = HostLayer(s, x, wr, bias, wg, wu, wd)
    if s.wdt == "bf16":
        out.wg, out.wu, out.wd = f32_to_bf16_bits(wg), f32_to_bf16_bits(wu), f32_to_bf16_bits(wd)
    elif s.wdt == "int4":
        out.wg, out.sg = int4_quantize(wg)
        out.wu, out.su = int4_quantize(wu)
        out.wd, out.sd = int4_quantize(wd)
    elif s.wdt in LOWBIT:
        b = LOWBIT[s.wdt]
        out.wg, out.sg = lowbit_quantize(wg, b)
        out.wu, out.su = lowbit_quantize(wu, b)
        out.wd, out.sd = lowbit_quantize(wd, b)
    return out


def steer_vector(H: int, seed: int = 0, cfg: int = 5, layer: int = 0) -> np.ndarray:
    """A synthetic steering direction: [H] fp32, N(0,1) entries scaled (in fp64)
    to unit length.  The pages' vectors come from a trained model; only their
    shape (one unit direction per steered layer) is reproduced."""
    v = np_rng(seed, cfg, layer, TID_V).standard_normal(H)
    return (v / np.linalg.norm(v)).astype(np.float32)


def make_host_logits(L: int, T: int, E: int, seed: int = 0, cfg: int = 3, zipf: bool = True,
                     layer0: int = 0) -> np.ndarray:
    """Given router logits [L][T][E] = fp32(z + b_l[e]), z ~ N(0,1) fp32."""
    out = np.empty((L, T, E), dtype=np.float32)
    for l in range(L):
        z = np_rng(seed, cfg, layer0 + l, TID_Z).standard_normal((T, E), dtype=np.float32)
        if zipf:
            z += zipf_bias_np(E, seed, cfg, layer0 + l)[None, :]
        out[l] = z
    return out


# ---------------------------------------------------------------- device generators (torch)
def _torch():
    import torch
    return torch


def _dev_normal(shape, sigma, seed, cfg, layer, tid, device, out_dtype, chunk_rows=None):
    """N(0, sigma) generated on `device` in fp32 chunks along dim 0 and cast
    (torch's float->bfloat16 cast rounds to nearest even)."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, cfg, layer, tid))
    out = torch.empty(shape, dtype=out_dtype, device=device)
    n0 = shape[0]
    step = chunk_rows or max(1, n0)
    for i in range(0, n0, step):
        j = min(n0, i + step)
        blk = torch.randn((j - i,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
        if sigma != 1.0:
            blk.mul_(sigma)
        out[i:j].copy_(blk)
        del blk
    return out


def int4_quantize_torch(w):
    """Torch version of int4_quantize (same format); w float32 [..., cols]."""
    torch = _torch()
    cols = w.shape[-1]
    blk = w.reshape(*w.shape[:-1], cols // INT4_BLOCK, INT4_BLOCK)
    amax = blk.abs().amax(dim=-1)
    d16 = (amax / 7.0).to(torch.float16)
    d32 = d16.to(torch.float32)
    safe = torch.where(d32 == 0, torch.ones_like(d32), d32)
    q = torch.round(blk / safe.unsqueeze(-1))
    q = torch.where(d32.unsqueeze(-1) == 0, torch.zeros_like(q), q)
    q = (q.clamp_(-8, 7) + 8).to(torch.uint8).reshape(*w.shape[:-1], cols)
    packed = q[..., 0::2] | (q[..., 1::2] << 4)
    return packed.contiguous(), d16.contiguous()


def lowbit_quantize_torch(w, bits: int):
    """Torch version of lowbit_quantize (same format); w float32 [..., cols]."""
    torch = _torch()
    cols = w.shape[-1]
    lead = tuple(w.shape[:-1])
    half = 1 << (bits - 1)
    blk = w.reshape(*lead, cols // INT4_BLOCK, INT4_BLOCK)
    amax = blk.abs().amax(dim=-1)
    d16 = (amax / float(half - 1)).to(torch.float16)
    d32 = d16.to(torch.float32)
    safe = torch.where(d32 == 0, torch.ones_like(d32), d32)
    q = torch.round(blk / safe.unsqueeze(-1))
    q = torch.where(d32.unsqueeze(-1) == 0, torch.zeros_like(q), q)
    u = (q.clamp_(-half, half - 1) + half).to(torch.uint8).reshape(*lead, cols)
    lo = (u & 3).reshape(*lead, cols // 16, 4, 4)
    plane2 = torch.zeros(lead + (cols // 16, 4), dtype=torch.uint8, device=w.device)
    for k in range(4):
        plane2 |= lo[..., k, :] << (2 * k)
    out = plane2.reshape(*lead, cols // 4)
    if bits == 3:
        hi = (u >> 2).reshape(*lead, cols // 32, 2, 4, 4)
        plane3 = torch.zeros(lead + (cols // 32, 4), dtype=torch.uint8, device=w.device)
        for g in range(2):
            for k in range(4):
                plane3 |= hi[..., g, k, :] << (4 * g + k)
        out = torch.cat([out, plane3.reshape(*lead, cols // 8)], dim=-1)
    return out.contiguous(), d16.contiguous()


@dataclasses.dataclass
class DeviceLayer:
    shape: LayerShape
    x: object
    wr: object
    bias: object
    wg: object
    wu: object
    wd: object
    sg: object = None
    su: object = None
    sd: object = None


def zipf_bias_torch(E, seed, cfg, layer, device):
    torch = _torch()
    return torch.from_numpy(zipf_bias_np(E, seed, cfg, layer)).to(device)


def make_device_weights(s: LayerShape, seed: int, cfg: int, layer: int, device, sigma_w: float = 0.02):
    """Expert weights generated on the device (fp32 draw per expert chunk)."""
    torch = _torch()
    shapes = {TID_WG: (s.E, s.F, s.H), TID_WU: (s.E, s.F, s.H), TID_WD: (s.E, s.H, s.F)}
    res = {}
    for tid, shp in shapes.items():
        if s.wdt in ("f32", "bf16"):
            dt = torch.float32 if s.wdt == "f32" else torch.bfloat16
            res[tid] = (_dev_normal(shp, sigma_w, seed, cfg, layer, tid, device, dt, chunk_rows=32), None)
        else:
            bits = LOWBIT.get(s.wdt, 4)
            g = torch.Generator(device=device)
            g.manual_seed(torch_seed(seed, cfg, layer, tid))
            packed = torch.empty(shp[:-1] + (shp[-1] * bits // 8,), dtype=torch.uint8, device=device)
            scales = torch.empty(shp[:-1] + (shp[-1] // INT4_BLOCK,), dtype=torch.float16, device=device)
            for i in range(0, shp[0], 32):
                j = min(shp[0], i + 32)
                blk = torch.randn((j - i,) + shp[1:], generator=g, device=device, dtype=torch.float32).mul_(sigma_w)
                p, d = int4_quantize_torch(blk) if bits == 4 else lowbit_quantize_torch(blk, bits)
                packed[i:j].copy_(p)
                scales[i:j].copy_(d)
                del blk, p, d
            res[tid] = (packed, scales)
    return res


def make_device_activations(s: LayerShape, seed: int = 0, cfg: int = 0, layer: int = 0, device="cuda"):
    """The layer's input rows [T][H] as make_device_layer draws them (same bytes)."""
    torch = _torch()
    xdt = torch.float32 if s.act == "f32" else torch.bfloat16
    return _dev_normal((s.T, s.H), 1.0, seed, cfg, layer, TID_X, device, xdt)


def make_device_router(s: LayerShape, seed: int = 0, cfg: int = 0, layer: int = 0, device="cuda"):
    """(router weights [E][H] fp32, Zipf offset [E] fp32 or None) as make_device_layer draws them."""
    torch = _torch()
    wr = _dev_normal((s.E, s.H), 0.02, seed, cfg, layer, TID_WR, device, torch.float32)
    bias = zipf_bias_torch(s.E, seed, cfg, layer, device) if s.zipf else None
    return wr, bias


def make_device_layer(s: LayerShape, seed: int = 0, cfg: int = 0, layer: int = 0, device="cuda",
                      x=None) -> DeviceLayer:
    if x is None:
        x = make_device_activations(s, seed, cfg, layer, device)
    wr, bias = make_device_router(s, seed, cfg, layer, device)
    w = make_device_weights(s, seed, cfg, layer, device)
    return DeviceLayer(s, x, wr, bias, w[TID_WG][0], w[TID_WU][0], w[TID_WD][0],
                       w[TID_WG][1], w[TID_WU][1], w[TID_WD][1])


def make_device_logits_layer(T: int, E: int, seed: int, cfg: int, layer: int, device, zipf: bool = True, out=None):
    """One layer of given router logits [T][E] fp32 = z + b_l, generated on the device."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, cfg, layer, TID_Z))
    if out is None:
        out = torch.empty((T, E), dtype=torch.float32, device=device)
    torch.randn((T, E), generator=g, device=device, dtype=torch.float32, out=out)
    if zipf:
        out.add_(zipf_bias_torch(E, seed, cfg, layer, device).unsqueeze(0))
    return out


def expert_bytes(s: LayerShape) -> int:
    """Bytes of one expert's gate+up+down weights in the layer's format."""
    n = 3 * s.F * s.H
    if s.wdt == "f32":
        return 4 * n
    if s.wdt == "bf16":
        return 2 * n
    return n * LOWBIT.get(s.wdt, 4) // 8 + 2 * (n // INT4_BLOCK)


def describe() -> str:
    return ("x ~ N(0,1); router and expert weights ~ N(0,0.02); fp32 draws cast by RNE to bf16 "
            "or quantised to int4 / int3 / int2 (blocks of 32 along the input dim, fp16 scale = max|w|/7, "
            "/3, /1); "
            "Zipf(1.1) router offset b[e] = -1.1 ln(1+pi(e)) with a seeded permutation pi")

