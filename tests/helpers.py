"""Shared helpers for the GPU parity tests: device<->host conversion of the
synthetic inputs and the tolerance metric.  No layer arithmetic here."""
import numpy as np
import torch

import oracle
from routed_expert_ffn_amd import synth

# Floating-point tolerances for layer outputs (max over rows of the row-relative
# max error) and routing weights (elementwise relative).
TOL_BF16 = 2e-2
TOL_F32 = 1e-4
TOL_W = 1e-4


def to_host(t):
    """Device tensor -> numpy in the oracle's formats (bf16 as uint16 bits, fp16 as float16)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def host_weights(layer) -> "oracle.Weights":
    wdt = layer.shape.wdt
    return oracle.Weights(wdt, to_host(layer.wg), to_host(layer.wu), to_host(layer.wd),
                          None if layer.sg is None else to_host(layer.sg),
                          None if layer.su is None else to_host(layer.su),
                          None if layer.sd is None else to_host(layer.sd))


def device_from_host(h, device="cuda"):
    """synth.HostLayer -> synth.DeviceLayer with the same bytes."""
    def dev(a, dt=None):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    s = h.shape
    x = dev(h.x)
    return synth.DeviceLayer(s, x, dev(h.wr), dev(h.bias), dev(h.wg), dev(h.wu), dev(h.wd), dev(h.sg), dev(h.su),
                             dev(h.sd))


def as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def row_rel_err(got, ref):
    """max over rows of max|got-ref| / max|ref| (an all-zero reference row needs an all-zero result)."""
    g, r = as_f64(got), as_f64(ref)
    num = np.abs(g - r).max(axis=1)
    den = np.abs(r).max(axis=1)
    zero = den == 0
    assert np.all(num[zero] == 0), "nonzero output where the reference row is zero"
    return float((num[~zero] / den[~zero]).max()) if np.any(~zero) else 0.0


def weight_rel_err(got, ref):
    g, r = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(g - r) / np.abs(r)))
