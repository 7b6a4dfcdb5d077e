"""moe_route_group_noalloc (routing + grouping on the library's own per-GPU
scratch, for callers that cannot allocate) against moe_route_group with a
caller workspace: identical ids, weights, counts, offsets, permutation and
inverse, on calls in a row whose sizes shrink and grow, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from routed_expert_ffn_amd import moe, synth

from .helpers import TOL_W, to_host, weight_rel_err

pytestmark = pytest.mark.gpu

NAMES = ("idx", "w", "counts", "offsets", "perm", "inv")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()
    yield
    torch.cuda.synchronize()


def inputs(T, E, zipf, layer):
    s = synth.LayerShape(T=T, H=2048, E=E, K=10, F=512, act="bf16", wdt="bf16", zipf=zipf)
    x = synth.make_device_activations(s, seed=0, cfg=21, layer=layer, device="cuda")
    wr, bias = synth.make_device_router(s, seed=0, cfg=21, layer=layer, device="cuda")
    return s, x, wr, bias


def both(s, x, wr, bias):
    ref = moe.route_group(x, wr, s.K, bias=bias)
    got = moe.route_group_noalloc(x, wr, s.K, bias=bias)
    torch.cuda.synchronize()
    return dict(zip(NAMES, ref)), dict(zip(NAMES, got))


def test_noalloc_matches_route_group_on_calls_in_a_row():
    # prefill chunk (estimate + rechecks), then a verify step (fused exact
    # path), then a mid-size call on the estimate path again
    for T, E, zipf, layer in ((8192, 512, True, 0), (5, 512, False, 1), (200, 256, False, 2)):
        s, x, wr, bias = inputs(T, E, zipf, layer)
        ref, got = both(s, x, wr, bias)
        for n in NAMES:
            assert torch.equal(got[n], ref[n]), f"T={T}: {n} differs from moe_route_group"
        if T <= 200:
            ref_idx, ref_w, _ = oracle.route(to_host(x), to_host(wr), s.K, None if bias is None else to_host(bias))
            assert np.array_equal(to_host(got["idx"]), ref_idx)
            assert weight_rel_err(to_host(got["w"]), ref_w) <= TOL_W


SCRATCH_BYTES = 32 << 20


def largest_fitting_T(E, H=2048, K=10):
    lo, hi = 1, 1 << 20
    while lo < hi:
        m = (lo + hi + 1) // 2
        if moe.route_group_workspace_size(m, H, E, K) <= SCRATCH_BYTES:
            lo = m
        else:
            hi = m - 1
    return lo


def test_noalloc_rejects_sizes_beyond_its_scratch():
    t_max = largest_fitting_T(512)
    s, x, wr, bias = inputs(t_max + 1, 512, False, 3)
    idx = torch.full((s.T, s.K), -7, dtype=torch.int32, device="cuda")
    w = torch.full((s.T, s.K), -7.0, dtype=torch.float32, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    rest = (torch.full((s.E,), -7, **i32), torch.full((s.E + 1,), -7, **i32), torch.full((s.T * s.K,), -7, **i32),
            torch.full((s.T * s.K,), -7, **i32))
    with pytest.raises(moe.MoeError) as ei:
        moe.route_group_noalloc(x, wr, s.K, out=(idx, w) + rest)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((idx == -7).all()) and bool((w == -7.0).all()) and all(bool((t == -7).all()) for t in rest)
    # the largest size that fits still runs, and matches
    s, x, wr, bias = inputs(t_max, 512, False, 3)
    ref, got = both(s, x, wr, bias)
    for n in NAMES:
        assert torch.equal(got[n], ref[n]), f"T={t_max}: {n} differs from moe_route_group"
