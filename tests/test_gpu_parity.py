"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Integers (expert ids, permutation, counts, ranks) must be
bit-exact; floats within the stated tolerances.

Workloads follow the pages' shapes: 10 of 512 experts per token, 256 after
pruning, 48 layers ("Strata Coder 编程模型深度剖析", §1, §3); 8,192-token prefill
chunks and a 4+1-token speculative verify (kwkr.cn Coder write-up,
"测试环境与运行配置").
"""
import numpy as np
import pytest
import torch

import oracle
from routed_expert_ffn_amd import moe, synth

from .helpers import (TOL_BF16, TOL_F32, TOL_W, as_f64, device_from_host, host_weights, row_rel_err, to_host,
                      weight_rel_err)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()
    if not __import__("os").path.exists(oracle.LIB):
        oracle.build()
    yield
    torch.cuda.synchronize()


def run_layer(d, residual=None, steer_v=None):
    """The layer in one call (moe_layer)."""
    s = d.shape
    lw = moe.LayerWorkspace(s.T, s.H, s.E, s.K, s.F, x_dtype=d.x.dtype,
                            w_dtype={"f32": moe.F32, "bf16": moe.BF16, "int4": moe.INT4_B32, "int3": moe.INT3_B32,
                                     "int2": moe.INT2_B32}[s.wdt])
    out, r = moe.layer(d.x, d.wr, d.wg, d.wu, d.wd, s.K, bias=d.bias, sg=d.sg, su=d.su, sd=d.sd,
                       residual=residual, lw=lw, steer_v=steer_v)
    torch.cuda.synchronize()
    return out, r


def run_separate(d, residual=None, y_dtype=None, steer_v=None):
    """The layer as the separate calls: route + group, experts into y_perm (y_dtype), combine."""
    s = d.shape
    idx, w, counts, offsets, perm, inv = moe.route_group(d.x, d.wr, s.K, bias=d.bias)
    y = moe.ffn(d.x, d.wg, d.wu, d.wd, offsets, perm, s.K, d.sg, d.su, d.sd, y_dtype=y_dtype or d.x.dtype)
    out = moe.combine(y, inv, w, residual=residual, out_dtype=d.x.dtype, steer_v=steer_v)
    torch.cuda.synchronize()
    return out, dict(idx=idx, w=w, counts=counts, offsets=offsets, perm=perm, inv=inv, y=y)


def check_routing_and_grouping(r, ref_idx, ref_w, E):
    idx = to_host(r["idx"])
    assert np.array_equal(idx, ref_idx), f"top-K ids differ at {np.argwhere(idx != ref_idx)[:5].tolist()}"
    assert weight_rel_err(to_host(r["w"]), ref_w) <= TOL_W
    counts, offsets, perm, inv = oracle.permute(ref_idx, E)
    assert np.array_equal(to_host(r["counts"]), counts)
    assert np.array_equal(to_host(r["offsets"]), offsets)
    assert np.array_equal(to_host(r["perm"]), perm)
    assert np.array_equal(to_host(r["inv"]), inv)


# ---------------------------------------------------------------- tiny fp32 layer
def test_tiny_fp32_layer_exact_routing_and_output():
    s = synth.TINY_FP32
    h = synth.make_host_layer(s, seed=0, cfg=1)
    d = device_from_host(h)
    ref_idx, ref_w, ref_lg = oracle.route(h.x, h.wr, s.K)
    lg = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    moe.route(d.x, d.wr, s.K, logits_out=lg)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(lg).view(np.uint32), ref_lg.view(np.uint32)), "logits are not bit-exact"
    out, r = run_layer(d)
    check_routing_and_grouping(r, ref_idx, ref_w, s.E)
    ref_out = oracle.layer_rows(h.x, ref_idx, ref_w, host_weights(d))
    assert row_rel_err(to_host(out), ref_out) <= TOL_F32


# ---------------------------------------------------------------- multi-tile bf16 / int4
SMALL = [
    synth.LayerShape(T=300, H=256, E=40, K=6, F=128, act="bf16", wdt="bf16", zipf=True),
    synth.LayerShape(T=300, H=256, E=40, K=6, F=128, act="bf16", wdt="int4", zipf=True),
    synth.LayerShape(T=77, H=384, E=100, K=10, F=192, act="bf16", wdt="bf16"),
    synth.LayerShape(T=130, H=128, E=8, K=8, F=64, act="bf16", wdt="int4"),
    # bf16 weights, H and 2F multiples of 512: the grouped-GEMM path (128-row
    # tiles, ragged last tile per expert, one item per block)
    synth.LayerShape(T=300, H=512, E=40, K=6, F=256, act="bf16", wdt="bf16", zipf=True),
    synth.LayerShape(T=97, H=1024, E=12, K=3, F=512, act="bf16", wdt="bf16"),
    # int4, most experts touched: the grouped GEMMs with int4 operands staged in LDS
    synth.LayerShape(T=300, H=1024, E=16, K=6, F=512, act="bf16", wdt="int4", zipf=True),
    # T <= 16: the weight-streaming path for the verify step
    synth.LayerShape(T=16, H=256, E=40, K=6, F=128, act="bf16", wdt="bf16", zipf=True),
    synth.LayerShape(T=16, H=256, E=40, K=6, F=128, act="bf16", wdt="int4", zipf=True),
    synth.LayerShape(T=3, H=512, E=24, K=8, F=192, act="bf16", wdt="int4"),
    synth.LayerShape(T=1, H=768, E=300, K=10, F=64, act="bf16", wdt="bf16"),
    # int4, T <= 8, H 2048, F 512: the streaming int4 path (one quant block per lane)
    synth.LayerShape(T=3, H=2048, E=24, K=8, F=512, act="bf16", wdt="int4"),
    synth.LayerShape(T=8, H=2048, E=6, K=4, F=512, act="bf16", wdt="int4", zipf=True),
    # int3 / int2 (the lower-bit verify variant), T <= 8, H 2048, F 512
    synth.LayerShape(T=3, H=2048, E=24, K=8, F=512, act="bf16", wdt="int3"),
    synth.LayerShape(T=8, H=2048, E=6, K=4, F=512, act="bf16", wdt="int3", zipf=True),
    synth.LayerShape(T=1, H=2048, E=40, K=10, F=512, act="bf16", wdt="int2"),
    synth.LayerShape(T=8, H=2048, E=6, K=4, F=512, act="bf16", wdt="int2", zipf=True),
    # bf16, T <= 8, whole 1 KB rows: the streaming bf16 path
    synth.LayerShape(T=7, H=1024, E=40, K=6, F=512, act="bf16", wdt="bf16", zipf=True),
    synth.LayerShape(T=3, H=512, E=16, K=4, F=1024, act="bf16", wdt="bf16"),
]


@pytest.mark.parametrize("s", SMALL, ids=lambda s: f"T{s.T}H{s.H}E{s.E}K{s.K}F{s.F}-{s.wdt}{'-zipf' if s.zipf else ''}")
def test_small_layers_span_tiles(s):
    h = synth.make_host_layer(s, seed=3, cfg=7)
    d = device_from_host(h)
    ref_idx, ref_w, ref_lg = oracle.route(h.x, h.wr, s.K, h.bias)
    out, r = run_layer(d)
    check_routing_and_grouping(r, ref_idx, ref_w, s.E)
    ref_out = oracle.layer_rows(h.x, ref_idx, ref_w, host_weights(d))
    assert row_rel_err(to_host(out), ref_out) <= TOL_BF16
    # the exact-logit path gives bit-exact logits and the same selection
    lg = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    idx2, _ = moe.route(d.x, d.wr, s.K, bias=d.bias, logits_out=lg)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(lg).view(np.uint32), ref_lg.view(np.uint32))
    assert np.array_equal(to_host(idx2), ref_idx)
    # the separate calls, with a bf16 and an fp32 y_perm: the same routing and in-tolerance outputs
    for y_dtype in (None, torch.float32):
        out_s, r_s = run_separate(d, y_dtype=y_dtype)
        check_routing_and_grouping(r_s, ref_idx, ref_w, s.E)
        assert row_rel_err(to_host(out_s), ref_out) <= TOL_BF16


# one whole layer for a few tokens in three launches (moe_layer's fused path:
# T <= 8, H 2048, F 512): (T, E, K, weights, Zipf offset, residual, steering)
FUSED = [
    (1, 64, 10, "bf16", False, False, False),
    (5, 64, 10, "int4", True, True, False),
    (8, 16, 16, "bf16", True, True, True),      # T*K = 128, up to 8 rows per expert
    (3, 40, 4, "int3", False, False, True),
    (7, 24, 8, "int2", True, True, False),
    (6, 9, 9, "int4", False, False, False),     # K = E: every expert in every token
    (4, 33, 1, "bf16", False, True, False),     # K = 1
]


@pytest.mark.parametrize("T,E,K,wdt,zipf,with_res,steer", FUSED,
                         ids=lambda v: str(v) if not isinstance(v, bool) else ("y" if v else "n"))
def test_layer_few_tokens_fused(T, E, K, wdt, zipf, with_res, steer):
    """moe_layer for a few tokens (selection and grouping inside the gate/up
    launch, the combine inside the down launch): routing and grouping exact
    and identical to the separate calls, the output (in place on the residual
    stream, optionally steered) within the bf16 bound of the oracle."""
    from oracle import steer as steer_oracle
    s = synth.LayerShape(T=T, H=2048, E=E, K=K, F=512, act="bf16", wdt=wdt, zipf=zipf)
    h = synth.make_host_layer(s, seed=T + E, cfg=9)
    d = device_from_host(h)
    ref_idx, ref_w, _ = oracle.route(h.x, h.wr, s.K, h.bias)
    v = torch.from_numpy(synth.steer_vector(s.H, layer=T)).cuda() if steer else None
    if with_res:
        stream = d.x.clone()
        lw = moe.LayerWorkspace(T, s.H, E, K, s.F, w_dtype={"bf16": moe.BF16, "int4": moe.INT4_B32,
                                                            "int3": moe.INT3_B32, "int2": moe.INT2_B32}[wdt])
        out, r = moe.layer(stream, d.wr, d.wg, d.wu, d.wd, K, bias=d.bias, sg=d.sg, su=d.su, sd=d.sd,
                           residual=stream, lw=lw, out=stream, steer_v=v)
        torch.cuda.synchronize()
    else:
        out, r = run_layer(d, steer_v=v)
    check_routing_and_grouping(r, ref_idx, ref_w, E)
    _, r_sep = run_separate(d)
    for k in ("idx", "w", "counts", "offsets", "perm", "inv"):
        assert torch.equal(r[k], r_sep[k]), f"{k} differs from the separate calls"
    res = h.x if with_res else None
    if steer:
        _, yk = oracle.layer_rows(h.x, ref_idx, ref_w, host_weights(d), want_y=True)
        hh = (ref_w.astype(np.float64)[:, :, None] * yk).sum(axis=1) + (as_f64(h.x) if with_res else 0.0)
        ref_out = steer_oracle.project_out(hh, to_host(v).astype(np.float64))
    else:
        ref_out = oracle.layer_rows(h.x, ref_idx, ref_w, host_weights(d), residual=res)
    assert row_rel_err(to_host(out), ref_out) <= TOL_BF16


@pytest.mark.parametrize("wdt", ["int4", "int3", "int2"])
def test_layer_few_tokens_fused_lowbit_eighty_slots(wdt):
    """moe_layer with block-quantised experts at T = 8, K = 10 (80 slots: the
    down launch stages more than 64 grouped rows, and the int4 / int2 levels
    are decoded in pair order against activations staged in that order, some
    experts holding several rows): routing exact, outputs within the bf16
    bound of the oracle.  (moe_ffn's separate low-bit path stops at 59 slots.)"""
    s = synth.LayerShape(T=8, H=2048, E=48, K=10, F=512, act="bf16", wdt=wdt, zipf=True)
    h = synth.make_host_layer(s, seed=80, cfg=9)
    d = device_from_host(h)
    ref_idx, ref_w, _ = oracle.route(h.x, h.wr, s.K, h.bias)
    out, r = run_layer(d, residual=d.x)
    check_routing_and_grouping(r, ref_idx, ref_w, s.E)
    assert int(to_host(r["counts"]).max()) >= 4, "want experts with several rows"
    ref_out = oracle.layer_rows(h.x, ref_idx, ref_w, host_weights(d), residual=h.x)
    assert row_rel_err(to_host(out), ref_out) <= TOL_BF16


def test_layer_few_tokens_fused_many_experts_and_ties():
    """The fused path's selection over more than 512 experts (16 logits per
    lane), with exact logit ties (duplicated router rows: the lower id wins)."""
    s = synth.LayerShape(T=8, H=2048, E=700, K=10, F=512, act="bf16", wdt="bf16")
    d = synth.make_device_layer(s, seed=2, cfg=9, layer=0, device="cuda")
    d.wr[1::7] = d.wr[0::7][: d.wr[1::7].shape[0]]          # pairs of equal router rows
    torch.cuda.synchronize()
    x, wr = to_host(d.x), to_host(d.wr)
    ref_idx, ref_w, ref_lg = oracle.route(x, wr, s.K)
    assert np.any(np.diff(np.sort(ref_lg, axis=1), axis=1) == 0)
    out, r = run_layer(d)
    check_routing_and_grouping(r, ref_idx, ref_w, s.E)
    ref_out = oracle.layer_rows(x, ref_idx, ref_w, host_weights(d))
    assert row_rel_err(to_host(out), ref_out) <= TOL_BF16


def test_layer_few_tokens_fused_max_experts():
    """The fused path at its largest expert count (1024: 16 logits per lane,
    a 16-word touched-expert bitmap), checked against the oracle on host
    copies of the touched experts only (the other experts' weights are zero
    pages the oracle never reads)."""
    s = synth.LayerShape(T=8, H=2048, E=1024, K=10, F=512, act="bf16", wdt="bf16")
    d = synth.make_device_layer(s, seed=4, cfg=9, layer=0, device="cuda")
    torch.cuda.synchronize()
    x, wr = to_host(d.x), to_host(d.wr)
    ref_idx, ref_w, _ = oracle.route(x, wr, s.K)
    out, r = run_layer(d)
    check_routing_and_grouping(r, ref_idx, ref_w, s.E)
    wg = np.zeros((s.E, s.F, s.H), np.uint16)
    wu = np.zeros((s.E, s.F, s.H), np.uint16)
    wd = np.zeros((s.E, s.H, s.F), np.uint16)
    for e in np.unique(ref_idx):
        wg[e], wu[e], wd[e] = to_host(d.wg[e]), to_host(d.wu[e]), to_host(d.wd[e])
    ref_out = oracle.layer_rows(x, ref_idx, ref_w, oracle.Weights("bf16", wg, wu, wd))
    assert row_rel_err(to_host(out), ref_out) <= TOL_BF16


@pytest.mark.parametrize("T,E,H,act", [(16, 520, 2048, "bf16"), (13, 513, 1024, "f32"), (5, 257, 512, "bf16"),
                                       (2, 1024, 256, "f32"), (1, 512, 2048, "bf16")])
def test_exact_logits_few_tokens_wave_splits(T, E, H, act):
    """The few-token exact logits where an expert's tokens are split over two
    waves (two experts per block; an odd expert count leaves the last block
    half empty) or four, with up to two groups of four tokens per wave:
    bit-exact against the oracle's pinned summation, same selection."""
    s = synth.LayerShape(T=T, H=H, E=E, K=8, F=8, act=act, wdt="bf16", zipf=True)
    h = synth.make_host_layer(s, seed=T + E, cfg=9)
    d = device_from_host(h)
    ref_idx, _, ref_lg = oracle.route(h.x, h.wr, s.K, h.bias)
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx, _ = moe.route(d.x, d.wr, s.K, bias=d.bias, logits_out=lg)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(lg).view(np.uint32), ref_lg.view(np.uint32)), "logits are not bit-exact"
    assert np.array_equal(to_host(idx), ref_idx)


@pytest.mark.parametrize("wdt", ["bf16", "int4"])
@pytest.mark.parametrize("T", [8, 9, 16, 17, 63, 65])
def test_path_boundaries(T, wdt):
    """Token counts on both sides of every path switch (streaming kernels up to
    8 tokens, the small-T kernels up to 16, the grouped GEMM above; the exact
    router below 64 tokens, the estimate with rechecks from 64)."""
    s = synth.LayerShape(T=T, H=1024, E=24, K=4, F=512, act="bf16", wdt=wdt, zipf=True)
    h = synth.make_host_layer(s, seed=11, cfg=8)
    d = device_from_host(h)
    ref_idx, ref_w, _ = oracle.route(h.x, h.wr, s.K, h.bias)
    out, r = run_layer(d)
    check_routing_and_grouping(r, ref_idx, ref_w, s.E)
    ref_out = oracle.layer_rows(h.x, ref_idx, ref_w, host_weights(d))
    assert row_rel_err(to_host(out), ref_out) <= TOL_BF16


@pytest.mark.parametrize("wdt", ["bf16", "int4"])
def test_gemm_path_blocks_walk_several_items(wdt):
    """More 128-row tiles than the chip holds blocks: every persistent block of
    the grouped GEMM handles several (expert, tile) items in turn (bf16: 128 x
    512 tiles, one block per CU; int4: 128 x 256 tiles, two blocks per CU)."""
    s = synth.LayerShape(T=4096, H=1024, E=16, K=8, F=512, act="bf16", wdt=wdt, zipf=True)
    h = synth.make_host_layer(s, seed=5, cfg=7)
    d = device_from_host(h)
    ref_idx, ref_w, _ = oracle.route(h.x, h.wr, s.K, h.bias)
    counts = np.bincount(ref_idx.ravel(), minlength=s.E)
    n_tiles, per_cu = (2, 1) if wdt == "bf16" else (4, 2)
    items_per_phase = int(np.sum((counts + 127) // 128)) * n_tiles
    assert items_per_phase > 2 * per_cu * torch.cuda.get_device_properties(0).multi_processor_count
    rows = np.unique(np.concatenate([[0, s.T - 1], np.random.default_rng(1).choice(s.T, 62, replace=False)]))
    ref_out = oracle.layer_rows(h.x, ref_idx, ref_w, host_weights(d), rows=rows)
    for y_dtype in (None, torch.float32):
        out, r = run_separate(d, y_dtype=y_dtype)
        check_routing_and_grouping(r, ref_idx, ref_w, s.E)
        assert row_rel_err(to_host(out)[rows], ref_out) <= TOL_BF16


# ---------------------------------------------------------------- routing edge cases
def _route_case(x_np, wr_np, K, bias_np=None):
    xd = torch.from_numpy(x_np.view(np.int16)).cuda().view(torch.bfloat16) if x_np.dtype == np.uint16 \
        else torch.from_numpy(x_np).cuda()
    wr = torch.from_numpy(wr_np).cuda()
    b = torch.from_numpy(bias_np).cuda() if bias_np is not None else None
    idx, w = moe.route(xd, wr, K, bias=b)
    torch.cuda.synchronize()
    ref_idx, ref_w, _ = oracle.route(x_np, wr_np, K, bias_np)
    assert np.array_equal(to_host(idx), ref_idx)
    assert weight_rel_err(to_host(w), ref_w) <= TOL_W
    return ref_idx


@pytest.mark.parametrize("T", [1, 70, 200])
def test_route_ties_go_to_lower_id(T):
    # x = 0 makes every logit 0 (plus an exactly tied bias): all ties
    H, E, K = 128, 96, 10
    x = synth.f32_to_bf16_bits(np.zeros((T, H), np.float32))
    wr = (np.random.default_rng(0).standard_normal((E, H)) * 0.02).astype(np.float32)
    bias = np.zeros(E, np.float32)
    bias[[5, 40, 77]] = 1.0
    ref = _route_case(x, wr, K, bias)
    assert ref[0].tolist() == [5, 40, 77, 0, 1, 2, 3, 4, 6, 7]


@pytest.mark.parametrize("E,K", [(16, 16), (100, 1), (64, 32), (4096, 10), (1, 1)])
def test_route_shapes(E, K):
    rng = np.random.default_rng(E * 7 + K)
    T, H = 150, 256
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    _route_case(x, wr, K)


def test_route_near_ties_are_rechecked():
    # duplicated router rows with a one-ulp bias difference: the fast estimate
    # cannot separate them, the exact recheck must
    rng = np.random.default_rng(11)
    T, H, E, K = 256, 512, 64, 8
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    wr[1::2] = wr[0::2]
    bias = np.zeros(E, np.float32)
    bias[1::2] = np.float32(1e-6)
    _route_case(x, wr, K, bias)


def test_route_recheck_falls_back_to_all_experts():
    # identical router rows: every estimate lies within the margin of the K-th,
    # more than 64 candidates, so each token is re-decided on all E exact
    # logits; the tiny distinct biases round to ties in places (lower id wins)
    rng = np.random.default_rng(12)
    T, H, E, K = 96, 256, 128, 4
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wr = np.tile((rng.standard_normal((1, H)) * 0.02).astype(np.float32), (E, 1))
    bias = (np.arange(E, dtype=np.float32) * np.float32(3e-8)).astype(np.float32)
    _route_case(x, wr, K, bias)


def _rechecked_tokens(xd, wr, K):
    """moe_route on the estimate path; returns (ids, weights, number of tokens re-decided on exact logits)."""
    T, E = xd.shape[0], wr.shape[0]
    ws = torch.empty(moe.route_workspace_size(T, xd.shape[1], E, K), dtype=torch.uint8, device="cuda")
    idx, w = moe.route(xd, wr, K, workspace=ws)
    torch.cuda.synchronize()
    off = (T * E * 4 + 255) // 256 * 256              # the per-token recheck flags follow the [T][E] estimates
    flags = ws[off:off + T * 4].view(torch.int32)
    return idx, w, int(flags.sum().item())


def test_route_margin_follows_input_magnitude():
    """The estimate's margin grows with |x_t| and the router rows' norms (its
    accumulation error does): with activations or router weights scaled by
    powers of two (exact in bf16 / fp32) the selection stays bit-exact, and at
    large scales a comparable share of tokens is still re-decided on exact
    logits (a fixed margin would let them through on estimates whose error has
    grown with the scale)."""
    rng = np.random.default_rng(31)
    T, H, E, K = 1024, 2048, 512, 10
    x32 = rng.standard_normal((T, H)).astype(np.float32)
    w32 = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    base = None
    for xs, ws in ((1.0, 1.0), (1024.0, 1.0), (1.0, 256.0), (2.0 ** -8, 1.0)):
        x = synth.f32_to_bf16_bits(x32 * np.float32(xs))
        wr = (w32 * np.float32(ws)).astype(np.float32)
        xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
        idx, w, n_re = _rechecked_tokens(xd, torch.from_numpy(wr).cuda(), K)
        ref_idx, ref_w, _ = oracle.route(x, wr, K)
        assert np.array_equal(to_host(idx), ref_idx), f"ids differ with x*{xs}, w*{ws}"
        # weights of tokens decided on estimates come from the estimates, whose
        # error (and so the weights' relative error) grows with the scale; at
        # large scales the smallest weights reach fp32's subnormal range, which
        # the GPU's exp may flush to zero (hence the absolute floor)
        tol = TOL_W * max(1.0, xs * ws)
        g, r = to_host(w).astype(np.float64), ref_w.astype(np.float64)
        assert np.all(np.abs(g - r) <= tol * np.abs(r) + 1e-30), f"weights off with x*{xs}, w*{ws}"
        if base is None:
            base = n_re
            assert base > 0
        elif xs * ws > 1:
            assert n_re >= base // 4, f"x*{xs}, w*{ws}: {n_re} tokens re-decided (unscaled: {base})"


def test_route_and_grouping_empty():
    wr = torch.zeros((8, 64), dtype=torch.float32, device="cuda")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    idx, w = moe.route(x, wr, 2)
    counts, offsets, perm, inv = moe.permute(idx, 8)
    torch.cuda.synchronize()
    assert idx.shape == (0, 2) and to_host(counts).tolist() == [0] * 8 and to_host(offsets).tolist() == [0] * 9


# ---------------------------------------------------------------- grouping edge cases
@pytest.mark.parametrize("T,K,E,mode", [(5, 10, 512, "rand"), (3000, 10, 512, "rand"), (4096, 1, 4096, "rand"),
                                        (2500, 4, 64, "one"), (700, 3, 1, "all"), (9000, 10, 300, "skew")])
def test_permute_matches_stable_counting_sort(T, K, E, mode):
    rng = np.random.default_rng(T + K + E)
    if mode == "rand":
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    elif mode == "one":
        idx = np.tile(np.arange(K, dtype=np.int32), (T, 1))
    elif mode == "all":
        idx = np.zeros((T, K), np.int32)
    else:
        p = 1.0 / np.arange(1, E + 1) ** 1.5
        idx = np.stack([rng.choice(E, K, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
    got = moe.permute(torch.from_numpy(idx).cuda(), E)
    torch.cuda.synchronize()
    ref = oracle.permute(idx, E)
    for g, r in zip(got, ref):
        assert np.array_equal(to_host(g), r)
    again = moe.permute(torch.from_numpy(idx).cuda(), E)
    torch.cuda.synchronize()
    for g, a in zip(got, again):
        assert torch.equal(g, a)


# ---------------------------------------------------------------- routing + grouping in one call
@pytest.mark.parametrize("T,E,K,H,act,ties", [
    (1, 512, 10, 2048, "bf16", False),
    (5, 512, 10, 2048, "bf16", True),       # the verify step, with tied router rows
    (16, 64, 32, 256, "bf16", True),        # 512 slots
    (16, 4096, 4, 256, "f32", False),       # the widest expert count
    (3, 300, 10, 512, "bf16", True),        # experts not a multiple of 64
    (17, 64, 8, 256, "bf16", False),        # past the one-block path: route, then permute
    (100, 512, 10, 2048, "bf16", False),    # the estimate path, then permute
    (0, 64, 4, 256, "bf16", False),
])
def test_route_group_matches_oracle_and_separate_calls(T, E, K, H, act, ties):
    rng = np.random.default_rng(T * 7 + E)
    x32 = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    if ties:
        wr[E // 2] = wr[1]                     # equal logits on two experts: the lower id must win
        wr[E - 1] = wr[0]
    x_h = synth.f32_to_bf16_bits(x32) if act == "bf16" else x32
    x = (torch.from_numpy(x_h.view(np.int16)).cuda().view(torch.bfloat16) if act == "bf16"
         else torch.from_numpy(x_h).cuda())
    wr_d = torch.from_numpy(wr).cuda()
    got = moe.route_group(x, wr_d, K)
    idx2, w2 = moe.route(x, wr_d, K)
    sep = moe.permute(idx2, E)
    torch.cuda.synchronize()
    names = ("idx", "w", "counts", "offsets", "perm", "inv")
    r = dict(zip(names, got))
    for a, b in zip(got, (idx2, w2) + tuple(sep)):
        assert torch.equal(a, b), "one call and two calls must agree bit for bit"
    if T == 0:
        assert not r["counts"].any() and not r["offsets"].any()
        return
    ref_idx, ref_w, _ = oracle.route(x_h, wr, K)
    check_routing_and_grouping(r, ref_idx, ref_w, E)


# ---------------------------------------------------------------- combine
def test_combine_in_place_residual_and_fp32():
    rng = np.random.default_rng(5)
    T, K, H = 37, 4, 256
    y = torch.from_numpy(rng.standard_normal((T * K, H)).astype(np.float32)).cuda()
    inv = torch.from_numpy(rng.permutation(T * K).astype(np.int32)).cuda()
    w = torch.from_numpy(rng.random((T, K)).astype(np.float32)).cuda()
    res = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).cuda()
    ref = (w.double().unsqueeze(-1) * y.double()[inv.long()].view(T, K, H)).sum(1) + res.double()
    out = moe.combine(y, inv, w, residual=res.clone())
    res2 = res.clone()
    moe.combine(y, inv, w, residual=res2, out=res2)        # out aliases residual
    torch.cuda.synchronize()
    assert torch.allclose(out.double(), ref, rtol=1e-5, atol=1e-5)
    assert torch.equal(out, res2)


# ---------------------------------------------------------------- steered combine
@pytest.mark.parametrize("ydt,odt,T,K,H,with_res", [
    ("f32", "f32", 37, 4, 256, True),        # one partial chunk
    ("bf16", "bf16", 5, 10, 2048, True),      # the verify step's shape
    ("bf16", "f32", 19, 10, 2560, False),     # two chunks, the second ragged (the pages' stream width)
    ("bf16", "bf16", 3, 8, 8192, True),       # the widest row one block holds
    ("f32", "bf16", 0, 4, 256, True),         # no tokens
])
def test_combine_steer_matches_oracle(ydt, odt, T, K, H, with_res):
    from oracle import steer
    rng = np.random.default_rng(T * 131 + H)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    y = torch.from_numpy(rng.standard_normal((T * K, H)).astype(np.float32)).to(tdt[ydt]).cuda()
    inv = torch.from_numpy(rng.permutation(T * K).astype(np.int32)).cuda()
    w = torch.from_numpy(rng.random((T, K)).astype(np.float32)).cuda()
    res = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(tdt[odt]).cuda() if with_res else None
    v = torch.from_numpy(synth.steer_vector(H, seed=T, layer=H)).cuda()
    out = moe.combine(y, inv, w, residual=res, out_dtype=tdt[odt], steer_v=v)
    again = moe.combine(y, inv, w, residual=res, out_dtype=tdt[odt], steer_v=v)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "the steered combine must not vary from run to run"
    if T == 0:
        return
    ref = steer.combine_steer(as_f64(to_host(y)), to_host(inv), to_host(w), to_host(v).astype(np.float64),
                              None if res is None else as_f64(to_host(res)))
    got = as_f64(to_host(out))
    assert row_rel_err(got, ref) <= (TOL_F32 if odt == "f32" else TOL_BF16)
    # what is left along v is the output's own rounding: with fp32 output a
    # few units of fp32 precision of the row, with bf16 a few of bf16
    along = np.abs(got @ to_host(v).astype(np.float64)) / np.linalg.norm(got, axis=1)
    assert along.max() <= (1e-5 if odt == "f32" else 2e-2)


def test_combine_steer_prefill_shape_sampled_rows():
    """The steered combine at the prefill chunk's shape (8192 tokens, K 10, H 2048,
    bf16), the launch the benchmark times: sampled rows against the oracle."""
    from oracle import steer
    T, K, H = 8192, 10, 2048
    g = torch.Generator(device="cuda")
    g.manual_seed(17)
    y = torch.randn((T * K, H), generator=g, device="cuda").to(torch.bfloat16)
    inv = torch.randperm(T * K, generator=g, device="cuda").to(torch.int32)
    w = torch.rand((T, K), generator=g, device="cuda")
    res = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.from_numpy(synth.steer_vector(H, seed=5)).cuda()
    out = moe.combine(y, inv, w, residual=res, steer_v=v)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(4).choice(T, 30, replace=False)]))
    inv_h, w_h = to_host(inv).reshape(T, K), to_host(w)
    y_rows = as_f64(to_host(y[torch.from_numpy(inv_h[rows].reshape(-1).astype(np.int64)).cuda()]))
    ref = steer.combine_steer(y_rows, np.arange(len(rows) * K), w_h[rows], to_host(v).astype(np.float64),
                              as_f64(to_host(res))[rows])
    assert row_rel_err(to_host(out)[rows], ref) <= TOL_BF16


def test_combine_steer_in_place_and_unit_axis():
    """out aliasing residual gives the same bytes; v = e_j zeroes column j exactly
    and leaves every other column as the plain combine rounds it."""
    rng = np.random.default_rng(77)
    T, K, H = 29, 6, 2560
    y = torch.from_numpy(rng.standard_normal((T * K, H)).astype(np.float32)).to(torch.bfloat16).cuda()
    inv = torch.from_numpy(rng.permutation(T * K).astype(np.int32)).cuda()
    w = torch.from_numpy(rng.random((T, K)).astype(np.float32)).cuda()
    res = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16).cuda()
    v = torch.from_numpy(synth.steer_vector(H, seed=3)).cuda()
    out = moe.combine(y, inv, w, residual=res, steer_v=v)
    res2 = res.clone()
    moe.combine(y, inv, w, residual=res2, out=res2, steer_v=v)
    e = torch.zeros(H, dtype=torch.float32, device="cuda")
    e[2049] = 1.0
    unit = moe.combine(y, inv, w, residual=res, steer_v=e)
    plain = moe.combine(y, inv, w, residual=res)
    torch.cuda.synchronize()
    assert torch.equal(out, res2)
    assert torch.all(unit[:, 2049] == 0)
    keep = torch.ones(H, dtype=torch.bool, device="cuda")
    keep[2049] = False
    assert torch.equal(unit[:, keep], plain[:, keep])


def test_steered_int4_verify_layer_full_size():
    """One steered layer of the pruned int4 stack at the verify shape, updating
    the stream in place: routing exact, output within the bf16 bound of the
    oracle's fp64 combine + residual + projection."""
    from oracle import steer
    s = synth.STACK_INT4_VERIFY
    d = synth.make_device_layer(s, seed=0, cfg=5, layer=1, device="cuda")
    v = torch.from_numpy(synth.steer_vector(s.H, layer=1)).cuda()
    torch.cuda.synchronize()
    x, wr = to_host(d.x), to_host(d.wr)
    ref_idx, ref_w, _ = oracle.route(x, wr, s.K)
    lw = moe.LayerWorkspace(s.T, s.H, s.E, s.K, s.F, x_dtype=d.x.dtype, w_dtype=moe.INT4_B32)
    h = d.x.clone()
    out, r = moe.layer(h, d.wr, d.wg, d.wu, d.wd, s.K, sg=d.sg, su=d.su, sd=d.sd, residual=h, lw=lw, out=h,
                       steer_v=v)
    torch.cuda.synchronize()
    check_routing_and_grouping(r, ref_idx, ref_w, s.E)
    _, yk = oracle.layer_rows(x, ref_idx, ref_w, host_weights(d), want_y=True)
    hh = (ref_w.astype(np.float64)[:, :, None] * yk).sum(axis=1) + as_f64(x)
    ref = steer.project_out(hh, to_host(v).astype(np.float64))
    assert row_rel_err(to_host(out), ref) <= TOL_BF16


# ---------------------------------------------------------------- decode/verify step, full size
def test_verify_step_full_size():
    s = synth.VERIFY_BF16
    d = synth.make_device_layer(s, seed=0, cfg=2, layer=0, device="cuda")
    torch.cuda.synchronize()
    x, wr = to_host(d.x), to_host(d.wr)
    ref_idx, ref_w, _ = oracle.route(x, wr, s.K)
    out, r = run_layer(d)
    check_routing_and_grouping(r, ref_idx, ref_w, s.E)
    ref_out = oracle.layer_rows(x, ref_idx, ref_w, host_weights(d))
    assert row_rel_err(to_host(out), ref_out) <= TOL_BF16


def test_int4_verify_layer_full_size():
    s = synth.STACK_INT4_VERIFY
    d = synth.make_device_layer(s, seed=0, cfg=5, layer=0, device="cuda")
    torch.cuda.synchronize()
    x, wr = to_host(d.x), to_host(d.wr)
    ref_idx, ref_w, _ = oracle.route(x, wr, s.K)
    out, r = run_layer(d)
    check_routing_and_grouping(r, ref_idx, ref_w, s.E)
    ref_out = oracle.layer_rows(x, ref_idx, ref_w, host_weights(d))
    assert row_rel_err(to_host(out), ref_out) <= TOL_BF16


@pytest.mark.parametrize("shape", [synth.STACK_INT3_VERIFY, synth.STACK_INT2_VERIFY], ids=["int3", "int2"])
def test_lowbit_verify_layer_full_size(shape):
    """A layer of the pruned stack at the verify shape with int3 / int2 experts:
    exact routing, output within the bf16 bound of the oracle on the same
    quantised weights."""
    d = synth.make_device_layer(shape, seed=0, cfg=5, layer=2, device="cuda")
    torch.cuda.synchronize()
    x, wr = to_host(d.x), to_host(d.wr)
    ref_idx, ref_w, _ = oracle.route(x, wr, shape.K)
    out, r = run_layer(d)
    check_routing_and_grouping(r, ref_idx, ref_w, shape.E)
    ref_out = oracle.layer_rows(x, ref_idx, ref_w, host_weights(d))
    assert row_rel_err(to_host(out), ref_out) <= TOL_BF16


def test_int4_prefill_layer_full_size():
    """One layer of the pruned int4 stack on an 8192-token chunk: the grouped
    GEMMs with each weight rounded once to bf16 from its int4 block (sampled rows)."""
    s = synth.STACK_INT4_PREFILL
    d = synth.make_device_layer(s, seed=0, cfg=5, layer=0, device="cuda")
    torch.cuda.synchronize()
    x, wr = to_host(d.x), to_host(d.wr)
    ref_idx, ref_w, _ = oracle.route(x, wr, s.K)
    out, r = run_layer(d)
    check_routing_and_grouping(r, ref_idx, ref_w, s.E)
    rows = np.unique(np.concatenate([[0, s.T - 1], np.random.default_rng(2).choice(s.T, 22, replace=False)]))
    ref_out = oracle.layer_rows(x, ref_idx, ref_w, host_weights(d), rows=rows)
    assert row_rel_err(to_host(out)[rows], ref_out) <= TOL_BF16


# ---------------------------------------------------------------- prefill chunk, full size
def test_prefill_chunk_full_size():
    s = synth.PREFILL_BF16
    d = synth.make_device_layer(s, seed=0, cfg=3, layer=0, device="cuda")
    torch.cuda.synchronize()
    x, wr, bias = to_host(d.x), to_host(d.wr), to_host(d.bias)
    ref_idx, ref_w, ref_lg = oracle.route(x, wr, s.K, bias)
    # the fp32 estimate stays far inside the recheck margin
    ws = torch.empty(moe.route_workspace_size(s.T, s.H, s.E, s.K), dtype=torch.uint8, device="cuda")
    idx, w = moe.route(d.x, d.wr, s.K, bias=d.bias, workspace=ws)
    torch.cuda.synchronize()
    fast = ws[: s.T * s.E * 4].view(torch.float32).view(s.T, s.E).cpu().numpy()
    err = np.abs(fast.astype(np.float64) - ref_lg.astype(np.float64)).max()
    assert err < (1.0 / 4096) / 8, f"fp32 logit estimate error {err}"
    assert np.array_equal(to_host(idx), ref_idx)
    out, r = run_layer(d)
    check_routing_and_grouping(r, ref_idx, ref_w, s.E)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, s.T - 1], rng.choice(s.T, 30, replace=False)]))
    ref_out = oracle.layer_rows(x, ref_idx, ref_w, host_weights(d), rows=rows)
    assert row_rel_err(to_host(out)[rows], ref_out) <= TOL_BF16
    # determinism: a second run is bit-identical
    out2, r2 = run_layer(d)
    assert torch.equal(out, out2) and torch.equal(r["perm"], r2["perm"])


# ---------------------------------------------------------------- pruning statistic
def test_freq_small_with_ties_and_accumulate():
    lg = synth.make_host_logits(3, 1500, 100, seed=1, cfg=4, zipf=True)
    lg[1, :300] = np.round(lg[1, :300])           # exact ties
    lg[2, :50] = 0.0
    K, keep = 10, 40
    ref_c, ref_r, ref_k = oracle.expert_freq(lg, K, keep=keep)
    c, rk, km = moe.expert_freq(torch.from_numpy(lg).cuda(), K, keep=keep)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(c), ref_c) and np.array_equal(to_host(rk), ref_r)
    assert np.array_equal(to_host(km), ref_k)
    c2, _, _ = moe.expert_freq(torch.from_numpy(np.ascontiguousarray(lg[:, :700])).cuda(), K)
    c2, rk2, km2 = moe.expert_freq(torch.from_numpy(np.ascontiguousarray(lg[:, 700:])).cuda(), K, keep=keep,
                                   counts=c2, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(c2), ref_c) and np.array_equal(to_host(km2), ref_k)


def test_freq_threshold_cut_rows_with_ties():
    """Wide rows with several rows per wave, so the threshold cut runs next to
    the full selection: plain Zipf rows, rows on a 0.25 grid (many exact
    ties at the cut), and a layer mixing constant rows (every key equal)
    with ordinary ones and occasional far outliers."""
    L, T, E, K, keep = 3, 40000, 300, 10, 150
    lg = synth.make_host_logits(L, T, E, seed=3, cfg=4, zipf=True)
    lg[1] = np.round(lg[1] * 4.0) / 4.0
    lg[2, ::7] = 1.5
    lg[2, 3::11, 17] = 40.0
    ref_c, ref_r, ref_k = oracle.expert_freq(lg, K, keep=keep)
    c, rk, km = moe.expert_freq(torch.from_numpy(lg).cuda(), K, keep=keep)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(c), ref_c)
    assert np.array_equal(to_host(rk), ref_r) and np.array_equal(to_host(km), ref_k)
    assert np.all(to_host(c).sum(axis=1) == T * K)


def test_freq_full_size_two_layers_and_invariants():
    T, E, K, keep = synth.FREQ_T, synth.FREQ_E, synth.FREQ_K, synth.FREQ_KEEP
    L = 2
    lg = torch.empty((L, T, E), dtype=torch.float32, device="cuda")
    for l in range(L):
        synth.make_device_logits_layer(T, E, seed=0, cfg=4, layer=l, device="cuda", out=lg[l])
    c, rk, km = moe.expert_freq(lg, K, keep=keep)
    torch.cuda.synchronize()
    ref_c, ref_r, ref_k = oracle.expert_freq(lg.cpu().numpy(), K, keep=keep)
    assert np.array_equal(to_host(c), ref_c)
    assert np.array_equal(to_host(rk), ref_r) and np.array_equal(to_host(km), ref_k)
    assert np.all(to_host(c).sum(axis=1) == T * K)


# ---------------------------------------------------------------- expert profile (global ranking, hit rate)
def test_profile_rank_matches_oracle():
    """Global (layer, expert) ranking on the GPU, bit-exact against the oracle:
    small counts (many ties across and within layers), a ragged shape, the
    statistic's 48 x 512, and a single wide layer."""
    from oracle import profile as P
    rng = np.random.default_rng(11)
    cases = [rng.integers(0, 3, size=(7, 300)), rng.integers(0, 50, size=(48, 512)),
             (rng.zipf(1.3, size=(48, 512)) % 100000).astype(np.int64), rng.integers(0, 5, size=(1, 4096)),
             np.zeros((3, 5), dtype=np.int64)]
    for counts in cases:
        rank, pairs = moe.profile_rank(torch.from_numpy(np.ascontiguousarray(counts, dtype=np.int64)).cuda())
        torch.cuda.synchronize()
        ref_pairs, ref_rank = P.global_rank(counts)
        assert np.array_equal(to_host(rank), ref_rank)
        assert np.array_equal(to_host(pairs).view(np.uint16), ref_pairs)


def test_profile_hits_match_oracle():
    """Reads of a routing trace that land on the first S ranked pairs, against
    the oracle, for a profile built from the trace itself and a random one."""
    from oracle import profile as P
    rng = np.random.default_rng(12)
    L, T, K, E = 4, 3000, 10, 256
    bias = -1.1 * np.log1p(rng.permutation(E))
    trace = np.stack([np.argsort(-(rng.standard_normal((T, E)) + bias), axis=1)[:, :K] for _ in range(L)])
    trace = trace.astype(np.int32)
    counts = np.stack([np.bincount(trace[l].reshape(-1), minlength=E) for l in range(L)]).astype(np.int64)
    perm = rng.permutation(L * E)
    rand_counts = np.empty(L * E, dtype=np.int64)
    rand_counts[perm] = np.arange(L * E)[::-1]
    td = torch.from_numpy(trace).cuda()
    for cnt in (counts, rand_counts.reshape(L, E)):
        rank, pairs = moe.profile_rank(torch.from_numpy(cnt).cuda())
        ref_pairs, _ = P.global_rank(cnt)
        for S in (0, 1, 100, 257, L * E):
            h = moe.profile_hits(td, rank, S)
            torch.cuda.synchronize()
            assert int(h.cpu().item()) == P.hits(trace, ref_pairs, S)[0]
