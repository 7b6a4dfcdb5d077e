"""Pins for the CPU oracle: each checks it against something other than itself
(hand-worked examples, closed forms, exact arithmetic, brute force, library
routines, invariants).  CPU only.

The layer's definition: tokens routed to their K highest-logit experts
("Strata Coder 编程模型深度剖析", §1), experts with gate/up/down matrices (§3),
a SwiGLU expert, softmax renormalised over the selected K, ties to the lower
id; the statistic counts selections, ranks and keeps the most-selected
experts listed in original order (§3).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from routed_expert_ffn_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


# ------------------------------------------------------------------ number formats
def test_bf16_rounding_hand_cases(orc):
    assert orc.round_bf16(1.0) == 0x3F80
    assert orc.round_bf16(-2.0) == 0xC000
    assert orc.round_bf16(1.0 + 2.0 ** -8) == 0x3F80            # tie -> even (down)
    assert orc.round_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82        # tie -> even (up)
    assert orc.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81  # one rounding, not via fp32
    assert orc.round_bf16(2.0 ** -133) == 0x0001                # smallest subnormal
    assert orc.round_bf16(2.0 ** -134) == 0x0000                # tie -> even (zero)
    assert orc.round_bf16(1.5 * 2.0 ** -134) == 0x0001
    assert orc.round_bf16(-0.0) == 0x8000
    assert orc.round_bf16(3.3895313892515355e38) == 0x7F7F      # largest finite
    assert orc.round_bf16(3.5e38) == 0x7F80                     # overflow -> inf
    assert orc.bf16_value(0x3F80) == 1.0 and orc.bf16_value(0xC0A0) == -5.0


def test_bf16_rounding_matches_torch_cast(orc):
    # torch's float32 -> bfloat16 cast is round-to-nearest-even: an independent implementation
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(3000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
                        np.float32(1.0) + np.arange(512, dtype=np.float32) * np.float32(2.0 ** -16)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.round_bf16(float(a)) for a in v], dtype=np.uint16)
    assert np.array_equal(got, ref)
    assert np.array_equal(synth.f32_to_bf16_bits(v), ref)


def test_fp16_decode_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.fp16_value(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert orc.fp16_value(0x0001) == 2.0 ** -24 and orc.fp16_value(0x7BFF) == 65504.0


def test_int4_format_and_round_trip(orc):
    # nibble order: element 2j low, 2j+1 high; stored value q+8
    w = np.array([-3.5, 3.5, 0.0, 0.5] + [0.0] * 28, dtype=np.float32)   # max|w| = 3.5 -> d = 0.5
    packed, sc = synth.int4_quantize(w[None, :])
    assert sc[0, 0] == np.float16(0.5)
    # q = (-7, 7, 0, 1) -> nibbles (1, 15, 8, 9) -> bytes 0xF1, 0x98, then 0x88 for zeros
    assert packed[0].tolist()[:3] == [0xF1, 0x98, 0x88]
    assert np.array_equal(orc.int4_dequant(packed, sc)[0], w.astype(np.float64))
    # round trip: values d*q with max |q| = 7 come back bit-exactly
    rng = np.random.default_rng(2)
    qq = rng.integers(-7, 8, size=(6, 64))
    qq[:, 0], qq[:, 32] = 7, -7
    # scales exactly representable in fp16 with 7*d / 7 == d in fp32
    dd = np.array([2.0 ** -7, 3 * 2.0 ** -10, 5 * 2.0 ** -12, 2.0 ** -5, 7 * 2.0 ** -11, 2.0 ** -9], np.float32)
    w2 = qq.astype(np.float32) * dd[:, None]
    p2, s2 = synth.int4_quantize(w2)
    deq2 = orc.int4_dequant(p2, s2)
    assert np.array_equal(deq2, w2.astype(np.float64))
    # an all-zero block has scale 0 and decodes to 0
    p3, s3 = synth.int4_quantize(np.zeros((1, 32), np.float32))
    assert s3[0, 0] == 0 and np.all(orc.int4_dequant(p3, s3) == 0)


def test_int4_numpy_and_torch_quantisers_agree():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((7, 96)) * 0.02).astype(np.float32)
    p, s = synth.int4_quantize(w)
    pt, st = synth.int4_quantize_torch(torch.from_numpy(w))
    assert np.array_equal(p, pt.numpy()) and np.array_equal(s.view(np.uint16), st.numpy().view(np.uint16))


def test_lowbit_formats_hand_bytes(orc):
    """int2 / int3 rows written out by hand from the layout rule (R16): the low
    two bits in 32-bit little-endian words of 16 elements, element 4k + j in
    byte j at bits 2k; int3's third bit in words of 32, element 16g + 4k + j in
    byte j at bit 4g + k; value d (u - 2) or d (u - 4).  The cases separate j
    from k and g, and the two scales of a 64-element row."""
    one, half, two, four = 0x3C00, 0x3800, 0x4000, 0x4400
    cases = [
        # (bits, row bytes, fp16 scales, expected values)
        (2, [0x00, 0x55, 0xAA, 0xFF] * 2, [one], [(i % 4) - 2 for i in range(32)]),
        (2, [0xE4] * 8, [half], [((i % 16) // 4 - 2) * 0.5 for i in range(32)]),
        (2, [0xFF] * 16, [one, two], [1.0] * 32 + [2.0] * 32),
        (3, [0x00, 0x55, 0xAA, 0xFF] * 2 + [0xF0] * 4, [one], [(i % 4) + (4 if i >= 16 else 0) - 4 for i in range(32)]),
        (3, [0x00] * 8 + [0x22] * 4, [one], [0 if (i % 16) // 4 == 1 else -4 for i in range(32)]),
        (3, [0x00] * 8 + [0x00, 0x00, 0xFF, 0x00], [four], [0 if i % 4 == 2 else -16 for i in range(32)]),
    ]
    for bits, row, sc, want in cases:
        packed = np.array([row], np.uint8)
        scales = np.array([sc], np.uint16)
        got = orc.lowbit_dequant(packed, scales, bits)[0]
        assert got.tolist() == [float(v) for v in want], (bits, row)
        # the input generator's packer writes the same bytes for these levels
        d = np.array([orc.fp16_value(v) for v in sc])
        u = np.rint(np.array(want, np.float64) / np.repeat(d, 32)).astype(np.int64) + (1 << (bits - 1))
        assert synth.lowbit_pack_np(u[None, :].astype(np.uint8), bits)[0].tolist() == row


def test_lowbit_round_trip_and_torch_agree(orc):
    rng = np.random.default_rng(11)
    for bits in (2, 3):
        half = 1 << (bits - 1)
        qq = rng.integers(-(half - 1), half, size=(5, 64))   # levels the scale max|w| / (half - 1) reaches exactly
        qq[:, 0], qq[:, 32] = half - 1, -(half - 1)
        dd = np.array([2.0 ** -7, 3 * 2.0 ** -10, 5 * 2.0 ** -12, 2.0 ** -5, 2.0 ** -9], np.float32)
        w = qq.astype(np.float32) * dd[:, None]
        p, sc = synth.lowbit_quantize(w, bits)
        assert p.shape == (5, 64 * bits // 8) and sc.shape == (5, 2)
        assert np.array_equal(orc.lowbit_dequant(p, sc, bits), w.astype(np.float64))
        z = synth.lowbit_quantize(np.zeros((1, 32), np.float32), bits)
        assert z[1][0, 0] == 0 and np.all(orc.lowbit_dequant(*z, bits) == 0)
        r = (rng.standard_normal((4, 96)) * 0.02).astype(np.float32)
        pn, sn = synth.lowbit_quantize(r, bits)
        pt, st = synth.lowbit_quantize_torch(torch.from_numpy(r), bits)
        assert np.array_equal(pn, pt.numpy()) and np.array_equal(sn.view(np.uint16), st.numpy().view(np.uint16))
        # every value within half a step of its block's scale
        deq = orc.lowbit_dequant(pn, sn, bits)
        step = np.repeat(sn.astype(np.float64), 32, axis=1)
        assert np.all(np.abs(deq - r) <= 0.5 * step * (1 + 1e-3))


# ------------------------------------------------------------------ a1: router logits
def _nearest_f32(fr: Fraction) -> np.float32:
    """Correctly rounded fp32 of an exact rational (ties to even), by exact comparison."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - fr), int(np.array(v).view(np.uint32)) & 1))
    return best


def test_logits_unit_vector_rows_exact(orc):
    # Wr rows = scaled unit vectors: every order of summation gives the chosen component exactly
    H, E = 128, 8
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, H)).astype(np.float32)
    wr = np.zeros((E, H), np.float32)
    cols = rng.choice(H, E, replace=False)
    for e, c in enumerate(cols):
        wr[e, c] = np.float32(2.0 ** (e - 3))
    got = orc.router_logits(x, wr)
    assert np.array_equal(got, (x[:, cols] * wr[np.arange(E), cols]).astype(np.float32))


def test_logits_close_to_exact_sum(orc):
    # fp32 of an fp64 sum vs the correctly rounded exact sum: equal except at rare
    # rounding-boundary cases, and never more than one fp32 ulp apart
    rng = np.random.default_rng(5)
    T, H, E = 4, 160, 6
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    xv = synth.bf16_bits_to_f32(x)
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    got = orc.router_logits(x, wr)
    same = 0
    for t in range(T):
        for e in range(E):
            ex = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xv[t], wr[e]))
            ref = _nearest_f32(ex)
            diff = abs(int(np.array(got[t, e]).view(np.int32)) - int(np.array(ref).view(np.int32)))
            assert diff <= 1
            same += diff == 0
    assert same >= T * E - 1


def test_logits_wave64_summation_order(orc):
    # Constructed so that the fixed order is visible:  products p with
    # p[0]=2^53, p[64]=-2^53, p[1]=1 : 64 strided partial sums give P_0 = 0, P_1 = 1
    # -> S = 1, while a left-to-right sum gives ((2^53 + 1) -> 2^53) - 2^53 = 0.
    H = 128
    x = np.zeros((3, H), np.float32)
    x[0, 0], x[0, 64], x[0, 1] = 2.0 ** 53, -(2.0 ** 53), 1.0
    # tree pairing P_j += P_{j+32} before +16: p[0]=2^53, p[32]=-2^53, p[16]=p[48]=1
    # -> tree: P_0 = 0, P_16 = 2, S = 2;  left-to-right: 2^53+1 -> 2^53, -2^53 -> 0, +1 -> 1
    x[1, 0], x[1, 32], x[1, 16], x[1, 48] = 2.0 ** 53, -(2.0 ** 53), 1.0, 1.0
    # neighbour pairing would pair (0,1): p[0]=2^53, p[1]=1, p[32]=-2^53 -> tree: P_0 = 0 after +32,
    # then P_0 += P_1 -> 1; left-to-right: 0
    x[2, 0], x[2, 1], x[2, 32] = 2.0 ** 53, 1.0, -(2.0 ** 53)
    wr = np.ones((1, H), np.float32)
    got = orc.router_logits(x, wr)[:, 0]
    assert got.tolist() == [1.0, 2.0, 1.0]


def test_logits_bias_added_in_fp32(orc):
    x = np.array([[1.0, 0.0]], np.float32)
    wr = np.array([[np.float32(1.0) + np.float32(2.0 ** -23)], [1.0]], np.float32).reshape(2, 1)
    wr = np.concatenate([wr, np.zeros((2, 1), np.float32)], axis=1)
    b = np.array([np.float32(2.0 ** -24), np.float32(3.0)], np.float32)
    got = orc.router_logits(x, wr, b)
    assert got[0, 0] == np.float32(np.float32(1.0 + 2.0 ** -23) + np.float32(2.0 ** -24))
    assert got[0, 1] == np.float32(4.0)


# ------------------------------------------------------------------ a2: selection and weights
def _brute_topk(lg, K):
    order = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def test_topk_matches_stable_sort_with_many_ties(orc):
    rng = np.random.default_rng(6)
    lg = (np.round(rng.standard_normal((400, 37)) * 4) / 4).astype(np.float32)   # heavy ties
    lg[:50] = 0.0
    lg[50:60, ::2] = -0.0
    for K in (1, 3, 10, 37):
        idx = orc.topk(lg, K, weights=False)
        assert np.array_equal(idx, _brute_topk(lg, K))


def test_topk_special_cases(orc):
    idx, w = orc.topk(np.zeros((2, 16), np.float32), 5)
    assert np.array_equal(idx, np.tile(np.arange(5), (2, 1)))
    assert np.allclose(w, 0.2, rtol=0, atol=1e-7)
    lg = np.array([[0.5, -1.0, 3.0, 3.0, 2.0]], np.float32)
    idx, _ = orc.topk(lg, 5)
    assert idx.tolist() == [[2, 3, 4, 0, 1]]
    idx, _ = orc.topk(np.array([[-0.0, 0.0, 0.0]], np.float32), 2)
    assert idx.tolist() == [[0, 1]]
    with pytest.raises(RuntimeError):
        orc.topk(np.array([[1.0, np.nan]], np.float32), 1)


def test_weights_equal_full_softmax_restricted(orc):
    rng = np.random.default_rng(7)
    lg = (rng.standard_normal((200, 64)) * 2).astype(np.float32)
    K = 6
    idx, w = orc.topk(lg, K)
    p = torch.softmax(torch.from_numpy(lg.astype(np.float64)), dim=1).numpy()
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    ref = sel / sel.sum(axis=1, keepdims=True)
    assert np.max(np.abs(w - ref) / ref) < 1e-6
    assert np.max(np.abs(w.astype(np.float64).sum(axis=1) - 1.0)) < 1e-6
    assert np.all(np.diff(w, axis=1) <= 0)     # weights follow the descending logit order


def test_hand_examples_routing(orc):
    g = GOLD["H1"]
    x = np.array(g["x"], np.float32)
    wr = np.array(g["wr"], np.float32)
    assert np.array_equal(orc.router_logits(x, wr), np.array(g["logits"], np.float32))
    for name in ("H1", "H2"):
        K = GOLD[name]["K"]
        idx, w, _ = orc.route(x, wr, K)
        assert idx.tolist() == GOLD[name]["idx"]
        assert np.allclose(w, np.array(GOLD[name]["w"]), rtol=1e-7, atol=0)
    h3 = GOLD["H3"]
    for k, key in ((1, "K1"), (2, "K2")):
        idx, w, _ = orc.route(np.array(h3["x"], np.float32), np.array(h3["wr"], np.float32), k)
        assert idx.tolist() == h3[key]["idx"] and np.allclose(w, h3[key]["w"], rtol=1e-7, atol=0)


# ------------------------------------------------------------------ a3: grouping
def test_permute_hand_examples(orc):
    for name in ("H1", "H2"):
        g = GOLD[name]
        counts, offsets, perm, inv = orc.permute(np.array(g["idx"], np.int32), 2)
        assert counts.tolist() == g["counts"] and offsets.tolist() == g["offsets"]
        assert perm.tolist() == g["perm"] and inv.tolist() == g["inv"]


@pytest.mark.parametrize("T,K,E", [(1, 1, 1), (37, 4, 64), (500, 10, 512), (3, 8, 8)])
def test_permute_invariants_and_brute_force(orc, T, K, E):
    rng = np.random.default_rng(T * 1000 + K)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = orc.permute(idx, E)
    flat = idx.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[-1] == T * K
    assert np.array_equal(np.sort(perm), np.arange(T * K))
    assert np.array_equal(inv[perm], np.arange(T * K))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0) and np.all(flat[seg] == e)


# ------------------------------------------------------------------ a4 + a5: the layer
def _dense_brute_force(x, wr, bias, K, wg, wu, wd, round_a=None):
    """Every expert on every token, then mask with the top-K weights (fp64, torch CPU)."""
    X = torch.from_numpy(x.astype(np.float64))
    lg = np.asarray(X @ torch.from_numpy(wr.astype(np.float64)).T, dtype=np.float64)
    if bias is not None:
        lg = lg + bias
    T, E = lg.shape
    order = np.argsort(-lg, axis=1, kind="stable")[:, :K]
    p = torch.softmax(torch.from_numpy(lg), dim=1).numpy()
    mask = np.zeros((T, E))
    np.put_along_axis(mask, order, 1.0, axis=1)
    wfull = p * mask
    wfull /= wfull.sum(axis=1, keepdims=True)
    out = torch.zeros(T, wd.shape[1], dtype=torch.float64)
    for e in range(E):
        g = X @ torch.from_numpy(wg[e].astype(np.float64)).T
        u = X @ torch.from_numpy(wu[e].astype(np.float64)).T
        a = torch.nn.functional.silu(g) * u
        if round_a is not None:
            a = round_a(a)
        y = a @ torch.from_numpy(wd[e].astype(np.float64)).T
        out += torch.from_numpy(wfull[:, e:e + 1]) * y
    return out.numpy(), order


def test_hand_examples_layer(orc):
    g = GOLD["H1"]
    x = np.array(g["x"], np.float32)
    wr = np.array(g["wr"], np.float32)
    W = orc.Weights("f32", np.array(g["wg"], np.float32), np.array(g["wu"], np.float32),
                    np.array(g["wd"], np.float32))
    for name in ("H1", "H2"):
        K = GOLD[name]["K"]
        idx, w, _ = orc.route(x, wr, K)
        out = orc.layer_rows(x, idx, w, W)
        assert np.allclose(out, np.array(GOLD[name]["out"]), rtol=2e-7, atol=1e-7)


def test_layer_equals_dense_brute_force_fp32(orc):
    s = synth.TINY_FP32
    L = synth.make_host_layer(s, seed=0, cfg=1)
    idx, w, _ = orc.route(L.x, L.wr, s.K)
    out = orc.layer_rows(L.x, idx, w, orc.Weights("f32", L.wg, L.wu, L.wd))
    ref, order = _dense_brute_force(L.x, L.wr, None, s.K, L.wg, L.wu, L.wd)
    assert np.array_equal(idx, order)
    rel = np.abs(out - ref).max(axis=1) / np.abs(ref).max(axis=1)
    assert rel.max() < 1e-6


def test_layer_equals_dense_brute_force_bf16_zipf(orc):
    s = synth.LayerShape(T=24, H=128, E=16, K=3, F=64, act="bf16", wdt="bf16", zipf=True)
    L = synth.make_host_layer(s, seed=0, cfg=9)
    idx, w, _ = orc.route(L.x, L.wr, s.K, L.bias)
    out = synth.bf16_bits_to_f32(orc.layer_rows(L.x, idx, w, orc.Weights("bf16", L.wg, L.wu, L.wd)))
    xv = synth.bf16_bits_to_f32(L.x)
    wgv, wuv, wdv = (synth.bf16_bits_to_f32(a) for a in (L.wg, L.wu, L.wd))
    rb = lambda a: a.to(torch.float32).to(torch.bfloat16).to(torch.float64)  # noqa: E731
    ref, order = _dense_brute_force(xv, L.wr, L.bias.astype(np.float64), s.K, wgv, wuv, wdv, round_a=rb)
    assert np.array_equal(idx, order)
    rel = np.abs(out - ref).max(axis=1) / np.abs(ref).max(axis=1)
    assert rel.max() < 2 ** -7     # output rounding to bf16, plus rare double rounding of a in ref


def test_single_expert_is_textbook_swiglu(orc):
    rng = np.random.default_rng(8)
    H, F = 64, 32
    x = rng.standard_normal((3, H)).astype(np.float32)
    wg, wu = (rng.standard_normal((1, F, H)) * 0.1).astype(np.float32), (rng.standard_normal((1, F, H)) * 0.1).astype(np.float32)
    wd = (rng.standard_normal((1, H, F)) * 0.1).astype(np.float32)
    idx, w, _ = orc.route(x, np.ones((1, H), np.float32), 1)
    assert np.all(idx == 0) and np.all(w == 1.0)
    out = orc.layer_rows(x, idx, w, orc.Weights("f32", wg, wu, wd))
    lin = lambda W: torch.nn.Linear(W.shape[1], W.shape[0], bias=False, dtype=torch.float64)  # noqa: E731
    gate, up, down = lin(wg[0]), lin(wu[0]), lin(wd[0])
    with torch.no_grad():
        gate.weight.copy_(torch.from_numpy(wg[0].astype(np.float64)))
        up.weight.copy_(torch.from_numpy(wu[0].astype(np.float64)))
        down.weight.copy_(torch.from_numpy(wd[0].astype(np.float64)))
        X = torch.from_numpy(x.astype(np.float64))
        ref = down(torch.nn.functional.silu(gate(X)) * up(X)).numpy()
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-7)


def test_zero_input_and_one_hot(orc):
    s = synth.LayerShape(T=4, H=64, E=8, K=2, F=32, act="f32", wdt="f32")
    L = synth.make_host_layer(s, seed=1, cfg=9)
    z = np.zeros_like(L.x)
    idx, w, _ = orc.route(z, L.wr, 2)
    W = orc.Weights("f32", L.wg, L.wu, L.wd)
    assert np.all(orc.layer_rows(z, idx, w, W) == 0)
    # residual passes through when the experts contribute nothing
    res = np.arange(4 * 64, dtype=np.float32).reshape(4, 64)
    assert np.array_equal(orc.layer_rows(z, idx, w, W, residual=res), res)
    # K=1: weight 1, output is exactly that expert's FFN
    idx1, w1, _ = orc.route(L.x, L.wr, 1)
    out = orc.layer_rows(L.x, idx1, w1, W)
    for t in range(4):
        assert np.array_equal(out[t], orc.expert_ffn(L.x[t], W, int(idx1[t, 0])).astype(np.float32))


def test_int4_path_equals_fp32_path_on_dequantised_weights(orc):
    s = synth.LayerShape(T=6, H=64, E=4, K=2, F=64, act="bf16", wdt="int4")
    L = synth.make_host_layer(s, seed=2, cfg=9)
    idx, w, _ = orc.route(L.x, L.wr, 2)
    W4 = orc.Weights("int4", L.wg, L.wu, L.wd, L.sg, L.su, L.sd)

    def deq(p, sc):   # independent numpy decode of the storage format
        q = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.float64)
        q[..., 0::2] = (p & 15).astype(np.float64) - 8
        q[..., 1::2] = (p >> 4).astype(np.float64) - 8
        return (q.reshape(*q.shape[:-1], -1, 32) * sc.astype(np.float64)[..., None]).reshape(q.shape)
    Wf = orc.Weights("f32", *(deq(p, sc).astype(np.float32) for p, sc in ((L.wg, L.sg), (L.wu, L.su), (L.wd, L.sd))))
    for p, sc in ((L.wg, L.sg), (L.wd, L.sd)):
        assert np.array_equal(deq(p, sc)[0], orc.int4_dequant(p[0], sc[0]))
    a = orc.layer_rows(L.x, idx, w, W4)
    b = orc.layer_rows(L.x, idx, w, Wf)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("wdt", ["int3", "int2"])
def test_lowbit_path_equals_fp32_path_on_dequantised_weights(orc, wdt):
    s = synth.LayerShape(T=6, H=64, E=4, K=2, F=64, act="bf16", wdt=wdt)
    L = synth.make_host_layer(s, seed=2, cfg=9)
    idx, w, _ = orc.route(L.x, L.wr, 2)
    Wq = orc.Weights(wdt, L.wg, L.wu, L.wd, L.sg, L.su, L.sd)
    bits = synth.LOWBIT[wdt]
    Wf = orc.Weights("f32", *(orc.lowbit_dequant(p.reshape(-1, p.shape[-1]), sc.reshape(-1, sc.shape[-1]), bits)
                              .reshape(p.shape[:-1] + (p.shape[-1] * 8 // bits,)).astype(np.float32)
                              for p, sc in ((L.wg, L.sg), (L.wu, L.su), (L.wd, L.sd))))
    a = orc.layer_rows(L.x, idx, w, Wq)
    b = orc.layer_rows(L.x, idx, w, Wf)
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ a6: pruning statistic
def test_freq_hand_examples(orc):
    f1 = GOLD["F1"]
    counts, rank_of, keep_map = orc.expert_freq(np.array(f1["logits"], np.float32), f1["K"], keep=f1["keep"])
    assert counts.tolist() == f1["counts"] and rank_of.tolist() == f1["rank_of"]
    assert keep_map.tolist() == f1["keep_map"]
    f2 = GOLD["F2"]
    r, k2 = orc.rank_keep(np.array(f2["counts"], np.int64), 2)
    assert r.tolist() == f2["rank_of"] and k2.tolist() == f2["keep2"]
    _, k3 = orc.rank_keep(np.array(f2["counts"], np.int64), 3)
    assert k3.tolist() == f2["keep3"]


def test_freq_closed_form_rotation(orc):
    # l[t][e] = -((e - t) mod E)  =>  top-K = {t, ..., t+K-1 mod E}  =>  counts = T*K/E each
    L, T, E, K = 2, 96, 32, 5
    t = np.arange(T)[:, None]
    e = np.arange(E)[None, :]
    lg = np.broadcast_to(-((e - t) % E).astype(np.float32), (L, T, E)).copy()
    counts, rank_of, keep_map = orc.expert_freq(lg, K, keep=8)
    assert np.all(counts == T * K // E)
    assert np.array_equal(rank_of, np.tile(np.arange(E), (L, 1)))      # all equal -> rank = id
    assert np.array_equal(keep_map, np.tile(np.arange(8), (L, 1)))


def test_freq_brute_force_and_accumulate(orc):
    lg = synth.make_host_logits(3, 700, 64, seed=0, cfg=3, zipf=True)
    lg[0, :20] = np.round(lg[0, :20])                # exact ties
    K, keep = 10, 32
    counts, rank_of, keep_map = orc.expert_freq(lg, K, keep=keep)
    for l in range(3):
        sel = _brute_topk(lg[l], K)
        c = np.bincount(sel.reshape(-1), minlength=64)
        assert np.array_equal(counts[l], c) and counts[l].sum() == 700 * K
        order = np.lexsort((np.arange(64), -c))
        r = np.empty(64, np.int64)
        r[order] = np.arange(64)
        assert np.array_equal(rank_of[l], r)
        assert np.array_equal(keep_map[l], np.sort(order[:keep]))
    # chunked calibration: two halves accumulated equal one pass
    c2, _, _ = orc.expert_freq(lg[:, :300], K)
    c2, r2, k2 = orc.expert_freq(lg[:, 300:], K, keep=keep, counts=c2, accumulate=True)
    assert np.array_equal(c2, counts) and np.array_equal(r2, rank_of) and np.array_equal(k2, keep_map)


def test_zipf_bias_is_log_zipf():
    b = synth.zipf_bias_np(512, 0, 3, 0)
    r = np.sort(-b / 1.1)                                # = ln(1 + pi(e)) sorted
    assert np.allclose(np.exp(r) - 1, np.arange(512), atol=1e-3)
    assert math.isclose(float(b.max()), 0.0, abs_tol=0.0)


def test_bf16_rounding_point_of_the_swiglu_product(orc):
    # a = silu(g) * u is rounded to bf16 before the down projection (bf16 activations).
    # g = (4, 4.0625), u = (1, 1), down row (-1, 1):  silu(4) = 3.92806 -> bf16 3.921875,
    # silu(4.0625) = 3.99378 -> bf16 4.0, so y = 4.0 - 3.921875 = 0.078125 exactly;
    # without that rounding y would be 0.0657.
    bf = lambda v: synth.f32_to_bf16_bits(np.array(v, np.float32))  # noqa: E731
    x = bf([[1.0, 0.0]])
    wg = bf([[[4.0, 0.0], [4.0625, 0.0]]])
    wu = bf([[[1.0, 0.0], [1.0, 0.0]]])
    wd = bf([[[-1.0, 1.0], [0.0, 0.0]]])
    out = orc.layer_rows(x, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32),
                         orc.Weights("bf16", wg, wu, wd))
    assert synth.bf16_bits_to_f32(out).tolist() == [[0.078125, 0.0]]


# ------------------------------------------------------------------ expert profile (global ranking, STRP, remap, hits)
def _prof():
    from oracle import profile
    return profile


def test_profile_rank_brute_force_and_ties():
    """Rank = number of pairs strictly ahead under (count desc, flat index asc),
    counted pair by pair, on tiny inputs with many equal counts."""
    P = _prof()
    rng = np.random.default_rng(3)
    for L, E in ((1, 1), (2, 3), (3, 5), (4, 7)):
        counts = rng.integers(0, 4, size=(L, E))
        pairs, rank = P.global_rank(counts)
        for l in range(L):
            for e in range(E):
                ahead = sum(1 for l2 in range(L) for e2 in range(E)
                            if counts[l2, e2] > counts[l, e] or (counts[l2, e2] == counts[l, e] and (l2, e2) < (l, e)))
                assert rank[l, e] == ahead
                assert tuple(pairs[ahead]) == (l, e)
    # invariants on a statistic-sized case: a permutation, counts non-increasing along the ranking
    counts = rng.integers(0, 50, size=(48, 64))
    pairs, rank = P.global_rank(counts)
    assert sorted(rank.reshape(-1).tolist()) == list(range(48 * 64))
    seq = [counts[l, e] for l, e in pairs.tolist()]
    assert all(a >= b for a, b in zip(seq, seq[1:]))


def test_strp_hand_example_bytes():
    """STRP v1 written out by hand for 2 layers x 3 experts (counts 5 0 2 / 2 7 0)."""
    P = _prof()
    pairs, _ = P.global_rank(np.array([[5, 0, 2], [2, 7, 0]]))
    # order: (1,1)=7, (0,0)=5, (0,2)=2, (1,0)=2, (0,1)=0, (1,2)=0
    expect = (b"STRP" + bytes([1, 0, 0, 0, 2, 0, 0, 0, 3, 0, 0, 0, 6, 0, 0, 0, 6, 0, 0, 0])
              + bytes([1, 0, 1, 0, 0, 0, 0, 0, 0, 0, 2, 0, 1, 0, 0, 0, 0, 0, 1, 0, 1, 0, 2, 0])
              + bytes([1, 0, 4, 0, 2, 0, 3, 0, 0, 0, 5, 0]))
    assert P.strp_bytes(pairs, 2, 3) == expect
    L, E, p2, inv = P.strp_parse(expect)
    assert (L, E) == (2, 3) and np.array_equal(p2, pairs)
    assert inv.tolist() == [[1, 4, 2], [3, 0, 5]]
    with pytest.raises(ValueError):
        P.strp_parse(expect[:-2])
    with pytest.raises(ValueError):
        P.strp_parse(b"STRQ" + expect[4:])


def test_strp_round_trip_and_unranked_entries():
    P = _prof()
    rng = np.random.default_rng(4)
    pairs, _ = P.global_rank(rng.integers(0, 9, size=(5, 11)))
    part = pairs[:20]                                   # a profile may rank only some pairs
    L, E, p2, inv = P.strp_parse(P.strp_bytes(part, 5, 11))
    assert np.array_equal(p2, part)
    assert int((inv >= 0).sum()) == 20 and int((inv == -1).sum()) == 55 - 20
    for r, (l, e) in enumerate(part.tolist()):
        assert inv[l, e] == r


def test_profile_remap_keeps_order_and_drops_pruned():
    """A 512-space profile through the keep list: every surviving pair is a kept
    expert at its position in the list, ranks keep their order, and the number
    of survivors is the number of ranked pairs whose expert is kept."""
    P = _prof()
    rng = np.random.default_rng(5)
    L, E, keep = 4, 16, 8
    counts = rng.integers(0, 30, size=(L, E))
    pairs, rank = P.global_rank(counts)
    keep_map = np.sort(np.stack([rng.choice(E, keep, replace=False) for _ in range(L)]), axis=1)
    top = pairs[:40]
    out = P.remap(top, keep_map)
    kept = [(l, e) for l, e in top.tolist() if e in set(keep_map[l].tolist())]
    assert len(out) == len(kept)
    for (l, j), (l0, e0) in zip(out.tolist(), kept):
        assert l == l0 and keep_map[l, j] == e0
    # a keep list of everything is the identity; of nothing leaves an empty profile
    assert np.array_equal(P.remap(top, np.tile(np.arange(E), (L, 1))), top)
    assert P.remap(top, np.zeros((L, 0), dtype=np.int64)).shape == (0, 2)


def test_profile_hit_rate_closed_forms():
    """Hit rate of the first S ranked pairs on a trace: a profile built from the
    trace's own counts reaches the sum of the S largest counts (the most any S
    pairs can); random profiles average S / (L E); S = 0 and S = L E give 0 and 1."""
    P = _prof()
    rng = np.random.default_rng(6)
    L, T, K, E = 3, 200, 4, 16
    bias = -1.1 * np.log1p(np.arange(E))
    trace = np.stack([np.argsort(-(rng.standard_normal((T, E)) + bias), axis=1)[:, :K] for _ in range(L)])
    counts = np.stack([np.bincount(trace[l].reshape(-1), minlength=E) for l in range(L)])
    pairs, _ = P.global_rank(counts)
    for S in (0, 1, 5, 17, L * E):
        h, n = P.hits(trace, pairs, S)
        assert n == L * T * K
        assert h == int(np.sort(counts.reshape(-1))[::-1][:S].sum())
    assert P.hits(trace, pairs, L * E)[0] == L * T * K
    S, acc = 12, []
    for _ in range(400):
        perm = rng.permutation(L * E)
        rp = np.stack([perm // E, perm % E], axis=1).astype(np.uint16)
        acc.append(P.hits(trace, rp, S)[0] / (L * T * K))
    assert abs(np.mean(acc) - S / (L * E)) < 0.01


# ------------------------------------------------------------------ steered combine
def test_steer_projection_closed_forms():
    """h - (h.v) v for a unit v: orthogonal to v, idempotent, no change for v
    orthogonal to h, the j-th coordinate zeroed for v = e_j, the same for -v,
    never longer than h; the combine part is a plain weighted gather."""
    from oracle import steer as St
    rng = np.random.default_rng(9)
    T, H = 6, 96
    h = rng.standard_normal((T, H))
    v = rng.standard_normal(H)
    v /= np.linalg.norm(v)
    p = St.project_out(h, v)
    assert np.max(np.abs(p @ v)) < 1e-12 * np.max(np.abs(h))
    assert np.allclose(St.project_out(p, v), p, rtol=0, atol=1e-13)
    assert np.array_equal(St.project_out(h, -v), p) or np.allclose(St.project_out(h, -v), p, rtol=0, atol=1e-14)
    assert np.all(np.linalg.norm(p, axis=1) <= np.linalg.norm(h, axis=1) + 1e-12)
    e = np.zeros(H); e[7] = 1.0
    pe = St.project_out(h, e)
    assert np.all(pe[:, 7] == 0) and np.array_equal(np.delete(pe, 7, axis=1), np.delete(h, 7, axis=1))
    u = np.zeros(H); u[3] = 1.0
    hz = h.copy(); hz[:, 3] = 0.0
    assert np.array_equal(St.project_out(hz, u), hz)
    # combine: two tokens, K = 2, hand-worked
    y = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0]])
    inv = np.array([2, 0, 1, 3])
    w = np.array([[0.5, 0.25], [1.0, -1.0]])
    res = np.array([[0.0, 1.0], [2.0, 0.0]])
    assert St.combine_rows(y, inv, w, res).tolist() == [[2.75, 4.5], [-2.0, -4.0]]
