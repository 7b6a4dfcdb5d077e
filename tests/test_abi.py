"""The C ABI library on the CPU: it loads, exports every function that
include/moe.h declares, sizes workspaces, and rejects bad arguments with the
documented status before anything reaches the GPU (no kernel is launched)."""
import ctypes
import os
import re

import pytest

from routed_expert_ffn_amd import build, moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(build.LIB):
        build.build()
    return moe.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_ffn", "moe_combine", "moe_expert_freq"):
        assert n in names


def test_library_exports_every_declared_function(L):
    names = declared_functions()
    assert names == sorted(moe.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", build.LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    assert set(names) <= exported


def test_version_and_status_strings(L):
    assert moe.abi_version() == 1
    assert moe.status_string(0) == "ok"
    assert "workspace" in moe.status_string(3)


def test_workspace_sizes(L):
    assert moe.route_workspace_size(8192, 2048, 512, 10) >= 8192 * 512 * 4
    assert moe.permute_workspace_size(5, 10, 512) > 0
    big = moe.permute_workspace_size(8192, 10, 512)
    assert big >= ((8192 * 10 + 2047) // 2048) * 512 * 4
    assert moe.ffn_workspace_size(8192, 10, 512, 2048, 512, moe.BF16, moe.BF16) >= 81920 * 512 * 2
    assert moe.ffn_workspace_size(32, 4, 64, 256, 128, moe.F32, moe.F32) >= 128 * 128 * 4


FAKE = ctypes.c_void_p(0x10000)   # aligned, never dereferenced: every call below returns before a launch


def test_route_rejects_bad_arguments(L):
    nb = moe.route_workspace_size(4, 64, 8, 2)
    args = lambda **k: dict(dict(x=FAKE, xd=moe.BF16, wr=FAKE, b=None, T=4, H=64, E=8, K=2, idx=FAKE, w=FAKE,  # noqa
                                 lo=None, ws=FAKE, nb=nb), **k)

    def call(a):
        return L.moe_route(a["x"], a["xd"], a["wr"], a["b"], a["T"], a["H"], a["E"], a["K"], a["idx"], a["w"],
                           a["lo"], a["ws"], a["nb"], None)
    assert call(args(x=None)) == moe.MOE_ERR_INVALID_ARG
    assert call(args(K=9)) == moe.MOE_ERR_INVALID_ARG          # K > E
    assert call(args(H=0)) == moe.MOE_ERR_INVALID_ARG
    assert call(args(xd=7)) == moe.MOE_ERR_INVALID_ARG
    assert call(args(K=33, E=64)) == moe.MOE_ERR_UNSUPPORTED
    assert call(args(E=5000, K=2)) == moe.MOE_ERR_UNSUPPORTED
    assert call(args(nb=nb - 1)) == moe.MOE_ERR_WORKSPACE
    assert call(args(ws=None)) == moe.MOE_ERR_WORKSPACE


def test_permute_ffn_combine_freq_reject_bad_arguments(L):
    assert L.moe_permute(None, 5, 10, 512, FAKE, FAKE, FAKE, FAKE, FAKE, 256, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_permute(FAKE, 5, 10, 5000, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_permute(FAKE, 8192, 10, 512, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == moe.MOE_ERR_WORKSPACE
    w = moe.ExpertWeights(moe.BF16, 0x10000, 0x10000, 0x10000, None, None, None)
    nb = moe.ffn_workspace_size(5, 10, 512, 2048, 512, moe.BF16, moe.BF16)
    ffn = lambda *a: L.moe_ffn(*a)  # noqa: E731
    assert ffn(FAKE, moe.BF16, None, FAKE, FAKE, 5, 10, 2048, 512, 512, FAKE, moe.BF16, FAKE, nb, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert ffn(FAKE, moe.BF16, ctypes.byref(w), FAKE, FAKE, 5, 10, 2000, 512, 512, FAKE, moe.BF16, FAKE, nb, None) == \
        moe.MOE_ERR_UNSUPPORTED                                  # H not a multiple of 128
    assert ffn(FAKE, moe.F32, ctypes.byref(w), FAKE, FAKE, 5, 10, 2048, 512, 512, FAKE, moe.F32, FAKE, nb, None) == \
        moe.MOE_ERR_UNSUPPORTED                                  # fp32 x with bf16 weights is not built
    assert ffn(FAKE, moe.BF16, ctypes.byref(w), FAKE, FAKE, 5, 10, 2048, 512, 512, FAKE, moe.BF16, FAKE, nb - 300,
               None) == moe.MOE_ERR_WORKSPACE
    w4 = moe.ExpertWeights(moe.INT4_B32, 0x10000, 0x10000, 0x10000, None, None, None)
    assert ffn(FAKE, moe.BF16, ctypes.byref(w4), FAKE, FAKE, 5, 10, 2048, 512, 512, FAKE, moe.BF16, FAKE, nb, None) == \
        moe.MOE_ERR_INVALID_ARG                                  # int4 needs its scales
    for dt in (moe.INT3_B32, moe.INT2_B32):
        wq = moe.ExpertWeights(dt, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000)
        nq = moe.ffn_workspace_size(9, 10, 256, 2048, 512, moe.BF16, dt)
        assert ffn(FAKE, moe.BF16, ctypes.byref(wq), FAKE, FAKE, 9, 10, 2048, 512, 256, FAKE, moe.BF16, FAKE, nq,
                   None) == moe.MOE_ERR_UNSUPPORTED              # int3 / int2: verify and decode steps only (T <= 8)
        assert ffn(FAKE, moe.BF16, ctypes.byref(wq), FAKE, FAKE, 5, 10, 1024, 512, 256, FAKE, moe.BF16, FAKE, nq,
                   None) == moe.MOE_ERR_UNSUPPORTED              # ... at H 2048, F 512
        wn = moe.ExpertWeights(dt, 0x10000, 0x10000, 0x10000, None, None, None)
        assert ffn(FAKE, moe.BF16, ctypes.byref(wn), FAKE, FAKE, 5, 10, 2048, 512, 256, FAKE, moe.BF16, FAKE, nq,
                   None) == moe.MOE_ERR_INVALID_ARG              # scales required
    assert L.moe_combine(FAKE, moe.BF16, FAKE, FAKE, None, 5, 10, 2044, FAKE, moe.BF16, None) == \
        moe.MOE_ERR_UNSUPPORTED                                  # H % 8
    rg = L.moe_route_group
    nrg = moe.route_group_workspace_size(5, 2048, 512, 10, moe.BF16)
    assert nrg >= moe.route_workspace_size(5, 2048, 512, 10, moe.BF16) + moe.permute_workspace_size(5, 10, 512)
    assert rg(FAKE, moe.BF16, FAKE, None, 5, 2048, 512, 10, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, nrg, None) == \
        moe.MOE_ERR_INVALID_ARG                                  # counts required
    assert rg(FAKE, moe.BF16, FAKE, None, 5, 2048, 512, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, nrg - 1,
              None) == moe.MOE_ERR_WORKSPACE
    assert rg(FAKE, moe.BF16, FAKE, None, 5, 2048, 512, 33, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, nrg, None) == \
        moe.MOE_ERR_UNSUPPORTED                                  # K > 32
    st = L.moe_combine_steer
    assert st(FAKE, moe.BF16, FAKE, FAKE, None, None, 5, 10, 2048, FAKE, moe.BF16, None) == \
        moe.MOE_ERR_INVALID_ARG                                  # the direction is required
    assert st(FAKE, moe.BF16, FAKE, FAKE, None, FAKE, 5, 10, 8200, FAKE, moe.BF16, None) == \
        moe.MOE_ERR_UNSUPPORTED                                  # one row per block: H <= 8192
    assert st(FAKE, moe.BF16, FAKE, FAKE, None, ctypes.c_void_p(0x10004), 5, 10, 2048, FAKE, moe.BF16, None) == \
        moe.MOE_ERR_UNSUPPORTED                                  # misaligned direction
    assert L.moe_combine(None, moe.BF16, FAKE, FAKE, None, 5, 10, 2048, FAKE, moe.BF16, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert L.moe_combine(FAKE, moe.BF16, FAKE, FAKE, ctypes.c_void_p(0x10004), 5, 10, 2048, FAKE, moe.BF16, None) == \
        moe.MOE_ERR_UNSUPPORTED                                  # misaligned residual
    assert L.moe_expert_freq(FAKE, 48, 262144, 512, 10, None, 0, 256, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_expert_freq(FAKE, 48, 262144, 512, 10, FAKE, 0, 513, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_expert_freq(FAKE, 48, 262144, 512, 10, FAKE, 0, 256, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_expert_freq(FAKE, 48, 262144, 512, 40, FAKE, 0, 256, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
