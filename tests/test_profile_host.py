"""The expert profile's host-side helpers through the C ABI, on the CPU: the
STRP v1 file (write, read, rejection of malformed files) and the remap of a
profile through a keep list, checked against the oracle (the kwkr.cn Coder
write-up, "专家配置文件：48 x 256 的全量排名")."""
import numpy as np
import pytest

from oracle import profile as P
from routed_expert_ffn_amd import build, moe


@pytest.fixture(scope="module", autouse=True)
def lib():
    import os
    if not os.path.exists(build.LIB):
        build.build()
    return moe.load()


def test_strp_write_read_match_the_oracle():
    rng = np.random.default_rng(7)
    for L, E, n in ((1, 1, 1), (2, 3, 6), (48, 256, 12288), (48, 512, 8000), (5, 11, 0)):
        pairs, _ = P.global_rank(rng.integers(0, 40, size=(L, E)))
        b = moe.strp_write(pairs[:n], L, E)
        assert b == P.strp_bytes(pairs[:n], L, E)
        L2, E2, p2, inv = moe.strp_read(b)
        assert (L2, E2) == (L, E) and np.array_equal(p2, pairs[:n])
        assert np.array_equal(inv, P.inverse_table(pairs[:n], L, E))


def test_strp_rejects_malformed_input():
    pairs, _ = P.global_rank(np.arange(6).reshape(2, 3))
    good = moe.strp_write(pairs, 2, 3)
    for bad in (good[:-1], good + b"\0", b"STRQ" + good[4:], good[:4] + b"\x02" + good[5:]):
        with pytest.raises(moe.MoeError) as ex:
            moe.strp_read(bad)
        assert ex.value.status == 1
    with pytest.raises(moe.MoeError) as ex:          # a pair ranked twice
        moe.strp_write(np.array([[0, 1], [0, 1]], dtype=np.uint16), 2, 3)
    assert ex.value.status == 1
    with pytest.raises(moe.MoeError) as ex:          # expert out of range
        moe.strp_write(np.array([[0, 3]], dtype=np.uint16), 2, 3)
    assert ex.value.status == 1
    big, _ = P.global_rank(np.zeros((64, 600), dtype=np.int64))
    with pytest.raises(moe.MoeError) as ex:          # ranks beyond int16
        moe.strp_write(big[:32768], 64, 600)
    assert ex.value.status == 2


def test_remap_matches_the_oracle():
    rng = np.random.default_rng(8)
    L, E, keep = 48, 512, 256
    counts = rng.integers(0, 1000, size=(L, E))
    pairs, _ = P.global_rank(counts)
    keep_map = np.sort(np.stack([rng.choice(E, keep, replace=False) for _ in range(L)]), axis=1)
    for n in (0, 1, 8000, L * E):
        got = moe.profile_remap(pairs[:n], keep_map, E)
        assert np.array_equal(got, P.remap(pairs[:n], keep_map))
    assert moe.profile_remap(pairs, keep_map, E).shape[0] == L * keep    # a full ranking keeps every kept pair
    with pytest.raises(moe.MoeError) as ex:          # keep list not ascending
        moe.profile_remap(pairs[:10], keep_map[:, ::-1], E)
    assert ex.value.status == 1
