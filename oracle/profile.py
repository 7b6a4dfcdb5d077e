"""CPU oracle for the expert profile (test infrastructure only).

The profile is a global ranking of every (layer, expert) pair by how often
the routing selects it; an engine fills its fast-memory expert slots in that
order, and a pruned model's profile is the full one mapped through the list
of kept experts ("Strata Coder 编程模型深度剖析", §3; kwkr.cn Coder write-up,
"专家配置文件：48 x 256 的全量排名" -- its format, construction and hit-rate
check).  Plain numpy and Python; shares nothing with the HIP library.

Readings where the pages leave a detail open:
  * order: count descending, ties to the lower flat index layer * E + expert;
  * STRP v1 layout, little-endian: b"STRP", five uint32 (version = 1, layers,
    experts, ranked pairs, inverse-table entries = layers * experts), the
    ranked pairs as (uint16 layer, uint16 expert), then per layer an
    experts-long int16 inverse table holding each pair's rank or -1;
  * hit rate: the share of routed (token, slot) reads whose (layer, expert)
    pair is among the first S ranked pairs.
"""
from __future__ import annotations

import struct

import numpy as np

MAGIC = b"STRP"
VERSION = 1


def global_rank(counts: np.ndarray):
    """counts [L][E] -> (pairs [L*E][2] uint16 in rank order, rank [L][E] int32)."""
    counts = np.asarray(counts, dtype=np.int64)
    L, E = counts.shape
    flat = counts.reshape(-1)
    idx = np.arange(L * E)
    order = sorted(idx.tolist(), key=lambda i: (-int(flat[i]), i))
    pairs = np.empty((L * E, 2), dtype=np.uint16)
    rank = np.empty(L * E, dtype=np.int32)
    for r, i in enumerate(order):
        pairs[r] = (i // E, i % E)
        rank[i] = r
    return pairs, rank.reshape(L, E)


def inverse_table(pairs: np.ndarray, L: int, E: int) -> np.ndarray:
    """[L][E] int16: the rank of each ranked pair, -1 for the others."""
    inv = np.full((L, E), -1, dtype=np.int16)
    for r, (l, e) in enumerate(np.asarray(pairs).tolist()):
        inv[l, e] = r
    return inv


def strp_bytes(pairs: np.ndarray, L: int, E: int) -> bytes:
    pairs = np.asarray(pairs, dtype=np.uint16).reshape(-1, 2)
    n = pairs.shape[0]
    if n > 32767:
        raise ValueError("int16 inverse table holds ranks below 32768")
    out = bytearray(MAGIC)
    out += struct.pack("<5I", VERSION, L, E, n, L * E)
    for l, e in pairs.tolist():
        out += struct.pack("<HH", l, e)
    for v in inverse_table(pairs, L, E).reshape(-1).tolist():
        out += struct.pack("<h", v)
    return bytes(out)


def strp_parse(buf: bytes):
    """-> (L, E, pairs [n][2] uint16, inverse [L][E] int16); raises on a malformed file."""
    if len(buf) < 24 or buf[:4] != MAGIC:
        raise ValueError("not an STRP file")
    version, L, E, n, entries = struct.unpack_from("<5I", buf, 4)
    if version != VERSION or entries != L * E or len(buf) != 24 + 4 * n + 2 * L * E:
        raise ValueError("inconsistent STRP header")
    pairs = np.array(struct.unpack_from("<%dH" % (2 * n), buf, 24), dtype=np.uint16).reshape(n, 2)
    inv = np.array(struct.unpack_from("<%dh" % (L * E), buf, 24 + 4 * n), dtype=np.int16).reshape(L, E)
    return L, E, pairs, inv


def remap(pairs: np.ndarray, keep_map: np.ndarray) -> np.ndarray:
    """Ranked pairs of an E-expert profile -> ranked pairs of the pruned model:
    expert e of layer l becomes its position in keep_map[l] (the kept ids in
    ascending order); pairs of pruned experts are dropped, the order kept."""
    keep_map = np.asarray(keep_map)
    new_index = [{int(e): j for j, e in enumerate(row)} for row in keep_map]
    out = []
    for l, e in np.asarray(pairs).tolist():
        j = new_index[l].get(e)
        if j is not None:
            out.append((l, j))
    return np.array(out, dtype=np.uint16).reshape(-1, 2)


def hits(trace: np.ndarray, pairs: np.ndarray, S: int):
    """trace [L][T][K] expert ids; -> (hits, reads): reads of the first S ranked pairs."""
    trace = np.asarray(trace)
    L = trace.shape[0]
    resident = set(map(tuple, np.asarray(pairs)[:S].tolist()))
    h = 0
    for l in range(L):
        ids, cnt = np.unique(trace[l], return_counts=True)
        for e, c in zip(ids.tolist(), cnt.tolist()):
            if (l, e) in resident:
                h += c
    return h, int(trace.size)
