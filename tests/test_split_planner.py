"""The split forward work list (host planner, no GPU) and its fp64 emulation against the oracle.

A split plan must cover exactly the key tiles of the ordinary forward list: every item of more than
chunk_tiles tiles becomes consecutive near-equal chunks with consecutive slots and one merge record, every
other item stays whole and writes its own rows.  Running the split list in fp64 (chunks leave unnormalised
partials, merges combine them) must reproduce the oracle, including rows that see none of a chunk's keys.
"""
import math
from collections import defaultdict

import numpy as np
import pytest

import head_causal_local_amd as aah
import oracle
from emulator import emulate_backward, emulate_forward_split

Q_TILE, KV_TILE = 128, 64

CASES = [
    # windows, B, H, H_kv, T, chunk_tiles
    ([4096, 512, 1024, 2048], 1, 4, 4, 4096, 24),
    ([1, 17, 2999, 5000], 2, 4, 2, 3000, 7),
    ([700, 700], 1, 2, 1, 700, 3),
    ([64, 1], 3, 2, 2, 333, 1),
]


@pytest.mark.parametrize("windows,B,H,H_kv,T,chunk", CASES)
def test_chunks_partition_items(windows, B, H, H_kv, T, chunk):
    base = aah.plan_fwd(windows, B, H, T, Q_TILE, KV_TILE, H_kv=H_kv)
    items, slots, merges = aah.plan_fwd_split(windows, B, H, T, Q_TILE, KV_TILE, chunk, H_kv=H_kv)
    assert len(items) % 8 == 0 and len(slots) == len(items)
    pieces = defaultdict(list)
    for i, (bh, tile, lo, hi) in enumerate(items):
        if bh < 0:
            assert slots[i] == -1
            continue
        pieces[(bh, tile)].append((lo, hi, int(slots[i]), i % 8))
    records = {(int(bh), int(t)): (int(first), int(n)) for bh, t, first, n in merges}
    assert len(records) == len(merges)
    used = []
    n_real = 0
    for bh, tile, lo, hi in base:
        if bh < 0:
            continue
        n_real += 1
        ps = sorted(pieces.pop((int(bh), int(tile))))
        assert ps[0][0] == lo and ps[-1][1] == hi
        assert all(a[1] == b[0] for a, b in zip(ps, ps[1:])), "chunks must be consecutive"
        assert len({p[3] for p in ps}) == 1, "an item's chunks share one queue"
        n = hi - lo
        if n <= chunk:
            assert len(ps) == 1 and ps[0][2] == -1 and (int(bh), int(tile)) not in records
            continue
        k = math.ceil(n / chunk)
        assert len(ps) == k and {p[1] - p[0] for p in ps} <= {n // k, -(-n // k)}
        first, count = records.pop((int(bh), int(tile)))
        assert count == k and [p[2] for p in ps] == list(range(first, first + k))
        used += [p[2] for p in ps]
    assert not pieces and not records, "no item beyond the ordinary list"
    assert sorted(used) == list(range(len(used)))
    # Longest first within each queue, as for the ordinary list.
    for qi in range(8):
        costs = [hi - lo for bh, t, lo, hi in items[qi::8] if bh >= 0]
        assert costs == sorted(costs, reverse=True)


@pytest.mark.parametrize("windows,B,H,H_kv,T,chunk", CASES[1:])
def test_split_emulation_matches_oracle(windows, B, H, H_kv, T, chunk):
    rng = np.random.default_rng(T + chunk)
    d = 8
    q = rng.standard_normal((B, H, T, d))
    k = rng.standard_normal((B, H_kv, T, d))
    v = rng.standard_normal((B, H_kv, T, d))
    scale = 1 / np.sqrt(d)
    items, slots, merges = aah.plan_fwd_split(windows, B, H, T, Q_TILE, KV_TILE, chunk, H_kv=H_kv)
    assert len(merges) > 0
    O, L = emulate_forward_split(items, slots, merges, q, k, v, windows, scale, Q_TILE, KV_TILE)
    Or, Lr = oracle.attn_fwd_ref(q, k, v, windows, scale)
    assert np.abs(O - Or).max() < 1e-12 and np.abs(L - Lr).max() < 1e-12


def test_split_plan_argument_errors():
    with pytest.raises(aah.AahError):
        aah.plan_fwd_split([0, 4], 1, 2, 100, Q_TILE, KV_TILE, 4)
    with pytest.raises(aah.AahError):
        aah.plan_fwd_split([4, 4], 1, 2, 100, Q_TILE, KV_TILE, 0)


BWD_CASES = [
    # windows, B, H, T, chunk_tiles (query tiles of 64 per chunk at most)
    ([4096, 512, 100], 1, 3, 4096, 24),
    ([700, 1, 5000], 2, 3, 700, 2),
    ([64, 300], 1, 2, 333, 1),
]


@pytest.mark.parametrize("windows,B,H,T,chunk", BWD_CASES)
def test_backward_chunks_partition_items(windows, B, H, T, chunk):
    base = aah.plan_bwd(windows, B, H, T, KV_TILE, Q_TILE)
    items, slots, merges = aah.plan_bwd_split(windows, B, H, T, KV_TILE, Q_TILE, chunk)
    pieces = defaultdict(list)
    for i, (bh, kt, lo, hi) in enumerate(items):
        if bh >= 0:
            pieces[(bh, kt)].append((lo, hi, int(slots[i])))
    records = {(int(bh), int(t)): (int(first), int(n)) for bh, t, first, n in merges}
    used = []
    for bh, kt, lo, hi in base:
        if bh < 0:
            continue
        ps = sorted(pieces.pop((int(bh), int(kt))))
        assert ps[0][0] == lo and ps[-1][1] == hi and all(a[1] == b[0] for a, b in zip(ps, ps[1:]))
        n = hi - lo
        if n <= chunk:
            assert len(ps) == 1 and ps[0][2] == -1
            continue
        first, count = records.pop((int(bh), int(kt)))
        assert count == math.ceil(n / chunk) == len(ps) and [p[2] for p in ps] == list(range(first, first + count))
        used += [p[2] for p in ps]
    assert not pieces and not records and sorted(used) == list(range(len(used)))


@pytest.mark.parametrize("windows,B,H,T,chunk", BWD_CASES[1:])
def test_backward_split_emulation_matches_oracle(windows, B, H, T, chunk):
    rng = np.random.default_rng(T + 7 * chunk)
    d = 8
    q, k, v, do = (rng.standard_normal((B, H, T, d)) for _ in range(4))
    scale = 1 / np.sqrt(d)
    items, slots, merges = aah.plan_bwd_split(windows, B, H, T, KV_TILE, Q_TILE, chunk)
    assert len(merges) > 0
    _, lse = oracle.attn_fwd_ref(q, k, v, windows, scale)
    dq, dk, dv = emulate_backward(items, q, k, v, do, lse, windows, scale, KV_TILE, Q_TILE, split=True)
    rq, rk, rv = oracle.attn_bwd_ref(q, k, v, windows, scale, do)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.abs(got - ref).max() < 1e-10
