"""The split work lists (host planner, no GPU) and their fp64 emulation against the oracle.

A split forward plan must cover exactly the key tiles of the ordinary forward list: every item of more than
chunk_tiles window tiles becomes consecutive near-equal chunks with consecutive slots and one merge record,
every other item stays whole and writes its own rows; an item's sink tiles go with its first chunk.  A split
backward plan cuts a key item's query-tile range, for every query head of its key/value group at once, into
consecutive chunks of near-equal steps.  Running the split lists in fp64 (chunks leave unnormalised partials
or partial gradient sums, merges combine them) must reproduce the oracle, including rows that see none of a
chunk's keys, with sink keys ("Autonomy-of-Heads", section 5) and grouped key/value heads.
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
    # windows, B, H, H_kv, T, chunk_tiles, sinks
    ([4096, 512, 1024, 2048], 1, 4, 4, 4096, 24, None),
    ([1, 17, 2999, 5000], 2, 4, 2, 3000, 7, None),
    ([700, 700], 1, 2, 1, 700, 3, None),
    ([64, 1], 3, 2, 2, 333, 1, None),
    # sink keys: sinks past T - W change nothing; a 200-key sink spans four key tiles
    ([1000, 100, 64, 5000], 1, 4, 2, 1100, 3, [200, 4, 130, 8]),
    ([300, 1], 2, 2, 2, 700, 2, [64, 65]),
]


def _eff_sink(sinks, h, W, T):
    return 0 if sinks is None else max(0, min(sinks[h], T - W))


def _fwd_cost(windows, sinks, H, T, bh, tile, lo, hi):
    """Tiles an item visits: its window tiles, and the sink tiles before them for a first chunk."""
    W = min(windows[bh % H], T)
    S = _eff_sink(sinks, bh % H, W, T)
    first = lo == max(0, tile * Q_TILE - W + 1) // KV_TILE
    return hi - lo + (min(-(-S // KV_TILE), lo) if first else 0)


@pytest.mark.parametrize("windows,B,H,H_kv,T,chunk,sinks", CASES)
def test_chunks_partition_items(windows, B, H, H_kv, T, chunk, sinks):
    base = aah.plan_fwd(windows, B, H, T, Q_TILE, KV_TILE, H_kv=H_kv, sinks=sinks)
    items, slots, merges = aah.plan_fwd_split(windows, B, H, T, Q_TILE, KV_TILE, chunk, H_kv=H_kv, sinks=sinks)
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
        costs = [_fwd_cost(windows, sinks, H, T, bh, t, lo, hi) for bh, t, lo, hi in items[qi::8] if bh >= 0]
        assert costs == sorted(costs, reverse=True)


@pytest.mark.parametrize("windows,B,H,H_kv,T,chunk,sinks", CASES[1:])
def test_split_emulation_matches_oracle(windows, B, H, H_kv, T, chunk, sinks):
    rng = np.random.default_rng(T + chunk)
    d = 8
    q = rng.standard_normal((B, H, T, d))
    k = rng.standard_normal((B, H_kv, T, d))
    v = rng.standard_normal((B, H_kv, T, d))
    scale = 1 / np.sqrt(d)
    items, slots, merges = aah.plan_fwd_split(windows, B, H, T, Q_TILE, KV_TILE, chunk, H_kv=H_kv, sinks=sinks)
    assert len(merges) > 0
    O, L = emulate_forward_split(items, slots, merges, q, k, v, windows, scale, Q_TILE, KV_TILE, sinks=sinks)
    Or, Lr = oracle.attn_fwd_ref(q, k, v, windows, scale, sinks=sinks)
    assert np.abs(O - Or).max() < 1e-12 and np.abs(L - Lr).max() < 1e-12


@pytest.mark.parametrize("windows,B,H,H_kv,T,chunk,sinks", [CASES[1], CASES[4]])
def test_split_diagnostics_emulation_matches_oracle(windows, B, H, H_kv, T, chunk, sinks):
    """The split diagnostic forward's merge ("Asymmetric Attention Heads", section 5.3: per-row attention
    entropy and output norm): chunks keep their weighted offsets against their own references, the merge
    moves them to the common one; entropy and norm equal the oracle's rows."""
    rng = np.random.default_rng(2 * T + chunk)
    d = 8
    q = rng.standard_normal((B, H, T, d))
    k = rng.standard_normal((B, H_kv, T, d))
    v = rng.standard_normal((B, H_kv, T, d))
    scale = 1 / np.sqrt(d)
    items, slots, merges = aah.plan_fwd_split(windows, B, H, T, Q_TILE, KV_TILE, chunk, H_kv=H_kv, sinks=sinks)
    assert len(merges) > 0
    O, L, E, N = emulate_forward_split(items, slots, merges, q, k, v, windows, scale, Q_TILE, KV_TILE, sinks=sinks,
                                       diag=True)
    Er, Nr = oracle.attn_row_stats_ref(q, k, v, windows, scale, sinks=sinks)
    assert np.abs(E - Er).max() < 1e-10 and np.abs(N - Nr).max() < 1e-12


def test_split_plan_argument_errors():
    with pytest.raises(aah.AahError):
        aah.plan_fwd_split([0, 4], 1, 2, 100, Q_TILE, KV_TILE, 4)
    with pytest.raises(aah.AahError):
        aah.plan_fwd_split([4, 4], 1, 2, 100, Q_TILE, KV_TILE, 0)
    with pytest.raises(aah.AahError):
        aah.plan_fwd_split([4, 4], 1, 2, 100, Q_TILE, KV_TILE, 4, sinks=[0, -1])
    with pytest.raises(aah.AahError):
        aah.plan_bwd_split([4, 4, 4], 1, 3, 100, KV_TILE, Q_TILE, 4, H_kv=2)


BWD_CASES = [
    # windows, B, H, H_kv, T, chunk_tiles (steps: query tiles of 64, summed over a group's heads), sinks
    ([4096, 512, 100], 1, 3, 3, 4096, 24, None),
    ([700, 1, 5000], 2, 3, 3, 700, 2, None),
    ([64, 300], 1, 2, 2, 333, 1, None),
    # grouped heads: a group's heads end at different query tiles
    ([4096, 512, 100, 1024, 2000, 64], 1, 6, 2, 2048, 9, None),
    ([300, 1, 700, 5], 2, 4, 1, 700, 3, None),
    # sink keys: key tiles that hold a sink run to the last query tile
    ([256, 100, 5000], 1, 3, 3, 1000, 4, [130, 0, 9]),
    ([200, 64, 300, 1], 1, 4, 2, 900, 5, [64, 1000, 0, 10]),
]


def _head_ranges(windows, sinks, H, H_kv, T, g, kt):
    """(lo, [hi_j]) of key tile kt of key/value head g: the query tiles each query head of the group needs
    (mask of section 5.8 with sinks; a key tile holding a sink is seen by every later query)."""
    G = H // H_kv
    k0, k1 = kt * Q_TILE, min(T, (kt + 1) * Q_TILE)
    his = []
    for h in range(g * G, (g + 1) * G):
        W = min(windows[h], T)
        last = T - 1 if k0 < _eff_sink(sinks, h, W, T) else min(T, k1 + W - 1) - 1
        his.append(last // KV_TILE + 1)
    return k0 // KV_TILE, his


@pytest.mark.parametrize("windows,B,H,H_kv,T,chunk,sinks", BWD_CASES)
def test_backward_chunks_partition_items(windows, B, H, H_kv, T, chunk, sinks):
    base = aah.plan_bwd(windows, B, H, T, KV_TILE, Q_TILE, H_kv=H_kv, sinks=sinks)
    items, slots, merges = aah.plan_bwd_split(windows, B, H, T, KV_TILE, Q_TILE, chunk, H_kv=H_kv, sinks=sinks)
    pieces = defaultdict(list)
    for i, (bh, kt, lo, hi) in enumerate(items):
        if bh >= 0:
            pieces[(bh, kt)].append((lo, hi, int(slots[i])))
    records = {(int(bh), int(t)): (int(first), int(n)) for bh, t, first, n in merges}
    used = []
    G = H // H_kv
    for bh, kt, lo, hi in base:
        if bh < 0:
            continue
        lo_ref, his = _head_ranges(windows, sinks, H, H_kv, T, int(bh) % H_kv, int(kt))
        assert lo == lo_ref and hi == max(his)
        ps = sorted(pieces.pop((int(bh), int(kt))))
        assert ps[0][0] == lo and ps[-1][1] == hi and all(a[1] == b[0] for a, b in zip(ps, ps[1:]))
        steps = [sum(max(0, min(c_hi, h_j) - c_lo) for h_j in his) for c_lo, c_hi, _ in ps]
        n = sum(h_j - lo for h_j in his)
        assert sum(steps) == n and min(steps) > 0
        if n <= chunk:
            assert len(ps) == 1 and ps[0][2] == -1
            continue
        first, count = records.pop((int(bh), int(kt)))
        k = math.ceil(n / chunk)
        assert count == len(ps) and [p[2] for p in ps] == list(range(first, first + count))
        assert count == k if G == 1 else count <= k
        assert max(steps) <= -(-n // k) + G - 1
        used += [p[2] for p in ps]
    assert not pieces and not records and sorted(used) == list(range(len(used)))


@pytest.mark.parametrize("windows,B,H,H_kv,T,chunk,sinks", BWD_CASES[1:])
def test_backward_split_emulation_matches_oracle(windows, B, H, H_kv, T, chunk, sinks):
    rng = np.random.default_rng(T + 7 * chunk)
    d = 8
    q, do = (rng.standard_normal((B, H, T, d)) for _ in range(2))
    k, v = (rng.standard_normal((B, H_kv, T, d)) for _ in range(2))
    scale = 1 / np.sqrt(d)
    items, slots, merges = aah.plan_bwd_split(windows, B, H, T, KV_TILE, Q_TILE, chunk, H_kv=H_kv, sinks=sinks)
    assert len(merges) > 0
    _, lse = oracle.attn_fwd_ref(q, k, v, windows, scale, sinks=sinks)
    dq, dk, dv = emulate_backward(items, q, k, v, do, lse, windows, scale, KV_TILE, Q_TILE, sinks=sinks, split=True)
    rq, rk, rv = oracle.attn_bwd_ref(q, k, v, windows, scale, do, sinks=sinks)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.abs(got - ref).max() < 1e-10
