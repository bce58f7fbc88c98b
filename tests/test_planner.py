"""Work-list invariants of the C++ planner, by brute force on small shapes, and
the fp64 emulator running those work lists against the oracle."""
import numpy as np
import pytest

import head_causal_local_amd as aah
import oracle
from emulator import emulate_backward, emulate_forward

CASES = [
    # (B, H, T, windows, q_tile, kv_tile, n_queues)
    (1, 4, 256, [16, 32, 64, 256], 64, 64, 8),
    (2, 3, 100, [1, 7, 1000], 16, 8, 8),
    (1, 5, 37, [1, 2, 5, 36, 37], 8, 16, 3),
    (3, 2, 5, [2, 9], 16, 16, 8),          # T smaller than one tile
    (1, 1, 1, [1], 128, 64, 8),            # a single token
    (2, 6, 130, [64, 65, 128, 129, 3, 1], 32, 32, 8),
]


def _needed_fwd(T, W, rows, kv_tile):
    first = max(0, rows[0] - W + 1)
    last = rows[-1]
    return first // kv_tile, last // kv_tile + 1


@pytest.mark.parametrize("B,H,T,windows,qt_,kt_,nq", CASES)
def test_forward_plan_invariants(B, H, T, windows, qt_, kt_, nq):
    items = aah.plan_fwd(windows, B, H, T, qt_, kt_, nq)
    real = items[items[:, 0] >= 0]
    n_qt = -(-T // qt_)
    # every (bh, query tile) exactly once
    seen = {(int(bh), int(t)) for bh, t, _, _ in real}
    assert len(seen) == len(real) == B * H * n_qt
    for bh, t, lo, hi in real:
        W = min(windows[bh % H], T)
        rows = np.arange(t * qt_, min(T, (t + 1) * qt_))
        # the listed range is exactly the union of the rows' needed key tiles
        assert (lo, hi) == _needed_fwd(T, W, rows, kt_)
        needed = set()
        for i in rows:
            for j in range(max(0, i - W + 1), i + 1):
                needed.add(j // kt_)
        assert needed == set(range(lo, hi))      # contiguous, complete, minimal
    # queue structure: slot s belongs to queue s % nq; heads never split; cost non-increasing
    head_queue = {}
    for s, (bh, t, lo, hi) in enumerate(items):
        if bh < 0:
            continue
        head_queue.setdefault(int(bh), set()).add(s % nq)
    assert all(len(v) == 1 for v in head_queue.values())
    for qi in range(nq):
        q = items[qi::nq]
        costs = [hi - lo for bh, _, lo, hi in q if bh >= 0]
        assert costs == sorted(costs, reverse=True)
        # padding only after the queue's real items
        flags = [bh >= 0 for bh, *_ in q]
        assert flags == sorted(flags, reverse=True)
    assert len(items) % nq == 0


@pytest.mark.parametrize("B,H,T,windows,qt_,kt_,nq", CASES)
def test_backward_plan_invariants(B, H, T, windows, qt_, kt_, nq):
    items = aah.plan_bwd(windows, B, H, T, qt_, kt_, nq)
    real = items[items[:, 0] >= 0]
    n_kt = -(-T // kt_)
    assert len({(int(bh), int(t)) for bh, t, _, _ in real}) == len(real) == B * H * n_kt
    for bh, t, lo, hi in real:
        W = min(windows[bh % H], T)
        keys = range(t * kt_, min(T, (t + 1) * kt_))
        needed = set()
        for j in keys:
            for i in range(j, min(T, j + W)):
                needed.add(i // qt_)
        assert needed == set(range(lo, hi))


def test_plan_rejects_bad_arguments():
    with pytest.raises(aah.AahError):
        aah.plan_fwd([3, 0], 1, 2, 16, 8, 8)
    with pytest.raises(aah.AahError):
        aah.plan_fwd([3], 1, 1, 16, 0, 8)


def test_plan_pairs_cover_window_stats():
    """Tiles listed x tile area >= exact pairs (no in-window pair is dropped)."""
    windows = [512, 1024, 2048, 4096]
    items = aah.plan_fwd(windows, 1, 4, 4096, 128, 64)
    tiles = sum(int(hi - lo) for bh, _, lo, hi in items if bh >= 0)
    pairs, _ = aah.window_stats(windows, 4096)
    assert tiles * 128 * 64 >= pairs
    assert tiles * 128 * 64 < 1.4 * pairs      # and not wildly more


@pytest.mark.parametrize("B,H,T,windows,qt_,kt_,nq", CASES)
def test_emulated_forward_equals_oracle(B, H, T, windows, qt_, kt_, nq):
    rng = np.random.default_rng(21)
    q, k, v = (rng.standard_normal((B, H, T, 8)) for _ in range(3))
    items = aah.plan_fwd(windows, B, H, T, qt_, kt_, nq)
    O, L = emulate_forward(items, q, k, v, windows, 0.4, qt_, kt_)
    Or, Lr = oracle.attn_fwd_ref(q, k, v, windows, 0.4)
    np.testing.assert_allclose(O, Or, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lr, rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,H,T,windows,qt_,kt_,nq", CASES[:4])
def test_emulated_backward_equals_oracle(B, H, T, windows, qt_, kt_, nq):
    rng = np.random.default_rng(22)
    q, k, v, do = (rng.standard_normal((B, H, T, 8)) for _ in range(4))
    _, L = oracle.attn_fwd_ref(q, k, v, windows, 0.4)
    items = aah.plan_bwd(windows, B, H, T, qt_, kt_, nq)
    dq, dk, dv = emulate_backward(items, q, k, v, do, L, windows, 0.4, qt_, kt_)
    rq, rk, rv = oracle.attn_bwd_ref(q, k, v, windows, 0.4, do)
    for a, r in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, r, rtol=0, atol=1e-11)


SINK_CASES = [
    # (B, H, T, windows, sinks, q_tile, kv_tile, n_queues)
    (1, 4, 256, [16, 32, 64, 256], [8, 40, 0, 100], 64, 64, 8),
    (2, 3, 100, [1, 7, 1000], [1, 30, 5], 16, 8, 8),
    (1, 5, 37, [1, 2, 5, 36, 37], [36, 3, 9, 1, 2], 8, 16, 3),
    (1, 2, 300, [20, 128], [128, 17], 32, 64, 8),
]


def _eff_sink(s, w, T):
    return max(0, min(s, T - min(w, T)))


@pytest.mark.parametrize("B,H,T,windows,sinks,qt_,kt_,nq", SINK_CASES)
def test_forward_plan_with_sinks(B, H, T, windows, sinks, qt_, kt_, nq):
    """The listed window range plus the implied sink tiles [0, min(ceil(S / kv), lo)) are exactly
    the key tiles the rows see (brute force over the visibility rule)."""
    items = aah.plan_fwd(windows, B, H, T, qt_, kt_, nq, sinks=sinks)
    real = items[items[:, 0] >= 0]
    assert len({(int(bh), int(t)) for bh, t, _, _ in real}) == len(real) == B * H * -(-T // qt_)
    # the window ranges do not depend on the sinks
    plain = aah.plan_fwd(windows, B, H, T, qt_, kt_, nq)
    assert {tuple(x) for x in plain[plain[:, 0] >= 0]} == {tuple(x) for x in real}
    for bh, t, lo, hi in real:
        h = bh % H
        W, S = min(windows[h], T), _eff_sink(sinks[h], windows[h], T)
        needed = set()
        for i in range(t * qt_, min(T, (t + 1) * qt_)):
            for j in range(i + 1):
                if j > i - W or j < sinks[h]:
                    needed.add(j // kt_)
        n_sink = min(-(-S // kt_), lo)
        assert needed == set(range(n_sink)) | set(range(lo, hi))
    for qi in range(nq):    # queues sorted by visited tiles, sink tiles included
        costs = [hi - lo + min(-(-_eff_sink(sinks[bh % H], windows[bh % H], T) // kt_), lo)
                 for bh, _, lo, hi in items[qi::nq] if bh >= 0]
        assert costs == sorted(costs, reverse=True)


@pytest.mark.parametrize("B,H,T,windows,sinks,qt_,kt_,nq", SINK_CASES)
def test_backward_plan_with_sinks(B, H, T, windows, sinks, qt_, kt_, nq):
    items = aah.plan_bwd(windows, B, H, T, qt_, kt_, nq, sinks=sinks)
    real = items[items[:, 0] >= 0]
    assert len({(int(bh), int(t)) for bh, t, _, _ in real}) == len(real) == B * H * -(-T // kt_)
    for bh, t, lo, hi in real:
        h = bh % H
        W = min(windows[h], T)
        needed = set()
        for j in range(t * kt_, min(T, (t + 1) * kt_)):
            for i in range(j, T):
                if j > i - W or j < sinks[h]:
                    needed.add(i // qt_)
        assert needed == set(range(lo, hi))


@pytest.mark.parametrize("B,H,T,windows,sinks,qt_,kt_,nq", SINK_CASES)
def test_emulated_forward_with_sinks_equals_oracle(B, H, T, windows, sinks, qt_, kt_, nq):
    rng = np.random.default_rng(23)
    q, k, v = (rng.standard_normal((B, H, T, 8)) for _ in range(3))
    items = aah.plan_fwd(windows, B, H, T, qt_, kt_, nq, sinks=sinks)
    O, L = emulate_forward(items, q, k, v, windows, 0.4, qt_, kt_, sinks=sinks)
    Or, Lr = oracle.attn_fwd_ref(q, k, v, windows, 0.4, sinks=sinks)
    np.testing.assert_allclose(O, Or, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lr, rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,H,T,windows,sinks,qt_,kt_,nq", SINK_CASES)
def test_emulated_backward_with_sinks_equals_oracle(B, H, T, windows, sinks, qt_, kt_, nq):
    rng = np.random.default_rng(24)
    q, k, v, do = (rng.standard_normal((B, H, T, 8)) for _ in range(4))
    _, L = oracle.attn_fwd_ref(q, k, v, windows, 0.4, sinks=sinks)
    items = aah.plan_bwd(windows, B, H, T, qt_, kt_, nq, sinks=sinks)
    dq, dk, dv = emulate_backward(items, q, k, v, do, L, windows, 0.4, qt_, kt_, sinks=sinks)
    rq, rk, rv = oracle.attn_bwd_ref(q, k, v, windows, 0.4, do, sinks=sinks)
    for a, r in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, r, rtol=0, atol=1e-11)


def test_plan_rejects_negative_sinks():
    with pytest.raises(aah.AahError):
        aah.plan_fwd([3, 4], 1, 2, 16, 8, 8, sinks=[0, -1])


GQA_CASES = [
    # (B, H, H_kv, T, windows, sinks, q_tile, kv_tile, n_queues)
    (2, 4, 2, 100, [1, 30, 7, 100], None, 16, 32, 8),
    (1, 6, 2, 77, [5, 5, 5, 60, 1, 200], [0, 3, 0, 0, 10, 2], 8, 16, 3),
    (1, 8, 1, 64, [2, 4, 8, 16, 32, 64, 3, 9], None, 16, 16, 8),
]


@pytest.mark.parametrize("B,H,H_kv,T,windows,sinks,qt_,kt_,nq", GQA_CASES)
def test_gqa_plans(B, H, H_kv, T, windows, sinks, qt_, kt_, nq):
    """Forward: the items are those of plain attention, with the G query heads of a key/value group in one queue.
    Backward: one item per (b, key/value head, key tile) whose range is the union of the group's per-head
    ranges."""
    G = H // H_kv
    f = aah.plan_fwd(windows, B, H, T, qt_, kt_, nq, sinks=sinks, H_kv=H_kv)
    plain = aah.plan_fwd(windows, B, H, T, qt_, kt_, nq, sinks=sinks)
    assert {tuple(x) for x in f[f[:, 0] >= 0]} == {tuple(x) for x in plain[plain[:, 0] >= 0]}
    queue_of = {}
    for slot, (bh, _, _, _) in enumerate(f):
        if bh >= 0:
            queue_of.setdefault((bh // H, (bh % H) // G), set()).add(slot % nq)
    assert all(len(v) == 1 for v in queue_of.values())
    b_items = aah.plan_bwd(windows, B, H, T, qt_, kt_, nq, sinks=sinks, H_kv=H_kv)
    real = b_items[b_items[:, 0] >= 0]
    assert len({(int(x[0]), int(x[1])) for x in real}) == len(real) == B * H_kv * -(-T // kt_)
    for bh, kt, lo, hi in real:
        g = bh % H_kv
        need = set()
        for h in range(g * G, (g + 1) * G):
            s = 0 if sinks is None else sinks[h]
            for j in range(kt * kt_, min(T, (kt + 1) * kt_)):
                for i in range(j, T):
                    if j > i - windows[h] or j < s:
                        need.add(i // qt_)
        assert need == set(range(lo, hi))


@pytest.mark.parametrize("B,H,H_kv,T,windows,sinks,qt_,kt_,nq", GQA_CASES)
def test_emulated_gqa_equals_oracle(B, H, H_kv, T, windows, sinks, qt_, kt_, nq):
    rng = np.random.default_rng(25)
    q, do = (rng.standard_normal((B, H, T, 8)) for _ in range(2))
    k, v = (rng.standard_normal((B, H_kv, T, 8)) for _ in range(2))
    f = aah.plan_fwd(windows, B, H, T, qt_, kt_, nq, sinks=sinks, H_kv=H_kv)
    O, L = emulate_forward(f, q, k, v, windows, 0.4, qt_, kt_, sinks=sinks)
    Or, Lr = oracle.attn_fwd_ref(q, k, v, windows, 0.4, sinks=sinks)
    np.testing.assert_allclose(O, Or, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lr, rtol=0, atol=1e-12)
    bi = aah.plan_bwd(windows, B, H, T, qt_, kt_, nq, sinks=sinks, H_kv=H_kv)
    dq, dk, dv = emulate_backward(bi, q, k, v, do, Lr, windows, 0.4, qt_, kt_, sinks=sinks)
    rq, rk, rv = oracle.attn_bwd_ref(q, k, v, windows, 0.4, do, sinks=sinks)
    for a, r in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, r, rtol=0, atol=1e-11)
