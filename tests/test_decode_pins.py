"""Pins of the decoding oracle (oracle/decode.py) against facts that do not come from it.

A library routine (torch scaled_dot_product_attention and scipy logsumexp in float64 on
the CPU, over exactly the keys the definition names), the forward definition's row at the
same position, closed forms (one key, identical keys), an invariant (key order), and a
brute-force replay of the cache's storage rule.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle


def _hist(B, H, L, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, L, d)) for _ in range(3)]


def test_decode_equals_sdpa_over_window_keys():
    """Library routine: one query, the keys max(0, p - C + 1) .. p, no mask."""
    B, H, L, d = 2, 3, 40, 8
    qh, kh, vh = _hist(B, H, L, d, 1)
    windows, T_max, scale = [1, 7, 100], 32, 0.37
    pos = np.array([5, 31])
    q = qh[np.arange(B), :, pos]                       # [B, H, d]
    o, lse = oracle.decode_ref(q, kh, vh, windows, pos, T_max, scale)
    for b in range(B):
        for h, w in enumerate(windows):
            c = min(w, T_max)
            lo = max(0, pos[b] - c + 1)
            kk = torch.from_numpy(kh[b, h, lo:pos[b] + 1])[None]
            vv = torch.from_numpy(vh[b, h, lo:pos[b] + 1])[None]
            qq = torch.from_numpy(q[b, h])[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)[0, 0].numpy()
            assert np.abs(o[b, h] - ref).max() < 1e-12
            assert abs(lse[b, h] - logsumexp(scale * kh[b, h, lo:pos[b] + 1] @ q[b, h])) < 1e-12


def test_decode_is_forward_row():
    """The forward definition (AAH section 5.8) at the new position, window min(W, T_max)."""
    B, H, L, d = 1, 4, 50, 16
    qh, kh, vh = _hist(B, H, L, d, 2)
    windows, T_max, scale = [3, 16, 49, 200], 48, 0.25
    for p in (0, 2, 15, 16, 47):
        pos = np.array([p])
        o, lse = oracle.decode_ref(qh[:, :, p], kh, vh, windows, pos, T_max, scale)
        for h, w in enumerate(windows):
            Of, Lf = oracle.attn_fwd_rows_ref(qh[0, h, :p + 1], kh[0, h, :p + 1], vh[0, h, :p + 1],
                                              min(w, T_max), scale, [p])
            assert np.abs(o[0, h] - Of[0]).max() < 1e-12
            assert abs(lse[0, h] - Lf[0]) < 1e-12


def test_decode_window_one_and_identical_keys():
    """Closed forms: W = 1 returns the new token's value; identical keys average the window's values."""
    B, H, L, d = 1, 2, 20, 4
    qh, kh, vh = _hist(B, H, L, d, 3)
    p = 12
    o, lse = oracle.decode_ref(qh[:, :, p], kh, vh, [1, 1], np.array([p]), 64, 0.5)
    assert np.array_equal(o[0], vh[0, :, p])
    assert np.allclose(lse[0], 0.5 * np.einsum("hd,hd->h", qh[0, :, p], kh[0, :, p]), atol=1e-14)
    kc = np.broadcast_to(kh[:, :, :1], kh.shape).copy()   # every key equal
    o, lse = oracle.decode_ref(qh[:, :, p], kc, vh, [5, 40], np.array([p]), 64, 0.5)
    assert np.allclose(o[0, 0], vh[0, 0, p - 4:p + 1].mean(0), atol=1e-12)
    assert np.allclose(o[0, 1], vh[0, 1, :p + 1].mean(0), atol=1e-12)
    s = 0.5 * np.einsum("hd,hd->h", qh[0, :, p], kh[0, :, 0])   # each head's one key value
    assert np.allclose(lse[0], [s[0] + np.log(5), s[1] + np.log(p + 1)], atol=1e-12)


def test_decode_key_order_invariant():
    """Invariant: permuting the history positions inside the window does not change the result."""
    B, H, L, d = 1, 1, 30, 8
    qh, kh, vh = _hist(B, H, L, d, 4)
    p, w = 25, 10
    o1, l1 = oracle.decode_ref(qh[:, :, p], kh, vh, [w], np.array([p]), 64, 0.3)
    perm = np.arange(L)
    perm[p - w + 1:p + 1] = np.random.default_rng(5).permutation(perm[p - w + 1:p + 1])
    o2, l2 = oracle.decode_ref(qh[:, :, p], kh[:, :, perm], vh[:, :, perm], [w], np.array([p]), 64, 0.3)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)


@pytest.mark.parametrize("windows,T_max", [([1, 3, 8], 6), ([5, 5], 100), ([200], 7)])
def test_cache_layout_brute_force(windows, T_max):
    """Brute force: replay every store one position at a time into a ring per head and compare."""
    B, H, L, d = 2, len(windows), 23, 2
    _, kh, _ = _hist(B, H, L, d, 6)
    off, sink, c = oracle.cache_rows_ref(windows, T_max)
    assert list(c) == [min(w, T_max) for w in windows] and list(sink) == [0] * H
    assert list(off) == [int(sum(c[:h])) for h in range(H)]
    n_written = np.array([0, 17])
    rows, valid = oracle.cache_content_ref(kh, windows, n_written, T_max)
    for b in range(B):
        ring = {}
        for t in range(n_written[b]):
            for h in range(H):
                ring[(h, t % c[h])] = kh[b, h, t]
        for h in range(H):
            for r in range(c[h]):
                if (h, r) in ring:
                    assert valid[b, off[h] + r] and np.array_equal(rows[b, off[h] + r], ring[(h, r)])
                else:
                    assert not valid[b, off[h] + r]


# ---------------------------------------------------------------- sinks and grouped key/value heads

def test_decode_with_sinks_is_forward_row():
    """With sinks: the forward definition's row p (window min(W, T_max), sinks S; pinned in
    test_sink_pins) over the history."""
    B, H, L, d = 1, 4, 60, 8
    qh, kh, vh = _hist(B, H, L, d, 9)
    windows, sinks, T_max, scale = [3, 16, 1, 200], [5, 2, 40, 3], 48, 0.3
    for p in (0, 4, 5, 20, 47):
        o, lse = oracle.decode_ref(qh[:, :, p], kh, vh, windows, np.array([p]), T_max, scale, sinks=sinks)
        for h, (w, s) in enumerate(zip(windows, sinks)):
            Of, Lf = oracle.attn_fwd_rows_ref(qh[0, h, :p + 1], kh[0, h, :p + 1], vh[0, h, :p + 1],
                                              min(w, T_max), scale, [p], sink=s)
            assert np.abs(o[0, h] - Of[0]).max() < 1e-12 and abs(lse[0, h] - Lf[0]) < 1e-12


def test_decode_grouped_equals_sdpa_gqa():
    """Grouped heads: torch SDPA with enable_gqa over each head's key set (as a boolean mask), and the same
    result as plain heads over K / V repeated per group."""
    B, H, H_kv, L, d = 2, 6, 2, 30, 8
    rng = np.random.default_rng(10)
    q = rng.standard_normal((B, H, d))
    kh, vh = rng.standard_normal((B, H_kv, L, d)), rng.standard_normal((B, H_kv, L, d))
    windows, sinks, T_max, scale = [1, 4, 30, 7, 2, 9], [0, 3, 0, 2, 5, 0], 32, 0.4
    pos = np.array([6, 25])
    o, lse = oracle.decode_ref(q, kh, vh, windows, pos, T_max, scale, sinks=sinks)
    kr, vr = np.repeat(kh, 3, axis=1), np.repeat(vh, 3, axis=1)
    o2, lse2 = oracle.decode_ref(q, kr, vr, windows, pos, T_max, scale, sinks=sinks)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    for b in range(B):
        mask = torch.zeros(1, H, 1, L, dtype=torch.bool)
        for h in range(H):
            mask[0, h, 0, oracle.decode_positions(int(pos[b]), windows[h], T_max, sinks[h])] = True
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b])[None, :, None], torch.from_numpy(kh[b])[None], torch.from_numpy(vh[b])[None],
            attn_mask=mask, scale=scale, enable_gqa=True)[0, :, 0].numpy()
        assert np.abs(o[b] - ref).max() < 1e-12


@pytest.mark.parametrize("windows,sinks,H_kv,T_max", [([1, 3, 8, 2], [2, 0, 4, 9], 2, 10),
                                                     ([5, 5, 5], [0, 1, 0], 1, 100), ([7, 2], [30, 0], 2, 7)])
def test_cache_layout_with_sinks_and_groups_brute_force(windows, sinks, H_kv, T_max):
    """Brute force: per key/value head, replay every store into a ring of max_h min(W_h, T_max) rows and a sink
    area of max_h min(S_h, T_max - min(W_h, T_max)) rows, and compare."""
    H = len(windows)
    G = H // H_kv
    B, L, d = 2, 23, 2
    kh = np.random.default_rng(11).standard_normal((B, H_kv, L, d))
    off, sink, ring = oracle.cache_rows_ref(windows, T_max, sinks, H_kv)
    c = [min(w, T_max) for w in windows]
    assert list(ring) == [max(c[g * G:(g + 1) * G]) for g in range(H_kv)]
    assert list(sink) == [max(max(0, min(s, T_max - ch)) for s, ch in zip(sinks[g * G:(g + 1) * G], c[g * G:(g + 1) * G]))
                          for g in range(H_kv)]
    assert list(off) == [int(sum(sink[:g]) + sum(ring[:g])) for g in range(H_kv)]
    n_written = np.array([0, 17])
    rows, valid = oracle.cache_content_ref(kh, windows, n_written, T_max, sinks)
    for b in range(B):
        store = {}
        for t in range(n_written[b]):
            for g in range(H_kv):
                store[off[g] + sink[g] + t % ring[g]] = kh[b, g, t]
                if t < sink[g]:
                    store[off[g] + t] = kh[b, g, t]
        for r in range(rows.shape[1]):
            assert valid[b, r] == (r in store)
            if r in store:
                assert np.array_equal(rows[b, r], store[r])


def test_decode_from_cache_rows_equals_decode_ref():
    """Attending over the cache rows the storage rule keeps, with the validity the layout implies (ring rows
    younger than C_h, sink rows before the window), gives decode_ref: the rows hold every position needed."""
    B, H, H_kv, L, d = 1, 4, 2, 40, 4
    rng = np.random.default_rng(12)
    q = rng.standard_normal((B, H, d))
    kh, vh = rng.standard_normal((B, H_kv, L, d)), rng.standard_normal((B, H_kv, L, d))
    windows, sinks, T_max, scale = [3, 10, 1, 5], [4, 0, 6, 2], 40, 0.5
    G = H // H_kv
    off, sink, ring = oracle.cache_rows_ref(windows, T_max, sinks, H_kv)
    for p in (0, 2, 3, 9, 25, 39):
        kc, _ = oracle.cache_content_ref(kh, windows, [p + 1], T_max, sinks)
        vc, _ = oracle.cache_content_ref(vh, windows, [p + 1], T_max, sinks)
        o, lse = oracle.decode_ref(q, kh, vh, windows, np.array([p]), T_max, scale, sinks=sinks)
        for h in range(H):
            g, ch = h // G, min(windows[h], T_max)
            s_eff = max(0, min(sinks[h], T_max - ch))
            idx = [off[g] + sink[g] + r for r in range(ring[g]) if (p - r) % ring[g] < ch and (p - r) % ring[g] <= p]
            idx += [off[g] + j for j in range(sink[g]) if j < s_eff and j <= p - ch]
            sc = scale * kc[0, idx] @ q[0, h]
            e = np.exp(sc - sc.max())
            assert np.abs((e / e.sum()) @ vc[0, idx] - o[0, h]).max() < 1e-12
            assert abs(sc.max() + np.log(e.sum()) - lse[0, h]) < 1e-12
