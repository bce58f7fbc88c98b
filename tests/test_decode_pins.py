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
    off, c = oracle.cache_rows_ref(windows, T_max)
    assert list(c) == [min(w, T_max) for w in windows]
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
