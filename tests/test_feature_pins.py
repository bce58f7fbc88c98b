"""Pins of the controller-feature oracle (oracle/features.py) against facts that do not come from it.

Library routines (scipy's softmax and entropy over each row's key set, torch scaled_dot_product_attention
for the output rows, torch's mean / population std of a head's slice), closed forms (uniform attention over
identical keys, a window of one, constant and two-valued activations, the EMA of a constant input), and the
mistakes a plausible implementation makes: |mean| instead of mean |x|, reducing over the wrong axis, an unbiased
instead of a population deviation, usage above 1 for windows longer than T, a nonzero usage with no stored
statistics.
"""
import numpy as np
import pytest
import torch
from scipy.special import softmax
from scipy.stats import entropy

import oracle


def _rand(B, H, T, d, seed=0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, T, d)) for _ in range(3)]


def _key_set(i, w, s):
    return sorted(set(range(max(0, i - w + 1), i + 1)) | set(range(min(s, i + 1))))


@pytest.mark.parametrize("windows,sinks", [([1, 5, 40], None), ([3, 8, 100], [2, 0, 9])])
def test_row_stats_equal_library_routines(windows, sinks):
    """Row entropy = scipy entropy of the softmax over the row's keys; row norm = ||SDPA output||."""
    B, T, d, scale = 2, 37, 8, 0.43
    q, k, v = _rand(B, len(windows), T, d, seed=1)
    ent, nrm = oracle.attn_row_stats_ref(q, k, v, windows, scale, sinks=sinks)
    for b in range(B):
        for h, w in enumerate(windows):
            s = 0 if sinks is None else sinks[h]
            for i in range(T):
                js = _key_set(i, w, s)
                p = softmax(scale * k[b, h, js] @ q[b, h, i])
                assert abs(ent[b, h, i] - entropy(p)) < 1e-12
                o = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(q[b, h, i])[None, None], torch.from_numpy(k[b, h, js])[None],
                    torch.from_numpy(v[b, h, js])[None], scale=scale)
                assert abs(nrm[b, h, i] - torch.linalg.norm(o).item()) < 1e-12


def test_row_stats_closed_forms():
    """Identical keys: uniform weights, entropy ln(n_i), norm ||mean of the row's values||.
    A window of one: entropy exactly 0, norm ||v_i||."""
    B, T, d = 1, 30, 6
    q, k, v = _rand(B, 3, T, d, seed=2)
    k[:] = k[:, :, :1]
    windows, sinks = [7, 1, 50], [3, 0, 0]
    ent, nrm = oracle.attn_row_stats_ref(q, k, v, windows, 0.9, sinks=sinks)
    for h, (w, s) in enumerate(zip(windows, sinks)):
        for i in range(T):
            js = _key_set(i, w, s)
            assert abs(ent[0, h, i] - np.log(len(js))) < 1e-12
            assert abs(nrm[0, h, i] - np.linalg.norm(v[0, h, js].mean(0))) < 1e-12
    q, k, v = _rand(B, 1, T, d, seed=3)
    ent, nrm = oracle.attn_row_stats_ref(q, k, v, [1], 0.5)
    assert np.array_equal(ent[0, 0], np.zeros(T))
    assert np.allclose(nrm[0, 0], np.linalg.norm(v[0, 0], axis=1), rtol=0, atol=1e-14)


def test_qkv_statistics_equal_torch_reductions():
    """mu(|x_h|) and sigma(x_h) equal torch's mean of abs and population std over (B, T, d) of head h,
    for heads with different distributions (a wrong reduction axis mixes them)."""
    rng = np.random.default_rng(4)
    B, H, T, d = 3, 4, 20, 8
    shift = np.array([0.0, 2.0, -1.5, 0.3])[None, :, None, None]
    spread = np.array([1.0, 0.5, 3.0, 0.1])[None, :, None, None]
    q, k, v = (rng.standard_normal((B, H, T, d)) * spread + shift * (i + 1) for i in range(3))
    x = oracle.head_features_ref(q, k, v, [5, 10, 20, 40])
    for h in range(H):
        for slot, t in enumerate((q, k, v)):
            th = torch.from_numpy(t[:, h])
            assert abs(x[h, 2 * slot] - th.abs().mean().item()) < 1e-12
            assert abs(x[h, 2 * slot + 1] - th.std(unbiased=False).item()) < 1e-12


def test_qkv_statistics_closed_forms():
    """Constant c: mean |x| = |c|, sigma = 0.  Values -1 and 3 in equal numbers: mean |x| = 2 (not
    |mean| = 1), population sigma = 2 (the unbiased form would give 2 sqrt(N / (N - 1)))."""
    B, H, T, d = 1, 2, 4, 4
    q = np.full((B, H, T, d), -2.5)
    k = np.where(np.arange(B * H * T * d).reshape(B, H, T, d) % 2 == 0, -1.0, 3.0)
    v = np.zeros((B, H, T, d))
    x = oracle.head_features_ref(q, k, v, [1, 4])
    assert np.array_equal(x[:, 0], [2.5, 2.5]) and np.array_equal(x[:, 1], [0.0, 0.0])
    assert np.array_equal(x[:, 2], [2.0, 2.0]) and np.array_equal(x[:, 3], [2.0, 2.0])
    assert np.array_equal(x[:, 4:6], np.zeros((2, 2)))


def test_diagnostics_usage_and_missing_entries():
    """"Asymmetric Attention Heads" section 5.3 (Head features and EMA smoothing): the previous-attention
    diagnostics (e_h, n_h, rho_h) start at zero when missing, so with no stored statistics all three entries
    are exactly 0 -- rho_h included.  With them, e_h and n_h are the means of the given rows over (B, T), and
    rho_h, the usage of the forward pass that produced them, is min(W_h, T) / T: a window longer than T is 1.
    Giving only one of the two row arrays is refused (they come from one forward pass)."""
    B, H, T, d = 2, 3, 16, 4
    q, k, v = _rand(B, H, T, d, seed=5)
    x0 = oracle.head_features_ref(q, k, v, [4, 16, 1000])
    assert np.array_equal(x0[:, 6:9], np.zeros((H, 3)))
    ent = np.arange(B * H * T, dtype=np.float64).reshape(B, H, T)
    nrm = ent[:, ::-1] * 0.5
    x1 = oracle.head_features_ref(q, k, v, [4, 16, 1000], row_entropy=ent, row_norm=nrm)
    for h in range(H):
        assert x1[h, 6] == pytest.approx(np.mean([ent[b, h, t] for b in range(B) for t in range(T)]), abs=1e-12)
        assert x1[h, 7] == pytest.approx(np.mean([nrm[b, h, t] for b in range(B) for t in range(T)]), abs=1e-12)
    assert np.array_equal(x1[:, 8], [0.25, 1.0, 1.0])
    assert np.array_equal(x1[:, :6], x0[:, :6])
    with pytest.raises(ValueError):
        oracle.head_features_ref(q, k, v, [4, 16, 1000], row_entropy=ent)


def test_ema_closed_forms():
    """The first update takes x; a constant input x after xbar_0 = a gives x + alpha^t (a - x); alpha = 0
    follows the input."""
    rng = np.random.default_rng(6)
    a, x = rng.standard_normal((4, 9)), rng.standard_normal((4, 9))
    assert np.array_equal(oracle.features_ema_ref(None, a, 0.9, init=True), a)
    xbar = a
    for t in range(1, 6):
        xbar = oracle.features_ema_ref(xbar, x, 0.9, init=False)
        assert np.allclose(xbar, x + 0.9 ** t * (a - x), atol=1e-14)
    assert np.array_equal(oracle.features_ema_ref(a, x, 0.0, init=False), x)


def test_row_stats_rows_match_full():
    """The row-restricted form is the full definition on the selected rows."""
    q, k, v = _rand(1, 2, 50, 8, seed=7)
    ent, nrm = oracle.attn_row_stats_ref(q, k, v, [6, 20], 0.7, sinks=[4, 0])
    rows = [0, 3, 17, 49]
    for h, (w, s) in enumerate(((6, 4), (20, 0))):
        e, n = oracle.attn_row_stats_rows_ref(q[0, h], k[0, h], v[0, h], w, 0.7, rows, sink=s)
        assert np.allclose(e, ent[0, h, rows], rtol=0, atol=1e-14)
        assert np.allclose(n, nrm[0, h, rows], rtol=0, atol=1e-14)
