"""Pins of the oracle's sink + recent-window variant against facts that do not come from it.

The variant ("Autonomy-of-Heads", section 5 and section 6.1): a streaming head sees the first
S keys (its sinks) and its recent window of W keys, causally.  Expected values come from a
library routine (torch scaled_dot_product_attention and scipy logsumexp in float64 on the CPU,
over key sets built as Python set unions or with torch's own causal mask), closed forms
(two keys, identical keys), a decomposition into the already pinned plain window plus the
sink keys outside it, autograd of the library routine, and central finite differences.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle


def _rand(B, H, T, d, seed=0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, T, d)) for _ in range(4)]


def _key_set(i, w, s):
    """Keys of query i as a set union: sinks {0 .. s-1} and the recent window, both causal."""
    recent = set(range(max(0, i - w + 1), i + 1))
    sinks = set(range(min(s, i + 1)))
    return sorted(recent | sinks)


@pytest.mark.parametrize("T,w,s", [(37, 5, 3), (64, 16, 16), (50, 1, 1), (40, 8, 30), (33, 33, 4), (20, 3, 0)])
def test_sink_rows_equal_sdpa_over_key_sets(T, w, s):
    """Library routine: each row is unmasked SDPA over its key set, built independently."""
    q, k, v, _ = _rand(1, 1, T, 8, seed=T + w + s)
    scale = 0.41
    O, L = oracle.attn_fwd_ref(q, k, v, [w], scale, sinks=[s])
    for i in range(T):
        js = _key_set(i, w, s)
        qq = torch.from_numpy(q[0, 0, i])[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, torch.from_numpy(k[0, 0, js])[None], torch.from_numpy(v[0, 0, js])[None], scale=scale)
        assert np.abs(O[0, 0, i] - ref[0, 0].numpy()).max() < 1e-12, i
        assert abs(L[0, 0, i] - logsumexp(scale * k[0, 0, js] @ q[0, 0, i])) < 1e-12, i


@pytest.mark.parametrize("s", [17, 64, 500])
def test_sinks_covering_the_sequence_are_causal(s):
    """Library routine: with S >= T every earlier key is a sink, so the head is plain causal
    (torch SDPA is_causal) whatever its window."""
    T = 17 if s == 17 else 48
    q, k, v, _ = _rand(2, 2, T, 8, seed=s)
    O, _ = oracle.attn_fwd_ref(q, k, v, [1, 7], 0.3, sinks=[s, s])
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), is_causal=True, scale=0.3).numpy()
    assert np.abs(O - ref).max() < 1e-12


def test_zero_sinks_is_the_plain_window():
    """S = 0 reproduces the pinned plain-window oracle exactly (forward and backward)."""
    q, k, v, do = _rand(1, 3, 40, 8, seed=3)
    w = [1, 9, 40]
    O0, L0 = oracle.attn_fwd_ref(q, k, v, w, 0.5)
    O1, L1 = oracle.attn_fwd_ref(q, k, v, w, 0.5, sinks=[0, 0, 0])
    assert np.array_equal(O0, O1) and np.array_equal(L0, L1)
    g0 = oracle.attn_bwd_ref(q, k, v, w, 0.5, do)
    g1 = oracle.attn_bwd_ref(q, k, v, w, 0.5, do, sinks=[0, 0, 0])
    assert all(np.array_equal(a, b) for a, b in zip(g0, g1))


def test_two_key_closed_form():
    """Closed form: W = 1 and S = 1 leave row i > 0 with keys {0, i}, so
    o_i = sigma(a) v_0 + (1 - sigma(a)) v_i with a = scale (k_0 - k_i) . q_i, and
    lse_i = log(exp(scale k_0 . q_i) + exp(scale k_i . q_i))."""
    T, scale = 30, 0.7
    q, k, v, _ = _rand(1, 1, T, 4, seed=5)
    O, L = oracle.attn_fwd_ref(q, k, v, [1], scale, sinks=[1])
    assert np.array_equal(O[0, 0, 0], v[0, 0, 0])
    for i in range(1, T):
        s0 = scale * k[0, 0, 0] @ q[0, 0, i]
        si = scale * k[0, 0, i] @ q[0, 0, i]
        g = 1.0 / (1.0 + np.exp(si - s0))
        assert np.allclose(O[0, 0, i], g * v[0, 0, 0] + (1 - g) * v[0, 0, i], atol=1e-13, rtol=0)
        assert abs(L[0, 0, i] - np.logaddexp(s0, si)) < 1e-13


@pytest.mark.parametrize("T,w,s", [(60, 7, 5), (45, 20, 25), (16, 2, 15)])
def test_identical_keys_average_the_key_set(T, w, s):
    """Closed form: equal keys give every allowed key the same weight, so row i averages the
    values of min(i + 1, W) recent keys and max(0, min(S, i + 1 - W)) sinks outside the window,
    and lse_i = score + log(count)."""
    q, k, v, _ = _rand(1, 1, T, 4, seed=6)
    k[:] = k[:, :, :1]
    scale = 0.5
    O, L = oracle.attn_fwd_ref(q, k, v, [w], scale, sinks=[s])
    for i in range(T):
        n_rec = min(i + 1, w)
        n_sink = max(0, min(s, i + 1 - w))
        idx = list(range(n_sink)) + list(range(i + 1 - n_rec, i + 1))
        assert np.allclose(O[0, 0, i], v[0, 0, idx].mean(0), atol=1e-12), i
        sc = scale * k[0, 0, 0] @ q[0, 0, i]
        assert abs(L[0, 0, i] - (sc + np.log(n_rec + n_sink))) < 1e-12, i


def test_sink_lse_decomposes_into_window_and_sinks():
    """Decomposition: row i's lse is the logaddexp of the plain window's lse (the pinned oracle
    without sinks) and the logsumexp over the sink keys that lie before the window."""
    T, w, s, scale = 80, 12, 20, 0.33
    q, k, v, _ = _rand(1, 1, T, 8, seed=7)
    _, Ls = oracle.attn_fwd_ref(q, k, v, [w], scale, sinks=[s])
    _, Lw = oracle.attn_fwd_ref(q, k, v, [w], scale)
    for i in range(T):
        extra = range(min(s, max(0, i - w + 1)))
        if len(extra) == 0:
            assert Ls[0, 0, i] == Lw[0, 0, i]
        else:
            ls = logsumexp(scale * k[0, 0, list(extra)] @ q[0, 0, i])
            assert abs(Ls[0, 0, i] - np.logaddexp(Lw[0, 0, i], ls)) < 1e-12


@pytest.mark.parametrize("windows,sinks", [([4, 1, 11], [3, 2, 0]), ([2, 6], [9, 4])])
def test_sink_gradients_equal_autograd_of_sdpa(windows, sinks):
    """Library routine: autograd of torch SDPA (float64, CPU) with a boolean mask made from each
    row's key set gives the oracle's dQ, dK, dV."""
    T, d, scale = 24, 8, 0.45
    q, k, v, do = _rand(1, len(windows), T, d, seed=8)
    dq, dk, dv = oracle.attn_bwd_ref(q, k, v, windows, scale, do, sinks=sinks)
    for h, (w, s) in enumerate(zip(windows, sinks)):
        mask = torch.zeros(T, T, dtype=torch.bool)
        for i in range(T):
            mask[i, _key_set(i, w, s)] = True
        qt, kt, vt = (torch.from_numpy(x[0, h].copy()).requires_grad_() for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None], attn_mask=mask, scale=scale)
        (o[0] * torch.from_numpy(do[0, h])).sum().backward()
        assert np.abs(qt.grad.numpy() - dq[0, h]).max() < 1e-11
        assert np.abs(kt.grad.numpy() - dk[0, h]).max() < 1e-11
        assert np.abs(vt.grad.numpy() - dv[0, h]).max() < 1e-11


def test_sink_gradients_finite_differences():
    """Central finite differences of sum(O * dO) at a few coordinates of Q, K and V, including a
    sink key (row 0) that only rows far outside its window reach."""
    T, d, w, s, scale, eps = 20, 4, 3, 2, 0.6, 1e-6
    q, k, v, do = _rand(1, 1, T, d, seed=9)
    grads = oracle.attn_bwd_ref(q, k, v, [w], scale, do, sinks=[s])

    def f(qq, kk, vv):
        return float((oracle.attn_fwd_ref(qq, kk, vv, [w], scale, sinks=[s])[0] * do).sum())

    for which, (t, e) in ((0, (15, 1)), (1, (0, 2)), (1, (1, 0)), (1, (10, 3)), (2, (0, 1)), (2, (18, 0))):
        args = [q.copy(), k.copy(), v.copy()]
        args[which][0, 0, t, e] += eps
        fp = f(*args)
        args[which][0, 0, t, e] -= 2 * eps
        fm = f(*args)
        assert abs((fp - fm) / (2 * eps) - grads[which][0, 0, t, e]) < 1e-7, (which, t, e)


@pytest.mark.parametrize("T,w,s", [(1, 1, 0), (9, 3, 2), (50, 10, 70), (64, 64, 5), (100, 1, 128), (300, 256, 128)])
def test_pair_count_with_sinks_brute_force(T, w, s):
    """Brute force: the pair count equals the size of every row's key set, summed."""
    assert oracle.pair_count_ref(T, w, s) == sum(len(_key_set(i, w, s)) for i in range(T))
    assert oracle.pair_count_ref(T, w, s) == int(oracle.window_allowed(T, w, s).sum())


@pytest.mark.parametrize("T,w,s", [(1, 1, 0), (9, 3, 2), (40, 7, 0), (40, 100, 5), (33, 1, 33)])
def test_window_rows_restriction_matches_full_mask_and_brute_force(T, w, s):
    """The row-restricted mask (used for spot checks of long sequences) is the full mask's rows, and both
    agree entry by entry with the visibility rule written as a loop."""
    full = oracle.window_allowed(T, w, s)
    rows = sorted({0, T // 2, T - 1})
    assert np.array_equal(oracle.window_allowed(T, w, s, rows=rows), full[rows])
    W = min(w, T)
    for i in range(T):
        for j in range(T):
            assert full[i, j] == (j <= i and (j > i - W or j < s))
