"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a library routine (PyTorch's
scaled_dot_product_attention and scipy's logsumexp, run in float64 on the CPU),
a closed form, an invariant, central finite differences, or the worked example
printed on the pages (tests/golden).  Together they fail on a dropped term, a
wrong sign, an off-by-one in the window, or a transposed operand anywhere in
the oracle.
"""
import json
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from synth import random_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(B, H, T, d, seed=0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, T, d)) for _ in range(4)]


def _sdpa_fp64(q, k, v, windows, scale, causal_only=False):
    """torch SDPA in float64 on the CPU with a boolean band mask built by tril/triu."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    T = q.shape[2]
    outs = []
    for h, w in enumerate(windows):
        if causal_only:
            o = torch.nn.functional.scaled_dot_product_attention(
                qt[:, h], kt[:, h], vt[:, h], is_causal=True, scale=scale)
        else:
            ones = torch.ones(T, T, dtype=torch.bool)
            band = torch.tril(ones) & torch.triu(ones, diagonal=-(min(w, T) - 1))
            o = torch.nn.functional.scaled_dot_product_attention(
                qt[:, h], kt[:, h], vt[:, h], attn_mask=band, scale=scale)
        outs.append(o.numpy())
    return np.stack(outs, axis=1)


# ---------------------------------------------------------------- forward

@pytest.mark.parametrize("windows", [[40, 41, 1000], [40, 40, 40]])
def test_full_window_equals_causal_sdpa(windows):
    """w >= T is standard causal attention (AAH section 5.2 and 5.8)."""
    q, k, v, _ = _rand(2, 3, 40, 8, seed=1)
    scale = 0.37
    O, LSE = oracle.attn_fwd_ref(q, k, v, windows, scale)
    ref = _sdpa_fp64(q, k, v, windows, scale, causal_only=True)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    # LSE of a causal row = logsumexp of the scaled scores over keys 0..i
    for b in range(2):
        for h in range(3):
            S = scale * q[b, h] @ k[b, h].T
            for i in (0, 7, 39):
                assert abs(LSE[b, h, i] - logsumexp(S[i, : i + 1])) < 1e-12


@pytest.mark.parametrize("T,d,windows", [(37, 5, [1, 2, 7, 36, 37, 90]), (64, 16, [3, 16, 17, 63])])
def test_band_mask_equals_sdpa(T, d, windows):
    """Any window equals SDPA with the band mask t_q - W + 1 <= t_k <= t_q (section 5.8, 7.7)."""
    q, k, v, _ = _rand(2, len(windows), T, d, seed=2)
    scale = 1.0 / np.sqrt(d)
    O, LSE = oracle.attn_fwd_ref(q, k, v, windows, scale)
    np.testing.assert_allclose(O, _sdpa_fp64(q, k, v, windows, scale), rtol=0, atol=1e-12)
    for b in range(2):
        for h, w in enumerate(windows):
            S = scale * q[b, h] @ k[b, h].T
            for i in range(T):
                lo = max(0, i - min(w, T) + 1)
                assert abs(LSE[b, h, i] - logsumexp(S[i, lo: i + 1])) < 1e-12


def test_window_one_returns_values():
    """w = 1: each query sees only itself, so O_i = V_i and LSE_i = scale q_i . k_i."""
    q, k, v, do = _rand(1, 2, 19, 6, seed=3)
    scale = 0.5
    O, LSE = oracle.attn_fwd_ref(q, k, v, [1, 1], scale)
    np.testing.assert_array_equal(O, v)
    np.testing.assert_allclose(LSE, scale * np.einsum("bhtd,bhtd->bht", q, k), atol=1e-14)
    dq, dk, dv = oracle.attn_bwd_ref(q, k, v, [1, 1], scale, do)
    np.testing.assert_allclose(dq, 0, atol=1e-14)
    np.testing.assert_allclose(dk, 0, atol=1e-14)
    np.testing.assert_allclose(dv, do, atol=1e-14)


@pytest.mark.parametrize("w", [1, 4, 9, 30])
def test_uniform_keys_closed_form(w):
    """All keys equal: O_i is the mean of V over the window, LSE_i = s q_i.k + ln(min(i+1, w))."""
    T, d = 30, 4
    q, _, v, _ = _rand(1, 1, T, d, seed=4)
    kvec = np.random.default_rng(5).standard_normal(d)
    k = np.broadcast_to(kvec, (1, 1, T, d)).copy()
    scale = 0.8
    O, LSE = oracle.attn_fwd_ref(q, k, v, [w], scale)
    for i in range(T):
        n = min(i + 1, w)
        np.testing.assert_allclose(O[0, 0, i], v[0, 0, i - n + 1: i + 1].mean(axis=0), atol=1e-13)
        assert abs(LSE[0, 0, i] - (scale * q[0, 0, i] @ kvec + np.log(n))) < 1e-12


def test_key_shift_invariance():
    """K -> K + 1 c^T shifts every score of row i by the same s q_i.c: O unchanged."""
    q, k, v, _ = _rand(1, 2, 25, 6, seed=6)
    c = np.random.default_rng(7).standard_normal(6)
    O1, L1 = oracle.attn_fwd_ref(q, k, v, [5, 25], 0.3)
    O2, L2 = oracle.attn_fwd_ref(q, k + c, v, [5, 25], 0.3)
    np.testing.assert_allclose(O1, O2, atol=1e-12)
    np.testing.assert_allclose(L2 - L1, 0.3 * np.einsum("bhtd,d->bht", q, c), atol=1e-12)


def test_row_weights():
    """With V = identity (d = T), O = P: rows sum to 1, P > 0 inside (i-w, i], 0 outside."""
    T, w = 12, 5
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, T, 3))
    k = rng.standard_normal((1, 1, T, 3))
    v = np.eye(T)[None, None]
    P, _ = oracle.attn_fwd_ref(q, k, v, [w], 1.0)
    P = P[0, 0]
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)
    for i in range(T):
        for j in range(T):
            if i - w < j <= i:
                assert P[i, j] > 0
            else:
                assert P[i, j] == 0.0


def test_constant_values():
    """V rows all equal c: O = c everywhere and dQ = dK = 0."""
    q, k, _, do = _rand(1, 2, 17, 5, seed=9)
    c = np.random.default_rng(10).standard_normal(5)
    v = np.broadcast_to(c, q.shape).copy()
    O, _ = oracle.attn_fwd_ref(q, k, v, [3, 17], 0.4)
    np.testing.assert_allclose(O, np.broadcast_to(c, O.shape), atol=1e-13)
    dq, dk, _ = oracle.attn_bwd_ref(q, k, v, [3, 17], 0.4, do)
    np.testing.assert_allclose(dq, 0, atol=1e-12)
    np.testing.assert_allclose(dk, 0, atol=1e-12)


def test_head_permutation_commutes():
    """Permuting heads (Q, K, V, windows) permutes every output: bucketing and
    scatter back to head order have no numerical effect (AAH Figure 1, section 5.8)."""
    q, k, v, do = _rand(2, 5, 21, 4, seed=11)
    windows = np.array([1, 3, 21, 7, 3])
    perm = np.array([3, 0, 4, 2, 1])
    O, L = oracle.attn_fwd_ref(q, k, v, windows, 0.6)
    Op, Lp = oracle.attn_fwd_ref(q[:, perm], k[:, perm], v[:, perm], windows[perm], 0.6)
    np.testing.assert_array_equal(Op, O[:, perm])
    np.testing.assert_array_equal(Lp, L[:, perm])
    g = oracle.attn_bwd_ref(q, k, v, windows, 0.6, do)
    gp = oracle.attn_bwd_ref(q[:, perm], k[:, perm], v[:, perm], windows[perm], 0.6, do[:, perm])
    for a, b in zip(g, gp):
        np.testing.assert_array_equal(b, a[:, perm])


def test_rows_variant_matches_full():
    q, k, v, _ = _rand(1, 1, 50, 8, seed=12)
    O, L = oracle.attn_fwd_ref(q, k, v, [13], 0.35)
    rows = [0, 5, 12, 13, 49]
    Or, Lr = oracle.attn_fwd_rows_ref(q[0, 0], k[0, 0], v[0, 0], 13, 0.35, rows)
    np.testing.assert_array_equal(Or, O[0, 0, rows])
    np.testing.assert_array_equal(Lr, L[0, 0, rows])


# ---------------------------------------------------------------- backward

@pytest.mark.parametrize("windows", [[1, 3], [3, 8], [8, 100]])
def test_backward_finite_differences(windows):
    """Central differences of f = sum(O * G) agree with the analytic dQ, dK, dV."""
    B, H, T, d = 1, 2, 8, 4
    q, k, v, g = _rand(B, H, T, d, seed=13)
    scale = 0.7
    dq, dk, dv = oracle.attn_bwd_ref(q, k, v, windows, scale, g)
    eps = 1e-6

    def f(q_, k_, v_):
        return float((oracle.attn_fwd_ref(q_, k_, v_, windows, scale)[0] * g).sum())

    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}; args_p[name] = xp
            args_m = {"q": q, "k": k, "v": v}; args_m[name] = xm
            num[idx] = (f(args_p["q"], args_p["k"], args_p["v"]) -
                        f(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        err = np.abs(num - grad).max() / max(np.abs(grad).max(), 1e-30)
        assert err < 1e-7, (name, err)


def test_gradient_sums():
    """sum_j dV_j = sum_i dO_i (rows of P sum to 1); sum_j dK_j = 0 (rows of dS sum to 0)."""
    q, k, v, do = _rand(2, 3, 33, 6, seed=14)
    dq, dk, dv = oracle.attn_bwd_ref(q, k, v, [1, 6, 40], 0.45, do)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-11)
    np.testing.assert_allclose(dk.sum(axis=2), 0, atol=1e-11)


def test_backward_full_window_matches_autograd():
    """w >= T: gradients equal autograd through causal SDPA in float64 (a library routine)."""
    q, k, v, do = _rand(1, 2, 24, 8, seed=15)
    scale = 0.35
    dq, dk, dv = oracle.attn_bwd_ref(q, k, v, [24, 50], scale, do)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-12)


# ---------------------------------------------------------------- coverage measures

@pytest.mark.parametrize("T,w", [(1, 1), (10, 1), (10, 3), (10, 10), (10, 25), (37, 16)])
def test_pair_count_brute_force(T, w):
    """sum_{t=1}^{T} min(t, W) equals the number of True entries of the band (section 5.10)."""
    assert oracle.pair_count_ref(T, w) == int(oracle.window_allowed(T, w).sum())
    W = min(w, T)
    assert oracle.pair_count_ref(T, w) == W * (W + 1) // 2 + (T - W) * W


def test_pair_count_at_4096():
    """Closed form W(W+1)/2 + (T-W)W at T = 4096 for the candidate set {512,...,4096}."""
    expected = {512: 1966336, 1024: 3670528, 2048: 6292480, 4096: 8390656}
    for w, n in expected.items():
        assert oracle.pair_count_ref(4096, w) == n


def test_acr_worked_example():
    """Figure 4 bucket fractions reproduce Table 6's printed inference ACR (tests/golden)."""
    with open(os.path.join(GOLDEN, "figure4_table6_acr.json")) as f:
        g = json.load(f)
    for name, row in g["rows"].items():
        fr = [p / 100.0 for p in row["fractions_percent"]]
        acr = oracle.acr_from_fractions_ref(fr, g["windows"], g["T"])
        assert abs(acr - row["acr"]) < g["tolerance"], (name, acr, row["acr"])


def test_acr_per_head_definition():
    """Per-head ACR (section 5.10) agrees with the fraction form (Table 6) and is 1 for full attention."""
    assert oracle.acr_ref([4096] * 32, 4096) == 1.0
    windows = [512] * 8 + [1024] * 8 + [2048] * 8 + [4096] * 8
    assert abs(oracle.acr_ref(windows, 4096) -
               oracle.acr_from_fractions_ref([0.25] * 4, [512, 1024, 2048, 4096], 4096)) < 1e-15
    assert oracle.acr_ref([9000], 4096) == 1.0   # windows above T are clamped to T


def test_oracle_on_bf16_workload_inputs():
    """The oracle consumes the generator's bf16-exact arrays without loss (exact promotion)."""
    wl = random_workload(1, 2, 16, 8, [4, 16], dtype="bf16", seed=3)
    O, _ = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale)
    O2, _ = oracle.attn_fwd_ref(wl.q.astype(np.float64), wl.k.astype(np.float64),
                                wl.v.astype(np.float64), wl.windows, wl.scale)
    np.testing.assert_array_equal(O, O2)
