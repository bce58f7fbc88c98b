"""Pins of the oracle's grouped K/V heads (query head h reads key/value head floor(h / G)) against facts that
do not come from it: torch scaled_dot_product_attention with enable_gqa (float64, CPU, boolean window and sink
masks) and its autograd, and the identity with plain multi-head attention over K/V repeated per group (the
gradient of a shared head is the sum of its copies' gradients).  A mapping h mod H_kv instead of floor(h / G)
fails the library comparison; a missing sum over the group fails the gradient identity.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(B, H, H_kv, T, d, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, T, d)), rng.standard_normal((B, H_kv, T, d)),
            rng.standard_normal((B, H_kv, T, d)), rng.standard_normal((B, H, T, d)))


def _mask(T, w, s):
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    return (j <= i) & ((j > i - w) | (j < s))


CASES = [(2, 4, 2, 23, 8, [1, 5, 23, 40], [0, 2, 0, 3]), (1, 6, 1, 17, 4, [2, 3, 4, 5, 6, 7], None),
         (1, 6, 3, 30, 8, [9, 9, 1, 30, 12, 4], [4, 0, 0, 0, 1, 7])]


@pytest.mark.parametrize("B,H,H_kv,T,d,windows,sinks", CASES)
def test_gqa_forward_and_gradients_equal_torch(B, H, H_kv, T, d, windows, sinks):
    q, k, v, do = _rand(B, H, H_kv, T, d, seed=H + T)
    scale = 0.37
    O, L = oracle.attn_fwd_ref(q, k, v, windows, scale, sinks=sinks)
    dq, dk, dv = oracle.attn_bwd_ref(q, k, v, windows, scale, do, sinks=sinks)
    s = [0] * H if sinks is None else sinks
    mask = torch.stack([_mask(T, w, sh) for w, sh in zip(windows, s)])[None]   # [1, H, T, T]
    qt, kt, vt = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    ot = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=True)
    (ot * torch.from_numpy(do)).sum().backward()
    assert np.abs(O - ot.detach().numpy()).max() < 1e-12
    assert np.abs(dq - qt.grad.numpy()).max() < 1e-11
    assert np.abs(dk - kt.grad.numpy()).max() < 1e-11
    assert np.abs(dv - vt.grad.numpy()).max() < 1e-11
    # lse against the key-set logsumexp computed directly
    G = H // H_kv
    for b in range(B):
        for h in range(H):
            sc = scale * q[b, h] @ k[b, h // G].T
            sc = np.where(mask[0, h].numpy(), sc, -np.inf)
            assert np.abs(L[b, h] - np.log(np.exp(sc - sc.max(1, keepdims=True)).sum(1)) - sc.max(1)).max() < 1e-12


@pytest.mark.parametrize("B,H,H_kv,T,d,windows,sinks", CASES)
def test_gqa_equals_mha_with_repeated_kv(B, H, H_kv, T, d, windows, sinks):
    """Identity: GQA = MHA over K/V repeated G times per group; dK, dV of a shared head = sum over its copies."""
    q, k, v, do = _rand(B, H, H_kv, T, d, seed=7 * H + T)
    G = H // H_kv
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    O, L = oracle.attn_fwd_ref(q, k, v, windows, 0.5, sinks=sinks)
    Om, Lm = oracle.attn_fwd_ref(q, kr, vr, windows, 0.5, sinks=sinks)
    assert np.array_equal(O, Om) and np.array_equal(L, Lm)
    dq, dk, dv = oracle.attn_bwd_ref(q, k, v, windows, 0.5, do, sinks=sinks)
    dqm, dkm, dvm = oracle.attn_bwd_ref(q, kr, vr, windows, 0.5, do, sinks=sinks)
    assert np.array_equal(dq, dqm)
    assert np.allclose(dk, dkm.reshape(B, H_kv, G, T, d).sum(2), rtol=0, atol=1e-13)
    assert np.allclose(dv, dvm.reshape(B, H_kv, G, T, d).sum(2), rtol=0, atol=1e-13)


def test_kv_head_mapping():
    assert [oracle.kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [oracle.kv_head(h, 3, 3) for h in range(3)] == [0, 1, 2]
    with pytest.raises(ValueError):
        oracle.kv_head(0, 6, 4)


def test_gqa_features_use_the_groups_kv_head():
    """Key/value statistics of a query head are its group's head's; query statistics stay per head."""
    q, k, v, _ = _rand(2, 4, 2, 10, 4, seed=3)
    k[:, 1] *= 3.0
    x = oracle.head_features_ref(q, k, v, [3, 3, 3, 3])
    for h in range(4):
        g = h // 2
        assert x[h, 2] == pytest.approx(np.abs(k[:, g]).mean(), abs=1e-14)
        assert x[h, 5] == pytest.approx(v[:, g].std(), abs=1e-14)
        assert x[h, 0] == pytest.approx(np.abs(q[:, h]).mean(), abs=1e-14)
    ent, nrm = oracle.attn_row_stats_ref(q, k, v, [3, 3, 3, 3], 0.5)
    entr, nrmr = oracle.attn_row_stats_ref(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), [3, 3, 3, 3], 0.5)
    assert np.array_equal(ent, entr) and np.array_equal(nrm, nrmr)
