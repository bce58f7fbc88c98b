"""GPU parity of the controller diagnostics ("Asymmetric Attention Heads" section 5.3) through the C ABI.

attn_fwd_diag: o and lse bit-identical to attn_fwd; per-row entropy and output norm against
oracle.attn_row_stats_ref.  Bounds (bf16): the kernel forms both from the same bf16-rounded weights w_j as
the row sum, each within a relative 2^-8 of the exact weight, so the normalised weights q_j are within
2 u p_j (u = 2^-8, a little over for the division) of the exact p_j:
  entropy: the result is the cross entropy of q against p plus ln(l~ / l), within 2 u H + u of H;
  norm:    ||sum_j (q_j - p_j) v_j|| <= 2 u max_j ||v_j||;
each plus 1e-4 for the fp32 arithmetic.  fp32 path: 2e-5 (entropy), 1e-5 (norm).
head_features: the Q/K/V statistics are fp32 sums about each lane's own first element merged in fp64:
relative 1e-5; e_h and n_h are means of the rows (checked against the oracle's means of the device's own
rows at 1e-6 relative, and against the exact rows within the row bounds); usage exact in fp32.
"""
import numpy as np
import pytest
import torch

import head_causal_local_amd as aah
import oracle
import synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -8 * 1.01


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a HIP device")


def dev(wl, key):
    if wl.dtype == "bf16":
        return torch.from_numpy(wl.bits[key].view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(getattr(wl, key)).to("cuda")


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_rows_bf16(ent, nrm, ent_ref, nrm_ref, vmax):
    e_bound = 2 * U * ent_ref + U + 1e-4
    assert (np.abs(ent - ent_ref) - e_bound).max() <= 0, f"entropy max err {np.abs(ent - ent_ref).max():.3e}"
    n_bound = 2 * U * vmax + 1e-4
    assert (np.abs(nrm - nrm_ref) - n_bound).max() <= 0, f"norm max err {np.abs(nrm - nrm_ref).max():.3e}"


def vmax_per_head(wl):
    """max_j ||v_j|| of every (b, h), broadcast over rows."""
    return np.linalg.norm(wl.v.astype(np.float64), axis=-1).max(axis=-1)[..., None]


SHAPES = [
    # B, H, T, d, windows, sinks
    (2, 4, 333, 64, [1, 7, 64, 1000], None),
    (1, 3, 200, 32, [5, 100, 200], [3, 0, 40]),
    (1, 2, 300, 128, [3, 300], [130, 0]),
    (2, 2, 1, 64, [1, 2], None),
]


@pytest.mark.parametrize("B,H,T,d,windows,sinks", SHAPES)
def test_bf16_forward_diagnostics(B, H, T, d, windows, sinks):
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=T + d, backward=False, sinks=sinks)
    q, k, v = dev(wl, "q"), dev(wl, "k"), dev(wl, "v")
    o0, l0 = aah.attn_fwd(q, k, v, wl.windows, sinks=wl.sinks)
    o, lse, ent, nrm = aah.attn_fwd_diag(q, k, v, wl.windows, sinks=wl.sinks)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, l0)
    ent_ref, nrm_ref = oracle.attn_row_stats_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, sinks=wl.sinks)
    check_rows_bf16(host(ent), host(nrm), ent_ref, nrm_ref, vmax_per_head(wl))


@pytest.mark.parametrize("B,H,T,d,windows,sinks", [(1, 3, 150, 32, [1, 17, 150], None),
                                                   (2, 2, 130, 64, [9, 64], [5, 0]),
                                                   (1, 2, 70, 128, [3, 70], None)])
def test_fp32_forward_diagnostics(B, H, T, d, windows, sinks):
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="f32", seed=T, backward=False, sinks=sinks)
    q, k, v = dev(wl, "q"), dev(wl, "k"), dev(wl, "v")
    o0, l0 = aah.attn_fwd(q, k, v, wl.windows, sinks=wl.sinks)
    o, lse, ent, nrm = aah.attn_fwd_diag(q, k, v, wl.windows, sinks=wl.sinks)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, l0)
    ent_ref, nrm_ref = oracle.attn_row_stats_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, sinks=wl.sinks)
    assert np.abs(host(ent) - ent_ref).max() < 2e-5
    assert np.abs(host(nrm) - nrm_ref).max() < 1e-5


@pytest.mark.parametrize("B,H,H_kv,T,d,windows,sinks", [
    (1, 4, 4, 3000, 64, [2000, 256, 3000, 1500], [64, 128, 0, 300]),
    (1, 4, 2, 2048, 128, [2048, 300, 1000, 2048], None),
])
def test_split_diagnostics(B, H, H_kv, T, d, windows, sinks):
    """Few-item shapes split the diagnostic forward too: each chunk leaves its rows' weighted offsets with
    (m, l, acc), and the merge forms the entropy and the norm of the combined row.  o and lse bitwise equal to
    the split attn_fwd (same chunks, same arithmetic); entropy and norm against the oracle within the same
    bounds as unsplit rows (each weight is still rounded within 2^-8 of its exact value, against its chunk's
    reference); repeated calls bitwise equal; an empty workspace gives the unsplit launch."""
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=T + H_kv, backward=False, sinks=sinks,
                               H_kv=H_kv)
    assert aah.fwd_workspace_size(wl.windows, B, H, T, d, sinks=sinks, H_kv=H_kv, diag=True) > \
        aah.fwd_workspace_size(wl.windows, B, H, T, d, sinks=sinks, H_kv=H_kv) > 0
    q, k, v = dev(wl, "q"), dev(wl, "k"), dev(wl, "v")
    o0, l0 = aah.attn_fwd(q, k, v, wl.windows, sinks=sinks)
    o, lse, ent, nrm = aah.attn_fwd_diag(q, k, v, wl.windows, sinks=sinks)
    _, _, ent2, nrm2 = aah.attn_fwd_diag(q, k, v, wl.windows, sinks=sinks)
    empty = torch.empty(0, dtype=torch.uint8, device="cuda")
    ou, lu, eu, nu = aah.attn_fwd_diag(q, k, v, wl.windows, sinks=sinks, workspace=empty)
    ou0, lu0 = aah.attn_fwd(q, k, v, wl.windows, sinks=sinks, workspace=empty)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, l0)
    assert torch.equal(ent, ent2) and torch.equal(nrm, nrm2)
    assert torch.equal(ou, ou0) and torch.equal(lu, lu0)
    ent_ref, nrm_ref = oracle.attn_row_stats_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, sinks=sinks)
    vmax = np.repeat(vmax_per_head(wl), H // H_kv, axis=1)
    check_rows_bf16(host(ent), host(nrm), ent_ref, nrm_ref, vmax)
    check_rows_bf16(host(eu), host(nu), ent_ref, nrm_ref, vmax)


def _check_features(x, wl, ent_dev, nrm_dev):
    ref_dev_rows = oracle.head_features_ref(wl.q, wl.k, wl.v, wl.windows, ent_dev, nrm_dev)
    assert np.allclose(x[:, :6], ref_dev_rows[:, :6], rtol=1e-5, atol=1e-6)
    assert np.allclose(x[:, 6:8], ref_dev_rows[:, 6:8], rtol=1e-6, atol=1e-6)
    assert np.array_equal(x[:, 8].astype(np.float32), ref_dev_rows[:, 8].astype(np.float32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_head_features_and_ema(dtype):
    """Features of the diagnostic forward's rows against the oracle; three EMA updates (init, then two more on
    changed inputs) against the recurrence applied to the device's previous state."""
    _require_gpu()
    B, H, T, d, windows = 2, 5, 700, 64, [1, 64, 300, 700, 5000]
    ema = torch.zeros((H, aah.N_FEATURES), dtype=torch.float32, device="cuda")
    prev = None
    for step, value_scale in enumerate((1.0, 0.5, 3.0)):
        wl = synth.random_workload(B, H, T, d, windows, dtype=dtype, seed=40 + step, backward=False,
                                   value_scale=value_scale)
        q, k, v = dev(wl, "q"), dev(wl, "k"), dev(wl, "v")
        _, _, ent, nrm = aah.attn_fwd_diag(q, k, v, wl.windows)
        x = aah.head_features(q, k, v, wl.windows, ent, nrm, features_ema=ema, alpha=0.9, init=step == 0)
        torch.cuda.synchronize()
        xh, ent_h, nrm_h = host(x), host(ent), host(nrm)
        _check_features(xh, wl, ent_h, nrm_h)
        # against the exact rows: the means inherit the row bounds
        ent_ref, nrm_ref = oracle.attn_row_stats_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale)
        exact = oracle.head_features_ref(wl.q, wl.k, wl.v, wl.windows, ent_ref, nrm_ref)
        if dtype == "bf16":
            assert (np.abs(xh[:, 6] - exact[:, 6]) <= 2 * U * exact[:, 6] + U + 1e-4).all()
            vmax = np.linalg.norm(wl.v.astype(np.float64), axis=-1).max(axis=(0, 2))
            assert (np.abs(xh[:, 7] - exact[:, 7]) <= 2 * U * vmax + 1e-4).all()
        else:
            assert np.allclose(xh[:, 6:8], exact[:, 6:8], rtol=0, atol=2e-5)
        want = oracle.features_ema_ref(prev, xh, 0.9, init=step == 0)
        assert np.allclose(host(ema), want, rtol=1e-6, atol=1e-7), step
        prev = host(ema)


def test_features_without_diagnostics_and_determinism():
    """No diagnostic rows: entropy, norm and usage features are 0 (AAH section 5.3 starts missing
    previous-attention diagnostics at zero).  Same inputs, same bits."""
    _require_gpu()
    wl = synth.random_workload(3, 4, 500, 32, [16, 128, 500, 2], dtype="bf16", seed=3, backward=False)
    q, k, v = dev(wl, "q"), dev(wl, "k"), dev(wl, "v")
    x1 = aah.head_features(q, k, v, wl.windows)
    x2 = aah.head_features(q, k, v, wl.windows)
    torch.cuda.synchronize()
    assert torch.equal(x1, x2)
    xh = host(x1)
    assert np.array_equal(xh[:, 6:9], np.zeros((4, 3)))
    ref = oracle.head_features_ref(wl.q, wl.k, wl.v, wl.windows)
    assert np.allclose(xh[:, :6], ref[:, :6], rtol=1e-5, atol=1e-6)
    assert np.array_equal(ref[:, 6:9], np.zeros((4, 3)))


SAMPLE_ROWS = [0, 1, 127, 128, 511, 512, 1023, 2048, 3000, 4095]


@pytest.mark.parametrize("idx", [3, 5])
def test_full_layer_diagnostics(idx):
    """The 1B-scale layer (grouped windows) and the streaming-head layer (sinks), B=4 H=32 T=4096 d=64:
    sampled rows against the oracle, all 32 heads' features against the oracle's reductions."""
    _require_gpu()
    wl = synth.make_workload(idx)
    q, k, v = dev(wl, "q"), dev(wl, "k"), dev(wl, "v")
    o0, l0 = aah.attn_fwd(q, k, v, wl.windows, sinks=wl.sinks)
    o, lse, ent, nrm = aah.attn_fwd_diag(q, k, v, wl.windows, sinks=wl.sinks)
    x = aah.head_features(q, k, v, wl.windows, ent, nrm)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, l0)
    ent_h, nrm_h = host(ent), host(nrm)
    vmax = vmax_per_head(wl)
    for b, h in ((0, 0), (1, 12), (2, 17), (3, 31)):
        s = 0 if wl.sinks is None else int(wl.sinks[h])
        e_ref, n_ref = oracle.attn_row_stats_rows_ref(wl.q[b, h], wl.k[b, h], wl.v[b, h], int(wl.windows[h]),
                                                      wl.scale, SAMPLE_ROWS, sink=s)
        check_rows_bf16(ent_h[b, h, SAMPLE_ROWS], nrm_h[b, h, SAMPLE_ROWS], e_ref, n_ref, vmax[b, h])
    _check_features(host(x), wl, ent_h, nrm_h)
