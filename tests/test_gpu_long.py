"""Long sequences: T = 2^17 positions per head, 32 times the bench layers, through the C ABI.

Forward: sampled rows (start, every power-of-two boundary region, middle, end) against
oracle.attn_fwd_rows_ref.  Backward: with window W a query row needs only the W keys ending at it, and a
key row only the queries within W after it, so the dense backward oracle run on a slice [a, b) of the
sequence gives the exact gradients of the slice's interior rows (`exact_rows` below, pinned on the CPU
against the oracle over a whole short sequence).  Tolerances as in the other bf16 parity tests.
"""
import numpy as np
import pytest
import torch

import head_causal_local_amd as aah
import oracle
import synth

O_TOL_BF16 = 1e-2
LSE_TOL_BF16 = 4e-3
GRAD_REL = 3e-2


def exact_rows(T, W, a, b):
    """Rows of the slice [a, b) whose gradients the slice alone determines: (dQ rows, dK/dV rows).

    dQ_i needs keys i - W + 1 .. i (all inside once i >= a + W - 1, or a = 0); dK_j / dV_j need the queries
    j .. j + W - 1 (inside once j + W - 1 < b, or b = T) with their exact softmax rows."""
    rows = np.arange(a, b)
    left = rows >= a + W - 1 if a > 0 else np.ones_like(rows, dtype=bool)
    right = rows + W - 1 < b if b < T else np.ones_like(rows, dtype=bool)
    return rows[left], rows[left & right]


def slice_bwd(wl, bh, W, a, b):
    """Oracle gradients of head (b, h) over the slice [a, b) of the sequence, as full slice arrays."""
    b_, h = bh
    sl = (slice(b_, b_ + 1), slice(h, h + 1), slice(a, b))
    dq, dk, dv = oracle.attn_bwd_ref(wl.q[sl], wl.k[sl], wl.v[sl], [W], wl.scale, wl.do[sl])
    return dq[0, 0], dk[0, 0], dv[0, 0]


@pytest.mark.parametrize("W", [1, 7, 40])
def test_slice_rows_equal_full_sequence_oracle(W):
    """CPU pin of the slicing rule: on a 300-position sequence every row `exact_rows` keeps has the
    whole-sequence oracle's gradient, for slices at the start, inside and at the end."""
    T = 300
    wl = synth.random_workload(1, 1, T, 8, [W], dtype="f32", seed=W, backward=True)
    fq, fk, fv = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, [W], wl.scale, wl.do)
    for a, b in ((0, 120), (90, 260), (200, T), (0, T)):
        dq, dk, dv = slice_bwd(wl, (0, 0), W, a, b)
        q_rows, k_rows = exact_rows(T, W, a, b)
        assert len(q_rows) and len(k_rows)
        assert np.allclose(dq[q_rows - a], fq[0, 0, q_rows], rtol=0, atol=1e-12)
        assert np.allclose(dk[k_rows - a], fk[0, 0, k_rows], rtol=0, atol=1e-12)
        assert np.allclose(dv[k_rows - a], fv[0, 0, k_rows], rtol=0, atol=1e-12)
        if a > 0 and W > 1:  # the first row of an inner slice lacks keys: the rule must drop it
            assert a not in q_rows and not np.allclose(dq[0], fq[0, 0, a], rtol=0, atol=1e-12)


T_LONG = 1 << 17
WINDOWS = [1, 512, 1024, 256]
SINKS = [0, 0, 0, 64]
ROWS = [0, 1, 63, 64, 511, 512, 1023, 1024, 32767, 32768, 65535, 65536, 98304, T_LONG - 2, T_LONG - 1]

_WL = {}


def _workload():
    if "wl" not in _WL:
        _WL["wl"] = synth.random_workload(1, len(WINDOWS), T_LONG, 64, WINDOWS, dtype="bf16", seed=29,
                                          backward=True, sinks=SINKS)
    return _WL["wl"]


def _dev(wl, key):
    return torch.from_numpy(wl.bits[key].view(np.int16)).view(torch.bfloat16).to("cuda")


@pytest.mark.gpu
def test_long_sequence_forward_rows():
    if not torch.cuda.is_available():
        pytest.fail("this test needs a HIP device")
    wl = _workload()
    q, k, v = _dev(wl, "q"), _dev(wl, "k"), _dev(wl, "v")
    o, lse = aah.attn_fwd(q, k, v, wl.windows, wl.scale, sinks=wl.sinks)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    for h, (W, S) in enumerate(zip(WINDOWS, SINKS)):
        ro, rl = oracle.attn_fwd_rows_ref(wl.q[0, h], wl.k[0, h], wl.v[0, h], W, wl.scale, ROWS, sink=S)
        got = o[0, h, ROWS].float().cpu().numpy().astype(np.float64)
        bound = np.maximum(O_TOL_BF16, np.abs(ro) * 2.0 ** -8)
        assert (np.abs(got - ro) - bound).max() <= 0, f"head {h}: max |err| {np.abs(got - ro).max():.3e}"
        assert np.abs(lse[0, h, ROWS].cpu().numpy() - rl).max() < LSE_TOL_BF16, f"head {h}"


@pytest.mark.gpu
def test_long_sequence_backward_slices():
    if not torch.cuda.is_available():
        pytest.fail("this test needs a HIP device")
    wl = _workload()
    q, k, v, do = _dev(wl, "q"), _dev(wl, "k"), _dev(wl, "v"), _dev(wl, "do")
    o, lse = aah.attn_fwd(q, k, v, wl.windows, wl.scale, sinks=wl.sinks)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, scale=wl.scale, sinks=wl.sinks)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    T = T_LONG
    checked = {"dq": [], "dk": [], "dv": []}  # (head, slice, device rows, oracle rows)
    for h, W in enumerate(WINDOWS[:3]):  # heads without sinks
        gq, gk, gv = (t[0, h].float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
        half = max(2 * W, 128)
        for c in (0, 40000, T // 2 + 7, T - 1):
            a, b = max(0, c - half), min(T, c + half)
            rq, rk, rv = slice_bwd(wl, (0, h), W, a, b)
            q_rows, k_rows = exact_rows(T, W, a, b)
            for name, got, ref, rows in (("dq", gq, rq, q_rows), ("dk", gk, rk, k_rows), ("dv", gv, rv, k_rows)):
                checked[name].append((h, (a, b), got[rows], ref[rows - a]))
    # Bound: 3e-2 of the gradient's largest magnitude over the checked rows of all heads (a window-1
    # head's exact dQ and dK are 0; the device's are fp32 rounding of dP - D).
    for name, items in checked.items():
        scale = max(np.abs(r).max() for _, _, _, r in items)
        for h, (a, b), g, r in items:
            err = np.abs(g - r).max()
            assert err <= GRAD_REL * scale, f"{name} head {h} slice [{a}, {b}): {err:.3e} vs {GRAD_REL * scale:.3e}"
