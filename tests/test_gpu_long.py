"""Long sequences through the C ABI: T = 2^17 positions per head (32 times the bench layers), and the
largest T the ABI accepts at d = 128 (4,194,303: one head's fp32 slice just under 2^31 bytes).

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


def fwd_row_slice(T, W, i):
    """The slice [a, i + 1) of the sequence holding every key row i of a window-W head sees (no sinks)."""
    return max(0, i - W + 1), i + 1


@pytest.mark.parametrize("W", [1, 7, 40])
def test_forward_row_slice_equals_full_sequence_oracle(W):
    """CPU pin of the forward slicing rule: the oracle run on `fwd_row_slice` gives row i exactly the whole
    sequence's output and log-sum-exp."""
    T = 300
    wl = synth.random_workload(1, 1, T, 8, [W], dtype="f32", seed=50 + W, backward=False)
    fo, fl = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, [W], wl.scale)
    for i in (0, 1, W - 1, W, 150, T - 1):
        if i < 0:
            continue
        a, b = fwd_row_slice(T, W, i)
        ro, rl = oracle.attn_fwd_rows_ref(wl.q[0, 0, a:b], wl.k[0, 0, a:b], wl.v[0, 0, a:b], W, wl.scale, [i - a])
        assert np.allclose(ro[0], fo[0, 0, i], rtol=0, atol=1e-12) and abs(rl[0] - fl[0, 0, i]) < 1e-12


# The largest T the ABI takes at d = 128: one head's fp32 [T, d] slice just under 2^31 bytes (its kernels
# address a slice with 32-bit byte offsets; T * d * 4 >= 2^31 is refused).
T_MAX_D128 = ((1 << 31) - 1) // (4 * 128)
MAX_WINDOWS = [40, 3]
MAX_ROWS = [0, 1, 39, 40, 41, 127, 128, T_MAX_D128 // 2, (1 << 21) + 5, T_MAX_D128 - 129, T_MAX_D128 - 128,
            T_MAX_D128 - 2, T_MAX_D128 - 1]


def _device_normal(shape, seed, dtype):
    """Seeded N(0, 1) inputs drawn on the device (a whole input set is 8-16 GiB); the oracle reads the same
    bits back, row slice by row slice."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(dtype)


def _rows64(t, h, a, b):
    return t[0, h, a:b].float().cpu().numpy().astype(np.float64)


@pytest.mark.gpu
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_largest_sequence_forward_and_backward(dt):
    """T = 4,194,303 at d = 128 (the fp32 slice's last row ends 512 bytes below 2^31): forward rows at the
    start, the middle and the end against the oracle on each row's slice, and backward slices at the start,
    past 2^21 rows and at the end (rows `exact_rows` keeps), bf16 and fp32."""
    if not torch.cuda.is_available():
        pytest.fail("this test needs a HIP device")
    T, d, H = T_MAX_D128, 128, len(MAX_WINDOWS)
    assert T * d * 4 < (1 << 31) <= (T + 1) * d * 4
    scale = 1.0 / np.sqrt(d)
    q, k, v, do = (_device_normal((1, H, T, d), 100 + i, dt) for i in range(4))
    o, lse = aah.attn_fwd(q, k, v, MAX_WINDOWS, scale)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, MAX_WINDOWS, scale=scale)
    torch.cuda.synchronize()
    o_tol = O_TOL_BF16 if dt == torch.bfloat16 else 1e-5
    l_tol = LSE_TOL_BF16 if dt == torch.bfloat16 else 1e-5
    for h, W in enumerate(MAX_WINDOWS):
        for i in MAX_ROWS:
            a, b = fwd_row_slice(T, W, i)
            ro, rl = oracle.attn_fwd_rows_ref(_rows64(q, h, a, b), _rows64(k, h, a, b), _rows64(v, h, a, b), W,
                                              scale, [i - a])
            got = o[0, h, i].float().cpu().numpy().astype(np.float64)
            bound = np.maximum(o_tol, np.abs(ro[0]) * 2.0 ** -8) if dt == torch.bfloat16 else o_tol
            assert (np.abs(got - ro[0]) - bound).max() <= 0, f"head {h} row {i}"
            assert abs(float(lse[0, h, i]) - rl[0]) < l_tol, f"head {h} row {i}"
        half = 2 * W + 64
        for c in (0, (1 << 21) + 5, T - 1):
            a, b = max(0, c - half), min(T, c + half)
            sl = (slice(0, 1), slice(h, h + 1), slice(a, b))
            rq, rk, rv = oracle.attn_bwd_ref(*(t[sl].float().cpu().numpy().astype(np.float64) for t in (q, k, v)),
                                             [W], scale, do[sl].float().cpu().numpy().astype(np.float64))
            q_rows, k_rows = exact_rows(T, W, a, b)
            for name, got, ref, rows in (("dq", dq, rq, q_rows), ("dk", dk, rk, k_rows), ("dv", dv, rv, k_rows)):
                g = _rows64(got, h, a, b)[rows - a]
                r = ref[0, 0, rows - a]
                err = np.abs(g - r).max()
                bound = (GRAD_REL if dt == torch.bfloat16 else 1e-4) * np.abs(r).max()
                assert err <= bound, f"{name} head {h} slice [{a}, {b}): {err:.3e} vs {bound:.3e}"
