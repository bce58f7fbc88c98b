"""GPU parity of the sink + recent-window variant ("Autonomy-of-Heads", section 5) through the C ABI.

Expected values come from oracle.attn_fwd_ref / attn_bwd_ref with the same sinks, on the
bf16-rounded inputs the device sees.  Tolerances are those of the plain-window tests: bf16
outputs max(1e-2, 2^-8 |ref|), lse 4e-3, gradients 3e-2 x max |gradient|; fp32 1e-5 (1e-4
relative for fp32 gradients).
"""
import numpy as np
import pytest
import torch

import head_causal_local_amd as aah
import oracle
import synth

pytestmark = pytest.mark.gpu

O_TOL_BF16 = 1e-2
LSE_TOL_BF16 = 4e-3
TOL_F32 = 1e-5
GRAD_REL = 3e-2


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a HIP device")


def dev(wl, key):
    if wl.dtype == "bf16":
        return torch.from_numpy(wl.bits[key].view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(getattr(wl, key)).to("cuda")


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_bf16_close(got, ref):
    bound = np.maximum(O_TOL_BF16, np.abs(ref) * 2.0 ** -8)
    excess = np.abs(got - ref) - bound
    assert excess.max() <= 0, f"max |err| {np.abs(got - ref).max():.3e}, worst excess {excess.max():.3e}"


def grad_close(got, ref, rel, name):
    bound = rel * max(np.abs(ref).max(), 1e-12)
    err = np.abs(got - ref).max()
    assert err <= bound, f"{name}: max err {err:.3e} vs bound {bound:.3e}"


SHAPES = [
    # B, H, T, d, windows, sinks    (sink tiles before the window, sinks inside the first window
    # tile, sinks reaching past T - W (trimmed), W = 1, ragged tails, several tiles)
    (2, 5, 333, 64, [1, 7, 64, 200, 1000], [1, 64, 70, 300, 5]),
    (1, 4, 700, 64, [256, 64, 1, 100], [128, 129, 700, 33]),
    (1, 3, 200, 32, [5, 100, 17], [3, 40, 200]),
    (1, 2, 300, 128, [3, 64], [130, 1]),
    (1, 2, 1, 64, [1, 2], [1, 4]),
    (2, 2, 640, 64, [65, 256], [0, 128]),
]


@pytest.mark.parametrize("B,H,T,d,windows,sinks", SHAPES)
def test_bf16_forward_with_sinks(B, H, T, d, windows, sinks):
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=B * 100 + T, backward=False, sinks=sinks)
    o, lse = aah.attn_fwd(dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), wl.windows, wl.scale, sinks=wl.sinks)
    torch.cuda.synchronize()
    O, L = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, sinks=wl.sinks)
    assert_bf16_close(host(o), O)
    assert np.abs(host(lse) - L).max() < LSE_TOL_BF16


@pytest.mark.parametrize("B,H,T,d,windows,sinks", [(1, 3, 200, 32, [5, 100, 17], [3, 40, 200]),
                                                   (2, 2, 150, 64, [1, 64], [65, 2]),
                                                   (1, 2, 140, 128, [9, 30], [1, 100])])
def test_fp32_forward_with_sinks(B, H, T, d, windows, sinks):
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="f32", seed=T, backward=False, sinks=sinks)
    o, lse = aah.attn_fwd(dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), wl.windows, wl.scale, sinks=wl.sinks)
    torch.cuda.synchronize()
    O, L = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, sinks=wl.sinks)
    assert np.abs(host(o) - O).max() < TOL_F32
    assert np.abs(host(lse) - L).max() < TOL_F32


@pytest.mark.parametrize("B,H,T,d,windows,sinks", [(1, 3, 333, 64, [1, 17, 100], [64, 3, 150]),
                                                   (2, 2, 300, 64, [64, 256], [128, 1]),
                                                   (1, 2, 150, 32, [3, 20], [2, 70]),
                                                   (1, 2, 260, 128, [9, 64], [129, 5])])
def test_bf16_backward_with_sinks(B, H, T, d, windows, sinks):
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=7 + T, backward=True, sinks=sinks)
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    o, lse = aah.attn_fwd(q, k, v, wl.windows, sinks=wl.sinks)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, sinks=wl.sinks)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, wl.do, sinks=wl.sinks)
    grad_close(host(dq), rq, GRAD_REL, "dq")
    grad_close(host(dk), rk, GRAD_REL, "dk")
    grad_close(host(dv), rv, GRAD_REL, "dv")


@pytest.mark.parametrize("B,H,T,d,windows,sinks", [(1, 3, 200, 32, [1, 17, 60], [5, 70, 1]),
                                                   (1, 2, 130, 64, [20, 64], [64, 3])])
def test_fp32_backward_with_sinks(B, H, T, d, windows, sinks):
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="f32", seed=3 + T, backward=True, sinks=sinks)
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    o, lse = aah.attn_fwd(q, k, v, wl.windows, sinks=wl.sinks)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, sinks=wl.sinks)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, wl.do, sinks=wl.sinks)
    grad_close(host(dq), rq, 1e-4, "dq")
    grad_close(host(dk), rk, 1e-4, "dk")
    grad_close(host(dv), rv, 1e-4, "dv")


def test_zero_and_redundant_sinks_equal_plain_window_bitwise():
    """All-zero sinks, and sinks that change nothing (heads whose window covers T), run the plain
    kernels: outputs and gradients equal the call without sinks bit for bit."""
    _require_gpu()
    wl = synth.random_workload(2, 3, 500, 64, [17, 500, 4096], dtype="bf16", seed=31, backward=True)
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    o0, l0 = aah.attn_fwd(q, k, v, wl.windows)
    g0 = aah.attn_bwd(q, k, v, o0, do, l0, wl.windows)
    for sinks in ([0, 0, 0], [0, 128, 7]):
        o1, l1 = aah.attn_fwd(q, k, v, wl.windows, sinks=sinks)
        g1 = aah.attn_bwd(q, k, v, o1, do, l1, wl.windows, sinks=sinks)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
        assert all(torch.equal(a, b) for a, b in zip(g0, g1))


def test_sinks_deterministic_and_steps():
    """Two runs are bitwise equal; dQ then dK/dV as separate calls reproduce the combined call."""
    _require_gpu()
    wl = synth.random_workload(2, 3, 700, 64, [64, 256, 300], dtype="bf16", seed=17, backward=True,
                               sinks=[128, 128, 1])
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    o, lse = aah.attn_fwd(q, k, v, wl.windows, sinks=wl.sinks)
    o2, lse2 = aah.attn_fwd(q, k, v, wl.windows, sinks=wl.sinks)
    g1 = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, sinks=wl.sinks)
    g2 = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, sinks=wl.sinks)
    ws = torch.empty(aah.workspace_size(2, 3, 700, 64, "bf16"), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    aah.attn_bwd_dq(q, k, v, o, do, lse, wl.windows, dq, ws, sinks=wl.sinks)
    aah.attn_bwd_dkdv(q, k, v, do, wl.windows, dk, dv, ws, sinks=wl.sinks)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b, c in zip(g1, g2, (dq, dk, dv)):
        assert torch.equal(a, b) and torch.equal(a, c)


SAMPLE_ROWS = [0, 1, 127, 128, 129, 255, 256, 383, 384, 385, 511, 512, 1000, 2047, 2048, 3000, 4095]


def test_streaming_workload_sampled():
    """B=4 H=32 T=4096 d=64: heads 0-15 full causal, heads 16-31 sink 128 + recent 256.
    Forward: sampled rows of retrieval and streaming heads; backward: four heads in full."""
    _require_gpu()
    wl = synth.make_workload(5)
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    o, lse = aah.attn_fwd(q, k, v, wl.windows, sinks=wl.sinks)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, sinks=wl.sinks)
    torch.cuda.synchronize()
    on, ln = host(o), host(lse)
    for b, h in ((0, 0), (1, 15), (2, 16), (3, 20), (0, 31)):
        Or, Lr = oracle.attn_fwd_rows_ref(wl.q[b, h], wl.k[b, h], wl.v[b, h], int(wl.windows[h]), wl.scale,
                                          SAMPLE_ROWS, sink=int(wl.sinks[h]))
        assert_bf16_close(on[b, h, SAMPLE_ROWS], Or)
        assert np.abs(ln[b, h, SAMPLE_ROWS] - Lr).max() < LSE_TOL_BF16, (b, h)
    for b, h in ((1, 3), (2, 16), (3, 29)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.attn_bwd_ref(wl.q[sl], wl.k[sl], wl.v[sl], wl.windows[h:h + 1], wl.scale, wl.do[sl],
                                         sinks=wl.sinks[h:h + 1])
        grad_close(host(dq[sl]), rq, GRAD_REL, f"dq b{b} h{h}")
        grad_close(host(dk[sl]), rk, GRAD_REL, f"dk b{b} h{h}")
        grad_close(host(dv[sl]), rv, GRAD_REL, f"dv b{b} h{h}")
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t.float()).all()
