"""local_window_attention: the autograd form of the forward and backward calls.

O against the oracle's forward and the gradients that autograd returns against the oracle's matrix-calculus
backward (bounds of tests/test_gpu_parity.py), grouped K/V heads and sinks included; and bitwise equal to the
explicit attn_fwd / attn_bwd calls it wraps (the binding only marshals arguments)."""
import numpy as np
import pytest
import torch

import head_causal_local_amd as aah
import oracle
import synth

O_TOL_BF16, GRAD_REL = 1e-2, 3e-2


def _dev(wl, key, dtype):
    if dtype == "bf16":
        return torch.from_numpy(wl.bits[key].view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(getattr(wl, key)).to("cuda")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,B,H,H_kv,T,d,windows,sinks", [
    ("bf16", 2, 4, 2, 333, 64, [1, 64, 200, 1000], [0, 3, 0, 0]),
    ("bf16", 1, 3, 3, 150, 128, [7, 150, 33], None),
    ("f32", 1, 4, 1, 200, 32, [5, 200, 17, 1], None),
])
def test_autograd_matches_oracle_and_explicit_calls(dtype, B, H, H_kv, T, d, windows, sinks):
    if not torch.cuda.is_available():
        pytest.fail("this test needs a HIP device")
    wl = synth.random_workload(B, H, T, d, windows, dtype=dtype, seed=T + d, backward=True, sinks=sinks, H_kv=H_kv)
    q, k, v, do = (_dev(wl, x, dtype) for x in ("q", "k", "v", "do"))
    qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = aah.local_window_attention(qg, kg, vg, wl.windows, sinks=wl.sinks)
    o.backward(do)
    torch.cuda.synchronize()
    # the explicit calls, bitwise
    o2, lse2 = aah.attn_fwd(q, k, v, wl.windows, wl.scale, sinks=wl.sinks)
    dq2, dk2, dv2 = aah.attn_bwd(q, k, v, o2, do, lse2, wl.windows, wl.scale, sinks=wl.sinks)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    assert torch.equal(qg.grad, dq2) and torch.equal(kg.grad, dk2) and torch.equal(vg.grad, dv2)
    assert qg.grad.dtype == q.dtype and kg.grad.shape == k.shape
    # the oracle
    O, _ = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, sinks=wl.sinks)
    got = o.detach().float().cpu().numpy().astype(np.float64)
    if dtype == "bf16":
        assert (np.abs(got - O) - np.maximum(O_TOL_BF16, np.abs(O) * 2.0 ** -8)).max() <= 0
    else:
        assert np.abs(got - O).max() <= 1e-5
    refs = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, wl.do, sinks=wl.sinks)
    rel = GRAD_REL if dtype == "bf16" else 1e-4
    for name, g, r in zip(("dq", "dk", "dv"), (qg.grad, kg.grad, vg.grad), refs):
        err = np.abs(g.float().cpu().numpy() - r).max()
        assert err <= rel * np.abs(r).max(), f"{name}: {err:.3e}"


def test_autograd_refuses_host_tensors():
    q = torch.zeros((1, 2, 8, 32), requires_grad=True)
    with pytest.raises(ValueError):
        aah.local_window_attention(q, q, q, [4, 4])
