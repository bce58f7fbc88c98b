"""Seeded random shapes through the C ABI against the oracle: batch, query heads, key/value heads, length,
head dimension, dtype, windows and sink sizes drawn from one generator (the list below is fixed by its seed),
forward and backward.  Small layers have few work items, so the binding's split launches run here too.
Bounds as in tests/test_gpu_parity.py."""
import numpy as np
import pytest
import torch

import head_causal_local_amd as aah
import oracle
import synth

pytestmark = pytest.mark.gpu

O_TOL_BF16, LSE_TOL_BF16, TOL_F32, GRAD_REL = 1e-2, 4e-3, 1e-5, 3e-2


def _shapes(n=48, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 4))
        H_kv = int(rng.integers(1, 4))
        H = H_kv * int(rng.integers(1, 5))
        T = int(rng.integers(1, 700))
        d = int(rng.choice([32, 64, 128]))
        dtype = str(rng.choice(["bf16", "f32"]))
        windows = [int(x) for x in rng.integers(1, T + 50, size=H)]
        sinks = None if rng.random() < 0.5 else [int(x) for x in rng.integers(0, T + 1, size=H)]
        out.append((B, H, H_kv, T, d, dtype, windows, sinks))
    return out


def _dev(wl, key, dtype):
    if dtype == "bf16":
        return torch.from_numpy(wl.bits[key].view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(getattr(wl, key)).to("cuda")


@pytest.mark.parametrize("case", range(48))
def test_random_shape_forward_backward(case):
    if not torch.cuda.is_available():
        pytest.fail("this test needs a HIP device")
    B, H, H_kv, T, d, dtype, windows, sinks = _shapes()[case]
    print(f"case {case}: B={B} H={H} H_kv={H_kv} T={T} d={d} {dtype} windows={windows} sinks={sinks}", flush=True)
    wl = synth.random_workload(B, H, T, d, windows, dtype=dtype, seed=1000 + case, backward=True, sinks=sinks,
                               H_kv=H_kv)
    q, k, v, do = (_dev(wl, x, dtype) for x in ("q", "k", "v", "do"))
    o, lse = aah.attn_fwd(q, k, v, wl.windows, wl.scale, sinks=wl.sinks)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, wl.scale, sinks=wl.sinks)
    torch.cuda.synchronize()
    O, L = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, sinks=wl.sinks)
    got = o.float().cpu().numpy().astype(np.float64)
    if dtype == "bf16":
        assert (np.abs(got - O) - np.maximum(O_TOL_BF16, np.abs(O) * 2.0 ** -8)).max() <= 0
        assert np.abs(lse.cpu().numpy() - L).max() < LSE_TOL_BF16
    else:
        assert np.abs(got - O).max() <= TOL_F32
        assert np.abs(lse.cpu().numpy() - L).max() <= TOL_F32
    refs = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, wl.do, sinks=wl.sinks)
    rel = GRAD_REL if dtype == "bf16" else 1e-4
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        scale = max(np.abs(r).max(), 1e-12)
        err = np.abs(g.float().cpu().numpy() - r).max()
        assert err <= rel * scale, f"{name}: {err:.3e} vs {rel * scale:.3e}"
