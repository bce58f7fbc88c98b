"""Seeded random shapes through the C ABI against the oracle: batch, query heads, key/value heads, length,
head dimension, dtype, windows and sink sizes drawn from one generator (the list below is fixed by its seed),
forward and backward.  Small layers have few work items, so the binding's split launches run here too.
Bounds as in tests/test_gpu_parity.py.  Random decoding layers likewise, against oracle.decode_ref and the
cache storage rule."""
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


def _decode_shapes(n=24, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H_kv = int(rng.integers(1, 4))
        H = H_kv * int(rng.integers(1, 6))
        T_max = int(rng.integers(8, 1500))
        d = int(rng.choice([32, 64, 128]))
        windows = [int(x) for x in rng.integers(1, T_max + 40, size=H)]
        sinks = None if rng.random() < 0.5 else [int(x) for x in rng.integers(0, T_max // 2 + 1, size=H)]
        T0 = int(rng.integers(0, T_max - 3))
        out.append((H, H_kv, T_max, d, windows, sinks, T0))
    return out


@pytest.mark.parametrize("case", range(24))
def test_random_decode_steps(case):
    """Random layers of trimmed caches: a prefill of T0 positions (none when T0 = 0), then three decoding
    steps per sequence (the second sequence a step behind), each against the oracle; the caches against the
    storage rule at the end."""
    if not torch.cuda.is_available():
        pytest.fail("this test needs a HIP device")
    H, H_kv, T_max, d, windows, sinks, T0 = _decode_shapes()[case]
    print(f"decode case {case}: H={H} H_kv={H_kv} T_max={T_max} d={d} T0={T0} windows={windows} sinks={sinks}",
          flush=True)
    B, steps = 2, 3
    L = T0 + steps
    rng = np.random.default_rng(500 + case)
    host, devs = [], []
    for heads in (H, H_kv, H_kv):
        bits = synth.bf16_bits(rng.standard_normal((B, heads, L, d), dtype=np.float32))
        host.append(synth.bf16_to_f32(bits).astype(np.float64))
        devs.append(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda"))
    (qh, kh, vh), (q, k, v) = host, devs
    scale = 1.0 / np.sqrt(d)
    R = aah.kv_cache_rows(windows, T_max, sinks=sinks, H_kv=H_kv)
    kc = torch.zeros((B, R, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    if T0 > 0:
        aah.kv_cache_fill(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(), windows, T_max, kcache=kc,
                          vcache=vc, sinks=sinks)
    ws = torch.zeros(aah.decode_workspace_size(windows, B, T_max, d, sinks=sinks, H_kv=H_kv), dtype=torch.uint8,
                     device="cuda")
    bi = np.arange(B)
    for i in range(steps):
        p = np.array([T0 + i, T0 + max(0, i - 1)])
        pos = torch.tensor(p, dtype=torch.int32, device="cuda")
        qt, kt, vt = q[bi, :, p].contiguous(), k[bi, :, p].contiguous(), v[bi, :, p].contiguous()
        o, lse = aah.attn_decode(qt, kt, vt, kc, vc, pos, windows, T_max, scale=scale, workspace=ws, sinks=sinks)
        ref_o, ref_l = oracle.decode_ref(qh[bi, :, p], kh, vh, windows, p, T_max, scale, sinks=sinks)
        got = o.float().cpu().numpy().astype(np.float64)
        assert (np.abs(got - ref_o) - np.maximum(O_TOL_BF16, np.abs(ref_o) * 2.0 ** -8)).max() <= 0, i
        assert np.abs(lse.cpu().numpy() - ref_l).max() < 1e-3, i
    torch.cuda.synchronize()
    for cache, hist in ((kc, kh), (vc, vh)):
        rows, valid = oracle.cache_content_ref(hist, windows, [T0 + steps, T0 + steps - 1], T_max, sinks)
        assert np.array_equal(cache.float().cpu().numpy().astype(np.float64)[valid], rows[valid])


def _split_shapes(n=10, seed=77):
    """One sequence, few heads, long windows: layers whose items are few and long, so the forward, the
    diagnostic forward and both backward kernels take their split launches (head 0 always sees every key)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H_kv = int(rng.choice([1, 2, 3]))
        H = H_kv * int(rng.integers(1, 4))
        T = int(rng.integers(1700, 2700))
        d = int(rng.choice([32, 64, 128]))
        windows = [T + 5] + [int(rng.choice([1, 64, 300, 1000, 1800, T + 50])) for _ in range(H - 1)]
        sinks = None if rng.random() < 0.3 else [int(x) for x in rng.choice([0, 1, 64, 130, 700], size=H)]
        out.append((H, H_kv, T, d, windows, sinks))
    return out


@pytest.mark.parametrize("case", range(10))
def test_random_split_layer(case):
    """Forward, diagnostics and backward of seeded small layers through the split launches, against the
    oracle (bounds as above; entropy and norm as in tests/test_gpu_features.py)."""
    if not torch.cuda.is_available():
        pytest.fail("this test needs a HIP device")
    H, H_kv, T, d, windows, sinks = _split_shapes()[case]
    print(f"split case {case}: H={H} H_kv={H_kv} T={T} d={d} windows={windows} sinks={sinks}", flush=True)
    wl = synth.random_workload(1, H, T, d, windows, dtype="bf16", seed=3000 + case, backward=True, sinks=sinks,
                               H_kv=H_kv)
    assert aah.fwd_workspace_size(wl.windows, 1, H, T, d, sinks=sinks, H_kv=H_kv) > 0
    assert aah.fwd_workspace_size(wl.windows, 1, H, T, d, sinks=sinks, H_kv=H_kv, diag=True) > 0
    q, k, v, do = (_dev(wl, x, "bf16") for x in ("q", "k", "v", "do"))
    o, lse, ent, nrm = aah.attn_fwd_diag(q, k, v, wl.windows, wl.scale, sinks=sinks)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, wl.scale, sinks=sinks)
    torch.cuda.synchronize()
    O, L = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, sinks=sinks)
    got = o.float().cpu().numpy().astype(np.float64)
    assert (np.abs(got - O) - np.maximum(O_TOL_BF16, np.abs(O) * 2.0 ** -8)).max() <= 0
    assert np.abs(lse.cpu().numpy() - L).max() < LSE_TOL_BF16
    E, N = oracle.attn_row_stats_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, sinks=sinks)
    u = 2.0 ** -8 * 1.01
    vmax = np.repeat(np.linalg.norm(wl.v.astype(np.float64), axis=-1).max(axis=-1)[..., None], H // H_kv, axis=1)
    e_err = np.abs(ent.cpu().numpy().astype(np.float64) - E)
    assert (e_err - (2 * u * E + u + 1e-4)).max() <= 0, f"entropy max err {e_err.max():.3e}"
    n_err = np.abs(nrm.cpu().numpy().astype(np.float64) - N)
    assert (n_err - (2 * u * vmax + 1e-4)).max() <= 0, f"norm max err {n_err.max():.3e}"
    refs = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, wl.do, sinks=sinks)
    for name, g, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        err = np.abs(g.float().cpu().numpy() - ref).max()
        assert err <= GRAD_REL * np.abs(ref).max(), (name, err)
