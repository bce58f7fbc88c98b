"""GPU parity of grouped key/value heads (query head h reads key/value head h / G) through the C ABI.

Expected values: oracle.attn_fwd_ref / attn_bwd_ref with K, V [B, H_kv, T, d] on the bf16-rounded inputs the
device sees; tolerances as for plain heads (bf16 outputs max(1e-2, 2^-8 |ref|), lse 4e-3, gradients
3e-2 x max |gradient| -- a shared head's dK / dV sum G query heads' contributions, each carrying the same bf16
rounding of P and dS, so the bound relative to the sum's largest entry is unchanged; fp32 1e-5 / 1e-4).
Identities: the same inputs with K / V repeated per group through the plain path give the same O, LSE and dQ
bit for bit, and dK / dV equal to the group sums of the plain path's.
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
    assert excess.max() <= 0, f"max |err| {np.abs(got - ref).max():.3e}"


def grad_close(got, ref, rel, name):
    bound = rel * max(np.abs(ref).max(), 1e-12)
    err = np.abs(got - ref).max()
    assert err <= bound, f"{name}: max err {err:.3e} vs bound {bound:.3e}"


SHAPES = [
    # B, H, H_kv, T, d, windows, sinks
    (2, 4, 2, 333, 64, [1, 64, 200, 1000], None),
    (1, 6, 3, 200, 32, [5, 100, 5, 17, 200, 3], [0, 0, 40, 0, 0, 2]),
    (1, 8, 1, 300, 128, [3, 300, 64, 9, 128, 1, 77, 256], None),
    (2, 4, 4, 150, 64, [7, 150, 1, 33], None),
]


@pytest.mark.parametrize("B,H,H_kv,T,d,windows,sinks", SHAPES)
def test_bf16_gqa_forward_backward(B, H, H_kv, T, d, windows, sinks):
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=H * 10 + T, backward=True, sinks=sinks,
                               H_kv=H_kv)
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    o, lse = aah.attn_fwd(q, k, v, wl.windows, sinks=wl.sinks)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, sinks=wl.sinks)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape
    O, L = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, sinks=wl.sinks)
    assert_bf16_close(host(o), O)
    assert np.abs(host(lse) - L).max() < LSE_TOL_BF16
    rq, rk, rv = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, wl.do, sinks=wl.sinks)
    grad_close(host(dq), rq, GRAD_REL, "dq")
    grad_close(host(dk), rk, GRAD_REL, "dk")
    grad_close(host(dv), rv, GRAD_REL, "dv")


@pytest.mark.parametrize("B,H,H_kv,T,d,windows,sinks", [(1, 4, 2, 130, 64, [9, 64, 130, 1], [0, 3, 0, 0]),
                                                       (1, 3, 1, 100, 32, [5, 50, 100], None)])
def test_fp32_gqa_forward_backward(B, H, H_kv, T, d, windows, sinks):
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="f32", seed=T, backward=True, sinks=sinks, H_kv=H_kv)
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    o, lse = aah.attn_fwd(q, k, v, wl.windows, sinks=wl.sinks)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, sinks=wl.sinks)
    torch.cuda.synchronize()
    O, L = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, sinks=wl.sinks)
    assert np.abs(host(o) - O).max() < 1e-5
    assert np.abs(host(lse) - L).max() < 1e-5
    rq, rk, rv = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, wl.do, sinks=wl.sinks)
    grad_close(host(dq), rq, 1e-4, "dq")
    grad_close(host(dk), rk, 1e-4, "dk")
    grad_close(host(dv), rv, 1e-4, "dv")


def test_gqa_matches_plain_heads_over_repeated_kv():
    """Grouped call vs the plain call with K / V repeated per group: O, LSE, dQ bitwise; dK, dV = group sums."""
    _require_gpu()
    B, H, H_kv, T, d = 2, 6, 2, 400, 64
    windows = [16, 400, 64, 1, 200, 128]
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=5, backward=True, H_kv=H_kv)
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    G = H // H_kv
    kr, vr = (x.repeat_interleave(G, dim=1).contiguous() for x in (k, v))
    o, lse = aah.attn_fwd(q, k, v, windows)
    o2, lse2 = aah.attn_fwd(q, kr, vr, windows)
    g1 = aah.attn_bwd(q, k, v, o, do, lse, windows)
    g2 = aah.attn_bwd(q, kr, vr, o2, do, lse2, windows)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    assert torch.equal(g1[0], g2[0])
    for a, b, name in ((g1[1], g2[1], "dk"), (g1[2], g2[2], "dv")):
        summed = b.float().reshape(B, H_kv, G, T, d).sum(2)
        grad_close(host(a), summed.cpu().numpy().astype(np.float64), 1e-2, name)


def test_gqa_deterministic_steps_and_features():
    """Two runs bitwise equal; dQ then dK/dV as separate calls equal the combined call; the diagnostic forward
    keeps O / LSE, and the features of a query head carry its group's K / V statistics."""
    _require_gpu()
    wl = synth.random_workload(2, 8, 500, 64, [64, 500, 32, 300, 1, 128, 256, 17], dtype="bf16", seed=8,
                               backward=True, H_kv=2)
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    o, lse = aah.attn_fwd(q, k, v, wl.windows)
    g1 = aah.attn_bwd(q, k, v, o, do, lse, wl.windows)
    g2 = aah.attn_bwd(q, k, v, o, do, lse, wl.windows)
    ws = torch.empty(aah.workspace_size(2, 8, 500, 64, "bf16"), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    aah.attn_bwd_dq(q, k, v, o, do, lse, wl.windows, dq, ws)
    aah.attn_bwd_dkdv(q, k, v, do, wl.windows, dk, dv, ws)
    o3, lse3, ent, nrm = aah.attn_fwd_diag(q, k, v, wl.windows)
    x = aah.head_features(q, k, v, wl.windows, ent, nrm)
    torch.cuda.synchronize()
    for a, b, c in zip(g1, g2, (dq, dk, dv)):
        assert torch.equal(a, b) and torch.equal(a, c)
    assert torch.equal(o, o3) and torch.equal(lse, lse3)
    ref = oracle.head_features_ref(wl.q, wl.k, wl.v, wl.windows, host(ent), host(nrm))
    assert np.allclose(host(x), ref, rtol=1e-5, atol=1e-6)
    e_ref, n_ref = oracle.attn_row_stats_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale)
    assert np.abs(host(ent) - e_ref).max() < 0.05 and np.abs(host(nrm) - n_ref).max() < 0.1


SAMPLE_ROWS = [0, 1, 127, 128, 511, 512, 1023, 2048, 3000, 4095]


def test_gqa_layer_sampled():
    """B=4 H=32 H_kv=8 T=4096 d=128 with per-query-head windows: sampled rows of several heads, and the full
    gradients of key/value head 2 (query heads 8-11) of batch entry 1."""
    _require_gpu()
    wl = synth.make_workload(6)
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    o, lse = aah.attn_fwd(q, k, v, wl.windows)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows)
    torch.cuda.synchronize()
    on, ln = host(o), host(lse)
    G = 4
    for b, h in ((0, 0), (1, 9), (2, 22), (3, 31)):
        Or, Lr = oracle.attn_fwd_rows_ref(wl.q[b, h], wl.k[b, h // G], wl.v[b, h // G], int(wl.windows[h]),
                                          wl.scale, SAMPLE_ROWS)
        assert_bf16_close(on[b, h, SAMPLE_ROWS], Or)
        assert np.abs(ln[b, h, SAMPLE_ROWS] - Lr).max() < LSE_TOL_BF16
    b, g = 1, 2
    rq, rk, rv = oracle.attn_bwd_ref(wl.q[b:b + 1, g * G:(g + 1) * G], wl.k[b:b + 1, g:g + 1], wl.v[b:b + 1, g:g + 1],
                                     wl.windows[g * G:(g + 1) * G], wl.scale, wl.do[b:b + 1, g * G:(g + 1) * G])
    grad_close(host(dq[b:b + 1, g * G:(g + 1) * G]), rq, GRAD_REL, "dq")
    grad_close(host(dk[b:b + 1, g:g + 1]), rk, GRAD_REL, "dk")
    grad_close(host(dv[b:b + 1, g:g + 1]), rv, GRAD_REL, "dv")
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t.float()).all()
