"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances: fp32 workloads max-abs 1e-5; bf16 outputs max-abs 1e-2 (per
element max(1e-2, 2^-8 |reference|): above |O| = 2.56 a bf16 output cannot be
held to 1e-2 by rounding alone, since its spacing there is 2^-7 |O| or more);
gradients 3e-2 x max |gradient|.  The log-sum-exp of the bf16 path is the log
of the sum of the bf16-rounded weights that also enter P V (round to nearest
keeps 8 significant bits, so each weight carries a relative error of at most
the unit roundoff 2^-8, and so does their sum): |error| <= -ln(1 - 2^-8) =
3.92e-3, reached only when one or two weights dominate a row, plus fp32
accumulation and exp2 rounding well below 1e-4, hence 4e-3.  The fp32 path
sums fp32 weights: 1e-5.
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
    """Device copy of a workload tensor with exactly the generator's bits."""
    if wl.dtype == "bf16":
        return torch.from_numpy(wl.bits[key].view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(getattr(wl, key)).to("cuda")


def assert_bf16_close(got, ref):
    bound = np.maximum(O_TOL_BF16, np.abs(ref) * 2.0 ** -8)
    excess = np.abs(got - ref) - bound
    assert excess.max() <= 0, f"max |err| {np.abs(got - ref).max():.3e}, worst excess {excess.max():.3e}"


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


_CACHE = {}


def workload(idx):
    if idx not in _CACHE:
        _CACHE[idx] = synth.make_workload(idx)
    return _CACHE[idx]


def run_fwd(wl):
    q, k, v = dev(wl, "q"), dev(wl, "k"), dev(wl, "v")
    o, lse = aah.attn_fwd(q, k, v, wl.windows, wl.scale)
    torch.cuda.synchronize()
    return o, lse


# ---------------------------------------------------------------- forward

def test_tiny_fp32_workload():
    """The tiny fp32 workload (B=1 H=4 T=256 d=32, windows 16/32/64/256) at max-abs 1e-5."""
    _require_gpu()
    wl = workload(0)
    o, lse = run_fwd(wl)
    O, L = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale)
    assert np.abs(host(o) - O).max() < TOL_F32
    assert np.abs(host(lse) - L).max() < TOL_F32


BF16_SHAPES = [
    # B, H, T, d, windows        (several tiles, ragged tails, windows below/at/above T)
    (2, 5, 333, 64, [1, 7, 64, 200, 1000]),
    (1, 3, 200, 32, [5, 100, 200]),
    (1, 2, 300, 128, [3, 300]),
    (1, 4, 1, 64, [1, 2, 3, 4]),
    (1, 3, 129, 64, [129, 128, 64]),
    (2, 2, 640, 64, [512, 65]),
]


@pytest.mark.parametrize("B,H,T,d,windows", BF16_SHAPES)
def test_bf16_forward_small(B, H, T, d, windows):
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=B * 1000 + T, backward=False)
    o, lse = run_fwd(wl)
    O, L = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale)
    assert_bf16_close(host(o), O)
    assert np.abs(host(lse) - L).max() < LSE_TOL_BF16


@pytest.mark.parametrize("B,H,T,d,windows", [(1, 3, 200, 32, [5, 100, 200]), (2, 2, 130, 64, [1, 64]),
                                             (1, 2, 70, 128, [3, 70])])
def test_fp32_forward_small(B, H, T, d, windows):
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="f32", seed=7, backward=False)
    o, lse = run_fwd(wl)
    O, L = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale)
    assert np.abs(host(o) - O).max() < TOL_F32
    assert np.abs(host(lse) - L).max() < TOL_F32


def test_window_one_returns_v_exactly():
    _require_gpu()
    wl = synth.random_workload(2, 3, 150, 64, [1, 1, 1], dtype="bf16", seed=5, backward=False)
    o, _ = run_fwd(wl)
    assert torch.equal(o, dev(wl, "v"))


def test_forward_deterministic_and_head_permutation():
    """Two runs are bitwise equal; permuting heads permutes outputs bitwise (bucket/scatter commutes)."""
    _require_gpu()
    wl = synth.random_workload(2, 6, 700, 64, [512, 1, 4096, 64, 700, 128], dtype="bf16", seed=9, backward=False)
    q, k, v = dev(wl, "q"), dev(wl, "k"), dev(wl, "v")
    o1, l1 = aah.attn_fwd(q, k, v, wl.windows)
    o2, l2 = aah.attn_fwd(q, k, v, wl.windows)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    perm = [4, 2, 0, 5, 1, 3]
    op, lp = aah.attn_fwd(q[:, perm].contiguous(), k[:, perm].contiguous(), v[:, perm].contiguous(),
                          wl.windows[perm])
    torch.cuda.synchronize()
    assert torch.equal(op, o1[:, perm]) and torch.equal(lp, l1[:, perm])


SAMPLE_ROWS = [0, 1, 31, 32, 63, 64, 127, 128, 511, 512, 513, 1000, 1023, 1024, 2047, 2048, 3000, 4095]


def _check_sampled_rows(wl, o, lse, heads):
    on, ln = host(o), host(lse)
    worst = 0.0
    for b, h in heads:
        Or, Lr = oracle.attn_fwd_rows_ref(wl.q[b, h], wl.k[b, h], wl.v[b, h], int(wl.windows[h]), wl.scale,
                                          SAMPLE_ROWS)
        assert_bf16_close(on[b, h, SAMPLE_ROWS], Or)
        assert np.abs(ln[b, h, SAMPLE_ROWS] - Lr).max() < LSE_TOL_BF16, (b, h)
        worst = max(worst, float(np.abs(on[b, h, SAMPLE_ROWS] - Or).max()))
    return worst


def test_single_layer_workload_sampled():
    """B=1 H=16 T=4096 d=64 bf16, windows drawn from {512,...,4096}: every head, sampled rows."""
    _require_gpu()
    wl = workload(1)
    o, lse = run_fwd(wl)
    _check_sampled_rows(wl, o, lse, [(0, h) for h in range(wl.H)])
    assert torch.isfinite(o.float()).all()


def test_1b_layer_workload_sampled():
    """B=4 H=32 T=4096 d=64 bf16 with the grouped window hierarchy: sampled heads and rows."""
    _require_gpu()
    wl = workload(3)
    o, lse = run_fwd(wl)
    heads = [(b, h) for b in (0, 3) for h in (0, 5, 12, 17, 28, 31)]
    _check_sampled_rows(wl, o, lse, heads)
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("idx", ["4a", "4b", "4c"])
def test_coverage_controls_sampled(idx):
    _require_gpu()
    wl = synth.make_workload(idx)
    o, lse = run_fwd(wl)
    _check_sampled_rows(wl, o, lse, [(1, 0), (2, 1), (3, 30), (0, 31)])


# ---------------------------------------------------------------- backward

def _grad_check(got, ref, rel=GRAD_REL, name=""):
    scale = max(np.abs(ref).max(), 1e-12)
    err = np.abs(got - ref).max()
    assert err <= rel * scale, f"{name}: max err {err:.3e} vs bound {rel * scale:.3e}"


@pytest.mark.parametrize("B,H,T,d,windows", [(1, 3, 200, 64, [1, 17, 200]), (2, 2, 333, 64, [64, 500]),
                                             (1, 2, 150, 32, [3, 150]), (1, 2, 140, 128, [9, 140])])
def test_bf16_backward_small(B, H, T, d, windows):
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=11 + T, backward=True)
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    o, lse = aah.attn_fwd(q, k, v, wl.windows)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, wl.do)
    _grad_check(host(dq), rq, name="dq")
    _grad_check(host(dk), rk, name="dk")
    _grad_check(host(dv), rv, name="dv")


@pytest.mark.parametrize("B,H,T,d,windows", [(1, 3, 200, 32, [1, 17, 200]), (1, 2, 130, 64, [64, 500])])
def test_fp32_backward_small(B, H, T, d, windows):
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="f32", seed=3 + T, backward=True)
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    o, lse = aah.attn_fwd(q, k, v, wl.windows)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, wl.do)
    _grad_check(host(dq), rq, rel=1e-4, name="dq")
    _grad_check(host(dk), rk, rel=1e-4, name="dk")
    _grad_check(host(dv), rv, rel=1e-4, name="dv")


def test_1b_layer_backward_sampled_heads():
    """Full-size B=4 H=32 T=4096 d=64 backward; heads of every window class checked in full."""
    _require_gpu()
    wl = workload(3)
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    o, lse = aah.attn_fwd(q, k, v, wl.windows)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows)
    torch.cuda.synchronize()
    distinct = {}
    for h, w in enumerate(wl.windows):
        distinct.setdefault(int(w), h)
    heads = [(b, h) for b, h in zip((0, 1, 2, 3), sorted(distinct.values()))]
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.attn_bwd_ref(wl.q[sl], wl.k[sl], wl.v[sl], wl.windows[h:h + 1], wl.scale, wl.do[sl])
        _grad_check(host(dq[sl]), rq, name=f"dq b{b} h{h}")
        _grad_check(host(dk[sl]), rk, name=f"dk b{b} h{h}")
        _grad_check(host(dv[sl]), rv, name=f"dv b{b} h{h}")
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()


def test_backward_deterministic_and_steps():
    """The backward writes every gradient once (no atomics): two runs are bitwise equal, and the
    two separate steps (dQ, then dK/dV) reproduce the combined call bitwise."""
    _require_gpu()
    wl = synth.random_workload(2, 3, 700, 64, [64, 700, 300], dtype="bf16", seed=17, backward=True)
    q, k, v, do = dev(wl, "q"), dev(wl, "k"), dev(wl, "v"), dev(wl, "do")
    o, lse = aah.attn_fwd(q, k, v, wl.windows)
    g1 = aah.attn_bwd(q, k, v, o, do, lse, wl.windows)
    g2 = aah.attn_bwd(q, k, v, o, do, lse, wl.windows)
    ws = torch.empty(aah.workspace_size(2, 3, 700, 64, "bf16"), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    aah.attn_bwd_dq(q, k, v, o, do, lse, wl.windows, dq, ws)   # also writes the workspace rows
    aah.attn_bwd_dkdv(q, k, v, do, wl.windows, dk, dv, ws)
    torch.cuda.synchronize()
    for a, b, c in zip(g1, g2, (dq, dk, dv)):
        assert torch.equal(a, b)
        assert torch.equal(a, c)


@pytest.mark.parametrize("B,T", [(0, 64), (2, 0)])
def test_empty_problems(B, T):
    """B = 0 or T = 0: every call returns empty results (nothing is computed; empty tensors have no storage),
    and a prefill of no tokens leaves the caches as they were."""
    _require_gpu()
    H, H_kv, d = 4, 2, 64
    windows = [3, 16, 64, 200]
    for dt in (torch.bfloat16, torch.float32):
        q = torch.zeros((B, H, T, d), dtype=dt, device="cuda")
        k = torch.zeros((B, H_kv, T, d), dtype=dt, device="cuda")
        v = torch.zeros_like(k)
        o, lse = aah.attn_fwd(q, k, v, windows)
        assert o.shape == (B, H, T, d) and lse.shape == (B, H, T)
        dq, dk, dv = aah.attn_bwd(q, k, v, o, torch.zeros_like(q), lse, windows)
        assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
    q = torch.zeros((B, H, T, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H_kv, T, d), dtype=torch.bfloat16, device="cuda")
    o, lse, ent, onorm = aah.attn_fwd_diag(q, k, k, windows)
    assert ent.shape == (B, H, T) and onorm.shape == (B, H, T)
    T_max = 128
    R = aah.kv_cache_rows(windows, T_max, H_kv=H_kv)
    kc = torch.full((B, R, d), 7.0, dtype=torch.bfloat16, device="cuda")
    vc = torch.full((B, R, d), -3.0, dtype=torch.bfloat16, device="cuda")
    aah.kv_cache_fill(k, k, windows, T_max, kcache=kc, vcache=vc)
    torch.cuda.synchronize()
    assert bool((kc == 7.0).all()) and bool((vc == -3.0).all())
    if B == 0:
        qd = torch.zeros((0, H, d), dtype=torch.bfloat16, device="cuda")
        kn = torch.zeros((0, H_kv, d), dtype=torch.bfloat16, device="cuda")
        pos = torch.zeros((0,), dtype=torch.int32, device="cuda")
        od, ld = aah.attn_decode(qd, kn, kn, kc, vc, pos, windows, T_max)
        assert od.shape == (0, H, d) and ld.shape == (0, H)
        aah.attn_decode_noalloc(qd, kn, kn, kc, vc, pos, windows, T_max, out=torch.empty_like(qd),
                                lse=torch.empty((0, H), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
