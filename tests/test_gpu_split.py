"""Split forward launches (long items' key ranges in chunks, merged afterwards) against the fp64 oracle.

A bf16 forward with fewer work items than the device holds workgroups splits every item longer than
the chunk length when the caller passes aah_attn_fwd_workspace_size bytes of workspace (the binding
does).  Tolerances as for every bf16 forward (tests/test_gpu_parity.py): O within max(1e-2, 2^-8 |O|),
LSE within 4e-3; each chunk's weights are rounded against the chunk's own reference, which the same
bounds cover.
"""
import ctypes

import numpy as np
import pytest
import torch

import head_causal_local_amd as aah
import oracle
import synth
from head_causal_local_amd._lib import lib

pytestmark = pytest.mark.gpu

O_TOL_BF16 = 1e-2
LSE_TOL_BF16 = 4e-3
BF16, F32 = 0, 1


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a HIP device")


def _dev(wl, key):
    return torch.from_numpy(wl.bits[key].view(np.int16)).view(torch.bfloat16).to("cuda")


def _ws_bytes(windows, B, H, T, d, sinks=None, dt=BF16, H_kv=None):
    w = np.ascontiguousarray(windows, dtype=np.int32)
    P = ctypes.POINTER(ctypes.c_int32)
    sp = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.int32).ctypes.data_as(P)
    return lib().aah_attn_fwd_workspace_size(w.ctypes.data_as(P), sp, B, H, H if H_kv is None else H_kv, T, d, dt)


def _fwd_unsplit(q, k, v, windows, scale, sinks=None):
    """The forward with no workspace: one workgroup per item, every item writes its own rows."""
    B, H, T, d = q.shape
    H_kv = k.shape[1]
    w = np.ascontiguousarray(windows, dtype=np.int32)
    P = ctypes.POINTER(ctypes.c_int32)
    sk = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.int32)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    st = lib().aah_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), w.ctypes.data_as(P),
                            None if sk is None else sk.ctypes.data_as(P), B, H, H_kv, T, d, BF16,
                            float(scale), o.data_ptr(), lse.data_ptr(), None, 0,
                            torch.cuda.current_stream().cuda_stream)
    aah.check(st)
    return o, lse


def _check_full(wl, o, lse):
    O, L = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, sinks=wl.sinks)
    got = o.float().cpu().numpy().astype(np.float64)
    bound = np.maximum(O_TOL_BF16, np.abs(O) * 2.0 ** -8)
    assert (np.abs(got - O) - bound).max() <= 0, f"max |dO| {np.abs(got - O).max():.3e}"
    assert np.abs(lse.cpu().numpy() - L).max() < LSE_TOL_BF16


def test_split_applies_only_where_it_should():
    """Workspace (and so a split launch) only for bf16 with too few items, some of them long."""
    _require_gpu()
    single = synth.make_workload(1)
    assert _ws_bytes(single.windows, 1, 16, 4096, 64) > 0          # 512 items: splits
    assert _ws_bytes([4096] * 32, 4, 32, 4096, 64) == 0            # 4096 items fill the device
    assert _ws_bytes([4096] * 16, 1, 16, 4096, 64, dt=F32) == 0   # the fp32 path never splits
    assert _ws_bytes([256] * 4, 1, 4, 4096, 64, sinks=[128] * 4) == 0  # sink + 256: no long item
    assert _ws_bytes([2048, 256] * 2, 1, 4, 4096, 64, sinks=[64, 128] * 2) > 0
    assert _ws_bytes([1024] * 4, 1, 4, 1024, 64) == 0              # no item longer than the shortest chunk
    assert _ws_bytes([0] * 4, 1, 4, 512, 64) == 0                  # invalid window: no workspace


@pytest.mark.parametrize("B,H,T,d,windows", [
    (1, 1, 4096, 64, [4096]),            # 64-tile items: several chunks each
    (1, 2, 2000, 64, [2000, 300]),        # ragged tail, mixed split / unsplit items
    (1, 3, 1777, 32, [1777, 64, 1]),
    (2, 2, 2048, 128, [2048, 100]),
    (1, 4, 3000, 64, [1, 17, 2999, 5000]),
])
def test_split_forward_matches_oracle(B, H, T, d, windows):
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=B * 131 + H * 7 + T + d, backward=False)
    assert _ws_bytes(wl.windows, B, H, T, d) > 0  # every case has items longer than the chunk
    o, lse = aah.attn_fwd(_dev(wl, "q"), _dev(wl, "k"), _dev(wl, "v"), wl.windows, wl.scale)
    torch.cuda.synchronize()
    _check_full(wl, o, lse)


def test_split_forward_grouped_heads_matches_oracle():
    """Grouped K/V heads take the split launch too (B=1, 8 query heads over 2 K/V heads, T=4096: 256 items,
    fewer than the device holds): every row of O and LSE against the oracle, which reads head h's keys from
    K/V head h // 4; split and unsplit launches agree within the bf16 bounds."""
    _require_gpu()
    B, H, H_kv, T, d = 1, 8, 2, 4096, 64
    windows = [4096, 512, 2048, 1, 4096, 3000, 100, 4096]
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=77, backward=False, H_kv=H_kv)
    assert _ws_bytes(wl.windows, B, H, T, d, H_kv=H_kv) > 0
    q, k, v = _dev(wl, "q"), _dev(wl, "k"), _dev(wl, "v")
    o, lse = aah.attn_fwd(q, k, v, wl.windows, wl.scale)
    ou, lu = _fwd_unsplit(q, k, v, wl.windows, wl.scale)
    torch.cuda.synchronize()
    _check_full(wl, o, lse)
    a, b = o.float().cpu().numpy(), ou.float().cpu().numpy()
    assert (np.abs(a - b) - np.maximum(2 * O_TOL_BF16, np.abs(b) * 2.0 ** -7)).max() <= 0
    assert (lse - lu).abs().max().item() < 2 * LSE_TOL_BF16


def test_caller_workspace_through_the_binding():
    """attn_fwd with a workspace the caller keeps: one of fwd_workspace_size bytes gives the split launch's
    results bitwise (the same as the binding's own allocation), an empty one the unsplit launch's."""
    _require_gpu()
    wl = synth.make_workload(1)
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    q, k, v = _dev(wl, "q"), _dev(wl, "k"), _dev(wl, "v")
    n = aah.fwd_workspace_size(wl.windows, B, H, T, d)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o1, l1 = aah.attn_fwd(q, k, v, wl.windows, wl.scale, workspace=ws)
    o2, l2 = aah.attn_fwd(q, k, v, wl.windows, wl.scale)
    o3, l3 = aah.attn_fwd(q, k, v, wl.windows, wl.scale, workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    ou, lu = _fwd_unsplit(q, k, v, wl.windows, wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, ou) and torch.equal(l3, lu)


def test_split_close_to_unsplit_and_deterministic():
    """The single-layer workload (B=1 H=16 T=4096): split and one-workgroup-per-item launches agree within
    the bf16 bounds, and repeated split launches are bitwise equal."""
    _require_gpu()
    wl = synth.make_workload(1)
    q, k, v = _dev(wl, "q"), _dev(wl, "k"), _dev(wl, "v")
    o1, l1 = aah.attn_fwd(q, k, v, wl.windows, wl.scale)
    o2, l2 = aah.attn_fwd(q, k, v, wl.windows, wl.scale)
    ou, lu = _fwd_unsplit(q, k, v, wl.windows, wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    a, b = o1.float().cpu().numpy(), ou.float().cpu().numpy()
    assert (np.abs(a - b) - np.maximum(2 * O_TOL_BF16, np.abs(b) * 2.0 ** -7)).max() <= 0
    assert (l1 - lu).abs().max().item() < 2 * LSE_TOL_BF16


def test_split_concurrent_streams_and_misaligned_workspace():
    """Two split forwards on two streams (each with its own workspace) equal the sequential results; a
    workspace that is large enough but not 256-byte aligned is refused before anything is written."""
    _require_gpu()
    wls = [synth.random_workload(1, 2, 4096, 64, [4096, 3000], dtype="bf16", seed=s, backward=False)
           for s in (5, 6)]
    ins = [tuple(_dev(wl, key) for key in ("q", "k", "v")) for wl in wls]
    seq = [aah.attn_fwd(*x, wl.windows, wl.scale) for x, wl in zip(ins, wls)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    par = []
    for st, x, wl in zip(streams, ins, wls):
        with torch.cuda.stream(st):
            par.append(aah.attn_fwd(*x, wl.windows, wl.scale))
    torch.cuda.synchronize()
    for (o1, l1), (o2, l2) in zip(seq, par):
        assert torch.equal(o1, o2) and torch.equal(l1, l2)

    wl, (q, k, v) = wls[0], ins[0]
    need = _ws_bytes(wl.windows, 1, 2, 4096, 64)
    assert need > 0
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 2, 4096), 7.0, dtype=torch.float32, device="cuda")
    w = np.ascontiguousarray(wl.windows, dtype=np.int32)
    st = lib().aah_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), None, 1, 2, 2, 4096, 64, BF16,
                            float(wl.scale), o.data_ptr(), lse.data_ptr(), ws.data_ptr() + 16, need,
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 1  # AAH_ERR_INVALID_ARG, as for every misaligned workspace
    assert bool((o.float() == 7.0).all()) and bool((lse == 7.0).all())


GRAD_REL = 3e-2


def _bwd_ws_bytes(windows, B, H, T, d, sinks=None, H_kv=None):
    w = np.ascontiguousarray(windows, dtype=np.int32)
    P = ctypes.POINTER(ctypes.c_int32)
    sp = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.int32).ctypes.data_as(P)
    return lib().aah_attn_bwd_split_workspace_size(w.ctypes.data_as(P), sp, B, H, H if H_kv is None else H_kv, T, d,
                                                   BF16)


@pytest.mark.parametrize("B,H,T,d,windows", [
    (1, 2, 4096, 64, [4096, 2048]),
    (1, 3, 2000, 32, [2000, 1, 700]),
    (1, 2, 3000, 128, [5000, 100]),
])
def test_split_backward_matches_oracle(B, H, T, d, windows):
    """Few-item backward shapes: the binding passes the split workspace, dQ and dK/dV chunks are summed."""
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=T + d, backward=True)
    assert _bwd_ws_bytes(wl.windows, B, H, T, d) > aah.workspace_size(B, H, T, d, "bf16")
    q, k, v, do = (_dev(wl, key) for key in ("q", "k", "v", "do"))
    o, lse = aah.attn_fwd(q, k, v, wl.windows, wl.scale)
    dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, wl.scale)
    torch.cuda.synchronize()
    gq, gk, gv = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, wl.do)
    for name, got, ref in (("dq", dq, gq), ("dk", dk, gk), ("dv", dv, gv)):
        err = np.abs(got.float().cpu().numpy() - ref).max()
        assert err <= GRAD_REL * np.abs(ref).max(), (name, err)


def test_split_backward_close_to_unsplit_and_deterministic():
    """B=1 H=16 T=4096 (the single layer with dO): split and unsplit backward agree within the gradient bound,
    and repeated split calls are bitwise equal; a layer with enough items asks for no split workspace."""
    _require_gpu()
    wl = synth.random_workload(1, 16, 4096, 64, synth.make_workload(1).windows, dtype="bf16", seed=3, backward=True)
    q, k, v, do = (_dev(wl, key) for key in ("q", "k", "v", "do"))
    o, lse = aah.attn_fwd(q, k, v, wl.windows, wl.scale)
    need_split = _bwd_ws_bytes(wl.windows, 1, 16, 4096, 64)
    assert need_split > 0
    g1 = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, wl.scale)
    g2 = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, wl.scale)
    plain = torch.empty(aah.workspace_size(1, 16, 4096, 64, "bf16"), dtype=torch.uint8, device="cuda")
    gu = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, wl.scale, workspace=plain)
    torch.cuda.synchronize()
    for a, b, c in zip(g1, g2, gu):
        assert torch.equal(a, b)
        ref = c.float()
        assert (a.float() - ref).abs().max().item() <= 2 * GRAD_REL * ref.abs().max().item()
    assert _bwd_ws_bytes([4096] * 32, 4, 32, 4096, 64) == 0


def test_split_forward_sinks_matches_oracle():
    """Sink heads ("Autonomy-of-Heads", section 5) take the split launch: only the first chunk of an item (the
    one that starts at its window's first tile) visits the sink tiles, so no sink key counts twice.  B=1,
    H=4, ragged T=3000: heads with sink 64 / window 2000 and sink 300 / window 1500 have items of 25-33 key
    tiles, cut into chunks; every row against the oracle, and split against unsplit within the bf16 bounds."""
    _require_gpu()
    B, H, T, d = 1, 4, 3000, 64
    windows, sinks = [2000, 256, 3000, 1500], [64, 128, 0, 300]
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=91, backward=False, sinks=sinks)
    assert _ws_bytes(wl.windows, B, H, T, d, sinks=sinks) > 0
    q, k, v = _dev(wl, "q"), _dev(wl, "k"), _dev(wl, "v")
    o, lse = aah.attn_fwd(q, k, v, wl.windows, wl.scale, sinks=sinks)
    o2, l2 = aah.attn_fwd(q, k, v, wl.windows, wl.scale, sinks=sinks)
    ou, lu = _fwd_unsplit(q, k, v, wl.windows, wl.scale, sinks=sinks)
    torch.cuda.synchronize()
    _check_full(wl, o, lse)
    assert torch.equal(o, o2) and torch.equal(lse, l2)
    a, b = o.float().cpu().numpy(), ou.float().cpu().numpy()
    assert (np.abs(a - b) - np.maximum(2 * O_TOL_BF16, np.abs(b) * 2.0 ** -7)).max() <= 0
    assert (lse - lu).abs().max().item() < 2 * LSE_TOL_BF16


@pytest.mark.parametrize("B,H,H_kv,T,d,windows,sinks", [
    (1, 4, 2, 2048, 64, [2048, 300, 1000, 64], None),            # groups whose heads end at different tiles
    (1, 4, 4, 2500, 64, [256, 2500, 1000, 128], [128, 0, 64, 300]),  # sink key tiles run to the last query
    (1, 4, 1, 2000, 128, [600, 2000, 64, 900], [0, 0, 200, 64]),     # one K/V head for all, with sinks
])
def test_split_backward_sinks_and_groups_match_oracle(B, H, H_kv, T, d, windows, sinks):
    """Few-item backward with grouped K/V heads (AAH appendix A.3) and sink keys: dQ chunks (sink tiles with
    the first chunk only) and dK/dV chunks (a grouped item's query-tile range cut, each chunk running every
    head of the group over its part) summed by the merges.  Gradients against the oracle; split against the
    unsplit launch within twice the bound; repeated split calls bitwise equal."""
    _require_gpu()
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=T + 3 * d + H_kv, backward=True,
                               sinks=sinks, H_kv=H_kv)
    need = _bwd_ws_bytes(wl.windows, B, H, T, d, sinks=sinks, H_kv=H_kv)
    assert need > aah.workspace_size(B, H, T, d, "bf16")
    q, k, v, do = (_dev(wl, key) for key in ("q", "k", "v", "do"))
    o, lse = aah.attn_fwd(q, k, v, wl.windows, wl.scale, sinks=sinks)
    g1 = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, wl.scale, sinks=sinks)
    g2 = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, wl.scale, sinks=sinks)
    plain = torch.empty(aah.workspace_size(B, H, T, d, "bf16"), dtype=torch.uint8, device="cuda")
    gu = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, wl.scale, workspace=plain, sinks=sinks)
    torch.cuda.synchronize()
    refs = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, wl.do, sinks=sinks)
    for name, a, b, c, ref in zip(("dq", "dk", "dv"), g1, g2, gu, refs):
        assert torch.equal(a, b), name
        err = np.abs(a.float().cpu().numpy() - ref).max()
        assert err <= GRAD_REL * np.abs(ref).max(), (name, err)
        ru = c.float()
        assert (a.float() - ru).abs().max().item() <= 2 * GRAD_REL * ru.abs().max().item(), name
