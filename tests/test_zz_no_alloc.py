"""The allocation-free decoding step (aah_attn_decode_noalloc) against aah_attn_decode, through the C ABI.

The two entry points run the same decode kernel over the same cache layout and chunking; the allocation-free
one builds its plan tables on the device and keeps counters, tables and partials in the library's per-device
scratch array.  So its outputs and cache rows must equal the workspace call's bit for bit, and both must meet
the decode bounds against the oracle (o within max(1e-2, 2^-8 |ref|), lse within 1e-3).  Two calls in a row,
the second with a smaller step, check that nothing left in the shared array from the first leaks into the
second; a step too large for the array is refused before any HIP call.
"""
import ctypes

import numpy as np
import pytest
import torch

import head_causal_local_amd as aah
import oracle
from head_causal_local_amd._lib import lib
from synth import bf16_bits, bf16_to_f32

pytestmark = pytest.mark.gpu

O_TOL = 1e-2
LSE_TOL = 1e-3


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a HIP device")


def _history(B, H, H_kv, L, d, seed):
    rng = np.random.default_rng(seed)
    host, devs = [], []
    for heads in (H, H_kv, H_kv):
        bits = bf16_bits(rng.standard_normal((B, heads, L, d), dtype=np.float32))
        host.append(bf16_to_f32(bits).astype(np.float64))
        devs.append(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda"))
    return host, devs


def _check_o(got, ref):
    got = got.float().cpu().numpy().astype(np.float64)
    bound = np.maximum(O_TOL, np.abs(ref) * 2.0 ** -8)
    assert (np.abs(got - ref) - bound).max() <= 0, f"max |err| {np.abs(got - ref).max():.3e}"


CASES = [
    # B, H, H_kv, d, windows, sinks, T_max, T0, steps -- the second step is smaller than the first
    (3, 8, 4, 64, [64, 700, 300, 1000, 1, 513, 40, 1000], [0, 4, 0, 16, 0, 0, 2, 0], 1024, 900, 4),
    (1, 2, 2, 32, [16, 200], None, 256, 100, 3),
]


def _run_case(B, H, H_kv, d, windows, sinks, T_max, T0, steps, seed):
    L = T0 + steps
    (qh, kh, vh), (q, k, v) = _history(B, H, H_kv, L, d, seed)
    scale = 1.0 / np.sqrt(d)
    kc1, vc1 = aah.kv_cache_fill(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(), windows, T_max, sinks=sinks)
    kc2, vc2 = kc1.clone(), vc1.clone()
    ws = torch.zeros(aah.decode_workspace_size(windows, B, T_max, d, sinks=sinks, H_kv=H_kv), dtype=torch.uint8,
                     device="cuda")
    bi = np.arange(B)
    for i in range(steps):
        p = np.array([T0 + i - (b % 2) * min(i, 2) for b in range(B)])  # sequences at different positions
        print(f"no-alloc decode: B={B} H={H} H_kv={H_kv} d={d} T_max={T_max} step {i} pos {p.tolist()}", flush=True)
        pos = torch.tensor(p, dtype=torch.int32, device="cuda")
        qt, kt, vt = q[bi, :, p].contiguous(), k[bi, :, p].contiguous(), v[bi, :, p].contiguous()
        o1, l1 = aah.attn_decode(qt, kt, vt, kc1, vc1, pos, windows, T_max, scale=scale, workspace=ws, sinks=sinks)
        o2 = torch.full_like(o1, 3.0)
        l2 = torch.full_like(l1, 3.0)
        aah.attn_decode_noalloc(qt, kt, vt, kc2, vc2, pos, windows, T_max, o2, l2, scale=scale, sinks=sinks)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), i
        ref_o, ref_l = oracle.decode_ref(qh[bi, :, p], kh, vh, windows, p, T_max, scale, sinks=sinks)
        _check_o(o2, ref_o)
        assert np.abs(l2.cpu().numpy() - ref_l).max() < LSE_TOL, i
    assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2)


def test_noalloc_decode_equals_workspace_decode_two_calls_in_a_row():
    _require_gpu()
    for n, case in enumerate(CASES):
        _run_case(*case, seed=100 + n)


def test_noalloc_decode_graph_replays():
    """Captured once, the allocation-free step replays with the plan built inside the graph: each replay
    equals the eager call, with the workspace call and other eager work in between."""
    _require_gpu()
    B, H, H_kv, d, windows, T_max, T0 = 2, 4, 2, 64, [32, 300, 128, 512], 512, 400
    (qh, kh, vh), (q, k, v) = _history(B, H, H_kv, T0 + 1, d, seed=7)
    kc, vc = aah.kv_cache_fill(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(), windows, T_max)
    pos = torch.full((B,), T0, dtype=torch.int32, device="cuda")
    qt, kt, vt = (x[:, :, T0].contiguous() for x in (q, k, v))
    o_e, l_e = torch.empty_like(qt), torch.empty((B, H), dtype=torch.float32, device="cuda")
    aah.attn_decode_noalloc(qt, kt, vt, kc, vc, pos, windows, T_max, o_e, l_e)
    torch.cuda.synchronize()
    o_g, l_g = torch.empty_like(o_e), torch.empty_like(l_e)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            aah.attn_decode_noalloc(qt, kt, vt, kc, vc, pos, windows, T_max, o_g, l_g, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(3):
        o_g.fill_(5.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(l_g, l_e), r
        # eager work on the same array between replays: a different, smaller step
        aah.attn_decode_noalloc(qt[:1], kt[:1], vt[:1], kc[:1].clone(), vc[:1].clone(), pos[:1], windows, T_max,
                                torch.empty_like(qt[:1]), torch.empty((1, H), dtype=torch.float32, device="cuda"))
        torch.cuda.synchronize()


def test_noalloc_decode_refuses_a_step_too_large_for_its_array():
    """A step whose partials exceed the library's array is refused (AAH_ERR_UNSUPPORTED) before any HIP call;
    the outputs stay as they were."""
    _require_gpu()
    B, H, d, T_max = 1, 2, 128, 1 << 21   # 2 x 8192 chunks: 8.5 MB of partials
    w = np.array([T_max, T_max], dtype=np.int32)
    small = torch.zeros(256, dtype=torch.bfloat16, device="cuda")
    o = torch.full((B, H, d), 9.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), 9.0, dtype=torch.float32, device="cuda")
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    st = lib().aah_attn_decode_noalloc(small.data_ptr(), small.data_ptr(), small.data_ptr(), small.data_ptr(),
                                       small.data_ptr(), pos.data_ptr(),
                                       w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), None, B, H, H, T_max, d, 0,
                                       0.1, o.data_ptr(), lse.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == 2
    assert "scratch" in lib().aah_last_error_detail().decode()
    assert bool((o.float() == 9.0).all()) and bool((lse == 9.0).all())
