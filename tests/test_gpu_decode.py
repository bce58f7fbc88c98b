"""GPU parity of decoding over per-head trimmed K/V caches, through the C ABI.

The expected values come from oracle.decode_ref / oracle.cache_content_ref on the same
bf16-rounded histories the device sees.  Outputs: bf16 o within 1e-2 max-abs (widened to
2^-8 |ref| above 2.56, as for the forward), fp32 lse within 1e-3 (the step sums fp32
weights, so only exp2 and accumulation rounding remain); cache rows bit-exact.
"""
import numpy as np
import pytest
import torch

import head_causal_local_amd as aah
import oracle
from synth import bf16_bits, bf16_to_f32

pytestmark = pytest.mark.gpu

O_TOL = 1e-2
LSE_TOL = 1e-3


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a HIP device")


def _history(B, H, L, d, seed):
    """bf16-exact fp32 histories q, k, v [B, H, L, d] and their device copies."""
    rng = np.random.default_rng(seed)
    host, devs = [], []
    for _ in range(3):
        bits = bf16_bits(rng.standard_normal((B, H, L, d), dtype=np.float32))
        host.append(bf16_to_f32(bits).astype(np.float64))
        devs.append(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda"))
    return host, devs


def _check_o(got, ref):
    got = got.float().cpu().numpy().astype(np.float64)
    bound = np.maximum(O_TOL, np.abs(ref) * 2.0 ** -8)
    assert (np.abs(got - ref) - bound).max() <= 0, f"max |err| {np.abs(got - ref).max():.3e}"


def _check_cache(kc, vc, kh, vh, windows, n_written, T_max):
    for cache, hist in ((kc, kh), (vc, vh)):
        rows, valid = oracle.cache_content_ref(hist, windows, n_written, T_max)
        got = cache.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(got[valid], rows[valid])


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("windows,T_max,T0", [
    ([1, 5, 256, 300], 300, 200),        # W = 1, a window filling the cache, one wider than T_max
    ([40, 513, 1000, 700], 1024, 700),   # rings of 40, 513 (3 chunks), 1000; ragged chunk tails
])
def test_prefill_then_decode_steps(d, windows, T_max, T0):
    """Prefill T0 positions, then 40 decoding steps; each step against the oracle, and the
    caches bit-exact against the storage rule at the end (several rings wrap around)."""
    _require_gpu()
    B, H, steps = 2, len(windows), 40
    L = T0 + steps
    (qh, kh, vh), (q, k, v) = _history(B, H, L, d, seed=d)
    scale = 1.0 / np.sqrt(d)
    kc, vc = aah.kv_cache_fill(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(), windows, T_max)
    _check_cache(kc, vc, kh, vh, windows, [T0, T0], T_max)
    ws = torch.zeros(aah.decode_workspace_size(windows, B, T_max, d), dtype=torch.uint8, device="cuda")
    # Sequence 1 repeats position T0 for its first 7 steps (a repeated step writes the same row and
    # gives the same output), so the two sequences sit at different positions afterwards.
    for i in range(steps):
        p = np.array([T0 + i, T0 + max(0, i - 7)])
        pos = torch.tensor(p, dtype=torch.int32, device="cuda")
        bi = np.arange(B)
        qt = q[bi, :, p].contiguous()
        kt = k[bi, :, p].contiguous()
        vt = v[bi, :, p].contiguous()
        o, lse = aah.attn_decode(qt, kt, vt, kc, vc, pos, windows, T_max, scale=scale, workspace=ws)
        ref_o, ref_l = oracle.decode_ref(qh[bi, :, p], kh, vh, windows, p, T_max, scale)
        _check_o(o, ref_o)
        assert np.abs(lse.cpu().numpy() - ref_l).max() < LSE_TOL, i
    torch.cuda.synchronize()
    _check_cache(kc, vc, kh, vh, windows, [T0 + steps, T0 + steps - 7], T_max)


def test_decode_from_empty_and_first_positions():
    """Positions 0, 1, 2 with nothing prefilled: the ring is filled by the steps themselves."""
    _require_gpu()
    B, H, d, T_max = 1, 3, 64, 64
    windows = [1, 2, 64]
    (qh, kh, vh), (q, k, v) = _history(B, H, 3, d, seed=11)
    R = aah.kv_cache_rows(windows, T_max)
    kc = torch.zeros((B, R, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for t in range(3):
        pos = torch.tensor([t], dtype=torch.int32, device="cuda")
        o, lse = aah.attn_decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                                 kc, vc, pos, windows, T_max, scale=0.125)
        ref_o, ref_l = oracle.decode_ref(qh[:, :, t], kh, vh, windows, np.array([t]), T_max, 0.125)
        _check_o(o, ref_o)
        assert np.abs(lse.cpu().numpy() - ref_l).max() < LSE_TOL
    # window 1: the output is the new token's value, bit for bit
    assert torch.equal(o[:, 0], v[:, 0, 2])


def test_decode_1b_layer_shape_sampled():
    """The 1B-scale layer's shape (B=4, H=32, d=64, T_max=4096, grouped windows) at position 4095
    after a full prefill; a sample of heads against the oracle, all heads finite."""
    _require_gpu()
    import synth
    wl = synth.make_workload(2)
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    k = torch.from_numpy(wl.bits["k"].view(np.int16)).view(torch.bfloat16).to("cuda")
    v = torch.from_numpy(wl.bits["v"].view(np.int16)).view(torch.bfloat16).to("cuda")
    q = torch.from_numpy(wl.bits["q"].view(np.int16)).view(torch.bfloat16).to("cuda")
    kc, vc = aah.kv_cache_fill(k[:, :, :T - 1].contiguous(), v[:, :, :T - 1].contiguous(), wl.windows, T)
    pos = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")
    o, lse = aah.attn_decode(q[:, :, T - 1].contiguous(), k[:, :, T - 1].contiguous(), v[:, :, T - 1].contiguous(),
                             kc, vc, pos, wl.windows, T, scale=wl.scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    for b, h in ((0, 0), (1, 12), (2, 28), (3, 31)):
        js = oracle.decode_positions(T - 1, int(wl.windows[h]), T)
        ref_o, ref_l = oracle.decode_ref(wl.q[b:b + 1, h:h + 1, T - 1], wl.k[b:b + 1, h:h + 1], wl.v[b:b + 1, h:h + 1],
                                         wl.windows[h:h + 1], np.array([T - 1]), T, wl.scale)
        _check_o(o[b:b + 1, h:h + 1], ref_o)
        assert abs(lse[b, h].item() - ref_l[0, 0]) < LSE_TOL
        assert len(js) == min(int(wl.windows[h]), T)


@pytest.mark.parametrize("idx", [3, 5, 6])
def test_decode_bench_layers_all_heads(idx):
    """The decode bench's layers at full size and in its launch configuration: the 1B-scale layer, the
    streaming-head layer (sinks 128 + recent 256 beside full-context heads) and the grouped layer (H = 32
    over H_kv = 8, d = 128); a prefill of positions 0 .. T - 2, then position T - 1; every (b, h) against
    the oracle."""
    _require_gpu()
    import synth
    wl = synth.make_workload(idx)
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    dev = lambda key: torch.from_numpy(wl.bits[key].view(np.int16)).view(torch.bfloat16).to("cuda")
    q, k, v = dev("q"), dev("k"), dev("v")
    kc, vc = aah.kv_cache_fill(k[:, :, :T - 1].contiguous(), v[:, :, :T - 1].contiguous(), wl.windows, T,
                               sinks=wl.sinks)
    pos = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")
    o, lse = aah.attn_decode(q[:, :, T - 1].contiguous(), k[:, :, T - 1].contiguous(), v[:, :, T - 1].contiguous(),
                             kc, vc, pos, wl.windows, T, scale=wl.scale, sinks=wl.sinks)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.decode_ref(wl.q[:, :, T - 1], wl.k, wl.v, wl.windows, np.full(B, T - 1), T, wl.scale,
                                     sinks=wl.sinks)
    _check_o(o, ref_o)
    assert np.abs(lse.cpu().numpy() - ref_l).max() < LSE_TOL


def test_decode_graph_replays_match_eager():
    """The step has no allocation or memset, so it can be captured in a HIP graph: every replay
    (with eager work and synchronisations in between) gives the eager result bit for bit."""
    _require_gpu()
    B, H, d, T_max = 2, 4, 64, 512
    windows = [16, 300, 512, 1000]
    (qh, kh, vh), (q, k, v) = _history(B, H, T_max, d, seed=21)
    p = T_max - 1
    kc, vc = aah.kv_cache_fill(k[:, :, :p].contiguous(), v[:, :, :p].contiguous(), windows, T_max)
    pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
    qt, kt, vt = (x[:, :, p].contiguous() for x in (q, k, v))
    ws = torch.zeros(aah.decode_workspace_size(windows, B, T_max, d), dtype=torch.uint8, device="cuda")
    o_eager, l_eager = aah.attn_decode(qt, kt, vt, kc, vc, pos, windows, T_max, workspace=ws)
    o_eager, l_eager = o_eager.clone(), l_eager.clone()
    o = torch.empty_like(o_eager)
    lse = torch.empty_like(l_eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            aah.attn_decode(qt, kt, vt, kc, vc, pos, windows, T_max, out=o, lse=lse, workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for r in range(4):
        o.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager) and torch.equal(lse, l_eager), r
        # eager work on the same workspace between replays
        aah.attn_decode(qt, kt, vt, kc, vc, pos, windows, T_max, workspace=ws)
    ref_o, ref_l = oracle.decode_ref(qh[:, :, p], kh, vh, windows, np.array([p, p]), T_max, 1.0 / np.sqrt(d))
    _check_o(o, ref_o)


# ---------------------------------------------------------------- sinks and grouped key/value heads

def _history_g(B, H, H_kv, L, d, seed):
    """bf16-exact histories q [B, H, L, d], k, v [B, H_kv, L, d] and their device copies."""
    rng = np.random.default_rng(seed)
    host, devs = [], []
    for heads in (H, H_kv, H_kv):
        bits = bf16_bits(rng.standard_normal((B, heads, L, d), dtype=np.float32))
        host.append(bf16_to_f32(bits).astype(np.float64))
        devs.append(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda"))
    return host, devs


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,H_kv,windows,sinks,T_max,T0", [
    # streaming heads (sinks), a head whose sinks reach past T_max - C (trimmed), full windows, W = 1
    (4, 4, [16, 300, 1, 40], [4, 10, 3, 300], 320, 12),
    # groups of three query heads over two key/value heads, different windows and sinks in a group
    (6, 2, [1, 64, 300, 7, 256, 33], [0, 5, 0, 128, 0, 2], 512, 200),
    # one key/value head for all query heads, rings of several chunks
    (4, 1, [600, 5, 1000, 129], [0, 130, 1, 0], 1024, 700),
    # groups larger than the kernel's rounds of four query heads: ten heads per group (rounds of 4, 4, 2),
    # mixed windows and sinks within the group
    (10, 1, [600, 5, 1000, 129, 1, 64, 300, 7, 256, 33], [0, 130, 1, 0, 0, 5, 0, 128, 0, 2], 1024, 700),
    # eight heads per group over two key/value heads (two full rounds each)
    (16, 2, [512, 64, 300, 1, 1024, 16, 700, 33] * 2, [0] * 16, 1024, 600),
])
def test_decode_sinks_and_groups(d, H, H_kv, windows, sinks, T_max, T0):
    """Prefill T0 positions, then 40 steps (sequence 1 repeats position T0 for its first 7 steps): every step
    against the oracle, and the caches bit-exact against the storage rule at the end."""
    _require_gpu()
    B, steps = 2, 40
    L = T0 + steps
    (qh, kh, vh), (q, k, v) = _history_g(B, H, H_kv, L, d, seed=d + H)
    scale = 1.0 / np.sqrt(d)
    kc, vc = aah.kv_cache_fill(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(), windows, T_max, sinks=sinks)
    for cache, hist in ((kc, kh), (vc, vh)):
        rows, valid = oracle.cache_content_ref(hist, windows, [T0, T0], T_max, sinks)
        assert np.array_equal(cache.float().cpu().numpy().astype(np.float64)[valid], rows[valid])
    ws = torch.zeros(aah.decode_workspace_size(windows, B, T_max, d, sinks=sinks, H_kv=H_kv), dtype=torch.uint8,
                     device="cuda")
    bi = np.arange(B)
    for i in range(steps):
        p = np.array([T0 + i, T0 + max(0, i - 7)])
        pos = torch.tensor(p, dtype=torch.int32, device="cuda")
        qt, kt, vt = q[bi, :, p].contiguous(), k[bi, :, p].contiguous(), v[bi, :, p].contiguous()
        o, lse = aah.attn_decode(qt, kt, vt, kc, vc, pos, windows, T_max, scale=scale, workspace=ws, sinks=sinks)
        ref_o, ref_l = oracle.decode_ref(qh[bi, :, p], kh, vh, windows, p, T_max, scale, sinks=sinks)
        _check_o(o, ref_o)
        assert np.abs(lse.cpu().numpy() - ref_l).max() < LSE_TOL, i
    torch.cuda.synchronize()
    for cache, hist in ((kc, kh), (vc, vh)):
        rows, valid = oracle.cache_content_ref(hist, windows, [T0 + steps, T0 + steps - 7], T_max, sinks)
        assert np.array_equal(cache.float().cpu().numpy().astype(np.float64)[valid], rows[valid])


def test_decode_sinks_from_empty_cache():
    """Positions 0 .. 11 with nothing prefilled and 5 sinks on a window of 2: the sink rows fill as the steps
    pass them, and are attended once the window has moved past them."""
    _require_gpu()
    B, H, d, T_max = 1, 2, 64, 64
    windows, sinks = [2, 64], [5, 0]
    (qh, kh, vh), (q, k, v) = _history_g(B, H, H, 12, d, seed=13)
    R = aah.kv_cache_rows(windows, T_max, sinks=sinks)
    kc = torch.zeros((B, R, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for t in range(12):
        pos = torch.tensor([t], dtype=torch.int32, device="cuda")
        o, lse = aah.attn_decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                                 kc, vc, pos, windows, T_max, scale=0.125, sinks=sinks)
        ref_o, ref_l = oracle.decode_ref(qh[:, :, t], kh, vh, windows, np.array([t]), T_max, 0.125, sinks=sinks)
        _check_o(o, ref_o)
        assert np.abs(lse.cpu().numpy() - ref_l).max() < LSE_TOL, t


def test_decode_grouped_graph_replays_match_eager():
    """Grouped heads with sinks captured in a HIP graph: every replay equals the eager call bit for bit."""
    _require_gpu()
    B, H, H_kv, d, T_max = 2, 8, 2, 128, 1024
    windows = [128, 1024, 256, 64, 512, 1024, 32, 256]
    sinks = [4, 0, 128, 0, 0, 0, 128, 16]
    (qh, kh, vh), (q, k, v) = _history_g(B, H, H_kv, T_max, d, seed=23)
    p = T_max - 1
    kc, vc = aah.kv_cache_fill(k[:, :, :p].contiguous(), v[:, :, :p].contiguous(), windows, T_max, sinks=sinks)
    pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
    qt, kt, vt = (x[:, :, p].contiguous() for x in (q, k, v))
    ws = torch.zeros(aah.decode_workspace_size(windows, B, T_max, d, sinks=sinks, H_kv=H_kv), dtype=torch.uint8,
                     device="cuda")
    o_eager, l_eager = aah.attn_decode(qt, kt, vt, kc, vc, pos, windows, T_max, workspace=ws, sinks=sinks)
    o_eager, l_eager = o_eager.clone(), l_eager.clone()
    o = torch.empty_like(o_eager)
    lse = torch.empty_like(l_eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            aah.attn_decode(qt, kt, vt, kc, vc, pos, windows, T_max, out=o, lse=lse, workspace=ws, stream=s,
                            sinks=sinks)
    torch.cuda.current_stream().wait_stream(s)
    for r in range(3):
        o.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager) and torch.equal(lse, l_eager), r
        aah.attn_decode(qt, kt, vt, kc, vc, pos, windows, T_max, workspace=ws, sinks=sinks)
    ref_o, ref_l = oracle.decode_ref(qh[:, :, p], kh, vh, windows, np.array([p, p]), T_max, 1.0 / np.sqrt(d),
                                     sinks=sinks)
    _check_o(o, ref_o)


@pytest.mark.parametrize("d,H,H_kv,windows,sinks", [
    # a full-context head of 65536 rows (256 chunks: the merge reads its partials in 16 batches) beside a
    # streaming head
    (64, 2, 2, [65536, 300], [0, 17]),
    # grouped heads: a group with the full-context ring and a sink head, a group with a ring of 5000 rows
    # (20 chunks: two merge batches) and a window of 1
    (128, 4, 2, [65536, 300, 5000, 1], [0, 17, 0, 0]),
])
def test_decode_long_context(d, H, H_kv, windows, sinks):
    """T_max = 65536: prefill 65533 positions, then 3 steps (sequence 1 repeats its first position once), each
    against the oracle over every attended position; the caches against the storage rule at the end."""
    _require_gpu()
    B, T_max, steps = 2, 65536, 3
    T0 = T_max - steps
    (qh, kh, vh), (q, k, v) = _history_g(B, H, H_kv, T_max, d, seed=7 + d)
    scale = 1.0 / np.sqrt(d)
    kc, vc = aah.kv_cache_fill(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(), windows, T_max, sinks=sinks)
    ws = torch.zeros(aah.decode_workspace_size(windows, B, T_max, d, sinks=sinks, H_kv=H_kv), dtype=torch.uint8,
                     device="cuda")
    bi = np.arange(B)
    for i in range(steps):
        p = np.array([T0 + i, T0 + max(0, i - 1)])
        pos = torch.tensor(p, dtype=torch.int32, device="cuda")
        qt, kt, vt = q[bi, :, p].contiguous(), k[bi, :, p].contiguous(), v[bi, :, p].contiguous()
        o, lse = aah.attn_decode(qt, kt, vt, kc, vc, pos, windows, T_max, scale=scale, workspace=ws, sinks=sinks)
        ref_o, ref_l = oracle.decode_ref(qh[bi, :, p], kh, vh, windows, p, T_max, scale, sinks=sinks)
        _check_o(o, ref_o)
        assert np.abs(lse.cpu().numpy() - ref_l).max() < LSE_TOL, i
    torch.cuda.synchronize()
    for cache, hist in ((kc, kh), (vc, vh)):
        rows, valid = oracle.cache_content_ref(hist, windows, [T0 + steps, T0 + steps - 1], T_max, sinks)
        assert np.array_equal(cache.float().cpu().numpy().astype(np.float64)[valid], rows[valid])
