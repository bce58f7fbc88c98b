"""The work-list cache under changing windows (the controller of "Asymmetric Attention Heads" sections 5.3 and
5.8 picks new per-head windows at every control update), through the C ABI.

Every call below uses a window vector not seen before, so every call builds, uploads (stream-ordered, from
pinned staging memory) and, once the cache is full, evicts a work list; every result is checked against the
fp64 oracle (bounds of tests/test_gpu_parity.py), and the cache never holds more than its capacity.  A list
built on one stream and used at once on another (which must wait for the upload) is checked too, as is the
refusal to build a list during graph capture, a list too large for the staging ring (synchronous upload), and
eight host threads on streams of their own building and using lists at the same time.
"""
import warnings

import numpy as np
import pytest
import torch

import head_causal_local_amd as aah
import oracle
import synth

pytestmark = pytest.mark.gpu

CAPACITY = 64  # work lists per kind
O_TOL, LSE_TOL, GRAD_REL = 1e-2, 4e-3, 3e-2


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a HIP device")


def _dev(wl, key):
    return torch.from_numpy(wl.bits[key].view(np.int16)).view(torch.bfloat16).to("cuda")


def _check_fwd(wl, o, lse):
    O, L = oracle.attn_fwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale)
    got = o.float().cpu().numpy().astype(np.float64)
    assert (np.abs(got - O) - np.maximum(O_TOL, np.abs(O) * 2.0 ** -8)).max() <= 0
    assert np.abs(lse.cpu().numpy() - L).max() < LSE_TOL


def test_new_windows_every_call_forward_bounded_cache():
    """150 forwards, each with a fresh window vector: all correct, the cache stays within its capacity."""
    _require_gpu()
    aah.cache_clear()
    B, H, T, d = 1, 4, 200, 64
    rng = np.random.default_rng(123)
    seen = set()
    wl = synth.random_workload(B, H, T, d, [1] * H, dtype="bf16", seed=5, backward=False)
    q, k, v = _dev(wl, "q"), _dev(wl, "k"), _dev(wl, "v")
    n = 0
    while n < 150:
        w = tuple(int(x) for x in rng.integers(1, 260, size=H))
        if w in seen:
            continue
        seen.add(w)
        wl.windows = np.asarray(w, dtype=np.int32)
        o, lse = aah.attn_fwd(q, k, v, wl.windows, wl.scale)
        torch.cuda.synchronize()
        _check_fwd(wl, o, lse)
        assert aah.cache_entries() <= CAPACITY, n
        n += 1
    assert aah.cache_entries() == CAPACITY


def test_new_windows_every_call_backward():
    """Forward and backward with a fresh window vector at every step (lists evicted as they go)."""
    _require_gpu()
    B, H, T, d = 1, 3, 160, 32
    rng = np.random.default_rng(7)
    for step in range(12):
        w = [int(x) for x in rng.integers(1, 200, size=H)]
        wl = synth.random_workload(B, H, T, d, w, dtype="bf16", seed=300 + step, backward=True)
        q, k, v, do = _dev(wl, "q"), _dev(wl, "k"), _dev(wl, "v"), _dev(wl, "do")
        o, lse = aah.attn_fwd(q, k, v, wl.windows, wl.scale)
        dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, wl.scale)
        torch.cuda.synchronize()
        _check_fwd(wl, o, lse)
        refs = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, wl.do)
        for got, ref in zip((dq, dk, dv), refs):
            err = np.abs(got.float().cpu().numpy() - ref).max()
            assert err <= GRAD_REL * np.abs(ref).max(), step


def test_list_built_on_one_stream_used_on_another():
    """A list uploaded on stream A (not yet synchronised) and used right away on stream B: B's kernels wait
    for the upload, so the result is correct."""
    _require_gpu()
    B, H, T, d = 2, 4, 700, 64
    wl = synth.random_workload(B, H, T, d, [17, 300, 4096, 1], dtype="bf16", seed=31, backward=False)
    q, k, v = _dev(wl, "q"), _dev(wl, "k"), _dev(wl, "v")
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    a.wait_stream(torch.cuda.current_stream())
    b.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(a):
        oa, la = aah.attn_fwd(q, k, v, wl.windows, wl.scale, stream=a)
    with torch.cuda.stream(b):
        ob, lb = aah.attn_fwd(q, k, v, wl.windows, wl.scale, stream=b)
    torch.cuda.synchronize()
    _check_fwd(wl, ob, lb)
    assert torch.equal(oa, ob) and torch.equal(la, lb)


def test_no_list_is_built_during_graph_capture():
    """Capturing a call whose windows have no cached list fails with AAH_ERR_UNSUPPORTED (nothing is
    recorded or allocated); after one eager call the same capture works and replays correctly."""
    _require_gpu()
    B, H, T, d = 1, 2, 300, 64
    wl = synth.random_workload(B, H, T, d, [211, 97], dtype="bf16", seed=41, backward=False)
    q, k, v = _dev(wl, "q"), _dev(wl, "k"), _dev(wl, "v")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s), warnings.catch_warnings():
        warnings.filterwarnings("ignore", message="The CUDA Graph is empty")  # nothing was recorded
        with pytest.raises(aah.AahError) as err:
            with torch.cuda.graph(g, stream=s):
                aah.attn_fwd(q, k, v, wl.windows, wl.scale, out=o, lse=lse, stream=s)
    assert err.value.name == "AAH_ERR_UNSUPPORTED"
    torch.cuda.synchronize()
    aah.attn_fwd(q, k, v, wl.windows, wl.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            aah.attn_fwd(q, k, v, wl.windows, wl.scale, out=o, lse=lse, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(2):
        o.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        _check_fwd(wl, o, lse)


def test_work_list_larger_than_staging_ring():
    """A work list over 4 MiB (more than a quarter of a million items: here B = 1100, H = 256, one tile per
    head) does not fit the pinned staging ring and takes the synchronous upload, and hipFree on release.
    Forward and backward, run twice (the second call reuses the cached list), checked against the oracle on
    sampled batch entries; the windows (1, 2 and 3 over T = 3 tokens) give every row a different key set."""
    _require_gpu()
    aah.cache_clear()
    B, H, T, d = 1100, 256, 3, 32
    assert B * H * 16 > 4 << 20
    windows = [1 + h % 3 for h in range(H)]
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=77, backward=True)
    q, k, v, do = _dev(wl, "q"), _dev(wl, "k"), _dev(wl, "v"), _dev(wl, "do")
    sel = [0, 1, 549, 1099]
    sub = dict(q=wl.q[sel], k=wl.k[sel], v=wl.v[sel])
    O, L = oracle.attn_fwd_ref(sub["q"], sub["k"], sub["v"], wl.windows, wl.scale)
    refs = oracle.attn_bwd_ref(sub["q"], sub["k"], sub["v"], wl.windows, wl.scale, wl.do[sel])
    for rep in range(2):
        o, lse = aah.attn_fwd(q, k, v, wl.windows, wl.scale)
        dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, wl.scale)
        torch.cuda.synchronize()
        got = o[sel].float().cpu().numpy().astype(np.float64)
        assert (np.abs(got - O) - np.maximum(O_TOL, np.abs(O) * 2.0 ** -8)).max() <= 0, rep
        assert np.abs(lse[sel].cpu().numpy() - L).max() < LSE_TOL, rep
        for g, ref in zip((dq, dk, dv), refs):
            err = np.abs(g[sel].float().cpu().numpy() - ref).max()
            assert err <= GRAD_REL * np.abs(ref).max(), rep
    assert aah.cache_entries() >= 1
    aah.cache_clear()
    assert aah.cache_entries() == 0


def test_concurrent_host_threads():
    """Eight host threads, each on a stream of its own, run forwards and backwards at the same time, each call
    with a window vector no other call uses (48 in all, within the cache's capacity, so no list is evicted
    while another stream may still read it): every list is built, uploaded and used under the library's lock,
    and every result matches the oracle."""
    from concurrent.futures import ThreadPoolExecutor

    _require_gpu()
    torch.cuda.synchronize()
    aah.cache_clear()
    B, H, T, d = 1, 3, 160, 64
    wl = synth.random_workload(B, H, T, d, [1] * H, dtype="bf16", seed=404, backward=True)
    q, k, v, do = _dev(wl, "q"), _dev(wl, "k"), _dev(wl, "v"), _dev(wl, "do")
    torch.cuda.synchronize()

    def windows(tid, it):
        return [1 + tid, 20 + 10 * it, 100 + 6 * tid + it]

    def worker(tid):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.default_stream())
        out = []
        with torch.cuda.stream(s):
            for it in range(6):
                w = windows(tid, it)
                o, lse = aah.attn_fwd(q, k, v, w, wl.scale, stream=s)
                dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, w, wl.scale, stream=s)
                out.append((w, o, lse, dq, dk, dv))
        s.synchronize()
        return out

    with ThreadPoolExecutor(max_workers=8) as ex:
        results = [r for rs in ex.map(worker, range(8)) for r in rs]
    assert len({tuple(r[0]) for r in results}) == 48
    for w, o, lse, dq, dk, dv in results:
        wl.windows = np.asarray(w, dtype=np.int32)
        _check_fwd(wl, o, lse)
        refs = oracle.attn_bwd_ref(wl.q, wl.k, wl.v, wl.windows, wl.scale, wl.do)
        for got, ref in zip((dq, dk, dv), refs):
            err = np.abs(got.float().cpu().numpy() - ref).max()
            assert err <= GRAD_REL * np.abs(ref).max(), w
    assert aah.cache_entries() <= 3 * CAPACITY
