"""The prefill calls under HIP graph capture: forward (plain and split) and backward, replayed against eager;
with sink keys and grouped heads also the split backward and the diagnostic forward's split.

After one eager call (which builds and uploads the work lists), a torch.cuda.CUDAGraph captures the
forward and the backward; each of several replays, with eager work and synchronisations between them,
must reproduce the eager results bitwise (the kernels are deterministic, and the split forward's
workspace is allocated inside the capture from the graph's own pool).
"""
import numpy as np
import pytest
import torch

import head_causal_local_amd as aah
import synth

pytestmark = pytest.mark.gpu


def _dev(wl, key):
    return torch.from_numpy(wl.bits[key].view(np.int16)).view(torch.bfloat16).to("cuda")


@pytest.mark.parametrize("B,H,H_kv,T,d,windows,sinks,split", [
    (2, 4, 4, 1000, 64, [1, 100, 512, 1000], None, False),   # every item short: one workgroup per item
    (1, 2, 2, 4096, 64, [4096, 2048], None, True),            # few long items: split forward + merge
    # split launches with sink keys and grouped heads, and the diagnostic forward's split
    (1, 4, 2, 2048, 64, [2048, 300, 1000, 2048], [64, 0, 32, 0], True),
])
def test_graph_replays_equal_eager(B, H, H_kv, T, d, windows, sinks, split):
    if not torch.cuda.is_available():
        pytest.fail("this test needs a HIP device")
    wl = synth.random_workload(B, H, T, d, windows, dtype="bf16", seed=T + H, backward=True, sinks=sinks,
                               H_kv=H_kv)
    assert (aah.fwd_workspace_size(wl.windows, B, H, T, d, sinks=sinks, H_kv=H_kv) > 0) == split
    q, k, v, do = (_dev(wl, key) for key in ("q", "k", "v", "do"))

    def run():
        o, lse = aah.attn_fwd(q, k, v, wl.windows, wl.scale, sinks=sinks)
        dq, dk, dv = aah.attn_bwd(q, k, v, o, do, lse, wl.windows, wl.scale, sinks=sinks)
        outs = [o, lse, dq, dk, dv]
        if sinks is not None:
            outs += list(aah.attn_fwd_diag(q, k, v, wl.windows, wl.scale, sinks=sinks)[2:])
        return outs

    eager = [t.clone() for t in run()]  # also builds and uploads the work lists outside the capture
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            outs = run()
    torch.cuda.current_stream().wait_stream(stream)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))  # eager work between replays; every replay must rewrite every output
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "lse", "dq", "dk", "dv", "entropy", "onorm"), outs, eager):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager call"
