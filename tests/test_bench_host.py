"""Host-side pieces of bench.py: the lookup of measured HBM traffic (profiles/hbm_traffic.txt) and the
refusal of more than one GPU.  No GPU needed."""
import hashlib
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _table():
    rows = []
    for line in open(os.path.join(ROOT, "profiles", "hbm_traffic.txt")):
        if line.startswith("#") or not line.strip():
            continue
        rows.append(line.rsplit(None, 4))
    return rows


def test_traffic_table_rows_are_well_formed():
    rows = _table()
    assert rows
    for kernel, workload, sha, fetch, write in rows:
        assert kernel.split("<")[0] in bench.KERNEL_SOURCES, kernel
        assert len(sha) == 16 and int(sha, 16) >= 0
        assert int(fetch) > 0 and int(write) > 0


def test_traffic_lookup_matches_kernel_workload_and_source_hash():
    for kernel, workload, sha, fetch, write in _table():
        h = hashlib.sha256()
        for f in (bench.KERNEL_SOURCES[kernel.split("<")[0]],) + bench.KERNEL_HEADERS:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        current = h.hexdigest()[:16]
        got = bench.measured_traffic(kernel, workload)
        if current == sha:
            assert got == int(fetch) + int(write)
        else:  # counters taken on an older source: not reported
            assert got is None
    assert bench.measured_traffic("decode_kernel<64, false>", "no-such-workload") is None
    assert bench.measured_traffic("no_such_kernel<1>", "3") is None


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)


def test_step_counts_are_checked():
    for flags in (["--steps", "0"], ["--warmup", "-1"]):
        res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *flags], capture_output=True,
                             text=True, timeout=120, cwd=ROOT)
        assert res.returncode == 2, flags
        assert "--steps must be" in res.stderr


def test_single_sequence_grouped_workload_shares_the_grouped_layers_windows():
    """Workload 6s is workload 6 for one sequence: the same per-query-head windows (workload 6 draws them
    after its tensors, so 6s holds them as a table), which this checks against workload 6's own draw."""
    import synth
    w6 = synth.make_workload(6)
    w6s = synth.make_workload("6s")
    assert w6s.windows.tolist() == w6.windows.tolist() == list(synth.GQA_WINDOWS)
    assert (w6s.B, w6s.H, w6s.T, w6s.d, w6s.k.shape[1]) == (1, 32, 4096, 128, 8)
