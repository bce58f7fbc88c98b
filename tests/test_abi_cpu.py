"""C ABI checks that need no GPU: every declared symbol is exported, argument
validation returns the documented status before any HIP call, and the
coverage helpers agree with the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import head_causal_local_amd as aah
import oracle
from head_causal_local_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "aah_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aah_\w+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 10
    lib = _lib.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_abi_version_and_status_strings():
    lib = _lib.lib()
    assert lib.aah_abi_version() == _lib.ABI_VERSION == 13
    for code, name in [(0, b"AAH_OK"), (1, b"AAH_ERR_INVALID_ARG"), (2, b"AAH_ERR_UNSUPPORTED"),
                       (3, b"AAH_ERR_WORKSPACE"), (4, b"AAH_ERR_HIP")]:
        assert lib.aah_status_string(code) == name
    assert lib.aah_status_string(99) == b"AAH_ERR_UNKNOWN"


FAKE = 0x10000  # an aligned, never-dereferenced stand-in for a device pointer


def _fwd(windows, B=1, H=None, T=64, d=64, dt=0, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, scale=0.125, sinks=None,
         H_kv=None):
    w = np.ascontiguousarray(np.asarray(windows, dtype=np.int32))
    H = len(w) if H is None else H
    wp = w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if len(w) else None
    sk = None if sinks is None else np.ascontiguousarray(np.asarray(sinks, dtype=np.int32))
    sp = None if sk is None else sk.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    H_kv = H if H_kv is None else H_kv
    return _lib.lib().aah_attn_fwd(q, k, v, wp, sp, B, H, H_kv, T, d, dt, scale, o, lse, None, 0, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(windows=[4, 0]), 1),                    # window < 1
    (dict(windows=[4, -3]), 1),
    (dict(windows=[4], B=-1), 1),                 # negative sizes (B = 0 or T = 0 is an empty problem)
    (dict(windows=[4], T=-1), 1),
    (dict(windows=[4], H=0), 1),                  # H < 1
    (dict(windows=[4], d=48), 2),                 # unsupported head dim
    (dict(windows=[4], d=256), 2),
    (dict(windows=[4], dt=7), 2),                 # unknown dtype
    (dict(windows=[4], q=0), 1),                  # NULL tensor
    (dict(windows=[4], lse=0), 1),
    (dict(windows=[4], v=FAKE + 8), 1),           # misaligned
    (dict(windows=[4], lse=FAKE + 2), 1),
    (dict(windows=[4], scale=float("nan")), 1),
    (dict(windows=[4], scale=float("inf")), 1),
    (dict(windows=[4, 8], sinks=[0, -1]), 1),     # sink size < 0
    (dict(windows=[4, 8], sinks=[2, 3], d=48), 2),
    (dict(windows=[4, 8, 8, 8], H_kv=3), 1),      # H_kv must divide H
    (dict(windows=[4, 8], H_kv=0), 1),
    (dict(windows=[4, 8], H_kv=4), 1),            # H_kv > H
])
def test_fwd_validation(kwargs, status):
    st = _fwd(**kwargs)
    assert st == status
    assert _lib.lib().aah_last_error_detail().decode() != ""


def test_fwd_null_windows():
    st = _lib.lib().aah_attn_fwd(FAKE, FAKE, FAKE, None, None, 1, 1, 1, 8, 64, 0, 0.1, FAKE, FAKE, None, 0, None)
    assert st == 1


def _bwd(windows, ws=FAKE, ws_bytes=None, B=1, T=64, d=64, dt=0, dq=FAKE, sinks=None, H_kv=None):
    w = np.ascontiguousarray(np.asarray(windows, dtype=np.int32))
    H = len(w)
    need = aah.workspace_size(B, H, T, d, "bf16" if dt == 0 else "f32")
    ws_bytes = need if ws_bytes is None else ws_bytes
    sk = None if sinks is None else np.ascontiguousarray(np.asarray(sinks, dtype=np.int32))
    sp = None if sk is None else sk.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    return _lib.lib().aah_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), sp, B, H,
                                   H if H_kv is None else H_kv, T, d, dt, 0.125, dq, FAKE, FAKE, ws, ws_bytes, None)


def test_bwd_validation():
    assert _bwd([4, 0]) == 1
    assert _bwd([4], ws=None) == 3
    assert _bwd([4], ws_bytes=10) == 3
    assert _bwd([4], dq=0) == 1
    assert _bwd([4], ws=FAKE + 16) == 1       # workspace must be 256-byte aligned
    assert _bwd([4], d=40) == 2
    assert _bwd([4, 2], sinks=[1, -5]) == 1
    assert _bwd([4, 2, 3], H_kv=2) == 1


def test_workspace_sizes():
    B, H, T, d = 4, 32, 4096, 64
    rows = B * H * T
    assert aah.workspace_size(B, H, T, d, "bf16", is_bwd=False) == 0
    assert aah.workspace_size(B, H, T, d, "bf16") == 2 * rows * 4     # lse2 and nD
    assert aah.workspace_size(B, H, T, d, "f32") == 2 * rows * 4
    assert aah.workspace_size(1, 1, 3, 32, "f32") == 512           # each array rounded to 256 bytes
    assert _lib.lib().aah_attn_workspace_size(0, 1, 1, 64, 0, 1) == 0
    assert _lib.lib().aah_attn_workspace_size(1, 1, 1, 48, 0, 1) == 0


def test_fwd_split_workspace_size_never_for_fp32_sinks_or_bad_arguments():
    # The split forward's workspace: 0 for fp32, for heads with sinks and for invalid arguments, on any
    # machine (a positive size also needs the device's occupancy, so it is tested on the GPU).
    assert aah.fwd_workspace_size([4096] * 16, 1, 16, 4096, 64, dtype="f32") == 0
    assert aah.fwd_workspace_size([256] * 4, 1, 4, 4096, 64, sinks=[128] * 4) == 0
    assert aah.fwd_workspace_size([0, 4096], 1, 2, 4096, 64) == 0
    assert aah.fwd_workspace_size([4096] * 2, 1, 2, 4096, 48) == 0
    assert aah.fwd_workspace_size([4096] * 3, 1, 3, 4096, 64, H_kv=2) == 0
    assert _lib.lib().aah_attn_fwd_workspace_size(None, None, 1, 2, 2, 4096, 64, 0) == 0
    # and the split backward's: 0 for fp32, sinks, grouped heads and invalid arguments
    P = ctypes.POINTER(ctypes.c_int32)
    def bws(windows, H, H_kv, dt=0, sinks=None, d=64):
        w = np.ascontiguousarray(windows, dtype=np.int32)
        sp = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.int32).ctypes.data_as(P)
        return _lib.lib().aah_attn_bwd_split_workspace_size(w.ctypes.data_as(P), sp, 1, H, H_kv, 4096, d, dt)
    assert bws([4096] * 2, 2, 2, dt=1) == 0
    assert bws([256] * 2, 2, 2, sinks=[128] * 2) == 0
    assert bws([4096] * 4, 4, 2) == 0
    assert bws([0, 4096], 2, 2) == 0
    assert bws([4096] * 2, 2, 2, d=48) == 0


def test_bwd_step_validation():
    lib = _lib.lib()
    w = np.array([4, 0], dtype=np.int32)
    wp = w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    need = aah.workspace_size(1, 2, 64, 64, "bf16")
    assert lib.aah_attn_bwd_dkdv(FAKE, FAKE, FAKE, FAKE, wp, None, 1, 2, 2, 64, 64, 0, 0.1, FAKE, FAKE, FAKE, need,
                                 None) == 1
    w[1] = 3
    bad = np.array([0, -1], dtype=np.int32)
    assert lib.aah_attn_bwd_dkdv(FAKE, FAKE, FAKE, FAKE, wp, bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 1, 2, 2, 64, 64, 0, 0.1, FAKE, FAKE, FAKE, need, None) == 1   # sink < 0
    # aah_attn_bwd_dq(q, k, v, o, dout, lse, windows, sinks, B, H, H_kv, T, d, dt, scale, dq, workspace, bytes,
    #                 stream)
    assert lib.aah_attn_bwd_dq(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wp, None, 1, 2, 2, 64, 64, 0, 0.1, 0, FAKE, need,
                               None) == 1                                                      # NULL dq
    assert lib.aah_attn_bwd_dq(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wp, None, 1, 2, 2, 64, 64, 0, 0.1, FAKE, FAKE, 8,
                               None) == 3                                                      # small ws
    assert lib.aah_attn_bwd_dq(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wp, None, 1, 2, 2, 64, 48, 0, 0.1, FAKE, FAKE, need,
                               None) == 2                                                      # d = 48
    assert lib.aah_attn_bwd_dq(FAKE, FAKE, FAKE, FAKE, FAKE, 0, wp, None, 1, 2, 2, 64, 64, 0, 0.1, FAKE, FAKE, need,
                               None) == 1                                                      # NULL lse
    assert lib.aah_attn_bwd_dq(FAKE, FAKE, FAKE, 0, FAKE, FAKE, wp, None, 1, 2, 2, 64, 64, 0, 0.1, FAKE, FAKE, need,
                               None) == 1                                                      # NULL o
    assert lib.aah_attn_bwd_dq(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wp, None, 1, 2, 2, 64, 64, 0, 0.0, FAKE, FAKE, need,
                               None) == 1                                                      # scale 0
    assert lib.aah_attn_bwd_dq(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wp, None, 1, 2, 2, 64, 64, 0, float("inf"), FAKE, FAKE,
                               need, None) == 1                                                # scale inf


def test_misaligned_workspace_is_one_status_everywhere():
    """A workspace that is large enough but not 256-byte aligned is AAH_ERR_INVALID_ARG (the header's status
    for every misalignment) in every entry point that takes one, and is found before any HIP call: the
    optional forward workspace included, whether or not the launch would split."""
    lib = _lib.lib()
    w = np.array([4, 64], dtype=np.int32)
    wp = w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    F, bad = FAKE, FAKE + 16
    need = aah.workspace_size(1, 2, 64, 64, "bf16")
    # aah_attn_fwd(q, k, v, windows, sinks, B, H, H_kv, T, d, dt, scale, o, lse, ws, bytes, stream): a short
    # bf16 call (never split) and an fp32 one (never split) with a misaligned workspace of any size.
    for dt, nbytes in ((0, 0), (0, 1 << 20), (1, 1 << 20)):
        assert lib.aah_attn_fwd(F, F, F, wp, None, 1, 2, 2, 64, 64, dt, 0.1, F, F, bad, nbytes, None) == 1
        assert "aligned" in lib.aah_last_error_detail().decode()
    assert lib.aah_attn_bwd(F, F, F, F, F, F, wp, None, 1, 2, 2, 64, 64, 0, 0.1, F, F, F, bad, need, None) == 1
    assert lib.aah_attn_bwd_dq(F, F, F, F, F, F, wp, None, 1, 2, 2, 64, 64, 0, 0.1, F, bad, need, None) == 1
    assert lib.aah_attn_bwd_dkdv(F, F, F, F, wp, None, 1, 2, 2, 64, 64, 0, 0.1, F, F, bad, need, None) == 1
    dneed = aah.decode_workspace_size(w, 2, 128, 64)
    assert lib.aah_attn_decode(F, F, F, F, F, F, wp, None, 2, 2, 2, 128, 64, 0, 0.125, F, F, bad, dneed, None) == 1
    fneed = aah.head_features_workspace_size(2, 2, 64, 64)
    assert lib.aah_head_features(F, F, F, None, None, wp, 2, 2, 2, 64, 64, 0, 0.9, 0, F, None, bad, fneed,
                                 None) == 1


def test_slice_limit():
    """One head's [T, d] slice is addressed with 32-bit offsets: T * d * 4 must stay below 2^31."""
    st = _fwd([4], T=(1 << 22), d=128)
    assert st == 2


def test_tile_shape():
    assert aah.tile_shape("bf16", 64, False) == (128, 64)
    r, c = aah.tile_shape("f32", 32, False)
    assert r >= 1 and c >= 1
    with pytest.raises(aah.AahError):
        aah.tile_shape("bf16", 48, False)


@pytest.mark.parametrize("T,windows", [(4096, [512, 1024, 2048, 4096]), (257, [1, 2, 256, 257, 300]),
                                       (1, [1, 5])])
def test_window_stats_match_oracle(T, windows):
    pairs, acr = aah.window_stats(windows, T)
    assert pairs == sum(oracle.pair_count_ref(T, w) for w in windows)
    assert abs(acr - oracle.acr_ref(windows, T)) < 1e-15


@pytest.mark.parametrize("T,windows,sinks", [(4096, [256, 256, 4096, 1024], [128, 0, 128, 3000]),
                                             (300, [1, 7, 299, 300], [1, 300, 2, 5]), (5, [1, 2], [9, 1])])
def test_window_stats_with_sinks_match_oracle(T, windows, sinks):
    pairs, acr = aah.window_stats(windows, T, sinks=sinks)
    assert pairs == sum(oracle.pair_count_ref(T, w, s) for w, s in zip(windows, sinks))
    assert abs(acr - oracle.acr_ref(windows, T)) < 1e-15


def test_window_stats_rejects_bad_window():
    with pytest.raises(aah.AahError) as e:
        aah.window_stats([3, 0], 16)
    assert e.value.status == 1
    with pytest.raises(aah.AahError) as e:
        aah.window_stats([3, 4], 16, sinks=[0, -2])
    assert e.value.status == 1


def test_plan_capacity_reporting():
    lib = _lib.lib()
    w = np.array([5, 9], dtype=np.int32)
    n = ctypes.c_int64()
    st = lib.aah_plan_fwd(w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), None, 2, 2, 2, 100, 16, 16, 8, None, 0,
                          ctypes.byref(n))
    assert st == 1 and n.value >= 2 * 2 * 7


def test_decode_cache_rows_and_workspace():
    """Cache rows = the layout oracle.cache_rows_ref states (per key/value head: sink rows + ring rows);
    workspace from the chunk count and group size."""
    import oracle
    w = np.array([512, 4096, 1, 300], dtype=np.int32)
    sk = np.array([128, 0, 3, 10], dtype=np.int32)
    wp = w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    sp = sk.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    lib = _lib.lib()
    for T_max in (1, 300, 1000, 8192):
        for sinks, H_kv in ((None, 4), (sk, 4), (sk, 2), (None, 1)):
            _, sink, ring = oracle.cache_rows_ref(w, T_max, sinks, H_kv)
            rows = int((sink + ring).sum())
            assert lib.aah_kv_cache_rows(wp, None if sinks is None else sp, 4, H_kv, T_max) == rows
            assert aah.kv_cache_rows(w, T_max, sinks=sinks, H_kv=H_kv) == rows
            cr = 256 if H_kv == 4 else 512  # rows per chunk: 512 with grouped heads
            chunks = int(sum((s_ + r + cr - 1) // cr for s_, r in zip(sink, ring)))
            need = aah.decode_workspace_size(w, 3, T_max, 64, sinks=sinks, H_kv=H_kv)
            counters = -(-3 * H_kv * 4 // 256) * 256
            partials = -(-3 * chunks * (4 // H_kv) * (2 + 64) * 4 // 256) * 256
            assert need == counters + partials
    bad = np.array([4, 0], dtype=np.int32)
    assert lib.aah_kv_cache_rows(bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), None, 2, 2, 10) == -1
    assert lib.aah_kv_cache_rows(wp, None, 4, 4, 0) == -1
    assert lib.aah_kv_cache_rows(wp, None, 4, 3, 100) == -1                   # H_kv must divide H
    neg = np.array([0, -1, 0, 0], dtype=np.int32)
    assert lib.aah_kv_cache_rows(wp, neg.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 4, 4, 100) == -1
    assert lib.aah_attn_decode_workspace_size(wp, None, 1, 4, 4, 100, 64, 1) == 0      # fp32: no decode kernel
    assert lib.aah_attn_decode_workspace_size(wp, None, 1, 4, 4, 100, 48, 0) == 0      # d = 48


def test_decode_validation():
    """Every decode / cache-fill argument error is reported before any HIP call."""
    lib = _lib.lib()
    w = np.array([16, 64], dtype=np.int32)
    wp = w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    need = aah.decode_workspace_size(w, 2, 128, 64)
    F = FAKE
    # aah_attn_decode(q, k_new, v_new, kcache, vcache, pos, windows, sinks, B, H, H_kv, T_max, d, dt, scale, o, lse,
    #                 ws, bytes, stream)
    ok = [F, F, F, F, F, F, wp, None, 2, 2, 2, 128, 64, 0, 0.125, F, F, F, need, None]

    def call(i=None, val=None):
        a = list(ok)
        if i is not None:
            a[i] = val
        return lib.aah_attn_decode(*a)
    for i, name in ((0, "q"), (1, "k_new"), (2, "v_new"), (3, "kcache"), (4, "vcache"), (5, "pos"), (15, "o"),
                    (16, "lse")):
        assert call(i, 0) == 1, name
    assert call(6, None) == 1                       # NULL windows
    assert call(13, 1) == 2                         # fp32 caches: unsupported
    assert call(12, 48) == 2                        # d = 48
    assert call(14, 0.0) == 1 and call(14, float("inf")) == 1
    assert call(18, need - 1) == 3                  # small workspace
    assert call(17, 0) == 3                         # NULL workspace
    assert call(11, 0) == 1                         # T_max = 0
    assert call(10, 3) == 1                         # H_kv does not divide H
    bad = np.array([16, 0], dtype=np.int32)
    assert call(6, bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))) == 1
    negs = np.array([0, -4], dtype=np.int32)
    assert call(7, negs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))) == 1
    # aah_kv_cache_fill(k, v, windows, sinks, B, H, H_kv, T, T_max, d, dt, kcache, vcache, stream)
    assert lib.aah_kv_cache_fill(F, F, wp, None, 2, 2, 2, 129, 128, 64, 0, F, F, None) == 1   # T > T_max
    assert lib.aah_kv_cache_fill(F, F, wp, None, 2, 2, 2, -1, 128, 64, 0, F, F, None) == 1    # T < 0
    assert lib.aah_kv_cache_fill(0, F, wp, None, 2, 2, 2, 64, 128, 64, 0, F, F, None) == 1    # NULL k
    assert lib.aah_kv_cache_fill(F, F, wp, None, 2, 2, 2, 64, 128, 64, 1, F, F, None) == 2    # fp32


def test_decode_noalloc_validation():
    """The allocation-free decode reports every argument error before any HIP call: the decode checks, more
    than 256 query heads, and a step whose counters, plan and partials exceed the library's array."""
    lib = _lib.lib()
    w = np.array([16, 64], dtype=np.int32)
    wp = w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    F = FAKE
    # aah_attn_decode_noalloc(q, k_new, v_new, kcache, vcache, pos, windows, sinks, B, H, H_kv, T_max, d, dt, scale,
    #                         o, lse, stream)
    ok = [F, F, F, F, F, F, wp, None, 2, 2, 2, 128, 64, 0, 0.125, F, F, None]

    def call(i=None, val=None):
        a = list(ok)
        if i is not None:
            a[i] = val
        return lib.aah_attn_decode_noalloc(*a)
    for i, name in ((0, "q"), (1, "k_new"), (2, "v_new"), (3, "kcache"), (4, "vcache"), (5, "pos"), (15, "o"),
                    (16, "lse")):
        assert call(i, 0) == 1, name
    assert call(4, F + 8) == 1                      # misaligned vcache
    assert call(6, None) == 1                       # NULL windows
    assert call(13, 1) == 2                         # fp32 caches: unsupported
    assert call(12, 48) == 2                        # d = 48
    assert call(14, 0.0) == 1 and call(14, float("nan")) == 1
    assert call(10, 3) == 1                         # H_kv does not divide H
    negs = np.array([0, -4], dtype=np.int32)
    assert call(7, negs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))) == 1
    many = np.full(257, 64, dtype=np.int32)         # 257 query heads
    a = list(ok)
    a[6], a[9], a[10] = many.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 257, 257
    assert lib.aah_attn_decode_noalloc(*a) == 2
    big = np.full(2, 1 << 21, dtype=np.int32)       # 16384 chunks of partials at d = 128: more than 8 MiB
    a = list(ok)
    a[6], a[8], a[11], a[12] = big.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 1, 1 << 21, 128
    assert lib.aah_attn_decode_noalloc(*a) == 2
    assert "scratch" in lib.aah_last_error_detail().decode()


def test_diag_and_feature_validation():
    lib = _lib.lib()
    w = np.array([4, 9], dtype=np.int32)
    wp = w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    # aah_attn_fwd_diag(q, k, v, windows, sinks, B, H, H_kv, T, d, dt, scale, o, lse, row_entropy, row_onorm,
    #                   workspace, workspace_bytes, stream)
    assert lib.aah_attn_fwd_diag(FAKE, FAKE, FAKE, wp, None, 1, 2, 2, 64, 64, 0, 0.1, FAKE, FAKE, 0, FAKE, None, 0,
                                 None) == 1
    assert lib.aah_attn_fwd_diag(FAKE, FAKE, FAKE, wp, None, 1, 2, 2, 64, 64, 0, 0.1, FAKE, FAKE, FAKE, FAKE + 2,
                                 None, 0, None) == 1                            # misaligned
    assert lib.aah_attn_fwd_diag(FAKE, FAKE, FAKE, wp, None, 1, 2, 2, 64, 48, 0, 0.1, FAKE, FAKE, FAKE, FAKE,
                                 None, 0, None) == 2                            # d = 48
    assert lib.aah_attn_fwd_diag(FAKE, FAKE, FAKE, wp, None, 1, 2, 2, 64, 64, 0, 0.1, FAKE, FAKE, FAKE, FAKE,
                                 FAKE + 16, 4096, None) == 1                    # misaligned workspace
    # The diagnostic forward's split workspace query: 0 for fp32 and for invalid arguments.
    assert lib.aah_attn_fwd_diag_workspace_size(wp, None, 1, 2, 2, 4096, 64, 1) == 0
    assert lib.aah_attn_fwd_diag_workspace_size(wp, None, 1, 2, 2, 4096, 48, 0) == 0
    need = aah.head_features_workspace_size(2, 2, 64, 64)
    assert need == 256 * -(-(14 * 2 * 2 * 1 * 8) // 256)                        # one 32768-element span per slice
    assert aah.head_features_workspace_size(1, 1, 4096, 128) == 256 * -(-(14 * 16 * 8) // 256)
    assert aah.head_features_workspace_size(0, 1, 1, 64) == 0

    def feat(ent=FAKE, on=FAKE, feats=FAKE, ema=FAKE, alpha=0.9, ws=FAKE, nbytes=need, d=64, H_kv=2):
        # aah_head_features(q, k, v, row_entropy, row_onorm, windows, B, H, H_kv, T, d, dt, alpha, init,
        #                   features, features_ema, workspace, bytes, stream)
        return lib.aah_head_features(FAKE, FAKE, FAKE, ent, on, wp, 2, 2, H_kv, 64, d, 0, alpha, 0, feats, ema, ws,
                                     nbytes, None)
    assert feat(ent=0) == 1                  # one diagnostic row array without the other
    assert feat(feats=0, ema=0) == 1         # nothing to write
    assert feat(alpha=1.5) == 1
    assert feat(alpha=float("nan")) == 1
    assert feat(nbytes=need - 8) == 3
    assert feat(ws=FAKE + 64) == 1           # workspace must be 256-byte aligned
    assert feat(d=40) == 2
    assert feat(H_kv=3) == 1


def test_missing_library_fails_loudly():
    """Without the built library every entry point raises (there is no CPU or PyTorch fallback)."""
    import subprocess
    import sys
    code = (
        "import head_causal_local_amd as aah\n"
        "from head_causal_local_amd import _lib\n"
        "_lib.LIB_PATH = '/nonexistent/libaah_attn.so'\n"
        "_lib._lib = None\n"
        "try:\n"
        "    aah.window_stats([4, 8], 16)\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    print('no error')\n")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert res.returncode == 0, res.stderr
    assert "raised:" in res.stdout and "missing" in res.stdout and "no fallback" in res.stdout


def test_empty_problems():
    """B = 0 or T = 0 (decoding: B = 0) is an empty problem: every other argument is still checked, then the call
    returns AAH_OK without touching a tensor or the workspace, so all of them may be NULL."""
    lib = _lib.lib()
    w = np.array([16, 64], dtype=np.int32)
    wp = w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    bad = np.array([16, 0], dtype=np.int32)
    bp = bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    N = None
    for B, T in ((0, 64), (3, 0), (0, 0)):
        # aah_attn_fwd(q, k, v, windows, sinks, B, H, H_kv, T, d, dt, scale, o, lse, ws, bytes, stream)
        assert lib.aah_attn_fwd(N, N, N, wp, N, B, 2, 2, T, 64, 0, 0.125, N, N, N, 0, N) == 0
        assert lib.aah_attn_fwd(N, N, N, wp, N, B, 2, 1, T, 32, 1, 0.125, N, N, N, 0, N) == 0
        assert lib.aah_attn_fwd_diag(N, N, N, wp, N, B, 2, 2, T, 64, 0, 0.125, N, N, N, N, N, 0, N) == 0
        # aah_attn_bwd(q, k, v, o, dout, lse, windows, sinks, B, H, H_kv, T, d, dt, scale, dq, dk, dv, ws, bytes, s)
        assert lib.aah_attn_bwd(N, N, N, N, N, N, wp, N, B, 2, 2, T, 64, 0, 0.125, N, N, N, N, 0, N) == 0
        assert lib.aah_attn_bwd_dq(N, N, N, N, N, N, wp, N, B, 2, 2, T, 64, 0, 0.125, N, N, 0, N) == 0
        assert lib.aah_attn_bwd_dkdv(N, N, N, N, wp, N, B, 2, 2, T, 64, 0, 0.125, N, N, N, 0, N) == 0
        # aah_kv_cache_fill(k, v, windows, sinks, B, H, H_kv, T, T_max, d, dt, kcache, vcache, stream)
        assert lib.aah_kv_cache_fill(N, N, wp, N, B, 2, 2, T, 128, 64, 0, N, N, N) == 0
        # the workspace queries agree: an empty problem needs none
        assert lib.aah_attn_workspace_size(B, 2, T, 64, 0, 1) == 0
        assert lib.aah_attn_fwd_workspace_size(wp, N, B, 2, 2, T, 64, 0) == 0
        assert lib.aah_attn_bwd_split_workspace_size(wp, N, B, 2, 2, T, 64, 0) == 0
        # the statistics of the controller features are means over tokens: no empty case
        assert lib.aah_head_features(N, N, N, N, N, wp, B, 2, 2, T, 64, 0, 0.9, 1, N, N, N, 0, N) == 1
        # the other arguments are still checked
        assert lib.aah_attn_fwd(N, N, N, bp, N, B, 2, 2, T, 64, 0, 0.125, N, N, N, 0, N) == 1   # window 0
        assert lib.aah_attn_fwd(N, N, N, N, N, B, 2, 2, T, 64, 0, 0.125, N, N, N, 0, N) == 1    # NULL windows
        assert lib.aah_attn_fwd(N, N, N, wp, N, B, 2, 2, T, 48, 0, 0.125, N, N, N, 0, N) == 2   # d = 48
        assert lib.aah_attn_fwd(N, N, N, wp, N, B, 2, 2, T, 64, 0, float("nan"), N, N, N, 0, N) == 1
        assert lib.aah_attn_fwd(N, N, N, wp, N, B, 2, 3, T, 64, 0, 0.125, N, N, N, 0, N) == 1   # H_kv > H
        assert lib.aah_attn_bwd(N, N, N, N, N, N, wp, N, B, 2, 2, T, 64, 0, 0.0, N, N, N, N, 0, N) == 1
        assert lib.aah_attn_bwd_dkdv(N, N, N, N, bp, N, B, 2, 2, T, 64, 0, 0.125, N, N, N, 0, N) == 1
    # decoding: no sequences
    # aah_attn_decode(q, k_new, v_new, kcache, vcache, pos, windows, sinks, B, H, H_kv, T_max, d, dt, scale, o, lse,
    #                 ws, bytes, stream)
    assert lib.aah_attn_decode(N, N, N, N, N, N, wp, N, 0, 2, 2, 128, 64, 0, 0.125, N, N, N, 0, N) == 0
    assert lib.aah_attn_decode_noalloc(N, N, N, N, N, N, wp, N, 0, 2, 2, 128, 64, 0, 0.125, N, N, N) == 0
    assert lib.aah_attn_decode_workspace_size(wp, N, 0, 2, 2, 128, 64, 0) == 0
    assert lib.aah_attn_decode(N, N, N, N, N, N, wp, N, 0, 2, 2, 0, 64, 0, 0.125, N, N, N, 0, N) == 1    # T_max = 0
    assert lib.aah_attn_decode_noalloc(N, N, N, N, N, N, wp, N, 0, 2, 2, 0, 64, 0, 0.125, N, N, N) == 1  # T_max = 0
    assert lib.aah_attn_decode(N, N, N, N, N, N, wp, N, 0, 2, 2, 128, 64, 1, 0.125, N, N, N, 0, N) == 2  # fp32
    assert lib.aah_attn_decode(N, N, N, N, N, N, wp, N, -1, 2, 2, 128, 64, 0, 0.125, N, N, N, 0, N) == 1
    assert lib.aah_kv_cache_fill(N, N, wp, N, 2, 2, 2, 0, 0, 64, 0, N, N, N) == 1    # T_max = 0
