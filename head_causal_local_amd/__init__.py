"""Per-head causal local-window attention for AMD MI355X (gfx950).

The execution branch of Asymmetric Attention Heads (AAH-v3): every head h
attends only to keys j with i - w_h < j <= i of its own causal local window
("Asymmetric Attention Heads", section 5.8).  Optionally a head also keeps its
first s_h keys visible to every later query (sink tokens plus a recent window,
"Autonomy-of-Heads", section 5): pass `sinks`, one int per head.  All arithmetic runs in the HIP
kernels of libaah_attn.so behind the C ABI of include/aah_attn.h; this module
only marshals arguments.  PyTorch provides device memory and the stream.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence, Tuple

import numpy as np

from ._lib import (AAH_BF16, AAH_F32, AahError, EXPORTS, LIB_PATH, WorkItem, check, lib)  # noqa: F401

__all__ = ["local_window_attention", "attn_fwd", "attn_fwd_diag", "head_features", "head_features_workspace_size", "N_FEATURES", "attn_bwd", "attn_bwd_dq", "attn_bwd_dkdv", "attn_decode", "kv_cache_fill", "kv_cache_rows",
           "decode_workspace_size", "workspace_size", "tile_shape", "plan_fwd", "plan_bwd", "window_stats",
           "cache_clear", "AahError", "LIB_PATH"]


_I32 = np.iinfo(np.int32)


def _windows_arg(windows) -> np.ndarray:
    if isinstance(windows, np.ndarray) and windows.dtype == np.int32 and windows.ndim == 1 \
            and windows.flags.c_contiguous:
        return windows
    w = np.ascontiguousarray(np.asarray(windows, dtype=np.int64))
    if w.ndim != 1:
        raise ValueError("windows must be a 1-D sequence with one entry per head")
    if w.size and (w.max() > _I32.max or w.min() < _I32.min):
        raise ValueError("window out of int32 range")
    return np.ascontiguousarray(w.astype(np.int32))


def _wptr(w: np.ndarray):
    return w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _sinks_arg(sinks, H: int):
    """int32 array of sink sizes (or None when there are none)."""
    if sinks is None:
        return None
    s = _windows_arg(sinks)
    if s.shape[0] != H:
        raise ValueError(f"sinks has {s.shape[0]} entries, expected H = {H}")
    return s


def _sptr(s):
    return None if s is None else _wptr(s)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return AAH_BF16
    if t.dtype == torch.float32:
        return AAH_F32
    raise AahError(2, "AAH_ERR_UNSUPPORTED", f"dtype {t.dtype} has no kernel (bfloat16 or float32)")


def _stream_ptr(t, stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return s.cuda_stream


def _check_operand(name, t, ref):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
        raise ValueError(f"{name} must match {'q' if ref.dim() == 4 else 'its reference'} in shape, dtype and device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, T, d]")


def _kv_heads(q, k, v) -> int:
    """H_kv of k, v [B, H_kv, T, d] against q [B, H, T, d] (grouped key/value heads: H_kv divides H)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, d] and [B, H_kv, T, d]")
    B, H, T, d = q.shape
    H_kv = k.shape[1]
    if k.shape != (B, H_kv, T, d) or H_kv < 1 or H % H_kv != 0:
        raise ValueError(f"k must be [B, H_kv, T, d] with H_kv dividing H = {H} (got {tuple(k.shape)})")
    if not k.is_cuda or k.dtype != q.dtype or k.device != q.device or not k.is_contiguous():
        raise ValueError("k must be a contiguous device tensor of q's dtype and device")
    _check_operand("v", v, k)
    return H_kv


def attn_fwd(q, k, v, windows, scale: Optional[float] = None, out=None, lse=None, stream=None, sinks=None,
             workspace=None):
    """O, LSE = local-window attention of q, k, v ([B, H, T, d] device tensors).

    windows: one int per head (>= 1; values above T act as T).  sinks: None or
    one int per head (>= 0), the number of leading keys every later query also
    sees.  scale defaults to 1/sqrt(d).  workspace: None (the call asks the
    library how much it needs for a split launch and allocates it), or a device
    tensor the caller keeps, of at least fwd_workspace_size(...) bytes (an empty
    one means no split).  Returns (O with q's dtype, LSE float32 [B, H, T])."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    _check_operand("q", q, q)
    H_kv = _kv_heads(q, k, v)
    B, H, T, d = q.shape
    w = _windows_arg(windows)
    if w.shape[0] != H:
        raise ValueError(f"windows has {w.shape[0]} entries, expected H = {H}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_operand("out", out, q)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, T) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, T] tensor")
    sk = _sinks_arg(sinks, H)
    if workspace is None:
        # Workspace for the split launch (partial results of long items' chunks) when the library asks for one.
        ws_bytes = lib().aah_attn_fwd_workspace_size(_wptr(w), _sptr(sk), B, H, H_kv, T, d, _dtype_code(q))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    else:
        ws_bytes = workspace.numel() * workspace.element_size()
        ws = workspace if ws_bytes else None
    st = lib().aah_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), _wptr(w), _sptr(sk), B, H, H_kv, T, d,
                            _dtype_code(q), float(scale), out.data_ptr(), lse.data_ptr(),
                            ws.data_ptr() if ws is not None else None, ws_bytes, _stream_ptr(q, stream))
    check(st)
    return out, lse


def attn_fwd_diag(q, k, v, windows, scale: Optional[float] = None, out=None, lse=None, row_entropy=None,
                  row_onorm=None, stream=None, sinks=None, workspace=None):
    """attn_fwd plus the per-row attention entropy and output norm (float32 [B, H, T] each).  workspace as
    for attn_fwd, sized by fwd_diag_workspace_size.

    Returns (O, LSE, row_entropy, row_onorm)."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    _check_operand("q", q, q)
    H_kv = _kv_heads(q, k, v)
    B, H, T, d = q.shape
    w = _windows_arg(windows)
    if w.shape[0] != H:
        raise ValueError(f"windows has {w.shape[0]} entries, expected H = {H}")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = torch.empty_like(q) if out is None else out
    _check_operand("out", out, q)
    rows = []
    for name, t in (("lse", lse), ("row_entropy", row_entropy), ("row_onorm", row_onorm)):
        if t is None:
            t = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
        elif t.shape != (B, H, T) or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 [B, H, T] tensor")
        rows.append(t)
    lse, row_entropy, row_onorm = rows
    sk = _sinks_arg(sinks, H)
    if workspace is None:
        # Workspace for the split launch when the library asks for one.
        ws_bytes = lib().aah_attn_fwd_diag_workspace_size(_wptr(w), _sptr(sk), B, H, H_kv, T, d, _dtype_code(q))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    else:
        ws_bytes = workspace.numel() * workspace.element_size()
        ws = workspace if ws_bytes else None
    check(lib().aah_attn_fwd_diag(q.data_ptr(), k.data_ptr(), v.data_ptr(), _wptr(w), _sptr(sk), B, H, H_kv, T, d,
                                  _dtype_code(q), float(scale), out.data_ptr(), lse.data_ptr(),
                                  row_entropy.data_ptr(), row_onorm.data_ptr(),
                                  ws.data_ptr() if ws is not None else None, ws_bytes, _stream_ptr(q, stream)))
    return out, lse, row_entropy, row_onorm


N_FEATURES = 9


def head_features_workspace_size(B: int, H: int, T: int, d: int) -> int:
    return int(lib().aah_head_features_workspace_size(B, H, T, d))


def head_features(q, k, v, windows, row_entropy=None, row_onorm=None, features_ema=None, alpha: float = 0.9,
                  init: bool = False, out=None, workspace=None, stream=None):
    """Per-head controller features x [H, 9] (float32) of q, k, v [B, H, T, d] and the diagnostic rows of
    the attn_fwd_diag call that ran with `windows` (None: entropy, norm and usage features are 0); if features_ema ([H, 9] float32) is given it is
    updated in place: init ? x : alpha * ema + (1 - alpha) * x.  Returns x."""
    import torch
    H_kv = _kv_heads(q, k, v)
    B, H, T, d = q.shape
    w = _windows_arg(windows)
    if w.shape[0] != H:
        raise ValueError(f"windows has {w.shape[0]} entries, expected H = {H}")
    if (row_entropy is None) != (row_onorm is None):
        raise ValueError("give both row_entropy and row_onorm, or neither")
    for name, t in (("row_entropy", row_entropy), ("row_onorm", row_onorm)):
        if t is not None and (t.shape != (B, H, T) or t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 [B, H, T] tensor")
    out = torch.empty((H, N_FEATURES), dtype=torch.float32, device=q.device) if out is None else out
    for name, t in (("out", out), ("features_ema", features_ema)):
        if t is not None and (t.shape != (H, N_FEATURES) or t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 [H, {N_FEATURES}] tensor")
    if workspace is None:
        workspace = torch.empty(max(head_features_workspace_size(B, H, T, d), 1), dtype=torch.uint8,
                                device=q.device)
    ptr, nbytes = _ws(workspace)
    check(lib().aah_head_features(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  None if row_entropy is None else row_entropy.data_ptr(),
                                  None if row_onorm is None else row_onorm.data_ptr(), _wptr(w), B, H, H_kv, T, d,
                                  _dtype_code(q), float(alpha), 1 if init else 0, out.data_ptr(),
                                  None if features_ema is None else features_ema.data_ptr(), ptr, nbytes,
                                  _stream_ptr(q, stream)))
    return out


def workspace_size(B: int, H: int, T: int, d: int, dtype: str = "bf16", is_bwd: bool = True) -> int:
    code = AAH_BF16 if dtype in ("bf16", "bfloat16") else AAH_F32
    return int(lib().aah_attn_workspace_size(B, H, T, d, code, 1 if is_bwd else 0))


def attn_bwd(q, k, v, o, do, lse, windows, scale: Optional[float] = None, dq=None, dk=None, dv=None,
             workspace=None, stream=None, sinks=None):
    """dQ, dK, dV of sum(O * do) for local-window attention (see attn_fwd); dK, dV have k's shape."""
    import torch
    for name, t in (("q", q), ("o", o), ("do", do)):
        _check_operand(name, t, q)
    H_kv = _kv_heads(q, k, v)
    B, H, T, d = q.shape
    w = _windows_arg(windows)
    if w.shape[0] != H:
        raise ValueError(f"windows has {w.shape[0]} entries, expected H = {H}")
    if lse.shape != (B, H, T) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, T] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_operand("dq", dq, q)
    for name, t in (("dk", dk), ("dv", dv)):
        _check_operand(name, t, k)
    code = _dtype_code(q)
    need = int(lib().aah_attn_workspace_size(B, H, T, d, code, 1))
    if workspace is None:
        # With few work items the library splits long ones when given room for their partial results.
        sk = _sinks_arg(sinks, H)
        split = int(lib().aah_attn_bwd_split_workspace_size(_wptr(w), _sptr(sk), B, H, H_kv, T, d,
                                                             code))
        workspace = torch.empty(max(need, split, 1), dtype=torch.uint8, device=q.device)
    sk = _sinks_arg(sinks, H)
    st = lib().aah_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                            _wptr(w), _sptr(sk), B, H, H_kv, T, d, code, float(scale), dq.data_ptr(), dk.data_ptr(),
                            dv.data_ptr(),
                            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                            _stream_ptr(q, stream))
    check(st)
    return dq, dk, dv


def _ws(workspace):
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


_AUTOGRAD_FN = None


def _autograd_fn():
    """The torch.autograd.Function behind local_window_attention (built on first use, so importing this
    module does not import torch)."""
    global _AUTOGRAD_FN
    if _AUTOGRAD_FN is None:
        import torch

        class _LocalWindowAttention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, windows, scale, sinks):
                o, lse = attn_fwd(q, k, v, windows, scale, sinks=sinks)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.windows, ctx.scale, ctx.sinks = windows, scale, sinks
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, o, lse = ctx.saved_tensors
                dq, dk, dv = attn_bwd(q, k, v, o, do.contiguous(), lse, ctx.windows, ctx.scale, sinks=ctx.sinks)
                return dq, dk, dv, None, None, None

        _AUTOGRAD_FN = _LocalWindowAttention
    return _AUTOGRAD_FN


def local_window_attention(q, k, v, windows, scale: Optional[float] = None, sinks=None):
    """O = local-window attention of q [B, H, T, d] and k, v [B, H_kv, T, d] (device tensors, bf16 or
    float32), differentiable: autograd's backward runs aah_attn_bwd on the saved O and log-sum-exp.

    windows: one int per query head (>= 1); sinks: None or one int per query head.  scale defaults to
    1/sqrt(d).  For the log-sum-exp as well, call attn_fwd (not differentiable)."""
    w = _windows_arg(windows)
    sk = None if sinks is None else _windows_arg(sinks)
    d = q.shape[-1]
    return _autograd_fn().apply(q, k, v, w, 1.0 / math.sqrt(d) if scale is None else float(scale), sk)


def _bwd_args(q, k, v, do, windows, scale):
    _check_operand("do", do, q)
    H_kv = _kv_heads(q, k, v)
    B, H, T, d = q.shape
    w = _windows_arg(windows)
    if w.shape[0] != H:
        raise ValueError(f"windows has {w.shape[0]} entries, expected H = {H}")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    return B, H, H_kv, T, d, w, float(scale)


def attn_bwd_dq(q, k, v, o, do, lse, windows, dq, workspace, scale: Optional[float] = None, stream=None,
                sinks=None):
    """Backward step 1: dQ, and the per-row -lse * log2(e) and -rowsum(do * o) into the workspace."""
    import torch
    B, H, H_kv, T, d, w, scale = _bwd_args(q, k, v, do, windows, scale)
    sk = _sinks_arg(sinks, H)
    _check_operand("o", o, q)
    _check_operand("dq", dq, q)
    if lse.shape != (B, H, T) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, T] tensor")
    ptr, nbytes = _ws(workspace)
    check(lib().aah_attn_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                lse.data_ptr(), _wptr(w), _sptr(sk), B, H, H_kv, T, d, _dtype_code(q), scale,
                                dq.data_ptr(), ptr, nbytes, _stream_ptr(q, stream)))


def attn_bwd_dkdv(q, k, v, do, windows, dk, dv, workspace, scale: Optional[float] = None, stream=None,
                  sinks=None):
    """Backward step 2: dK and dV (reads the workspace rows attn_bwd_dq wrote; run it after that step)."""
    B, H, H_kv, T, d, w, scale = _bwd_args(q, k, v, do, windows, scale)
    sk = _sinks_arg(sinks, H)
    _check_operand("dk", dk, k)
    _check_operand("dv", dv, k)
    ptr, nbytes = _ws(workspace)
    check(lib().aah_attn_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), _wptr(w), _sptr(sk),
                                  B, H, H_kv, T, d, _dtype_code(q), scale, dk.data_ptr(), dv.data_ptr(), ptr, nbytes,
                                  _stream_ptr(q, stream)))


def _decode_heads(windows, sinks, H_kv):
    w = _windows_arg(windows)
    H = w.shape[0]
    H_kv = H if H_kv is None else int(H_kv)
    return w, _sinks_arg(sinks, H), H, H_kv


def kv_cache_rows(windows, T_max: int, sinks=None, H_kv: Optional[int] = None) -> int:
    """Rows per batch entry of the trimmed decode caches (see aah_kv_cache_rows)."""
    w, sk, H, H_kv = _decode_heads(windows, sinks, H_kv)
    r = int(lib().aah_kv_cache_rows(_wptr(w), _sptr(sk), H, H_kv, int(T_max)))
    if r < 0:
        raise ValueError("invalid windows, sinks, H_kv or T_max")
    return r


def decode_workspace_size(windows, B: int, T_max: int, d: int, sinks=None, H_kv: Optional[int] = None) -> int:
    """Workspace bytes of one decoding step (bf16)."""
    w, sk, H, H_kv = _decode_heads(windows, sinks, H_kv)
    return int(lib().aah_attn_decode_workspace_size(_wptr(w), _sptr(sk), B, H, H_kv, int(T_max), d, AAH_BF16))


def kv_cache_fill(k, v, windows, T_max: int, kcache=None, vcache=None, stream=None, sinks=None):
    """Store a prefill's K/V [B, H_kv, T, d] (positions 0..T-1) into trimmed caches [B, R, d]; windows (and
    sinks) have one entry per query head, H = len(windows) a multiple of H_kv."""
    import torch
    _check_operand("v", v, k)
    B, H_kv, T, d = k.shape
    w, sk, H, H_kv = _decode_heads(windows, sinks, H_kv)
    R = kv_cache_rows(w, T_max, sinks=sk, H_kv=H_kv)
    if kcache is None:
        kcache = torch.zeros((B, R, d), dtype=k.dtype, device=k.device)
    if vcache is None:
        vcache = torch.zeros((B, R, d), dtype=k.dtype, device=k.device)
    for name, t in (("kcache", kcache), ("vcache", vcache)):
        if t.shape != (B, R, d) or t.dtype != k.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [{B}, {R}, {d}] tensor of k's dtype")
    check(lib().aah_kv_cache_fill(k.data_ptr(), v.data_ptr(), _wptr(w), _sptr(sk), B, H, H_kv, T, int(T_max), d,
                                  _dtype_code(k), kcache.data_ptr(), vcache.data_ptr(), _stream_ptr(k, stream)))
    return kcache, vcache


def attn_decode(q, k_new, v_new, kcache, vcache, pos, windows, T_max: int, scale: Optional[float] = None,
                out=None, lse=None, workspace=None, stream=None, sinks=None):
    """One decoding step: q [B, H, d], k_new, v_new [B, H_kv, d] at positions pos (int32 device tensor [B]).

    Stores k_new / v_new into the caches and returns (o [B, H, d], lse [B, H])."""
    import torch
    _check_operand("v_new", v_new, k_new)
    B, H, d = q.shape
    H_kv = k_new.shape[1]
    if k_new.shape != (B, H_kv, d) or H % H_kv != 0 or k_new.dtype != q.dtype or not k_new.is_contiguous():
        raise ValueError("k_new must be a contiguous [B, H_kv, d] tensor of q's dtype with H_kv dividing H")
    if not q.is_cuda or not q.is_contiguous():
        raise ValueError("q must be a contiguous device tensor")
    w, sk, Hw, H_kv = _decode_heads(windows, sinks, H_kv)
    if Hw != H:
        raise ValueError(f"windows has {Hw} entries, expected H = {H}")
    R = kv_cache_rows(w, T_max, sinks=sk, H_kv=H_kv)
    for name, t in (("kcache", kcache), ("vcache", vcache)):
        if t.shape != (B, R, d) or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [{B}, {R}, {d}] tensor of q's dtype")
    if pos.shape != (B,) or pos.dtype != torch.int32 or not pos.is_contiguous() or pos.device != q.device:
        raise ValueError("pos must be a contiguous int32 [B] tensor on q's device")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_operand("out", out, q)
    if lse.shape != (B, H) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H] tensor")
    if workspace is None:   # zeroed: its first B*H_kv int32 are the kernels' merge counters
        workspace = torch.zeros(max(decode_workspace_size(w, B, T_max, d, sinks=sk, H_kv=H_kv), 1),
                                dtype=torch.uint8, device=q.device)
    ptr, nbytes = _ws(workspace)
    check(lib().aah_attn_decode(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), kcache.data_ptr(),
                                vcache.data_ptr(), pos.data_ptr(), _wptr(w), _sptr(sk), B, H, H_kv, int(T_max), d,
                                _dtype_code(q), scale, out.data_ptr(), lse.data_ptr(), ptr, nbytes,
                                _stream_ptr(q, stream)))
    return out, lse


def attn_decode_noalloc(q, k_new, v_new, kcache, vcache, pos, windows, T_max: int, out, lse,
                        scale: Optional[float] = None, stream=None, sinks=None):
    """attn_decode without a workspace (aah_attn_decode_noalloc): the library's per-device scratch array holds
    the counters, plan and partials, so this call allocates nothing.  out [B, H, d] and lse [B, H] must be
    given.  Returns (out, lse)."""
    import torch
    _check_operand("v_new", v_new, k_new)
    B, H, d = q.shape
    H_kv = k_new.shape[1]
    if k_new.shape != (B, H_kv, d) or H % H_kv != 0 or k_new.dtype != q.dtype or not k_new.is_contiguous():
        raise ValueError("k_new must be a contiguous [B, H_kv, d] tensor of q's dtype with H_kv dividing H")
    if not q.is_cuda or not q.is_contiguous():
        raise ValueError("q must be a contiguous device tensor")
    w, sk, Hw, H_kv = _decode_heads(windows, sinks, H_kv)
    if Hw != H:
        raise ValueError(f"windows has {Hw} entries, expected H = {H}")
    R = kv_cache_rows(w, T_max, sinks=sk, H_kv=H_kv)
    for name, t in (("kcache", kcache), ("vcache", vcache)):
        if t.shape != (B, R, d) or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [{B}, {R}, {d}] tensor of q's dtype")
    if pos.shape != (B,) or pos.dtype != torch.int32 or not pos.is_contiguous() or pos.device != q.device:
        raise ValueError("pos must be a contiguous int32 [B] tensor on q's device")
    _check_operand("out", out, q)
    if lse.shape != (B, H) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H] tensor")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    check(lib().aah_attn_decode_noalloc(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), kcache.data_ptr(),
                                        vcache.data_ptr(), pos.data_ptr(), _wptr(w), _sptr(sk), B, H, H_kv,
                                        int(T_max), d, _dtype_code(q), scale, out.data_ptr(), lse.data_ptr(),
                                        _stream_ptr(q, stream)))
    return out, lse


def tile_shape(dtype: str, d: int, is_bwd: bool) -> Tuple[int, int]:
    """(row tile, column tile) the kernels use for this dtype / head dim / pass."""
    code = AAH_BF16 if dtype in ("bf16", "bfloat16") else AAH_F32
    r, c = ctypes.c_int(), ctypes.c_int()
    check(lib().aah_tile_shape(code, d, 1 if is_bwd else 0, ctypes.byref(r), ctypes.byref(c)))
    return r.value, c.value


def _plan(fn, windows, sinks, B, H, T, q_tile, kv_tile, n_queues, H_kv) -> np.ndarray:
    w = _windows_arg(windows)
    sk = None if sinks is None else _windows_arg(sinks)
    H_kv = H if H_kv is None else H_kv
    n = ctypes.c_int64()
    st = fn(_wptr(w), _sptr(sk), B, H, H_kv, T, q_tile, kv_tile, n_queues, None, 0, ctypes.byref(n))
    if st not in (0, 1):
        check(st)
    buf = (WorkItem * max(n.value, 1))()
    check(fn(_wptr(w), _sptr(sk), B, H, H_kv, T, q_tile, kv_tile, n_queues, buf, n.value, ctypes.byref(n)))
    arr = np.frombuffer(buf, dtype=np.int32).reshape(-1, 4)[: n.value].copy()
    return arr


def bwd_split_workspace_size(windows: Sequence[int], B: int, H: int, T: int, d: int, dtype: str = "bf16",
                             sinks: Optional[Sequence[int]] = None, H_kv: Optional[int] = None) -> int:
    """Workspace bytes with which the backward (and each of its two steps) splits long items on the current
    device, 0 when it does not; such a workspace also serves the unsplit calls."""
    w = _windows_arg(windows)
    sk = _sinks_arg(sinks, H)
    code = AAH_BF16 if dtype == "bf16" else AAH_F32
    return int(lib().aah_attn_bwd_split_workspace_size(_wptr(w), _sptr(sk), B, H, H if H_kv is None else H_kv, T,
                                                       d, code))


def plan_fwd(windows: Sequence[int], B: int, H: int, T: int, q_tile: int, kv_tile: int, n_queues: int = 8,
             sinks: Optional[Sequence[int]] = None, H_kv: Optional[int] = None):
    """Forward work list as an int32 array [n, 4] of (bh, q_tile_index, kv_lo, kv_hi)."""
    return _plan(lib().aah_plan_fwd, windows, sinks, B, H, T, q_tile, kv_tile, n_queues, H_kv)


def plan_bwd(windows: Sequence[int], B: int, H: int, T: int, q_tile: int, kv_tile: int, n_queues: int = 8,
             sinks: Optional[Sequence[int]] = None, H_kv: Optional[int] = None):
    """Backward work list as an int32 array [n, 4] of (b * H_kv + g, kv_tile_index, q_lo, q_hi)."""
    return _plan(lib().aah_plan_bwd, windows, sinks, B, H, T, q_tile, kv_tile, n_queues, H_kv)


def fwd_workspace_size(windows: Sequence[int], B: int, H: int, T: int, d: int, dtype: str = "bf16",
                       sinks: Optional[Sequence[int]] = None, H_kv: Optional[int] = None, diag: bool = False) -> int:
    """Workspace bytes with which the forward (diag: the diagnostic forward) splits long items on the current
    device (0: it does not)."""
    w = _windows_arg(windows)
    sk = _sinks_arg(sinks, H)
    code = AAH_BF16 if dtype == "bf16" else AAH_F32
    fn = lib().aah_attn_fwd_diag_workspace_size if diag else lib().aah_attn_fwd_workspace_size
    return int(fn(_wptr(w), _sptr(sk), B, H, H if H_kv is None else H_kv, T, d, code))


def _plan_split(fn, windows, sinks, B, H, T, q_tile, kv_tile, chunk_tiles, n_queues, H_kv):
    w = _windows_arg(windows)
    sk = _sinks_arg(sinks, H)
    H_kv = H if H_kv is None else H_kv
    n, m = ctypes.c_int64(), ctypes.c_int64()
    st = fn(_wptr(w), _sptr(sk), B, H, H_kv, T, q_tile, kv_tile, n_queues, chunk_tiles, None, None, 0,
            ctypes.byref(n), None, 0, ctypes.byref(m))
    if st not in (0, 1):
        check(st)
    items = (WorkItem * max(n.value, 1))()
    slots = np.zeros(max(n.value, 1), dtype=np.int32)
    merges = (WorkItem * max(m.value, 1))()
    check(fn(_wptr(w), _sptr(sk), B, H, H_kv, T, q_tile, kv_tile, n_queues, chunk_tiles, items,
             slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n.value, ctypes.byref(n), merges, m.value,
             ctypes.byref(m)))
    as_arr = lambda buf, k: np.frombuffer(buf, dtype=np.int32).reshape(-1, 4)[:k].copy()  # noqa: E731
    return as_arr(items, n.value), slots[: n.value].copy(), as_arr(merges, m.value)


def plan_fwd_split(windows: Sequence[int], B: int, H: int, T: int, q_tile: int, kv_tile: int, chunk_tiles: int,
                   n_queues: int = 8, H_kv: Optional[int] = None, sinks: Optional[Sequence[int]] = None):
    """Split forward work list: (items int32 [n, 4] as plan_fwd, slots int32 [n] (-1: the item writes its own
    rows), merge records int32 [m, 4] of (bh, q_tile_index, first slot, chunks))."""
    return _plan_split(lib().aah_plan_fwd_split, windows, sinks, B, H, T, q_tile, kv_tile, chunk_tiles, n_queues,
                       H_kv)


def plan_bwd_split(windows: Sequence[int], B: int, H: int, T: int, q_tile: int, kv_tile: int, chunk_tiles: int,
                   n_queues: int = 8, H_kv: Optional[int] = None, sinks: Optional[Sequence[int]] = None):
    """Split dK/dV work list: (items int32 [n, 4] as plan_bwd, slots int32 [n], merge records int32 [m, 4] of
    (b * H_kv + g, key_tile_index, first slot, chunks))."""
    return _plan_split(lib().aah_plan_bwd_split, windows, sinks, B, H, T, q_tile, kv_tile, chunk_tiles, n_queues,
                       H_kv)


def window_stats(windows: Sequence[int], T: int, sinks: Optional[Sequence[int]] = None) -> Tuple[int, float]:
    """(exact visible query/key pairs per batch entry, ACR) of a window vector (and sink sizes)."""
    w = _windows_arg(windows)
    sk = _sinks_arg(sinks, w.shape[0])
    pairs = ctypes.c_int64()
    acr = ctypes.c_double()
    check(lib().aah_window_stats(_wptr(w), _sptr(sk), w.shape[0], T, ctypes.byref(pairs), ctypes.byref(acr)))
    return pairs.value, acr.value


def cache_clear() -> None:
    lib().aah_cache_clear()


def cache_entries() -> int:
    """Work lists the library currently caches (all kinds; at most 64 per kind besides graph-pinned ones)."""
    return int(lib().aah_cache_entries())
