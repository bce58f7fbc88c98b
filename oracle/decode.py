"""fp64 reference of one decoding step over per-head trimmed K/V caches.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  * "Asymmetric Attention Heads" (AAH), section 5.8 (Head mapping and
    execution): a query at position t_q sees the keys t_q - W + 1 .. t_q of
    its head, W clamped to the sequence length.  A decoding step is that
    definition for the newest position only.
  * AAH Table 6 (inference with per-head candidate windows) and
    "Autonomy-of-Heads", section 5 (Deploying LLMs with AoH): during decoding a
    head whose attention is bounded keeps only the K/V entries its window can
    still reach, so per-head cache storage is bounded by the window.

Definition used here.  A decoding step for sequence b puts its new token at
position p = pos[b] (0-based) with maximum context T_max.  Head h, window W_h,
attends over positions max(0, p - C_h + 1) .. p with C_h = min(W_h, T_max):
    o = softmax(scale * k_j . q) over those j, applied to v_j;
    lse = natural log of sum_j exp(scale * k_j . q).
This is row p of the forward definition with window C_h over the sequence's
history, which is what the tests pin it to.

The trimmed cache (the library's storage contract, restated so that the tests
can check the bytes the kernels write): head h owns C_h rows; position t of
head h is stored in row off_h + (t mod C_h), off_h = sum of C over the heads
before h.  After positions 0 .. n - 1 have been written, row off_h + r holds
the largest t < n with t mod C_h = r (rows with no such t are unspecified).
"""
from __future__ import annotations

import numpy as np


def cache_rows_ref(windows, T_max: int):
    """(offsets [H], rows [H]): C_h = min(W_h, T_max) rows per head, heads back to back."""
    w = np.asarray(windows, dtype=np.int64)
    if (w < 1).any() or T_max < 1:
        raise ValueError("windows and T_max must be >= 1")
    c = np.minimum(w, T_max)
    off = np.concatenate([[0], np.cumsum(c)[:-1]])
    return off, c


def decode_positions(p: int, w: int, T_max: int):
    """Positions a decoding query at position p attends to: max(0, p - C + 1) .. p, C = min(w, T_max)."""
    c = min(int(w), int(T_max))
    return np.arange(max(0, p - c + 1), p + 1)


def decode_ref(q, k_hist, v_hist, windows, pos, T_max: int, scale: float):
    """One decoding step.

    q [B, H, d]: the new tokens' queries.  k_hist, v_hist [B, H, L, d]: every
    position's K/V up to and including the new token (L > max(pos)).
    pos [B]: position of each sequence's new token.  Returns (o [B, H, d],
    lse [B, H]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k_hist = np.asarray(k_hist, dtype=np.float64)
    v_hist = np.asarray(v_hist, dtype=np.float64)
    B, H, d = q.shape
    o = np.empty((B, H, v_hist.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            js = decode_positions(int(pos[b]), int(windows[h]), T_max)
            s = scale * (k_hist[b, h, js] @ q[b, h])     # explicit scores
            m = s.max()
            e = np.exp(s - m)
            o[b, h] = (e / e.sum()) @ v_hist[b, h, js]
            lse[b, h] = m + np.log(e.sum())
    return o, lse


def cache_content_ref(x_hist, windows, n_written, T_max: int):
    """Expected trimmed-cache rows after positions 0 .. n_written[b] - 1 were stored.

    x_hist [B, H, L, d] (K or V history).  Returns (rows [B, R, d], valid [B, R])
    where valid marks the rows that hold some position."""
    x_hist = np.asarray(x_hist)
    B, H, L, d = x_hist.shape
    off, c = cache_rows_ref(windows, T_max)
    R = int(c.sum())
    rows = np.zeros((B, R, d), dtype=x_hist.dtype)
    valid = np.zeros((B, R), dtype=bool)
    for b in range(B):
        n = int(n_written[b])
        for h in range(H):
            for t in range(max(0, n - int(c[h])), n):   # the last C_h positions
                r = int(off[h]) + t % int(c[h])
                rows[b, r] = x_hist[b, h, t]
                valid[b, r] = True
    return rows, valid
