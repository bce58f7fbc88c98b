"""fp64 reference of one decoding step over per-head trimmed K/V caches.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  * "Asymmetric Attention Heads" (AAH), section 5.8 (Head mapping and
    execution): a query at position t_q sees the keys t_q - W + 1 .. t_q of
    its head, W clamped to the sequence length.  A decoding step is that
    definition for the newest position only.
  * AAH Table 6 (inference with per-head candidate windows) and
    "Autonomy-of-Heads" (AoH), section 5 (Deploying LLMs with AoH): during
    decoding a streaming head keeps only its sink tokens and its recent
    window, so per-head cache storage is bounded by s_sink + s_recent.
  * Grouped key/value heads (AAH section 3.3 and appendix A.3, AoH section 4):
    query head h reads key/value head floor(h / G), G = H / H_kv.

Definition used here.  A decoding step for sequence b puts its new token at
position p = pos[b] (0-based) with maximum context T_max.  Query head h, window
W_h and sink size S_h, attends over the positions
    {max(0, p - C_h + 1) .. p}  union  {0 .. min(S_h, p + 1) - 1},  C_h = min(W_h, T_max),
of its key/value head:
    o = softmax(scale * k_j . q) over those j, applied to v_j;
    lse = natural log of sum_j exp(scale * k_j . q).
This is row p of the forward definition (window C_h, sinks S_h) over the
sequence's history, which is what the tests pin it to.

The trimmed cache (the library's storage contract, restated so that the tests
can check the bytes the kernels write).  Key/value head g, whose query heads
are h = g G .. g G + G - 1, owns S_g + R_g rows starting at row off_g (off_g =
sum of S + R over the heads before g):
    R_g = max over its query heads of C_h (the ring),
    S_g = max over its query heads of min(S_h, T_max - C_h) (the sinks; a sink
          key at or past T_max - C_h is always inside the window, so it never
          needs a row of its own).
After positions 0 .. n - 1 have been written, ring row off_g + S_g + r holds
the largest t < n with t mod R_g = r, and sink row off_g + j (j < S_g) holds
position j if j < n (rows with no such position are unspecified).
"""
from __future__ import annotations

import numpy as np

from .attention import kv_head


def _sinks(sinks, H):
    return np.zeros(H, dtype=np.int64) if sinks is None else np.asarray(sinks, dtype=np.int64)


def cache_rows_ref(windows, T_max: int, sinks=None, H_kv=None):
    """(offsets [H_kv], sink rows [H_kv], ring rows [H_kv]) of the cache layout."""
    w = np.asarray(windows, dtype=np.int64)
    H = len(w)
    H_kv = H if H_kv is None else int(H_kv)
    s = _sinks(sinks, H)
    if (w < 1).any() or T_max < 1 or (s < 0).any():
        raise ValueError("windows and T_max must be >= 1, sinks >= 0")
    G = H // H_kv
    if H_kv < 1 or G * H_kv != H:
        raise ValueError("H must be a multiple of H_kv")
    c = np.minimum(w, T_max)
    s_eff = np.maximum(0, np.minimum(s, T_max - c))
    ring = c.reshape(H_kv, G).max(axis=1)
    sink = s_eff.reshape(H_kv, G).max(axis=1)
    off = np.concatenate([[0], np.cumsum(sink + ring)[:-1]])
    return off, sink, ring


def decode_positions(p: int, w: int, T_max: int, sink: int = 0):
    """Positions a decoding query at position p attends to: the window max(0, p - C + 1) .. p,
    C = min(w, T_max), and the sinks 0 .. min(sink, p + 1) - 1."""
    c = min(int(w), int(T_max))
    window = set(range(max(0, p - c + 1), p + 1))
    return np.array(sorted(window | set(range(min(int(sink), p + 1)))), dtype=np.int64)


def decode_ref(q, k_hist, v_hist, windows, pos, T_max: int, scale: float, sinks=None):
    """One decoding step.

    q [B, H, d]: the new tokens' queries.  k_hist, v_hist [B, H_kv, L, d]: every
    position's K/V up to and including the new token (L > max(pos)).
    pos [B]: position of each sequence's new token.  Returns (o [B, H, d],
    lse [B, H]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k_hist = np.asarray(k_hist, dtype=np.float64)
    v_hist = np.asarray(v_hist, dtype=np.float64)
    B, H, d = q.shape
    s = _sinks(sinks, H)
    o = np.empty((B, H, v_hist.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, k_hist.shape[1])
            js = decode_positions(int(pos[b]), int(windows[h]), T_max, int(s[h]))
            sc = scale * (k_hist[b, g, js] @ q[b, h])     # explicit scores
            m = sc.max()
            e = np.exp(sc - m)
            o[b, h] = (e / e.sum()) @ v_hist[b, g, js]
            lse[b, h] = m + np.log(e.sum())
    return o, lse


def cache_content_ref(x_hist, windows, n_written, T_max: int, sinks=None):
    """Expected cache rows after positions 0 .. n_written[b] - 1 were stored.

    x_hist [B, H_kv, L, d] (K or V history; the number of query heads is len(windows)).
    Returns (rows [B, R, d], valid [B, R]) where valid marks the rows that hold some position."""
    x_hist = np.asarray(x_hist)
    B, H_kv, L, d = x_hist.shape
    off, sink, ring = cache_rows_ref(windows, T_max, sinks, H_kv)
    R = int((sink + ring).sum())
    rows = np.zeros((B, R, d), dtype=x_hist.dtype)
    valid = np.zeros((B, R), dtype=bool)
    for b in range(B):
        n = int(n_written[b])
        for g in range(H_kv):
            for j in range(min(int(sink[g]), n)):          # the first positions, in order
                rows[b, int(off[g]) + j] = x_hist[b, g, j]
                valid[b, int(off[g]) + j] = True
            base = int(off[g] + sink[g])
            for t in range(max(0, n - int(ring[g])), n):   # the last R_g positions
                r = base + t % int(ring[g])
                rows[b, r] = x_hist[b, g, t]
                valid[b, r] = True
    return rows, valid
