"""fp64 reference of the per-head controller features and their EMA.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Asymmetric Attention Heads" (AAH), section 5.3 (Head features and EMA
smoothing).  Each head h gets a base feature
    x_h = [mu(|q_h|), sigma(q_h), mu(|k_h|), sigma(k_h), mu(|v_h|), sigma(v_h), e_h, n_h, rho_h],
where the Q/K/V entries are scalar reductions over the batch, sequence and
per-head feature axes of that head (mu(|.|) is the mean ABSOLUTE activation,
not the absolute value of the mean), and e_h, n_h, rho_h are the previous
attention diagnostics: entropy, output norm and usage.  The features are
smoothed as xbar_t = alpha xbar_{t-1} + (1 - alpha) x_t, with xbar_0 = x_0 at the
first control update.  When there are no previous attention diagnostics, all
three of them (e_h, n_h and rho_h) are zero.

Readings where the page is silent (each listed in the design notes):
  * sigma is the population standard deviation (divide by the count N); with
    N = B T d of the order of 10^6 the unbiased form differs by 1/(2N) relative;
  * e_h is the mean over batch entries and query rows of the row's attention
    entropy -sum_j p_ij ln p_ij (natural log) over its visible keys;
  * n_h is the mean over batch entries and query rows of the Euclidean norm of
    the head's output row O_i;
  * rho_h, the usage, is the fraction of the context the window of the stored
    statistics' forward pass covered, min(W_h, T) / T: the head's term of the
    coverage ratio of section 5.10, matching the pages' window-branch usage
    (Table 6 caption).  It belongs to the stored statistics like e_h and n_h:
    with no diagnostics given it is zero, and with them it is taken from the
    windows of the forward pass that produced them (the `windows` argument).
"""
from __future__ import annotations

import numpy as np

from .attention import _head_probs, _sink, kv_head

N_FEATURES = 9


def attn_row_stats_ref(q, k, v, windows, scale, sinks=None):
    """Per query row of every (b, h): (entropy [B,H,T], output norm [B,H,T]) in float64.

    entropy_i = -sum_j p_ij ln p_ij over the row's visible keys (masked weights
    are exactly zero and contribute nothing); norm_i = ||sum_j p_ij v_j||_2."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, _ = q.shape
    ent = np.empty((B, H, T))
    nrm = np.empty((B, H, T))
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, k.shape[1])
            P, _, _ = _head_probs(q[b, h], k[b, g], int(windows[h]), scale, sink=_sink(sinks, h))
            with np.errstate(divide="ignore", invalid="ignore"):
                plogp = np.where(P > 0, P * np.log(P), 0.0)
            ent[b, h] = -plogp.sum(axis=1)
            nrm[b, h] = np.linalg.norm(P @ v[b, g], axis=1)
    return ent, nrm


def attn_row_stats_rows_ref(q_h, k_h, v_h, w, scale, rows, sink: int = 0):
    """attn_row_stats_ref restricted to selected query rows of ONE head (arrays [T, d]), so that
    large inputs can be spot-checked row by row.  Returns (entropy [len(rows)], norm [len(rows)])."""
    q_h = np.asarray(q_h, dtype=np.float64)
    k_h = np.asarray(k_h, dtype=np.float64)
    v_h = np.asarray(v_h, dtype=np.float64)
    P, _, _ = _head_probs(q_h, k_h, int(w), scale, rows=np.asarray(rows), sink=int(sink))
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(P > 0, P * np.log(P), 0.0)
    return -plogp.sum(axis=1), np.linalg.norm(P @ v_h, axis=1)


def _mean_abs_std(x_h):
    x_h = np.asarray(x_h, dtype=np.float64).ravel()
    mu = x_h.mean()
    return np.abs(x_h).mean(), np.sqrt(((x_h - mu) ** 2).mean())


def head_features_ref(q, k, v, windows, row_entropy=None, row_norm=None):
    """Base features x [H, 9] (section 5.3) from Q [B,H,T,d], K/V [B,H_kv,T,d] and, if given, the
    per-row diagnostics of the most recent forward pass ([B,H,T] each), run with `windows`.  Without
    them (both None) e_h, n_h and rho_h are zero.  With grouped K/V heads, query head h's key and
    value statistics are those of its group's head."""
    if (row_entropy is None) != (row_norm is None):
        raise ValueError("row_entropy and row_norm are the stored statistics of one forward pass: give both or neither")
    have_diag = row_entropy is not None
    q = np.asarray(q, dtype=np.float64)
    B, H, T, _ = q.shape
    x = np.zeros((H, N_FEATURES))
    for h in range(H):
        g = kv_head(h, H, np.asarray(k).shape[1])
        for slot, (t, hh) in enumerate(((q, h), (k, g), (v, g))):
            x[h, 2 * slot], x[h, 2 * slot + 1] = _mean_abs_std(np.asarray(t)[:, hh])
        if have_diag:
            x[h, 6] = np.asarray(row_entropy, dtype=np.float64)[:, h].mean()
            x[h, 7] = np.asarray(row_norm, dtype=np.float64)[:, h].mean()
            x[h, 8] = min(int(windows[h]), T) / T
    return x


def features_ema_ref(xbar_prev, x, alpha, init):
    """xbar_t = alpha xbar_{t-1} + (1 - alpha) x_t; the first update (init) takes x_t itself."""
    x = np.asarray(x, dtype=np.float64)
    if init:
        return x.copy()
    return alpha * np.asarray(xbar_prev, dtype=np.float64) + (1.0 - alpha) * x
