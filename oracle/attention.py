"""fp64 reference definition of grouped local causal attention (AAH-v3 execution).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Asymmetric Attention Heads: Structured Head-Wise Context Allocation for
Transformer Attention" (AAH).
  * Section 4 (Background: Standard Multi-Head Attention): O_h = softmax(Q_h K_h^T
    / sqrt(d_h) + M) V_h; the softmax scale is passed in explicitly here.
  * Section 5.8 (Head mapping and execution): for a head with window W, key t_k is
    allowed for query t_q iff t_q - W + 1 <= t_k <= t_q; A = softmax(Q K^T/sqrt(d_h)
    + M_W), Y = A V; W is clamped to at most T, and W = T is standard causal
    attention.  Heads are bucketed by W and scattered back to head order, which
    has no numerical effect: head h's output depends only on (Q_h, K_h, V_h, W_h).
  * Section 7.7 (Backend-realized local attention): the same predicate written as
    k <= q and k >= q - (W - 1).
  * Section 5.10 (Measuring Attention Coverage and Hardware FLOPs): the exact
    allowed-pair count of a window W over length T is the sum over t = 1..T of
    min(t, W); ACR is the rectangular proxy sum_h T * T_k / (H T^2).
  * Table 6 caption: inference ACR reconstructed as sum_W f_W * W / T.

Sink tokens ("Autonomy-of-Heads: Data-Free Sparse Attention from Frozen Query-Key
Geometry", section 5, Deploying LLMs With AoH, and section 6.1): a streaming head
attends to the first s_sink tokens and to its recent window.  With a sink size S
per head, key t_k is allowed for query t_q iff t_k <= t_q and (t_k >= t_q - W + 1
or t_k < S); S = 0 is the plain local window.

Grouped K/V heads ("Asymmetric Attention Heads" section 3.3 relates the method to
grouped-query attention; its appendix A.3 inserts it into a grouped-query model,
and "Autonomy-of-Heads" section 4 and section 5 assign query heads to KV groups):
with H query heads and H_kv = H / G key/value heads, query head h reads key/value
head floor(h / G) (the G query heads of a group are consecutive); windows and
sink sizes stay per query head.  The gradients of a key/value head sum over the
query heads of its group.

Readings where the pages are silent (each listed in the design notes):
  * the additive mask value is -inf, so masked weights are exactly zero;
  * the log-sum-exp is the natural log of sum_j exp(scaled score) over the
    window, one value per query row;
  * the backward pass is plain matrix calculus of the forward definition.

Everything is computed in float64 from whatever inputs are passed (the tests
pass the same bf16-rounded values the device sees, promoted exactly).
"""
from __future__ import annotations

import numpy as np


def window_allowed(T: int, w: int, sink: int = 0, rows=None) -> np.ndarray:
    """Boolean [T, T] matrix (or [len(rows), T] for the given query rows only); entry (i, j) is True
    when key j is in query i's window.

    AAH section 5.8: t_q - W + 1 <= t_k <= t_q, with W clamped to T; with a sink
    size S (AoH section 5), keys t_k < S are allowed too (still t_k <= t_q)."""
    if w < 1:
        raise ValueError("window must be >= 1")
    if sink < 0:
        raise ValueError("sink must be >= 0")
    w = min(int(w), T)
    i = (np.arange(T) if rows is None else np.asarray(rows))[:, None]
    j = np.arange(T)[None, :]
    return (j <= i) & ((j >= i - w + 1) | (j < sink))


def _sink(sinks, h) -> int:
    return 0 if sinks is None else int(sinks[h])


def _head_probs(q: np.ndarray, k: np.ndarray, w: int, scale: float, rows=None, sink: int = 0):
    """Scores, mask and softmax of one head (AAH section 5.8).

    Returns (P, m, l) where P[r, j] is the attention weight of query row r on
    key j, m the row max of the scaled masked scores and l the row sum of
    exp(score - m)."""
    T = k.shape[0]
    allowed = window_allowed(T, w, sink, rows=rows)
    if rows is not None:
        q = q[rows]
    S = scale * (q @ k.T)                      # explicit scores
    S = np.where(allowed, S, -np.inf)          # additive -inf mask M_W
    m = S.max(axis=1, keepdims=True)           # the diagonal is always allowed: finite
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return E / l, m[:, 0], l[:, 0]


def kv_head(h: int, H: int, H_kv: int) -> int:
    """Key/value head read by query head h: floor(h / G), G = H / H_kv query heads per group."""
    if H_kv < 1 or H % H_kv != 0:
        raise ValueError("H must be a multiple of H_kv")
    return h // (H // H_kv)


def attn_fwd_ref(q, k, v, windows, scale, sinks=None):
    """Forward pass for Q [B, H, T, d] and K/V [B, H_kv, T, d] (H_kv divides H; H_kv = H is
    plain multi-head attention) with one window (and sink size) per query head.

    Returns (O [B,H,T,d], LSE [B,H,T]) in float64.  AAH section 5.8; AoH section 5 for sinks."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, d = q.shape
    H_kv = k.shape[1]
    O = np.empty((B, H, T, v.shape[-1]), dtype=np.float64)
    LSE = np.empty((B, H, T), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, H_kv)
            P, m, l = _head_probs(q[b, h], k[b, g], int(windows[h]), scale, sink=_sink(sinks, h))
            O[b, h] = P @ v[b, g]
            LSE[b, h] = m + np.log(l)
    return O, LSE


def attn_fwd_rows_ref(q_h, k_h, v_h, w, scale, rows, sink: int = 0):
    """Forward pass of selected query rows of ONE head (arrays [T, d]).

    Same definition as attn_fwd_ref restricted to the given rows, so that large
    inputs can be spot-checked row by row.  Returns (O [len(rows), d], LSE)."""
    q_h = np.asarray(q_h, dtype=np.float64)
    k_h = np.asarray(k_h, dtype=np.float64)
    v_h = np.asarray(v_h, dtype=np.float64)
    P, m, l = _head_probs(q_h, k_h, int(w), scale, rows=np.asarray(rows), sink=int(sink))
    return P @ v_h, m + np.log(l)


def attn_bwd_ref(q, k, v, windows, scale, do, sinks=None):
    """Gradients (dQ, dK, dV) of sum(O * dO) by matrix calculus of section 5.8.

    With P the masked row softmax of S = scale Q K^T and O = P V, per query head:
      dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
      dS = P * (dP - D 1^T)  (zero where masked, since P is),
      dQ = scale dS K,  dK = scale dS^T Q;
    a key/value head shared by a group of query heads gets the sum of their dK, dV."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, T, d = q.shape
    H_kv = k.shape[1]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, H_kv)
            P, _, _ = _head_probs(q[b, h], k[b, g], int(windows[h]), scale, sink=_sink(sinks, h))
            dv[b, g] += P.T @ do[b, h]
            dP = do[b, h] @ v[b, g].T
            D = (P * dP).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            dq[b, h] = scale * (dS @ k[b, g])
            dk[b, g] += scale * (dS.T @ q[b, h])
    return dq, dk, dv


def pair_count_ref(T: int, w: int, sink: int = 0) -> int:
    """Exact allowed query-key pairs of one head: sum_{t=1}^{T} min(t, W), plus the sink
    keys row t sees before its window (keys 0 .. t - W - 1): sum_t max(0, min(S, t - W)).

    AAH section 5.10 (with W clamped to T, section 5.8); AoH section 5 for sinks."""
    W = min(int(w), T)
    S = int(sink)
    return int(sum(min(t, W) + max(0, min(S, t - W)) for t in range(1, T + 1)))


def acr_ref(windows, T: int) -> float:
    """Attention Coverage Ratio of one layer, decoder-only (T_q = T, T_k = W_h).

    AAH section 5.10: sum_h T * T_k / (H * T^2)."""
    windows = [min(int(w), T) for w in windows]
    return float(sum(T * w for w in windows)) / (len(windows) * T * T)


def acr_from_fractions_ref(fractions, windows, T: int) -> float:
    """Inference ACR from window-bucket fractions: sum_W f_W * W / T (AAH Table 6 caption)."""
    return float(sum(f * w for f, w in zip(fractions, windows))) / T
