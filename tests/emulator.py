"""fp64 tile-loop emulator of the device work lists (a test tool, not the oracle).

It executes the C++ planner's forward work list the way the kernels do --
online softmax over the listed key tiles, mask evaluated per element -- and
the backward work list key-tile by key-tile, so that a tile-range bug in the
planner shows up as a difference from the oracle on the CPU.  It shares no
code with the oracle and does not import it.

With sink sizes, the forward items visit the implied sink tiles
[0, min(ceil(S / kv_tile), lo)) first, S = min(sinks[h], T - W) (the library's
effective sink), exactly as the kernels do.  With grouped key/value heads
(k, v [B, H_kv, T, d]) forward items read head h // G, and a backward item
(bh = b H_kv + g) walks the group's query heads, each over its own query-tile
range from lo, as the kernels do.
"""
import numpy as np


def _eff_sink(sinks, h, T, W):
    return 0 if sinks is None else max(0, min(int(sinks[h]), T - W))


def _visible(rows, keys, W, S):
    return (keys[None, :] <= rows[:, None]) & ((keys[None, :] > rows[:, None] - W) | (keys[None, :] < S))


def emulate_forward(items, q, k, v, windows, scale, q_tile, kv_tile, sinks=None):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, T, d = q.shape
    O = np.full((B, H, T, d), np.nan)
    L = np.full((B, H, T), np.nan)
    for bh, qt, lo, hi in items:
        if bh < 0:
            continue
        b, h = divmod(int(bh), H)
        g = h // (H // k.shape[1])
        W = min(int(windows[h]), T)
        S = _eff_sink(sinks, h, T, W)
        rows = np.arange(qt * q_tile, min(T, (qt + 1) * q_tile))
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        acc = np.zeros((len(rows), d))
        n_sink = min(-(-S // kv_tile), int(lo))
        for kt in list(range(n_sink)) + list(range(lo, hi)):
            keys = np.arange(kt * kv_tile, min(T, (kt + 1) * kv_tile))
            s = scale * q[b, h, rows] @ k[b, g, keys].T
            ok = _visible(rows, keys, W, S)
            s = np.where(ok, s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            m_use = np.where(np.isneginf(m_new), 0.0, m_new)
            alpha = np.exp(m - m_use)
            p = np.exp(s - m_use[:, None])
            l = l * alpha + p.sum(axis=1)
            acc = acc * alpha[:, None] + p @ v[b, g, keys]
            m = m_new
        O[b, h, rows] = acc / l[:, None]
        L[b, h, rows] = m + np.log(l)
    return O, L


def emulate_forward_split(items, slots, merges, q, k, v, windows, scale, q_tile, kv_tile, sinks=None, diag=False):
    """The split forward: each item runs its own key tiles; an item with a slot leaves (m, l, acc) of its
    rows there, and every merge record (bh, q tile, first slot, chunks) combines its chunks as
    M = max m_c, L = sum exp(m_c - M) l_c, O = sum exp(m_c - M) acc_c / L, LSE = M + ln L.  With sink
    sizes, the chunk whose range starts at the window's first tile (every unsplit item's does) also visits
    the sink tiles [0, min(ceil(S / kv_tile), lo)).

    diag: also the per-row entropy and output norm, each chunk keeping a = sum_j p_j (s_j - m) against its
    own reference m and the merge taking it to M as A = sum_c exp(m_c - M) (a_c + (m_c - M) l_c), so that
    entropy = ln L - A / L and norm = |acc| / L; returns (O, LSE, entropy, norm)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, T, d = q.shape
    O = np.full((B, H, T, d), np.nan)
    L = np.full((B, H, T), np.nan)
    ENT = np.full((B, H, T), np.nan)
    NRM = np.full((B, H, T), np.nan)
    parts = {}
    for (bh, qt, lo, hi), slot in zip(items, slots):
        if bh < 0:
            continue
        b, h = divmod(int(bh), H)
        g = h // (H // k.shape[1])
        W = min(int(windows[h]), T)
        S = _eff_sink(sinks, h, T, W)
        rows = np.arange(qt * q_tile, min(T, (qt + 1) * q_tile))
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        a = np.zeros(len(rows))
        acc = np.zeros((len(rows), d))
        first = int(lo) == max(0, int(rows[0]) - W + 1) // kv_tile
        n_sink = min(-(-S // kv_tile), int(lo)) if first else 0
        for kt in list(range(n_sink)) + list(range(lo, hi)):
            keys = np.arange(kt * kv_tile, min(T, (kt + 1) * kv_tile))
            s = np.where(_visible(rows, keys, W, S), scale * q[b, h, rows] @ k[b, g, keys].T, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            m_use = np.where(np.isneginf(m_new), 0.0, m_new)
            alpha = np.exp(m - m_use)
            p = np.exp(s - m_use[:, None])
            # a about the new reference: the old terms move by (m - m_use) each (rows with a reference only)
            shift = np.where(np.isneginf(m), 0.0, m - m_use)
            with np.errstate(invalid="ignore"):  # masked keys: p = 0 times s - m = -inf, dropped by the where
                a = alpha * (a + shift * l) + np.where(p > 0, p * (s - m_use[:, None]), 0.0).sum(axis=1)
            l = l * alpha + p.sum(axis=1)
            acc = acc * alpha[:, None] + p @ v[b, g, keys]
            m = m_new
        if slot < 0:
            O[b, h, rows] = acc / l[:, None]
            L[b, h, rows] = m + np.log(l)
            ENT[b, h, rows] = np.log(l) - a / l
            NRM[b, h, rows] = np.linalg.norm(acc, axis=1) / l
        else:
            assert int(slot) not in parts, "slot written twice"
            parts[int(slot)] = (m, l, acc, a)
    for bh, qt, first, n in merges:
        b, h = divmod(int(bh), H)
        rows = np.arange(qt * q_tile, min(T, (qt + 1) * q_tile))
        ms = np.stack([parts[first + c][0] for c in range(n)])
        M = ms.max(axis=0)
        w = np.exp(ms - M)  # 0 for a chunk a row did not see (m = -inf)
        l = sum(w[c] * parts[first + c][1] for c in range(n))
        acc = sum(w[c][:, None] * parts[first + c][2] for c in range(n))
        with np.errstate(invalid="ignore"):  # a chunk the row did not see: -inf times 0, dropped by the where
            A = sum(np.where(np.isneginf(ms[c]), 0.0,
                             w[c] * (parts[first + c][3] + (ms[c] - M) * parts[first + c][1])) for c in range(n))
        O[b, h, rows] = acc / l[:, None]
        L[b, h, rows] = M + np.log(l)
        ENT[b, h, rows] = np.log(l) - A / l
        NRM[b, h, rows] = np.linalg.norm(acc, axis=1) / l
    return (O, L, ENT, NRM) if diag else (O, L)


def emulate_backward(items, q, k, v, do, lse, windows, scale, q_tile, kv_tile, sinks=None, split=False):
    """Key-stationary backward over the backward work list: dK, dV per key tile of a key/value head
    (summed over its query heads), dQ accumulated from every key tile.  split: the list may hold several
    chunks of one key tile, each over its own query tiles [lo, hi); their dK, dV sums add up."""
    q, k, v, do, lse = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do, lse))
    B, H, T, d = q.shape
    H_kv = k.shape[1]
    G = H // H_kv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k) if split else np.full_like(k, np.nan)
    dv = np.zeros_like(v) if split else np.full_like(v, np.nan)
    for bh, kt, lo, hi in items:
        if bh < 0:
            continue
        b, g = divmod(int(bh), H_kv)
        keys = np.arange(kt * kv_tile, min(T, (kt + 1) * kv_tile))
        k0, k1 = int(keys[0]), int(keys[-1]) + 1
        dk_t = np.zeros((len(keys), d))
        dv_t = np.zeros((len(keys), d))
        for h in range(g * G, (g + 1) * G):
            W = min(int(windows[h]), T)
            S = _eff_sink(sinks, h, T, W)
            last = T - 1 if k0 < S else min(T, k1 + W - 1) - 1
            for qt in range(lo, min(hi, last // q_tile + 1) if split else last // q_tile + 1):
                rows = np.arange(qt * q_tile, min(T, (qt + 1) * q_tile))
                s = scale * q[b, h, rows] @ k[b, g, keys].T
                ok = _visible(rows, keys, W, S)
                p = np.where(ok, np.exp(s - lse[b, h, rows][:, None]), 0.0)
                # D for these rows: sum over the row's whole key set of P * dP
                Drow = np.empty(len(rows))
                for n, i in enumerate(rows):
                    kk = np.union1d(np.arange(max(0, i - W + 1), i + 1), np.arange(min(S, i + 1)))
                    pi = np.exp(scale * k[b, g, kk] @ q[b, h, i] - lse[b, h, i])
                    Drow[n] = pi @ (v[b, g, kk] @ do[b, h, i])
                dp = do[b, h, rows] @ v[b, g, keys].T
                ds = p * (dp - Drow[:, None])
                dv_t += p.T @ do[b, h, rows]
                dk_t += scale * ds.T @ q[b, h, rows]
                dq[b, h, rows] += scale * ds @ k[b, g, keys]
        if split:
            dk[b, g, keys] += dk_t
            dv[b, g, keys] += dv_t
        else:
            dk[b, g, keys] = dk_t
            dv[b, g, keys] = dv_t
    return dq, dk, dv
