"""fp64 oracle of paged decode attention with attention sinks and a sliding window.
TEST INFRASTRUCTURE ONLY (same rules as ``oracle.paged_attention``).

Sources on the xserv pages (xserv compare phase10...cf1e9e41, diff of
crates/xserv-kernels/src/attention.rs):

* `paged_decode_attention_sinks` and its FFI `launch_paged_decode_attention_sinks_bf16`:
  the same paged decode as `paged_decode_attention`, plus a pointer to one bf16
  sink value per query head (null: no sinks) and a `window_size` (0: full
  attention, > 0: sliding window).
* `flash_attention_sinks` (same diff): the per-head sinks are the gpt-oss
  attention sinks, folded into the softmax denominator.

Readings where the pages are silent:

* The sink sigma_h is a logit in the same units as the scaled scores
  s_t = scale * q_h . K_t. It joins the softmax as one more entry that has no
  value row, so it only enlarges the denominator:
      out = sum_t e^(s_t - M) V_t / (e^(sigma_h - M) + sum_t e^(s_t - M)),
      M = max(sigma_h, max_t s_t).
* A window W > 0 keeps the last W positions, the query's own included: the
  token at L - 1 attends to t in [max(0, L - W), L). W = 0 keeps all L.
* L = 0 gives zeros (there is no value row to weigh), with or without a sink.
* Split-K with a window: partition j still covers [j*P, (j+1)*P) of the
  sequence, cut to the window; partitions wholly before the window start do
  not exist. The sink enters once, in the merge:
      M = max(sigma, max_j m_j),  out = sum_j l_j e^(m_j - M) o_j
                                        / (e^(sigma - M) + sum_j l_j e^(m_j - M)).
"""

from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np

from .paged_attention import _scores, decode_values, gather_kv


def window_start(L: int, window: int) -> int:
    """First position the query at L - 1 attends to."""
    return max(0, L - window) if window > 0 else 0


def _sink_values(sinks, dtype: str, Hq: int) -> Optional[np.ndarray]:
    if sinks is None:
        return None
    s = decode_values(np.asarray(sinks), dtype)
    if s.shape != (Hq,):
        raise ValueError("sinks must hold one value per query head")
    return s


def _sequence_kv(k_cache, v_cache, bt_row, L, block_size, dtype):
    nblk = (L + block_size - 1) // block_size
    ids = np.asarray(bt_row[:nblk], dtype=np.int64)
    K = gather_kv(decode_values(k_cache[ids], dtype), np.arange(nblk), L, block_size)
    V = gather_kv(decode_values(v_cache[ids], dtype), np.arange(nblk), L, block_size)
    return K, V


def paged_decode_attention_sinks(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, dtype,
                                 sinks=None, window: int = 0):
    """Decode attention over the paged pool with per-head sinks and a sliding window, in fp64.

    out[b, h] = sum_{t in [t0, L)} e^(s_t - M) V_t / (e^(sigma_h - M) + sum_{t in [t0, L)} e^(s_t - M))
    with t0 = window_start(L, window) and M = max(sigma_h, max s_t). Without sinks the sigma term
    is absent.
    """
    qv = decode_values(q, dtype)
    B, Hq, D = qv.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    n_rep = Hq // Hkv
    sig = _sink_values(sinks, dtype, Hq)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L <= 0:
            continue
        t0 = window_start(L, window)
        K, V = _sequence_kv(k_cache, v_cache, block_tables[b], L, block_size, dtype)
        for h in range(Hq):
            g = h // n_rep
            s = _scores(qv[b, h], K[g, t0:], scale)
            M = s.max() if sig is None else max(s.max(), sig[h])
            w = np.exp(s - M)
            den = w.sum() + (0.0 if sig is None else np.exp(sig[h] - M))
            out[b, h] = (w @ V[g, t0:]) / den
    return out


def partition_stats_window(s: np.ndarray, V: np.ndarray, t0: int, partition_size: int):
    """Partitions of one row under a window: j runs over [t0 // P, ceil(L / P)), partition j covers
    tokens [max(j*P, t0), min((j+1)*P, L)). Returns (j0, o [n, D], m [n], l [n])."""
    L = s.shape[0]
    j0 = t0 // partition_size
    n_end = (L + partition_size - 1) // partition_size
    o, m, l = [], [], []
    for j in range(j0, n_end):
        sl = slice(max(j * partition_size, t0), min((j + 1) * partition_size, L))
        mj = s[sl].max()
        e = np.exp(s[sl] - mj)
        o.append((e @ V[sl]) / e.sum())
        m.append(mj)
        l.append(e.sum())
    return j0, np.array(o).reshape(-1, V.shape[1]), np.array(m), np.array(l)


def lse_merge_sink(o: np.ndarray, m: np.ndarray, l: np.ndarray, sink: Optional[float]) -> np.ndarray:
    """M = max(sink, max m_j), out = sum l_j e^(m_j - M) o_j / (e^(sink - M) + sum l_j e^(m_j - M))."""
    if m.size == 0:
        return np.zeros(o.shape[1] if o.ndim == 2 else 0)
    M = m.max() if sink is None else max(m.max(), sink)
    w = l * np.exp(m - M)
    den = w.sum() + (0.0 if sink is None else np.exp(sink - M))
    return (w @ o) / den


def split_paged_decode_attention_sinks(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, dtype,
                                       partition_size, sinks=None, window: int = 0) -> Tuple[np.ndarray, List]:
    """Partition-by-partition decode under the window, merged with the sink.

    Returns (out [B, Hq, D], stats) with stats[b][h] = (j0, o, m, l) for partitions j0, j0+1, ...
    """
    qv = decode_values(q, dtype)
    B, Hq, D = qv.shape
    n_rep = Hq // k_cache.shape[1]
    sig = _sink_values(sinks, dtype, Hq)
    out = np.zeros((B, Hq, D))
    stats = []
    for b in range(B):
        L = int(context_lens[b])
        row = []
        if L > 0:
            t0 = window_start(L, window)
            K, V = _sequence_kv(k_cache, v_cache, block_tables[b], L, block_size, dtype)
        for h in range(Hq):
            if L <= 0:
                row.append((0, np.zeros((0, D)), np.zeros(0), np.zeros(0)))
                continue
            g = h // n_rep
            s = _scores(qv[b, h], K[g], scale)
            j0, o, m, l = partition_stats_window(s, V[g], t0, partition_size)
            row.append((j0, o, m, l))
            out[b, h] = lse_merge_sink(o, m, l, None if sig is None else sig[h])
        stats.append(row)
    return out, stats
