"""fp64 oracle of the paged-KV decode step. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module. It shares no code with the HIP path.

Sources on the xserv pages:

* Pool layout: one pool each for K and V, logical shape
  [num_blocks, num_kv_heads, block_size, head_dim]. Block table: int32
  [batch, max_blocks_per_seq], rows already in batch order. context_lens:
  int32 [batch]. From xserv compare phase10...cf1e9e41, diff of
  crates/xserv-kernels/src/attention.rs, doc comments of
  `reshape_and_cache_bf16` and `paged_decode_attention`.
* Append: the batched scatter writes one new K/V row per sequence. kv_lens
  is the current length plus one, which is the index of the just-written
  token plus one. Same diff, doc comment of `reshape_and_cache_batched_bf16`.
  The source layout [num_kv_heads, num_tokens, head_dim] of the single-sequence
  scatter, with one token per sequence, gives k_new/v_new = [batch,
  num_kv_heads, head_dim].
* Decode attention: q has one token per sequence, [batch, num_q_heads, 1,
  head_dim]. num_q_heads is a multiple of num_kv_heads. The output has q's
  shape. Same diff, `paged_decode_attention` and `decode_attention`. The
  single query sits at the last position, so the causal mask lets it see all
  L keys.
* GQA: q head h reads kv head h // n_rep, with n_rep = num_q_heads /
  num_kv_heads. From xserv compare phase8...phase13, `repeat_kv` in the Qwen3
  model and the `repeat_kv_bf16` kernel: out head kv_h * n_rep + r copies kv
  head kv_h.
* Naive attention: the full score matrix, the causal mask, softmax, then
  weights times V. From xserv compare phase10...cf1e9e41, attention.rs,
  `attention(q, k, v, causal)`. The phase-9 benchmark doc (xserv compare
  phase5...phase9) states that decoding with the cache gives the same result
  as recomputing everything.

Readings where the pages are silent:

* Softmax is taken max-subtracted. That is the same function, written in a
  stable form.
* L = 0 gives an all-zero output.
* Split partitions and their log-sum-exp merge are not on the pages. Partition
  j covers tokens [j*P, min((j+1)*P, L)). It keeps m_j = max s,
  l_j = sum exp(s - m_j) and o_j = sum exp(s - m_j) V / l_j. The merge is
  M = max m_j, w_j = l_j exp(m_j - M), out = sum w_j o_j / sum w_j. This is
  an exact identity of the unsplit softmax.

bf16 values are given as uint16 bit patterns and float32 as float32. Every
stored value is exact in fp64, and all arithmetic here is fp64.
"""

from __future__ import annotations

from typing import List, Tuple

import numpy as np


def decode_values(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of stored bf16 (uint16 bits) or float32 data."""
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must be given as uint16 bit patterns")
        # A bf16 value is the float32 whose top 16 bits are the pattern.
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def kv_append(k_cache, v_cache, k_new, v_new, block_tables, context_lens, block_size):
    """Decode-step append: copy each sequence's new K/V row into slot L_b - 1.

    For sequence b with L = context_lens[b] >= 1, position p = L - 1 lives in
    physical block block_tables[b, p // block_size], at offset p % block_size.
    Row [blk, g, off, :] of each pool becomes k_new[b, g, :] (v_new likewise)
    for every kv head g. No other byte changes. The arrays are copied, so the
    inputs are left as they were. The copy moves raw stored values and no
    rounding takes place.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    for b in range(len(context_lens)):
        L = int(context_lens[b])
        if L <= 0:
            continue
        p = L - 1
        blk = int(block_tables[b, p // block_size])
        off = p % block_size
        k_out[blk, :, off, :] = k_new[b]
        v_out[blk, :, off, :] = v_new[b]
    return k_out, v_out


def gather_kv(cache_values: np.ndarray, block_table_row: np.ndarray, L: int, block_size: int) -> np.ndarray:
    """Logical K (or V) of one sequence, [num_kv_heads, L, head_dim].

    Token t comes from physical block block_table_row[t // block_size], slot
    t % block_size. ``cache_values`` is the pool as fp64 values.
    """
    if L <= 0:
        return np.zeros((cache_values.shape[1], 0, cache_values.shape[3]), dtype=np.float64)
    nblk = (L + block_size - 1) // block_size
    ids = np.asarray(block_table_row[:nblk], dtype=np.int64)
    chunks = cache_values[ids]  # [nblk, Hkv, BS, D]
    seq = np.transpose(chunks, (1, 0, 2, 3)).reshape(cache_values.shape[1], nblk * block_size, -1)
    return seq[:, :L, :]


def _scores(q_h: np.ndarray, K_g: np.ndarray, scale: float) -> np.ndarray:
    # s_t = scale * sum_d q[d] K_t[d]
    return scale * (K_g @ q_h)


def paged_decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, dtype):
    """Single-token GQA decode attention over the paged pool, in fp64.

    Returns out [B, Hq, D]. out[b, h] = sum_t w_t V_t / sum_t w_t, where
    w_t = exp(s_t - max s), s_t = scale * q[b, h] . K_t, and K_t, V_t are
    token t of kv head h // (Hq / Hkv) of sequence b, for t in [0, L_b).
    """
    qv = decode_values(q, dtype)
    B, Hq, D = qv.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    n_rep = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L <= 0:
            continue
        nblk = (L + block_size - 1) // block_size
        ids = np.asarray(block_tables[b, :nblk], dtype=np.int64)
        # Decode only the blocks this sequence owns (keeps memory bounded on big pools).
        K = gather_kv(decode_values(k_cache[ids], dtype), np.arange(nblk), L, block_size)
        V = gather_kv(decode_values(v_cache[ids], dtype), np.arange(nblk), L, block_size)
        for h in range(Hq):
            g = h // n_rep
            s = _scores(qv[b, h], K[g], scale)
            w = np.exp(s - s.max())
            out[b, h] = (w @ V[g]) / w.sum()
    return out


def attention_weights(q, k_cache, block_tables, context_lens, scale, block_size, dtype):
    """Softmax weights per (b, h): a list over b of arrays [Hq, L_b]."""
    qv = decode_values(q, dtype)
    B, Hq, D = qv.shape
    n_rep = Hq // k_cache.shape[1]
    res = []
    for b in range(B):
        L = int(context_lens[b])
        K = gather_kv(decode_values(k_cache, dtype), block_tables[b], L, block_size)
        W = np.zeros((Hq, L))
        for h in range(Hq):
            if L == 0:
                continue
            s = _scores(qv[b, h], K[h // n_rep], scale)
            w = np.exp(s - s.max())
            W[h] = w / w.sum()
        res.append(W)
    return res


def partition_stats(s: np.ndarray, V: np.ndarray, partition_size: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Softmax statistics of each partition of one (sequence, head) row.

    s: scores [L]; V: values [L, D]. Partition j covers tokens
    [j*P, min((j+1)*P, L)). Returns (o [n, D], m [n], l [n]) with
    m_j = max s, l_j = sum exp(s - m_j) and o_j = sum exp(s - m_j) V / l_j.
    """
    L = s.shape[0]
    n = (L + partition_size - 1) // partition_size
    o = np.zeros((n, V.shape[1]))
    m = np.zeros(n)
    l = np.zeros(n)
    for j in range(n):
        sl = slice(j * partition_size, min((j + 1) * partition_size, L))
        m[j] = s[sl].max()
        e = np.exp(s[sl] - m[j])
        l[j] = e.sum()
        o[j] = (e @ V[sl]) / l[j]
    return o, m, l


def lse_merge(o: np.ndarray, m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """Merge partition results. M = max m_j, w_j = l_j exp(m_j - M), out = sum w_j o_j / sum w_j."""
    if m.size == 0:
        return np.zeros(o.shape[1] if o.ndim == 2 else 0)
    M = m.max()
    w = l * np.exp(m - M)
    return (w @ o) / w.sum()


def split_paged_decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, dtype,
                                 partition_size) -> Tuple[np.ndarray, List]:
    """Decode attention computed partition by partition, then merged.

    Returns (out [B, Hq, D], stats), where stats[b][h] = (o, m, l) of that row's partitions.
    """
    qv = decode_values(q, dtype)
    B, Hq, D = qv.shape
    n_rep = Hq // k_cache.shape[1]
    out = np.zeros((B, Hq, D))
    stats = []
    for b in range(B):
        L = int(context_lens[b])
        row = []
        if L > 0:
            nblk = (L + block_size - 1) // block_size
            ids = np.asarray(block_tables[b, :nblk], dtype=np.int64)
            K = gather_kv(decode_values(k_cache[ids], dtype), np.arange(nblk), L, block_size)
            V = gather_kv(decode_values(v_cache[ids], dtype), np.arange(nblk), L, block_size)
        for h in range(Hq):
            if L <= 0:
                row.append((np.zeros((0, D)), np.zeros(0), np.zeros(0)))
                continue
            g = h // n_rep
            s = _scores(qv[b, h], K[g], scale)
            o, m, l = partition_stats(s, V[g], partition_size)
            row.append((o, m, l))
            out[b, h] = lse_merge(o, m, l)
        stats.append(row)
    return out, stats


def naive_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Naive multi-head causal attention on contiguous fp64 tensors.

    q: [Hq, S, D]; k, v: [Hkv, S, D]. K/V heads are first repeated so that
    head h uses kv head h // n_rep. Then the full S x S score matrix is
    formed, every entry above the diagonal is masked to -inf, softmax runs
    along rows, and the weights multiply V. Returns [Hq, S, D].
    """
    Hq, S, D = q.shape
    n_rep = Hq // k.shape[0]
    kr = np.repeat(k, n_rep, axis=0)
    vr = np.repeat(v, n_rep, axis=0)
    scores = scale * np.einsum("hsd,htd->hst", q, kr)
    mask = np.triu(np.ones((S, S), dtype=bool), k=1)
    scores = np.where(mask[None], -np.inf, scores)
    scores = scores - scores.max(axis=-1, keepdims=True)
    w = np.exp(scores)
    w = w / w.sum(axis=-1, keepdims=True)
    return np.einsum("hst,htd->hsd", w, vr)
