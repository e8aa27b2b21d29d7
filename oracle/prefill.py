"""fp64 oracle of the chunked-prefill step over the paged pool: multi-token append, then causal
attention of the chunk's queries over everything cached so far. TEST INFRASTRUCTURE ONLY (same
rules as ``oracle.paged_attention``).

Sources on the xserv pages (xserv compare phase10...cf1e9e41, attention.rs):

* `reshape_and_cache_bf16`: scatter K/V of shape [num_kv_heads, num_tokens, head_dim] into one
  sequence's paged blocks, starting at position `start_pos`; token i goes to position
  start_pos + i, that is block block_ids[(start_pos + i) / block_size], slot
  (start_pos + i) % block_size, for every kv head.
* `flash_attention(q, k, v, causal)`: q [batch, num_q_heads, q_len, head_dim] against K/V of
  kv_len positions, GQA, optional causal mask; output has q's shape.

Readings where the pages are silent:

* Batching: k_src, v_src are [batch, num_kv_heads, chunk, head_dim], q and out are
  [batch, num_q_heads, chunk, head_dim]; sequence b's chunk starts at start_pos[b] and has
  chunk_lens[b] <= chunk valid rows (a last chunk may be short). Rows at or past chunk_lens[b]
  are not part of the chunk: the append skips them and their output is zero.
* Causal alignment with a cached prefix: row i of sequence b sits at position p = start_pos[b] + i
  and sees keys t in [0, p] (the bottom-right aligned mask of `flash_attention` with
  kv_len = start_pos[b] + chunk_lens[b]). With start_pos = 0 this is the pages' naive causal
  attention.

Sinks and a sliding window (same diff, `flash_attention_sinks`: the prefill attention of the
gpt-oss layers, always causal, one sink per query head folded into the softmax denominator,
window_size 0 for full causal attention and > 0 for a sliding window), over the paged pool:

* The window reads as in the decode with sinks: the query at position p keeps the last W
  positions up to and including its own, t in [max(0, p + 1 - W), p]; W = 0 keeps [0, p].
* The sink sigma_h of query head h is a logit in the units of the scaled scores and only enlarges
  the denominator: out = sum_t e^(s_t - M) V_t / (e^(sigma_h - M) + sum_t e^(s_t - M)),
  M = max(sigma_h, max_t s_t).
"""

from __future__ import annotations

import numpy as np

from .paged_attention import _scores, decode_values, gather_kv


def kv_append_chunk(k_cache, v_cache, k_src, v_src, block_tables, start_pos, chunk_lens, block_size):
    """Returns new pools with each sequence's chunk written at positions start_pos[b] + i."""
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    for b in range(len(start_pos)):
        s0, n = int(start_pos[b]), int(chunk_lens[b])
        for i in range(max(n, 0)):
            p = s0 + i
            blk = int(block_tables[b, p // block_size])
            k_out[blk, :, p % block_size, :] = k_src[b, :, i, :]
            v_out[blk, :, p % block_size, :] = v_src[b, :, i, :]
    return k_out, v_out


def paged_prefill_attention(q, k_cache, v_cache, block_tables, start_pos, chunk_lens, scale, block_size, dtype):
    """out[b, h, i] = sum_{t <= p} e^(s_t - m) V_t / sum_{t <= p} e^(s_t - m), p = start_pos[b] + i,
    s_t = scale * q[b, h, i] . K_t, K_t / V_t token t of kv head h // (Hq / Hkv) of sequence b, for
    i < chunk_lens[b]; zero for the other rows."""
    qv = decode_values(q, dtype)
    B, Hq, C, D = qv.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    n_rep = Hq // Hkv
    out = np.zeros((B, Hq, C, D))
    for b in range(B):
        s0, n = int(start_pos[b]), int(chunk_lens[b])
        if n <= 0:
            continue
        L = s0 + n
        nblk = (L + block_size - 1) // block_size
        ids = np.asarray(block_tables[b, :nblk], dtype=np.int64)
        K = gather_kv(decode_values(k_cache[ids], dtype), np.arange(nblk), L, block_size)
        V = gather_kv(decode_values(v_cache[ids], dtype), np.arange(nblk), L, block_size)
        for h in range(Hq):
            g = h // n_rep
            for i in range(n):
                p = s0 + i
                s = _scores(qv[b, h, i], K[g, :p + 1], scale)
                w = np.exp(s - s.max())
                out[b, h, i] = (w @ V[g, :p + 1]) / w.sum()
    return out


def window_first(p: int, window: int) -> int:
    """First key position that the query at position p sees under a window of W (0: none)."""
    return max(0, p + 1 - window) if window > 0 else 0


def paged_prefill_attention_sinks(q, k_cache, v_cache, block_tables, start_pos, chunk_lens, scale, block_size,
                                  dtype, sinks=None, window: int = 0):
    """Chunked-prefill attention with per-head sinks and a sliding window, in fp64:
    out[b, h, i] = sum_{t in [t0, p]} e^(s_t - M) V_t / (e^(sigma_h - M) + sum_{t in [t0, p]} e^(s_t - M))
    with p = start_pos[b] + i, t0 = window_first(p, window), s_t = scale * q[b, h, i] . K_t and
    M = max(sigma_h, max s_t); without sinks the sigma term is absent. Rows at or past
    chunk_lens[b] are zero."""
    qv = decode_values(q, dtype)
    B, Hq, C, D = qv.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if window < 0:
        raise ValueError("window must be >= 0")
    n_rep = Hq // Hkv
    sig = None
    if sinks is not None:
        sig = decode_values(np.asarray(sinks), dtype)
        if sig.shape != (Hq,):
            raise ValueError("sinks must hold one value per query head")
    out = np.zeros((B, Hq, C, D))
    for b in range(B):
        s0, n = int(start_pos[b]), int(chunk_lens[b])
        if n <= 0:
            continue
        L = s0 + n
        nblk = (L + block_size - 1) // block_size
        ids = np.asarray(block_tables[b, :nblk], dtype=np.int64)
        K = gather_kv(decode_values(k_cache[ids], dtype), np.arange(nblk), L, block_size)
        V = gather_kv(decode_values(v_cache[ids], dtype), np.arange(nblk), L, block_size)
        for h in range(Hq):
            g = h // n_rep
            for i in range(n):
                p = s0 + i
                t0 = window_first(p, window)
                s = _scores(qv[b, h, i], K[g, t0:p + 1], scale)
                M = s.max() if sig is None else max(s.max(), sig[h])
                w = np.exp(s - M)
                den = w.sum() + (0.0 if sig is None else np.exp(sig[h] - M))
                out[b, h, i] = (w @ V[g, t0:p + 1]) / den
    return out
