"""A per-element error bound for the bf16 attention outputs, derived from the kernels' own rounding.

The output tolerance (2e-2 absolute + 2e-2 relative) cannot tell a right long-context result from a
wrong one: with N(0, 1) data the output of a row over L keys has a spread of about sqrt(e / L),
0.009 at L = 32768, so a kernel that skipped a whole block (or a 512-token partition) would still
pass it. The bound below is what the arithmetic of the matrix-core kernels allows, and no more.

What the kernels round (the rest is fp32 on exact bf16 inputs, errors of order 1e-6 relative):
  (a) each softmax weight p_t = exp(s_t - m) is rounded to bf16 before the P.V contraction on the
      matrix cores: p_t (1 + d_t) with |d_t| <= u = 2^-8 (bf16 keeps 8 significant bits; round to
      nearest even). The normaliser sum_t p_t uses the unrounded weights. So the fp32 result is
      x = y + e with e = sum_t w_t d_t V_t, where y is the exact output and w_t = p_t / sum p the
      softmax weights (with a sink: p_t over the denominator that includes e^(sigma - m)).
  (b) x is rounded to bf16 once: |round(x) - x| <= u |x| <= u |y| + u |e|.
Treating the d_t as independent, zero-mean and bounded by u (the probabilistic model of rounding
errors of Higham and Mary, "A new approach to probabilistic rounding error analysis", SIAM J. Sci.
Comput. 2019), Hoeffding's inequality gives, for each element d,
    P(|e_d| >= k u tau_d) <= 2 exp(-k^2 / 2),  tau_d = sqrt(sum_t w_t^2 V_t[d]^2),
which is 4.6e-11 for k = 7: over a million elements, a false failure has odds below 1e-4. Hence
    |got - y| <= u |y| + (1 + u) 7 u tau + 1e-5 |y| + 1e-5,
the last two terms for the fp32 score, exponential and accumulation errors. Paths that do not
round the weights (the fp32 and generic bf16 decode) satisfy it a fortiori.

tau is about sqrt(e / L) u-sized for N(0, 1) data, i.e. it shrinks with the context like the
output itself, which is what gives the bound its power (tests/test_rounding_bound.py shows a
dropped block failing it at the long-context sizes where the output tolerance passes).

The spread tau is computed here from the oracle's gather (decode_values, gather_kv) and the plain
softmax; it is test machinery, not the oracle's arithmetic.
"""

from __future__ import annotations

import numpy as np

import oracle

U = 2.0 ** -8
K_SIGMA = 7.0
FP32_REL = 1e-5
FP32_ABS = 1e-5


def row_spread(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, first: np.ndarray,
               last: np.ndarray, sink=None) -> np.ndarray:
    """tau for query rows q_rows [n, D] over keys K, V [L, D]; row r sees keys first[r] .. last[r];
    sink: None, one logit for every row, or one per row."""
    S = scale * (q_rows @ K.T)  # [n, L]
    t = np.arange(K.shape[0])
    mask = (t[None, :] >= np.asarray(first)[:, None]) & (t[None, :] <= np.asarray(last)[:, None])
    S = np.where(mask, S, -np.inf)
    M = S.max(axis=1, keepdims=True)
    sg = None if sink is None else np.broadcast_to(np.asarray(sink, np.float64), (S.shape[0],))[:, None]
    if sg is not None:
        M = np.maximum(M, sg)
    W = np.where(mask, np.exp(S - M), 0.0)
    den = W.sum(axis=1, keepdims=True)
    if sg is not None:
        den = den + np.exp(sg - M)
    W = W / den
    return np.sqrt((W * W) @ (V * V))


def decode_spread(q, k_pool, v_pool, block_tables, context_lens, scale, block_size, dtype, sinks=None,
                  window: int = 0) -> np.ndarray:
    """tau [B, Hq, D] of the decode outputs (pools after the append; sinks as bits, or None)."""
    qv = oracle.decode_values(q, dtype)
    B, Hq, D = qv.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    sig = None if sinks is None else oracle.decode_values(np.asarray(sinks), dtype)
    tau = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(context_lens[b])
        if L <= 0:
            continue
        nblk = (L + block_size - 1) // block_size
        ids = np.asarray(block_tables[b, :nblk], dtype=np.int64)
        K = oracle.gather_kv(oracle.decode_values(k_pool[ids], dtype), np.arange(nblk), L, block_size)
        V = oracle.gather_kv(oracle.decode_values(v_pool[ids], dtype), np.arange(nblk), L, block_size)
        t0 = max(0, L - window) if window > 0 else 0
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            tau[b, hs] = row_spread(qv[b, hs], K[g], V[g], scale, np.full(G, t0), np.full(G, L - 1),
                                    None if sig is None else sig[hs])
    return tau


def prefill_spread(q, k_pool, v_pool, block_tables, start_pos, chunk_lens, scale, block_size, dtype, sinks=None,
                   window: int = 0, b_rows=None) -> np.ndarray:
    """tau [B, Hq, C, D] of the chunked-prefill outputs; b_rows: optional {b: (i0, i1)} to compute
    only rows i0 .. i1-1 of sequence b (the others stay 0)."""
    qv = oracle.decode_values(q, dtype)
    B, Hq, C, D = qv.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    sig = None if sinks is None else oracle.decode_values(np.asarray(sinks), dtype)
    tau = np.zeros((B, Hq, C, D))
    for b in range(B):
        s0, n = int(start_pos[b]), int(chunk_lens[b])
        if n <= 0 or (b_rows is not None and b not in b_rows):
            continue
        i0, i1 = (0, n) if b_rows is None else b_rows[b]
        L = s0 + n
        nblk = (L + block_size - 1) // block_size
        ids = np.asarray(block_tables[b, :nblk], dtype=np.int64)
        K = oracle.gather_kv(oracle.decode_values(k_pool[ids], dtype), np.arange(nblk), L, block_size)
        V = oracle.gather_kv(oracle.decode_values(v_pool[ids], dtype), np.arange(nblk), L, block_size)
        p = s0 + np.arange(i0, i1)
        first = np.maximum(p + 1 - window, 0) if window > 0 else np.zeros_like(p)
        for h in range(Hq):
            tau[b, h, i0:i1] = row_spread(qv[b, h, i0:i1], K[h // G], V[h // G], scale, first, p,
                                          None if sig is None else float(sig[h]))
    return tau


def bound(ref: np.ndarray, tau: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    return U * a + (1 + U) * K_SIGMA * U * tau + FP32_REL * a + FP32_ABS


def violations(got: np.ndarray, ref: np.ndarray, tau: np.ndarray) -> int:
    return int(np.sum(~(np.abs(got - ref) <= bound(ref, tau))))


def assert_rounding_bound(got: np.ndarray, ref: np.ndarray, tau: np.ndarray, what: str) -> float:
    """Raises unless every element is within the bound; returns the largest error / bound."""
    assert got.shape == ref.shape == tau.shape, (what, got.shape, ref.shape, tau.shape)
    err = np.abs(got - ref)
    lim = bound(ref, tau)
    bad = ~(err <= lim)
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond the rounding bound; first at {idx}: got "
                             f"{got[idx]!r} ref {ref[idx]!r} err {err[idx]:.3g} bound {lim[idx]:.3g} "
                             f"(max err/bound {float((err / lim).max()):.3g})")
    return float((err / lim).max()) if err.size else 0.0
