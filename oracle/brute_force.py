"""40-digit ``decimal`` brute force of paged decode attention. TEST INFRASTRUCTURE ONLY.

This is a second, independent statement of the same definition as
``paged_attention.paged_decode_attention``. It is used only to check that
function on tiny inputs. It reads the pools through flat row-major offsets
of the logical shape [num_blocks, num_kv_heads, block_size, head_dim]
(xserv compare phase10...cf1e9e41, attention.rs, doc comment of
`paged_decode_attention`), so it does not reuse numpy's 4-D indexing.
It maps GQA as kv head = h // n_rep (xserv compare phase8...phase13,
`repeat_kv`). ``Decimal.exp`` is correctly rounded at the working precision.
"""

from __future__ import annotations

from decimal import Decimal, getcontext
from typing import List


def brute_decode_attention(q_vals: List[List[List[float]]], k_flat: List[float], v_flat: List[float],
                           block_tables: List[List[int]], context_lens: List[int], scale: float,
                           num_kv_heads: int, block_size: int, head_dim: int) -> List[List[List[Decimal]]]:
    """q_vals[b][h][d] and the flat pools hold the exact stored values as Python floats."""
    getcontext().prec = 40
    B = len(q_vals)
    Hq = len(q_vals[0]) if B else 0
    n_rep = Hq // num_kv_heads
    sc = Decimal(scale)
    out = []
    for b in range(B):
        L = context_lens[b]
        rows = []
        for h in range(Hq):
            if L <= 0:
                rows.append([Decimal(0)] * head_dim)
                continue
            g = h // n_rep
            scores = []
            for t in range(L):
                blk = block_tables[b][t // block_size]
                base = ((blk * num_kv_heads + g) * block_size + (t % block_size)) * head_dim
                acc = Decimal(0)
                for d in range(head_dim):
                    acc += Decimal(q_vals[b][h][d]) * Decimal(k_flat[base + d])
                scores.append(sc * acc)
            mx = max(scores)
            weights = [(s - mx).exp() for s in scores]
            total = sum(weights, Decimal(0))
            o = []
            for d in range(head_dim):
                num = Decimal(0)
                for t in range(L):
                    blk = block_tables[b][t // block_size]
                    base = ((blk * num_kv_heads + g) * block_size + (t % block_size)) * head_dim
                    num += weights[t] * Decimal(v_flat[base + d])
                o.append(num / total)
            rows.append(o)
        out.append(rows)
    return out


def brute_decode_attention_sinks(q_vals: List[List[List[float]]], k_flat: List[float], v_flat: List[float],
                                 block_tables: List[List[int]], context_lens: List[int], scale: float,
                                 num_kv_heads: int, block_size: int, head_dim: int, sinks, window: int
                                 ) -> List[List[List[Decimal]]]:
    """Decode attention with attention sinks and a sliding window, at 40 digits.

    Sources and readings as in ``oracle.sinks_window``: head h's sink (``sinks[h]``, or none when
    ``sinks`` is None) is one more softmax logit with no value row; the window keeps positions
    t >= L - window (all when window is 0).
    """
    getcontext().prec = 40
    B = len(q_vals)
    Hq = len(q_vals[0]) if B else 0
    n_rep = Hq // num_kv_heads
    sc = Decimal(scale)
    out = []
    for b in range(B):
        L = context_lens[b]
        first = L - window if (window > 0 and L > window) else 0
        rows = []
        for h in range(Hq):
            if L <= 0:
                rows.append([Decimal(0)] * head_dim)
                continue
            g = h // n_rep
            positions = list(range(first, L))
            scores = []
            for t in positions:
                blk = block_tables[b][t // block_size]
                base = ((blk * num_kv_heads + g) * block_size + (t % block_size)) * head_dim
                acc = Decimal(0)
                for d in range(head_dim):
                    acc += Decimal(q_vals[b][h][d]) * Decimal(k_flat[base + d])
                scores.append(sc * acc)
            logits = scores + ([Decimal(sinks[h])] if sinks is not None else [])
            mx = max(logits)
            weights = [(s - mx).exp() for s in scores]
            total = sum(((x - mx).exp() for x in logits), Decimal(0))
            o = []
            for d in range(head_dim):
                num = Decimal(0)
                for i, t in enumerate(positions):
                    blk = block_tables[b][t // block_size]
                    base = ((blk * num_kv_heads + g) * block_size + (t % block_size)) * head_dim
                    num += weights[i] * Decimal(v_flat[base + d])
                o.append(num / total)
            rows.append(o)
        out.append(rows)
    return out
