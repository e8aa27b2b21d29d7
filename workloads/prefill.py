"""Seeded synthetic inputs for one chunked-prefill step (multi-token append + causal attention).

Like the decode workloads, this module only draws and lays out random inputs; it holds none of
the attention arithmetic. The layout follows the xserv pages (xserv compare phase10...cf1e9e41,
attention.rs, `reshape_and_cache_bf16`: a sequence's tokens are written from `start_pos` on
through its block ids; `flash_attention`: q [batch, num_q_heads, q_len, head_dim]).

Recipe:

1. ``rng = numpy.random.default_rng(seed)`` (PCG64).
2. Lengths after the step: L_b = start_pos[b] + chunk_lens[b]. Pool size: given, or
   ceil(1.25 * sum_b ceil(L_b / BS)). Placement: one permutation of [0, NB); its first
   sum_b ceil(L_b / BS) entries are the sequences' blocks in batch order; table padding -1.
3. Values, in this order, float32 N(0, 1) rounded to bf16 (nearest-even) for bf16: q
   [B, Hq, C, D], k_src and v_src [B, Hkv, C, D], then each sequence's K blocks and V blocks in
   batch order. Rows past chunk_lens[b] are drawn too (and must be ignored).
4. Poison: every pool slot at a position >= start_pos[b] (the chunk's own slots, which the
   append must fill, and the tail) and every unused block is NaN.
5. Workloads with sinks (the gpt-oss layers): last, one sink logit per query head, float32
   N(0, 1) rounded to bf16. The window is a fixed size of the workload.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

from . import _encode, _nan_fill, _normal


@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    name: str
    description: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    chunk: int  # C: rows of q / k_src / v_src per sequence
    start_pos: tuple  # per sequence
    chunk_lens: tuple  # per sequence, <= chunk
    max_blocks_per_seq: int
    seed: int
    num_blocks: Optional[int] = None
    window: int = 0  # sliding window W (0: full causal attention)
    sinks: bool = False  # one sink logit per query head

    @property
    def batch(self) -> int:
        return len(self.start_pos)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "PrefillWorkload":
        return dataclasses.replace(self, **kw)

    def key_visits(self) -> int:
        """sum over chunk rows (b, i < n_b) of the keys the row sees (one head): start_pos[b] + i + 1,
        at most W with a sliding window."""
        tot = 0
        for s0, n in zip(self.start_pos, self.chunk_lens):
            n = max(int(n), 0)
            if self.window > 0:
                tot += sum(min(int(s0) + i + 1, self.window) for i in range(n))
            else:
                tot += n * (int(s0) + 1) + n * (n - 1) // 2
        return tot

    def attention_flops(self) -> int:
        """Algorithmic flops of the causal attention: 2 D for q.K plus 2 D for p.V per (head, row, key)."""
        return 4 * self.head_dim * self.num_q_heads * self.key_visits()

    def append_bytes(self) -> int:
        """Bytes the append moves: each chunk row of K and V read once and written once."""
        rows = sum(max(int(n), 0) for n in self.chunk_lens)
        return 2 * 2 * rows * self.num_kv_heads * self.head_dim * self.elt_bytes


@dataclasses.dataclass
class PrefillCase:
    workload: PrefillWorkload
    q: np.ndarray  # [B, Hq, C, D]
    k_src: np.ndarray  # [B, Hkv, C, D]
    v_src: np.ndarray
    k_cache: np.ndarray  # [NB, Hkv, BS, D], before the append
    v_cache: np.ndarray
    block_tables: np.ndarray  # int32 [B, MBPS]
    start_pos: np.ndarray  # int32 [B]
    chunk_lens: np.ndarray  # int32 [B]
    sinks: Optional[np.ndarray] = None  # bf16 bits [Hq] when the workload has sinks


PREFILL_WORKLOADS: Dict[str, PrefillWorkload] = {
    w.name: w
    for w in [
        PrefillWorkload(
            name="qwen3_8b_prefill_c512",
            description="Qwen3-8B shape, bf16 chunked prefill: 4 sequences, 512-token chunks starting at "
            "0, 1024, 2048 and 3584 cached tokens, 32 q / 8 KV heads, head_dim 128, block_size 16",
            dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, chunk=512,
            start_pos=(0, 1024, 2048, 3584), chunk_lens=(512, 512, 512, 512), max_blocks_per_seq=256, seed=6,
        ),
        PrefillWorkload(
            name="qwen3_8b_prefill_long16k",
            description="Qwen3-8B shape, bf16 chunked prefill deep into one long context: 1 sequence, a "
            "512-token chunk after 15872 cached tokens (16384 after the step), 32 q / 8 KV heads, head_dim "
            "128, block_size 16 (64 row blocks: the split-K case)",
            dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, chunk=512,
            start_pos=(15872,), chunk_lens=(512,), max_blocks_per_seq=1024, seed=7,
        ),
        PrefillWorkload(
            name="gptoss_20b_prefill_window128_c512",
            description="gpt-oss-20b sliding-window layer shape, bf16 chunked prefill: 4 sequences, 512-token "
            "chunks starting at 0, 1024, 2048 and 3584 cached tokens, 64 q / 8 KV heads, head_dim 64, "
            "block_size 16, a 128-token window and one sink per query head",
            dtype="bf16", num_q_heads=64, num_kv_heads=8, head_dim=64, block_size=16, chunk=512,
            start_pos=(0, 1024, 2048, 3584), chunk_lens=(512, 512, 512, 512), max_blocks_per_seq=256, seed=8,
            window=128, sinks=True,
        ),
        PrefillWorkload(
            name="gptoss_20b_prefill_full_c512",
            description="gpt-oss-20b full-attention layer shape, bf16 chunked prefill: the same 4 sequences and "
            "chunks, 64 q / 8 KV heads, head_dim 64, block_size 16, no window, one sink per query head",
            dtype="bf16", num_q_heads=64, num_kv_heads=8, head_dim=64, block_size=16, chunk=512,
            start_pos=(0, 1024, 2048, 3584), chunk_lens=(512, 512, 512, 512), max_blocks_per_seq=256, seed=9,
            sinks=True,
        ),
    ]
}


def make_prefill_case(w: PrefillWorkload, seed: Optional[int] = None) -> PrefillCase:
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, Hq, Hkv, D, BS, C = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.chunk
    s0 = np.asarray(w.start_pos, dtype=np.int64)
    n = np.asarray(w.chunk_lens, dtype=np.int64)
    if s0.shape != (B,) or n.shape != (B,) or (n > C).any() or (n < 0).any() or (s0 < 0).any():
        raise ValueError("start_pos / chunk_lens do not fit the chunk")
    L = s0 + n
    if int(L.max(initial=0)) > w.max_blocks_per_seq * BS:
        raise ValueError("a sequence exceeds max_blocks_per_seq * block_size")
    nblk = (L + BS - 1) // BS
    need = int(nblk.sum())
    NB = w.num_blocks if w.num_blocks is not None else max(1, math.ceil(1.25 * need))
    if need > NB:
        raise ValueError(f"{w.name}: {need} blocks needed, pool has {NB}")
    perm = rng.permutation(NB).astype(np.int32)
    bt = np.full((B, w.max_blocks_per_seq), -1, dtype=np.int32)
    start = 0
    for b in range(B):
        bt[b, : nblk[b]] = perm[start : start + nblk[b]]
        start += int(nblk[b])
    q = _encode(_normal(rng, (B, Hq, C, D)), w.dtype)
    k_src = _encode(_normal(rng, (B, Hkv, C, D)), w.dtype)
    v_src = _encode(_normal(rng, (B, Hkv, C, D)), w.dtype)
    k_cache = _nan_fill((NB, Hkv, BS, D), w.dtype)
    v_cache = _nan_fill((NB, Hkv, BS, D), w.dtype)
    for b in range(B):
        nb = int(nblk[b])
        if nb == 0:
            continue
        ids = bt[b, :nb]
        kb = _encode(_normal(rng, (nb, Hkv, BS, D)), w.dtype)
        vb = _encode(_normal(rng, (nb, Hkv, BS, D)), w.dtype)
        # Positions >= start_pos[b] are not cached yet.
        flat_k = kb.transpose(0, 2, 1, 3).reshape(nb * BS, Hkv, D)
        flat_v = vb.transpose(0, 2, 1, 3).reshape(nb * BS, Hkv, D)
        flat_k[int(s0[b]):] = _nan_fill((), w.dtype)
        flat_v[int(s0[b]):] = _nan_fill((), w.dtype)
        k_cache[ids] = flat_k.reshape(nb, BS, Hkv, D).transpose(0, 2, 1, 3)
        v_cache[ids] = flat_v.reshape(nb, BS, Hkv, D).transpose(0, 2, 1, 3)
    sinks = _encode(_normal(rng, (Hq,)), w.dtype) if w.sinks else None
    return PrefillCase(workload=w, q=q, k_src=k_src, v_src=v_src, k_cache=k_cache, v_cache=v_cache,
                       block_tables=bt, start_pos=s0.astype(np.int32), chunk_lens=n.astype(np.int32), sinks=sinks)


PREFILL_ORDER: List[str] = list(PREFILL_WORKLOADS)
