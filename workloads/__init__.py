"""Seeded synthetic inputs for paged-KV decode attention.

This module only draws and lays out random inputs. It holds none of the
attention arithmetic: no dot products, no softmax, no append. Both sides of
every parity check take their inputs from here: the HIP path (through the
tests and the bench) and the fp64 oracle.

Workload shapes follow the xserv pages:

* GPT-2 124M: 12 heads, head_dim 64 (xserv compare phase5...phase8,
  docs and `ModelConfig`, where head_dim = hidden / heads).
* Qwen3-8B: 32 query heads, 8 KV heads, head_dim 128, Qwen3 `q_norm`/`k_norm`
  weights of shape [head_dim] (xserv compare phase8...phase13, Qwen3 model
  and the phase-10 benchmark doc).

The paged pool has logical shape [num_blocks, num_kv_heads, block_size,
head_dim] and the block table is int32 [batch, max_blocks_per_seq]
(xserv compare phase10...cf1e9e41, crates/xserv-kernels/src/attention.rs,
doc comments of `reshape_and_cache_bf16` and `paged_decode_attention`).

Recipe (the same for every workload):

1. ``rng = numpy.random.default_rng(seed)`` (PCG64).
2. Context lengths: fixed, or integers uniform on [lo, hi] inclusive.
3. Pool size: given, or ceil(1.25 * sum_b ceil(L_b / BS)).
4. Placement: one permutation of [0, NB). Its first sum_b ceil(L_b / BS)
   entries are the sequences' blocks, taken in batch order. Table padding is -1.
5. Values, drawn in this order: config-3 gains (if any), q, k_new, v_new,
   then each sequence's K blocks and V blocks in batch order. Normal draws
   are float32 (numpy's ``standard_normal(dtype=float32)``). For bf16 they
   are rounded to bf16, nearest-even, on the float32 bit pattern.
   The "rmsnorm_gain" rows: z ~ N(0,1) per row of D in fp64, x = z / rms(z),
   times a gain vector of shape [D] drawn from N(1, 0.1) once per tensor kind
   (one for q, one for k). V stays N(0, 1).
6. Sinks (workloads that have them): one N(0, 1) value per query head, drawn after
   everything else, then rounded like the other values.
7. Poison: every pool slot that no sequence owns is NaN. That is all unused
   blocks, the tail slots t >= L_b of each last block, and the slot L_b - 1
   itself, which the decode step's append must fill.

bf16 tensors travel as uint16 bit patterns, float32 ones as float32.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
F32_NAN_BITS = np.uint32(0x7FC00000)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic decode-step workload."""

    name: str
    description: str
    dtype: str  # "f32" or "bf16"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    ctx: tuple  # ("fixed", [L_0, ...]) or ("uniform", lo, hi)
    num_blocks: Optional[int]  # None: ceil(1.25 * blocks needed)
    max_blocks_per_seq: int
    values: str  # "normal" or "rmsnorm_gain"
    seed: int
    partition_size: int  # tokens per split-K partition used by the bench and tests
    window: int = 0  # > 0: the query attends to the last `window` positions only
    sinks: bool = False  # one attention-sink logit per query head (drawn last, N(0, 1) -> dtype)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(
            name="gpt2_fp32_ctx32",
            description="GPT-2-124M shape, fp32: 1 sequence, 12 heads MHA, head_dim 64, "
            "context 32, block_size 16, 2 blocks at random slots of a 64-block pool",
            dtype="f32", batch=1, num_q_heads=12, num_kv_heads=12, head_dim=64, block_size=16,
            ctx=("fixed", [32]), num_blocks=64, max_blocks_per_seq=2, values="normal", seed=0,
            partition_size=16,
        ),
        Workload(
            name="gpt2_bf16_b8",
            description="GPT-2-124M shape, bf16: batch 8, 12 heads MHA, head_dim 64, "
            "context_lens uniform in [64,1024], block_size 16, 1024-block pool",
            dtype="bf16", batch=8, num_q_heads=12, num_kv_heads=12, head_dim=64, block_size=16,
            ctx=("uniform", 64, 1024), num_blocks=1024, max_blocks_per_seq=64, values="normal",
            seed=1, partition_size=128,
        ),
        Workload(
            name="qwen3_8b_b1_ctx4096",
            description="Qwen3-8B shape, bf16 single-stream decode: batch 1, 32 q / 8 KV heads, "
            "head_dim 128, context 4096, block_size 16, scattered blocks, RMS-normalised q/k",
            dtype="bf16", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
            ctx=("fixed", [4096]), num_blocks=None, max_blocks_per_seq=256, values="rmsnorm_gain",
            seed=2, partition_size=64,
        ),
        Workload(
            name="qwen3_8b_b64",
            description="Qwen3-8B shape, bf16 continuous batch: 64 sequences, 32 q / 8 KV heads, "
            "head_dim 128, context_lens uniform in [128,8192], block_size 16, pool 1.25x need",
            dtype="bf16", batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
            ctx=("uniform", 128, 8192), num_blocks=None, max_blocks_per_seq=512, values="normal",
            seed=3, partition_size=1024,
        ),
        Workload(
            name="qwen3_8b_b4_long",
            description="Qwen3-8B shape, bf16 long context with split-K: batch 4, 32 q / 8 KV heads, "
            "head_dim 128, context_lens {8192,16384,24576,32768}, 512-token partitions",
            dtype="bf16", batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
            ctx=("fixed", [8192, 16384, 24576, 32768]), num_blocks=None, max_blocks_per_seq=2048,
            values="normal", seed=4, partition_size=512,
        ),
        Workload(
            name="qwen3_8b_b64_tp8_share",
            description="one GPU's share of the 64-sequence Qwen3-8B batch at tensor parallelism 8: "
            "4 q / 1 KV head, head_dim 128, the same context_lens (uniform in [128,8192], seed 3)",
            dtype="bf16", batch=64, num_q_heads=4, num_kv_heads=1, head_dim=128, block_size=16,
            ctx=("uniform", 128, 8192), num_blocks=None, max_blocks_per_seq=512, values="normal",
            seed=3, partition_size=256,
        ),
        Workload(
            name="gptoss_20b_window128_b64",
            description="gpt-oss-20b sliding-window layer shape, bf16: 64 sequences, 64 q / 8 KV heads, "
            "head_dim 64, 128-token window, one sink per head, context_lens uniform in [128,8192]",
            dtype="bf16", batch=64, num_q_heads=64, num_kv_heads=8, head_dim=64, block_size=16,
            ctx=("uniform", 128, 8192), num_blocks=None, max_blocks_per_seq=512, values="normal",
            seed=5, partition_size=0, window=128, sinks=True,
        ),
    ]
}

ORDER: List[str] = list(WORKLOADS)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return the uint16 bits.

    Inputs are finite here; NaN payloads are not handled.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _context_lens(w: Workload, rng: np.random.Generator) -> np.ndarray:
    kind = w.ctx[0]
    if kind == "fixed":
        lens = np.asarray(w.ctx[1], dtype=np.int64)
        if lens.size != w.batch:
            raise ValueError(f"{w.name}: {lens.size} fixed lengths for batch {w.batch}")
    elif kind == "uniform":
        lo, hi = w.ctx[1], w.ctx[2]
        lens = rng.integers(lo, hi + 1, size=w.batch)
    else:
        raise ValueError(kind)
    return lens.astype(np.int32)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _rms_rows(rng: np.random.Generator, shape, gain: np.ndarray) -> np.ndarray:
    z = rng.standard_normal(size=shape)  # fp64
    x = z / np.sqrt(np.mean(z * z, axis=-1, keepdims=True))
    return (x * gain).astype(np.float32)


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def _nan_fill(shape, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return np.full(shape, BF16_NAN, dtype=np.uint16)
    return np.full(shape, F32_NAN_BITS, dtype=np.uint32).view(np.float32)


@dataclasses.dataclass
class Case:
    """Inputs of one decode step, as host arrays."""

    workload: Workload
    q: np.ndarray  # [B, Hq, D]
    k_new: np.ndarray  # [B, Hkv, D]
    v_new: np.ndarray  # [B, Hkv, D]
    k_cache: np.ndarray  # [NB, Hkv, BS, D], before this step's append
    v_cache: np.ndarray
    block_tables: np.ndarray  # int32 [B, MBPS], -1 padded
    context_lens: np.ndarray  # int32 [B], length after this step's append
    sinks: Optional[np.ndarray] = None  # [Hq] sink logits (dtype bits), or None

    @property
    def num_blocks(self) -> int:
        return self.k_cache.shape[0]

    @property
    def scale(self) -> float:
        return self.workload.scale

    def attended_tokens(self) -> int:
        """sum_b of the positions the query sees: L_b, or min(L_b, window) with a window."""
        L = np.maximum(self.context_lens.astype(np.int64), 0)
        w = self.workload.window
        return int((np.minimum(L, w) if w > 0 else L).sum())

    def kv_bytes(self) -> int:
        """K+V bytes attention must stream: sum_b L_b * Hkv * D * elt * 2 (window-limited)."""
        w = self.workload
        return self.attended_tokens() * w.num_kv_heads * w.head_dim * w.elt_bytes * 2


@dataclasses.dataclass
class Layout:
    """Lengths, pool size and block placement of a workload (no values)."""

    context_lens: np.ndarray  # int32 [B]
    num_blocks: int
    block_tables: np.ndarray  # int32 [B, MBPS], -1 padded
    blocks_per_seq: np.ndarray  # int64 [B]


def make_layout(w: Workload, rng: np.random.Generator, lens: Optional[np.ndarray] = None) -> Layout:
    """Steps 2-4 of the recipe. Consumes the rng in the same order as ``make_case``."""
    if lens is None:
        lens = _context_lens(w, rng)
    else:
        lens = np.asarray(lens, dtype=np.int32)
        if lens.shape != (w.batch,):
            raise ValueError("lens must have shape [batch]")
    BS = w.block_size
    if int(lens.max(initial=0)) > w.max_blocks_per_seq * BS:
        raise ValueError("a context length exceeds max_blocks_per_seq * block_size")
    nblk = (lens.astype(np.int64) + BS - 1) // BS
    need = int(nblk.sum())
    NB = w.num_blocks if w.num_blocks is not None else max(1, math.ceil(1.25 * need))
    if need > NB:
        raise ValueError(f"{w.name}: {need} blocks needed, pool has {NB}")
    perm = rng.permutation(NB).astype(np.int32)
    bt = np.full((w.batch, w.max_blocks_per_seq), -1, dtype=np.int32)
    start = 0
    for b in range(w.batch):
        bt[b, : nblk[b]] = perm[start : start + nblk[b]]
        start += nblk[b]
    return Layout(context_lens=lens, num_blocks=NB, block_tables=bt, blocks_per_seq=nblk)


def make_case(w: Workload, seed: Optional[int] = None, lens: Optional[np.ndarray] = None) -> Case:
    """Draw the inputs of workload ``w`` (seed defaults to the workload's own)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    lay = make_layout(w, rng, lens)
    lens, NB, bt, nblk = lay.context_lens, lay.num_blocks, lay.block_tables, lay.blocks_per_seq
    B, Hq, Hkv, D, BS = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size

    if w.values == "rmsnorm_gain":
        gain_q = 1.0 + 0.1 * rng.standard_normal(D)
        gain_k = 1.0 + 0.1 * rng.standard_normal(D)
        q = _rms_rows(rng, (B, Hq, D), gain_q)
        k_new = _rms_rows(rng, (B, Hkv, D), gain_k)
        v_new = _normal(rng, (B, Hkv, D))
    elif w.values == "normal":
        gain_k = None
        q = _normal(rng, (B, Hq, D))
        k_new = _normal(rng, (B, Hkv, D))
        v_new = _normal(rng, (B, Hkv, D))
    else:
        raise ValueError(w.values)

    k_cache = _nan_fill((NB, Hkv, BS, D), w.dtype)
    v_cache = _nan_fill((NB, Hkv, BS, D), w.dtype)
    for b in range(B):
        n = int(nblk[b])
        if n == 0:
            continue
        ids = bt[b, :n]
        if gain_k is not None:
            kb = _rms_rows(rng, (n, Hkv, BS, D), gain_k)
        else:
            kb = _normal(rng, (n, Hkv, BS, D))
        vb = _normal(rng, (n, Hkv, BS, D))
        kb = _encode(kb, w.dtype)
        vb = _encode(vb, w.dtype)
        # Slots from L_b - 1 on in the last block: the new token's slot and the tail.
        first_unowned = (int(lens[b]) - 1) - (n - 1) * BS
        kb[n - 1, :, first_unowned:, :] = _nan_fill((), w.dtype)
        vb[n - 1, :, first_unowned:, :] = _nan_fill((), w.dtype)
        k_cache[ids] = kb
        v_cache[ids] = vb

    sinks = _encode(_normal(rng, (Hq,)), w.dtype) if w.sinks else None
    return Case(
        workload=w,
        sinks=sinks,
        q=_encode(q, w.dtype),
        k_new=_encode(k_new, w.dtype),
        v_new=_encode(v_new, w.dtype),
        k_cache=k_cache,
        v_cache=v_cache,
        block_tables=bt,
        context_lens=lens,
    )


def small(name: str, **kw) -> Workload:
    """A named workload with some fields replaced (for reduced-size test cases)."""
    return WORKLOADS[name].with_(**kw)
