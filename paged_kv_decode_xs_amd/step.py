"""One decode step: KV append, split-K decode attention, log-sum-exp reduce.

`DecodeStep` owns the step's output and partial buffers (allocated once, through torch) and
chains the library calls on one stream. With partition_size == 0 it issues the unsplit decode
and no reduce. With fused=True the append and the decode are one call
(xs_paged_attn_decode_append); otherwise they are xs_kv_append then xs_paged_attn_decode.
With sinks (bf16 [Hq]) or window > 0 the decode and the reduce are xs_paged_attn_decode_sinks and
xs_paged_attn_reduce_sinks.
`DecodeStep.capture()` records the same step as one HIP graph (xs_step_graph_create); replaying it
runs the step on the buffers as they are at replay time.
`suggest_partition_size` picks a split partition size from a batch's context lengths (host side).
`DecodeStep.check_inputs` checks, on the host, the step's preconditions that live in device memory
(`checks.check_device_inputs`).
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from . import _binding as xb
from .checks import check_device_inputs

# Split items per compute unit that the partition-size rule aims at (at most).
ITEMS_PER_CU = 12.5


def suggest_partition_size(context_lens: Sequence[int], num_kv_heads: int, block_size: int = 16,
                           num_cus: int = 256) -> int:
    """Partition size for the split decode of a batch with these context lengths (host values):
    the smallest power-of-two multiple of block_size, at least 64 tokens, for which the split
    items num_kv_heads * sum_b ceil(L_b / P) number at most ITEMS_PER_CU per compute unit.

    A host-side rule from measurements on one MI355X (256 CUs), Qwen3-8B shape (8 kv heads,
    lengths uniform in [128, 8192]): 64, 128 and 256 sequences ran fastest at P = 1024, 2048 and
    4096, the rule's picks; the one-GPU share at tensor parallelism 8 (1 kv head) gets 128, where
    128 to 256 were within 3%. Enough items keep every CU's wavefronts streaming; more than that
    add partial partitions, merge traffic and per-item start-up."""
    if num_kv_heads < 1 or block_size < 1 or num_cus < 1:
        raise ValueError("num_kv_heads, block_size and num_cus must be positive")
    lens = [max(int(x), 0) for x in context_lens]
    longest = max(lens, default=0)
    P = block_size
    while P < 64:
        P *= 2
    while P < longest and num_kv_heads * sum(-(-x // P) for x in lens) > ITEMS_PER_CU * num_cus:
        P *= 2
    return P


class DecodeStep:
    def __init__(self, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                 context_lens: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, scale: float,
                 partition_size: int = 0, max_context_len: Optional[int] = None, fused: bool = False,
                 sinks: Optional[torch.Tensor] = None, window: int = 0):
        self.q, self.k_cache, self.v_cache = q, k_cache, v_cache
        self.block_tables, self.context_lens = block_tables, context_lens
        self.k_new, self.v_new = k_new, v_new
        self.scale = float(scale)
        self.partition_size = int(partition_size)
        self.fused = bool(fused)
        self.sinks, self.window = sinks, int(window)
        self.sw = sinks is not None or self.window > 0
        B, Hq, D = q.shape
        self.out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
        if self.partition_size > 0:
            BS = k_cache.shape[2]
            if max_context_len is None:
                max_context_len = block_tables.shape[1] * BS
            NP = xb.num_partitions(max_context_len, self.partition_size)
            self.part_o = torch.empty((B, Hq, NP, D), dtype=torch.float32, device=q.device)
            self.part_m = torch.empty((B, Hq, NP), dtype=torch.float32, device=q.device)
            self.part_l = torch.empty((B, Hq, NP), dtype=torch.float32, device=q.device)
        else:
            self.part_o = self.part_m = self.part_l = None

    def append(self, stream=None) -> None:
        xb.xs_kv_append(self.k_new, self.v_new, self.k_cache, self.v_cache, self.block_tables, self.context_lens,
                        stream=stream)

    def _attend_sw(self, fused: bool, stream=None) -> None:
        xb.xs_paged_attn_decode_sinks(self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens,
                                      self.scale, sinks=self.sinks, window_size=self.window,
                                      out=None if self.partition_size > 0 else self.out,
                                      part_o=self.part_o, part_m=self.part_m, part_l=self.part_l,
                                      partition_size=self.partition_size,
                                      k_new=self.k_new if fused else None, v_new=self.v_new if fused else None,
                                      stream=stream)

    def attend(self, stream=None) -> None:
        if self.sw:
            return self._attend_sw(False, stream)
        xb.xs_paged_attn_decode(self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens,
                                self.scale, out=None if self.partition_size > 0 else self.out,
                                part_o=self.part_o, part_m=self.part_m, part_l=self.part_l,
                                partition_size=self.partition_size, stream=stream)

    def reduce(self, stream=None) -> None:
        if self.partition_size > 0 and self.sw:
            xb.xs_paged_attn_reduce_sinks(self.part_o, self.part_m, self.part_l, self.context_lens, self.out,
                                          self.partition_size, sinks=self.sinks, window_size=self.window,
                                          stream=stream)
        elif self.partition_size > 0:
            xb.xs_paged_attn_reduce(self.part_o, self.part_m, self.part_l, self.context_lens, self.out,
                                    self.partition_size, stream=stream)

    def append_and_attend(self, stream=None) -> None:
        if self.sw:
            return self._attend_sw(True, stream)
        xb.xs_paged_attn_decode_append(self.q, self.k_new, self.v_new, self.k_cache, self.v_cache,
                                       self.block_tables, self.context_lens, self.scale,
                                       out=None if self.partition_size > 0 else self.out,
                                       part_o=self.part_o, part_m=self.part_m, part_l=self.part_l,
                                       partition_size=self.partition_size, stream=stream)

    def check_inputs(self, limit: int = 20) -> List[str]:
        """check_device_inputs on this step's tables (synchronises; see there)."""
        NB, _, BS, _ = self.k_cache.shape
        mp = self.part_m.shape[-1] if self.partition_size > 0 else 0
        return check_device_inputs(self.block_tables, self.context_lens, NB, BS, self.partition_size, mp, limit)

    def capture(self) -> "StepGraph":
        """This step as one HIP graph."""
        return StepGraph([self])

    def run(self, stream=None) -> torch.Tensor:
        if self.fused:
            self.append_and_attend(stream)
        else:
            self.append(stream)
            self.attend(stream)
        self.reduce(stream)
        return self.out


def _step_desc(step: "DecodeStep") -> "xb.XsStepDesc":
    """The C descriptor of one step's buffers and sizes."""
    q = step.q
    B, Hq, D = q.shape
    NB, Hkv, BS, _ = step.k_cache.shape
    split = step.partition_size > 0
    return xb.XsStepDesc(
        q=q.data_ptr(), k_new=step.k_new.data_ptr(), v_new=step.v_new.data_ptr(),
        k_cache=step.k_cache.data_ptr(), v_cache=step.v_cache.data_ptr(),
        block_tables=step.block_tables.data_ptr(), context_lens=step.context_lens.data_ptr(),
        sinks=None if step.sinks is None else step.sinks.data_ptr(), window_size=step.window,
        scale=step.scale, out=step.out.data_ptr(),
        part_o=step.part_o.data_ptr() if split else None, part_m=step.part_m.data_ptr() if split else None,
        part_l=step.part_l.data_ptr() if split else None, batch=B, num_q_heads=Hq, num_kv_heads=Hkv,
        head_dim=D, block_size=BS, max_blocks_per_seq=step.block_tables.shape[1], num_blocks=NB,
        partition_size=step.partition_size, max_partitions=step.part_m.shape[-1] if split else 0,
        dtype=xb._dtype_code(q), fused=int(step.fused))


class StepGraph:
    """Decode steps captured in order as one HIP graph, e.g. one per layer (owns the handle;
    close() or garbage collection frees it)."""

    def __init__(self, steps):
        self._steps = list(steps)  # keeps the captured buffers alive
        self._handle = xb.xs_step_graph_create([_step_desc(s) for s in self._steps])

    def launch(self, stream=None) -> torch.Tensor:
        """Replays the steps; returns the last step's output."""
        xb.xs_step_graph_launch(self._handle, stream)
        return self._steps[-1].out

    def close(self) -> None:
        if self._handle:
            xb.xs_step_graph_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass
