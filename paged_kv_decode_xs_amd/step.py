"""One decode step: KV append, split-K decode attention, log-sum-exp reduce.

`DecodeStep` owns the step's output and partial buffers (allocated once, through torch) and
chains the library calls on one stream. With partition_size == 0 it issues the unsplit decode
and no reduce. With fused=True the append and the decode are one call
(xs_paged_attn_decode_append); otherwise they are xs_kv_append then xs_paged_attn_decode.
With schedule="balanced" the step is xs_paged_attn_decode_balanced (append included when fused;
otherwise xs_kv_append first), which writes `out` itself; partition_size is then unused.
With sinks (bf16 [Hq]) or window > 0 the decode and the reduce are xs_paged_attn_decode_sinks and
xs_paged_attn_reduce_sinks (split schedule only).
"""

from __future__ import annotations

from typing import Optional

import torch

from . import _binding as xb


class DecodeStep:
    def __init__(self, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                 context_lens: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, scale: float,
                 partition_size: int = 0, max_context_len: Optional[int] = None, fused: bool = False,
                 schedule: str = "split", sinks: Optional[torch.Tensor] = None, window: int = 0):
        self.q, self.k_cache, self.v_cache = q, k_cache, v_cache
        self.block_tables, self.context_lens = block_tables, context_lens
        self.k_new, self.v_new = k_new, v_new
        self.scale = float(scale)
        self.partition_size = int(partition_size)
        self.fused = bool(fused)
        if schedule not in ("split", "balanced"):
            raise ValueError(f"unknown schedule {schedule!r}")
        self.schedule = schedule
        self.sinks, self.window = sinks, int(window)
        self.sw = sinks is not None or self.window > 0
        if self.sw and schedule != "split":
            raise ValueError("sinks and windows run on the split schedule")
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
        self.workspace = None
        if schedule == "balanced":
            self.partition_size = 0
            self.part_o = self.part_m = self.part_l = None
            nbytes = xb.xs_paged_attn_balanced_workspace_size(B, Hq, k_cache.shape[1], D)
            self.workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)

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

    def balanced(self, stream=None) -> None:
        xb.xs_paged_attn_decode_balanced(self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens,
                                         self.scale, self.out, self.workspace,
                                         k_new=self.k_new if self.fused else None,
                                         v_new=self.v_new if self.fused else None, stream=stream)

    def run(self, stream=None) -> torch.Tensor:
        if self.schedule == "balanced":
            if not self.fused:
                self.append(stream)
            self.balanced(stream)
            return self.out
        if self.fused:
            self.append_and_attend(stream)
        else:
            self.append(stream)
            self.attend(stream)
        self.reduce(stream)
        return self.out
