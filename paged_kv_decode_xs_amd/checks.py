"""Host checks of the preconditions that live in device memory.

The library checks every argument it can before a launch, but lengths, start positions and block
ids live in device memory: reading them would need a synchronisation, so a violation gives
undefined results (never an out-of-bounds access) instead of an error. These helpers copy the
tables to the host (they synchronise) and return one message per violation found, at most
`limit`; an empty list means none. They are for tests, debugging and callers that can afford the
copy, not for the step itself.
"""

from __future__ import annotations

from typing import List

import torch


def _host(t: torch.Tensor):
    return t.detach().to("cpu").numpy()


def check_device_inputs(block_tables: torch.Tensor, context_lens: torch.Tensor, num_blocks: int, block_size: int,
                        partition_size: int = 0, max_partitions: int = 0, limit: int = 20) -> List[str]:
    """A decode step's preconditions (xs_kv_append, xs_paged_attn_decode*, xs_paged_attn_reduce*):
    - 0 <= L_b <= max_blocks_per_seq * block_size;
    - the ids of the blocks holding positions 0 .. L_b - 1 lie in [0, num_blocks);
    - the slot that receives position L_b - 1 (the append's target) is neither inside another
      sequence's context (that sequence would read it while it is written) nor another
      sequence's target;
    - with split-K (partition_size > 0), ceil(L_b / partition_size) <= max_partitions. A longer
      sequence gets NaN rows."""
    bt = _host(block_tables)
    lens = _host(context_lens)
    if bt.ndim != 2 or lens.ndim != 1 or bt.shape[0] != lens.shape[0]:
        raise ValueError("block_tables must be [batch, max_blocks_per_seq] and context_lens [batch]")
    mbps = bt.shape[1]
    problems: List[str] = []

    def note(msg: str) -> None:
        if len(problems) < limit:
            problems.append(msg)

    users = {}  # block -> [(sequence, logical index)] over every block a context covers
    targets = {}  # sequence -> (block, slot) of its position L_b - 1
    for b, L in enumerate(int(x) for x in lens):
        if L < 0 or L > mbps * block_size:
            note(f"context_lens[{b}] = {L} is outside [0, {mbps * block_size}]")
            continue
        for j in range(-(-L // block_size)):
            blk = int(bt[b, j])
            if blk < 0 or blk >= num_blocks:
                note(f"block_tables[{b}, {j}] = {blk} is outside [0, {num_blocks})")
                continue
            users.setdefault(blk, []).append((b, j))
        if L >= 1:
            targets[b] = (int(bt[b, (L - 1) // block_size]), (L - 1) % block_size)
        if partition_size > 0 and -(-L // partition_size) > max_partitions:
            note(f"sequence {b}: {L} tokens need {-(-L // partition_size)} partitions of {partition_size}, "
                 f"max_partitions is {max_partitions}")
    seen = {}
    for b, (blk, slot) in targets.items():
        if (blk, slot) in seen:
            note(f"sequences {seen[(blk, slot)]} and {b} both append into block {blk}, slot {slot}")
        seen.setdefault((blk, slot), b)
        for c, j in users.get(blk, []):
            if c != b and j * block_size + slot < int(lens[c]):
                note(f"block {blk}, slot {slot} receives sequence {b}'s new token inside sequence {c}'s context")
    return problems


def check_prefill_inputs(block_tables: torch.Tensor, start_pos: torch.Tensor, chunk_lens: torch.Tensor,
                         chunk_size: int, num_blocks: int, block_size: int, limit: int = 20) -> List[str]:
    """A chunked prefill's preconditions (xs_kv_append_chunk, xs_paged_attn_prefill*):
    - 0 <= start_pos[b], 0 <= chunk_lens[b] <= chunk_size and start_pos[b] + chunk_lens[b] <=
      max_blocks_per_seq * block_size (a sequence outside them is skipped: nothing is appended and
      its rows are zeros);
    - the ids of the blocks holding positions 0 .. start_pos[b] + chunk_lens[b] - 1 lie in
      [0, num_blocks);
    - no two appended positions map the same slot, and no appended slot lies inside another
      sequence's context (positions 0 .. start_pos + chunk_lens - 1 of that sequence)."""
    bt = _host(block_tables)
    sp = _host(start_pos)
    cl = _host(chunk_lens)
    if bt.ndim != 2 or sp.shape != (bt.shape[0],) or cl.shape != (bt.shape[0],):
        raise ValueError("block_tables must be [batch, max_blocks_per_seq], start_pos and chunk_lens [batch]")
    mbps = bt.shape[1]
    problems: List[str] = []

    def note(msg: str) -> None:
        if len(problems) < limit:
            problems.append(msg)

    ends = {}
    users = {}  # block -> [(sequence, logical index)]
    writes = {}  # (block, slot) -> first (sequence, position) appending there
    for b in range(bt.shape[0]):
        s, n = int(sp[b]), int(cl[b])
        if s < 0 or n < 0 or n > chunk_size or s + n > mbps * block_size:
            note(f"sequence {b}: start_pos {s}, chunk_lens {n} break 0 <= start_pos, 0 <= chunk_lens <= "
                 f"{chunk_size}, start_pos + chunk_lens <= {mbps * block_size} (the sequence is skipped)")
            continue
        ends[b] = s + n
        for j in range(-(-(s + n) // block_size)):
            blk = int(bt[b, j])
            if blk < 0 or blk >= num_blocks:
                note(f"block_tables[{b}, {j}] = {blk} is outside [0, {num_blocks})")
                continue
            users.setdefault(blk, []).append((b, j))
        for p in range(s, s + n):
            blk = int(bt[b, p // block_size])
            if blk < 0 or blk >= num_blocks:
                continue
            key = (blk, p % block_size)
            if key in writes:
                c, q = writes[key]
                note(f"positions {q} of sequence {c} and {p} of sequence {b} both append into block {blk}, "
                     f"slot {key[1]}")
            else:
                writes[key] = (b, p)
    for (blk, slot), (b, p) in writes.items():
        for c, j in users.get(blk, []):
            if c != b and j * block_size + slot < ends[c]:
                note(f"block {blk}, slot {slot} receives position {p} of sequence {b} inside sequence {c}'s context")
    return problems
