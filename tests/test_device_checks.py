"""The host checks of the device-resident preconditions, on CPU tensors.

`check_device_inputs` (decode step): lengths in range, block ids in range over each context, the
append's slot outside every other context, enough partitions for split-K.
`check_prefill_inputs` (chunked prefill): start and chunk length in range, block ids in range over
each context, no slot appended twice, no appended slot inside another sequence's context.
Tables of the synthetic workloads pass; each planted violation is named, and violations outside
what the kernels use are not."""

import numpy as np
import torch

import workloads as wl
from paged_kv_decode_xs_amd import check_device_inputs, check_prefill_inputs
from workloads.prefill import PREFILL_WORKLOADS, make_prefill_case


def _tables(lens, bs=16, mbps=8, nb=64, seed=0):
    rng = np.random.default_rng(seed)
    bt = np.full((len(lens), mbps), -1, np.int32)
    perm = rng.permutation(nb)
    k = 0
    for b, L in enumerate(lens):
        n = -(-L // bs)
        bt[b, :n] = perm[k:k + n]
        k += n
    return torch.from_numpy(bt), torch.tensor(lens, dtype=torch.int32)


def test_workload_layouts_pass():
    for name in ("gpt2_fp32_ctx32", "gpt2_bf16_b8", "qwen3_8b_b1_ctx4096"):
        w = wl.WORKLOADS[name]
        lay = wl.make_layout(w, np.random.default_rng(w.seed))
        bt, lens = torch.from_numpy(lay.block_tables), torch.from_numpy(lay.context_lens)
        assert check_device_inputs(bt, lens, lay.num_blocks, w.block_size) == [], name
        P = w.partition_size or 128
        npart = -(-int(lens.max()) // P)
        assert check_device_inputs(bt, lens, lay.num_blocks, w.block_size, P, npart) == [], name
        assert check_device_inputs(bt, lens, lay.num_blocks, w.block_size, P, npart - 1) != [] or npart == 1


def test_length_out_of_range():
    bt, lens = _tables([10, 20])
    lens[1] = 8 * 16 + 1
    assert check_device_inputs(bt, lens, 64, 16) == ["context_lens[1] = 129 is outside [0, 128]"]
    lens[1] = -3
    assert check_device_inputs(bt, lens, 64, 16) == ["context_lens[1] = -3 is outside [0, 128]"]
    lens[1] = 0
    assert check_device_inputs(bt, lens, 64, 16) == []


def test_block_ids_checked_only_inside_the_context():
    bt, lens = _tables([40, 17])
    bt[0, 1] = -1
    bt[1, 1] = 64
    bt[1, 5] = 999  # past sequence 1's two blocks: never used
    got = check_device_inputs(bt, lens, 64, 16)
    assert got == ["block_tables[0, 1] = -1 is outside [0, 64)", "block_tables[1, 1] = 64 is outside [0, 64)"]


def test_append_slot_inside_another_context():
    # Sequences 0 and 1 share their first block (a shared prefix). Sequence 0 has 12 tokens, so its
    # new token goes to slot 11 of the shared block, which sequence 1 (40 tokens) reads.
    bt, lens = _tables([12, 40])
    bt[1, 0] = bt[0, 0]
    got = check_device_inputs(bt, lens, 64, 16)
    assert got == [f"block {int(bt[0, 0])}, slot 11 receives sequence 0's new token inside sequence 1's context"]
    # A shared full prefix block is fine when both sequences append into blocks of their own:
    # 30 and 40 tokens share block 0 and write slots 13 and 7 of their own second and third blocks.
    bt, lens = _tables([30, 40])
    bt[1, 0] = bt[0, 0]
    assert check_device_inputs(bt, lens, 64, 16) == []
    # Sequence 1 appending into the shared block (4 tokens: slot 3) writes inside sequence 0's context.
    lens[1] = 4
    assert check_device_inputs(bt, lens, 64, 16) == [
        f"block {int(bt[0, 0])}, slot 3 receives sequence 1's new token inside sequence 0's context"]


def test_two_sequences_appending_into_one_slot():
    bt, lens = _tables([20, 20])
    bt[1, 1] = bt[0, 1]
    got = check_device_inputs(bt, lens, 64, 16)
    blk = int(bt[0, 1])
    assert f"sequences 0 and 1 both append into block {blk}, slot 3" in got


def test_partitions_and_limit():
    bt, lens = _tables([100, 250, 0, 128], mbps=16, nb=64)
    got = check_device_inputs(bt, lens, 64, 16, partition_size=64, max_partitions=2)
    assert got == ["sequence 1: 250 tokens need 4 partitions of 64, max_partitions is 2"]
    bt[:, :] = 1000
    assert len(check_device_inputs(bt, lens, 64, 16, limit=5)) == 5


def test_prefill_workload_layouts_pass():
    for name, w in PREFILL_WORKLOADS.items():
        case = make_prefill_case(w)
        nb = case.k_cache.shape[0]
        got = check_prefill_inputs(torch.from_numpy(case.block_tables), torch.from_numpy(case.start_pos),
                                   torch.from_numpy(case.chunk_lens), w.chunk, nb, w.block_size)
        assert got == [], (name, got)


def _prefill_tables(starts, lens, bs=16, mbps=8, nb=64, seed=1):
    bt, _ = _tables([s + n for s, n in zip(starts, lens)], bs, mbps, nb, seed)
    return bt, torch.tensor(starts, dtype=torch.int32), torch.tensor(lens, dtype=torch.int32)


def test_prefill_ranges():
    bt, sp, cl = _prefill_tables([0, 20, 5], [10, 30, 0])
    assert check_prefill_inputs(bt, sp, cl, 32, 64, 16) == []
    sp[0] = -1
    cl[1] = 33
    got = check_prefill_inputs(bt, sp, cl, 32, 64, 16)
    assert len(got) == 2 and got[0].startswith("sequence 0: start_pos -1") and got[1].startswith(
        "sequence 1: start_pos 20, chunk_lens 33")
    sp[0], cl[1] = 120, 9  # sequence 0: 120 + 10 > 8 * 16; sequence 1 back in range
    assert check_prefill_inputs(bt, sp, cl, 32, 64, 16) == [
        "sequence 0: start_pos 120, chunk_lens 10 break 0 <= start_pos, 0 <= chunk_lens <= 32, "
        "start_pos + chunk_lens <= 128 (the sequence is skipped)"]


def test_prefill_block_ids_and_slots():
    bt, sp, cl = _prefill_tables([0, 20], [10, 30])
    bt[1, 2] = 64  # block of positions 32..47 of sequence 1
    got = check_prefill_inputs(bt, sp, cl, 32, 64, 16)
    assert got == ["block_tables[1, 2] = 64 is outside [0, 64)"]
    # Sequence 1's table repeats a block: positions 20 and 36 both map slot 4 of one block.
    bt, sp, cl = _prefill_tables([0, 20], [10, 30])
    bt[1, 2] = bt[1, 1]
    got = check_prefill_inputs(bt, sp, cl, 32, 64, 16)
    assert got[0] == f"positions 20 of sequence 1 and 36 of sequence 1 both append into block {int(bt[1, 1])}, slot 4"


def test_prefill_write_inside_another_context():
    # Sequence 1 (chunk at 20..49) shares sequence 0's first block (positions 0..15 of a 10-token
    # context that sequence 0 appends at 0..9): sequence 0 writes slots 0..9 that sequence 1 reads.
    bt, sp, cl = _prefill_tables([0, 20], [10, 30])
    bt[1, 0] = bt[0, 0]
    got = check_prefill_inputs(bt, sp, cl, 32, 64, 16, limit=100)
    assert len(got) == 10 and all("inside sequence 1's context" in g for g in got)
    # A shared, full prefix block that neither sequence appends into is fine.
    bt, sp, cl = _prefill_tables([16, 20], [10, 30])
    bt[1, 0] = bt[0, 0]
    assert check_prefill_inputs(bt, sp, cl, 32, 64, 16) == []
