"""Chunked prefill (xs_kv_append_chunk + xs_paged_attn_prefill) against the prefill oracle (needs an
MI355X).

The append must reproduce the oracle's pools bit for bit (only the chunk's slots change, the NaN
poison elsewhere stays). The attention output is compared element by element with the fp64
oracle at the bf16 bar (2e-2 absolute + 2e-2 relative); rows past chunk_lens[b] must be exactly
zero. Shapes span several 128-row workgroups and 32-token key tiles with ragged tails, GQA groups
that do and do not divide 16 (1, 3, 4, 6, 8, 12), head_dim 64/128, block_size 8/16/32, chunks
that start at 0 or deep into a cached prefix, empty chunks and sequences outside the valid range.
The Qwen3-8B 512-token chunk workload (the timed one) is checked in full for the append and on
sampled rows for the attention: a run of rows [a, a+k) of the chunk is what the oracle gives for
a chunk that starts at start_pos + a (the chunking invariance pinned on the CPU).
A block id outside [0, num_blocks) in the cached prefix is skipped (checked against the decode
oracle over the table without it). The prefill kernel's rows also agree with the decode kernel's
output for the same queries on the
same pools (twice the bf16 bar: each is within it of the oracle). The split-K entry point
(xs_paged_attn_prefill_split) is held to the same bar with partition
sizes of 64 and 128 keys, so the small shapes already split into several pieces and rows see
pieces with and without keys of their own. Two shapes cover the workgroup orders in full: 448
workgroups of mixed sizes (taken largest first, unsplit and split, with an empty and an invalid
sequence), and 264 row blocks per kv head (the fixed order).
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_xs_amd as xs
from tests.gpu_common import TOL, as_f64, assert_close, log
from tests.rounding_bound import assert_rounding_bound, prefill_spread
from workloads.device import to_numpy_bits, to_torch
from workloads.prefill import PREFILL_WORKLOADS, PrefillWorkload, make_prefill_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _library():
    xs.load_library()
    torch.cuda.init()
    yield


def _to_dev(case):
    dt = case.workload.dtype
    return {
        "q": to_torch(case.q, dt).cuda(),
        "k_src": to_torch(case.k_src, dt).cuda(),
        "v_src": to_torch(case.v_src, dt).cuda(),
        "k_cache": to_torch(case.k_cache, dt).cuda(),
        "v_cache": to_torch(case.v_cache, dt).cuda(),
        "bt": torch.from_numpy(case.block_tables).cuda(),
        "sp": torch.from_numpy(case.start_pos).cuda(),
        "cl": torch.from_numpy(case.chunk_lens).cuda(),
    }


def _attend(dev, scale, split=None):
    # Output and partials start as NaN: whatever the kernels leave unwritten shows in the result.
    out = torch.full_like(dev["q"], float("nan"))
    if split:
        B, Hq, C, D = dev["q"].shape
        NP = xs.num_partitions(dev["bt"].shape[1] * dev["k_cache"].shape[2], split)
        po = torch.full((B, Hq, C, NP, D), float("nan"), dtype=torch.float32, device="cuda")
        pml = torch.full((B, Hq, C, NP, 2), float("nan"), dtype=torch.float32, device="cuda")
        return xs.xs_paged_attn_prefill_split(dev["q"], dev["k_cache"], dev["v_cache"], dev["bt"], dev["sp"], dev["cl"],
                                              scale, split, out=out, part_o=po, part_ml=pml)
    return xs.xs_paged_attn_prefill(dev["q"], dev["k_cache"], dev["v_cache"], dev["bt"], dev["sp"], dev["cl"], scale,
                                    out=out)


def _run(dev, scale, split=None):
    xs.xs_kv_append_chunk(dev["k_src"], dev["v_src"], dev["k_cache"], dev["v_cache"], dev["bt"], dev["sp"], dev["cl"])
    out = _attend(dev, scale, split)
    torch.cuda.synchronize()
    return out


def _check_pools(dev, kp, vp):
    for name, exp in (("k_cache", kp), ("v_cache", vp)):
        got = to_numpy_bits(dev[name])
        assert np.array_equal(got.view(np.uint8), exp.view(np.uint8)), f"{name} differs after the chunk append"


def _full_check(w, label, split=None):
    log(f"[gpu] prefill {label}: Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim} BS={w.block_size} "
        f"C={w.chunk} start={w.start_pos} n={w.chunk_lens} split={split}")
    case = make_prefill_case(w)
    kp, vp = oracle.kv_append_chunk(case.k_cache, case.v_cache, case.k_src, case.v_src, case.block_tables,
                                    case.start_pos, case.chunk_lens, w.block_size)
    exp = oracle.paged_prefill_attention(case.q, kp, vp, case.block_tables, case.start_pos, case.chunk_lens, w.scale,
                                         w.block_size, "bf16")
    dev = _to_dev(case)
    assert xs.check_prefill_inputs(dev["bt"], dev["sp"], dev["cl"], w.chunk, case.k_cache.shape[0], w.block_size) == []
    out = _run(dev, w.scale, split)
    _check_pools(dev, kp, vp)
    got = as_f64(out)
    atol, rtol = TOL["bf16"]
    err = assert_close(got, exp, atol, rtol, f"prefill {label} split={split}")
    tau = prefill_spread(case.q, kp, vp, case.block_tables, case.start_pos, case.chunk_lens, w.scale, w.block_size,
                         "bf16")
    assert_rounding_bound(got, exp, tau, f"prefill {label} split={split}, rounding bound")
    for b, n in enumerate(case.chunk_lens.tolist()):
        assert not got[b, :, n:].any(), f"rows past chunk_lens[{b}] = {n} are not zero"
    # Deterministic: a second run on the same inputs gives the same bits.
    out2 = _attend(dev, w.scale, split)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    return err


SHAPES = [
    # Hq, Hkv, D, BS, C, start_pos, chunk_lens
    (8, 2, 64, 16, 24, (0, 37, 5), (24, 11, 1)),
    (6, 2, 128, 8, 21, (3, 64), (21, 20)),
    (12, 1, 64, 32, 9, (40, 0), (9, 0)),
    (2, 2, 64, 16, 40, (0, 60), (40, 33)),
    (32, 8, 128, 16, 70, (0, 130, 257), (70, 64, 3)),
    (64, 8, 64, 16, 33, (100, 0), (33, 17)),
    (12, 2, 128, 32, 50, (31, 200, 0, 77), (50, 49, 50, 1)),
    (16, 16, 128, 16, 130, (0,), (130,)),
]


def _shape_workload(shape):
    Hq, Hkv, D, BS, C, sp, cl = shape
    mbps = -(-max(s + n for s, n in zip(sp, cl)) // BS) + 2
    return PrefillWorkload(name="t", description="", dtype="bf16", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                           block_size=BS, chunk=C, start_pos=sp, chunk_lens=cl, max_blocks_per_seq=mbps,
                           seed=hash(shape) % 1000)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"Hq{s[0]}_Hkv{s[1]}_D{s[2]}_BS{s[3]}_C{s[4]}")
def test_prefill_matches_oracle(shape):
    Hq, Hkv, D, BS, C = shape[:5]
    _full_check(_shape_workload(shape), f"Hq{Hq} Hkv{Hkv} D{D} BS{BS} C{C}")


@pytest.mark.parametrize("split", [64, 128])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"Hq{s[0]}_Hkv{s[1]}_D{s[2]}_BS{s[3]}_C{s[4]}")
def test_prefill_split_matches_oracle(shape, split):
    Hq, Hkv, D, BS, C = shape[:5]
    _full_check(_shape_workload(shape), f"Hq{Hq} Hkv{Hkv} D{D} BS{BS} C{C}", split)


# Dispatch orders: many row blocks of mixed sizes in a grid larger than one workgroup per CU
# (the unsplit row blocks and the split-K pieces are taken largest first, a sequence without rows
# and an invalid one still get their zero rows), and more than 256 row blocks per kv head (the
# fixed order).
ORDER_SHAPES = {
    "ranked": (64, 16, 64, 16, 200, (0, 300, 50, 700, 0, 10, -5), (200, 64, 0, 200, 33, 200, 10)),
    "fixed": (8, 1, 128, 16, 2100, (0, 37, 900, 5), (2100, 1500, 2100, 7)),
}


@pytest.mark.parametrize("split", [None, 64, 256])
@pytest.mark.parametrize("order", sorted(ORDER_SHAPES))
def test_prefill_dispatch_orders(order, split):
    Hq, Hkv, D, BS, C, sp, cl = ORDER_SHAPES[order]
    mbps = -(-max(max(s, 0) + n for s, n in zip(sp, cl)) // BS) + 2
    w = PrefillWorkload(name="t", description="", dtype="bf16", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                        block_size=BS, chunk=C, start_pos=tuple(max(s, 0) for s in sp), chunk_lens=cl,
                        max_blocks_per_seq=mbps, seed=31 if order == "ranked" else 32)
    row_blocks = -(-C * (Hq // Hkv) // 256)
    assert (len(sp) * row_blocks <= 256) == (order == "ranked")
    log(f"[gpu] prefill dispatch order {order}: {len(sp)} seqs x {row_blocks} row blocks x {Hkv} kv heads, split={split}")
    case = make_prefill_case(w)
    kp, vp = oracle.kv_append_chunk(case.k_cache, case.v_cache, case.k_src, case.v_src, case.block_tables,
                                    case.start_pos, case.chunk_lens, w.block_size)
    exp = oracle.paged_prefill_attention(case.q, kp, vp, case.block_tables, case.start_pos, case.chunk_lens, w.scale,
                                         w.block_size, "bf16")
    dev = _to_dev(case)
    # The last sequence of "ranked" gets an invalid start: its rows must come out zero.
    bad = [b for b, s in enumerate(sp) if s < 0]
    for b in bad:
        dev["sp"][b] = -5
        exp[b] = 0.0
    problems = xs.check_prefill_inputs(dev["bt"], dev["sp"], dev["cl"], C, case.k_cache.shape[0], BS)
    assert [p.split(":")[0] for p in problems] == [f"sequence {b}" for b in bad], problems
    out = _run(dev, w.scale, split)
    got = as_f64(out)
    assert_close(got, exp, *TOL["bf16"], f"prefill order {order} split={split}")
    for b, n in enumerate(cl):
        assert not got[b, :, (0 if b in bad else n):].any(), f"rows past chunk_lens[{b}] are not zero"


@pytest.mark.parametrize("split", [None, 64])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.5])
def test_prefill_scale_sign_and_zero(scale, split):
    # A negative scale (q negated inside the kernel), scale 0 (uniform weights over the visible
    # keys) and a large one (sharp softmax, many rescales).
    w = PrefillWorkload(name="t", description="", dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128,
                        block_size=16, chunk=40, start_pos=(0, 70), chunk_lens=(40, 29), max_blocks_per_seq=8,
                        seed=21)
    log(f"[gpu] prefill scale={scale} split={split}")
    case = make_prefill_case(w)
    kp, vp = oracle.kv_append_chunk(case.k_cache, case.v_cache, case.k_src, case.v_src, case.block_tables,
                                    case.start_pos, case.chunk_lens, w.block_size)
    exp = oracle.paged_prefill_attention(case.q, kp, vp, case.block_tables, case.start_pos, case.chunk_lens, scale,
                                         w.block_size, "bf16")
    dev = _to_dev(case)
    out = _run(dev, scale, split)
    assert_close(as_f64(out), exp, *TOL["bf16"], f"prefill scale={scale} split={split}")


@pytest.mark.parametrize("split", [None, 64])
def test_invalid_sequences_get_zero_rows_and_no_append(split):
    w = PrefillWorkload(name="t", description="", dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=64,
                        block_size=16, chunk=20, start_pos=(0, 10, 5, 16), chunk_lens=(20, 20, 7, 12),
                        max_blocks_per_seq=3, seed=11)
    log(f"[gpu] prefill invalid ranges split={split}")
    case = make_prefill_case(w)
    dev = _to_dev(case)
    # Sequence 1: start_pos < 0. Sequence 2: chunk_lens > chunk. Sequence 3: start + n > 48 slots.
    sp = torch.tensor([0, -1, 5, 40], dtype=torch.int32)
    cl = torch.tensor([20, 20, 21, 12], dtype=torch.int32)
    dev["sp"].copy_(sp)
    dev["cl"].copy_(cl)
    out = _run(dev, w.scale, split)
    valid = np.array([True, False, False, False])
    kp, vp = oracle.kv_append_chunk(case.k_cache, case.v_cache, case.k_src[valid], case.v_src[valid],
                                    case.block_tables[valid], case.start_pos[valid], case.chunk_lens[valid],
                                    w.block_size)
    _check_pools(dev, kp, vp)
    exp = oracle.paged_prefill_attention(case.q[:1], kp, vp, case.block_tables[:1], case.start_pos[:1],
                                         case.chunk_lens[:1], w.scale, w.block_size, "bf16")
    got = as_f64(out)
    assert_close(got[:1], exp, *TOL["bf16"], "prefill valid sequence")
    assert not got[1:].any()


def test_append_chunk_f32_bit_exact():
    rng = np.random.default_rng(12)
    NB, Hkv, BS, D, C = 40, 3, 8, 64, 17
    log("[gpu] append chunk f32")
    k = rng.standard_normal((NB, Hkv, BS, D)).astype(np.float32)
    v = rng.standard_normal((NB, Hkv, BS, D)).astype(np.float32)
    ks = rng.standard_normal((3, Hkv, C, D)).astype(np.float32)
    vs = rng.standard_normal((3, Hkv, C, D)).astype(np.float32)
    bt = rng.permutation(NB)[:3 * 8].reshape(3, 8).astype(np.int32)
    sp = np.array([0, 9, 40], np.int32)
    cl = np.array([17, 5, 0], np.int32)
    kc, vc = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    xs.xs_kv_append_chunk(torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda(), kc, vc, torch.from_numpy(bt).cuda(),
                          torch.from_numpy(sp).cuda(), torch.from_numpy(cl).cuda())
    torch.cuda.synchronize()
    ek, ev = oracle.kv_append_chunk(k, v, ks, vs, bt, sp, cl, BS)
    assert np.array_equal(kc.cpu().numpy().view(np.uint32), ek.view(np.uint32))
    assert np.array_equal(vc.cpu().numpy().view(np.uint32), ev.view(np.uint32))


@pytest.mark.parametrize("name,split", [("qwen3_8b_prefill_c512", None), ("qwen3_8b_prefill_c512", 512),
                                        ("qwen3_8b_prefill_c512", 1024), ("qwen3_8b_prefill_c512", 2048),
                                        ("qwen3_8b_prefill_long16k", None), ("qwen3_8b_prefill_long16k", 4096),
                                        ("qwen3_8b_prefill_long16k", 2048), ("qwen3_8b_prefill_long16k", 1024)])
def test_qwen3_prefill_workload_sampled_rows(name, split):
    w = PREFILL_WORKLOADS[name]
    log(f"[gpu] prefill {w.name} (full size, sampled rows) split={split}")
    case = make_prefill_case(w)
    kp, vp = oracle.kv_append_chunk(case.k_cache, case.v_cache, case.k_src, case.v_src, case.block_tables,
                                    case.start_pos, case.chunk_lens, w.block_size)
    dev = _to_dev(case)
    out = _run(dev, w.scale, split)
    _check_pools(dev, kp, vp)
    got = as_f64(out)
    assert np.isfinite(got).all()
    atol, rtol = TOL["bf16"]
    rng = np.random.default_rng(13)
    for b in range(w.batch):
        n = int(case.chunk_lens[b])
        for a in sorted({0, n - 3, *rng.integers(0, n - 3, 2).tolist()}):
            k = 3
            exp = oracle.paged_prefill_attention(case.q[b:b + 1, :, a:a + k], kp, vp, case.block_tables[b:b + 1],
                                                 case.start_pos[b:b + 1] + a, np.array([k], np.int32), w.scale,
                                                 w.block_size, "bf16")
            assert_close(got[b:b + 1, :, a:a + k], exp[:, :, :k], atol, rtol, f"{w.name} b={b} rows {a}..{a + k - 1}")
            tau = prefill_spread(case.q[b:b + 1], kp, vp, case.block_tables[b:b + 1], case.start_pos[b:b + 1],
                                 case.chunk_lens[b:b + 1], w.scale, w.block_size, "bf16", b_rows={0: (a, a + k)})
            assert_rounding_bound(got[b:b + 1, :, a:a + k], exp[:, :, :k], tau[:, :, a:a + k],
                                  f"{w.name} b={b} rows {a}..{a + k - 1}, rounding bound")


@pytest.mark.parametrize("decode_split", [0, 64])
def test_prefill_rows_agree_with_decode(decode_split):
    # Row i of a chunk is a decode query at position start_pos + i: on the same pools, the prefill
    # kernel's row and the decode kernel's output for that query (context length start_pos + i + 1)
    # are the same attention, computed by two different kernels.
    w = PrefillWorkload(name="t", description="", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                        block_size=16, chunk=70, start_pos=(0, 130, 257), chunk_lens=(70, 64, 3),
                        max_blocks_per_seq=24, seed=41)
    log(f"[gpu] prefill rows vs decode (decode partition {decode_split})")
    case = make_prefill_case(w)
    dev = _to_dev(case)
    out = _run(dev, w.scale)
    B, Hq, D = w.batch, w.num_q_heads, w.head_dim
    atol, rtol = TOL["bf16"]
    for i in (0, 1, 2, 31, 63, 69):
        rows = [b for b in range(B) if i < w.chunk_lens[b]]
        q_i = dev["q"][:, :, i, :].contiguous()
        lens = torch.tensor([w.start_pos[b] + min(i, w.chunk_lens[b] - 1) + 1 for b in range(B)], dtype=torch.int32,
                            device="cuda")
        dec = torch.empty((B, Hq, D), dtype=q_i.dtype, device="cuda")
        if decode_split:
            NP = xs.num_partitions(w.max_blocks_per_seq * w.block_size, decode_split)
            po = torch.empty((B, Hq, NP, D), dtype=torch.float32, device="cuda")
            pm = torch.empty((B, Hq, NP), dtype=torch.float32, device="cuda")
            pl = torch.empty((B, Hq, NP), dtype=torch.float32, device="cuda")
            xs.xs_paged_attn_decode(q_i, dev["k_cache"], dev["v_cache"], dev["bt"], lens, w.scale, part_o=po, part_m=pm,
                                    part_l=pl, partition_size=decode_split)
            xs.xs_paged_attn_reduce(po, pm, pl, lens, dec, decode_split)
        else:
            xs.xs_paged_attn_decode(q_i, dev["k_cache"], dev["v_cache"], dev["bt"], lens, w.scale, out=dec)
        torch.cuda.synchronize()
        got = as_f64(out)[rows, :, i]
        ref = as_f64(dec)[rows]
        assert_close(got, ref, 2 * atol, 2 * rtol, f"prefill row {i} vs decode")


@pytest.mark.parametrize("split", [None, 64])
def test_prefill_skips_bad_block_ids(split):
    # A block id outside [0, num_blocks) inside the cached prefix is skipped: with the table
    # [b0, -1, b2, b3, b4] (block_size 16) and the chunk at positions 32..71, row i (position p)
    # sees positions 0..15 and 32..p, which is a decode query over the table [b0, b2, b3, b4]
    # with context length p + 1 - 16 (the decode oracle, pinned on the CPU).
    w = PrefillWorkload(name="t", description="", dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128,
                        block_size=16, chunk=40, start_pos=(32,), chunk_lens=(40,), max_blocks_per_seq=6, seed=43)
    log(f"[gpu] prefill with a bad block id, split={split}")
    case = make_prefill_case(w)
    bt = case.block_tables.copy()
    bad = bt.copy()
    bad[0, 1] = -1
    dev = _to_dev(case)
    dev["bt"].copy_(torch.from_numpy(bad))
    out = _run(dev, w.scale, split)
    got = as_f64(out)
    kp, vp = oracle.kv_append_chunk(case.k_cache, case.v_cache, case.k_src, case.v_src, bt, case.start_pos,
                                    case.chunk_lens, w.block_size)
    remap = np.full_like(bt, -1)
    remap[0, :4] = [bt[0, 0], bt[0, 2], bt[0, 3], bt[0, 4]]
    atol, rtol = TOL["bf16"]
    for i in range(40):
        p = 32 + i
        exp = oracle.paged_decode_attention(case.q[:, :, i, :], kp, vp, remap, np.array([p + 1 - 16], np.int32),
                                            w.scale, w.block_size, "bf16")
        assert_close(got[:, :, i], exp, atol, rtol, f"row {i} (position {p}) with a bad block id, split={split}")
