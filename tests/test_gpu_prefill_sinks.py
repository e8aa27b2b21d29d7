"""Chunked prefill with attention sinks and a sliding window (xs_paged_attn_prefill_sinks) against
the fp64 oracle (needs an MI355X).

Every output element is compared with ``oracle.paged_prefill_attention_sinks`` at the bf16 bar
(2e-2 absolute + 2e-2 relative); rows past chunk_lens[b] must be exactly zero. The shapes are
those of the plain prefill tests (several row blocks and key tiles with ragged tails, GQA groups
1-12, head_dim 64/128, block_size 8/16/32, chunks that start at 0 or deep into a cached prefix),
each with windows of 1, 7 and 100 positions (a window inside one tile, one that crosses tile and
row-block edges, and one longer than some contexts) and with and without sinks, unsplit and
split-K at 64 keys (so rows see pieces wholly before their window, partly inside it, and inside
it). The gpt-oss-20b layer shapes (64 q / 8 kv heads, head_dim 64, a 128-token window, sinks)
are checked on sampled rows at their full size. Without sinks and window the call must give the
plain prefill's bits, and a window longer than every context must too.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_xs_amd as xs
from tests.gpu_common import TOL, as_f64, assert_close, log
from tests.rounding_bound import assert_rounding_bound, prefill_spread
from tests.test_gpu_prefill import SHAPES, _shape_workload, _to_dev
from workloads import f32_to_bf16_bits
from workloads.device import to_torch
from workloads.prefill import PREFILL_WORKLOADS, PrefillWorkload, make_prefill_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _library():
    xs.load_library()
    torch.cuda.init()
    yield


def _sinks_dev(case):
    return None if case.sinks is None else to_torch(case.sinks, "bf16").cuda()


def _attend(dev, case, window, split=0):
    # Output and partials start as NaN: whatever the kernels leave unwritten shows in the result.
    w = case.workload
    out = torch.full_like(dev["q"], float("nan"))
    po = pml = None
    if split:
        B, Hq, C, D = dev["q"].shape
        NP = xs.num_partitions(dev["bt"].shape[1] * dev["k_cache"].shape[2], split)
        po = torch.full((B, Hq, C, NP, D), float("nan"), dtype=torch.float32, device="cuda")
        pml = torch.full((B, Hq, C, NP, 2), float("nan"), dtype=torch.float32, device="cuda")
    return xs.xs_paged_attn_prefill_sinks(dev["q"], dev["k_cache"], dev["v_cache"], dev["bt"], dev["sp"], dev["cl"],
                                          w.scale, sinks=_sinks_dev(case), window_size=window, partition_size=split,
                                          out=out, part_o=po, part_ml=pml)


def _append(dev):
    xs.xs_kv_append_chunk(dev["k_src"], dev["v_src"], dev["k_cache"], dev["v_cache"], dev["bt"], dev["sp"], dev["cl"])


@pytest.mark.parametrize("sinks", [False, True], ids=["nosink", "sinks"])
@pytest.mark.parametrize("window", [1, 7, 100])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"Hq{s[0]}_Hkv{s[1]}_D{s[2]}_BS{s[3]}_C{s[4]}")
def test_prefill_sinks_matches_oracle(shape, window, sinks):
    w = _shape_workload(shape).with_(window=window, sinks=sinks)
    log(f"[gpu] prefill sinks: shape={shape} window={window} sinks={sinks}")
    case = make_prefill_case(w)
    kp, vp = oracle.kv_append_chunk(case.k_cache, case.v_cache, case.k_src, case.v_src, case.block_tables,
                                    case.start_pos, case.chunk_lens, w.block_size)
    exp = oracle.paged_prefill_attention_sinks(case.q, kp, vp, case.block_tables, case.start_pos, case.chunk_lens,
                                               w.scale, w.block_size, "bf16", sinks=case.sinks, window=window)
    dev = _to_dev(case)
    _append(dev)
    atol, rtol = TOL["bf16"]
    tau = prefill_spread(case.q, kp, vp, case.block_tables, case.start_pos, case.chunk_lens, w.scale, w.block_size,
                         "bf16", sinks=case.sinks, window=window)
    for split in (0, 64):
        out = _attend(dev, case, window, split)
        torch.cuda.synchronize()
        got = as_f64(out)
        assert_close(got, exp, atol, rtol, f"prefill sinks window={window} sinks={sinks} split={split}")
        assert_rounding_bound(got, exp, tau, f"prefill sinks window={window} sinks={sinks} split={split}, bound")
        for b, n in enumerate(case.chunk_lens.tolist()):
            assert not got[b, :, n:].any(), f"rows past chunk_lens[{b}] = {n} are not zero"
        again = _attend(dev, case, window, split)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "not deterministic"


@pytest.mark.parametrize("split", [0, 64, 128])
def test_prefill_sinks_without_window(split):
    """Sinks with full causal attention (the gpt-oss full layers), split and unsplit."""
    w = _shape_workload(SHAPES[4]).with_(sinks=True)
    log(f"[gpu] prefill sinks, no window: split={split}")
    case = make_prefill_case(w)
    kp, vp = oracle.kv_append_chunk(case.k_cache, case.v_cache, case.k_src, case.v_src, case.block_tables,
                                    case.start_pos, case.chunk_lens, w.block_size)
    exp = oracle.paged_prefill_attention_sinks(case.q, kp, vp, case.block_tables, case.start_pos, case.chunk_lens,
                                               w.scale, w.block_size, "bf16", sinks=case.sinks)
    dev = _to_dev(case)
    _append(dev)
    out = _attend(dev, case, 0, split)
    torch.cuda.synchronize()
    assert_close(as_f64(out), exp, *TOL["bf16"], f"prefill sinks split={split}")


def test_prefill_sinks_dominant_sink():
    """Sinks far above the scores: outputs shrink towards zero by e^(s - sigma), still at the bar."""
    w = _shape_workload(SHAPES[0]).with_(window=7, sinks=True)
    log("[gpu] prefill sinks: dominant sinks")
    case = make_prefill_case(w)
    case.sinks = f32_to_bf16_bits(np.full(w.num_q_heads, 9.0, np.float32))
    kp, vp = oracle.kv_append_chunk(case.k_cache, case.v_cache, case.k_src, case.v_src, case.block_tables,
                                    case.start_pos, case.chunk_lens, w.block_size)
    exp = oracle.paged_prefill_attention_sinks(case.q, kp, vp, case.block_tables, case.start_pos, case.chunk_lens,
                                               w.scale, w.block_size, "bf16", sinks=case.sinks, window=7)
    assert np.abs(exp).max() < 0.05  # the sink takes nearly all the weight
    dev = _to_dev(case)
    _append(dev)
    for split in (0, 64):
        out = _attend(dev, case, 7, split)
        torch.cuda.synchronize()
        assert_close(as_f64(out), exp, *TOL["bf16"], f"dominant sinks split={split}")


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[4], SHAPES[6]], ids=["Hq8_D64", "Hq32_D128", "Hq12_BS32"])
def test_prefill_sinks_reduces_to_plain_bits(shape):
    """No sinks and no window: the plain kernel's bits. A window past every context (no sinks):
    the same bits from the windowed kernel (same tiles, same arithmetic)."""
    w = _shape_workload(shape)
    log(f"[gpu] prefill sinks reduces to plain: shape={shape}")
    case = make_prefill_case(w)
    dev = _to_dev(case)
    _append(dev)
    plain = xs.xs_paged_attn_prefill(dev["q"], dev["k_cache"], dev["v_cache"], dev["bt"], dev["sp"], dev["cl"], w.scale)
    big = int(max(s + n for s, n in zip(w.start_pos, w.chunk_lens))) + 1
    for window in (0, big, 1 << 30):
        out = _attend(dev, case, window)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), plain.view(torch.int16)), f"window={window}"


# Full-size gpt-oss layer shapes: sampled rows of the chunk (every head) against the oracle.
SAMPLED = {"gptoss_20b_prefill_window128_c512": (0, 64, 128), "gptoss_20b_prefill_full_c512": (0, 256, 2048)}


@pytest.mark.parametrize("name,split", [(n, s) for n, splits in SAMPLED.items() for s in splits])
def test_prefill_sinks_gptoss_sampled_rows(name, split):
    w = PREFILL_WORKLOADS[name]
    log(f"[gpu] prefill sinks {name} split={split}")
    case = make_prefill_case(w)
    kp, vp = oracle.kv_append_chunk(case.k_cache, case.v_cache, case.k_src, case.v_src, case.block_tables,
                                    case.start_pos, case.chunk_lens, w.block_size)
    dev = _to_dev(case)
    _append(dev)
    out = _attend(dev, case, w.window, split)
    torch.cuda.synchronize()
    got = as_f64(out)
    rng = np.random.default_rng(21)
    atol, rtol = TOL["bf16"]
    for b in range(w.batch):
        n = int(case.chunk_lens[b])
        # Runs of rows [a, a + k): the oracle's chunk that starts at start_pos + a.
        for a in sorted({0, n - 3, int(rng.integers(1, n - 3))}):
            k = 3
            sub_q = np.ascontiguousarray(case.q[b:b + 1, :, a:a + k])
            exp = oracle.paged_prefill_attention_sinks(sub_q, kp, vp, case.block_tables[b:b + 1],
                                                       np.array([int(case.start_pos[b]) + a], np.int32),
                                                       np.array([k], np.int32), w.scale, w.block_size, "bf16",
                                                       sinks=case.sinks, window=w.window)
            assert_close(got[b:b + 1, :, a:a + k], exp, atol, rtol, f"{name} b={b} rows {a}..{a + k} split={split}")


# The merge of split rows runs eight d per lane when its four-wide grid would exceed one round of
# resident workgroups (more than 8 * 256 * 8 rows at head_dim 128, 8 * 256 * 16 at 64). The shapes
# above reach that width only with head_dim 64 and sinks; these two reach it with head_dim 128
# and a window and sinks, and with head_dim 64 and neither. Sampled rows against the oracle.
WIDE_MERGE = [
    # Hq, Hkv, D, window, sinks: 2 x Hq x 512 rows
    (32, 8, 128, 300, True),   # 32 768 rows: 4096 workgroups of 8 rows at four d per lane
    (64, 8, 64, 0, False),     # 65 536 rows: 4096 workgroups of 16 rows
]


@pytest.mark.parametrize("Hq,Hkv,D,window,sinks", WIDE_MERGE)
def test_wide_merge_sampled_rows(Hq, Hkv, D, window, sinks):
    w = PrefillWorkload(name="wide_merge", description="", dtype="bf16", num_q_heads=Hq, num_kv_heads=Hkv,
                        head_dim=D, block_size=16, chunk=512, start_pos=(1800, 700), chunk_lens=(512, 509),
                        max_blocks_per_seq=160, seed=61, window=window, sinks=sinks)
    rows = w.batch * Hq * w.chunk
    assert rows // (256 // (D // 4)) > 8 * 256, "the shape must take the eight-wide merge"
    split = 512
    log(f"[gpu] prefill wide merge Hq={Hq} D={D} window={window} sinks={sinks} split={split}")
    case = make_prefill_case(w)
    kp, vp = oracle.kv_append_chunk(case.k_cache, case.v_cache, case.k_src, case.v_src, case.block_tables,
                                    case.start_pos, case.chunk_lens, w.block_size)
    dev = _to_dev(case)
    _append(dev)
    if window or sinks:
        out = _attend(dev, case, window, split)
    else:
        B, Hq_, C, D_ = dev["q"].shape
        NP = xs.num_partitions(dev["bt"].shape[1] * w.block_size, split)
        out = torch.full_like(dev["q"], float("nan"))
        po = torch.full((B, Hq_, C, NP, D_), float("nan"), dtype=torch.float32, device="cuda")
        pml = torch.full((B, Hq_, C, NP, 2), float("nan"), dtype=torch.float32, device="cuda")
        xs.xs_paged_attn_prefill_split(dev["q"], dev["k_cache"], dev["v_cache"], dev["bt"], dev["sp"], dev["cl"],
                                       w.scale, split, out=out, part_o=po, part_ml=pml)
    torch.cuda.synchronize()
    got = as_f64(out)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(62)
    atol, rtol = TOL["bf16"]
    for b in range(w.batch):
        n = int(case.chunk_lens[b])
        assert not got[b, :, n:].any(), f"rows past chunk_lens[{b}] = {n} are not zero"
        for a in sorted({0, n - 3, *rng.integers(1, n - 3, 2).tolist()}):
            k = 3
            sub_q = np.ascontiguousarray(case.q[b:b + 1, :, a:a + k])
            start = np.array([int(case.start_pos[b]) + a], np.int32)
            if window or sinks:
                exp = oracle.paged_prefill_attention_sinks(sub_q, kp, vp, case.block_tables[b:b + 1], start,
                                                           np.array([k], np.int32), w.scale, w.block_size, "bf16",
                                                           sinks=case.sinks, window=window)
            else:
                exp = oracle.paged_prefill_attention(sub_q, kp, vp, case.block_tables[b:b + 1], start,
                                                     np.array([k], np.int32), w.scale, w.block_size, "bf16")
            assert_close(got[b:b + 1, :, a:a + k], exp, atol, rtol, f"wide merge D={D} b={b} rows {a}..{a + k - 1}")
