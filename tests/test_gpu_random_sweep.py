"""Seeded random sweep of the decode step and the chunked prefill against the oracle (needs an
MI355X).

The fixed-shape parity tests pick their shapes by hand. This file draws them: each case number
seeds its own generator, which picks dtype, head_dim, block_size, the GQA group and kv head count,
the batch, a mix of context lengths, the partition size, the fused or separate append, and for
bf16 sometimes a sliding window and sinks. The lengths are drawn to hit the edges: 0, 1, one less
and one more than a block or a 64-token tile, and a partition's end. Each case is held to the
fixed tests' bars:
- the appended pools are bit-exact;
- the output is within the bf16/fp32 tolerance and the rounding bound;
- the split partials match the oracle's partition statistics (no window or sinks);
- prefill rows past a sequence's chunk are exactly zero.
The case number and drawn shape are printed before each GPU call. A failure names its case,
which reproduces from the number alone.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_xs_amd as xs
import workloads as wl
from tests.gpu_common import TOL, OracleResult, as_f64, assert_close, check_partials, log, nan_fill
from tests.rounding_bound import assert_rounding_bound, decode_spread, prefill_spread
from workloads.device import case_to_device, to_numpy_bits, to_torch
from workloads.prefill import PrefillWorkload, make_prefill_case

pytestmark = pytest.mark.gpu

N_DECODE = 96
N_PREFILL = 48


@pytest.fixture(scope="module", autouse=True)
def _library():
    xs.load_library()
    torch.cuda.init()
    yield


def _edge_lengths(rng, n, lmax, bs):
    """n context lengths in [0, lmax]: uniform draws mixed with block, tile and small edges."""
    edges = [0, 1, bs - 1, bs, bs + 1, 63, 64, 65, 2 * bs + 1, lmax - 1, lmax]
    out = []
    for _ in range(n):
        if rng.random() < 0.4:
            out.append(int(rng.choice([e for e in edges if 0 <= e <= lmax])))
        else:
            out.append(int(rng.integers(0, lmax + 1)))
    return out


def _decode_draw(i):
    rng = np.random.default_rng(77_000 + i)
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    D = int(rng.choice([64, 128]))
    BS = int(rng.choice([8, 16, 32]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    while G * Hkv > 64:
        Hkv //= 2
    B = int(rng.integers(1, 40))
    lmax = int(rng.choice([16, 100, 700, 2100]))
    lens = _edge_lengths(rng, B, lmax, BS)
    P = 0 if rng.random() < 0.3 else BS * int(rng.choice([1, 2, 4, 8, 16, 32]))
    fused = bool(rng.random() < 0.5)
    window, sinks = 0, False
    if dtype == "bf16" and BS in (16, 32) and rng.random() < 0.35:
        window = int(rng.choice([0, 1, 7, 16, 100, 1000]))
        sinks = bool(rng.random() < 0.7)
        if window == 0 and not sinks:
            sinks = True
    return dict(dtype=dtype, D=D, BS=BS, Hq=G * Hkv, Hkv=Hkv, lens=lens, P=P, fused=fused, window=window,
                sinks=sinks, seed=77_000 + i)


@pytest.mark.parametrize("i", range(N_DECODE))
def test_decode_random_case(i):
    c = _decode_draw(i)
    log(f"[gpu] random decode case {i}: {c['dtype']} Hq={c['Hq']} Hkv={c['Hkv']} D={c['D']} BS={c['BS']} "
        f"P={c['P']} fused={c['fused']} window={c['window']} sinks={c['sinks']} B={len(c['lens'])} "
        f"lens={c['lens'][:10]}{'...' if len(c['lens']) > 10 else ''}")
    mbps = max(1, -(-max(c["lens"]) // c["BS"]) + 1)
    w = wl.Workload(name=f"random{i}", description="", dtype=c["dtype"], batch=len(c["lens"]), num_q_heads=c["Hq"],
                    num_kv_heads=c["Hkv"], head_dim=c["D"], block_size=c["BS"], ctx=("fixed", c["lens"]),
                    num_blocks=None, max_blocks_per_seq=mbps, values="normal", seed=c["seed"],
                    partition_size=c["BS"], window=c["window"], sinks=c["sinks"])
    case = wl.make_case(w)
    sw = c["window"] > 0 or c["sinks"]
    P = c["P"]
    k_pool, v_pool = oracle.kv_append(case.k_cache, case.v_cache, case.k_new, case.v_new, case.block_tables,
                                      case.context_lens, w.block_size)
    if sw:
        ref = oracle.paged_decode_attention_sinks(case.q, k_pool, v_pool, case.block_tables, case.context_lens,
                                                  w.scale, w.block_size, w.dtype, sinks=case.sinks, window=c["window"])
    else:
        oref = OracleResult(case, P)
        ref = oref.out
    dev = case_to_device(case)
    sinks_t = None if case.sinks is None else to_torch(case.sinks, "bf16").cuda()
    step = xs.DecodeStep(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                         dev["k_new"], dev["v_new"], w.scale, partition_size=P,
                         max_context_len=max(1, max(c["lens"])) if P else None, fused=c["fused"], sinks=sinks_t,
                         window=c["window"])
    nan_fill(step)
    step.run()
    torch.cuda.synchronize()
    for name, exp in (("k_cache", k_pool), ("v_cache", v_pool)):
        assert np.array_equal(to_numpy_bits(dev[name]).view(np.uint8), exp.view(np.uint8)), \
            f"case {i}: {name} after the append"
    got = as_f64(step.out)
    assert_close(got, ref, *TOL[w.dtype], f"random decode case {i}")
    if w.dtype == "bf16":
        tau = decode_spread(case.q, k_pool, v_pool, case.block_tables, case.context_lens, w.scale, w.block_size,
                            "bf16", sinks=case.sinks, window=c["window"])
        assert_rounding_bound(got, ref, tau, f"random decode case {i}, rounding bound")
    if P and not sw:
        check_partials(step, oref, case)


def _prefill_draw(i):
    rng = np.random.default_rng(88_000 + i)
    D = int(rng.choice([64, 128]))
    BS = int(rng.choice([8, 16, 32]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    while G * Hkv > 64:
        Hkv //= 2
    B = int(rng.integers(1, 6))
    C = int(rng.choice([1, 9, 33, 64, 65, 130, 300]))
    chunk_lens = tuple(int(x) for x in _edge_lengths(rng, B, C, BS))
    start_pos = tuple(int(rng.choice([0, 1, BS, 63, 64, int(rng.integers(0, 1500))])) for _ in range(B))
    split = 0 if rng.random() < 0.4 else int(rng.choice([64, 128, 256, 512]))
    window, sinks = 0, False
    if rng.random() < 0.35:
        window = int(rng.choice([0, 1, 7, 64, 100, 1000]))
        sinks = bool(rng.random() < 0.7)
    mbps = -(-max(s + n for s, n in zip(start_pos, chunk_lens)) // BS) + 2
    return PrefillWorkload(name=f"random{i}", description="", dtype="bf16", num_q_heads=G * Hkv, num_kv_heads=Hkv,
                           head_dim=D, block_size=BS, chunk=C, start_pos=start_pos, chunk_lens=chunk_lens,
                           max_blocks_per_seq=mbps, seed=88_000 + i, window=window, sinks=sinks), split


@pytest.mark.parametrize("i", range(N_PREFILL))
def test_prefill_random_case(i):
    w, split = _prefill_draw(i)
    log(f"[gpu] random prefill case {i}: Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim} "
        f"BS={w.block_size} C={w.chunk} start={w.start_pos} n={w.chunk_lens} split={split} window={w.window} "
        f"sinks={w.sinks}")
    case = make_prefill_case(w)
    kp, vp = oracle.kv_append_chunk(case.k_cache, case.v_cache, case.k_src, case.v_src, case.block_tables,
                                    case.start_pos, case.chunk_lens, w.block_size)
    sw = w.window > 0 or w.sinks
    if sw:
        exp = oracle.paged_prefill_attention_sinks(case.q, kp, vp, case.block_tables, case.start_pos, case.chunk_lens,
                                                   w.scale, w.block_size, "bf16", sinks=case.sinks, window=w.window)
    else:
        exp = oracle.paged_prefill_attention(case.q, kp, vp, case.block_tables, case.start_pos, case.chunk_lens,
                                             w.scale, w.block_size, "bf16")
    dev = {
        "q": to_torch(case.q, "bf16").cuda(), "k_src": to_torch(case.k_src, "bf16").cuda(),
        "v_src": to_torch(case.v_src, "bf16").cuda(), "k_cache": to_torch(case.k_cache, "bf16").cuda(),
        "v_cache": to_torch(case.v_cache, "bf16").cuda(), "bt": torch.from_numpy(case.block_tables).cuda(),
        "sp": torch.from_numpy(case.start_pos).cuda(), "cl": torch.from_numpy(case.chunk_lens).cuda(),
    }
    xs.xs_kv_append_chunk(dev["k_src"], dev["v_src"], dev["k_cache"], dev["v_cache"], dev["bt"], dev["sp"], dev["cl"])
    out = torch.full_like(dev["q"], float("nan"))
    po = pml = None
    if split:
        B, Hq, C, D = dev["q"].shape
        NP = xs.num_partitions(dev["bt"].shape[1] * w.block_size, split)
        po = torch.full((B, Hq, C, NP, D), float("nan"), dtype=torch.float32, device="cuda")
        pml = torch.full((B, Hq, C, NP, 2), float("nan"), dtype=torch.float32, device="cuda")
    if sw:
        sinks_t = None if case.sinks is None else to_torch(case.sinks, "bf16").cuda()
        xs.xs_paged_attn_prefill_sinks(dev["q"], dev["k_cache"], dev["v_cache"], dev["bt"], dev["sp"], dev["cl"],
                                       w.scale, sinks=sinks_t, window_size=w.window, partition_size=split, out=out,
                                       part_o=po, part_ml=pml)
    elif split:
        xs.xs_paged_attn_prefill_split(dev["q"], dev["k_cache"], dev["v_cache"], dev["bt"], dev["sp"], dev["cl"],
                                       w.scale, split, out=out, part_o=po, part_ml=pml)
    else:
        xs.xs_paged_attn_prefill(dev["q"], dev["k_cache"], dev["v_cache"], dev["bt"], dev["sp"], dev["cl"], w.scale,
                                 out=out)
    torch.cuda.synchronize()
    for name, exp_pool in (("k_cache", kp), ("v_cache", vp)):
        assert np.array_equal(to_numpy_bits(dev[name]).view(np.uint8), exp_pool.view(np.uint8)), \
            f"case {i}: {name} after the chunk append"
    got = as_f64(out)
    assert_close(got, exp, *TOL["bf16"], f"random prefill case {i}")
    tau = prefill_spread(case.q, kp, vp, case.block_tables, case.start_pos, case.chunk_lens, w.scale, w.block_size,
                         "bf16", sinks=case.sinks, window=w.window)
    assert_rounding_bound(got, exp, tau, f"random prefill case {i}, rounding bound")
    for b, n in enumerate(case.chunk_lens.tolist()):
        assert not got[b, :, n:].any(), f"case {i}: rows past chunk_lens[{b}] = {n} are not zero"
