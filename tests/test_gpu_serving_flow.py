"""The serving flow end to end on one set of pools (needs an MI355X), plain and with the gpt-oss
sinks and sliding window. Each sequence's prompt goes in through chunked prefill
(xs_kv_append_chunk, then xs_paged_attn_prefill / _split / _sinks; several chunks, the sequences
finishing their prompts at different chunks), then every sequence decodes several tokens (the
append fused with the decode attention, unsplit or split-K with its reduce), and the pools carry
over from call to call. Every attention output is compared with the fp64 oracle run through the
same steps at the bf16 bar, and the pools must equal the oracle's bit for bit after the last step.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_xs_amd as xs
from tests.gpu_common import TOL, as_f64, assert_close, log
from workloads import f32_to_bf16_bits
from workloads.device import to_numpy_bits, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _library():
    xs.load_library()
    torch.cuda.init()
    yield


def _bf16(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("split", [0, 64])
@pytest.mark.parametrize("Hq,Hkv,D", [(8, 2, 128), (16, 4, 64)])
def test_prefill_then_decode(Hq, Hkv, D, split):
    rng = np.random.default_rng(77 + D + split)
    prompts = [37, 130, 5]
    B, BS, C, steps = len(prompts), 16, 64, 4
    scale = 1.0 / np.sqrt(D)
    max_len = max(prompts) + steps
    MBPS = -(-max_len // BS)
    NB = B * MBPS + 3
    bt = np.full((B, MBPS), -1, np.int32)
    perm = rng.permutation(NB).astype(np.int32)
    for b in range(B):
        bt[b] = perm[b * MBPS:(b + 1) * MBPS]
    k_pool = np.full((NB, Hkv, BS, D), 0x7FC0, np.uint16)  # NaN until written
    v_pool = k_pool.copy()
    kc, vc = to_torch(k_pool, "bf16").cuda(), to_torch(v_pool, "bf16").cuda()
    bt_d = torch.from_numpy(bt).cuda()
    atol, rtol = TOL["bf16"]
    log(f"[gpu] serving flow: Hq={Hq} Hkv={Hkv} D={D} prompts={prompts} chunk={C} decode steps={steps} split={split}")

    # Prefill: chunk by chunk until every prompt is in.
    done = [0] * B
    while any(d < p for d, p in zip(done, prompts)):
        start = np.array(done, np.int32)
        n = np.array([min(C, p - d) for d, p in zip(done, prompts)], np.int32)
        q = _bf16(rng, (B, Hq, C, D))
        ks, vs = _bf16(rng, (B, Hkv, C, D)), _bf16(rng, (B, Hkv, C, D))
        k_pool, v_pool = oracle.kv_append_chunk(k_pool, v_pool, ks, vs, bt, start, n, BS)
        exp = oracle.paged_prefill_attention(q, k_pool, v_pool, bt, start, n, scale, BS, "bf16")
        sp_d, n_d = torch.from_numpy(start).cuda(), torch.from_numpy(n).cuda()
        xs.xs_kv_append_chunk(to_torch(ks, "bf16").cuda(), to_torch(vs, "bf16").cuda(), kc, vc, bt_d, sp_d, n_d)
        qd = to_torch(q, "bf16").cuda()
        if split:
            out = xs.xs_paged_attn_prefill_split(qd, kc, vc, bt_d, sp_d, n_d, scale, split)
        else:
            out = xs.xs_paged_attn_prefill(qd, kc, vc, bt_d, sp_d, n_d, scale)
        torch.cuda.synchronize()
        got = as_f64(out)
        assert_close(got, exp, atol, rtol, f"prefill chunk at {start.tolist()}")
        for b in range(B):
            assert not got[b, :, int(n[b]):].any()
        done = [d + int(k) for d, k in zip(done, n)]

    # Decode: one token per sequence per step, the append fused with the attention.
    lens = np.array(prompts, np.int32)
    P = split or 0
    for step in range(steps):
        lens = lens + 1
        q = _bf16(rng, (B, Hq, D))
        kn, vn = _bf16(rng, (B, Hkv, D)), _bf16(rng, (B, Hkv, D))
        k_pool, v_pool = oracle.kv_append(k_pool, v_pool, kn, vn, bt, lens, BS)
        exp = oracle.paged_decode_attention(q, k_pool, v_pool, bt, lens, scale, BS, "bf16")
        lens_d = torch.from_numpy(lens).cuda()
        qd = to_torch(q, "bf16").cuda()
        out = torch.empty_like(qd)
        if P:
            NP = xs.num_partitions(MBPS * BS, P)
            po = torch.empty((B, Hq, NP, D), dtype=torch.float32, device="cuda")
            pm = torch.empty((B, Hq, NP), dtype=torch.float32, device="cuda")
            pl = torch.empty((B, Hq, NP), dtype=torch.float32, device="cuda")
            xs.xs_paged_attn_decode_append(qd, to_torch(kn, "bf16").cuda(), to_torch(vn, "bf16").cuda(), kc, vc, bt_d,
                                           lens_d, scale, part_o=po, part_m=pm, part_l=pl, partition_size=P)
            xs.xs_paged_attn_reduce(po, pm, pl, lens_d, out, P)
        else:
            xs.xs_paged_attn_decode_append(qd, to_torch(kn, "bf16").cuda(), to_torch(vn, "bf16").cuda(), kc, vc, bt_d,
                                           lens_d, scale, out=out)
        torch.cuda.synchronize()
        assert_close(as_f64(out), exp, atol, rtol, f"decode step {step} (lens {lens.tolist()})")

    # The pools after the whole flow: bit for bit the oracle's (every slot written once, NaN elsewhere).
    assert np.array_equal(to_numpy_bits(kc), k_pool) and np.array_equal(to_numpy_bits(vc), v_pool)


@pytest.mark.parametrize("split", [0, 64])
@pytest.mark.parametrize("window", [0, 20])
def test_prefill_then_decode_with_sinks_and_window(window, split):
    """The same flow for a gpt-oss layer: per-head sinks, and a sliding window or none
    (xs_paged_attn_prefill_sinks for the prompt chunks, xs_paged_attn_decode_sinks with the fused
    append and xs_paged_attn_reduce_sinks for the decode steps)."""
    rng = np.random.default_rng(91 + window + split)
    Hq, Hkv, D = 16, 2, 64
    prompts = [45, 150, 9]
    B, BS, C, steps = len(prompts), 16, 64, 4
    scale = 1.0 / np.sqrt(D)
    max_len = max(prompts) + steps
    MBPS = -(-max_len // BS)
    NB = B * MBPS + 3
    perm = rng.permutation(NB).astype(np.int32)
    bt = np.stack([perm[b * MBPS:(b + 1) * MBPS] for b in range(B)]).astype(np.int32)
    sinks = _bf16(rng, (Hq,))
    k_pool = np.full((NB, Hkv, BS, D), 0x7FC0, np.uint16)
    v_pool = k_pool.copy()
    kc, vc = to_torch(k_pool, "bf16").cuda(), to_torch(v_pool, "bf16").cuda()
    bt_d = torch.from_numpy(bt).cuda()
    sinks_d = to_torch(sinks, "bf16").cuda()
    atol, rtol = TOL["bf16"]
    log(f"[gpu] serving flow with sinks: window={window} split={split}")

    done = [0] * B
    while any(d < p for d, p in zip(done, prompts)):
        start = np.array(done, np.int32)
        n = np.array([min(C, p - d) for d, p in zip(done, prompts)], np.int32)
        q = _bf16(rng, (B, Hq, C, D))
        ks, vs = _bf16(rng, (B, Hkv, C, D)), _bf16(rng, (B, Hkv, C, D))
        k_pool, v_pool = oracle.kv_append_chunk(k_pool, v_pool, ks, vs, bt, start, n, BS)
        exp = oracle.paged_prefill_attention_sinks(q, k_pool, v_pool, bt, start, n, scale, BS, "bf16", sinks=sinks,
                                                   window=window)
        sp_d, n_d = torch.from_numpy(start).cuda(), torch.from_numpy(n).cuda()
        xs.xs_kv_append_chunk(to_torch(ks, "bf16").cuda(), to_torch(vs, "bf16").cuda(), kc, vc, bt_d, sp_d, n_d)
        out = xs.xs_paged_attn_prefill_sinks(to_torch(q, "bf16").cuda(), kc, vc, bt_d, sp_d, n_d, scale, sinks=sinks_d,
                                             window_size=window, partition_size=split)
        torch.cuda.synchronize()
        assert_close(as_f64(out), exp, atol, rtol, f"prefill chunk at {start.tolist()}")
        done = [d + int(k) for d, k in zip(done, n)]

    lens = np.array(prompts, np.int32)
    for step in range(steps):
        lens = lens + 1
        q = _bf16(rng, (B, Hq, D))
        kn, vn = _bf16(rng, (B, Hkv, D)), _bf16(rng, (B, Hkv, D))
        k_pool, v_pool = oracle.kv_append(k_pool, v_pool, kn, vn, bt, lens, BS)
        exp = oracle.paged_decode_attention_sinks(q, k_pool, v_pool, bt, lens, scale, BS, "bf16", sinks=sinks,
                                                  window=window)
        lens_d = torch.from_numpy(lens).cuda()
        qd = to_torch(q, "bf16").cuda()
        out = torch.empty_like(qd)
        kn_d, vn_d = to_torch(kn, "bf16").cuda(), to_torch(vn, "bf16").cuda()
        if split:
            NP = xs.num_partitions(MBPS * BS, split)
            po = torch.empty((B, Hq, NP, D), dtype=torch.float32, device="cuda")
            pm = torch.empty((B, Hq, NP), dtype=torch.float32, device="cuda")
            pl = torch.empty((B, Hq, NP), dtype=torch.float32, device="cuda")
            xs.xs_paged_attn_decode_sinks(qd, kc, vc, bt_d, lens_d, scale, sinks=sinks_d, window_size=window, part_o=po,
                                          part_m=pm, part_l=pl, partition_size=split, k_new=kn_d, v_new=vn_d)
            xs.xs_paged_attn_reduce_sinks(po, pm, pl, lens_d, out, split, sinks=sinks_d, window_size=window)
        else:
            xs.xs_paged_attn_decode_sinks(qd, kc, vc, bt_d, lens_d, scale, sinks=sinks_d, window_size=window, out=out,
                                          k_new=kn_d, v_new=vn_d)
        torch.cuda.synchronize()
        assert_close(as_f64(out), exp, atol, rtol, f"decode step {step} (lens {lens.tolist()})")

    assert np.array_equal(to_numpy_bits(kc), k_pool) and np.array_equal(to_numpy_bits(vc), v_pool)
