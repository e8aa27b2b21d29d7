"""The decode step captured as one HIP graph (xs_step_graph_*) against the same step run eagerly
(needs an MI355X).

A decode loop: each iteration writes new q / k_new / v_new into the captured buffers, advances
context_lens by one, and replays the graph. The same inputs go to an eager DecodeStep on separate
copies of the pools. Every replay must match the eager step bit for bit (output and pools), with
the program's own eager work and synchronizations between replays; the last iteration is also
checked against the fp64 oracle. Variants: unsplit and split-K, fused and separate append,
sinks + sliding window, and two graphs alive at once.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_xs_amd as xs
import workloads as wl
from tests.gpu_common import TOL, as_f64, assert_close, log
from workloads.device import case_to_device, to_numpy_bits, to_torch

pytestmark = pytest.mark.gpu

STEPS = 4


@pytest.fixture(scope="module", autouse=True)
def _library():
    xs.load_library()
    torch.cuda.init()
    yield


def _setup(Hq, Hkv, D, lens0, P, fused, window=0, sinks=False, seed=0):
    BS = 16
    final = [L + STEPS for L in lens0]
    mbps = -(-max(final) // BS) + 1
    w = wl.Workload(name="graph", description="", dtype="bf16", batch=len(lens0), num_q_heads=Hq,
                    num_kv_heads=Hkv, head_dim=D, block_size=BS, ctx=("fixed", final), num_blocks=None,
                    max_blocks_per_seq=mbps, values="normal", seed=seed, partition_size=P, window=window,
                    sinks=sinks)
    case = wl.make_case(w)
    dev = case_to_device(case)
    dev["context_lens"].copy_(torch.tensor(lens0, dtype=torch.int32))
    sk = None
    if case.sinks is not None:
        sk = torch.from_numpy(case.sinks.view(np.int16).copy()).view(torch.bfloat16).cuda()
    mk = lambda d: xs.DecodeStep(d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],  # noqa: E731
                                 d["k_new"], d["v_new"], w.scale, partition_size=P,
                                 max_context_len=max(final) if P else None, fused=fused, sinks=sk, window=window)
    ref = {k: v.clone() for k, v in dev.items()}
    return case, dev, ref, mk(dev), mk(ref)


def _new_inputs(rng, case):
    w = case.workload
    q = wl.f32_to_bf16_bits(rng.standard_normal((w.batch, w.num_q_heads, w.head_dim)).astype(np.float32))
    kn = wl.f32_to_bf16_bits(rng.standard_normal((w.batch, w.num_kv_heads, w.head_dim)).astype(np.float32))
    vn = wl.f32_to_bf16_bits(rng.standard_normal((w.batch, w.num_kv_heads, w.head_dim)).astype(np.float32))
    return q, kn, vn


def _write(dev, q, kn, vn, lens):
    dev["q"].copy_(to_torch(q, "bf16"))
    dev["k_new"].copy_(to_torch(kn, "bf16"))
    dev["v_new"].copy_(to_torch(vn, "bf16"))
    dev["context_lens"].copy_(torch.tensor(lens, dtype=torch.int32))


def _loop(label, Hq, Hkv, D, lens0, P, fused, window=0, sinks=False, seed=0):
    log(f"[gpu] graph {label}: Hq={Hq} Hkv={Hkv} D={D} lens0={lens0} P={P} fused={fused} window={window} "
        f"sinks={sinks}")
    case, dev, ref, step, eager = _setup(Hq, Hkv, D, lens0, P, fused, window, sinks, seed)
    # Warm the library outside the capture (code objects load and device attributes are read on
    # first use). Both copies take the same step, so their pools stay equal.
    step.run()
    eager.run()
    torch.cuda.synchronize()
    graph = step.capture()
    rng = np.random.default_rng(seed + 1)
    w = case.workload
    for i in range(STEPS):
        lens = [L + 1 + i for L in lens0]
        q, kn, vn = _new_inputs(rng, case)
        _write(dev, q, kn, vn, lens)
        _write(ref, q, kn, vn, lens)
        if i == STEPS - 1:
            k_before = to_numpy_bits(dev["k_cache"])
            v_before = to_numpy_bits(dev["v_cache"])
        graph.launch()
        eager.run()
        torch.cuda.synchronize()
        assert torch.equal(step.out.view(torch.int16), eager.out.view(torch.int16)), f"replay {i}: out differs"
        for name in ("k_cache", "v_cache"):
            assert torch.equal(dev[name].view(torch.int16), ref[name].view(torch.int16)), f"replay {i}: {name}"
        # Some unrelated eager work on the same stream between replays.
        torch.cuda.synchronize()
        _ = (dev["q"].float() * 2).sum().item()
    lens_np = np.array(lens, np.int32)
    kp, vp = oracle.kv_append(k_before, v_before, kn, vn, case.block_tables, lens_np, w.block_size)
    exp = oracle.paged_decode_attention_sinks(q, kp, vp, case.block_tables, lens_np, w.scale, w.block_size, "bf16",
                                              sinks=case.sinks, window=window)
    atol, rtol = TOL["bf16"]
    assert_close(as_f64(step.out), exp, atol, rtol, f"graph {label} vs oracle")
    graph.close()


@pytest.mark.parametrize("P,fused", [(0, True), (64, True), (64, False), (0, False)])
def test_graph_replays_match_eager(P, fused):
    _loop(f"P={P} fused={fused}", 32, 8, 128, [100, 17, 640, 1], P, fused, seed=10 + P + int(fused))


def test_graph_with_sinks_and_window():
    _loop("sinks+window split", 64, 8, 64, [300, 40, 129], 64, True, window=48, sinks=True, seed=20)
    _loop("sinks+window unsplit", 64, 8, 64, [300, 40, 129], 0, False, window=100, sinks=True, seed=21)


def test_two_graphs_alternate():
    _, devA, refA, stepA, eagerA = _setup(32, 8, 128, [50, 200], 0, True, seed=30)
    _, devB, refB, stepB, eagerB = _setup(12, 12, 64, [500, 33, 90], 64, True, seed=31)
    for s in (stepA, stepB, eagerA, eagerB):
        s.run()
    torch.cuda.synchronize()
    gA, gB = stepA.capture(), stepB.capture()
    for i in range(3):
        for dev, ref, lens0 in ((devA, refA, [50, 200]), (devB, refB, [500, 33, 90])):
            lens = torch.tensor([L + 1 + i for L in lens0], dtype=torch.int32)
            dev["context_lens"].copy_(lens)
            ref["context_lens"].copy_(lens)
        gA.launch()
        gB.launch()
        eagerA.run()
        eagerB.run()
        torch.cuda.synchronize()
        assert torch.equal(stepA.out.view(torch.int16), eagerA.out.view(torch.int16))
        assert torch.equal(stepB.out.view(torch.int16), eagerB.out.view(torch.int16))
    gA.close()
    gB.close()


def test_layer_stack_graph():
    # Three steps (layers) on their own pools, captured in order as one graph.
    sets = [_setup(32, 8, 128, [90, 300], 64 if i % 2 else 0, True, seed=40 + i) for i in range(3)]
    for _, _, _, step, eager in sets:
        step.run()
        eager.run()
    torch.cuda.synchronize()
    graph = xs.StepGraph([s[3] for s in sets])
    for i in range(3):
        for _, dev, ref, _, _ in sets:
            lens = torch.tensor([91 + i, 301 + i], dtype=torch.int32)
            dev["context_lens"].copy_(lens)
            ref["context_lens"].copy_(lens)
        out = graph.launch()
        for _, _, _, _, eager in sets:
            eager.run()
        torch.cuda.synchronize()
        assert out.data_ptr() == sets[-1][3].out.data_ptr()
        for _, dev, ref, step, eager in sets:
            assert torch.equal(step.out.view(torch.int16), eager.out.view(torch.int16))
            assert torch.equal(dev["k_cache"].view(torch.int16), ref["k_cache"].view(torch.int16))
    graph.close()
