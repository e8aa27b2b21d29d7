"""Decode with attention sinks and a sliding window (xs_paged_attn_decode_sinks, and the split-K
merge xs_paged_attn_reduce_sinks) against the fp64 oracle (needs an MI355X).

The gpt-oss-shaped windowed workload at full size, unsplit and split, with and without the
fused append; reduced shapes cover windows that start inside a tile, inside a block and at a
block boundary, windows of one token and windows longer than the context, block_size 32, GQA
groups 1..16, empty and single-token sequences, no sinks, and sinks far above or below the
scores. Split partials are checked against the oracle's per-partition statistics.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_common import P_BF16_REL, PART_TOL, TOL, as_f64, assert_close, log, nan_fill
from tests.rounding_bound import assert_rounding_bound, decode_spread
from workloads.device import case_to_device, to_numpy_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _library():
    import paged_kv_decode_xs_amd as xs

    xs.load_library()
    torch.cuda.init()
    yield


def _sinks_tensor(bits):
    if bits is None:
        return None
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16).copy()).view(torch.bfloat16).cuda()


def run_case(case, window, sink_bits, P, fused, check_parts=True, label=""):
    import paged_kv_decode_xs_amd as xs

    w = case.workload
    log(f"[gpu] sinks {label}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim} "
        f"BS={w.block_size} window={window} sinks={sink_bits is not None} P={P} fused={fused} "
        f"lens={case.context_lens[:6].tolist()}")
    k_pool, v_pool = oracle.kv_append(case.k_cache, case.v_cache, case.k_new, case.v_new, case.block_tables,
                                      case.context_lens, w.block_size)
    ref = oracle.paged_decode_attention_sinks(case.q, k_pool, v_pool, case.block_tables, case.context_lens, w.scale,
                                              w.block_size, w.dtype, sinks=sink_bits, window=window)
    dev = case_to_device(case)
    maxlen = int(case.context_lens.max(initial=1))
    step = xs.DecodeStep(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                         dev["k_new"], dev["v_new"], w.scale, partition_size=P, max_context_len=maxlen if P else None,
                         fused=fused, sinks=_sinks_tensor(sink_bits), window=window)
    nan_fill(step)
    step.run()
    torch.cuda.synchronize()
    for name, exp in (("k_cache", k_pool), ("v_cache", v_pool)):
        assert np.array_equal(to_numpy_bits(dev[name]).view(np.uint8), exp.view(np.uint8)), f"{name} after append"
    atol, rtol = TOL[w.dtype]
    got = as_f64(step.out)
    err = assert_close(got, ref, atol, rtol, f"{label} out")
    tau = decode_spread(case.q, k_pool, v_pool, case.block_tables, case.context_lens, w.scale, w.block_size, "bf16",
                        sinks=sink_bits, window=window)
    assert_rounding_bound(got, ref, tau, f"{label} out, rounding bound")
    if P > 0 and check_parts:
        _, stats = oracle.split_paged_decode_attention_sinks(case.q, k_pool, v_pool, case.block_tables,
                                                             case.context_lens, w.scale, w.block_size, w.dtype, P,
                                                             sinks=sink_bits, window=window)
        po = step.part_o.cpu().double().numpy()
        pm = step.part_m.cpu().double().numpy()
        pl = step.part_l.cpu().double().numpy()
        vmax = float(np.nanmax(np.abs(oracle.decode_values(v_pool, "bf16"))))
        patol, prtol = PART_TOL
        for b in range(w.batch):
            for h in range(w.num_q_heads):
                j0, o, m, l = stats[b][h]
                n = len(m)
                if n == 0:
                    continue
                assert_close(pm[b, h, j0:j0 + n], m, patol, prtol, f"part_m[{b},{h}]")
                assert_close(pl[b, h, j0:j0 + n], l, patol, 1e-5, f"part_l[{b},{h}]")
                assert_close(po[b, h, j0:j0 + n], o, patol + P_BF16_REL * vmax, prtol, f"part_o[{b},{h}]")
    return err, step


@pytest.mark.parametrize("P,fused", [(0, True), (0, False), (256, True)])
def test_gptoss_window_full_size(P, fused):
    w = wl.WORKLOADS["gptoss_20b_window128_b64"]
    case = wl.make_case(w)
    err, _ = run_case(case, w.window, case.sinks, P, fused, label=f"{w.name} P={P}")
    log(f"[gpu] {w.name} P={P} fused={fused}: max |err| {err:.3g}")


def _case(Hq, Hkv, D, BS, lens, seed):
    mbps = max(1, -(-max(lens) // BS) + 1)
    w = wl.Workload(name="sinks", description="", dtype="bf16", batch=len(lens), num_q_heads=Hq,
                    num_kv_heads=Hkv, head_dim=D, block_size=BS, ctx=("fixed", lens), num_blocks=None,
                    max_blocks_per_seq=mbps, values="normal", seed=seed, partition_size=0)
    return wl.make_case(w)


def _bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)  # exact for these values


SHAPES = [
    # Hq, Hkv, D, BS, lens, window, sinks ("rand", "none", "high", "low")
    (32, 8, 128, 16, [1, 15, 16, 17, 300, 513, 0, 2], 7, "rand"),
    (32, 8, 128, 16, [40, 1000, 33], 16, "high"),
    (32, 8, 128, 32, [70, 31, 900], 33, "rand"),
    (16, 2, 64, 32, [5, 64, 65, 200], 1, "rand"),
    (64, 8, 64, 16, [129, 2000, 128, 127], 128, "none"),
    (64, 8, 64, 16, [129, 700], 5000, "rand"),           # window longer than every context
    (32, 2, 128, 16, [400, 9], 100, "low"),              # group 16: two head chunks
    (12, 12, 64, 16, [64, 333, 1], 50, "rand"),          # MHA
    (24, 8, 64, 16, [77, 130], 0, "high"),               # sinks without a window
]


@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_sinks_window_shapes(idx):
    Hq, Hkv, D, BS, lens, window, kind = SHAPES[idx]
    case = _case(Hq, Hkv, D, BS, lens, seed=300 + idx)
    rng = np.random.default_rng(900 + idx)
    if kind == "none":
        sinks = None
    elif kind == "high":
        sinks = _bits(np.round(rng.uniform(2.0, 6.0, Hq) * 8) / 8)
    elif kind == "low":
        sinks = _bits(np.full(Hq, -60.0))
    else:
        sinks = _bits(np.round(rng.standard_normal(Hq) * 16) / 8)
    for P in (0, 32 if BS == 16 else 64, 128):
        for fused in (False, True):
            run_case(case, window, sinks, P, fused, label=f"shape{idx} P={P}")


def test_window_one_is_the_last_value():
    # A window of one token without sinks returns V_{L-1} (the appended v_new) exactly.
    case = _case(32, 8, 128, 16, [1, 17, 250], seed=77)
    _, step = run_case(case, 1, None, 0, True, label="window 1")
    exp = np.repeat(case.v_new, 4, axis=1)  # q head h reads kv head h // 4
    assert np.array_equal(to_numpy_bits(step.out), exp)


def test_sink_far_above_scores_gives_zero():
    case = _case(32, 8, 128, 16, [50, 400], seed=78)
    _, step = run_case(case, 0, _bits(np.full(32, 120.0)), 0, True, label="sink 120")
    assert torch.count_nonzero(step.out.float().abs() > 1e-30).item() == 0
