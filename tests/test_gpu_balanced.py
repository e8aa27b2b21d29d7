"""The balanced decode (xs_paged_attn_decode_balanced) against the fp64 oracle (needs an MI355X).

Every bf16 workload at full size, with and without the fused append. Reduced shapes cover the
supported head_dim / block_size, GQA groups 1..16, empty sequences, single tokens, and batches
with fewer tiles than workers. The schedule depends only on the lengths, so a rerun and a
block-table permutation must give bitwise the same output.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_common import OracleResult, check_case, log, run_step
from workloads.device import case_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _library():
    import paged_kv_decode_xs_amd as xs

    xs.load_library()
    torch.cuda.init()
    yield


@pytest.mark.parametrize("name", [n for n in wl.ORDER if wl.WORKLOADS[n].dtype == "bf16"])
def test_balanced_full_size(name):
    w = wl.WORKLOADS[name]
    case = wl.make_case(w)
    ref = OracleResult(case)
    e0, _, _ = check_case(case, 0, ref, label=f"{name} balanced", schedule="balanced")
    e1, _, _ = check_case(case, 0, ref, label=f"{name} balanced fused", fused=True, schedule="balanced")
    log(f"[gpu] {name}: balanced max |err| {e0:.3g}, fused {e1:.3g}")


SHAPES = [
    # Hq, Hkv, D, BS, lens
    (32, 8, 128, 16, [1, 15, 16, 17, 4095, 513, 0, 2]),
    (32, 8, 128, 32, [0, 31, 33, 700, 64]),
    (12, 12, 64, 16, [64, 1000, 333, 1]),
    (16, 2, 64, 32, [33, 31, 100]),
    (16, 2, 128, 16, [300, 45]),          # group 8
    (32, 2, 128, 16, [129, 2, 1]),        # group 16: two chunks of 8
    (8, 4, 128, 16, [5]),                 # far fewer tiles than workers
    (32, 8, 128, 16, [0, 0, 0, 40, 0]),   # mostly empty
    (24, 8, 64, 16, [77, 130]),           # group 3: one head per chunk
]


def _case(Hq, Hkv, D, BS, lens, seed):
    mbps = max(1, -(-max(lens) // BS) + 1)
    w = wl.Workload(name="balanced", description="", dtype="bf16", batch=len(lens), num_q_heads=Hq,
                    num_kv_heads=Hkv, head_dim=D, block_size=BS, ctx=("fixed", lens), num_blocks=None,
                    max_blocks_per_seq=mbps, values="normal", seed=seed, partition_size=BS)
    return wl.make_case(w)


@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_balanced_shapes(idx):
    Hq, Hkv, D, BS, lens = SHAPES[idx]
    case = _case(Hq, Hkv, D, BS, lens, seed=200 + idx)
    ref = OracleResult(case)
    for fused in (False, True):
        _, step, _ = check_case(case, 0, ref, label=f"balanced shape{idx} fused={fused}", fused=fused,
                                schedule="balanced")
        empty = np.flatnonzero(case.context_lens <= 0)
        if empty.size:
            assert torch.count_nonzero(step.out[torch.from_numpy(empty).cuda()]).item() == 0


def test_balanced_bitwise_rerun_and_permutation():
    w = wl.WORKLOADS["qwen3_8b_b64"].with_(batch=7, ctx=("uniform", 1, 2500), max_blocks_per_seq=160)
    case = wl.make_case(w, seed=23)
    dev = case_to_device(case)
    s1 = run_step(dev, w.scale, 0, fused=True, schedule="balanced")
    out1 = s1.out.clone()
    s1.run()
    torch.cuda.synchronize()
    assert torch.equal(s1.out.view(torch.int16), out1.view(torch.int16)), "second run differs"
    perm = np.random.default_rng(6).permutation(case.num_blocks)
    case2 = wl.Case(workload=w, q=case.q, k_new=case.k_new, v_new=case.v_new,
                    k_cache=np.empty_like(case.k_cache), v_cache=np.empty_like(case.v_cache),
                    block_tables=np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1)
                    .astype(np.int32), context_lens=case.context_lens)
    case2.k_cache[perm] = case.k_cache
    case2.v_cache[perm] = case.v_cache
    s2 = run_step(case_to_device(case2), w.scale, 0, fused=True, schedule="balanced")
    assert torch.equal(s2.out.view(torch.int16), out1.view(torch.int16)), "permutation changed bits"


def test_balanced_fused_append_matches_separate_append():
    case = _case(32, 8, 128, 16, [1, 16, 17, 2000, 0, 300], seed=41)
    a = case_to_device(case)
    s1 = run_step(a, case.workload.scale, 0, fused=False, schedule="balanced")
    b = case_to_device(case)
    s2 = run_step(b, case.workload.scale, 0, fused=True, schedule="balanced")
    assert torch.equal(s1.out.view(torch.int16), s2.out.view(torch.int16))
    for name in ("k_cache", "v_cache"):
        assert torch.equal(a[name].view(torch.int16), b[name].view(torch.int16)), name


def test_balanced_many_short_sequences():
    # Workers cross hundreds of segment boundaries: pieces, slots and merges of short segments.
    w = wl.WORKLOADS["qwen3_8b_b64"].with_(batch=2000, ctx=("uniform", 1, 48), max_blocks_per_seq=3)
    case = wl.make_case(w, seed=31)
    check_case(case, 0, OracleResult(case), label="balanced 2000 short", fused=True, schedule="balanced")


@pytest.mark.slow
def test_balanced_long_sequences():
    # 32 x ~14k tokens: every worker's range lies inside one or two long segments.
    w = wl.WORKLOADS["qwen3_8b_b64"].with_(batch=32, ctx=("uniform", 12000, 16000), max_blocks_per_seq=1000)
    case = wl.make_case(w, seed=37)
    check_case(case, 0, OracleResult(case), label="balanced long", fused=True, schedule="balanced")
