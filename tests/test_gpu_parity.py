"""HIP path against the fp64 oracle, through the C ABI (needs an MI355X).

* all five workloads at full size: the append bit-exact over the whole pool, attention within
  tolerance unsplit and split-K, and the split partials against the oracle's partition
  statistics;
* reduced shapes that span several blocks and partitions with ragged tails, every supported
  head_dim / block_size / dtype, GQA groups 1..16, L = 0 and L = 1;
* invariants on the GPU: a block-table permutation gives bitwise the same output, as does a
  second run; one key returns its V exactly;
* block ids outside [0, num_blocks) inside a context are skipped (no access, no contribution),
  unsplit, split and fused; the split item orders for small and large batches.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_common import TOL, OracleResult, as_f64, assert_close, check_case, log, run_step
from workloads.device import case_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _library():
    import paged_kv_decode_xs_amd as xs

    xs.load_library()
    torch.cuda.init()
    yield


# ---------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("name", wl.ORDER)
def test_workload_full_size(name):
    w = wl.WORKLOADS[name]
    case = wl.make_case(w)
    ref = OracleResult(case, w.partition_size)
    err0, _, _ = check_case(case, 0, ref, label=f"{name} unsplit")
    err1, _, _ = check_case(case, w.partition_size, ref, check_pools=False, label=f"{name} split")
    err2, step, _ = check_case(case, w.partition_size, ref, label=f"{name} split fused", fused=True)
    assert step.check_inputs() == [], "the workload's tables break a device-resident precondition"
    log(f"[gpu] {name}: max |err| unsplit {err0:.3g}, split {err1:.3g}, split+fused append {err2:.3g}")


# ---------------------------------------------------------------- reduced shapes and edge cases

SHAPES = [
    # dtype, Hq, Hkv, D, BS, lens, P
    ("f32", 12, 12, 64, 16, [32], 16),
    ("f32", 8, 2, 128, 16, [1, 17, 100, 16], 32),
    ("f32", 4, 4, 64, 8, [0, 9, 40], 8),
    ("f32", 6, 2, 64, 32, [65, 3], 32),
    ("bf16", 12, 12, 64, 16, [64, 1000, 333, 1], 128),
    ("bf16", 32, 8, 128, 16, [1, 15, 16, 17, 4095, 513], 64),
    ("bf16", 32, 8, 128, 8, [200, 7], 16),
    ("bf16", 32, 8, 128, 32, [0, 31, 33, 700], 96),
    ("bf16", 16, 16, 128, 16, [50, 51], 16),
    ("bf16", 24, 8, 128, 16, [77, 130], 32),   # group 3: one head per wavefront, 3 chunks
    ("bf16", 12, 2, 64, 16, [90, 260], 64),    # group 6: two heads per wavefront
    ("bf16", 16, 2, 128, 16, [300, 45, 0], 64),   # group 8 (an empty row of 8 heads: zeros past 64 lanes)
    ("bf16", 32, 2, 128, 16, [129, 2, 0], 48),    # group 16: two chunks of 8
    ("f32", 32, 2, 64, 16, [70, 18], 32),
]


def _shape_case(dtype, Hq, Hkv, D, BS, lens, seed):
    mbps = max(1, -(-max(lens) // BS) + 1)
    w = wl.Workload(name="shape", description="", dtype=dtype, batch=len(lens), num_q_heads=Hq,
                    num_kv_heads=Hkv, head_dim=D, block_size=BS, ctx=("fixed", lens), num_blocks=None,
                    max_blocks_per_seq=mbps, values="normal", seed=seed, partition_size=BS)
    return wl.make_case(w)


@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_shapes(idx):
    dtype, Hq, Hkv, D, BS, lens, P = SHAPES[idx]
    case = _shape_case(dtype, Hq, Hkv, D, BS, lens, seed=100 + idx)
    ref = OracleResult(case, P)
    check_case(case, 0, ref, label=f"shape{idx} unsplit")
    check_case(case, 0, ref, label=f"shape{idx} unsplit fused", fused=True)
    check_case(case, P, ref, check_pools=False, label=f"shape{idx} split")
    # Partition = one block: many partitions per sequence.
    check_case(case, BS, OracleResult(case, BS), check_pools=False, label=f"shape{idx} P=BS")


def test_empty_contexts_give_zeros():
    case = _shape_case("bf16", 8, 2, 128, 16, [0, 0, 5], seed=7)
    ref = OracleResult(case, 32)
    for P in (0, 32):
        _, step, _ = check_case(case, P, ref, label=f"empty P={P}")
        assert torch.count_nonzero(step.out[:2]).item() == 0


def test_single_key_returns_v_exactly():
    case = _shape_case("f32", 8, 2, 128, 16, [1, 1], seed=8)
    _, step, _ = check_case(case, 0, OracleResult(case), label="L=1")
    got = step.out.cpu().numpy()
    for b in range(2):
        for h in range(8):
            assert np.array_equal(got[b, h], case.v_new[b, h // 4]), (b, h)


def test_permutation_and_rerun_are_bitwise_identical():
    w = wl.WORKLOADS["qwen3_8b_b64"].with_(batch=6, ctx=("uniform", 1, 1500), max_blocks_per_seq=96)
    case = wl.make_case(w, seed=21)
    P = 64
    ref = OracleResult(case, P)
    _, step1, dev = check_case(case, P, ref, label="perm base")
    out1 = step1.out.clone()
    step1.run()
    torch.cuda.synchronize()
    assert torch.equal(step1.out.view(torch.int16), out1.view(torch.int16)), "second run differs"
    # Re-place every block by a permutation of pool ids and rewrite the table.
    rng = np.random.default_rng(5)
    perm = rng.permutation(case.num_blocks)
    case2 = wl.Case(workload=w, q=case.q, k_new=case.k_new, v_new=case.v_new,
                    k_cache=np.empty_like(case.k_cache), v_cache=np.empty_like(case.v_cache),
                    block_tables=np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1)
                    .astype(np.int32), context_lens=case.context_lens)
    case2.k_cache[perm] = case.k_cache
    case2.v_cache[perm] = case.v_cache
    for P2 in (0, P):
        dev2 = case_to_device(case2)
        s2 = run_step(dev2, w.scale, P2, int(case.context_lens.max()))
        s1 = run_step(case_to_device(case), w.scale, P2, int(case.context_lens.max()))
        assert torch.equal(s2.out.view(torch.int16), s1.out.view(torch.int16)), f"permutation changed bits (P={P2})"
    log("[gpu] permutation and rerun: bitwise identical")


def test_stream_argument_is_honoured():
    case = _shape_case("bf16", 32, 8, 128, 16, [300, 1000], seed=9)
    ref = OracleResult(case, 128)
    dev = case_to_device(case)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        import paged_kv_decode_xs_amd as xs

        step = xs.DecodeStep(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                             dev["k_new"], dev["v_new"], case.workload.scale, partition_size=128)
        step.run(stream=s)
    s.synchronize()
    from tests.gpu_common import TOL, assert_close

    assert_close(as_f64(step.out), ref.out, *TOL["bf16"], "side stream")


@pytest.mark.parametrize("dtype,Hq,Hkv,D,BS,lens,P", [
    ("bf16", 32, 8, 128, 16, [1, 16, 17, 2000, 0], 64),   # matrix-core kernel
    ("bf16", 16, 2, 64, 32, [33, 31, 100], 32),           # matrix-core kernel, group 8, two tiles per block
    ("bf16", 12, 12, 64, 8, [9, 200], 16),                # generic kernel (block_size 8)
    ("f32", 8, 2, 128, 16, [5, 77], 32),                  # generic kernel (fp32)
])
def test_fused_append_is_bitwise_the_two_calls(dtype, Hq, Hkv, D, BS, lens, P):
    case = _shape_case(dtype, Hq, Hkv, D, BS, lens, seed=31)
    maxlen = max(lens)
    for part in (0, P):
        a = case_to_device(case)
        s1 = run_step(a, case.workload.scale, part, maxlen, fused=False)
        b = case_to_device(case)
        s2 = run_step(b, case.workload.scale, part, maxlen, fused=True)
        view = torch.int16 if dtype == "bf16" else torch.int32
        assert torch.equal(s1.out.view(view), s2.out.view(view)), f"outputs differ (P={part})"
        for name in ("k_cache", "v_cache"):
            assert torch.equal(a[name].view(view), b[name].view(view)), f"{name} differs (P={part})"
    log(f"[gpu] fused append: bitwise equal to append + decode for {dtype} D={D} BS={BS}")


def test_split_order_for_large_and_small_batches():
    # The split grid maps workgroup ids onto the partitions that exist for batches of up to 256
    # sequences (full partitions first, then the partial ones, ranked by size for up to 64
    # sequences, with every second whole round of CU-count ids reversed) and keeps
    # partition-major ids above that. Every order must give the oracle's result, with partitions
    # past a sequence's end, empty sequences, tied partial sizes and a last round that is not
    # whole mixed in.
    # Partition size 64 on small grids takes partition-major ids; 256 the ranked order (2 to 256
    # sequences).
    rng = np.random.default_rng(31)
    for B in (2, 64, 65, 256, 300):
        lens = rng.integers(0, 1400, B).tolist()
        lens[1] = 0
        if B > 5:
            lens[5] = 1
        case = _shape_case("bf16", 8, 2, 64, 16, lens, seed=32 + B)
        for P in (64, 256):
            ref = OracleResult(case, P)
            check_case(case, P, ref, check_pools=False, label=f"split order B={B} P={P}")
            check_case(case, P, ref, label=f"split order B={B} P={P} fused", fused=True)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("P", [0, 16, 32])
def test_bad_block_ids_are_skipped(P, fused):
    # Block ids outside [0, num_blocks) inside a context are skipped: sequence 0's table
    # [b0, -1, b2, NB + 5] with L = 64 attends over the 32 tokens of b0 and b2 only, which is the
    # oracle's result for the table [b0, b2] with L = 32 (decode attention does not depend on the
    # order of its keys). The append into a bad block is skipped too; sequence 1 is unaffected.
    case = _shape_case("bf16", 8, 2, 128, 16, [64, 40], seed=51)
    w = case.workload
    NB = case.num_blocks
    bt = case.block_tables.copy()
    b0, b2 = int(bt[0, 0]), int(bt[0, 2])
    bad = bt.copy()
    bad[0, 1] = -1
    bad[0, 3] = NB + 5
    log(f"[gpu] bad block ids: P={P} fused={fused} table0={bad[0, :4].tolist()}")
    kp, vp = oracle.kv_append(case.k_cache, case.v_cache, case.k_new, case.v_new, bt, case.context_lens, w.block_size)
    exp_bt = np.full_like(bt, -1)
    exp_bt[0, :2] = [b0, b2]
    exp_bt[1] = bt[1]
    exp = oracle.paged_decode_attention(case.q, kp, vp, exp_bt, np.array([32, 40], np.int32), w.scale, w.block_size,
                                        w.dtype)
    dev = case_to_device(case)
    dev["block_tables"].copy_(torch.from_numpy(bad))
    step = run_step(dev, w.scale, P, 64 if P else None, fused=fused)
    problems = step.check_inputs()
    assert len(problems) == 2 and "block_tables[0, 1] = -1" in problems[0] and f"= {NB + 5} " in problems[1], problems
    got = as_f64(step.out)
    assert np.isfinite(got).all()
    assert_close(got, exp, *TOL["bf16"], f"bad block ids P={P} fused={fused}")


def test_partition_overflow_gives_nan_rows():
    # Sequence 1 needs 4 partitions of 64 tokens but the partials hold 2: the reduce writes its
    # rows as NaN (a truncated context must not pass for a result); the others are unaffected.
    import paged_kv_decode_xs_amd as xs
    from tests.gpu_common import nan_fill

    case = _shape_case("bf16", 8, 2, 128, 16, [100, 250, 0, 128], seed=81)
    w = case.workload
    ref = OracleResult(case)
    dev = case_to_device(case)
    step = xs.DecodeStep(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                         dev["k_new"], dev["v_new"], w.scale, partition_size=64, max_context_len=128, fused=True)
    assert step.part_m.shape[-1] == 2
    problems = step.check_inputs()
    assert len(problems) == 1 and problems[0].startswith("sequence 1: 250 tokens need 4 partitions"), problems
    nan_fill(step)
    step.run()
    torch.cuda.synchronize()
    got = as_f64(step.out)
    assert np.isnan(got[1]).all(), "the truncated sequence must give NaN rows"
    keep = [0, 2, 3]
    assert_close(got[keep], ref.out[keep], *TOL["bf16"], "partition overflow: the other sequences")
    log("[gpu] partition overflow: NaN rows")
