"""Invariants of the decode step on the GPU (through the C ABI), checked against values the
mathematics fixes rather than against the oracle:

* keys that are all equal give every position the same weight, so each head's output is the
  plain mean of the V rows its sequence holds (including the row appended in this step);
* values that are all one constant c give c back whatever the keys, because the softmax weights
  of a row sum to one.

Both run unsplit and split-K (partials merged by the reduce), with the append separate and fused,
for bf16 (matrix-core path) and fp32 (generic path). The expected values are computed here from
the inputs; the only tolerance is the rounding the kernels do: for bf16 the output's own rounding
(unit roundoff 2^-8 relative) plus, for the constant case, the weights rounded to bf16 for the P.V
product on the matrix cores (2^-8 relative); for fp32, accumulation order.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_common import as_f64, log, run_step
from workloads import f32_to_bf16_bits
from workloads.device import case_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _library():
    import paged_kv_decode_xs_amd as xs

    xs.load_library()
    torch.cuda.init()
    yield


# dtype, Hq, Hkv, D, BS, lens
SHAPES = [
    ("bf16", 32, 8, 128, 16, [1, 17, 300, 2049]),
    ("bf16", 12, 12, 64, 16, [64, 1000]),
    ("bf16", 16, 2, 128, 32, [129, 700]),
    ("bf16", 32, 8, 128, 8, [40, 513]),
    ("f32", 8, 2, 128, 16, [1, 100, 257]),
    ("f32", 12, 12, 64, 16, [33, 640]),
]
PATHS = [(0, False), (0, True), (64, False), (64, True), (512, True)]


def _case(dtype, Hq, Hkv, D, BS, lens, seed):
    mbps = max(1, -(-max(lens) // BS) + 1)
    w = wl.Workload(name="invariant", description="", dtype=dtype, batch=len(lens), num_q_heads=Hq,
                    num_kv_heads=Hkv, head_dim=D, block_size=BS, ctx=("fixed", lens), num_blocks=None,
                    max_blocks_per_seq=mbps, values="normal", seed=seed, partition_size=BS)
    return wl.make_case(w)


def _values(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _encode(x, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _cached_slots(case, b):
    """(block, slot) of every position of sequence b before this step's append."""
    BS = case.workload.block_size
    L = int(case.context_lens[b])
    return [(int(case.block_tables[b, t // BS]), t % BS) for t in range(max(L - 1, 0))]


def _run(case, P, fused):
    dev = case_to_device(case)
    step = run_step(dev, case.workload.scale, P, int(case.context_lens.max()) if P else None, fused=fused)
    return as_f64(step.out)


@pytest.mark.parametrize("P,fused", PATHS)
@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_identical_keys_give_the_mean_of_v(idx, P, fused):
    dtype, Hq, Hkv, D, BS, lens = SHAPES[idx]
    case = _case(dtype, Hq, Hkv, D, BS, lens, seed=300 + idx)
    G = Hq // Hkv
    expect = np.zeros((len(lens), Hq, D))
    for b in range(len(lens)):
        slots = _cached_slots(case, b)
        for g in range(Hkv):
            key = case.k_new[b, g].copy()  # every cached key of (b, g) becomes the new one
            for blk, s in slots:
                case.k_cache[blk, g, s] = key
            vs = [_values(case.v_cache[blk, g, s], dtype) for blk, s in slots] + [_values(case.v_new[b, g], dtype)]
            expect[b, g * G:(g + 1) * G] = np.mean(vs, axis=0)
    got = _run(case, P, fused)
    if dtype == "bf16":
        tol = 2.0 ** -8 * np.abs(expect) + 2e-6 * np.sqrt(max(lens)) + 1e-6
    else:
        tol = 1e-6 * np.abs(expect) + 1e-6 * np.sqrt(max(lens))
    err = np.abs(got - expect)
    assert np.all(np.isfinite(got)), "non-finite output"
    assert np.all(err <= tol), (f"{dtype} {SHAPES[idx]} P={P} fused={fused}: max err {err.max():.3g}, "
                                f"{int((err > tol).sum())} elements beyond the bound")
    log(f"[gpu] identical keys {SHAPES[idx]} P={P} fused={fused}: max |out - mean V| {err.max():.3g}")


@pytest.mark.parametrize("P,fused", PATHS)
@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_constant_values_are_returned(idx, P, fused):
    dtype, Hq, Hkv, D, BS, lens = SHAPES[idx]
    case = _case(dtype, Hq, Hkv, D, BS, lens, seed=400 + idx)
    c = np.float32(-1.3125)  # exact in bf16
    cv = _encode(np.full(D, c), dtype)
    for b in range(len(lens)):
        for g in range(Hkv):
            for blk, s in _cached_slots(case, b):
                case.v_cache[blk, g, s] = cv
            case.v_new[b, g] = cv
    got = _run(case, P, fused)
    if dtype == "bf16":
        tol = (2.0 ** -8 + 2.0 ** -8 + 1e-5) * abs(float(c))
    else:
        tol = 1e-5 * abs(float(c))
    err = np.abs(got - float(c))
    assert np.all(np.isfinite(got)), "non-finite output"
    assert np.all(err <= tol), (f"{dtype} {SHAPES[idx]} P={P} fused={fused}: max |out - c| {err.max():.3g} "
                                f"beyond {tol:.3g}")
    log(f"[gpu] constant values {SHAPES[idx]} P={P} fused={fused}: max |out - c| {err.max():.3g}")
