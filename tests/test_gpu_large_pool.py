"""Pools larger than 32-bit offsets can address (needs an MI355X; up to 32 GiB of device memory).

The kernels address a pool element as ((block * num_kv_heads + g) * block_size + slot) * head_dim
+ d, which for a pool of a few hundred thousand blocks passes 2^31 and 2^32 elements (8 and 16 GiB
of bf16): an intermediate held in 32 bits would wrap there and read or write a block near the
start of the pool instead. Here a small case's blocks are moved to the top of a pool sized so that
every used block lies past element 2^32, the rest of the pool is NaN, and the block tables are
renumbered to match. The results must equal those of the same case in its own small pool (checked
against the oracle at the usual bars), the appended slots must land in the moved blocks bit for
bit, and the untouched part of the pool must still be NaN. Covered: the matrix-core decode (split
and unsplit, separate and fused append), the generic decode (fp32, and bf16 with block_size 8),
the sliding-window decode with sinks, chunked prefill (append and attention, unsplit and split)
and the block swap in both directions.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_xs_amd as xs
import workloads as wl
from oracle import swap as oswap
from tests.gpu_common import TOL, OracleResult, as_f64, assert_close, check_rounding_bound, log, run_step
from tests.rounding_bound import assert_rounding_bound, decode_spread, prefill_spread
from workloads.device import case_to_device, to_numpy_bits, to_torch
from workloads.prefill import PrefillWorkload, make_prefill_case

pytestmark = pytest.mark.gpu

ELEMS_PAST = 2 ** 32  # every moved block starts at or past this element of the pool


@pytest.fixture(scope="module", autouse=True)
def _library():
    xs.load_library()
    torch.cuda.init()
    yield


@pytest.fixture(autouse=True)
def _release():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class BigPools:
    """The pools of a case moved to the top of pools of ``total`` blocks (block j -> total - 1 - j)."""

    def __init__(self, k_small: torch.Tensor, v_small: torch.Tensor):
        nb, hkv, bs, d = k_small.shape
        per_block = hkv * bs * d
        self.low = -(-ELEMS_PAST // per_block)  # blocks below the moved ones
        self.total = self.low + nb + 3
        self.nb = nb
        self.ids = torch.arange(self.total - 1, self.total - 1 - nb, -1, dtype=torch.long, device="cuda")
        self.k = torch.full((self.total, hkv, bs, d), float("nan"), dtype=k_small.dtype, device="cuda")
        self.v = torch.full_like(self.k, float("nan"))
        self.k[self.ids] = k_small
        self.v[self.ids] = v_small
        assert int(self.ids.min()) * per_block >= ELEMS_PAST
        log(f"[gpu] large pool: {self.total} blocks of {per_block} elements "
            f"({2 * self.k.numel() * self.k.element_size() / 2**30:.1f} GiB for K+V), moved blocks from "
            f"{int(self.ids.min())}")

    def table(self, bt: np.ndarray) -> torch.Tensor:
        """Block table renumbered into the big pools (entries outside [0, nb) stay as they are)."""
        bt = np.asarray(bt, np.int64)
        ok = (bt >= 0) & (bt < self.nb)
        big = np.where(ok, self.total - 1 - np.where(ok, bt, 0), bt)
        return torch.from_numpy(big.astype(np.int32)).cuda()

    def moved(self, which: str) -> np.ndarray:
        return to_numpy_bits((self.k if which == "k" else self.v)[self.ids])

    def assert_rest_is_nan(self) -> None:
        for t in (self.k, self.v):
            step = 1 << 15
            for a in range(0, self.total - self.nb, step):
                part = t[a:min(a + step, self.total - self.nb)]
                assert bool(torch.isnan(part).all()), f"blocks {a}.. of the big pool were written"


def _decode_case(dtype, Hq, Hkv, D, BS, lens, seed, sinks=False):
    mbps = max(1, -(-max(lens) // BS) + 1)
    w = wl.Workload(name="large_pool", description="", dtype=dtype, batch=len(lens), num_q_heads=Hq,
                    num_kv_heads=Hkv, head_dim=D, block_size=BS, ctx=("fixed", lens), num_blocks=None,
                    max_blocks_per_seq=mbps, values="normal", seed=seed, partition_size=BS, sinks=sinks)
    return wl.make_case(w)


DECODE = [
    # dtype, Hq, Hkv, D, BS, lens
    ("bf16", 32, 8, 128, 16, [1, 300, 2049, 700]),
    ("bf16", 16, 2, 64, 8, [5, 640, 129]),
    ("f32", 8, 2, 128, 16, [1, 257, 1000]),
]


@pytest.mark.parametrize("P,fused", [(0, False), (0, True), (512, False), (512, True)])
@pytest.mark.parametrize("idx", range(len(DECODE)))
def test_decode_past_2e32_elements(idx, P, fused):
    dtype, Hq, Hkv, D, BS, lens = DECODE[idx]
    case = _decode_case(dtype, Hq, Hkv, D, BS, lens, seed=500 + idx)
    w = case.workload
    ref = OracleResult(case, P)
    small = case_to_device(case)
    big = BigPools(small["k_cache"], small["v_cache"])
    dev = dict(small, k_cache=big.k, v_cache=big.v, block_tables=big.table(case.block_tables))
    del small
    step = run_step(dev, w.scale, P, max(lens) if P else None, fused=fused)
    got = as_f64(step.out)
    assert_close(got, ref.out, *TOL[dtype], f"large pool {DECODE[idx]} P={P} fused={fused}")
    check_rounding_bound(got, ref, f"large pool {DECODE[idx]} P={P} fused={fused}")
    assert np.array_equal(big.moved("k").view(np.uint8), ref.k_pool.view(np.uint8)), "k pool after append"
    assert np.array_equal(big.moved("v").view(np.uint8), ref.v_pool.view(np.uint8)), "v pool after append"
    big.assert_rest_is_nan()


@pytest.mark.parametrize("P", [0, 512])
def test_windowed_decode_with_sinks_past_2e32_elements(P):
    case = _decode_case("bf16", 64, 8, 64, 16, [1, 100, 1500, 4100], seed=510, sinks=True)
    w = case.workload
    window = 128
    k_pool, v_pool = oracle.kv_append(case.k_cache, case.v_cache, case.k_new, case.v_new, case.block_tables,
                                      case.context_lens, w.block_size)
    ref = oracle.paged_decode_attention_sinks(case.q, k_pool, v_pool, case.block_tables, case.context_lens, w.scale,
                                              w.block_size, w.dtype, sinks=case.sinks, window=window)
    small = case_to_device(case)
    big = BigPools(small["k_cache"], small["v_cache"])
    sinks = torch.from_numpy(case.sinks.view(np.int16).copy()).view(torch.bfloat16).cuda()
    step = xs.DecodeStep(small["q"], big.k, big.v, big.table(case.block_tables), small["context_lens"],
                         small["k_new"], small["v_new"], w.scale, partition_size=P,
                         max_context_len=int(case.context_lens.max()) if P else None, fused=True, sinks=sinks,
                         window=window)
    for t in (step.out, step.part_o, step.part_m, step.part_l):
        if t is not None:
            t.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    got = as_f64(step.out)
    assert_close(got, ref, *TOL["bf16"], f"large pool window+sinks P={P}")
    tau = decode_spread(case.q, k_pool, v_pool, case.block_tables, case.context_lens, w.scale, w.block_size, "bf16",
                        sinks=case.sinks, window=window)
    assert_rounding_bound(got, ref, tau, f"large pool window+sinks P={P}, rounding bound")
    assert np.array_equal(big.moved("k").view(np.uint8), k_pool.view(np.uint8)), "k pool after append"
    assert np.array_equal(big.moved("v").view(np.uint8), v_pool.view(np.uint8)), "v pool after append"
    big.assert_rest_is_nan()


@pytest.mark.parametrize("split", [None, 64])
def test_prefill_past_2e32_elements(split):
    w = PrefillWorkload(name="large_pool", description="", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                        block_size=16, chunk=70, start_pos=(0, 130, 257), chunk_lens=(70, 64, 3),
                        max_blocks_per_seq=24, seed=520)
    case = make_prefill_case(w)
    kp, vp = oracle.kv_append_chunk(case.k_cache, case.v_cache, case.k_src, case.v_src, case.block_tables,
                                    case.start_pos, case.chunk_lens, w.block_size)
    exp = oracle.paged_prefill_attention(case.q, kp, vp, case.block_tables, case.start_pos, case.chunk_lens, w.scale,
                                         w.block_size, "bf16")
    big = BigPools(to_torch(case.k_cache, "bf16").cuda(), to_torch(case.v_cache, "bf16").cuda())
    q = to_torch(case.q, "bf16").cuda()
    bt = big.table(case.block_tables)
    sp, cl = torch.from_numpy(case.start_pos).cuda(), torch.from_numpy(case.chunk_lens).cuda()
    xs.xs_kv_append_chunk(to_torch(case.k_src, "bf16").cuda(), to_torch(case.v_src, "bf16").cuda(), big.k, big.v, bt,
                          sp, cl)
    out = torch.full_like(q, float("nan"))
    if split:
        B, Hq, C, D = q.shape
        NP = xs.num_partitions(bt.shape[1] * w.block_size, split)
        po = torch.full((B, Hq, C, NP, D), float("nan"), dtype=torch.float32, device="cuda")
        pml = torch.full((B, Hq, C, NP, 2), float("nan"), dtype=torch.float32, device="cuda")
        xs.xs_paged_attn_prefill_split(q, big.k, big.v, bt, sp, cl, w.scale, split, out=out, part_o=po, part_ml=pml)
    else:
        xs.xs_paged_attn_prefill(q, big.k, big.v, bt, sp, cl, w.scale, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(big.moved("k").view(np.uint8), kp.view(np.uint8)), "k pool after the chunk append"
    assert np.array_equal(big.moved("v").view(np.uint8), vp.view(np.uint8)), "v pool after the chunk append"
    got = as_f64(out)
    assert_close(got, exp, *TOL["bf16"], f"large pool prefill split={split}")
    tau = prefill_spread(case.q, kp, vp, case.block_tables, case.start_pos, case.chunk_lens, w.scale, w.block_size,
                         "bf16")
    assert_rounding_bound(got, exp, tau, f"large pool prefill split={split}, rounding bound")
    for b, n in enumerate(case.chunk_lens.tolist()):
        assert not got[b, :, n:].any(), f"rows past chunk_lens[{b}] = {n} are not zero"
    big.assert_rest_is_nan()


def test_swap_past_2e32_elements():
    rng = np.random.default_rng(530)
    nb, S, shape = 40, 24, (8, 16, 128)
    k = rng.integers(0, 65536, (nb,) + shape, dtype=np.uint16)
    v = rng.integers(0, 65536, (nb,) + shape, dtype=np.uint16)
    big = BigPools(to_torch(k, "bf16").cuda(), to_torch(v, "bf16").cuda())
    kh0 = rng.integers(0, 65536, (S,) + shape, dtype=np.uint16)
    vh0 = rng.integers(0, 65536, (S,) + shape, dtype=np.uint16)
    kh = torch.empty((S,) + shape, dtype=torch.bfloat16, pin_memory=True)
    vh = torch.empty((S,) + shape, dtype=torch.bfloat16, pin_memory=True)
    kh.copy_(to_torch(kh0, "bf16"))
    vh.copy_(to_torch(vh0, "bf16"))
    # Out: 16 moved blocks to host slots (small-pool ids, renumbered into the big pool).
    src = rng.choice(nb, 16, replace=False).astype(np.int32)
    dst = rng.choice(S, 16, replace=False).astype(np.int32)
    xs.xs_kv_swap_out(big.k, big.v, kh, vh, big.table(src), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    ek, ev = oswap.swap_out(k, v, kh0, vh0, src, dst)
    assert np.array_equal(kh.view(torch.int16).numpy().view(np.uint16), ek)
    assert np.array_equal(vh.view(torch.int16).numpy().view(np.uint16), ev)
    # In: host slots to other moved blocks.
    src2 = rng.choice(S, 12, replace=False).astype(np.int32)
    dst2 = rng.choice(nb, 12, replace=False).astype(np.int32)
    xs.xs_kv_swap_in(kh, vh, big.k, big.v, torch.from_numpy(src2).cuda(), big.table(dst2))
    torch.cuda.synchronize()
    ek2, ev2 = oswap.swap_in(ek, ev, k, v, src2, dst2)
    assert np.array_equal(big.moved("k"), ek2)
    assert np.array_equal(big.moved("v"), ev2)
    big.assert_rest_is_nan()
