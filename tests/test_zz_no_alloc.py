"""xs_paged_attn_decode_append_noalloc (partials in the library's own device scratch) against the
same step with caller-owned partials (xs_paged_attn_decode_append + xs_paged_attn_reduce), through
the C ABI: two calls in a row, the second on a smaller input (the scratch then still holds the
first call's partials), each bitwise equal to the caller-buffer step in `out` and in the pools,
and within tolerance of the fp64 oracle (needs an MI355X)."""

import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_common import TOL, OracleResult, as_f64, assert_close, log
from workloads.device import case_to_device, to_numpy_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _library():
    import paged_kv_decode_xs_amd as xs

    xs.load_library()
    torch.cuda.init()
    yield


def _case(batch, lens, seed):
    w = wl.WORKLOADS["qwen3_8b_b64"].with_(batch=batch, ctx=("fixed", lens), max_blocks_per_seq=256)
    return wl.make_case(w, seed=seed)


def _caller_buffers(case, P, NP):
    import paged_kv_decode_xs_amd as xs

    w = case.workload
    dev = case_to_device(case)
    step = xs.DecodeStep(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                         dev["k_new"], dev["v_new"], w.scale, partition_size=P,
                         max_context_len=NP * P if P else None, fused=True)
    step.run()
    torch.cuda.synchronize()
    return step.out.clone(), dev


def _noalloc(case, P, NP):
    import paged_kv_decode_xs_amd as xs

    w = case.workload
    dev = case_to_device(case)
    out = torch.full(tuple(case.q.shape), float("nan"), dtype=torch.bfloat16, device="cuda")
    xs.xs_paged_attn_decode_append_noalloc(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                                           dev["block_tables"], dev["context_lens"], w.scale, out,
                                           partition_size=P, max_partitions=NP)
    torch.cuda.synchronize()
    return out, dev


@pytest.mark.parametrize("P", [256, 0])
def test_noalloc_matches_caller_buffers_on_two_calls(P):
    calls = [(12, [3000, 1, 700, 0, 4096, 17, 2500, 1024, 333, 4000, 128, 65], 11),  # first: the larger input
             (3, [900, 5, 260], 12)]                                                 # then a smaller one
    for i, (batch, lens, seed) in enumerate(calls):
        case = _case(batch, lens, seed)
        NP = -(-max(lens) // P) if P else 0
        log(f"[gpu] noalloc call {i}: batch={batch} P={P} max_partitions={NP} lens={lens}")
        ref_out, ref_dev = _caller_buffers(case, P, NP)
        out, dev = _noalloc(case, P, NP)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"call {i}: out differs"
        for name in ("k_cache", "v_cache"):
            assert np.array_equal(to_numpy_bits(dev[name]), to_numpy_bits(ref_dev[name])), f"call {i}: {name}"
        assert_close(as_f64(out), OracleResult(case).out, *TOL["bf16"], f"noalloc call {i} vs oracle")
