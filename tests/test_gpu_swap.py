"""KV block swap-out / swap-in (xs_kv_swap_out / xs_kv_swap_in) against the swap oracle, bit for
bit (needs an MI355X).

Random pools and pinned host swap spaces; pair lists with valid, distinct destinations mixed
with out-of-range entries (skipped); bf16 and fp32; a round trip through host memory into other
blocks; a side stream; and a Qwen3-8B-shaped list of 4096 blocks (256 MB each way).
"""

import numpy as np
import pytest
import torch

import oracle.swap as oswap
import paged_kv_decode_xs_amd as xs
from tests.gpu_common import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _library():
    xs.load_library()
    torch.cuda.init()
    yield


def _bits(rng, shape, dtype):
    if dtype == "bf16":
        return rng.integers(0, 65536, shape, dtype=np.uint16)
    return rng.standard_normal(shape).astype(np.float32)


def _to_dev(a, dtype):
    t = torch.from_numpy(a.view(np.int16) if dtype == "bf16" else a)
    t = t.view(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def _to_pinned(a, dtype):
    t = torch.from_numpy(a.view(np.int16).copy() if dtype == "bf16" else a.copy())
    t = t.view(torch.bfloat16) if dtype == "bf16" else t
    p = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    p.copy_(t)
    return p


def _host_bits(t, dtype):
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _dev_bits(t, dtype):
    return _host_bits(t.cpu(), dtype)


def _pairs(rng, n_valid, n_src, n_dst, junk=6):
    src = rng.choice(n_src, n_valid, replace=False).astype(np.int32)
    dst = rng.choice(n_dst, n_valid, replace=False).astype(np.int32)
    bad_src = np.array([-1, n_src, n_src + 5, 0, 1, -7][:junk], np.int32)
    bad_dst = np.array([0, 1, 2, -1, n_dst, n_dst + 100][:junk], np.int32)
    # Junk pairs have an out-of-range index on one side, so they never land on a valid destination.
    src = np.concatenate([src, bad_src])
    dst = np.concatenate([dst, bad_dst])
    perm = rng.permutation(len(src))
    return src[perm], dst[perm]


@pytest.mark.parametrize("dtype,Hkv,BS,D", [("bf16", 8, 16, 128), ("f32", 2, 16, 64), ("bf16", 12, 32, 64)])
def test_swap_out_and_in_match_oracle(dtype, Hkv, BS, D):
    rng = np.random.default_rng(hash((dtype, Hkv, BS, D)) % 1000)
    NB, S = 300, 200
    log(f"[gpu] swap {dtype} Hkv={Hkv} BS={BS} D={D} NB={NB} S={S}")
    k, v = _bits(rng, (NB, Hkv, BS, D), dtype), _bits(rng, (NB, Hkv, BS, D), dtype)
    kh0, vh0 = _bits(rng, (S, Hkv, BS, D), dtype), _bits(rng, (S, Hkv, BS, D), dtype)
    kc, vc = _to_dev(k, dtype), _to_dev(v, dtype)
    kh, vh = _to_pinned(kh0, dtype), _to_pinned(vh0, dtype)
    src, dst = _pairs(rng, 150, NB, S)
    xs.xs_kv_swap_out(kc, vc, kh, vh, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    ek, ev = oswap.swap_out(k, v, kh0, vh0, src, dst)
    assert np.array_equal(_host_bits(kh, dtype).view(np.uint8), ek.view(np.uint8))
    assert np.array_equal(_host_bits(vh, dtype).view(np.uint8), ev.view(np.uint8))
    # Swap in from the (now updated) host space into other pool blocks.
    src2, dst2 = _pairs(rng, 120, S, NB)
    xs.xs_kv_swap_in(kh, vh, kc, vc, torch.from_numpy(src2).cuda(), torch.from_numpy(dst2).cuda())
    torch.cuda.synchronize()
    ek2, ev2 = oswap.swap_in(ek, ev, k, v, src2, dst2)
    assert np.array_equal(_dev_bits(kc, dtype).view(np.uint8), ek2.view(np.uint8))
    assert np.array_equal(_dev_bits(vc, dtype).view(np.uint8), ev2.view(np.uint8))


def test_round_trip_on_a_side_stream():
    rng = np.random.default_rng(9)
    NB, S, shape = 64, 32, (8, 16, 128)
    k, v = _bits(rng, (NB,) + shape, "bf16"), _bits(rng, (NB,) + shape, "bf16")
    kc, vc = _to_dev(k, "bf16"), _to_dev(v, "bf16")
    kh = torch.empty((S,) + shape, dtype=torch.bfloat16, pin_memory=True)
    vh = torch.empty((S,) + shape, dtype=torch.bfloat16, pin_memory=True)
    blocks = rng.choice(NB, 20, replace=False).astype(np.int32)
    slots = np.arange(20, dtype=np.int32)
    targets = np.setdiff1d(np.arange(NB), blocks)[:20].astype(np.int32)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        xs.xs_kv_swap_out(kc, vc, kh, vh, torch.from_numpy(blocks).cuda(), torch.from_numpy(slots).cuda(), stream=side)
        xs.xs_kv_swap_in(kh, vh, kc, vc, torch.from_numpy(slots).cuda(), torch.from_numpy(targets).cuda(), stream=side)
    side.synchronize()
    got = _dev_bits(kc, "bf16")
    assert np.array_equal(got[targets], k[blocks]) and np.array_equal(_dev_bits(vc, "bf16")[targets], v[blocks])
    others = np.setdiff1d(np.arange(NB), targets)
    assert np.array_equal(got[others], k[others])


def test_large_list_qwen_shape():
    rng = np.random.default_rng(10)
    NB, S, n, shape = 6000, 4096, 4096, (8, 16, 128)
    k = torch.randint(-32768, 32767, (NB,) + shape, dtype=torch.int16, device="cuda")
    v = torch.randint(-32768, 32767, (NB,) + shape, dtype=torch.int16, device="cuda")
    kc, vc = k.view(torch.bfloat16), v.view(torch.bfloat16)
    kh = torch.empty((S,) + shape, dtype=torch.bfloat16, pin_memory=True)
    vh = torch.empty((S,) + shape, dtype=torch.bfloat16, pin_memory=True)
    src = rng.choice(NB, n, replace=False).astype(np.int32)
    dst = rng.permutation(S)[:n].astype(np.int32)
    xs.xs_kv_swap_out(kc, vc, kh, vh, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    kk = k.cpu().numpy()
    assert np.array_equal(kh.view(torch.int16).numpy()[dst], kk[src])
    assert np.array_equal(vh.view(torch.int16).numpy()[dst], v.cpu().numpy()[src])
