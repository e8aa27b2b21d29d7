"""The seeded input generator (CPU only): determinism, sizes, placement and poison."""

import math

import numpy as np
import pytest
import torch

import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32),
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8), 3.0e38, 1e-40], np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


@pytest.mark.parametrize("name", ["gpt2_fp32_ctx32", "gpt2_bf16_b8", "qwen3_8b_b1_ctx4096"])
def test_case_layout_and_poison(name):
    w = wl.WORKLOADS[name]
    c = wl.make_case(w)
    c2 = wl.make_case(w)
    for a, b in [(c.q, c2.q), (c.k_cache, c2.k_cache), (c.v_new, c2.v_new), (c.block_tables, c2.block_tables)]:
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    B, Hq, Hkv, D, BS = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    assert c.q.shape == (B, Hq, D) and c.k_new.shape == (B, Hkv, D)
    assert c.k_cache.shape == (c.num_blocks, Hkv, BS, D)
    assert c.block_tables.shape == (B, w.max_blocks_per_seq)
    isnan = lambda a: np.isnan(a) if a.dtype == np.float32 else ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)  # noqa
    owned = np.zeros(c.k_cache.shape, bool)
    used = set()
    for b in range(B):
        L = int(c.context_lens[b])
        n = -(-L // BS)
        ids = c.block_tables[b, :n]
        assert np.all(c.block_tables[b, n:] == -1)
        used.update(ids.tolist())
        for t in range(L - 1):
            owned[ids[t // BS], :, t % BS, :] = True
    assert len(used) == sum(-(-int(L) // BS) for L in c.context_lens)  # no block shared
    assert not np.any(isnan(c.k_cache) & owned) and not np.any(isnan(c.v_cache) & owned)
    assert np.all(isnan(c.k_cache)[~owned]) and np.all(isnan(c.v_cache)[~owned])


def test_sizes_of_big_workloads():
    # Layouts only (no values), checked against the sizes the workloads are quoted with.
    w4 = wl.WORKLOADS["qwen3_8b_b64"]
    lay = wl.make_layout(w4, np.random.default_rng(w4.seed))
    L = lay.context_lens
    assert L.shape == (64,) and L.min() >= 128 and L.max() <= 8192
    need = int(lay.blocks_per_seq.sum())
    assert lay.num_blocks == math.ceil(1.25 * need)
    w5 = wl.WORKLOADS["qwen3_8b_b4_long"]
    lay5 = wl.make_layout(w5, np.random.default_rng(w5.seed))
    assert lay5.num_blocks == 6400 and list(lay5.context_lens) == [8192, 16384, 24576, 32768]
    w3 = wl.WORKLOADS["qwen3_8b_b1_ctx4096"]
    assert wl.make_layout(w3, np.random.default_rng(w3.seed)).num_blocks == 320


def test_rmsnorm_rows():
    c = wl.make_case(wl.WORKLOADS["qwen3_8b_b1_ctx4096"].with_(ctx=("fixed", [40]), max_blocks_per_seq=4))
    q = torch.from_numpy(c.q.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    # Each row is x * gain with unit-RMS x and gain ~ N(1, 0.1): row RMS stays near 1.
    rms = np.sqrt((q ** 2).mean(-1))
    assert np.all(np.abs(rms - 1) < 0.2)
    # All rows share one gain vector, so the per-column RMS over rows deviates coherently.
    col = np.sqrt((q.reshape(-1, q.shape[-1]) ** 2).mean(0))
    assert col.std() > 0.03


# Chunked-prefill inputs.
from workloads.prefill import PREFILL_WORKLOADS, PrefillWorkload, make_prefill_case  # noqa: E402


def _tiny_prefill(**kw):
    a = dict(name="t", description="", dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
             chunk=20, start_pos=(0, 13, 40), chunk_lens=(20, 7, 0), max_blocks_per_seq=5, seed=1)
    a.update(kw)
    return PrefillWorkload(**a)


def test_prefill_case_is_seeded_and_poisons_uncached_slots():
    w = _tiny_prefill()
    a, b = make_prefill_case(w), make_prefill_case(w)
    for f in ("q", "k_src", "v_src", "k_cache", "v_cache", "block_tables"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    BS = w.block_size
    for s in range(w.batch):
        s0, n = int(a.start_pos[s]), int(a.chunk_lens[s])
        nblk = -(-(s0 + n) // BS)
        for p in range(nblk * BS):
            blk = int(a.block_tables[s, p // BS])
            row = a.k_cache[blk, :, p % BS, :]
            assert (row == 0x7FC0).all() == (p >= s0), (s, p)
        assert (a.block_tables[s, nblk:] == -1).all()
    used = set(a.block_tables[a.block_tables >= 0].tolist())
    assert len(used) == int(sum(-(-(s0 + n) // BS) for s0, n in zip(w.start_pos, w.chunk_lens)))
    for blk in set(range(a.k_cache.shape[0])) - used:
        assert (a.k_cache[blk] == 0x7FC0).all()


def test_prefill_key_visits_and_flops():
    w = _tiny_prefill()
    brute = sum(s0 + i + 1 for s0, n in zip(w.start_pos, w.chunk_lens) for i in range(n))
    assert w.key_visits() == brute
    assert w.attention_flops() == 4 * 64 * 4 * brute
    assert w.append_bytes() == 2 * 2 * 27 * 2 * 64 * 2


def test_prefill_key_visits_with_a_window_and_sinks_drawn_last():
    w = _tiny_prefill(window=9)
    brute = sum(len(range(max(0, s0 + i + 1 - 9), s0 + i + 1)) for s0, n in zip(w.start_pos, w.chunk_lens)
                for i in range(n))
    assert w.key_visits() == brute
    a, b = make_prefill_case(_tiny_prefill()), make_prefill_case(_tiny_prefill(sinks=True))
    assert a.sinks is None and b.sinks.shape == (4,) and b.sinks.dtype == np.uint16
    for f in ("q", "k_src", "v_src", "k_cache", "v_cache", "block_tables"):
        assert np.array_equal(getattr(a, f), getattr(b, f))  # the sinks do not move the other draws


def test_prefill_workloads_are_valid():
    for w in PREFILL_WORKLOADS.values():
        assert w.batch == len(w.chunk_lens)
        assert max(s + n for s, n in zip(w.start_pos, w.chunk_lens)) <= w.max_blocks_per_seq * w.block_size


def test_prefill_case_rejects_bad_ranges():
    with pytest.raises(ValueError):
        make_prefill_case(_tiny_prefill(chunk_lens=(21, 7, 0)))
    with pytest.raises(ValueError):
        make_prefill_case(_tiny_prefill(start_pos=(0, 13, 90)))


# Host-side partition-size rule of the decode step helper.
from paged_kv_decode_xs_amd.step import suggest_partition_size  # noqa: E402


def test_suggested_partition_sizes_match_the_measured_best():
    base = wl.WORKLOADS["qwen3_8b_b64"]
    for batch, seed, want in ((64, 3, 1024), (128, 5, 2048), (256, 6, 4096)):
        w = base.with_(batch=batch, seed=seed)
        lens = wl.make_layout(w, np.random.default_rng(w.seed)).context_lens
        assert suggest_partition_size(lens, w.num_kv_heads, w.block_size) == want, batch
    tp = wl.WORKLOADS["qwen3_8b_b64_tp8_share"]
    lens = wl.make_layout(tp, np.random.default_rng(tp.seed)).context_lens
    assert suggest_partition_size(lens, tp.num_kv_heads, tp.block_size) == 128
    # One 4096-token Qwen3-8B sequence: 64 measured fastest (11.32 us per step against 11.81 at 128).
    one = wl.WORKLOADS["qwen3_8b_b1_ctx4096"]
    assert suggest_partition_size([4096], one.num_kv_heads, one.block_size) == 64 == one.partition_size


def test_suggested_partition_size_edges():
    assert suggest_partition_size([], 8) == 64
    assert suggest_partition_size([0, 0], 8) == 64
    assert suggest_partition_size([10], 8, block_size=32) == 64
    assert suggest_partition_size([100000] * 64, 8, num_cus=1) >= 100000 // 2  # capped near the longest
    for bs in (8, 16, 32):
        p = suggest_partition_size([5000] * 300, 8, block_size=bs)
        assert p % bs == 0 and p & (p - 1) == 0
    with pytest.raises(ValueError):
        suggest_partition_size([1], 0)
