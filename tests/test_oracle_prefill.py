"""Pins of the chunked-prefill oracle (CPU): torch SDPA with an explicit bottom-right causal mask,
the pinned naive causal attention, the pinned decode oracle at the last row, the 40-digit brute
force row by row, explicit flat-offset appends, zero rows past the chunk, chunking invariance;
for the variant with sinks and a sliding window: the 40-digit brute force with sinks row by row,
the pinned decode-with-sinks oracle at every row, the plain prefill where the two coincide, and
closed forms for a window of one; and planted mistakes that the pins must catch."""

import inspect
import math
import types

import numpy as np
import pytest
import torch

import oracle.paged_attention as plain
import oracle.prefill as prefill_mod
import oracle.sinks_window as sinks_mod
from oracle.brute_force import brute_decode_attention, brute_decode_attention_sinks
from tests.oracle_pins import _bf16_bits, _rand_case, _values_torch
from tests.oracle_pins_sinks import _sink_vals, _sinks


def _case(rng, lens_total, starts, C, Hq=4, Hkv=2, D=8, BS=4, dtype="bf16"):
    """Pools holding each sequence's first lens_total[b] tokens; chunk rows are the tokens
    start..start+n-1 (already in the pool, as after the append) and q is random."""
    c = _rand_case(rng, len(lens_total), Hq, Hkv, D, BS, lens_total, dtype)
    B = len(lens_total)
    q = rng.standard_normal((B, Hq, C, D)).astype(np.float32)
    c["qc"] = _bf16_bits(q) if dtype == "bf16" else q
    c["starts"] = np.array(starts, np.int32)
    c["n"] = np.array([L - s for L, s in zip(lens_total, starts)], np.int32)
    return c


def pin_sdpa_bottom_right(po):
    rng = np.random.default_rng(3)
    for dtype in ("bf16", "f32"):
        c = _case(rng, [13, 20, 6], [5, 0, 2], 20, dtype=dtype)
        scale = 0.4
        out = po.paged_prefill_attention(c["qc"], c["k"], c["v"], c["bt"], c["starts"], c["n"], scale, 4, dtype)
        for b in range(3):
            s0, n = int(c["starts"][b]), int(c["n"][b])
            L = s0 + n
            qv = _values_torch(c["qc"][b], dtype)[:, :n]          # [Hq, n, D]
            kv = _values_torch(c["ks"][b], dtype)                  # [Hkv, L, D]
            vv = _values_torch(c["vs"][b], dtype)
            mask = torch.arange(L)[None, :] <= (s0 + torch.arange(n))[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qv, kv, vv, attn_mask=mask, scale=scale,
                                                                   enable_gqa=True).numpy()
            assert np.allclose(out[b, :, :n], ref, rtol=0, atol=1e-12), (dtype, b, np.abs(out[b, :, :n] - ref).max())


def pin_naive_from_zero(po):
    rng = np.random.default_rng(4)
    c = _case(rng, [11], [0], 11, Hq=6, Hkv=3, dtype="f32")
    out = po.paged_prefill_attention(c["qc"], c["k"], c["v"], c["bt"], c["starts"], c["n"], 0.3, 4, "f32")
    ref = plain.naive_causal_attention(c["qc"][0].astype(np.float64), c["ks"][0].astype(np.float64),
                                       c["vs"][0].astype(np.float64), 0.3)
    assert np.allclose(out[0], ref, rtol=0, atol=1e-13)


def pin_last_row_is_decode(po):
    rng = np.random.default_rng(5)
    c = _case(rng, [30, 9, 17], [21, 0, 16], 12, Hq=8, Hkv=2)
    out = po.paged_prefill_attention(c["qc"], c["k"], c["v"], c["bt"], c["starts"], c["n"], 0.35, 4, "bf16")
    lens = c["starts"] + c["n"]
    last_q = np.stack([c["qc"][b, :, int(c["n"][b]) - 1] for b in range(3)])
    dec = plain.paged_decode_attention(last_q, c["k"], c["v"], c["bt"], lens, 0.35, 4, "bf16")
    for b in range(3):
        assert np.allclose(out[b, :, int(c["n"][b]) - 1], dec[b], rtol=0, atol=1e-14)


def pin_brute_force_rows(po):
    rng = np.random.default_rng(6)
    c = _case(rng, [7, 10], [3, 6], 4, Hq=4, Hkv=2, D=5, BS=2)
    scale = 1 / math.sqrt(5)
    out = po.paged_prefill_attention(c["qc"], c["k"], c["v"], c["bt"], c["starts"], c["n"], scale, 2, "bf16")
    kf = _values_torch(c["k"], "bf16").reshape(-1).tolist()
    vf = _values_torch(c["v"], "bf16").reshape(-1).tolist()
    for b in range(2):
        for i in range(int(c["n"][b])):
            qv = _values_torch(c["qc"][b, :, i], "bf16").tolist()
            ref = brute_decode_attention([qv], kf, vf, [c["bt"][b].tolist()], [int(c["starts"][b]) + i + 1], scale,
                                         2, 2, 5)
            ref = np.array([[float(x) for x in row] for row in ref[0]])
            assert np.allclose(out[b, :, i], ref, rtol=0, atol=1e-12), (b, i)


def pin_rows_past_chunk_are_zero_and_chunking(po):
    rng = np.random.default_rng(7)
    c = _case(rng, [26, 12], [0, 0], 26, Hq=4, Hkv=1)
    n_short = np.array([26, 9], np.int32)  # sequence 1: only its first 9 rows are in the chunk
    out = po.paged_prefill_attention(c["qc"], c["k"], c["v"], c["bt"], c["starts"], n_short, 0.5, 4, "bf16")
    assert not out[1, :, 9:].any()
    # Three chunks in turn give the rows of the single chunk.
    for a, b2 in [(0, 10), (10, 19), (19, 26)]:
        part = po.paged_prefill_attention(c["qc"][:1, :, a:], c["k"], c["v"], c["bt"][:1], np.array([a], np.int32),
                                          np.array([b2 - a], np.int32), 0.5, 4, "bf16")
        assert np.allclose(part[0, :, :b2 - a], out[0, :, a:b2], rtol=0, atol=1e-14)


def pin_append_chunk(po):
    rng = np.random.default_rng(8)
    NB, Hkv, BS, D, C = 10, 2, 4, 3, 7
    k = rng.integers(0, 65536, (NB, Hkv, BS, D), dtype=np.uint16)
    v = rng.integers(0, 65536, (NB, Hkv, BS, D), dtype=np.uint16)
    ks = rng.integers(0, 65536, (2, Hkv, C, D), dtype=np.uint16)
    vs = rng.integers(0, 65536, (2, Hkv, C, D), dtype=np.uint16)
    bt = np.array([[4, 9, 1, -1], [0, 7, 3, 8]], np.int32)
    starts, n = np.array([3, 9], np.int32), np.array([7, 2], np.int32)
    ko, vo = po.kv_append_chunk(k, v, ks, vs, bt, starts, n, BS)
    kf, vf = k.reshape(-1).copy(), v.reshape(-1).copy()
    for b in range(2):
        for i in range(int(n[b])):
            p = int(starts[b]) + i
            blk = int(bt[b, p // BS])
            for g in range(Hkv):
                base = ((blk * Hkv + g) * BS + p % BS) * D
                kf[base:base + D] = ks[b, g, i]
                vf[base:base + D] = vs[b, g, i]
    assert np.array_equal(ko.reshape(-1), kf) and np.array_equal(vo.reshape(-1), vf)


def pin_psw_brute_force_rows(po):
    """Every row against the 40-digit brute force with sinks, at context p + 1 and the same window."""
    rng = np.random.default_rng(12)
    scale = 1 / math.sqrt(5)
    for dtype in ("bf16", "f32"):
        for window in (0, 1, 3, 6):
            c = _case(rng, [9, 12], [5, 8], 4, Hq=4, Hkv=2, D=5, BS=2, dtype=dtype)
            kf = _values_torch(c["k"], dtype).reshape(-1).tolist()
            vf = _values_torch(c["v"], dtype).reshape(-1).tolist()
            for sinks in (None, _sinks(rng, 4, dtype)):
                out = po.paged_prefill_attention_sinks(c["qc"], c["k"], c["v"], c["bt"], c["starts"], c["n"], scale,
                                                       2, dtype, sinks=sinks, window=window)
                sv = None if sinks is None else _sink_vals(sinks, dtype).tolist()
                for b in range(2):
                    for i in range(int(c["n"][b])):
                        qv = _values_torch(c["qc"][b, :, i], dtype).tolist()
                        ref = brute_decode_attention_sinks([qv], kf, vf, [c["bt"][b].tolist()],
                                                           [int(c["starts"][b]) + i + 1], scale, 2, 2, 5, sv, window)
                        ref = np.array([[float(x) for x in row] for row in ref[0]])
                        assert np.allclose(out[b, :, i], ref, rtol=0, atol=1e-12), (dtype, window, b, i)


def pin_psw_rows_are_decode_sinks(po):
    """Row i of sequence b is the (pinned) decode with sinks of that query at context start + i + 1."""
    rng = np.random.default_rng(13)
    c = _case(rng, [30, 17, 9], [18, 0, 3], 17, Hq=8, Hkv=2, D=16, BS=4)
    sinks = _sinks(rng, 8, "bf16")
    for window in (0, 5, 16):
        out = po.paged_prefill_attention_sinks(c["qc"], c["k"], c["v"], c["bt"], c["starts"], c["n"], 0.3, 4, "bf16",
                                               sinks=sinks, window=window)
        for b in range(3):
            for i in range(int(c["n"][b])):
                dec = sinks_mod.paged_decode_attention_sinks(c["qc"][b:b + 1, :, i], c["k"], c["v"], c["bt"][b:b + 1],
                                                             np.array([int(c["starts"][b]) + i + 1], np.int32), 0.3,
                                                             4, "bf16", sinks=sinks, window=window)
                assert np.allclose(out[b, :, i], dec[0], rtol=0, atol=1e-13), (window, b, i)
        assert not out[1, :, int(c["n"][1]):].any() and not out[2, :, int(c["n"][2]):].any()


def pin_psw_reduces_to_prefill(po):
    """No sinks with no window, or a window longer than every context, or a sink far below every
    score: the plain causal prefill."""
    rng = np.random.default_rng(14)
    c = _case(rng, [21, 14], [7, 2], 14, Hq=6, Hkv=3, D=8, BS=4, dtype="f32")
    ref = po.paged_prefill_attention(c["qc"], c["k"], c["v"], c["bt"], c["starts"], c["n"], 0.45, 4, "f32")
    low = np.full(6, -3.0e38, np.float32)
    for sinks, window in ((None, 0), (None, 21), (None, 500), (low, 0), (low, 22)):
        out = po.paged_prefill_attention_sinks(c["qc"], c["k"], c["v"], c["bt"], c["starts"], c["n"], 0.45, 4, "f32",
                                               sinks=sinks, window=window)
        assert np.allclose(out, ref, rtol=0, atol=1e-14), (window, sinks is None)


def pin_psw_window_of_one(po):
    """W = 1: a row sees only its own key, so it is V_p; with a sink sigma it is
    V_p / (1 + e^(sigma - s_p)), s_p = scale * q . K_p (K_p, V_p from the contiguous source)."""
    rng = np.random.default_rng(15)
    c = _case(rng, [10, 7], [4, 0], 7, Hq=4, Hkv=2, D=6, BS=4, dtype="f32")
    sinks = _sinks(rng, 4, "f32", scale=1.0)
    scale = 0.7
    plain_out = po.paged_prefill_attention_sinks(c["qc"], c["k"], c["v"], c["bt"], c["starts"], c["n"], scale, 4,
                                                 "f32", window=1)
    sink_out = po.paged_prefill_attention_sinks(c["qc"], c["k"], c["v"], c["bt"], c["starts"], c["n"], scale, 4, "f32",
                                                sinks=sinks, window=1)
    for b in range(2):
        for i in range(int(c["n"][b])):
            p = int(c["starts"][b]) + i
            for h in range(4):
                g = h // 2
                kp = c["ks"][b][g, p].astype(np.float64)
                vp = c["vs"][b][g, p].astype(np.float64)
                sp = scale * float(np.dot(c["qc"][b, h, i].astype(np.float64), kp))
                assert np.array_equal(plain_out[b, h, i], vp), (b, i, h)
                want = vp / (1.0 + math.exp(float(sinks[h]) - sp))
                assert np.allclose(sink_out[b, h, i], want, rtol=1e-14, atol=1e-15), (b, i, h)


PREFILL_PINS = [pin_sdpa_bottom_right, pin_naive_from_zero, pin_last_row_is_decode, pin_brute_force_rows,
                pin_rows_past_chunk_are_zero_and_chunking, pin_append_chunk, pin_psw_brute_force_rows,
                pin_psw_rows_are_decode_sinks, pin_psw_reduces_to_prefill, pin_psw_window_of_one]


@pytest.mark.parametrize("pin", PREFILL_PINS, ids=lambda p: p.__name__)
def test_prefill_pin(pin):
    pin(prefill_mod)


SOURCE = inspect.getsource(prefill_mod)
MUTANTS = {
    "causal_excludes_self": ("paged_prefill_attention", "K[g, :p + 1]", "K[g, :max(p, 1)]"),
    "top_left_alignment": ("paged_prefill_attention", "                p = s0 + i\n", "                p = i\n"),
    "gqa_modulo": ("paged_prefill_attention", "g = h // n_rep", "g = h % Hkv"),
    "v_not_causal": ("paged_prefill_attention", "(w @ V[g, :p + 1])", "(w @ V[g, L - p - 1:])"),
    "append_shifted": ("kv_append_chunk", "            p = s0 + i\n", "            p = s0 + i + 1\n"),
    "append_ignores_chunk_len": ("kv_append_chunk", "for i in range(max(n, 0)):",
                                 "for i in range(k_src.shape[2]):"),
    "unnormalised": ("paged_prefill_attention", "/ w.sum()", ""),
    "sw_window_off_by_one": ("window_first", "max(0, p + 1 - window)", "max(0, p - window)"),
    "sw_window_from_chunk_start": ("paged_prefill_attention_sinks", "                t0 = window_first(p, window)\n",
                                   "                t0 = window_first(s0, window)\n"),
    "sw_sink_dropped": ("paged_prefill_attention_sinks", "/ den", "/ w.sum()"),
    "sw_sink_of_kv_head": ("paged_prefill_attention_sinks", "np.exp(sig[h] - M)", "np.exp(sig[g] - M)"),
    "sw_sink_unshifted": ("paged_prefill_attention_sinks", "np.exp(sig[h] - M)", "np.exp(sig[h])"),
    "sw_gqa_modulo": ("paged_prefill_attention_sinks", "g = h // n_rep", "g = h % Hkv"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_prefill_mutant_is_caught(name):
    func, old, new = MUTANTS[name]
    start = SOURCE.index(f"\ndef {func}(")
    end = SOURCE.find("\ndef ", start + 1)
    end = len(SOURCE) if end < 0 else end
    body = SOURCE[start:end]
    assert body.count(old) == 1, name
    src = SOURCE[:start] + body.replace(old, new) + SOURCE[end:]
    src = src.replace("from .paged_attention import", "from oracle.paged_attention import")
    mod = types.ModuleType(f"prefill_mutant_{name}")
    exec(compile(src, name, "exec"), mod.__dict__)
    failed = []
    for pin in PREFILL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001
            failed.append(type(e).__name__)
    assert failed, f"mutant {name} passed every pin"
