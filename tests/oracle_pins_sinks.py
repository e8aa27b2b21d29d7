"""Pins for the sinks / sliding-window oracle (``oracle.sinks_window``).

Each ``pin_sw_*`` takes the module (or a mutated copy of its source) and raises AssertionError
when it disagrees with a fact that does not come from it:

* the 40-digit brute force (``oracle.brute_force.brute_decode_attention_sinks``);
* the already-pinned plain oracle, on the special cases that reduce to it (no sink, a window at
  least as long as the context, a sink far below every score);
* closed forms: one key with a sink, a window of one, identical keys, a sink far above every
  score;
* the window as truncation: the last W tokens copied into a fresh pool through explicit flat
  offsets, then the plain oracle;
* split-K: merged partitions equal the unsplit result, and with identical keys each partition's
  l_j is exactly its token count, which fixes the partition boundaries under the window.
"""

from __future__ import annotations

import math

import numpy as np

import oracle.paged_attention as plain
from oracle.brute_force import brute_decode_attention_sinks
from tests.oracle_pins import _bf16_bits, _flat_scatter, _rand_case, _values_torch


def _sinks(rng, Hq, dtype, scale=2.0):
    x = (rng.standard_normal(Hq) * scale).astype(np.float32)
    return _bf16_bits(x) if dtype == "bf16" else x


def _sink_vals(s, dtype):
    return _values_torch(np.asarray(s), dtype).numpy()


def pin_sw_brute_force(sw):
    rng = np.random.default_rng(4321)
    for dtype in ("bf16", "f32"):
        for (B, Hq, Hkv, D, BS, lens), window in [((2, 4, 2, 8, 4, [7, 13]), 3), ((1, 3, 1, 5, 2, [1]), 1),
                                                  ((2, 2, 2, 4, 8, [20, 9]), 16), ((2, 4, 1, 6, 4, [0, 11]), 0),
                                                  ((1, 2, 1, 4, 4, [9]), 9), ((1, 2, 2, 4, 4, [12]), 5)]:
            c = _rand_case(rng, B, Hq, Hkv, D, BS, lens, dtype)
            scale = 1.0 / math.sqrt(D)
            for sinks in (None, _sinks(rng, Hq, dtype)):
                out = sw.paged_decode_attention_sinks(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, BS, dtype,
                                                      sinks=sinks, window=window)
                qv = _values_torch(c["q"], dtype).tolist()
                kf = _values_torch(c["k"], dtype).reshape(-1).tolist()
                vf = _values_torch(c["v"], dtype).reshape(-1).tolist()
                sv = None if sinks is None else _sink_vals(sinks, dtype).tolist()
                ref = brute_decode_attention_sinks(qv, kf, vf, c["bt"].tolist(), c["lens"].tolist(), scale, Hkv, BS,
                                                   D, sv, window)
                ref = np.array([[[float(x) for x in row] for row in b] for b in ref])
                assert np.allclose(out, ref, rtol=0, atol=1e-12), (dtype, window, np.abs(out - ref).max())


def pin_sw_reduces_to_plain(sw):
    rng = np.random.default_rng(77)
    c = _rand_case(rng, 3, 8, 2, 16, 4, [5, 0, 23], "bf16")
    scale = 0.25
    ref = plain.paged_decode_attention(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, 4, "bf16")
    for window in (0, 23, 24, 1000):
        out = sw.paged_decode_attention_sinks(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, 4, "bf16",
                                              sinks=None, window=window)
        assert np.allclose(out, ref, rtol=0, atol=1e-14), window
    # A sink far below every score changes nothing (its weight underflows against the max score).
    low = _bf16_bits(np.full(8, -1.0e4, np.float32))
    out = sw.paged_decode_attention_sinks(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, 4, "bf16",
                                          sinks=low, window=0)
    assert np.allclose(out, ref, rtol=0, atol=1e-14)


def pin_sw_closed_forms(sw):
    rng = np.random.default_rng(5)
    D, BS = 8, 4
    scale = 1.0 / math.sqrt(D)
    # One key with a sink: out = V_0 / (1 + e^(sigma - s_0)).
    c = _rand_case(rng, 1, 2, 1, D, BS, [1], "f32")
    sig = np.array([0.75, -1.5], np.float32)
    out = sw.paged_decode_attention_sinks(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, BS, "f32", sinks=sig)
    k0 = c["ks"][0][0, 0].astype(np.float64)
    v0 = c["vs"][0][0, 0].astype(np.float64)
    for h in range(2):
        s0 = scale * float(np.dot(c["q"][0, h].astype(np.float64), k0))
        exp = v0 / (1.0 + math.exp(float(sig[h]) - s0))
        assert np.allclose(out[0, h], exp, rtol=0, atol=1e-14), h
    # A window of one: the last token alone (exactly V_{L-1} without a sink).
    c = _rand_case(rng, 1, 2, 1, D, BS, [11], "f32")
    vl = c["vs"][0][0, 10].astype(np.float64)
    kl = c["ks"][0][0, 10].astype(np.float64)
    out = sw.paged_decode_attention_sinks(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, BS, "f32", window=1)
    assert np.array_equal(out[0, 0], vl) and np.array_equal(out[0, 1], vl)
    out = sw.paged_decode_attention_sinks(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, BS, "f32", sinks=sig,
                                          window=1)
    for h in range(2):
        sl = scale * float(np.dot(c["q"][0, h].astype(np.float64), kl))
        assert np.allclose(out[0, h], vl / (1.0 + math.exp(float(sig[h]) - sl)), rtol=0, atol=1e-14)
    # Identical keys under a window W with a sink: out = mean(V over the window) * W e^s / (W e^s + e^sigma).
    L, W = 14, 6
    c = _rand_case(rng, 1, 1, 1, D, BS, [L], "f32")
    key = rng.standard_normal(D).astype(np.float32)
    ks = np.repeat(key[None, None, :], L, axis=1)
    k_pool = _flat_scatter(ks, c["bt"][0], c["NB"], BS, np.float32("nan"))
    sig1 = np.array([0.3], np.float32)
    out = sw.paged_decode_attention_sinks(c["q"], k_pool, c["v"], c["bt"], c["lens"], scale, BS, "f32", sinks=sig1,
                                          window=W)
    s = scale * float(np.dot(c["q"][0, 0].astype(np.float64), key.astype(np.float64)))
    mean_v = c["vs"][0][0, L - W:].astype(np.float64).mean(axis=0)
    frac = W * math.exp(s) / (W * math.exp(s) + math.exp(float(sig1[0])))
    assert np.allclose(out[0, 0], mean_v * frac, rtol=0, atol=1e-13)
    # A sink far above every score takes all the weight.
    big = np.array([1.0e4], np.float32)
    out = sw.paged_decode_attention_sinks(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, BS, "f32", sinks=big)
    assert np.all(np.abs(out) < 1e-300)
    # No context: zeros, sink or not.
    c = _rand_case(rng, 2, 2, 1, D, BS, [0, 3], "f32")
    out = sw.paged_decode_attention_sinks(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, BS, "f32", sinks=sig,
                                          window=2)
    assert np.array_equal(out[0], np.zeros((2, D)))


def pin_sw_window_is_truncation(sw):
    rng = np.random.default_rng(11)
    BS, D, Hq, Hkv = 4, 8, 4, 2
    scale = 0.3
    for L, W in [(19, 5), (19, 8), (8, 3), (30, 17)]:
        c = _rand_case(rng, 1, Hq, Hkv, D, BS, [L], "bf16")
        out = sw.paged_decode_attention_sinks(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, BS, "bf16",
                                              window=W)
        # The last W tokens, copied into a fresh pool at new positions 0..W-1 via flat offsets.
        tail_k = c["ks"][0][:, L - W:, :]
        tail_v = c["vs"][0][:, L - W:, :]
        nblk = (W + BS - 1) // BS
        ids = list(rng.permutation(nblk + 2)[:nblk])
        nan = np.uint16(0x7FC0)
        kp = _flat_scatter(tail_k, ids, nblk + 2, BS, nan)
        vp = _flat_scatter(tail_v, ids, nblk + 2, BS, nan)
        bt = np.array([ids], np.int32)
        ref = plain.paged_decode_attention(c["q"], kp, vp, bt, np.array([W], np.int32), scale, BS, "bf16")
        assert np.allclose(out, ref, rtol=0, atol=1e-14), (L, W)


def pin_sw_split_merge(sw):
    rng = np.random.default_rng(21)
    BS, D, Hq, Hkv = 4, 8, 4, 2
    scale = 0.35
    c = _rand_case(rng, 3, Hq, Hkv, D, BS, [37, 9, 64], "bf16")
    sinks = _sinks(rng, Hq, "bf16")
    for window in (0, 1, 7, 20, 100):
        for P in (4, 8, 12):
            ref = sw.paged_decode_attention_sinks(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, BS, "bf16",
                                                  sinks=sinks, window=window)
            out, _ = sw.split_paged_decode_attention_sinks(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, BS,
                                                           "bf16", P, sinks=sinks, window=window)
            assert np.allclose(out, ref, rtol=0, atol=1e-12), (window, P)
    # Identical keys: every weight inside a partition is exactly 1, so l_j counts its tokens.
    L = 29
    c = _rand_case(rng, 1, 2, 1, D, BS, [L], "f32")
    key = rng.standard_normal(D).astype(np.float32)
    k_pool = _flat_scatter(np.repeat(key[None, None, :], L, axis=1), c["bt"][0], c["NB"], BS, np.float32("nan"))
    for window, P in [(0, 8), (13, 8), (5, 4), (16, 8), (29, 12), (1, 4)]:
        _, stats = sw.split_paged_decode_attention_sinks(c["q"], k_pool, c["v"], c["bt"], c["lens"], scale, BS, "f32",
                                                         P, window=window)
        t0 = L - window if 0 < window < L else 0
        j0, o, m, l = stats[0][0]
        assert j0 == t0 // P, (window, P, j0)
        expect = [min((j + 1) * P, L) - max(j * P, t0) for j in range(t0 // P, (L + P - 1) // P)]
        assert np.array_equal(l, np.array(expect, np.float64)), (window, P, l, expect)


SINK_PINS = [pin_sw_brute_force, pin_sw_reduces_to_plain, pin_sw_closed_forms, pin_sw_window_is_truncation,
             pin_sw_split_merge]
