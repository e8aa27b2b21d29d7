"""Pins for the fp64 oracle: checks against facts that do not come from the oracle itself.

Each ``pin_*`` takes an oracle namespace (the real ``oracle.paged_attention``
module, or a mutated copy of its source) and raises AssertionError when the
oracle disagrees with:

* the pages' worked structure (the hand-derived fixture in tests/golden),
* a library routine on the contiguous special case (torch SDPA in fp64, with
  its own GQA and causal options),
* a 40-digit brute force over flat offsets,
* closed forms (one key, identical keys, zero query, a dominant key),
* invariants (block-table permutation, weights summing to one, split and
  merge equal to unsplit, cached decode equal to full recompute),
* explicit flat-offset arithmetic for the append.

tests/test_oracle_pins.py runs every pin on the real oracle. The mutant test
plants plausible mistakes in copies of the oracle and requires each to fail
at least one pin.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from oracle.brute_force import brute_decode_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers (test-side, independent of the oracle)

def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits through torch (its own rounding code, not the generator's)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _values_torch(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Exact fp64 values through torch's own bf16 decoding."""
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.float64)


def _flat_scatter(contig_k: np.ndarray, ids, num_blocks: int, block_size: int, fill) -> np.ndarray:
    """Build a pool from contiguous [Hkv, L, D] data with explicit row-major offsets.

    Element (blk, g, off, d) of a [NB, Hkv, BS, D] row-major array sits at flat
    offset ((blk * Hkv + g) * BS + off) * D + d.
    """
    Hkv, L, D = contig_k.shape
    flat = np.full(num_blocks * Hkv * block_size * D, fill, dtype=contig_k.dtype)
    for g in range(Hkv):
        for t in range(L):
            blk = ids[t // block_size]
            base = ((blk * Hkv + g) * block_size + (t % block_size)) * D
            flat[base:base + D] = contig_k[g, t]
    return flat.reshape(num_blocks, Hkv, block_size, D)


def _rand_case(rng, B, Hq, Hkv, D, BS, lens, dtype, NB=None):
    """Random paged case: contiguous per-sequence K/V, scattered through a random table."""
    lens = list(lens)
    nblk = [(L + BS - 1) // BS for L in lens]
    NB = NB or sum(nblk) + 3
    perm = rng.permutation(NB)
    MBPS = max(max(nblk), 1)
    bt = np.full((B, MBPS), -1, dtype=np.int32)
    s = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[s:s + nblk[b]]
        s += nblk[b]
    qf = rng.standard_normal((B, Hq, D)).astype(np.float32)
    seqs_k = [rng.standard_normal((Hkv, L, D)).astype(np.float32) for L in lens]
    seqs_v = [rng.standard_normal((Hkv, L, D)).astype(np.float32) for L in lens]
    if dtype == "bf16":
        enc = _bf16_bits
        nan = np.uint16(0x7FC0)
    else:
        enc = lambda x: np.ascontiguousarray(x, np.float32)  # noqa: E731
        nan = np.float32("nan")
    q = enc(qf)
    pool_dtype = np.uint16 if dtype == "bf16" else np.float32
    kc = np.full((NB, Hkv, BS, D), nan, dtype=pool_dtype)
    vc = np.full((NB, Hkv, BS, D), nan, dtype=pool_dtype)
    ks, vs = [], []
    for b in range(B):
        if lens[b] == 0:
            ks.append(enc(seqs_k[b]))
            vs.append(enc(seqs_v[b]))
            continue
        kb = enc(seqs_k[b])
        vb = enc(seqs_v[b])
        ks.append(kb)
        vs.append(vb)
        pk = _flat_scatter(kb, bt[b], NB, BS, nan)
        pv = _flat_scatter(vb, bt[b], NB, BS, nan)
        used = np.zeros(NB, bool)
        used[bt[b, :nblk[b]]] = True
        # Merge: only the slots this sequence owns come from its scatter.
        own = np.zeros((NB, Hkv, BS, D), bool)
        for t in range(lens[b]):
            own[bt[b, t // BS], :, t % BS, :] = True
        kc = np.where(own, pk, kc)
        vc = np.where(own, pv, vc)
    return dict(q=q, k=kc, v=vc, bt=bt, lens=np.asarray(lens, np.int32), ks=ks, vs=vs, NB=NB)


def _sdpa(q_vals, k_vals, v_vals, scale, causal=False):
    """torch SDPA in fp64 on contiguous tensors, GQA by torch's own enable_gqa."""
    return torch.nn.functional.scaled_dot_product_attention(
        q_vals, k_vals, v_vals, scale=scale, is_causal=causal,
        enable_gqa=q_vals.shape[-3] != k_vals.shape[-3])


# ---------------------------------------------------------------- pins

def pin_golden(ora):
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    nanify = lambda x: np.array([[[[np.nan if e is None else e for e in row] for row in head] for head in blk]  # noqa: E731
                                 for blk in x], dtype=np.float32)
    k = nanify(g["k_cache"])
    v = nanify(g["v_cache"])
    q = np.array(g["q"], dtype=np.float32)
    out = ora.paged_decode_attention(q, k, v, np.array(g["block_tables"], np.int32),
                                     np.array(g["context_lens"], np.int32), g["scale"], g["block_size"], "f32")
    exp = np.array([[[float(x) for x in row] for row in b] for b in g["expected"]])
    assert np.all(np.isfinite(out)), "poisoned slot reached the result"
    assert np.allclose(out, exp, rtol=0, atol=1e-13), (out, exp)
    # The closed forms in the fixture's derivation, evaluated again here.
    e = math.e
    h0 = [(7 + e) / (1 + 2 * e), 7 * e / (1 + 2 * e)]
    a, c = math.exp(-4), math.exp(-12)
    Z = 1 + a + c
    h1 = [(7 + c) / Z, (14 * a - 7 * c) / Z]
    assert np.allclose(exp[0], [h0, h1], rtol=0, atol=1e-14)


def pin_brute_force(ora):
    rng = np.random.default_rng(1234)
    for dtype in ("f32", "bf16"):
        for (B, Hq, Hkv, D, BS, lens) in [(2, 4, 2, 8, 4, [7, 13]), (1, 3, 1, 5, 2, [1]),
                                          (2, 2, 2, 4, 8, [20, 9]), (2, 4, 1, 6, 4, [0, 11])]:
            c = _rand_case(rng, B, Hq, Hkv, D, BS, lens, dtype)
            scale = 1.0 / math.sqrt(D)
            out = ora.paged_decode_attention(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, BS, dtype)
            qv = _values_torch(c["q"], dtype).tolist()
            kf = _values_torch(c["k"], dtype).reshape(-1).tolist()
            vf = _values_torch(c["v"], dtype).reshape(-1).tolist()
            ref = brute_decode_attention(qv, kf, vf, c["bt"].tolist(), c["lens"].tolist(), scale, Hkv, BS, D)
            ref = np.array([[[float(x) for x in row] for row in b] for b in ref])
            assert np.allclose(out, ref, rtol=0, atol=1e-12), np.abs(out - ref).max()


def pin_sdpa_contiguous(ora):
    """Paged result == contiguous decode attention (torch SDPA, fp64, enable_gqa)."""
    rng = np.random.default_rng(99)
    for dtype, (B, Hq, Hkv, D, BS, lens) in [("bf16", (3, 8, 2, 16, 4, [5, 16, 23])),
                                             ("f32", (2, 6, 6, 8, 16, [33, 1])),
                                             ("bf16", (1, 12, 3, 32, 8, [64]))]:
        c = _rand_case(rng, B, Hq, Hkv, D, BS, lens, dtype)
        scale = 0.37
        out = ora.paged_decode_attention(c["q"], c["k"], c["v"], c["bt"], c["lens"], scale, BS, dtype)
        for b in range(B):
            qv = _values_torch(c["q"][b], dtype)[:, None, :]  # [Hq, 1, D]
            kv = _values_torch(c["ks"][b], dtype)  # [Hkv, L, D]
            vv = _values_torch(c["vs"][b], dtype)
            ref = _sdpa(qv[None], kv[None], vv[None], scale)[0, :, 0, :].numpy()
            assert np.allclose(out[b], ref, rtol=0, atol=1e-12), (b, np.abs(out[b] - ref).max())


def pin_naive_vs_sdpa(ora):
    rng = np.random.default_rng(5)
    Hq, Hkv, S, D = 6, 3, 11, 8
    q = rng.standard_normal((Hq, S, D))
    k = rng.standard_normal((Hkv, S, D))
    v = rng.standard_normal((Hkv, S, D))
    out = ora.naive_causal_attention(q, k, v, 0.3)
    ref = _sdpa(torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], 0.3,
                causal=True)[0].numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def pin_full_recompute(ora):
    """Decoding with the paged cache equals naive full attention at the last position, at every step."""
    rng = np.random.default_rng(7)
    Hq, Hkv, S, D, BS = 4, 2, 19, 8, 4
    qf = _bf16_bits(rng.standard_normal((Hq, S, D)).astype(np.float32))
    kf = _bf16_bits(rng.standard_normal((Hkv, S, D)).astype(np.float32))
    vf = _bf16_bits(rng.standard_normal((Hkv, S, D)).astype(np.float32))
    scale = 1 / math.sqrt(D)
    full = ora.naive_causal_attention(_values_torch(qf, "bf16").numpy(), _values_torch(kf, "bf16").numpy(),
                                      _values_torch(vf, "bf16").numpy(), scale)
    NB = 9
    ids = np.array([6, 2, 8, 0, 4], np.int32)
    bt = ids[None, :]
    kc = np.full((NB, Hkv, BS, D), 0x7FC0, np.uint16)
    vc = np.full((NB, Hkv, BS, D), 0x7FC0, np.uint16)
    for p in range(S):
        lens = np.array([p + 1], np.int32)
        kc, vc = ora.kv_append(kc, vc, kf[None, :, p, :], vf[None, :, p, :], bt, lens, BS)
        out = ora.paged_decode_attention(qf[None, :, p, :], kc, vc, bt, lens, scale, BS, "bf16")
        assert np.allclose(out[0], full[:, p, :], rtol=0, atol=1e-12), p


def pin_permutation(ora):
    rng = np.random.default_rng(11)
    c = _rand_case(rng, 3, 4, 2, 8, 4, [9, 16, 3], "bf16", NB=20)
    out = ora.paged_decode_attention(c["q"], c["k"], c["v"], c["bt"], c["lens"], 0.5, 4, "bf16")
    perm = rng.permutation(c["NB"])  # new id of old block i is perm[i]
    k2 = np.empty_like(c["k"])
    v2 = np.empty_like(c["v"])
    k2[perm] = c["k"]
    v2[perm] = c["v"]
    bt2 = np.where(c["bt"] >= 0, perm[np.maximum(c["bt"], 0)], -1).astype(np.int32)
    out2 = ora.paged_decode_attention(c["q"], k2, v2, bt2, c["lens"], 0.5, 4, "bf16")
    assert np.array_equal(out, out2)


def pin_closed_forms(ora):
    rng = np.random.default_rng(3)
    B, Hq, Hkv, D, BS = 1, 4, 2, 8, 4
    # (1) One key: the output is that key's V exactly.
    c = _rand_case(rng, B, Hq, Hkv, D, BS, [1], "f32")
    out = ora.paged_decode_attention(c["q"], c["k"], c["v"], c["bt"], c["lens"], 0.7, BS, "f32")
    for h in range(Hq):
        assert np.array_equal(out[0, h], c["vs"][0][h // 2, 0].astype(np.float64))
    # (2) Identical keys: the output is the mean of V. (3) Zero query: the same.
    L = 10
    c = _rand_case(rng, B, Hq, Hkv, D, BS, [L], "f32")
    k = c["k"].copy()
    for t in range(L):
        k[c["bt"][0, t // BS], :, t % BS, :] = c["ks"][0][:, 0, :]
    out = ora.paged_decode_attention(c["q"], k, c["v"], c["bt"], c["lens"], 0.7, BS, "f32")
    mean_v = c["vs"][0].astype(np.float64).mean(axis=1)  # [Hkv, D]
    for h in range(Hq):
        assert np.allclose(out[0, h], mean_v[h // 2], rtol=0, atol=1e-14)
    q0 = np.zeros_like(c["q"])
    out = ora.paged_decode_attention(q0, c["k"], c["v"], c["bt"], c["lens"], 0.7, BS, "f32")
    for h in range(Hq):
        assert np.allclose(out[0, h], mean_v[h // 2], rtol=0, atol=1e-14)
    # (4) A dominant key k_a = c * q: the output tends to V_a.
    a = 6
    k = c["k"].copy()
    for g in range(Hkv):
        k[c["bt"][0, a // BS], g, a % BS, :] = 200.0 * c["q"][0, 2 * g]
    out = ora.paged_decode_attention(c["q"], k, c["v"], c["bt"], c["lens"], 1.0, BS, "f32")
    for g in range(Hkv):
        assert np.allclose(out[0, 2 * g], c["vs"][0][g, a], rtol=0, atol=1e-12)


def pin_weights_sum(ora):
    rng = np.random.default_rng(4)
    c = _rand_case(rng, 2, 4, 2, 8, 4, [13, 30], "bf16")
    W = ora.attention_weights(c["q"], c["k"], c["bt"], c["lens"], 0.5, 4, "bf16")
    for b in range(2):
        assert W[b].shape == (4, int(c["lens"][b]))
        assert np.all(W[b] > 0)
        assert np.allclose(W[b].sum(axis=1), 1.0, rtol=0, atol=1e-12)


def pin_split_merge(ora):
    rng = np.random.default_rng(8)
    BS = 4
    c = _rand_case(rng, 3, 4, 2, 8, BS, [37, 4, 64], "bf16")
    ref = ora.paged_decode_attention(c["q"], c["k"], c["v"], c["bt"], c["lens"], 0.5, BS, "bf16")
    for P in (4, 8, 12, 64, 100 * BS):
        out, stats = ora.split_paged_decode_attention(c["q"], c["k"], c["v"], c["bt"], c["lens"], 0.5, BS, "bf16", P)
        assert np.allclose(out, ref, rtol=0, atol=1e-12), P
        for b in range(3):
            n = -(-int(c["lens"][b]) // P)
            assert stats[b][0][1].shape == (n,)
    # The merge is independent of the order of its parts.
    o, m, l = stats[0][1]
    _, st8 = ora.split_paged_decode_attention(c["q"], c["k"], c["v"], c["bt"], c["lens"], 0.5, BS, "bf16", 8)
    o, m, l = st8[0][1]
    p = rng.permutation(len(m))
    assert np.allclose(ora.lse_merge(o[p], m[p], l[p]), ora.lse_merge(o, m, l), rtol=0, atol=1e-13)
    # A merge of one part returns it; the merge of two parts with equal max is the l-weighted mean.
    assert np.allclose(ora.lse_merge(o[:1], m[:1], l[:1]), o[0], rtol=0, atol=1e-15)
    two = ora.lse_merge(np.array([[1.0, 2.0], [3.0, 6.0]]), np.array([0.5, 0.5]), np.array([1.0, 3.0]))
    assert np.allclose(two, [2.5, 5.0], rtol=0, atol=1e-15)
    # Partition statistics against their definitions on a hand-sized row.
    s = np.array([0.0, 1.0, 2.0])
    V = np.array([[1.0], [2.0], [4.0]])
    o, m, l = ora.partition_stats(s, V, 2)
    assert np.allclose(m, [1.0, 2.0]) and np.allclose(l, [1 + math.exp(-1), 1.0])
    assert np.allclose(o[:, 0], [(math.exp(-1) + 2) / (1 + math.exp(-1)), 4.0])


def pin_append(ora):
    rng = np.random.default_rng(2)
    NB, Hkv, BS, D, B = 7, 3, 4, 5, 3
    kc = rng.integers(0, 2**16, size=(NB, Hkv, BS, D), dtype=np.uint16)
    vc = rng.integers(0, 2**16, size=(NB, Hkv, BS, D), dtype=np.uint16)
    kn = rng.integers(0, 2**16, size=(B, Hkv, D), dtype=np.uint16)
    vn = rng.integers(0, 2**16, size=(B, Hkv, D), dtype=np.uint16)
    bt = np.array([[5, 2, -1], [0, 6, 3], [4, -1, -1]], np.int32)
    lens = np.array([6, 12, 0], np.int32)  # last tokens: seq0 pos 5 -> blk 2 off 1; seq1 pos 11 -> blk 3 off 3
    k2, v2 = ora.kv_append(kc, vc, kn, vn, bt, lens, BS)
    fk, fv = kc.reshape(-1).copy(), vc.reshape(-1).copy()
    for (b, blk, off) in [(0, 2, 1), (1, 3, 3)]:
        for g in range(Hkv):
            base = ((blk * Hkv + g) * BS + off) * D
            fk[base:base + D] = kn[b, g]
            fv[base:base + D] = vn[b, g]
    assert np.array_equal(k2.reshape(-1), fk) and np.array_equal(v2.reshape(-1), fv)
    assert k2.dtype == kc.dtype and k2.shape == kc.shape
    assert not np.shares_memory(k2, kc)


def pin_empty_and_decode(ora):
    q = np.ones((2, 2, 4), np.float32)
    kc = np.full((3, 1, 4, 4), np.nan, np.float32)
    bt = np.array([[1, -1], [-1, -1]], np.int32)
    out = ora.paged_decode_attention(q, kc, kc, bt, np.array([0, 0], np.int32), 0.5, 4, "f32")
    assert np.array_equal(out, np.zeros((2, 2, 4)))
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F], np.uint16)
    vals = ora.decode_values(bits, "bf16")
    assert vals[0] == 1.0 and vals[1] == -2.0
    assert vals[2] == 2.0 ** -133 and vals[3] == (2 - 2.0 ** -7) * 2.0 ** 127


ALL_PINS = [pin_golden, pin_brute_force, pin_sdpa_contiguous, pin_naive_vs_sdpa, pin_full_recompute,
            pin_permutation, pin_closed_forms, pin_weights_sum, pin_split_merge, pin_append,
            pin_empty_and_decode]
