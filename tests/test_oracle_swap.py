"""Pins of the swap oracle (CPU): explicit flat-offset copies, a round trip, skipped pairs, and
planted mistakes that the pins must catch."""

import inspect
import types

import numpy as np
import pytest

import oracle.swap as swap_mod


def _pools(rng, NB=9, Hkv=3, BS=4, D=8):
    k = rng.integers(0, 65536, (NB, Hkv, BS, D), dtype=np.uint16)
    v = rng.integers(0, 65536, (NB, Hkv, BS, D), dtype=np.uint16)
    return k, v


def pin_flat_offsets(sw):
    # Element (blk, g, off, d) of a row-major [NB, Hkv, BS, D] array sits at ((blk*Hkv + g)*BS + off)*D + d.
    rng = np.random.default_rng(1)
    k, v = _pools(rng)
    NB, Hkv, BS, D = k.shape
    S = 5
    kh = rng.integers(0, 65536, (S, Hkv, BS, D), dtype=np.uint16)
    vh = rng.integers(0, 65536, (S, Hkv, BS, D), dtype=np.uint16)
    pairs = [(7, 2), (0, 4), (3, 0)]
    ko, vo = sw.swap_out(k, v, kh, vh, [p[0] for p in pairs], [p[1] for p in pairs])
    kf, khf, kof = k.reshape(-1), kh.reshape(-1).copy(), ko.reshape(-1)
    vf, vhf, vof = v.reshape(-1), vh.reshape(-1).copy(), vo.reshape(-1)
    n = Hkv * BS * D
    for blk, slot in pairs:
        khf[slot * n:(slot + 1) * n] = kf[blk * n:(blk + 1) * n]
        vhf[slot * n:(slot + 1) * n] = vf[blk * n:(blk + 1) * n]
    assert np.array_equal(kof, khf) and np.array_equal(vof, vhf)
    kc, vc = sw.swap_in(kh, vh, k, v, [1, 4], [8, 2])
    kcf, vcf = k.reshape(-1).copy(), v.reshape(-1).copy()
    for slot, blk in [(1, 8), (4, 2)]:
        kcf[blk * n:(blk + 1) * n] = kh.reshape(-1)[slot * n:(slot + 1) * n]
        vcf[blk * n:(blk + 1) * n] = vh.reshape(-1)[slot * n:(slot + 1) * n]
    assert np.array_equal(kc.reshape(-1), kcf) and np.array_equal(vc.reshape(-1), vcf)


def pin_round_trip_and_skips(sw):
    rng = np.random.default_rng(2)
    k, v = _pools(rng, NB=12)
    S = 6
    kh = np.zeros((S,) + k.shape[1:], np.uint16)
    vh = np.zeros_like(kh)
    blocks = [5, 11, 0, 7]
    ko, vo = sw.swap_out(k, v, kh, vh, blocks, [0, 1, 2, 3])
    # Swap back into other blocks of a blank pool: those blocks equal the originals.
    kb = np.zeros_like(k)
    vb = np.zeros_like(v)
    kc, vc = sw.swap_in(ko, vo, kb, vb, [3, 2, 1, 0], [1, 2, 3, 4])
    for dst, src in zip([1, 2, 3, 4], [7, 0, 11, 5]):
        assert np.array_equal(kc[dst], k[src]) and np.array_equal(vc[dst], v[src])
    untouched = [i for i in range(12) if i not in (1, 2, 3, 4)]
    assert not kc[untouched].any() and not vc[untouched].any()
    # Out-of-range pairs change nothing.
    ko2, vo2 = sw.swap_out(k, v, kh, vh, [-1, 12, 3], [0, 1, 6])
    assert not ko2.any() and not vo2.any()
    kc2, vc2 = sw.swap_in(ko, vo, k, v, [-1, 9, 2], [0, 3, 12])
    assert np.array_equal(kc2, k) and np.array_equal(vc2, v)


SWAP_PINS = [pin_flat_offsets, pin_round_trip_and_skips]


@pytest.mark.parametrize("pin", SWAP_PINS, ids=lambda p: p.__name__)
def test_swap_pin(pin):
    pin(swap_mod)


SOURCE = inspect.getsource(swap_mod)
MUTANTS = {
    "out_v_dropped": ("swap_out", "            v_out[slot] = v_cache[blk]\n", ""),
    "in_reversed": ("swap_in", "k_out[blk] = k_host[slot]", "k_out[slot % NB] = k_host[blk % S]"),
    "out_no_bounds": ("swap_out", "if 0 <= blk < NB and 0 <= slot < S:", "if True:"),
    "in_slot_bound_off": ("swap_in", "0 <= slot < S", "0 <= slot < S - 1"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_swap_mutant_is_caught(name):
    func, old, new = MUTANTS[name]
    start = SOURCE.index(f"\ndef {func}(")
    end = SOURCE.find("\ndef ", start + 1)
    end = len(SOURCE) if end < 0 else end
    body = SOURCE[start:end]
    assert body.count(old) == 1, name
    mod = types.ModuleType(f"swap_mutant_{name}")
    exec(compile(SOURCE[:start] + body.replace(old, new) + SOURCE[end:], name, "exec"), mod.__dict__)
    failed = []
    for pin in SWAP_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001
            failed.append(type(e).__name__)
    assert failed, f"mutant {name} passed every pin"
