"""Planted mistakes in copies of the oracle must each fail at least one pin (CPU only).

Each mutant is the oracle's source with one plausible mistake: a wrong GQA
mapping, transposed pool axes, a dropped scale or normalisation, a wrong
sign, an off-by-one in the append slot or a partition boundary, a merge
without its rescale, a wrong bf16 decode, a wrong causal mask. The mutant
is loaded as a fresh module, and the real oracle is never modified.
"""

import inspect
import types

import pytest

import oracle.paged_attention as ora
from tests.oracle_pins import ALL_PINS

SOURCE = inspect.getsource(ora)

# (function the mistake sits in, original text, mutated text)
MUTANTS = {
    "gqa_modulo": ("paged_decode_attention", "g = h // n_rep", "g = h % Hkv"),
    "pool_axes_swapped": ("gather_kv", "(1, 0, 2, 3)", "(2, 0, 1, 3)"),
    "table_ignored": ("paged_decode_attention", "ids = np.asarray(block_tables[b, :nblk], dtype=np.int64)",
                      "ids = np.arange(nblk)"),
    "scale_dropped": ("_scores", "return scale * (K_g @ q_h)", "return (K_g @ q_h)"),
    "exp_sign": ("paged_decode_attention", "w = np.exp(s - s.max())", "w = np.exp(s.max() - s)"),
    "not_normalised": ("paged_decode_attention", "out[b, h] = (w @ V[g]) / w.sum()", "out[b, h] = (w @ V[g])"),
    "append_slot_L": ("kv_append", "        p = L - 1\n", "        p = L if L < 4 else L - 1\n"),
    "append_v_dropped": ("kv_append", "v_out[blk, :, off, :] = v_new[b]", "pass"),
    "append_head0_only": ("kv_append", "k_out[blk, :, off, :] = k_new[b]", "k_out[blk, 0, off, :] = k_new[b, 0]"),
    "merge_no_rescale": ("lse_merge", "w = l * np.exp(m - M)", "w = l"),
    "merge_no_l": ("lse_merge", "w = l * np.exp(m - M)", "w = np.exp(m - M)"),
    "partition_boundary": ("partition_stats", "min((j + 1) * partition_size, L)",
                           "min((j + 1) * partition_size, L - 1)"),
    "bf16_shift": ("decode_values", "<< np.uint32(16)", "<< np.uint32(15)"),
    "causal_diag_masked": ("naive_causal_attention", "k=1)", "k=0)"),
    "causal_mask_off": ("naive_causal_attention", "scores = np.where(mask[None], -np.inf, scores)", "pass"),
    "gather_skips_tail_rule": ("gather_kv", "return seq[:, :L, :]", "return seq[:, :max(L - 1, 1), :]"),
    "weights_unnormalised": ("attention_weights", "W[h] = w / w.sum()", "W[h] = w"),
}


def _mutate(name):
    func, old, new = MUTANTS[name]
    start = SOURCE.index(f"\ndef {func}(")
    end = SOURCE.find("\ndef ", start + 1)
    end = len(SOURCE) if end < 0 else end
    body = SOURCE[start:end]
    assert body.count(old) == 1, f"mutation text for {name} must occur exactly once in {func}"
    src = SOURCE[:start] + body.replace(old, new) + SOURCE[end:]
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


# A planted mistake may overflow or produce NaN on its way to failing a pin: its numpy warnings
# are expected.
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutate(name)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts as a catch
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"


# Mistakes planted in the sinks / sliding-window oracle; each must fail one of SINK_PINS.
import oracle.sinks_window as sw_mod  # noqa: E402
from tests.oracle_pins_sinks import SINK_PINS  # noqa: E402

SW_SOURCE = inspect.getsource(sw_mod)
SW_MUTANTS = {
    "sink_dropped": ("paged_decode_attention_sinks", "den = w.sum() + (0.0 if sig is None else np.exp(sig[h] - M))",
                     "den = w.sum()"),
    "sink_scaled": ("paged_decode_attention_sinks", "np.exp(sig[h] - M))", "np.exp(scale * sig[h] - M))"),
    "sink_sign": ("paged_decode_attention_sinks", "np.exp(sig[h] - M))", "np.exp(-sig[h] - M))"),
    "window_one_more": ("window_start", "max(0, L - window)", "max(0, L - window - 1)"),
    "window_one_less": ("window_start", "max(0, L - window)", "max(0, L - window + 1)"),
    "window_ignored": ("paged_decode_attention_sinks", "        t0 = window_start(L, window)\n", "        t0 = 0\n"),
    "merge_sink_dropped": ("lse_merge_sink", "den = w.sum() + (0.0 if sink is None else np.exp(sink - M))",
                           "den = w.sum()"),
    "partition_start_unwindowed": ("partition_stats_window", "max(j * partition_size, t0)", "j * partition_size"),
    "partition_first_index": ("partition_stats_window", "j0 = t0 // partition_size", "j0 = 0"),
}


def _mutate_sw(name):
    func, old, new = SW_MUTANTS[name]
    start = SW_SOURCE.index(f"\ndef {func}(")
    end = SW_SOURCE.find("\ndef ", start + 1)
    end = len(SW_SOURCE) if end < 0 else end
    body = SW_SOURCE[start:end]
    assert body.count(old) == 1, f"mutation text for {name} must occur exactly once in {func}"
    src = SW_SOURCE[:start] + body.replace(old, new) + SW_SOURCE[end:]
    src = src.replace("from .paged_attention import", "from oracle.paged_attention import")
    mod = types.ModuleType(f"oracle_sw_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(SW_MUTANTS))
def test_sinks_window_mutant_is_caught(name):
    mod = _mutate_sw(name)
    failed = []
    for pin in SINK_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts as a catch
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"
