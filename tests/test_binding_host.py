"""The Python binding's own work, on the CPU: shape and dtype checks before any library call, and
the order and values of the arguments it hands to the C ABI (argument marshalling is all it
does). The device-placement check and the library are replaced by a recorder here, so CPU tensors
stand in for device ones and nothing runs."""

import pytest
import torch

from paged_kv_decode_xs_amd import _binding as xb


class Recorder:
    """Stands in for libxs.so: records each call's arguments and returns XS_OK."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def call(*args):
            self.calls.append((name, args))
            return 0
        return call


@pytest.fixture
def rec(monkeypatch):
    r = Recorder()
    monkeypatch.setattr(xb, "_dev", lambda *ts: None)
    monkeypatch.setattr(xb, "load_library", lambda path=None: r)
    return r


def _decode_inputs(B=3, Hq=8, Hkv=2, D=128, NB=20, BS=16, MBPS=5, NP=4, dtype=torch.bfloat16):
    return dict(
        q=torch.zeros(B, Hq, D, dtype=dtype), k=torch.zeros(NB, Hkv, BS, D, dtype=dtype),
        v=torch.zeros(NB, Hkv, BS, D, dtype=dtype), bt=torch.zeros(B, MBPS, dtype=torch.int32),
        cl=torch.zeros(B, dtype=torch.int32), out=torch.zeros(B, Hq, D, dtype=dtype),
        po=torch.zeros(B, Hq, NP, D), pm=torch.zeros(B, Hq, NP), pl=torch.zeros(B, Hq, NP),
        kn=torch.zeros(B, Hkv, D, dtype=dtype), vn=torch.zeros(B, Hkv, D, dtype=dtype))


def test_decode_split_marshalling(rec):
    a = _decode_inputs()
    xb.xs_paged_attn_decode(a["q"], a["k"], a["v"], a["bt"], a["cl"], 0.125, part_o=a["po"], part_m=a["pm"],
                            part_l=a["pl"], partition_size=64, stream=0)
    (name, args), = rec.calls
    assert name == "xs_paged_attn_decode"
    ptr = lambda t: t.data_ptr()  # noqa: E731
    assert args == (ptr(a["q"]), ptr(a["k"]), ptr(a["v"]), ptr(a["bt"]), ptr(a["cl"]), 0.125, None, ptr(a["po"]),
                    ptr(a["pm"]), ptr(a["pl"]), 3, 8, 2, 128, 16, 5, 20, 64, 4, xb.XS_BF16, None)


def test_decode_append_unsplit_marshalling(rec):
    a = _decode_inputs(dtype=torch.float32, D=64)
    xb.xs_paged_attn_decode_append(a["q"], a["kn"], a["vn"], a["k"], a["v"], a["bt"], a["cl"], 0.5, out=a["out"],
                                   stream=0)
    (name, args), = rec.calls
    assert name == "xs_paged_attn_decode_append"
    assert args[:3] == (a["q"].data_ptr(), a["kn"].data_ptr(), a["vn"].data_ptr())
    assert args[8] == a["out"].data_ptr() and args[9:12] == (None, None, None)
    assert args[12:] == (3, 8, 2, 64, 16, 5, 20, 0, 0, xb.XS_F32, None)


def test_reduce_and_append_marshalling(rec):
    a = _decode_inputs()
    xb.xs_paged_attn_reduce(a["po"], a["pm"], a["pl"], a["cl"], a["out"], 64, stream=0)
    xb.xs_kv_append(a["kn"], a["vn"], a["k"], a["v"], a["bt"], a["cl"], stream=0)
    (n1, a1), (n2, a2) = rec.calls
    assert n1 == "xs_paged_attn_reduce" and a1[5:] == (3, 8, 128, 64, 4, xb.XS_BF16, None)
    assert n2 == "xs_kv_append" and a2[6:] == (3, 2, 128, 16, 5, 20, xb.XS_BF16, None)


def test_prefill_split_marshalling(rec):
    B, Hq, Hkv, C, D, NB, BS, MBPS = 2, 8, 2, 40, 64, 30, 16, 12
    q = torch.zeros(B, Hq, C, D, dtype=torch.bfloat16)
    k = torch.zeros(NB, Hkv, BS, D, dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    bt = torch.zeros(B, MBPS, dtype=torch.int32)
    sp, cl = torch.zeros(B, dtype=torch.int32), torch.zeros(B, dtype=torch.int32)
    out = xb.xs_paged_attn_prefill_split(q, k, v, bt, sp, cl, 0.125, 64, stream=0)
    (name, args), = rec.calls
    assert name == "xs_paged_attn_prefill_split" and out.shape == q.shape
    NP = -(-MBPS * BS // 64)
    assert args[10:] == (B, Hq, Hkv, D, C, BS, MBPS, NB, 64, NP, xb.XS_BF16, None)


@pytest.mark.parametrize("change,message", [
    (dict(k=torch.zeros(20, 2, 16, 64, dtype=torch.bfloat16)), "pool shapes do not match q"),
    (dict(q=torch.zeros(3, 8, 128)), "dtypes differ"),
    (dict(bt=torch.zeros(3, 5, dtype=torch.int64)), "block_tables must be int32"),
    (dict(cl=torch.zeros(4, dtype=torch.int32)), "context_lens must be int32 [batch]"),
    (dict(pm=torch.zeros(3, 8, 5)), "partials must be"),
    (dict(po=torch.zeros(3, 8, 4, 128, dtype=torch.float64)), "partials are float32"),
])
def test_decode_checks_come_before_the_library(rec, change, message):
    a = {**_decode_inputs(), **change}
    with pytest.raises(ValueError, match=message.replace("[", r"\[").replace("]", r"\]")):
        xb.xs_paged_attn_decode(a["q"], a["k"], a["v"], a["bt"], a["cl"], 0.125, part_o=a["po"], part_m=a["pm"],
                                part_l=a["pl"], partition_size=64, stream=0)
    assert rec.calls == []


def test_unsplit_decode_needs_a_q_shaped_out(rec):
    a = _decode_inputs()
    with pytest.raises(ValueError, match="out must be q-shaped"):
        xb.xs_paged_attn_decode(a["q"], a["k"], a["v"], a["bt"], a["cl"], 0.125, out=None, stream=0)
    with pytest.raises(TypeError, match="unsupported dtype"):
        xb._dtype_code(torch.zeros(2, dtype=torch.float16))
    assert rec.calls == []


def test_device_check_rejects_host_tensors():
    with pytest.raises(ValueError, match="on the GPU"):
        xb._dev(torch.zeros(4))


@pytest.mark.parametrize("P,fused,sw,expected", [
    (0, False, False, ["xs_kv_append", "xs_paged_attn_decode"]),
    (0, True, False, ["xs_paged_attn_decode_append"]),
    (64, False, False, ["xs_kv_append", "xs_paged_attn_decode", "xs_paged_attn_reduce"]),
    (64, True, False, ["xs_paged_attn_decode_append", "xs_paged_attn_reduce"]),
    (0, True, True, ["xs_paged_attn_decode_sinks"]),
    (64, False, True, ["xs_kv_append", "xs_paged_attn_decode_sinks", "xs_paged_attn_reduce_sinks"]),
    (64, True, True, ["xs_paged_attn_decode_sinks", "xs_paged_attn_reduce_sinks"]),
])
def test_decode_step_call_chain(rec, P, fused, sw, expected):
    from paged_kv_decode_xs_amd.step import DecodeStep

    a = _decode_inputs()
    sinks = torch.zeros(8, dtype=torch.bfloat16) if sw else None
    step = DecodeStep(a["q"], a["k"], a["v"], a["bt"], a["cl"], a["kn"], a["vn"], 0.125, partition_size=P,
                      max_context_len=200 if P else None, fused=fused, sinks=sinks, window=16 if sw else 0)
    step.run(stream=0)
    assert [name for name, _ in rec.calls] == expected
    if P:
        assert step.part_m.shape == (3, 8, 4)  # ceil(200 / 64) partitions
    if sw:
        # The fused windowed decode gets k_new / v_new; the separate one gets none (the append ran).
        sink_call = [args for name, args in rec.calls if name == "xs_paged_attn_decode_sinks"][0]
        assert (sink_call[1] is not None) == fused
