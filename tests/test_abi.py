"""C ABI checks that need no GPU: the library loads, exports what include/xs/xs.h declares, and
rejects bad arguments on the host with a status and a message, before any HIP call."""

import ctypes
import os
import re

import pytest

from paged_kv_decode_xs_amd import _binding as xb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "xs", "xs.h")

pytestmark = pytest.mark.skipif(not os.path.exists(xb.LIB_PATH), reason="libxs.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(xs_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("xs_kv_append", "xs_paged_attn_decode", "xs_paged_attn_reduce", "xs_last_error", "xs_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(xb.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in xb.SIGNATURES, f"binding lacks {name}"


def test_library_exports_nothing_else():
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", xb.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert {n for n in exported if n.startswith("xs_")} == set(declared_functions())


def test_version():
    assert xb.load_library().xs_version() >= 100


# Calls below are all rejected by the host checks, which run before any HIP call.
F, B = 0, 1
FAKE = 1 << 20  # a 16-byte aligned non-null address that is never dereferenced


def _decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, scale=0.125, out=FAKE, po=None, pm=None, pl=None, batch=2,
             hq=8, hkv=2, d=128, bs=16, mbps=4, nb=16, p=0, np_=0, dt=B, stream=None)
    a.update(kw)
    lib = xb.load_library()
    return lib.xs_paged_attn_decode(a["q"], a["k"], a["v"], a["bt"], a["cl"], a["scale"], a["out"], a["po"], a["pm"],
                                    a["pl"], a["batch"], a["hq"], a["hkv"], a["d"], a["bs"], a["mbps"], a["nb"],
                                    a["p"], a["np_"], a["dt"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(hq=6, hkv=4), 1, "multiple"),
    (dict(d=96), 2, "head_dim"),
    (dict(bs=12), 2, "block_size"),
    (dict(dt=7), 2, "dtype"),
    (dict(batch=-1), 1, "batch"),
    (dict(hkv=0), 1, "num_kv_heads"),
    (dict(nb=0), 1, "num_blocks"),
    (dict(q=None), 1, "NULL"),
    (dict(out=None), 1, "out is NULL"),
    (dict(p=24, np_=2, po=FAKE, pm=FAKE, pl=FAKE), 1, "multiple of block_size"),
    (dict(p=32, np_=0, po=FAKE, pm=FAKE, pl=FAKE), 1, "max_partitions"),
    (dict(p=32, np_=2), 1, "needs part_o"),
    (dict(po=FAKE), 1, "must be NULL"),
    (dict(q=FAKE + 4), 1, "aligned"),
    (dict(scale=float("inf")), 1, "scale"),
    (dict(p=-16), 1, "partition_size"),
    (dict(batch=1 << 20, hkv=8, hq=8, p=16, np_=1 << 10, po=FAKE, pm=FAKE, pl=FAKE), 1, "launch limit"),
])
def test_decode_rejects(kw, status, needle):
    assert _decode(**kw) == status
    assert needle in xb.xs_last_error()


def test_empty_batch_is_a_noop():
    assert _decode(batch=0, q=None, out=None) == 0
    assert xb.xs_last_error() == ""


def _append(**kw):
    a = dict(kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, batch=2, hkv=2, d=64, bs=16, mbps=4, nb=8, dt=B,
             stream=None)
    a.update(kw)
    return xb.load_library().xs_kv_append(a["kn"], a["vn"], a["kc"], a["vc"], a["bt"], a["cl"], a["batch"], a["hkv"],
                                          a["d"], a["bs"], a["mbps"], a["nb"], a["dt"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(kc=None), 1, "NULL"),
    (dict(d=80), 2, "head_dim"),
    (dict(bs=64), 2, "block_size"),
    (dict(vn=FAKE + 2), 1, "aligned"),
    (dict(mbps=0), 1, "max_blocks_per_seq"),
    (dict(dt=-1), 2, "dtype"),
])
def test_append_rejects(kw, status, needle):
    assert _append(**kw) == status
    assert needle in xb.xs_last_error()


def _reduce(**kw):
    a = dict(po=FAKE, pm=FAKE, pl=FAKE, cl=FAKE, out=FAKE, batch=2, hq=4, d=64, p=16, np_=3, dt=F, stream=None)
    a.update(kw)
    return xb.load_library().xs_paged_attn_reduce(a["po"], a["pm"], a["pl"], a["cl"], a["out"], a["batch"], a["hq"],
                                                  a["d"], a["p"], a["np_"], a["dt"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(pm=None), 1, "NULL"),
    (dict(p=0), 1, "partition_size"),
    (dict(np_=0), 1, "max_partitions"),
    (dict(d=32), 2, "head_dim"),
    (dict(hq=0), 1, "num_q_heads"),
])
def test_reduce_rejects(kw, status, needle):
    assert _reduce(**kw) == status
    assert needle in xb.xs_last_error()


def test_binding_raises_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        xb.load_library(str(tmp_path / "nope.so"))


def test_probe_rejects():
    lib = xb.load_library()
    assert lib.xs_stream_read_probe(None, 64, FAKE, 1, 0, None) == 1
    assert "NULL" in xb.xs_last_error()
    assert lib.xs_stream_read_probe(FAKE, 24, FAKE, 1, 0, None) == 1
    assert "multiple of 16" in xb.xs_last_error()
    assert lib.xs_stream_read_probe(FAKE, 64, FAKE, 1, 2, None) == 1
    assert "shape = 2" in xb.xs_last_error()
    assert lib.xs_stream_read_probe(FAKE, 0, FAKE, 1, 1, None) == 0  # nothing to read: no launch


def test_decode_append_rejects_missing_new_rows():
    lib = xb.load_library()
    args = [FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 0.125, FAKE, None, None, None, 2, 8, 2, 128, 16, 4, 16, 0, 0, B,
            None]
    assert lib.xs_paged_attn_decode_append(*args) == 1
    assert "k_new" in xb.xs_last_error()
    args[0] = None  # q
    assert lib.xs_paged_attn_decode_append(*args) == 1
    assert "NULL" in xb.xs_last_error()


def _decode_sinks(**kw):
    a = dict(q=FAKE, kn=None, vn=None, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, sinks=FAKE, w=0, scale=0.125, out=FAKE,
             po=None, pm=None, pl=None, batch=2, hq=8, hkv=2, d=128, bs=16, mbps=4, nb=16, p=0, np_=0, dt=B,
             stream=None)
    a.update(kw)
    return xb.load_library().xs_paged_attn_decode_sinks(
        a["q"], a["kn"], a["vn"], a["k"], a["v"], a["bt"], a["cl"], a["sinks"], a["w"], a["scale"], a["out"],
        a["po"], a["pm"], a["pl"], a["batch"], a["hq"], a["hkv"], a["d"], a["bs"], a["mbps"], a["nb"], a["p"],
        a["np_"], a["dt"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dt=F), 2, "XS_BF16"),
    (dict(bs=8), 2, "block_size"),
    (dict(w=-1), 1, "window_size"),
    (dict(kn=FAKE), 1, "both"),
    (dict(sinks=FAKE + 1), 1, "2-byte"),
    (dict(hq=6, hkv=4), 1, "multiple"),
    (dict(p=24, np_=2, po=FAKE, pm=FAKE, pl=FAKE, out=None), 1, "multiple of block_size"),
])
def test_decode_sinks_rejects(kw, status, needle):
    assert _decode_sinks(**kw) == status
    assert needle in xb.xs_last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dt=F), 2, "XS_BF16"),
    (dict(w=-3), 1, "window_size"),
    (dict(pm=None), 1, "NULL"),
    (dict(d=96), 2, "head_dim"),
])
def test_reduce_sinks_rejects(kw, status, needle):
    a = dict(po=FAKE, pm=FAKE, pl=FAKE, cl=FAKE, sinks=None, w=0, out=FAKE, batch=2, hq=4, d=64, p=16, np_=3, dt=B,
             stream=None)
    a.update(kw)
    st = xb.load_library().xs_paged_attn_reduce_sinks(a["po"], a["pm"], a["pl"], a["cl"], a["sinks"], a["w"],
                                                       a["out"], a["batch"], a["hq"], a["d"], a["p"], a["np_"],
                                                       a["dt"], a["stream"])
    assert st == status
    assert needle in xb.xs_last_error()


def test_step_graph_rejects_before_any_hip_call():
    lib = xb.load_library()
    h = ctypes.c_void_p(123)
    assert lib.xs_step_graph_create(None, 1, ctypes.byref(h)) == 1 and "descs is NULL" in xb.xs_last_error()
    assert h.value is None
    d = xb.XsStepDesc(q=FAKE, k_new=FAKE, v_new=FAKE, k_cache=FAKE, v_cache=FAKE, block_tables=FAKE,
                      context_lens=FAKE, sinks=None, window_size=0, scale=0.125, out=FAKE, part_o=None, part_m=None,
                      part_l=None, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                      max_blocks_per_seq=4, num_blocks=16, partition_size=0, max_partitions=0, dtype=B, fused=1)
    for field, value, status, needle in [("k_new", None, 1, "k_new and v_new"), ("batch", 0, 1, "nothing to capture"),
                                         ("head_dim", 96, 2, "head_dim"), ("window_size", -2, 1, "window_size"),
                                         ("dtype", F, 2, "XS_BF16")]:
        saved = getattr(d, field)
        setattr(d, field, value)
        if field == "dtype":
            d.window_size = 8
        assert lib.xs_step_graph_create(ctypes.byref(d), 1, ctypes.byref(h)) == status, field
        assert needle in xb.xs_last_error(), (field, xb.xs_last_error())
        setattr(d, field, saved)
        d.window_size = 0
    assert lib.xs_step_graph_launch(None, None) == 1
    assert lib.xs_step_graph_destroy(None) == 0


def test_step_desc_layout_matches_header():
    # The binding's structure must match the C declaration field for field.
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{(.*?)\} xs_step_desc;", text, re.S).group(1)
    names = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        head, _, rest = decl.rpartition(" ")
        parts = [p.strip().lstrip("*") for p in decl.split(",")]
        first = parts[0].split()[-1].lstrip("*")
        names.append(first)
        names.extend(p.split()[-1].lstrip("*") for p in parts[1:])
    assert names == [f for f, _ in xb.XsStepDesc._fields_]


def test_step_graph_rejects_step_count_and_names_the_bad_step():
    lib = xb.load_library()
    h = ctypes.c_void_p()
    good = dict(q=FAKE, k_new=FAKE, v_new=FAKE, k_cache=FAKE, v_cache=FAKE, block_tables=FAKE, context_lens=FAKE,
                sinks=None, window_size=0, scale=0.125, out=FAKE, part_o=None, part_m=None, part_l=None, batch=2,
                num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, max_blocks_per_seq=4, num_blocks=16,
                partition_size=0, max_partitions=0, dtype=B, fused=1)
    arr = (xb.XsStepDesc * 3)(xb.XsStepDesc(**good), xb.XsStepDesc(**good), xb.XsStepDesc(**dict(good, head_dim=80)))
    assert lib.xs_step_graph_create(arr, 0, ctypes.byref(h)) == 1 and "num_steps" in xb.xs_last_error()
    assert lib.xs_step_graph_create(arr, 3, ctypes.byref(h)) == 2 and "head_dim" in xb.xs_last_error()
    arr[2].head_dim = 128
    arr[1].batch = 0
    assert lib.xs_step_graph_create(arr, 3, ctypes.byref(h)) == 1 and "step 1" in xb.xs_last_error()


@pytest.mark.parametrize("fn", ["xs_kv_swap_out", "xs_kv_swap_in"])
@pytest.mark.parametrize("kw,status,needle", [
    (dict(n=-1), 1, "num_pairs"),
    (dict(slots=0), 1, ">= 1"),
    (dict(dt=9), 2, "dtype"),
    (dict(d=3, bs=1, hkv=1, dt=B), 1, "multiple of 16"),
    (dict(src=None), 1, "NULL"),
    (dict(kh=FAKE + 8), 1, "aligned"),
])
def test_swap_rejects(fn, kw, status, needle):
    a = dict(kc=FAKE, vc=FAKE, kh=FAKE, vh=FAKE, src=FAKE, dst=FAKE, n=4, nb=16, slots=8, hkv=2, bs=16, d=64, dt=B)
    a.update(kw)
    f = getattr(xb.load_library(), fn)
    if fn == "xs_kv_swap_out":
        st = f(a["kc"], a["vc"], a["kh"], a["vh"], a["src"], a["dst"], a["n"], a["nb"], a["slots"], a["hkv"], a["bs"],
               a["d"], a["dt"], None)
    else:
        st = f(a["kh"], a["vh"], a["kc"], a["vc"], a["src"], a["dst"], a["n"], a["nb"], a["slots"], a["hkv"], a["bs"],
               a["d"], a["dt"], None)
    assert st == status
    assert needle in xb.xs_last_error()


def test_swap_empty_list_is_a_noop():
    assert xb.load_library().xs_kv_swap_out(None, None, None, None, None, None, 0, 4, 4, 1, 16, 64, B, None) == 0


def _append_chunk(**kw):
    a = dict(ks=FAKE, vs=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sp=FAKE, cl=FAKE, batch=2, hkv=2, d=128, c=16, bs=16,
             mbps=4, nb=16, dt=B)
    a.update(kw)
    return xb.load_library().xs_kv_append_chunk(a["ks"], a["vs"], a["kc"], a["vc"], a["bt"], a["sp"], a["cl"],
                                                 a["batch"], a["hkv"], a["d"], a["c"], a["bs"], a["mbps"], a["nb"],
                                                 a["dt"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(batch=-1), 1, "batch"),
    (dict(c=-2), 1, "chunk_size"),
    (dict(d=96), 2, "head_dim"),
    (dict(bs=12), 2, "block_size"),
    (dict(dt=7), 2, "dtype"),
    (dict(sp=None), 1, "NULL"),
    (dict(cl=None), 1, "NULL"),
    (dict(ks=FAKE + 4), 1, "aligned"),
    (dict(nb=0), 1, "num_blocks"),
])
def test_append_chunk_rejects(kw, status, needle):
    assert _append_chunk(**kw) == status
    assert needle in xb.xs_last_error()


def test_append_chunk_empty_is_a_noop():
    assert _append_chunk(batch=0, ks=None, vs=None) == 0
    assert _append_chunk(c=0, ks=None, vs=None, sp=None) == 0


def _prefill(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sp=FAKE, cl=FAKE, scale=0.125, out=FAKE, batch=2, hq=8, hkv=2, d=128,
             c=16, bs=16, mbps=4, nb=16, dt=B)
    a.update(kw)
    return xb.load_library().xs_paged_attn_prefill(a["q"], a["kc"], a["vc"], a["bt"], a["sp"], a["cl"], a["scale"],
                                                    a["out"], a["batch"], a["hq"], a["hkv"], a["d"], a["c"], a["bs"],
                                                    a["mbps"], a["nb"], a["dt"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dt=F), 2, "XS_BF16"),
    (dict(d=80), 2, "head_dim"),
    (dict(bs=64), 2, "block_size"),
    (dict(hq=6, hkv=4), 1, "multiple"),
    (dict(hq=0), 1, "num_q_heads"),
    (dict(c=-1), 1, "chunk_size"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(out=None), 1, "NULL"),
    (dict(bt=None), 1, "NULL"),
    (dict(q=FAKE + 2), 1, "aligned"),
    (dict(out=FAKE + 8), 1, "aligned"),
    (dict(c=1 << 30, hq=8, hkv=1), 1, "too large"),
    (dict(batch=1 << 20, hkv=64, hq=64, c=1 << 16), 1, "launch limit"),
])
def test_prefill_rejects(kw, status, needle):
    assert _prefill(**kw) == status
    assert needle in xb.xs_last_error()


def _prefill_split(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sp=FAKE, cl=FAKE, scale=0.125, out=FAKE, po=FAKE, pml=FAKE, batch=2,
             hq=8, hkv=2, d=128, c=16, bs=16, mbps=4, nb=16, p=64, np_=1, dt=B)
    a.update(kw)
    return xb.load_library().xs_paged_attn_prefill_split(
        a["q"], a["kc"], a["vc"], a["bt"], a["sp"], a["cl"], a["scale"], a["out"], a["po"], a["pml"], a["batch"],
        a["hq"], a["hkv"], a["d"], a["c"], a["bs"], a["mbps"], a["nb"], a["p"], a["np_"], a["dt"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(p=0), 1, "partition_size = 0"),
    (dict(p=96), 1, "multiple of 64"),
    (dict(p=-64), 1, "multiple of 64"),
    (dict(p=32, np_=2), 1, "multiple of 64"),
    (dict(mbps=8), 1, "max_partitions = 1 < 2"),
    (dict(po=None), 1, "part_o and part_ml"),
    (dict(pml=None), 1, "part_o and part_ml"),
    (dict(po=FAKE + 8), 1, "aligned"),
    (dict(pml=FAKE + 4), 1, "aligned"),
    (dict(dt=F), 2, "XS_BF16"),
    (dict(out=None), 1, "NULL"),
    (dict(batch=1 << 16, hkv=64, hq=64, c=1 << 12, np_=1 << 10, mbps=1 << 12, p=64), 1, "launch limit"),
])
def test_prefill_split_rejects(kw, status, needle):
    assert _prefill_split(**kw) == status
    assert needle in xb.xs_last_error()


def test_prefill_split_empty_is_a_noop():
    assert _prefill_split(batch=0, q=None, out=None, po=None, pml=None) == 0
    assert _prefill_split(c=0, q=None, out=None, po=None, pml=None) == 0


def test_prefill_empty_is_a_noop():
    assert _prefill(batch=0, q=None, out=None) == 0
    assert _prefill(c=0, q=None, out=None) == 0


def _prefill_sinks(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sp=FAKE, cl=FAKE, sinks=FAKE, w=128, scale=0.125, out=FAKE, po=None,
             pml=None, batch=2, hq=8, hkv=2, d=64, c=16, bs=16, mbps=4, nb=16, p=0, np_=0, dt=B)
    a.update(kw)
    return xb.load_library().xs_paged_attn_prefill_sinks(
        a["q"], a["kc"], a["vc"], a["bt"], a["sp"], a["cl"], a["sinks"], a["w"], a["scale"], a["out"], a["po"],
        a["pml"], a["batch"], a["hq"], a["hkv"], a["d"], a["c"], a["bs"], a["mbps"], a["nb"], a["p"], a["np_"],
        a["dt"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(w=-1), 1, "window_size = -1"),
    (dict(sinks=FAKE + 1), 1, "sinks must be 2-byte aligned"),
    (dict(dt=F), 2, "XS_BF16"),
    (dict(d=96), 2, "head_dim"),
    (dict(hq=6, hkv=4), 1, "multiple"),
    (dict(p=96, np_=1), 1, "multiple of 64"),
    (dict(p=64, np_=1), 1, "part_o and part_ml"),
    (dict(p=64, np_=0, po=FAKE, pml=FAKE), 1, "max_partitions = 0 < 1"),
    (dict(out=None), 1, "NULL"),
    (dict(scale=float("inf")), 1, "scale"),
])
def test_prefill_sinks_rejects(kw, status, needle):
    assert _prefill_sinks(**kw) == status
    assert needle in xb.xs_last_error()


def test_prefill_sinks_empty_is_a_noop():
    assert _prefill_sinks(batch=0, q=None, out=None) == 0
    assert _prefill_sinks(c=0, q=None, out=None, p=64, np_=1) == 0


def test_noalloc_rejects_partials_beyond_its_scratch():
    # 64 sequences x 32 heads x 1024 partitions x 130 floats is far beyond the scratch: XS_EINVAL,
    # decided on the host before any device work.
    lib = xb.load_library()
    st = lib.xs_paged_attn_decode_append_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.125, FAKE, 64, 32, 8,
                                                 128, 16, 4096, 8192, 64, 1024, B, None)
    assert st == 1
    assert "scratch holds" in xb.xs_last_error()


@pytest.mark.parametrize("kw,needle", [
    (dict(out=None), "out must be"),
    (dict(k_new=None), "k_new and v_new"),
    (dict(p=24), "multiple of block_size"),
])
def test_noalloc_host_checks(kw, needle):
    a = dict(q=FAKE, k_new=FAKE, v_new=FAKE, out=FAKE, p=32)
    a.update(kw)
    lib = xb.load_library()
    st = lib.xs_paged_attn_decode_append_noalloc(a["q"], a["k_new"], FAKE, FAKE, FAKE, FAKE, FAKE, 0.125, a["out"],
                                                 2, 8, 2, 128, 16, 4, 16, a["p"], 2, B, None)
    assert st == 1
    assert needle in xb.xs_last_error()
