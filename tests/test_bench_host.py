"""Host logic of bench.py (CPU only): the refusal of several GPUs, the algorithmic byte counts
behind roofline.achieved, and the reading of the committed rocprofv3 summaries (taken only when
they were made on the current decode sources)."""

import os
import subprocess
import sys

import numpy as np

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_headline_algorithmic_bytes():
    # Qwen3-8B batch: 64 sequences, 8 kv heads, head_dim 128, bf16, lengths from seed 3.
    w = wl.WORKLOADS["qwen3_8b_b64"]
    case = wl.make_case(w)
    L = case.context_lens.astype(np.int64)
    ab = bench.algorithmic_bytes(case, 1024)
    kv = int(L.sum()) * 8 * 128 * 2 * 2
    assert ab["kv"] == kv == 1_008_586_752
    ids = 4 * int(((L + 15) // 16).sum())
    q = 64 * 32 * 128 * 2
    nparts = int(((L + 1023) // 1024).sum())
    partials = nparts * 32 * (128 + 2) * 4
    assert ab["decode"] == kv + ids + q + 4 * 64 + partials
    assert ab["reduce"] == partials + 4 * 64 + 64 * 32 * 128 * 2
    append = 4 * 64 * 8 * 128 * 2 + 4 * 64 + 4 * 64
    assert ab["append"] == append
    # The decode launch's bytes quoted with the roofline (K+V, q, ids, lengths, partials, append).
    assert ab["decode"] + ab["append"] == 1_014_240_500


def test_window_bytes_count_only_the_window():
    w = wl.WORKLOADS["gptoss_20b_window128_b64"]
    case = wl.make_case(w)
    ab = bench.algorithmic_bytes(case, 0)
    L = np.maximum(case.context_lens.astype(np.int64), 0)
    assert ab["kv"] == int(np.minimum(L, 128).sum()) * 8 * 64 * 2 * 2
    assert ab["reduce"] == 0


def test_profiles_are_read_only_for_the_current_sources(tmp_path, monkeypatch):
    # The committed summaries carry the current decode sources' hash: they are read.
    for name, P in bench.CONFIGS + bench.EXTRA_WORKLOADS:
        trace = bench.read_trace(name, P)
        assert trace is not None and trace["decode_us"] > 0, name
    assert bench.read_traffic("qwen3_8b_b64", 1024) is not None
    # Another partition size, or another source hash, and they are not.
    assert bench.read_trace("qwen3_8b_b64", 512) is None
    monkeypatch.setattr(bench, "decode_source_hash", lambda: "0" * 16)
    assert bench.read_trace("qwen3_8b_b64", 1024) is None
    assert bench.read_traffic("qwen3_8b_b64", 1024) is None
