"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI, compare with the oracle."""

from __future__ import annotations

import sys
from typing import Dict

import numpy as np
import torch

import oracle
import paged_kv_decode_xs_amd as xs
from tests.rounding_bound import assert_rounding_bound, decode_spread
from workloads.device import case_to_device, to_numpy_bits

# Tolerances: fp32 1e-5 absolute; bf16 2e-2 absolute + 2e-2 relative, elementwise against the fp64 oracle.
TOL = {"f32": (1e-5, 0.0), "bf16": (2e-2, 2e-2)}
# fp32 partials of the split path (exact bf16/fp32 inputs, fp32 arithmetic): a much tighter check
# than the output bar. For bf16 pools the matrix-core PV rounds the weights p to bf16 (round to
# nearest even with 8 significant bits: relative error <= 2^-8), so o_j = sum p V / l can move by
# up to 2^-8 * max|V|; that bound is added to part_o's tolerance. m_j and l_j come from unrounded
# fp32 weights and keep the tight bound.
PART_TOL = (5e-5, 1e-5)
P_BF16_REL = 2.0 ** -8


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def assert_close(got: np.ndarray, ref: np.ndarray, atol: float, rtol: float, what: str) -> float:
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in the GPU result"
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; first at {tuple(idx)}: "
                             f"got {got[tuple(idx)]!r} ref {ref[tuple(idx)]!r}; max err {err.max():.3g}")
    return float(err.max()) if err.size else 0.0


class OracleResult:
    """fp64 oracle results for one case: appended pools, unsplit output, split partials."""

    def __init__(self, case, partition_size: int = 0):
        w = case.workload
        self.k_pool, self.v_pool = oracle.kv_append(case.k_cache, case.v_cache, case.k_new, case.v_new,
                                                    case.block_tables, case.context_lens, w.block_size)
        self.out = oracle.paged_decode_attention(case.q, self.k_pool, self.v_pool, case.block_tables,
                                                 case.context_lens, w.scale, w.block_size, w.dtype)
        self._tau = None
        self._case = case
        self.stats = None
        if partition_size > 0:
            _, self.stats = oracle.split_paged_decode_attention(case.q, self.k_pool, self.v_pool, case.block_tables,
                                                                case.context_lens, w.scale, w.block_size, w.dtype,
                                                                partition_size)


def check_rounding_bound(got: np.ndarray, ref: "OracleResult", what: str) -> None:
    """bf16 outputs: the per-element bound of the kernels' rounding (tests/rounding_bound.py), which
    at long contexts is far tighter than the output tolerance."""
    case = ref._case
    w = case.workload
    if w.dtype != "bf16":
        return
    if ref._tau is None:
        ref._tau = decode_spread(case.q, ref.k_pool, ref.v_pool, case.block_tables, case.context_lens, w.scale,
                                 w.block_size, w.dtype)
    ratio = assert_rounding_bound(got, ref.out, ref._tau, what)
    log(f"[gpu] {what}: max error / bound {ratio:.3f}")


def run_step(dev: Dict[str, torch.Tensor], scale: float, partition_size: int, max_context_len: int = None,
             fused: bool = False):
    step = xs.DecodeStep(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                         dev["k_new"], dev["v_new"], scale, partition_size=partition_size,
                         max_context_len=max_context_len, fused=fused)
    nan_fill(step)
    step.run()
    torch.cuda.synchronize()
    return step


def nan_fill(step) -> None:
    """Poison a step's output and partials, so that anything the kernels leave unwritten shows."""
    for t in (step.out, step.part_o, step.part_m, step.part_l):
        if t is not None:
            t.fill_(float("nan"))



def check_case(case, partition_size: int, ref: OracleResult = None, check_pools: bool = True, label: str = "",
               fused: bool = False):
    """Append + decode (+ reduce) on the GPU, compared with the oracle. Returns the max output error."""
    w = case.workload
    log(f"[gpu] {label or w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim} "
        f"BS={w.block_size} dtype={w.dtype} P={partition_size} fused={fused} "
        f"lens={case.context_lens[:8].tolist()}...")
    ref = ref or OracleResult(case, partition_size)
    dev = case_to_device(case)
    step = run_step(dev, w.scale, partition_size, int(case.context_lens.max(initial=1)) if partition_size else None,
                    fused=fused)
    if check_pools:
        for name, exp in (("k_cache", ref.k_pool), ("v_cache", ref.v_pool)):
            got = to_numpy_bits(dev[name])
            assert np.array_equal(got.view(np.uint8), exp.view(np.uint8)), f"{name} differs after append"
    atol, rtol = TOL[w.dtype]
    got = as_f64(step.out)
    err = assert_close(got, ref.out, atol, rtol, f"{label or w.name} out (P={partition_size})")
    check_rounding_bound(got, ref, f"{label or w.name} out (P={partition_size}) rounding bound")
    if partition_size > 0 and ref.stats is not None:
        check_partials(step, ref, case)
    return err, step, dev


def check_partials(step, ref: OracleResult, case) -> None:
    """GPU partials against the oracle's partition statistics."""
    po = step.part_o.cpu().double().numpy()
    pm = step.part_m.cpu().double().numpy()
    pl = step.part_l.cpu().double().numpy()
    atol, rtol = PART_TOL
    atol_o = atol
    if case.workload.dtype == "bf16":
        vmax = float(np.nanmax(np.abs(oracle.decode_values(ref.v_pool, "bf16"))))
        atol_o = atol + P_BF16_REL * vmax
    for b in range(case.workload.batch):
        for h in range(case.workload.num_q_heads):
            o, m, l = ref.stats[b][h]
            n = len(m)
            if n == 0:
                continue
            assert_close(pm[b, h, :n], m, atol, rtol, f"part_m[{b},{h}]")
            assert_close(pl[b, h, :n], l, atol, 1e-5, f"part_l[{b},{h}]")
            assert_close(po[b, h, :n], o, atol_o, rtol, f"part_o[{b},{h}]")
