"""The rounding bound of tests/rounding_bound.py: its spread in closed form, a simulation of the
kernels' rounding that satisfies it, and its power: at the long-context sizes (the 64-sequence
batch's longest rows, the 32K row of the long-context batch) an output that misses one 16-token
block, or one 512-token partition, violates it, while the output tolerance alone lets them pass.
CPU only."""

import numpy as np
import pytest

from tests import rounding_bound as rb
from workloads import f32_to_bf16_bits


def bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 (through fp32, round to nearest even) -> fp64."""
    bits = f32_to_bf16_bits(np.asarray(x, np.float64).astype(np.float32))
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def rand_bf16(rng, shape):
    return bf16(rng.standard_normal(shape))


def exact(q, K, V, scale, keep=None):
    s = scale * (K @ q)
    if keep is not None:
        s = np.where(keep, s, -np.inf)
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def kernel_like(q, K, V, scale, P):
    """What the split-K matrix-core path computes, in fp64 except for its two bf16 roundings: per
    partition of P keys the weights p = exp(s - m_j) are rounded to bf16 for P.V while l_j keeps
    the unrounded sum; the partitions merge by the log-sum-exp rule; the result is rounded to bf16."""
    s = scale * (K @ q)
    o, m, l = [], [], []
    for j0 in range(0, len(s), P):
        sj = s[j0:j0 + P]
        mj = sj.max()
        p = np.exp(sj - mj)
        o.append((bf16(p) @ V[j0:j0 + P]) / p.sum())
        m.append(mj)
        l.append(p.sum())
    m, l = np.array(m), np.array(l)
    w = l * np.exp(m - m.max())
    return bf16((w @ np.array(o)) / w.sum())


def test_spread_closed_forms():
    rng = np.random.default_rng(0)
    K, V = rand_bf16(rng, (1, 8)), rand_bf16(rng, (1, 8))
    tau = rb.row_spread(rand_bf16(rng, (1, 8)), K, V, 0.3, np.array([0]), np.array([0]))
    assert np.allclose(tau[0], np.abs(V[0]), rtol=0, atol=1e-15)          # one key: weight 1
    K = np.repeat(rand_bf16(rng, (1, 8)), 5, axis=0)
    V = rand_bf16(rng, (5, 8))
    tau = rb.row_spread(rand_bf16(rng, (1, 8)), K, V, 0.3, np.array([0]), np.array([4]))
    assert np.allclose(tau[0], np.sqrt((V ** 2).sum(axis=0)) / 5, rtol=1e-14)  # equal weights 1/5
    # A window keeps keys first .. last only; a sink far below the scores changes nothing.
    K, V = rand_bf16(rng, (9, 8)), rand_bf16(rng, (9, 8))
    q = rand_bf16(rng, (1, 8))
    a = rb.row_spread(q, K, V, 0.3, np.array([3]), np.array([6]))
    b = rb.row_spread(q, K[3:7], V[3:7], 0.3, np.array([0]), np.array([3]))
    c = rb.row_spread(q, K[3:7], V[3:7], 0.3, np.array([0]), np.array([3]), sink=-200.0)
    assert np.allclose(a, b, rtol=1e-14) and np.allclose(b, c, rtol=1e-14)
    # A sink far above the scores takes all the weight: tau -> 0.
    d = rb.row_spread(q, K, V, 0.3, np.array([0]), np.array([8]), sink=60.0)
    assert np.all(d < 1e-20)


# (context length, partition size): the longest rows of the 64-sequence batch and the long-context
# batch's rows, Qwen3-8B head_dim 128, four query heads of one kv head.
CASES = [(4000, 1024), (8192, 1024), (32768, 512)]


@pytest.mark.parametrize("L,P", CASES)
def test_kernel_like_rounding_passes_and_dropped_keys_fail(L, P):
    rng = np.random.default_rng(L)
    D, H = 128, 4
    scale = 1 / np.sqrt(D)
    K, V = rand_bf16(rng, (L, D)), rand_bf16(rng, (L, D))
    Q = rand_bf16(rng, (H, D))
    ref = np.stack([exact(Q[h], K, V, scale) for h in range(H)])
    tau = rb.row_spread(Q, K, V, scale, np.zeros(H, int), np.full(H, L - 1))
    got = np.stack([kernel_like(Q[h], K, V, scale, P) for h in range(H)])
    assert rb.violations(got, ref, tau) == 0
    atol, rtol = 2e-2, 2e-2
    for drop in (16, P):  # one block, one partition
        keep = np.ones(L, bool)
        keep[L // 2: L // 2 + drop] = False
        wrong = np.stack([bf16(exact(Q[h], K, V, scale, keep)) for h in range(H)])
        n = rb.violations(wrong, ref, tau)
        assert n > 0, f"L={L}: dropping {drop} keys goes unnoticed by the rounding bound"
        if drop * 64 <= L:
            # A sixty-fourth of the keys or less: the output tolerance alone cannot see it.
            assert np.all(np.abs(wrong - ref) <= atol + rtol * np.abs(ref))


def test_sinks_and_window_rows_follow_the_same_rule():
    # With a sink the weights' denominator includes e^(sigma - M); the kernel-like computation over
    # a window with a sink stays within the bound and a dropped block in the window does not.
    rng = np.random.default_rng(5)
    D, W, L = 64, 2048, 6000
    scale = 1 / 8
    K, V = rand_bf16(rng, (L, D)), rand_bf16(rng, (L, D))
    q = rand_bf16(rng, (D,))
    sig = 1.5
    t0 = L - W
    s = scale * (K[t0:] @ q)
    M = max(s.max(), sig)
    p = np.exp(s - M)
    den = p.sum() + np.exp(sig - M)
    ref = (p @ V[t0:]) / den
    got = bf16((bf16(p) @ V[t0:]) / den)
    tau = rb.row_spread(q[None], K, V, scale, np.array([t0]), np.array([L - 1]), sink=sig)[0]
    assert rb.violations(got, ref, tau) == 0
    keep = np.ones(W, bool)
    keep[100:116] = False
    wrong = bf16((p * keep) @ V[t0:] / ((p * keep).sum() + np.exp(sig - M)))
    assert rb.violations(wrong, ref, tau) > 0
