"""The work-item orders of the split grids, emulated on the CPU (no GPU).

Two kernels map a workgroup id onto a work item with wavefront-wide integer code (ballot counts,
a binary search over sizes, prefix sums, reversed rounds): the split decode's ranked order
(`dense_item` in xs_decode_mfma.hip) and the chunked prefill's largest-first order
(`ranked_piece` in xs_prefill.hip). A mistake there (an item taken twice, one skipped) is a
silently wrong output for particular mixes of lengths, which the parity tests may not happen to
meet. Here each mapping is re-implemented step by step in Python, the way the wavefront does it,
and checked over many random batches against what it must be:
  * a bijection between the ids that find an item and the items the kernel needs;
  * the items in the order the kernel documents (full partitions / pieces first, then the partial
    ones by non-increasing size, ties by index), every second whole round of CU-count ids reversed.
"""

from __future__ import annotations

import numpy as np
import pytest

# ----------------------------------------------------------------------------------------------
# Split decode: xs_decode_mfma.hip, dense_item (and the launcher's choice of it).


def seq_partitions(L, mbps, BS, pb, maxp):
    """(full partitions, partial last partition 0/1, its size in blocks) the split grid computes."""
    L = min(L, mbps * BS)
    nblk = (L + BS - 1) // BS if L > 0 else 0
    nfull = min(nblk // pb, maxp)
    npartial = 1 if nblk % pb != 0 and nblk // pb < maxp else 0
    return nfull, npartial, nblk - nfull * pb


def dense_item(k, lens, mbps, BS, pb, maxp, segs, ncu, grid):
    """Workgroup id k -> (b, p, seg), b = -1 past the last item; the steps of the kernel."""
    batch = len(lens)
    ncu = max(ncu, 1)
    rnd, col = divmod(k, ncu)
    if (rnd & 1) and (rnd + 1) * ncu <= grid:
        k = rnd * ncu + (ncu - 1 - col)
    parts = [seq_partitions(L, mbps, BS, pb, maxp) for L in lens]
    F = sum(nf for nf, _, _ in parts) * segs
    if k < F:
        # Prefix sums of nf * segs in chunks of 64 lanes; the first sequence whose inclusive sum
        # exceeds k.
        base = 0
        for b0 in range(0, batch, 64):
            own = [parts[b][0] * segs for b in range(b0, min(b0 + 64, batch))]
            incl = np.cumsum(own)
            hit = [i for i, v in enumerate(incl) if base + v > k]
            if hit:
                first = hit[0]
                r = k - base - (incl[first] - own[first])
                return b0 + first, r // segs, r % segs
            base += int(incl[-1])
        raise AssertionError("unreachable")
    k -= F
    psz = [ps if np1 else 0 for _, np1, ps in parts]  # partial sizes in blocks, 0 for none
    count_ge = lambda sz: sum(1 for s in psz if s >= sz)  # noqa: E731
    r = k // segs
    if r >= count_ge(1):
        return -1, 0, 0
    lo, hi = 1, pb - 1
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if count_ge(mid) > r:
            lo = mid
        else:
            hi = mid - 1
    jth = r - count_ge(lo + 1)
    same = [b for b, s in enumerate(psz) if s == lo]
    b = same[jth]
    return b, parts[b][0], k % segs


def decode_uses_dense(batch, P, grid, ncu):
    """The launcher's choice (xs_decode_mfma.hip, launch_sw)."""
    small_items = P <= 128 and grid <= 4 * ncu
    return batch > 1 and batch <= 256 and not small_items


def decode_items(lens, mbps, BS, pb, maxp, segs):
    """The items the split decode must compute, from the definition (not from seq_partitions):
    every (b, p, seg) with p < min(ceil(L_b / P), max_partitions), of min(pb, blocks left) blocks."""
    out = {}
    for b, L in enumerate(lens):
        L = min(L, mbps * BS)
        nblk = -(-L // BS) if L > 0 else 0
        for p in range(min(-(-nblk // pb), maxp)):
            for seg in range(segs):
                out[(b, p, seg)] = min(pb, nblk - p * pb)
    return out


def check_decode_order(lens, BS, P, maxp, mbps, Hkv, chunks, ncu):
    pb = P // BS
    segs = Hkv * chunks
    grid = len(lens) * segs * maxp
    items = decode_items(lens, mbps, BS, pb, maxp, segs)
    taken = {}
    by_rank = []
    for k in range(grid):
        b, p, seg = dense_item(k, lens, mbps, BS, pb, maxp, segs, ncu, grid)
        if b < 0:
            continue
        key = (b, p, seg)
        assert key in items, f"id {k} maps to {key}, which is not an item"
        assert key not in taken, f"ids {taken[key]} and {k} both map to {key}"
        taken[key] = k
    assert len(taken) == len(items), f"{len(items) - len(taken)} items are never taken"
    # Rank order (undo the reversal): full partitions sequence-major, then partial ones by size.
    for r in range(len(items)):
        rnd, col = divmod(r, ncu)
        k = rnd * ncu + (ncu - 1 - col) if (rnd & 1) and (rnd + 1) * ncu <= grid else r
        by_rank.append(dense_item(k, lens, mbps, BS, pb, maxp, segs, ncu, grid))
    sizes = [items[x] for x in by_rank]
    nfull = sum(1 for s in sizes if s == pb)
    assert all(s == pb for s in sizes[:nfull])
    partial = sizes[nfull:]
    assert all(a >= b for a, b in zip(partial, partial[1:])), "partial partitions not by decreasing size"
    full_keys = by_rank[:nfull]
    assert full_keys == sorted(full_keys), "full partitions not sequence-major"
    ties = [(-items[x], x[0]) for x in by_rank[nfull:][::segs]]
    assert ties == sorted(ties), "partial partitions of equal size not by sequence"


@pytest.mark.parametrize("seed", range(12))
def test_decode_ranked_order_is_a_bijection(seed):
    rng = np.random.default_rng(seed)
    BS = int(rng.choice([16, 32]))
    P = BS * int(rng.choice([1, 2, 4, 8, 16, 64]))
    B = int(rng.choice([2, 3, 17, 63, 64, 65, 200, 256]))
    lens = rng.integers(0, 6 * P, B)
    lens[rng.random(B) < 0.1] = 0                           # empty sequences
    lens[rng.random(B) < 0.1] = P * rng.integers(1, 4)      # exact multiples: no partial partition
    mbps = -(-int(lens.max(initial=1)) // BS) + 1
    need = -(-int(lens.max(initial=1)) // P)
    maxp = max(1, need - int(rng.integers(0, 2)))            # sometimes cut by max_partitions
    Hkv, chunks = int(rng.choice([1, 2, 8])), int(rng.choice([1, 2]))
    ncu = int(rng.choice([7, 64, 256, 304]))
    check_decode_order(lens.tolist(), BS, P, maxp, mbps, Hkv, chunks, ncu)


def test_decode_ranked_order_edges():
    # Ties everywhere, all empty, a single partial, grids around CU multiples.
    check_decode_order([0] * 40, 16, 64, 1, 4, 2, 1, 64)
    check_decode_order([50] * 70, 16, 64, 1, 4, 2, 1, 64)
    check_decode_order([17] + [0] * 9, 16, 1024, 1, 2, 8, 1, 256)
    for ncu in (1, 5, 8, 35, 36, 37):
        check_decode_order([1, 100, 64, 65, 0, 31, 32, 33], 16, 32, 4, 8, 1, 1, ncu)
    # Every id an item, the last round odd and incomplete (12 ids, 8 CUs): that round keeps its order.
    check_decode_order([128, 128, 128], 16, 32, 4, 8, 1, 1, 8)
    check_decode_order([128, 128, 128], 16, 32, 4, 8, 2, 1, 5)


def test_decode_order_choice():
    # Partition-major ids: one sequence, more than 256, or small grids of small items; else ranked.
    assert not decode_uses_dense(1, 1024, 10_000, 256)
    assert not decode_uses_dense(257, 1024, 10_000, 256)
    assert not decode_uses_dense(8, 128, 768, 256)            # the GPT-2 bf16 batch
    assert decode_uses_dense(64, 1024, 4096, 256)             # the 64-sequence Qwen3-8B batch
    assert decode_uses_dense(4, 512, 2048, 256)               # the long-context batch
    assert decode_uses_dense(64, 128, 4096, 256)              # small items, but a large grid


# ----------------------------------------------------------------------------------------------
# Chunked prefill: xs_prefill.hip, ranked_piece (kv head fastest, then the rank).

ROWS_PER_GROUP = 256
TILE = 64


def row_block_tiles(s0, n, chunk, group, rb, mbps, BS):
    if s0 < 0 or n < 0 or n > chunk or s0 + n > mbps * BS:
        return 0
    rows_total = chunk * group
    rho0 = rb * ROWS_PER_GROUP
    i_hi = min((min(rho0 + ROWS_PER_GROUP, rows_total) - 1) // group, n - 1)
    return (s0 + i_hi) // TILE + 1 if i_hi >= rho0 // group else 0


def ranked_piece(k, starts, lens, chunk, group, mbps, BS, part_tiles):
    PT = part_tiles if part_tiles > 0 else 1 << 24
    RBN = -(-chunk * group // ROWS_PER_GROUP)
    nx = len(starts) * RBN
    nfull, last = [], []
    for x in range(nx):
        b, rb = divmod(x, RBN)
        nt = row_block_tiles(starts[b], lens[b], chunk, group, RBN - 1 - rb, mbps, BS)
        nfull.append(nt // PT)
        last.append(nt % PT if (nt % PT != 0 or nt == 0) else -1)
    F = sum(nfull)
    x = -1
    piece = 0
    if k < F:
        incl = np.cumsum(nfull)
        x = int(np.argmax(incl > k))
        piece = k - int(incl[x] - nfull[x])
    else:
        r = k - F
        count_ge = lambda sz: sum(1 for s in last if s >= sz)  # noqa: E731
        if r < count_ge(0):
            lo, hi = 0, max(max(last), 0)
            while lo < hi:
                mid = (lo + hi + 1) >> 1
                if count_ge(mid) > r:
                    lo = mid
                else:
                    hi = mid - 1
            jth = r - count_ge(lo + 1)
            x = [i for i, s in enumerate(last) if s == lo][jth]
            piece = nfull[x]
    if x < 0:
        return -1, 0, 0
    return x // RBN, RBN - 1 - x % RBN, piece


def check_prefill_order(starts, lens, chunk, group, mbps, BS, P, maxp):
    part_tiles = P // TILE if P else 0
    RBN = -(-chunk * group // ROWS_PER_GROUP)
    pieces = maxp if part_tiles else 1
    per_head = len(starts) * RBN * pieces  # the grid is this times the kv heads, kv head fastest
    items = {}
    for b in range(len(starts)):
        for rb in range(RBN):
            nt = row_block_tiles(starts[b], lens[b], chunk, group, rb, mbps, BS)
            PT = part_tiles if part_tiles else 1 << 24
            n_pieces = max(1, -(-nt // PT))
            for j in range(n_pieces):
                items[(b, rb, j)] = min(PT, nt - j * PT) if nt else 0
    taken = {}
    order = []
    for k in range(per_head):
        b, rb, piece = ranked_piece(k, starts, lens, chunk, group, mbps, BS, part_tiles)
        if b < 0:
            continue
        key = (b, rb, piece)
        assert key in items, f"id {k} maps to {key}, not an item"
        assert key not in taken, f"ids {taken[key]} and {k} both map to {key}"
        taken[key] = k
        order.append(key)
    assert len(taken) == len(items), f"{len(items) - len(taken)} pieces never taken"
    sizes = [items[x] for x in order]
    if part_tiles:
        nfull = sum(1 for x in order if items[x] == part_tiles and (x[2] + 1) * part_tiles <= row_block_tiles(
            starts[x[0]], lens[x[0]], chunk, group, x[1], mbps, BS))
        rest = sizes[nfull:]
    else:
        rest = sizes
    assert all(a >= b for a, b in zip(rest, rest[1:])), "pieces not largest first"


@pytest.mark.parametrize("seed", range(10))
def test_prefill_ranked_order_is_a_bijection(seed):
    rng = np.random.default_rng(100 + seed)
    BS = int(rng.choice([8, 16, 32]))
    group = int(rng.choice([1, 4, 8]))
    chunk = int(rng.choice([9, 64, 200, 512]))
    B = int(rng.integers(1, 9))
    starts = rng.integers(0, 3000, B).tolist()
    lens = rng.integers(0, chunk + 1, B).tolist()
    if B > 2:
        starts[1] = -5                           # an invalid sequence: its row blocks have no keys
    mbps = -(-(max(s + n for s, n in zip(starts, lens)) + 1) // BS) + 1
    RBN = -(-chunk * group // ROWS_PER_GROUP)
    if B * RBN > 256:
        pytest.skip("more than 256 row blocks per kv head take the fixed order")
    P = int(rng.choice([0, 64, 128, 512, 2048]))
    maxp = -(-mbps * BS // P) if P else 0
    check_prefill_order(starts, lens, chunk, group, mbps, BS, P, maxp)
