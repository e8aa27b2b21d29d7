"""Oracle of KV block swap-out / swap-in between the paged pools and host swap space.
TEST INFRASTRUCTURE ONLY (same rules as ``oracle.paged_attention``).

Source: the xserv README on the compare page xserv compare phase10...cf1e9e41 (status list:
paged KV cache with CPU swap-out / swap-in for elastic GPU memory; server option
``--swap-space-gb``: pinned host memory for swapped-out KV, 0 turns it off). The pages show no
code for it, so the operation is the plainest one that reading supports:

* Swap space: host arrays k_host, v_host of shape [num_slots, num_kv_heads, block_size, head_dim]
  in the pools' dtype. One slot holds one pool block, all kv heads.
* Swap-out of pairs (src_block[i], dst_slot[i]): slot dst_slot[i] becomes a bit copy of pool block
  src_block[i], K and V.
* Swap-in of pairs (src_slot[i], dst_block[i]): pool block dst_block[i] becomes a bit copy of slot
  src_slot[i], K and V.
* A pair with an index outside its array is skipped. Nothing else changes. (Two pairs with the
  same destination are not allowed: their order is not fixed.)
"""

from __future__ import annotations

import numpy as np


def swap_out(k_cache, v_cache, k_host, v_host, src_blocks, dst_slots):
    """Returns new (k_host, v_host) after the swap-out; the inputs are left as they were."""
    k_out, v_out = np.array(k_host, copy=True), np.array(v_host, copy=True)
    NB, S = k_cache.shape[0], k_host.shape[0]
    for blk, slot in zip(np.asarray(src_blocks).tolist(), np.asarray(dst_slots).tolist()):
        if 0 <= blk < NB and 0 <= slot < S:
            k_out[slot] = k_cache[blk]
            v_out[slot] = v_cache[blk]
    return k_out, v_out


def swap_in(k_host, v_host, k_cache, v_cache, src_slots, dst_blocks):
    """Returns new (k_cache, v_cache) after the swap-in; the inputs are left as they were."""
    k_out, v_out = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    NB, S = k_cache.shape[0], k_host.shape[0]
    for slot, blk in zip(np.asarray(src_slots).tolist(), np.asarray(dst_blocks).tolist()):
        if 0 <= blk < NB and 0 <= slot < S:
            k_out[blk] = k_host[slot]
            v_out[blk] = v_host[slot]
    return k_out, v_out
