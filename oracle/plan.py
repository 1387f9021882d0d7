"""Re-derivation of the split / tile scheduling metadata (oracle; test infrastructure).

[SGLang-sched-meta] (intro, code §1-3 and the "why" part) hoists the split-KV
tile-scheduling metadata out of the per-layer attention call: it depends only
on the batch's sequence lengths (and, for varlen queries, cu_seqlens_q), so
it is computed once per batch and reused by every layer.  The pages do not
give the scheduling rule itself; the integer rule below is this library's
design, restated plainly so the GPU plan kernel can be compared with it bit
for bit.  Its pins are invariants, not values from the pages.

Decode rule (tile = 32 tokens):

* L_b is clamped to [0, max_kv_len]; tiles_b = ceil(L_b / 32).
* units = Hkv · ceil(G / 16) work items per split (one per kv head and
  16-row head group).  ``target_items`` is the number of split items the
  chunk is sized for: ceil(split_target / units) when the caller gives a
  split_target, otherwise the number of items whose waves the device holds
  at once (the library queries the decode kernel's occupancy; it is an
  input here and the GPU plan records it in its header).
* automatic chunk: the smallest c >= 1 with Σ_b max(1, ceil(tiles_b / c))
  <= target_items; if even c = max_b tiles_b gives more (every request is
  then one item), c = max(1, max_b tiles_b).
  fixed chunk (``kv_chunk`` tokens, a multiple of 32): c = kv_chunk / 32.
* splits_b = max(1, ceil(tiles_b / c)); split s covers tiles
  [⌊s·tiles_b/splits_b⌋, ⌊(s+1)·tiles_b/splits_b⌋), i.e. tokens
  [32·t0, min(32·t1, L_b)) (balanced, interior bounds on tile multiples).
* items are created request-major (b, s); a request with one split writes
  its output directly (part index -1), otherwise split s of request b owns
  partial slot split_off[b] + s with split_off the exclusive prefix sum.
  When there are more items than target_items the list is ordered by split
  length (tokens) descending, ties by creation order (longest first, so the
  short splits fill the tail); otherwise it stays in creation order.
* capacity (host-visible, never exceeded):
  automatic: min(max(target_items, B), B · max(1, ceil(max_kv_len / 32)));
  fixed: B · max(1, ceil(max_kv_len / kv_chunk)).

Extend rule: rows of a work item are (head, token) pairs of one kv head,
block_tokens = max(1, 256 // G) new tokens × G heads.  Request b contributes
ceil(n_b / block_tokens) items (b, t) with kv_end = min(p_b + min((t+1)·block,
n_b), L_b), p_b = L_b - n_b; items are ordered by kv_end descending (longest
causal range first), ties by creation order.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

DECODE_TILE = 32
EXTEND_BLOCK_M = 256  # rows ((head, token) pairs) per extend work item


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def decode_target_items(num_kv_heads: int, group: int, split_target: int, resident_items: int) -> int:
    units = num_kv_heads * _ceil_div(group, 16)
    return max(1, _ceil_div(split_target, units) if split_target > 0 else resident_items)


def decode_capacity(batch: int, max_kv_len: int, target_items: int, kv_chunk: int = 0) -> int:
    if kv_chunk > 0:
        return batch * max(1, _ceil_div(max_kv_len, kv_chunk))
    max_tiles = max(1, _ceil_div(max_kv_len, DECODE_TILE))
    return min(max(target_items, batch), batch * max_tiles)


def plan_decode(seq_lens, max_kv_len: int, target_items: int, kv_chunk: int = 0) -> Dict:
    L = np.clip(np.asarray(seq_lens, dtype=np.int64), 0, max_kv_len)
    B = len(L)
    tiles = [_ceil_div(int(x), DECODE_TILE) for x in L]

    def count_items(c):
        return sum(max(1, _ceil_div(t, c)) for t in tiles)

    if kv_chunk > 0:
        assert kv_chunk % DECODE_TILE == 0
        chunk = kv_chunk // DECODE_TILE
    else:
        top = max([1] + tiles)
        chunk = next((c for c in range(1, top + 1) if count_items(c) <= target_items), top)
    splits = [max(1, _ceil_div(t, chunk)) for t in tiles]
    split_off = [0]
    for s in splits:
        split_off.append(split_off[-1] + s)
    items = []
    for b in range(B):
        for s in range(splits[b]):
            t0 = (s * tiles[b]) // splits[b]
            t1 = ((s + 1) * tiles[b]) // splits[b]
            kb = t0 * DECODE_TILE
            ke = min(t1 * DECODE_TILE, int(L[b]))
            part = split_off[b] + s if splits[b] > 1 else -1
            items.append((b, kb, ke, part))
    if len(items) > target_items:
        order = sorted(range(len(items)), key=lambda i: (-(items[i][2] - items[i][1]), i))
        items = [items[i] for i in order]
    cap = decode_capacity(B, max_kv_len, target_items, kv_chunk)
    return {"chunk_tiles": chunk, "splits": np.array(splits, np.int64),
            "split_off": np.array(split_off, np.int64), "target_items": target_items,
            "items": np.array(items, np.int64).reshape(-1, 4), "capacity": cap}


def extend_block_tokens(group: int) -> int:
    return max(1, EXTEND_BLOCK_M // group)


def extend_capacity(batch: int, max_total_q: int, group: int) -> int:
    bt = extend_block_tokens(group)
    return _ceil_div(max_total_q, bt) + batch


def plan_extend(seq_lens, cu_seqlens_q, group: int, max_kv_len: int, total_q: int) -> Dict:
    L = np.clip(np.asarray(seq_lens, dtype=np.int64), 0, max_kv_len)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    B = len(L)
    bt = extend_block_tokens(group)
    items = []
    for b in range(B):
        q0 = min(max(int(cu[b]), 0), total_q)
        q1 = min(max(int(cu[b + 1]), q0), total_q)
        n = q1 - q0
        p = int(L[b]) - n
        for t in range(_ceil_div(n, bt)):
            kv_end = min(max(p + min((t + 1) * bt, n), 0), int(L[b]))
            items.append((b, t, kv_end))
    order = sorted(range(len(items)), key=lambda i: (-items[i][2], i))
    arr = np.array([items[i] for i in order], np.int64).reshape(-1, 3)
    return {"block_tokens": bt, "items": arr,
            "capacity": extend_capacity(B, total_q, group)}
