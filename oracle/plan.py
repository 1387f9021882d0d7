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
* units = Hkv · ceil(G / 16) waves per item (one per kv head and 16-row head
  group).  ``target_items`` is the number of chunks the work is cut into at
  most: ceil(split_target / units) when the caller gives a split_target,
  otherwise the number of items whose waves the device holds at once (the
  library queries the decode kernel's occupancy; it is an input here and the
  GPU plan records it in its header).
* automatic (kv_chunk = 0), balanced chunks over tiles of ``tile`` tokens
  (the decode kernel's tile: 32 for bf16 K/V, 64 for 8-bit; "32" below
  stands for it in this mode): request b occupies global tiles
  [o_b, o_b + tiles_b) with o the exclusive prefix sum of tiles, T = Σ tiles_b.
  Chunk size C = max(1, ceil(T / target_items)); nchunks = max(1, ceil(T / C)).
  Chunk c covers global tiles [c·C, (c+1)·C).  Request b is cut into the
  segments it shares with the chunks it overlaps: segment s lies in chunk
  ⌊o_b / C⌋ + s and covers tokens [32·(g0 - o_b), min(32·(g1 - o_b), L_b)),
  g0/g1 the overlap's global tile bounds.  An empty request is one empty
  segment in chunk min(⌊o_b / C⌋, nchunks - 1).  Segments are listed request
  by request (so chunks are non-decreasing along the list) and chunk c owns
  the segments [tab[c], tab[c+1]).
* fixed chunk (``kv_chunk`` tokens, a multiple of 32): c = kv_chunk / 32,
  splits_b = max(1, ceil(tiles_b / c)); split s covers tiles
  [⌊s·tiles_b/splits_b⌋, ⌊(s+1)·tiles_b/splits_b⌋), i.e. tokens
  [32·t0, min(32·t1, L_b)).  Each split is its own chunk; when there are more
  splits than target_items they are ordered by length (tokens) descending,
  ties by creation order, otherwise they stay in request order.
* a request with one segment writes its output directly (part index -1);
  otherwise segment s of request b owns partial slot split_off[b] + s, with
  split_off the exclusive prefix sum of segments per request.
* capacity (host-visible, never exceeded):
  automatic: min(target_items + B, B · max(1, ceil(max_kv_len / tile)));
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


def decode_capacity(batch: int, max_kv_len: int, target_items: int, kv_chunk: int = 0,
                    tile: int = DECODE_TILE) -> int:
    if kv_chunk > 0:
        return batch * max(1, _ceil_div(max_kv_len, kv_chunk))
    max_tiles = max(1, _ceil_div(max_kv_len, tile))
    return min(target_items + batch, batch * max_tiles)


def plan_decode(seq_lens, max_kv_len: int, target_items: int, kv_chunk: int = 0,
                tile: int = DECODE_TILE) -> Dict:
    L = [int(x) for x in np.clip(np.asarray(seq_lens, dtype=np.int64), 0, max_kv_len)]
    B = len(L)
    if kv_chunk > 0:
        tile = DECODE_TILE
    tiles = [_ceil_div(x, tile) for x in L]
    items, seg_chunk = [], []
    splits = []
    if kv_chunk > 0:
        assert kv_chunk % DECODE_TILE == 0
        chunk = kv_chunk // DECODE_TILE
        for b in range(B):
            n = max(1, _ceil_div(tiles[b], chunk))
            splits.append(n)
            for s in range(n):
                t0 = (s * tiles[b]) // n
                t1 = ((s + 1) * tiles[b]) // n
                items.append([b, t0 * DECODE_TILE, min(t1 * DECODE_TILE, L[b]), s])
        if len(items) > target_items:
            order = sorted(range(len(items)), key=lambda i: (-(items[i][2] - items[i][1]), i))
            items = [items[i] for i in order]
        nchunks = len(items)
        chunk_tab = list(range(nchunks + 1))
    else:
        T = sum(tiles)
        chunk = max(1, _ceil_div(T, target_items))
        nchunks = max(1, _ceil_div(T, chunk))
        o = 0
        for b in range(B):
            if tiles[b] == 0:
                splits.append(1)
                items.append([b, 0, 0, 0])
                seg_chunk.append(min(o // chunk, nchunks - 1))
                continue
            first_c, last_c = o // chunk, (o + tiles[b] - 1) // chunk
            splits.append(last_c - first_c + 1)
            for s, c in enumerate(range(first_c, last_c + 1)):
                g0 = max(o, c * chunk)
                g1 = min(o + tiles[b], (c + 1) * chunk)
                items.append([b, (g0 - o) * tile, min((g1 - o) * tile, L[b]), s])
                seg_chunk.append(c)
            o += tiles[b]
        chunk_tab = [next((i for i, c in enumerate(seg_chunk) if c >= cc), len(items))
                     for cc in range(nchunks)] + [len(items)]
    split_off = [0]
    for n in splits:
        split_off.append(split_off[-1] + n)
    for it in items:  # segment index -> partial slot, or -1 for a whole request
        b, s = it[0], it[3]
        it[3] = split_off[b] + s if splits[b] > 1 else -1
    cap = decode_capacity(B, max_kv_len, target_items, kv_chunk, tile)
    assert len(items) <= cap
    return {"chunk_tiles": chunk, "tile": tile, "splits": np.array(splits, np.int64),
            "split_off": np.array(split_off, np.int64), "target_items": target_items,
            "items": np.array(items, np.int64).reshape(-1, 4), "capacity": cap,
            "nchunks": nchunks, "chunk_tab": np.array(chunk_tab, np.int64)}


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
