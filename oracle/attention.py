"""Materialising paged attention in float64 (oracle; test infrastructure only).

Definition followed ([FA-vs-PA], FlashAttention §1): for queries Q and keys K,
V of one head, S = Q·Kᵀ scaled by 1/sqrt(d_k), P = row-softmax(S), O = P·V,
with the full score matrix S held in memory.  Tiling ([FA-vs-PA],
FlashAttention §2) changes where S lives, never its value, so this plain
form is the reference for both the tiled extend and the split-KV decode.

Two-level lookup ([SGLang-FA-basics], KV-cache part; [SGLang-FA-DE], the
KV-cache paragraph): a request row of ``req_to_token`` maps token position j
to a KV slot; the per-layer pools map a slot to a K row and a V row
([slots, Hkv, d]).  The oracle reads one slot per position and never assumes
that a page holds consecutive slots.

Forward modes ([SGLang-FA-basics]; [SGLang-FA-DE], forward-mode paragraph):
EXTEND appends n_b new tokens to a cached prefix of p_b tokens; DECODE is the
case n_b = 1.  Readings where the pages are silent:

* ``seq_lens[b]`` = L_b counts the new tokens (the length attended after the
  new K/V rows are stored), so p_b = L_b - n_b.
* Causal alignment is bottom-right: new token i sits at absolute position
  p_b + i and sees keys 0 .. p_b + i.
* Query head h reads kv head h // G with G = Hq / Hkv (contiguous groups).
* ``sm_scale`` defaults to 1/sqrt(d).
* A request with L_b = 0 in decode yields O = 0 and lse = -inf.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def paged_attention(q, k_pool, v_pool, req_to_token, seq_lens, cu_seqlens_q,
                    sm_scale: Optional[float] = None, req_pool_indices=None,
                    return_probs: bool = False):
    """Causal attention of new tokens over their request's paged KV, in fp64.

    q: [T, Hq, d]; k_pool, v_pool: [slots, Hkv, d]; req_to_token: [rows, stride]
    int; seq_lens: [B]; cu_seqlens_q: [B+1] (decode: 0..B).
    Returns (o [T, Hq, d] float64, lse [T, Hq] float64[, probs list]) where
    ``probs[b][h]`` is the [n_b, L_b] probability matrix.
    """
    q = np.asarray(q)
    T, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    B = len(seq_lens)
    out = np.zeros((T, Hq, d), dtype=np.float64)
    lse = np.full((T, Hq), -np.inf, dtype=np.float64)
    probs = [] if return_probs else None
    for b in range(B):
        row = b if req_pool_indices is None else int(req_pool_indices[b])
        L = int(seq_lens[b])
        q0, q1 = int(cu[b]), int(cu[b + 1])
        n = q1 - q0
        p = L - n
        per_head = []
        if n == 0:
            if return_probs:
                probs.append(per_head)
            continue
        if L == 0:
            # no keys at all: zero output, lse = -inf (already initialised)
            if return_probs:
                probs.append([np.zeros((n, 0)) for _ in range(Hq)])
            continue
        slots = np.asarray(req_to_token[row, :L], dtype=np.int64)
        K = np.asarray(k_pool[slots], dtype=np.float64)  # [L, Hkv, d]
        V = np.asarray(v_pool[slots], dtype=np.float64)
        i = np.arange(n)[:, None]
        j = np.arange(L)[None, :]
        visible = j <= p + i  # [n, L]
        for h in range(Hq):
            g = h // G
            Qh = np.asarray(q[q0:q1, h], dtype=np.float64)  # [n, d]
            S = sm_scale * (Qh @ K[:, g, :].T)  # [n, L], materialised
            S = np.where(visible, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            l = E.sum(axis=1, keepdims=True)
            P = E / l
            out[q0:q1, h] = P @ V[:, g, :]
            lse[q0:q1, h] = (m + np.log(l))[:, 0]
            if return_probs:
                per_head.append(P)
        if return_probs:
            probs.append(per_head)
    if return_probs:
        return out, lse, probs
    return out, lse

