"""Block-sparse decode in float64 — TEST INFRASTRUCTURE ONLY.

[FlashInfer-Sage] (the README block and the list of measured cases) runs the
decode kernel in a dense and in a block-sparse mode, with bf16 or with the
8-bit formula, and measures the "exact" block-sparse mode at densities 0.125
and 0.10.  The page gives no mask format.  Reading taken here (the plainest
one the rest supports):

* one block mask per request, shared by all heads: a list of KV block numbers,
  a block being ``block_size`` consecutive logical positions of the request
  (CSR over the batch: ``blk_indptr`` [B + 1], ``blk_indices`` [nnz]);
* "exact": the query of request b attends to key j (j < L_b) exactly when
  ⌊j / block_size⌋ is listed, with the ordinary softmax over those keys and
  nothing else; a block number outside [0, ⌈L_b / block_size⌉) selects no key;
* a request with no selected key gives O = 0 and lse = -inf (as an empty
  request), or v_mean on the 8-bit path;
* dense decode is the mask that lists every block.

The mask is applied here on logical positions as the definition reads: every
score of the request is formed and the unlisted ones are set to -inf before
the softmax; no compaction of positions is done.  On the 8-bit path sfK is
indexed by the key's logical position, ⌊j / k_block⌋.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .e4m3 import e4m3_decode, e4m3_encode
from .sage import qk_values


def key_mask(L: int, blocks, block_size: int) -> np.ndarray:
    """Boolean [L]: key j is attended iff ⌊j / block_size⌋ is in ``blocks``."""
    listed = {int(k) for k in np.asarray(blocks).ravel()}
    return np.array([(j // block_size) in listed for j in range(L)], dtype=bool)


def _request_blocks(blk_indptr, blk_indices, b):
    e0, e1 = int(blk_indptr[b]), int(blk_indptr[b + 1])
    return np.asarray(blk_indices[e0:e1])


def block_sparse_decode(q, k_pool, v_pool, req_to_token, seq_lens, blk_indptr, blk_indices,
                        block_size: int, sm_scale: Optional[float] = None, req_pool_indices=None):
    """bf16 (or any float) decode over the selected blocks.

    q [B, Hq, d]; pools [slots, Hkv, d]; req_to_token [rows, >= max L];
    returns (o [B, Hq, d], lse [B, Hq]) in float64, lse = m + ln l.
    """
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, d), np.float64)
    lse = np.full((B, Hq), -np.inf, np.float64)
    for b in range(B):
        row = b if req_pool_indices is None else int(req_pool_indices[b])
        L = int(seq_lens[b])
        keep = key_mask(L, _request_blocks(blk_indptr, blk_indices, b), block_size)
        if not keep.any():
            continue
        slots = np.asarray(req_to_token[row, :L], np.int64)
        K = np.asarray(k_pool, np.float64)[slots]  # [L, Hkv, d]
        V = np.asarray(v_pool, np.float64)[slots]
        for h in range(Hq):
            g = h // G
            s = sm_scale * (K[:, g, :] @ q[b, h])
            s = np.where(keep, s, -np.inf)
            m = s.max()
            p = np.exp(s - m)  # exactly 0 on unlisted keys
            l = p.sum()
            out[b, h] = (p @ V[:, g, :]) / l
            lse[b, h] = m + math.log(l)
    return out, lse


def block_sparse_sage_decode(q8, k8_pool, v8_pool, req_to_token, seq_lens, blk_indptr, blk_indices,
                             block_size: int, sfq, sfk, sfv, k_block: int, sm_scale: Optional[float] = None,
                             v_mean=None, quantize_p: bool = True, req_pool_indices=None,
                             qk_codes: str = "e4m3"):
    """The 8-bit formula of [FlashInfer-Sage] (README block) over the selected
    blocks: S = sm_scale·sfQ[b,h]·sfK[b,g,⌊j/k_block⌋]·(q8·k8_j) on listed keys,
    m the row max over them, P8 = E4M3(448·e^{S-m}), l = Σ e^{S-m} (unquantised),
    O = sfV·(Σ P8_j·v8_j)/(448·l) (+ v_mean).  Same shapes and ``qk_codes``
    as ``sage_decode``.
    """
    q8 = np.asarray(q8)
    B, Hq, d = q8.shape
    Hkv = k8_pool.shape[1]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, d), np.float64)
    lse = np.full((B, Hq), -np.inf, np.float64)
    for b in range(B):
        row = b if req_pool_indices is None else int(req_pool_indices[b])
        L = int(seq_lens[b])
        keep = key_mask(L, _request_blocks(blk_indptr, blk_indices, b), block_size)
        if not keep.any():
            if v_mean is not None:
                out[b] = np.repeat(np.asarray(v_mean[b], np.float64), G, axis=0)
            continue
        slots = np.asarray(req_to_token[row, :L], np.int64)
        K = qk_values(np.asarray(k8_pool)[slots], qk_codes)
        V = e4m3_decode(np.asarray(v8_pool)[slots])
        kblk = np.arange(L) // k_block
        for h in range(Hq):
            g = h // G
            dots = K[:, g, :] @ qk_values(q8[b, h], qk_codes)
            S = sm_scale * float(sfq[b, h]) * np.asarray(sfk[b, g, kblk], np.float64) * dots
            S = np.where(keep, S, -np.inf)
            m = S.max()
            p = np.exp(S - m)
            l = p.sum()
            P8 = 448.0 * p
            if quantize_p:
                P8 = e4m3_decode(e4m3_encode(P8))
            o = np.asarray(sfv[b, g], np.float64) * (P8 @ V[:, g, :]) / (448.0 * l)
            if v_mean is not None:
                o = o + np.asarray(v_mean[b, g], np.float64)
            out[b, h] = o
            lse[b, h] = m + math.log(l)
    return out, lse
