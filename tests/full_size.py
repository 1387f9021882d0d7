"""Whole-batch oracle references for the full-size workloads (test helper).

The device batches of the measured workloads are too large to hand to the
oracle in one piece, but every output row depends only on its request's
rows of the pools.  So each request's K/V rows are gathered on the device
through its page-table row, copied to the host, and the oracle is run on
them one (request, kv head) at a time with that head's group of query
heads, in a pool of threads (numpy releases the interpreter lock inside its
array work).  The result covers every output element of the batch.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle

WORKERS = max(1, min(16, os.cpu_count() or 1))


def _torch():
    import torch
    return torch


def _rows_host(pool, rows):
    """Pool rows [L, Hkv, d] on the host: float32 for bf16 pools (exact), the
    raw codes for 8-bit pools."""
    torch = _torch()
    t = pool[rows]
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def _q_host(q):
    torch = _torch()
    return (q.float() if q.dtype == torch.bfloat16 else q).cpu().numpy()


def _run(jobs):
    with cf.ThreadPoolExecutor(WORKERS) as ex:
        return [f.result() for f in [ex.submit(*j) for j in jobs]]


def decode_reference(db, layer: int = 0, q_len: int = 1, sage: bool = False, qk_codes: str = "e4m3"):
    """fp64 oracle output and lse of a device decode batch, every (row, head).

    q_len new tokens per request (rows request-major); bf16 batches go through
    ``paged_attention`` (causal over the new tokens), 8-bit ones through
    ``sage_decode`` (one token per request).  Returns (o [B·q_len, Hq, d],
    lse [B·q_len, Hq]) in float64.
    """
    lay = db.layout
    spec = lay.spec
    B, Hq, Hkv, d = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    G = Hq // Hkv
    q = _q_host(db.q)
    out = np.zeros((B * q_len, Hq, d), np.float64)
    lse = np.full((B * q_len, Hq), -np.inf, np.float64)
    sfq = db.sfq.cpu().numpy() if sage else None
    sfk = db.sfk.cpu().numpy() if sage else None
    sfv = db.sfv.cpu().numpy() if sage else None

    def one(b, g, K, V):
        L = K.shape[0]
        hs = slice(g * G, (g + 1) * G)
        rs = slice(b * q_len, (b + 1) * q_len)
        if sage:
            o, l = oracle.sage_decode(q[rs, hs], K[:, g:g + 1], V[:, g:g + 1], np.arange(L)[None], [L],
                                      sfq[b:b + 1, hs], sfk[b:b + 1, g:g + 1], sfv[b:b + 1, g:g + 1],
                                      spec.k_block, qk_codes=qk_codes)
        else:
            o, l = oracle.paged_attention(q[rs, hs], K[:, g:g + 1], V[:, g:g + 1], np.arange(L)[None], [L],
                                          [0, q_len])
        out[rs, hs] = o
        lse[rs, hs] = l

    torch = _torch()
    for b in range(B):
        L = int(lay.seq_lens[b])
        if L == 0:
            continue
        rows = db.req_to_token[b, :L].long()
        K = _rows_host(db.k_pools[layer], rows)
        V = _rows_host(db.v_pools[layer], rows)
        _run([(one, b, g, K, V) for g in range(Hkv)])
        del K, V
    torch.cuda.synchronize()
    return out, lse


def extend_reference(db, layer: int = 0, requests=None, sage: bool = False):
    """fp64 oracle output and lse of a device extend batch (bf16, or the 8-bit
    formula with ``sage``) for every new row of the listed requests (default:
    all).  Rows of other requests stay NaN.  Returns (o [T, Hq, d], lse [T, Hq])."""
    lay = db.layout
    spec = lay.spec
    Hq, Hkv, d = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    G = Hq // Hkv
    T = lay.total_q
    q = _q_host(db.q)
    out = np.full((T, Hq, d), np.nan)
    lse = np.full((T, Hq), np.nan)
    cu = lay.cu_seqlens_q
    sfq = db.sfq.cpu().numpy() if sage else None
    sfk = db.sfk.cpu().numpy() if sage else None
    sfv = db.sfv.cpu().numpy() if sage else None

    def one(b, g, K, V):
        L = K.shape[0]
        q0, q1 = int(cu[b]), int(cu[b + 1])
        hs = slice(g * G, (g + 1) * G)
        if sage:
            o, l = oracle.sage_extend(q[q0:q1, hs], K[:, g:g + 1], V[:, g:g + 1], np.arange(L)[None], [L],
                                      [0, q1 - q0], sfq[q0:q1, hs], sfk[b:b + 1, g:g + 1], sfv[b:b + 1, g:g + 1],
                                      spec.k_block)
        else:
            o, l = oracle.paged_attention(q[q0:q1, hs], K[:, g:g + 1], V[:, g:g + 1], np.arange(L)[None], [L],
                                          [0, q1 - q0])
        out[q0:q1, hs] = o
        lse[q0:q1, hs] = l

    reqs = range(spec.batch) if requests is None else requests
    for b in reqs:
        L = int(lay.seq_lens[b])
        if L == 0 or cu[b + 1] == cu[b]:
            continue
        rows = db.req_to_token[b, :L].long()
        K = _rows_host(db.k_pools[layer], rows)
        V = _rows_host(db.v_pools[layer], rows)
        _run([(one, b, g, K, V) for g in range(Hkv)])
        del K, V
    return out, lse


def block_sparse_reference(db, layer: int = 0, sage: bool = False, qk_codes: str = "e4m3"):
    """fp64 oracle of a device block-sparse decode batch, every (request,
    head): the dense page table and the listed blocks, as the definition
    reads (no compaction)."""
    lay = db.layout
    spec = lay.spec
    B, Hq, Hkv, d = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    G = Hq // Hkv
    q = _q_host(db.q)
    out = np.zeros((B, Hq, d), np.float64)
    lse = np.full((B, Hq), -np.inf, np.float64)
    indptr, indices = lay.blk_indptr, lay.blk_indices
    sfq = db.sfq.cpu().numpy() if sage else None
    sfk = db.sfk.cpu().numpy() if sage else None
    sfv = db.sfv.cpu().numpy() if sage else None

    def one(b, g, K, V):
        L = K.shape[0]
        hs = slice(g * G, (g + 1) * G)
        blocks = indices[indptr[b]:indptr[b + 1]]
        ptr = np.array([0, len(blocks)], np.int32)
        if sage:
            o, l = oracle.block_sparse_sage_decode(q[b:b + 1, hs], K[:, g:g + 1], V[:, g:g + 1], np.arange(L)[None],
                                                   [L], ptr, blocks, spec.sparse_block, sfq[b:b + 1, hs],
                                                   sfk[b:b + 1, g:g + 1], sfv[b:b + 1, g:g + 1], spec.k_block,
                                                   qk_codes=qk_codes)
        else:
            o, l = oracle.block_sparse_decode(q[b:b + 1, hs], K[:, g:g + 1], V[:, g:g + 1], np.arange(L)[None], [L],
                                              ptr, blocks, spec.sparse_block)
        out[b, hs] = o[0]
        lse[b, hs] = l[0]

    for b in range(B):
        L = int(lay.seq_lens[b])
        rows = db.req_to_token[b, :L].long()
        K = _rows_host(db.k_pools[layer], rows)
        V = _rows_host(db.v_pools[layer], rows)
        _run([(one, b, g, K, V) for g in range(Hkv)])
        del K, V
    return out, lse
