"""8-bit scaled ("Sage") decode attention in float64 (oracle; test infrastructure).

What is computed ([FlashInfer-Sage], code §1 and the README "Sage attention"
block), for one query row and the keys it sees: each score is the dot product
of the row's Q codes with a key's K codes, multiplied by the Q scale of the
row's block and by the K scale of the key's block.  The probabilities
exp(score - row max) are kept as E4M3 codes of 448 times their value; the
output channel d is the sum over keys of those codes times the key's V code
in channel d, divided by 448 times the row sum l of the unquantised
probabilities, times the channel's V scale (plus an optional per-channel
mean of V).

Scale conventions ([FlashInfer-Sage], code §1 and §4): the caller quantises
and supplies the scales; Q and K scales enter before the row max and the
exponential; V scales apply per channel after the sum; scale values are not
checked.

Readings where the pages are silent or at odds:

* The 8-bit formula carries no 1/sqrt(d) although the attention definition
  ([FA-vs-PA], FlashAttention §1) does: ``sm_scale`` multiplies the
  dequantised S (``sm_scale=1`` gives the formula literally).
* Dividing by 448·l only makes sense if P8 holds the *unnormalised*
  exp(S - m), so l is the float sum of the unquantised p = exp(S - m), and
  m is the row max of S.  This oracle takes m as the final row max.
* blkK(c) = c // k_block on the logical position c in the request; sfK is
  [B, Hkv, nblk]; decode has one query row per request so sfQ is [B, Hq];
  sfV and v_mean are [B, Hkv, d].
* E4M3 is the OCP E4M3FN variant (largest finite value 448).
* INT8 Q and K ([FlashInfer-Sage], code §3 and §4: Q/K may be INT8, whose
  scores accumulate in 32-bit and enter the softmax as fp32): the same
  formula with Q8 and K8 read as two's-complement integers (``qk_codes=
  "int8"``).  The pages name INT8 for Q and K only, so V8 and P8 stay E4M3.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .e4m3 import e4m3_decode, e4m3_encode


def qk_values(codes, qk_codes: str = "e4m3"):
    """Exact float64 values of Q or K codes: E4M3 bytes, or two's-complement
    int8 ([FlashInfer-Sage], code §3) for ``qk_codes="int8"``."""
    c = np.asarray(codes)
    if qk_codes == "e4m3":
        return e4m3_decode(c)
    if qk_codes != "int8":
        raise ValueError(f"qk_codes must be 'e4m3' or 'int8', got {qk_codes!r}")
    if c.dtype == np.uint8:
        c = c.view(np.int8)
    if c.dtype != np.int8:
        raise ValueError("int8 codes must be an int8 or uint8 array")
    return c.astype(np.float64)


def sage_decode(q8, k8_pool, v8_pool, req_to_token, seq_lens, sfq, sfk, sfv,
                k_block: int, sm_scale: Optional[float] = None, v_mean=None,
                quantize_p: bool = True, req_pool_indices=None, qk_codes: str = "e4m3"):
    """One query row per request. q8: [B, Hq, d] uint8 codes; pools [slots, Hkv, d].
    ``qk_codes``: how q8 and the K pool's bytes read ("e4m3" or "int8").

    Returns (o [B, Hq, d] float64, lse [B, Hq] float64) with lse = m + ln l in
    the (scaled) S domain.  ``quantize_p=False`` keeps 448·p unrounded.
    """
    q8 = np.asarray(q8)
    B, Hq, d = q8.shape
    Hkv = k8_pool.shape[1]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        row = b if req_pool_indices is None else int(req_pool_indices[b])
        L = int(seq_lens[b])
        if L == 0:
            if v_mean is not None:
                out[b] = np.repeat(np.asarray(v_mean[b], np.float64), G, axis=0)
            continue
        slots = np.asarray(req_to_token[row, :L], dtype=np.int64)
        K = qk_values(np.asarray(k8_pool)[slots], qk_codes)  # [L, Hkv, d] exact
        V = e4m3_decode(np.asarray(v8_pool)[slots])
        blk = np.arange(L) // k_block
        for h in range(Hq):
            g = h // G
            qv = qk_values(q8[b, h], qk_codes)  # [d]
            dots = K[:, g, :] @ qv  # exact in fp64 (4-bit significands, or integers below 2^22)
            S = sm_scale * float(sfq[b, h]) * np.asarray(sfk[b, g, blk], np.float64) * dots
            m = S.max()
            p = np.exp(S - m)
            l = p.sum()
            P8 = 448.0 * p
            if quantize_p:
                P8 = e4m3_decode(e4m3_encode(P8))
            acc = P8 @ V[:, g, :]  # [d]
            o = np.asarray(sfv[b, g], np.float64) * acc / (448.0 * l)
            if v_mean is not None:
                o = o + np.asarray(v_mean[b, g], np.float64)
            out[b, h] = o
            lse[b, h] = m + math.log(l)
    return out, lse


def sage_extend(q8, k8_pool, v8_pool, req_to_token, seq_lens, cu_seqlens_q, sfq, sfk, sfv,
                k_block: int, sm_scale: Optional[float] = None, v_mean=None,
                quantize_p: bool = True, req_pool_indices=None, qk_codes: str = "e4m3"):
    """The same 8-bit formula for the new-token rows of an extend batch.

    q8: [T, Hq, d] codes, rows request-major (cu_seqlens_q); sfq: [T, Hq] (one
    Q block per row, the page's default q_block = 1); sfk [B, Hkv, nblk], sfv
    and v_mean [B, Hkv, d].  New token i of request b sits at absolute
    position p_b + i (p_b = L_b - n_b) and sees keys 0 .. p_b + i (causal,
    bottom-right aligned, as the bf16 extend).  Returns (o [T, Hq, d],
    lse [T, Hq]) in float64.
    """
    q8 = np.asarray(q8)
    T, Hq, d = q8.shape
    Hkv = k8_pool.shape[1]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    out = np.zeros((T, Hq, d), dtype=np.float64)
    lse = np.full((T, Hq), -np.inf, dtype=np.float64)
    for b in range(len(seq_lens)):
        row = b if req_pool_indices is None else int(req_pool_indices[b])
        q0, q1 = int(cu[b]), int(cu[b + 1])
        L = int(seq_lens[b])
        p0 = L - (q1 - q0)
        slots = np.asarray(req_to_token[row, :L], dtype=np.int64)
        K = qk_values(np.asarray(k8_pool)[slots], qk_codes)  # [L, Hkv, d] exact
        V = e4m3_decode(np.asarray(v8_pool)[slots])
        blk = np.arange(L) // k_block
        for t in range(q0, q1):
            vis = p0 + (t - q0) + 1  # keys 0 .. p_b + i
            for h in range(Hq):
                g = h // G
                dots = K[:vis, g, :] @ qk_values(q8[t, h], qk_codes)
                S = sm_scale * float(sfq[t, h]) * np.asarray(sfk[b, g, blk[:vis]], np.float64) * dots
                m = S.max()
                p = np.exp(S - m)
                l = p.sum()
                P8 = 448.0 * p
                if quantize_p:
                    P8 = e4m3_decode(e4m3_encode(P8))
                o = np.asarray(sfv[b, g], np.float64) * (P8 @ V[:vis, g, :]) / (448.0 * l)
                if v_mean is not None:
                    o = o + np.asarray(v_mean[b, g], np.float64)
                out[t, h] = o
                lse[t, h] = m + math.log(l)
    return out, lse
