"""8-bit batches whose row maximum sits at the first key (test helper).

The 8-bit kernels quantise P against the running maximum of the scores they
have read so far.  When every row's maximum is at position 0 (in the first
tile read) and a request is not split, that running maximum is the row's
final maximum from the first tile on, so the kernels' E4M3 codes of P are
the oracle's, and the only differences left are fp32 and bf16 roundings.

``put_row_max_first`` sets the component of every query row of a (request,
kv head) along a random direction w to one shared value (so all those rows
project equally on w) and rewrites position 0's K codes to c·w, with c just
large enough that position 0 out-scores every other key for each of those
rows.  Position 0 then leads each row's scores by a similar margin, and a
small ``sm_scale`` in the tests keeps every probability a normal E4M3 value.
"""
from __future__ import annotations

import numpy as np

import oracle


def _encode(x, qk_codes):
    if qk_codes == "int8":
        return np.clip(np.rint(x), -127, 127).astype(np.int8)
    return oracle.e4m3_encode(np.clip(x, -448.0, 448.0))


def put_row_max_first(hb, qk_codes: str = "e4m3", margin: float = 0.05, seed: int = 0):
    """In place on a host 8-bit batch (decode or extend); returns the
    smallest relative gap, over all rows, between position 0's raw score and
    the largest other one (positive by construction)."""
    lay = hb.layout
    spec = lay.spec
    G = spec.num_q_heads // spec.num_kv_heads
    d = spec.head_dim
    kb = spec.k_block
    cu = lay.cu_seqlens_q
    rng = np.random.default_rng(seed)
    worst = np.inf
    for b in range(spec.batch):
        L = int(lay.seq_lens[b])
        rows = np.arange(int(cu[b]), int(cu[b + 1]))  # the request's query rows (decode: one per new token)
        if L < 2 or len(rows) == 0:
            continue
        slots = lay.req_to_token[b, :L]
        sk = hb.sfk[b][:, np.arange(L) // kb]  # [Hkv, L]
        for g in range(spec.num_kv_heads):
            heads = slice(g * G, (g + 1) * G)
            w = rng.standard_normal(d)
            w /= np.linalg.norm(w)
            qv0 = oracle.qk_values(hb.q_codes[rows, heads], qk_codes)  # [n, G, d]
            rms = np.sqrt((qv0 ** 2).mean(axis=-1, keepdims=True))
            K = oracle.qk_values(hb.k_codes[slots[1:], g], qk_codes)
            limit = 127.0 if qk_codes == "int8" else 448.0
            found = False
            lift = 3.0
            for _ in range(12):  # a larger shared component until c·w fits the codes
                along = (qv0 @ w)[..., None] * w  # [n, G, d]
                qc = _encode(qv0 - along + lift * float(rms.mean()) * w, qk_codes)
                qv = oracle.qk_values(qc, qk_codes).reshape(-1, d)
                others = (K @ qv.T) * sk[g, 1:, None]  # raw scores up to each row's positive scale
                top = others.max(axis=0)
                c = 1.0
                while np.abs(c * w).max() <= limit and np.all(qv @ w > 0):
                    k0 = _encode(c * w, qk_codes)
                    gap = sk[g, 0] * (oracle.qk_values(k0, qk_codes) @ qv.T) - top
                    if np.all(gap > margin * np.abs(top) + 1e-9):
                        found = True
                        break
                    c *= 1.05
                if found:
                    break
                lift *= 1.5
            if not found:
                raise AssertionError(f"no position-0 key dominates request {b}, kv head {g}")
            worst = min(worst, float((gap / np.maximum(np.abs(top), 1e-9)).min()))
            hb.q_codes[rows, heads] = qc
            hb.k_codes[slots[0], g] = k0
    hb.k_new_codes = hb.k_codes[lay.new_slots].copy()
    return worst
