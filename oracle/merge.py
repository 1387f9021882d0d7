"""Log-sum-exp merge of split-KV partial results (oracle; test infrastructure).

Split-KV decode ([SGLang-sched-meta], intro and code §3: scheduling metadata
that cuts each request's KV range into chunks) computes, for each chunk s,
the normalised partial output O_s and lse_s = log Σ_{j∈s} exp(S_j).  The
pages do not spell out how the chunks are recombined; the plain reading is
exact softmax algebra: with lse = log Σ_s exp(lse_s),

    O = Σ_s exp(lse_s - lse) · O_s.

A chunk with no keys has lse_s = -inf and contributes nothing.
"""
from __future__ import annotations

import numpy as np


def lse_merge(outs, lses):
    """Merge partials. outs: [S, ..., d]; lses: [S, ...] (float64 arrays).

    Returns (O [..., d], lse [...]).  All-empty inputs give O = 0, lse = -inf.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max(axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Ms), 0.0)  # [S, ...]
    tot = w.sum(axis=0)
    lse = np.where(finite, Ms + np.log(np.where(finite, tot, 1.0)), -np.inf)
    wn = np.where(finite, w / np.where(finite, tot, 1.0), 0.0)
    O = (wn[..., None] * outs).sum(axis=0)
    return O, lse
