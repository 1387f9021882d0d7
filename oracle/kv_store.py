"""Writing new tokens' K/V rows into their slots (oracle; test infrastructure).

[SGLang-FA-DE] (KV-cache paragraph) says the cache is read and updated
within the forward methods; [SGLang-FA-basics] (KV-cache part) gives the
second pool level, slot -> per-layer K/V data.  Storing token t therefore
means pool[slot_t] = new_t for every kv head, as a plain copy.
"""
from __future__ import annotations

import numpy as np


def kv_store(pool, new_rows, slots):
    """Return a copy of ``pool`` ([slots, Hkv, d]) with ``pool[slots[t]] = new_rows[t]``."""
    out = np.array(pool, copy=True)
    out[np.asarray(slots, dtype=np.int64)] = new_rows
    return out
