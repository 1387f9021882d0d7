"""CPU oracle for paged-KV attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The library
(``flashattention_paged_kv_amd``) never calls it, shares no code with it and
has no CPU fallback through it.

Everything here is plain numpy in float64 and materialises the full score
matrix, which is exactly the "standard attention" that tiled FlashAttention
avoids; tiling only changes where S lives, not its value.  Each function
names the passage of the source pages it follows.  The source pages are:

* [SGLang-FA-basics]  "Implement Flash Attention Back End in SGLang – Basics
  and KV Cache" (hnr.moe summary): forward modes, the two-level KV pool.
* [SGLang-sched-meta] "SGLang의 FA3 디코드 최적화: get_scheduler_metadata 도입"
  (analysis of sglang PR #21103): split-KV scheduling metadata, once per batch.
* [FlashInfer-Sage]   "FlashInfer PrimTS, Sage Attention 도입으로 8비트 양자화
  및 성능 최적화 달성" (analysis of flashinfer PR #5123): the 8-bit formula.
* [FA-vs-PA]          "FlashAttention: 优化计算过程中的临时显存占用" /
  "PagedAttention: 优化 KV Cache 的管理和利用率" (Adam Chow's Life Journals).
* [SGLang-FA-DE]      "Flash Attention Backend in SGLang: Grundlagen und KV
  Cache optimal nutzen" (dasgeld.co).

Parity status per function (what pins it, see ``tests/test_oracle_*.py``):

* ``paged_attention``: pinned (torch SDPA special case, closed forms,
  page-permutation invariance, GQA == repeated-head MHA, P rows sum to 1).
* ``lse_merge``: pinned (partition invariance against the unsplit oracle).
* ``e4m3_encode`` / ``e4m3_decode``: pinned (exhaustive against torch's
  float8_e4m3fn cast, OCP format landmarks).
* ``sage_decode``: pinned by reductions (scales 1 and P unquantised equals
  ``paged_attention``; constant scores give sfV·mean(V8); hand-worked two-key
  example; power-of-two sfV scaling).  The difference between quantising P
  against the final row max (here) and a running max (an online kernel) is
  bounded only by the stated fp8 tolerance: parity unpinned beyond it.
* ``sage_extend``: pinned by reductions to pinned functions (one new token
  per request equals ``sage_decode``; every row equals ``sage_decode`` on
  the request cut at that row's causal limit; unit scales and P
  unquantised equal ``paged_attention``; q8 = 0 gives sfV·mean(V8) over the
  visible keys).  Same running-max caveat as ``sage_decode``.
* INT8 Q/K (``qk_codes="int8"`` of the three 8-bit functions): pinned by a
  hand-worked two-key example with negative and extreme codes, equality with
  the E4M3 reading where the integer codes' values are exact E4M3 values,
  and the integer dot product (sign, range) against exact integer arithmetic.
* ``plan_decode`` / ``plan_extend``: the split heuristic is a design choice,
  not from the pages; pinned by invariants (every token covered once, in
  order; bounds on tile multiples; capacity; the chunk is the smallest that
  meets the item target; longest-first order when items overflow it).
* ``kv_store``: pinned by a round trip.
* ``block_sparse_decode`` / ``block_sparse_sage_decode``: pinned by
  reductions to pinned functions (every block listed equals
  ``paged_attention`` / ``sage_decode``; equal to them on a page table cut
  down by hand to the listed positions, with sfK of the logical blocks), the
  log-sum-exp merge identity over a disjoint split of the listed blocks, and
  one-hot scores inside and outside the mask.  The mask format and "exact"
  semantics are a reading (the pages give only densities); the 8-bit
  running-max caveat of ``sage_decode`` applies.
"""
from .attention import paged_attention
from .merge import lse_merge
from .e4m3 import e4m3_encode, e4m3_decode, E4M3_MAX
from .sage import sage_decode, sage_extend, qk_values
from .plan import plan_decode, plan_extend, decode_target_items, DECODE_TILE, EXTEND_BLOCK_M
from .kv_store import kv_store
from .memory import score_matrix_bytes
from .block_sparse import block_sparse_decode, block_sparse_sage_decode

__all__ = [
    "paged_attention", "lse_merge", "e4m3_encode",
    "e4m3_decode", "E4M3_MAX", "sage_decode", "sage_extend", "qk_values", "plan_decode", "plan_extend",
    "DECODE_TILE", "EXTEND_BLOCK_M", "decode_target_items", "kv_store",
    "score_matrix_bytes", "block_sparse_decode", "block_sparse_sage_decode",
]
