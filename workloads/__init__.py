"""Seeded synthetic workloads for paged-KV attention.

This module only draws inputs: request lengths, a shuffled page pool, the
two-level page table and N(0, 1) values (rounded to the storage type by a
plain cast).  It holds none of the attention arithmetic, so the CPU oracle
and the HIP library can both be fed from it without sharing any method code.

Shapes and distributions follow the workloads the library is measured on:

=====================  =====================================================
name                   description
=====================  =====================================================
``tiny_decode``        B=2, 4 q / 2 kv heads, d=64, page 1, cached {37,100},
                       one new token each; fp32 N(0,1); the page table is a
                       random permutation of a 256-slot pool
``tiny_extend``        as above with {5,12} new tokens
``decode_bf16``        B=64, 32 q / 8 kv heads, d=128, page 16, cached
                       lengths U[512,4096]; pool = 2x the pages needed
``extend_bf16``        16 requests, 32/8 heads, d=128, page 16, prefix
                       U[0,2048] cached, U[128,2048] new tokens
``long_decode_bf16``   B=8, 64/8 heads, d=128, page 64, cached U[32768,131072]
``single_decode_bf16`` one request, 64/8 heads, d=128, page 64, 131071 cached
                       tokens: every split of the device comes from one
                       request, so the merge and the plan serve one row
``decode_fp8``         B=64, 32/8 heads, d=128, page 16, cached U[1024,8192];
                       E4M3 codes of N(0,1)/scale with per-64-token sfK,
                       per-(b,h) sfQ and per-channel sfV drawn from U[0.5,2]
``decode_int8``        as ``decode_fp8`` with INT8 Q and K codes (Sage INT8:
                       clip(rint(N(0,1)/sf), -127, 127), sf = U[0.5,2]/16)
                       and E4M3 V
``decode_n4_bf16``     as ``decode_bf16`` with 4 new tokens per request
                       checked in one decode call (a verify step)
``extend_fp8``         as ``extend_bf16`` with E4M3 K/V, sfQ per new-token
                       row, sfK per 16 keys (the Sage page's default blocks),
                       per-channel sfV
=====================  =====================================================

Decode workloads append n new tokens per request (one unless stated): the
drawn value is the cached length and the attended length is ``cached + n``
(the new tokens' K/V rows are written by ``kv_store`` before attention
reads them).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple, Union

import numpy as np

LenSpec = Union[int, Tuple[int, int], Sequence[int]]


@dataclass(frozen=True)
class Spec:
    """Shape of one synthetic batch.

    ``prefix`` / ``new``: an int (same for all requests), a ``(lo, hi)`` tuple
    (uniform integers, inclusive) or a list with one value per request.
    ``pool``: ``"2x"`` for a shuffled pool with twice the pages needed, or an
    int giving the total number of slots (the page table is then a random
    permutation of that pool's pages).
    """

    name: str
    mode: str  # "decode" or "extend"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    prefix: LenSpec
    new: LenSpec
    dtype: str = "bf16"  # "fp32" (host-only tiny case), "bf16", "fp8" or "int8" (Sage INT8 Q/K, E4M3 V)
    pool: Union[str, int] = "2x"
    k_block: int = 64  # fp8: tokens per sfK block
    q_block: int = 1  # fp8: q rows per sfQ block
    scale_range: Tuple[float, float] = (0.5, 2.0)
    sparse_block: int = 0  # block-sparse decode: logical positions per KV block (0 = dense)
    density: float = 0.0  # block-sparse decode: share of each request's blocks selected


SPECS = {
    "tiny_decode": Spec("tiny_decode", "decode", 2, 4, 2, 64, 1, [37, 100], 1,
                        dtype="fp32", pool=256),
    "tiny_extend": Spec("tiny_extend", "extend", 2, 4, 2, 64, 1, [37, 100], [5, 12],
                        dtype="fp32", pool=256),
    "decode_bf16": Spec("decode_bf16", "decode", 64, 32, 8, 128, 16, (512, 4096), 1),
    "extend_bf16": Spec("extend_bf16", "extend", 16, 32, 8, 128, 16, (0, 2048), (128, 2048)),
    "long_decode_bf16": Spec("long_decode_bf16", "decode", 8, 64, 8, 128, 64,
                             (32768, 131072), 1),
    "single_decode_bf16": Spec("single_decode_bf16", "decode", 1, 64, 8, 128, 64, (131071, 131071), 1),
    "decode_n4_bf16": Spec("decode_n4_bf16", "decode", 64, 32, 8, 128, 16, (512, 4096), 4),
    "extend_fp8": Spec("extend_fp8", "extend", 16, 32, 8, 128, 16, (0, 2048), (128, 2048), dtype="fp8",
                       k_block=16, q_block=1),
    "decode_fp8": Spec("decode_fp8", "decode", 64, 32, 8, 128, 16, (1024, 8192), 1,
                       dtype="fp8", k_block=64, q_block=1),
    "decode_int8": Spec("decode_int8", "decode", 64, 32, 8, 128, 16, (1024, 8192), 1,
                        dtype="int8", k_block=64, q_block=1),
    "sparse_decode_bf16": Spec("sparse_decode_bf16", "decode", 8, 40, 40, 128, 16, (15360, 75600), 1,
                               sparse_block=64, density=0.10),
    "sparse_decode_fp8": Spec("sparse_decode_fp8", "decode", 8, 40, 40, 128, 16, (15360, 75600), 1,
                              dtype="fp8", k_block=64, q_block=1, sparse_block=64, density=0.10),
}

# Index used to derive the seed of each named workload (1000 + index).
SPEC_INDEX = {"tiny_decode": 1, "tiny_extend": 1, "decode_bf16": 2, "extend_bf16": 3, "decode_n4_bf16": 6, "extend_fp8": 7,
              "long_decode_bf16": 4, "decode_fp8": 5, "sparse_decode_bf16": 8, "sparse_decode_fp8": 10,
              "single_decode_bf16": 11, "decode_int8": 12}


def seed_sequence(spec: Spec, seed: int) -> list:
    base = 1000 + SPEC_INDEX.get(spec.name, 9)
    return [base, int(seed)]


@dataclass
class Layout:
    """Integer structure of a batch: lengths and the two-level page table."""

    spec: Spec
    prefix_lens: np.ndarray  # int32 [B]   cached tokens before this step
    new_lens: np.ndarray  # int32 [B]   tokens appended this step
    seq_lens: np.ndarray  # int32 [B]   attended length = prefix + new
    cu_seqlens_q: np.ndarray  # int32 [B+1] prefix sums of new_lens
    req_to_token: np.ndarray  # int32 [B, stride]; -1 past seq_len
    pool_slots: int  # rows in each per-layer K/V pool
    new_slots: np.ndarray  # int32 [T] slot of each new token, request-major
    slot_owner: np.ndarray  # int32 [pool_slots] request owning a slot, -1 if free
    slot_pos: np.ndarray  # int32 [pool_slots] position of a slot in its request
    blk_indptr: Optional[np.ndarray] = None  # block-sparse decode: int32 [B+1]
    blk_indices: Optional[np.ndarray] = None  # int32 [nnz], ascending per request

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_kv_len(self) -> int:
        return int(self.seq_lens.max()) if len(self.seq_lens) else 0


def _draw(rng: np.random.Generator, spec_val: LenSpec, batch: int) -> np.ndarray:
    if isinstance(spec_val, (int, np.integer)):
        return np.full(batch, int(spec_val), dtype=np.int64)
    if isinstance(spec_val, tuple):
        lo, hi = spec_val
        return rng.integers(lo, hi + 1, size=batch, dtype=np.int64)
    arr = np.asarray(spec_val, dtype=np.int64)
    assert arr.shape == (batch,), (arr.shape, batch)
    return arr


def block_mask(seq_lens, block_size: int, density: float, rng: np.random.Generator):
    """Selected KV blocks per request (CSR): ceil(density · n) of the n =
    ceil(L / block_size) blocks, at least one; the newest block (holding the
    decoded token) is always kept, the others are drawn uniformly without
    replacement; ascending per request."""
    indptr = [0]
    indices = []
    for L in np.asarray(seq_lens, np.int64):
        n = int((L + block_size - 1) // block_size)
        if n == 0:
            indptr.append(len(indices))
            continue
        count = min(n, max(1, int(np.ceil(density * n))))
        rest = rng.choice(n - 1, size=count - 1, replace=False) if count > 1 else np.zeros(0, np.int64)
        indices.extend(sorted(int(x) for x in rest) + [n - 1])
        indptr.append(len(indices))
    return np.asarray(indptr, np.int32), np.asarray(indices, np.int32)


def make_layout(spec: Spec, seed: int = 0, rng: Optional[np.random.Generator] = None,
                stride: Optional[int] = None) -> Tuple[Layout, np.random.Generator]:
    """Draw lengths, then the page permutation, then build ``req_to_token``.

    Positions j and j+1 of a request that fall in one page get consecutive
    slots (slot = page * page_size + j % page_size).
    """
    if rng is None:
        rng = np.random.default_rng(seed_sequence(spec, seed))
    B, P = spec.batch, spec.page_size
    prefix = _draw(rng, spec.prefix, B)
    new = _draw(rng, spec.new, B)
    if spec.mode == "decode":
        # one new token per request, or the same n for every request (several
        # tokens checked in one decode call)
        assert B == 0 or (np.all(new == new[0]) and new[0] >= 1), "decode appends the same n >= 1 tokens per request"
    seq = prefix + new
    pages_per_req = (seq + P - 1) // P
    pages_needed = int(pages_per_req.sum())
    if spec.pool == "2x":
        num_pages = max(2 * pages_needed, 1)
    else:
        assert int(spec.pool) % P == 0
        num_pages = int(spec.pool) // P
        assert num_pages >= pages_needed, "pool too small for the drawn lengths"
    perm = rng.permutation(num_pages)
    max_len = int(seq.max()) if B else 0
    if stride is None:
        stride = max(max_len, 1)
    assert stride >= max_len
    rtt = np.full((B, stride), -1, dtype=np.int64)
    slot_owner = np.full(num_pages * P, -1, dtype=np.int32)
    slot_pos = np.full(num_pages * P, -1, dtype=np.int32)
    nxt = 0
    for b in range(B):
        L = int(seq[b])
        npg = int(pages_per_req[b])
        pages = perm[nxt:nxt + npg]
        nxt += npg
        j = np.arange(L)
        slots = pages[j // P] * P + (j % P)
        rtt[b, :L] = slots
        slot_owner[slots] = b
        slot_pos[slots] = j
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(new)
    new_slots = np.concatenate(
        [rtt[b, prefix[b]:seq[b]] for b in range(B)]) if B else np.zeros(0, np.int64)
    lay = Layout(spec=spec, prefix_lens=prefix.astype(np.int32), new_lens=new.astype(np.int32),
                 seq_lens=seq.astype(np.int32), cu_seqlens_q=cu.astype(np.int32),
                 req_to_token=rtt.astype(np.int32), pool_slots=num_pages * P,
                 new_slots=new_slots.astype(np.int32), slot_owner=slot_owner, slot_pos=slot_pos)
    if spec.sparse_block > 0:
        # drawn from a stream of its own, so the other draws match the dense layout
        mrng = np.random.default_rng(seed_sequence(spec, seed) + [77])
        lay.blk_indptr, lay.blk_indices = block_mask(lay.seq_lens, spec.sparse_block, spec.density, mrng)
    return lay, rng


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even) by a cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """OCP E4M3 (``float8_e4m3fn``) byte codes of float32 values, by a torch cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@dataclass
class HostBatch:
    """Layout plus host values (float32 arrays; bf16-exact when dtype is bf16).

    ``k_pool``/``v_pool`` hold every referenced row *including* the new tokens
    (the state after ``kv_store``); ``k_new``/``v_new`` are those new rows, in
    ``new_slots`` order.  Unreferenced rows are NaN when ``poison`` was set.
    fp8 batches carry E4M3 codes (uint8) in ``*_codes`` and the scales;
    int8 batches carry int8 codes of Q and K (scales U[lo, hi] / INT8_LEVELS,
    so code·scale is about N(0,1)) and E4M3 codes of V.
    """

    layout: Layout
    q: np.ndarray  # [T, Hq, d]
    k_pool: np.ndarray  # [slots, Hkv, d]
    v_pool: np.ndarray
    k_new: np.ndarray  # [T, Hkv, d]
    v_new: np.ndarray
    q_codes: Optional[np.ndarray] = None  # fp8 only, uint8
    k_codes: Optional[np.ndarray] = None
    v_codes: Optional[np.ndarray] = None
    k_new_codes: Optional[np.ndarray] = None
    v_new_codes: Optional[np.ndarray] = None
    sfq: Optional[np.ndarray] = None  # [B, Hq] float32 (decode: one q block)
    sfk: Optional[np.ndarray] = None  # [B, Hkv, nblk] float32
    sfv: Optional[np.ndarray] = None  # [B, Hkv, d] float32


# int8 Sage codes: code = clip(rint(x / sf), -127, 127) with sf = U[lo, hi] /
# INT8_LEVELS, i.e. a standard normal x spans about +-4 * 16 / U codes.
INT8_LEVELS = 16.0


def int8_codes(x: np.ndarray) -> np.ndarray:
    return np.clip(np.rint(x), -127, 127).astype(np.int8)


def make_host_batch(spec: Spec, seed: int = 0, poison: bool = True,
                    stride: Optional[int] = None) -> HostBatch:
    """Draw a complete batch on the host (small and medium sizes).

    Draw order: lengths, page permutation, Q, K pool, V pool, then scales.
    """
    lay, rng = make_layout(spec, seed, stride=stride)
    T, Hq, Hkv, d = lay.total_q, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    S = lay.pool_slots
    q = rng.standard_normal((T, Hq, d), dtype=np.float32)
    k = rng.standard_normal((S, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((S, Hkv, d), dtype=np.float32)
    used = lay.slot_owner >= 0
    if spec.dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    hb = HostBatch(layout=lay, q=q, k_pool=k, v_pool=v, k_new=None, v_new=None)
    if spec.dtype in ("fp8", "int8"):
        i8 = spec.dtype == "int8"
        B = spec.batch
        lo, hi = spec.scale_range
        nblk = max((lay.max_kv_len + spec.k_block - 1) // spec.k_block, 1)
        # sfQ: one scale per (request, head) for decode, per (new-token row,
        # head) for extend (q_block = 1)
        sfq = rng.uniform(lo, hi, size=(T if spec.mode == "extend" else B, Hq)).astype(np.float32)
        sfk = rng.uniform(lo, hi, size=(B, Hkv, nblk)).astype(np.float32)
        sfv = rng.uniform(lo, hi, size=(B, Hkv, d)).astype(np.float32)
        if i8:
            sfq = (sfq / INT8_LEVELS).astype(np.float32)
            sfk = (sfk / INT8_LEVELS).astype(np.float32)
        qk_codes = int8_codes if i8 else e4m3_codes
        req_of_row = np.repeat(np.arange(B), lay.new_lens)
        q_codes = qk_codes(q / (sfq if spec.mode == "extend" else sfq[req_of_row])[:, :, None])
        owner = np.where(used, lay.slot_owner, 0)
        blk = np.where(used, lay.slot_pos, 0) // spec.k_block
        ks = sfk[owner, :, blk]  # [S, Hkv]
        vs = sfv[owner]  # [S, Hkv, d]
        k_codes = qk_codes(k / ks[:, :, None])
        v_codes = e4m3_codes(v / vs)
        k_codes[~used] = -128 if i8 else 0x7F  # extreme int8 / E4M3 NaN in unreferenced rows
        v_codes[~used] = 0x7F
        hb.q_codes, hb.k_codes, hb.v_codes = q_codes, k_codes, v_codes
        hb.sfq, hb.sfk, hb.sfv = sfq, sfk, sfv
        hb.k_new_codes = k_codes[lay.new_slots].copy()
        hb.v_new_codes = v_codes[lay.new_slots].copy()
    if poison:
        k[~used] = np.nan
        v[~used] = np.nan
    hb.k_new = k[lay.new_slots].copy()
    hb.v_new = v[lay.new_slots].copy()
    return hb


def pool_before_store(pool: np.ndarray, new_slots: np.ndarray, fill=np.nan) -> np.ndarray:
    """Copy of a pool whose new-token rows are overwritten with ``fill``."""
    out = pool.copy()
    out[new_slots] = fill
    return out


def permute_pages(layout: Layout, rng: np.random.Generator) -> Tuple[Layout, np.ndarray]:
    """Relabel the physical pages of a layout by a random permutation.

    Returns the new layout and ``slot_map`` with ``new_slot = slot_map[old_slot]``;
    moving every pool row ``r`` to ``slot_map[r]`` keeps the logical contents.
    """
    P = layout.spec.page_size
    num_pages = layout.pool_slots // P
    page_perm = rng.permutation(num_pages)
    old = np.arange(layout.pool_slots)
    slot_map = (page_perm[old // P] * P + old % P).astype(np.int64)
    rtt = layout.req_to_token.astype(np.int64)
    rtt_new = np.where(rtt >= 0, slot_map[np.maximum(rtt, 0)], -1).astype(np.int32)
    owner = np.full_like(layout.slot_owner, -1)
    pos = np.full_like(layout.slot_pos, -1)
    owner[slot_map] = layout.slot_owner
    pos[slot_map] = layout.slot_pos
    new = replace(layout, req_to_token=rtt_new,
                  new_slots=slot_map[layout.new_slots].astype(np.int32),
                  slot_owner=owner, slot_pos=pos)
    return new, slot_map


# ---------------------------------------------------------------- device-side batches
@dataclass
class DeviceBatch:
    """A batch whose integer structure comes from :func:`make_layout` and whose
    values are drawn on the GPU with a seeded torch generator (for sizes where
    host generation would be slow).  One set of pools per layer."""

    layout: Layout
    q: "object"  # [T, Hq, d] bf16 (fp8: uint8 E4M3 codes)
    k_pools: list  # per layer [slots, Hkv, d]
    v_pools: list
    k_new: list  # per layer [T, Hkv, d]
    v_new: list
    req_to_token: "object"  # int32 [B, stride]
    seq_lens: "object"  # int32 [B]
    cu_seqlens_q: "object"  # int32 [B+1]
    new_slots: "object"  # int32 [T]
    sfq: "object" = None
    sfk: "object" = None
    blk_indptr: "object" = None  # block-sparse decode, int32 [B+1]
    blk_indices: "object" = None  # int32 [nnz]
    sfv: "object" = None


def _torch_seed(spec: Spec, seed: int) -> int:
    return int(np.random.SeedSequence(seed_sequence(spec, seed)).generate_state(1)[0])


def make_device_batch(spec: Spec, seed: int = 0, device="cuda", layers: int = 1,
                      stride: Optional[int] = None) -> DeviceBatch:
    """Draw lengths and the page table on the host, values on ``device``.

    Draw order on the device: Q, then per layer the K pool and the V pool;
    for fp8 the scales are drawn first on the host (U[lo, hi]) and the codes
    are E4M3 casts of N(0,1)/scale; for int8 the Q and K scales are divided by
    INT8_LEVELS and their codes are clip(rint(N(0,1)/scale), -127, 127).
    """
    import torch
    lay, rng = make_layout(spec, seed, stride=stride)
    T, Hq, Hkv, d = lay.total_q, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    S = lay.pool_slots
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(spec, seed))
    dev = torch.device(device)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    new_slots = i32(lay.new_slots)
    db = DeviceBatch(layout=lay, q=None, k_pools=[], v_pools=[], k_new=[], v_new=[],
                     req_to_token=i32(lay.req_to_token), seq_lens=i32(lay.seq_lens),
                     cu_seqlens_q=i32(lay.cu_seqlens_q), new_slots=new_slots)
    if lay.blk_indptr is not None:
        db.blk_indptr, db.blk_indices = i32(lay.blk_indptr), i32(lay.blk_indices)
    if spec.dtype in ("fp8", "int8"):
        i8 = spec.dtype == "int8"
        B = spec.batch
        lo, hi = spec.scale_range
        nblk = max((lay.max_kv_len + spec.k_block - 1) // spec.k_block, 1)
        sfq = rng.uniform(lo, hi, size=(T if spec.mode == "extend" else B, Hq)).astype(np.float32)
        sfk = rng.uniform(lo, hi, size=(B, Hkv, nblk)).astype(np.float32)
        sfv = rng.uniform(lo, hi, size=(B, Hkv, d)).astype(np.float32)
        if i8:
            sfq = (sfq / INT8_LEVELS).astype(np.float32)
            sfk = (sfk / INT8_LEVELS).astype(np.float32)

        def qk_cast(x):
            if i8:
                return torch.clamp(torch.round(x), -127, 127).to(torch.int8)
            return x.to(torch.float8_e4m3fn).view(torch.uint8)
        db.sfq, db.sfk, db.sfv = (torch.from_numpy(x).to(dev) for x in (sfq, sfk, sfv))
        used = lay.slot_owner >= 0
        owner = torch.from_numpy(np.where(used, lay.slot_owner, 0).astype(np.int64)).to(dev)
        blk = torch.from_numpy((np.where(used, lay.slot_pos, 0) // spec.k_block).astype(np.int64)).to(dev)
        k_scale = db.sfk[owner, :, blk]  # [S, Hkv]
        v_scale = db.sfv[owner]  # [S, Hkv, d]
        req_of_row = torch.from_numpy(np.repeat(np.arange(B), lay.new_lens)).to(dev)
        qf = torch.randn((T, Hq, d), generator=g, device=dev, dtype=torch.float32)
        q_scale = db.sfq if spec.mode == "extend" else db.sfq[req_of_row]
        db.q = qk_cast(qf / q_scale[:, :, None])
        for _ in range(layers):
            kf = torch.randn((S, Hkv, d), generator=g, device=dev, dtype=torch.float32)
            kc = qk_cast(kf / k_scale[:, :, None])
            del kf
            vf = torch.randn((S, Hkv, d), generator=g, device=dev, dtype=torch.float32)
            vc = (vf / v_scale).to(torch.float8_e4m3fn).view(torch.uint8)
            del vf
            db.k_pools.append(kc)
            db.v_pools.append(vc)
            db.k_new.append(kc[new_slots.long()].contiguous())
            db.v_new.append(vc[new_slots.long()].contiguous())
        return db
    db.q = torch.randn((T, Hq, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    for _ in range(layers):
        kp = torch.randn((S, Hkv, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        vp = torch.randn((S, Hkv, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        db.k_pools.append(kp)
        db.v_pools.append(vp)
        db.k_new.append(kp[new_slots.long()].contiguous())
        db.v_new.append(vp[new_slots.long()].contiguous())
    return db
