"""ctypes binding of libpkv (argument marshalling only).

Each function takes torch tensors that already live on the GPU, checks their
dtype, shape (every buffer the kernels write or index against the sizes the
call implies) and contiguity, and forwards raw device pointers and torch's
current HIP stream to the C entry point of the same name.  All arithmetic
runs in the library's kernels; there is no fallback: if ``libpkv.so`` is
missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; PKV_LIBRARY names another build of the same library (the
# host-AddressSanitizer build of the ABI tests)
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(PKG, "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_EHIP = range(5)
PKV_BF16, PKV_FP8_E4M3, PKV_SAGE_INT8 = 0, 1, 2
PKV_DECODE, PKV_EXTEND = 0, 1

EXPORTED = ("pkv_workspace_size", "pkv_plan_metadata", "pkv_kv_store", "pkv_block_sparse_table",
            "pkv_attn_decode", "pkv_attn_decode_noalloc", "pkv_attn_extend", "pkv_last_error", "pkv_version")
STATIC_SCRATCH_BYTES = 32 << 20  # PKV_STATIC_SCRATCH_BYTES


class PkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pkv error {code}: {msg}")
        self.code = code
        self.msg = msg


class Params(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("q_block", ctypes.c_int32),
                ("k_block", ctypes.c_int32), ("max_kv_len", ctypes.c_int32),
                ("kv_chunk", ctypes.c_int32), ("split_target", ctypes.c_int32),
                ("decode_q_len", ctypes.c_int32)]

    def __init__(self, num_q_heads, num_kv_heads, head_dim, page_size, max_kv_len,
                 kv_dtype=PKV_BF16, q_block=0, k_block=0, kv_chunk=0, split_target=0, decode_q_len=0):
        super().__init__(num_q_heads, num_kv_heads, head_dim, page_size, kv_dtype, q_block,
                         k_block, max_kv_len, kv_chunk, split_target, decode_q_len)


_P = ctypes.c_void_p
_I32, _I64, _SZ, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpkv.so (built in-tree by ``build.py``); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m flashattention_paged_kv_amd.build` "
                           "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(path)
    pp = ctypes.POINTER(Params)
    lib.pkv_workspace_size.argtypes = [pp, _I32, _I32, _I64, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]
    lib.pkv_plan_metadata.argtypes = [pp, _I32, _I32, _I64, _P, _P, _P, _SZ, _P]
    lib.pkv_kv_store.argtypes = [pp, _P, _P, _I64, _P, _P, _P, _I64, _P]
    lib.pkv_block_sparse_table.argtypes = [pp, _I32, _P, _P, _I64, _P, _P, _P, _I64, _I32, _P, _P, _P, _P, _P]
    lib.pkv_attn_decode.argtypes = [pp, _P, _P, _P, _P, _P, _I64, _P, _I64, _P, _P, _I32, _F,
                                    _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P]
    lib.pkv_attn_decode_noalloc.argtypes = [pp, _P, _P, _P, _P, _P, _I64, _P, _I64, _P, _P, _I32, _F,
                                            _P, _P, _P, _P, _P, _SZ, _P]
    lib.pkv_attn_extend.argtypes = [pp, _P, _P, _P, _P, _P, _I64, _P, _I64, _P, _P, _P, _I32, _I64,
                                    _F, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P]
    for f in ("pkv_workspace_size", "pkv_plan_metadata", "pkv_kv_store", "pkv_block_sparse_table",
              "pkv_attn_decode", "pkv_attn_decode_noalloc", "pkv_attn_extend", "pkv_version"):
        getattr(lib, f).restype = ctypes.c_int
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_last_error.argtypes = []
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().pkv_last_error().decode()


def _check(rc: int):
    if rc != PKV_OK:
        raise PkvError(rc, last_error())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t):
    """The current stream of tensor t's device, as a raw handle.  torch's
    accessor of the raw handle skips building a Stream object (about 2 us per
    call); the public API serves where it is absent."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, name, dtype=None, ndim=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _is_8bit(params: Params) -> bool:
    return params.kv_dtype in (PKV_FP8_E4M3, PKV_SAGE_INT8)


def _need_rows(t, name, params: Params):
    """K/V pools and new rows: [n, Hkv, d] of the params' element type."""
    _need(t, name, ndim=3)
    esize = 1 if _is_8bit(params) else 2
    if tuple(t.shape[1:]) != (params.num_kv_heads, params.head_dim) or t.element_size() != esize:
        raise ValueError(f"{name} must be [n, {params.num_kv_heads}, {params.head_dim}] with {esize}-byte elements, "
                         f"got {tuple(t.shape)} with {t.element_size()}-byte elements")


def _check_q_out_lse(params: Params, q, out, lse, rows: int):
    """q and out are [rows, Hq, d] and lse, when given, is [rows, Hq]: the
    kernels write every element of those shapes, so a smaller buffer would be
    written past its end."""
    want = (rows, params.num_q_heads, params.head_dim)
    if tuple(q.shape) != want:
        raise ValueError(f"q must be {want}, got {tuple(q.shape)}")
    if out is not None and tuple(out.shape) != want:
        raise ValueError(f"out must be {want} (the shape of q), got {tuple(out.shape)}")
    if lse is not None and tuple(lse.shape) != (rows, params.num_q_heads):
        raise ValueError(f"lse must be {(rows, params.num_q_heads)}, got {tuple(lse.shape)}")


def _check_page_table(params: Params, req_to_token, req_pool_indices, batch: int):
    """Every request has a req_to_token row (directly, or through
    req_pool_indices) of at least max_kv_len entries."""
    if req_pool_indices is None:
        if req_to_token.shape[0] < batch:
            raise ValueError(f"req_to_token needs a row per request ({batch}) when req_pool_indices is None, "
                             f"got {req_to_token.shape[0]}")
    elif req_pool_indices.shape[0] < batch:
        raise ValueError(f"req_pool_indices needs an entry per request ({batch}), got {req_pool_indices.shape[0]}")
    if req_to_token.shape[1] < params.max_kv_len:
        raise ValueError(f"req_to_token rows must hold max_kv_len = {params.max_kv_len} entries, "
                         f"got {req_to_token.shape[1]}")


def workspace_size(params: Params, mode: int, max_batch: int, max_total_q: int = 0) -> Tuple[int, int]:
    lib = load_library()
    ws, sc = _SZ(0), _SZ(0)
    _check(lib.pkv_workspace_size(ctypes.byref(params), mode, max_batch, max_total_q, ctypes.byref(ws),
                                  ctypes.byref(sc)))
    return ws.value, sc.value


@dataclass
class Plan:
    """Output of :func:`plan_metadata`: the device workspace and what it was planned for."""
    workspace: "object"
    mode: int
    batch: int
    total_q: int
    scratch_bytes: int


def plan_metadata(params: Params, mode: int, seq_lens, cu_seqlens_q=None, total_q: int = 0,
                  workspace=None) -> Plan:
    import torch
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    batch = seq_lens.shape[0]
    ws_bytes, sc_bytes = workspace_size(params, mode, batch, total_q if mode == PKV_EXTEND else 0)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=seq_lens.device)
    _need(workspace, "workspace")
    lib = load_library()
    _check(lib.pkv_plan_metadata(ctypes.byref(params), mode, batch, total_q, _ptr(seq_lens), _ptr(cu_seqlens_q),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(seq_lens)))
    return Plan(workspace, mode, batch, total_q, sc_bytes)


def kv_store(params: Params, k_pool, v_pool, k_new, v_new, slots):
    import torch
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool"), (k_new, "k_new"), (v_new, "v_new")):
        _need_rows(t, n, params)
    _need(slots, "slots", torch.int32, 1)
    if k_new.shape[0] != slots.shape[0] or v_new.shape[0] != slots.shape[0]:
        raise ValueError("k_new/v_new rows must match slots")
    lib = load_library()
    _check(lib.pkv_kv_store(ctypes.byref(params), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0], _ptr(k_new),
                            _ptr(v_new), _ptr(slots), slots.shape[0], _stream(k_pool)))


def block_sparse_table(params: Params, seq_lens, req_to_token, blk_indptr, blk_indices, block_size: int,
                       req_pool_indices=None, sfk=None):
    """Compacted page table of a block-sparse decode batch (ascending block
    lists per request, shared by all heads).  Returns (sparse_req_to_token
    [B, max_kv_len], sparse_seq_lens [B], sparse_sfk or None); pass them to
    plan_metadata / attn_decode in place of req_to_token, seq_lens and sfk."""
    import torch
    fp8 = _is_8bit(params)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(req_to_token, "req_to_token", torch.int32, 2)
    _need(blk_indptr, "blk_indptr", torch.int32, 1)
    _need(blk_indices, "blk_indices", torch.int32, 1)
    _need(req_pool_indices, "req_pool_indices", torch.int32, 1)
    _need(sfk, "sfk", torch.float32)
    B = seq_lens.shape[0]
    if blk_indptr.shape[0] != B + 1:
        raise ValueError("blk_indptr must have batch + 1 entries")
    _check_page_table(params, req_to_token, req_pool_indices, B)
    dev = seq_lens.device
    sparse_rtt = torch.empty((B, params.max_kv_len), dtype=torch.int32, device=dev)
    sparse_lens = torch.empty((B,), dtype=torch.int32, device=dev)
    sparse_sfk = None
    if fp8:
        nblk = -(-params.max_kv_len // params.k_block)
        if sfk is None or tuple(sfk.shape) != (B, params.num_kv_heads, nblk):
            raise ValueError(f"sfk must be [B, Hkv, ceil(max_kv_len/k_block)] = {(B, params.num_kv_heads, nblk)}")
        sparse_sfk = torch.empty_like(sfk)
    lib = load_library()
    _check(lib.pkv_block_sparse_table(ctypes.byref(params), B, _ptr(seq_lens), _ptr(req_to_token),
                                      req_to_token.shape[1], _ptr(req_pool_indices), _ptr(blk_indptr),
                                      _ptr(blk_indices), blk_indices.shape[0], int(block_size), _ptr(sfk),
                                      _ptr(sparse_rtt), _ptr(sparse_lens), _ptr(sparse_sfk), _stream(seq_lens)))
    return sparse_rtt, sparse_lens, sparse_sfk


def attn_decode(params: Params, q, k_pool, v_pool, req_to_token, seq_lens, plan: Plan, scratch=None,
                out=None, lse=None, sm_scale: Optional[float] = None, req_pool_indices=None,
                sfq=None, sfk=None, sfv=None, v_mean=None):
    """Decode attention: q [B, Hq, d] (bf16, uint8 E4M3 codes, or int8 codes for PKV_SAGE_INT8)
    -> out [B, Hq, d] bf16."""
    return _attn_decode(params, q, k_pool, v_pool, req_to_token, seq_lens, plan, scratch, out, lse, sm_scale,
                        req_pool_indices, sfq, sfk, sfv, v_mean, noalloc=False)


def attn_decode_noalloc(params: Params, q, k_pool, v_pool, req_to_token, seq_lens, plan: Plan, out,
                        lse=None, sm_scale: Optional[float] = None, req_pool_indices=None,
                        sfq=None, sfk=None, sfv=None, v_mean=None):
    """``pkv_attn_decode_noalloc``: the decode of :func:`attn_decode` with its
    split partials in the library's static device scratch; ``out`` must be
    given (nothing is allocated here or in the library).  Calls that overlap
    on one GPU race on that scratch."""
    if out is None:
        raise ValueError("attn_decode_noalloc writes into a caller's out buffer; pass out=")
    return _attn_decode(params, q, k_pool, v_pool, req_to_token, seq_lens, plan, None, out, lse, sm_scale,
                        req_pool_indices, sfq, sfk, sfv, v_mean, noalloc=True)


def _attn_decode(params, q, k_pool, v_pool, req_to_token, seq_lens, plan, scratch, out, lse, sm_scale,
                 req_pool_indices, sfq, sfk, sfv, v_mean, noalloc):
    import torch
    qt = {PKV_FP8_E4M3: torch.uint8, PKV_SAGE_INT8: torch.int8}.get(params.kv_dtype, torch.bfloat16)
    _need(q, "q", qt, 3)
    _need_rows(k_pool, "k_pool", params)
    _need_rows(v_pool, "v_pool", params)
    _need(req_to_token, "req_to_token", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(req_pool_indices, "req_pool_indices", torch.int32, 1)
    for t, n in ((sfq, "sfq"), (sfk, "sfk"), (sfv, "sfv"), (v_mean, "v_mean"), (lse, "lse")):
        _need(t, n, torch.float32)
    B = seq_lens.shape[0]
    if plan.mode != PKV_DECODE or plan.batch != B:
        raise ValueError("plan was not made by plan_metadata(PKV_DECODE) for this batch")
    n = max(params.decode_q_len, 1)
    _check_q_out_lse(params, q, out, lse, B * n)
    _check_page_table(params, req_to_token, req_pool_indices, B)
    if _is_8bit(params) and sfk is not None:
        nblk = -(-params.max_kv_len // params.k_block)
        if tuple(sfk.shape) != (B, params.num_kv_heads, nblk):
            raise ValueError(f"sfk must be [B, Hkv, ceil(max_kv_len/k_block)] = {(B, params.num_kv_heads, nblk)}")
        if sfq is None or tuple(sfq.shape) != (B * n, params.num_q_heads):
            raise ValueError("sfq must be [B * decode_q_len, Hq] (one scale per new-token row and head)")
        if sfv is None or tuple(sfv.shape) != (B, params.num_kv_heads, params.head_dim):
            raise ValueError("sfv must be [B, Hkv, d]")
        if v_mean is not None and tuple(v_mean.shape) != (B, params.num_kv_heads, params.head_dim):
            raise ValueError("v_mean must be [B, Hkv, d]")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, 3)
    if scratch is None and not noalloc:
        scratch = torch.empty(max(plan.scratch_bytes, 16), dtype=torch.uint8, device=q.device)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(params.head_dim)
    lib = load_library()
    ws = plan.workspace
    if noalloc:
        _check(lib.pkv_attn_decode_noalloc(
            ctypes.byref(params), _ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0],
            _ptr(req_to_token), req_to_token.shape[1], _ptr(req_pool_indices), _ptr(seq_lens), B, float(sm_scale),
            _ptr(sfq), _ptr(sfk), _ptr(sfv), _ptr(v_mean), _ptr(ws), ws.numel() * ws.element_size(), _stream(q)))
        return out
    _check(lib.pkv_attn_decode(ctypes.byref(params), _ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                               k_pool.shape[0], _ptr(req_to_token), req_to_token.shape[1], _ptr(req_pool_indices),
                               _ptr(seq_lens), B, float(sm_scale), _ptr(sfq), _ptr(sfk), _ptr(sfv), _ptr(v_mean),
                               _ptr(ws), ws.numel() * ws.element_size(), _ptr(scratch),
                               scratch.numel() * scratch.element_size(), _stream(q)))
    return out


def attn_extend(params: Params, q, k_pool, v_pool, req_to_token, seq_lens, cu_seqlens_q, plan: Plan,
                out=None, lse=None, sm_scale: Optional[float] = None, req_pool_indices=None,
                sfq=None, sfk=None, sfv=None, v_mean=None):
    """Causal extend attention: q [total_q, Hq, d] (bf16, or uint8 E4M3 codes with
    sfq [total_q, Hq], sfk, sfv and optional v_mean) -> out [total_q, Hq, d] bf16."""
    import torch
    fp8 = params.kv_dtype == PKV_FP8_E4M3
    _need(q, "q", torch.uint8 if fp8 else torch.bfloat16, 3)
    _need_rows(k_pool, "k_pool", params)
    _need_rows(v_pool, "v_pool", params)
    for t, nm in ((sfq, "sfq"), (sfk, "sfk"), (sfv, "sfv"), (v_mean, "v_mean")):
        _need(t, nm, torch.float32)
    _need(req_to_token, "req_to_token", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _need(req_pool_indices, "req_pool_indices", torch.int32, 1)
    _need(lse, "lse", torch.float32)
    B = seq_lens.shape[0]
    total_q = q.shape[0]
    if plan.mode != PKV_EXTEND or plan.batch != B or plan.total_q != total_q:
        raise ValueError("plan was not made by plan_metadata(PKV_EXTEND) for this batch and total_q")
    if cu_seqlens_q.shape[0] != B + 1:
        raise ValueError(f"cu_seqlens_q must have batch + 1 = {B + 1} entries, got {cu_seqlens_q.shape[0]}")
    _check_q_out_lse(params, q, out, lse, total_q)
    _check_page_table(params, req_to_token, req_pool_indices, B)
    if fp8 and sfk is not None:
        nblk = -(-params.max_kv_len // params.k_block)
        if tuple(sfk.shape) != (B, params.num_kv_heads, nblk):
            raise ValueError(f"sfk must be [B, Hkv, ceil(max_kv_len/k_block)] = {(B, params.num_kv_heads, nblk)}")
        if sfq is None or tuple(sfq.shape) != (total_q, params.num_q_heads):
            raise ValueError("sfq must be [total_q, Hq]")
        if sfv is None or tuple(sfv.shape) != (B, params.num_kv_heads, params.head_dim):
            raise ValueError("sfv must be [B, Hkv, d]")
        if v_mean is not None and tuple(v_mean.shape) != (B, params.num_kv_heads, params.head_dim):
            raise ValueError("v_mean must be [B, Hkv, d]")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, 3)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(params.head_dim)
    lib = load_library()
    ws = plan.workspace
    _check(lib.pkv_attn_extend(ctypes.byref(params), _ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                               k_pool.shape[0], _ptr(req_to_token), req_to_token.shape[1], _ptr(req_pool_indices),
                               _ptr(seq_lens), _ptr(cu_seqlens_q), B, total_q, float(sm_scale), _ptr(sfq),
                               _ptr(sfk), _ptr(sfv), _ptr(v_mean), _ptr(ws), ws.numel() * ws.element_size(),
                               None, 0, _stream(q)))
    return out
