"""The C ABI without a GPU: the library loads, exports every entry point that
include/pkv.h declares, and rejects bad host arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import flashattention_paged_kv_amd as pkv
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


@pytest.fixture(scope="module")
def lib():
    return pkv.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(pkv.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def _ws(lib, params, mode=pkv.PKV_DECODE, batch=4, total_q=0):
    ws, sc = ctypes.c_size_t(0), ctypes.c_size_t(0)
    rc = lib.pkv_workspace_size(ctypes.byref(params), mode, batch, total_q, ctypes.byref(ws), ctypes.byref(sc))
    return rc, ws.value, sc.value


@pytest.mark.parametrize("kw,code,msg", [
    (dict(num_q_heads=30, num_kv_heads=8), pkv.PKV_EINVAL, "is not a multiple of"),
    (dict(num_q_heads=0), pkv.PKV_EINVAL, "must be >= 1"),
    (dict(head_dim=96), pkv.PKV_EUNSUPPORTED, "head_dim=96 is unsupported"),
    (dict(page_size=24), pkv.PKV_EINVAL, "power of two"),
    (dict(page_size=512), pkv.PKV_EINVAL, "power of two"),
    (dict(max_kv_len=0), pkv.PKV_EINVAL, "max_kv_len"),
    (dict(kv_chunk=48), pkv.PKV_EINVAL, "kv_chunk"),
    (dict(k_block=16), pkv.PKV_EINVAL, "k_block is unsupported by a bf16 plan"),
    (dict(q_block=1), pkv.PKV_EINVAL, "q_block is unsupported by a bf16 plan"),
    (dict(kv_dtype=7), pkv.PKV_EUNSUPPORTED, "kv_dtype=7"),
    (dict(kv_dtype=pkv.PKV_FP8_E4M3, k_block=20, q_block=1), pkv.PKV_EINVAL, "k_block=20"),
    (dict(kv_dtype=pkv.PKV_FP8_E4M3, k_block=64, q_block=1, head_dim=64), pkv.PKV_EUNSUPPORTED, "head_dim=128"),
    (dict(kv_dtype=pkv.PKV_SAGE_INT8, k_block=64, q_block=1, head_dim=64), pkv.PKV_EUNSUPPORTED, "head_dim=128"),
    (dict(kv_dtype=pkv.PKV_SAGE_INT8, k_block=24, q_block=1), pkv.PKV_EINVAL, "k_block=24"),
    (dict(decode_q_len=-1), pkv.PKV_EINVAL, "decode_q_len=-1"),
    (dict(decode_q_len=65), pkv.PKV_EINVAL, "decode_q_len=65"),
])
def test_params_validation(lib, kw, code, msg):
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, max_kv_len=4096)
    base.update(kw)
    p = pkv.Params(**base)
    rc, _, _ = _ws(lib, p)
    assert rc == code
    assert msg in pkv.last_error()


def test_decode_q_len_sizes_scratch_per_token_and_is_decode_only(lib):
    p1 = pkv.Params(32, 8, 128, 16, 4096, split_target=2048)
    p4 = pkv.Params(32, 8, 128, 16, 4096, split_target=2048, decode_q_len=4)
    _, _, sc1 = _ws(lib, p1, batch=16)
    rc, _, sc4 = _ws(lib, p4, batch=16)
    assert rc == pkv.PKV_OK
    # same units (4 tokens x 4 heads fill one 16-column group), 4x the partial rows
    assert sc4 >= 4 * sc1 - 4 * 512
    rc, _, _ = _ws(lib, p4, mode=pkv.PKV_EXTEND, batch=16, total_q=64)
    assert rc == pkv.PKV_EINVAL and "DECODE plans only" in pkv.last_error()


def test_fp8_extend_plans_take_one_sfq_per_row(lib):
    """The 8-bit extend takes q_block = 1 (the Sage page's default); a larger Q
    block is rejected when planning, like the page's plan-time checks (code §2)."""
    p = pkv.Params(32, 8, 128, 16, 4096, kv_dtype=pkv.PKV_FP8_E4M3, q_block=1, k_block=16)
    rc, ws, _ = _ws(lib, p, mode=pkv.PKV_EXTEND, total_q=100)
    assert rc == pkv.PKV_OK and ws > 0
    p = pkv.Params(32, 8, 128, 16, 4096, kv_dtype=pkv.PKV_FP8_E4M3, q_block=64, k_block=64)
    rc, _, _ = _ws(lib, p, mode=pkv.PKV_EXTEND, total_q=100)
    assert rc == pkv.PKV_EUNSUPPORTED and "q_block=1" in pkv.last_error()
    rc, ws, sc = _ws(lib, p, mode=pkv.PKV_DECODE)
    assert rc == pkv.PKV_OK and ws > 0 and sc > 0


def test_int8_sage_is_a_decode_path(lib):
    """INT8 Q/K (the Sage page's code §3) is planned for DECODE; an EXTEND plan
    is rejected, as is an int8 extend call."""
    p = pkv.Params(32, 8, 128, 16, 4096, kv_dtype=pkv.PKV_SAGE_INT8, q_block=1, k_block=64)
    rc, ws, sc = _ws(lib, p, mode=pkv.PKV_DECODE)
    assert rc == pkv.PKV_OK and ws > 0 and sc > 0
    rc, _, _ = _ws(lib, p, mode=pkv.PKV_EXTEND, total_q=100)
    assert rc == pkv.PKV_EUNSUPPORTED and "sage_int8 is a DECODE path" in pkv.last_error()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    rc = lib.pkv_attn_extend(ctypes.byref(p), fake, None, fake, fake, fake, 100, fake, 4096, None, fake, fake, 4,
                             16, 0.1, fake, fake, fake, None, fake, 1 << 20, None, 0, None)
    assert rc == pkv.PKV_EUNSUPPORTED and "DECODE path" in pkv.last_error()
    # the decode needs its scales, like the E4M3 one
    rc = lib.pkv_attn_decode(ctypes.byref(p), fake, None, fake, fake, fake, 100, fake, 4096, None, fake, 4,
                             0.1, None, fake, fake, None, fake, 1 << 20, fake, 1 << 20, None)
    assert rc == pkv.PKV_EINVAL and "needs sfq, sfk and sfv" in pkv.last_error()


def test_run_call_argument_errors(lib):
    p = pkv.Params(32, 8, 128, 16, 4096)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    # scales given to a bf16 decode
    rc = lib.pkv_attn_decode(ctypes.byref(p), fake, None, fake, fake, fake, 100, fake, 4096, None, fake, 4,
                             0.1, fake, None, None, None, fake, 1 << 20, fake, 1 << 20, None)
    assert rc == pkv.PKV_EINVAL and "sfq is unsupported by a bf16 plan" in pkv.last_error()
    # rtt_stride below max_kv_len
    rc = lib.pkv_attn_decode(ctypes.byref(p), fake, None, fake, fake, fake, 100, fake, 100, None, fake, 4,
                             0.1, None, None, None, None, fake, 1 << 20, fake, 1 << 20, None)
    assert rc == pkv.PKV_EINVAL and "rtt_stride" in pkv.last_error()
    # workspace too small
    rc = lib.pkv_attn_decode(ctypes.byref(p), fake, None, fake, fake, fake, 100, fake, 4096, None, fake, 4,
                             0.1, None, None, None, None, fake, 8, fake, 1 << 30, None)
    assert rc == pkv.PKV_EWORKSPACE and "workspace_bytes=8" in pkv.last_error()
    # non-finite scale
    rc = lib.pkv_attn_decode(ctypes.byref(p), fake, None, fake, fake, fake, 100, fake, 4096, None, fake, 4,
                             float("nan"), None, None, None, None, fake, 1 << 20, fake, 1 << 20, None)
    assert rc == pkv.PKV_EINVAL and "sm_scale" in pkv.last_error()
    # fp8 without scales
    p8 = pkv.Params(32, 8, 128, 16, 4096, kv_dtype=pkv.PKV_FP8_E4M3, q_block=1, k_block=64)
    rc = lib.pkv_attn_decode(ctypes.byref(p8), fake, None, fake, fake, fake, 100, fake, 4096, None, fake, 4,
                             0.1, None, None, None, None, fake, 1 << 20, fake, 1 << 20, None)
    assert rc == pkv.PKV_EINVAL and "needs sfq, sfk and sfv" in pkv.last_error()
    # misaligned pointer
    odd = ctypes.c_void_p(0x1002)
    rc = lib.pkv_attn_decode(ctypes.byref(p), fake, None, odd, fake, fake, 100, fake, 4096, None, fake, 4,
                             0.1, None, None, None, None, fake, 1 << 20, fake, 1 << 20, None)
    assert rc == pkv.PKV_EINVAL and "16-byte aligned" in pkv.last_error()
    # extend: NULL cu_seqlens_q
    rc = lib.pkv_attn_extend(ctypes.byref(p), fake, None, fake, fake, fake, 100, fake, 4096, None, fake, None, 4,
                             64, 0.1, None, None, None, None, fake, 1 << 20, None, 0, None)
    assert rc == pkv.PKV_EINVAL and "cu_seqlens_q" in pkv.last_error()
    # extend: scales given to a bf16 plan; an 8-bit plan without them
    rc = lib.pkv_attn_extend(ctypes.byref(p), fake, None, fake, fake, fake, 100, fake, 4096, None, fake, fake, 4,
                             64, 0.1, fake, None, None, None, fake, 1 << 20, None, 0, None)
    assert rc == pkv.PKV_EINVAL and "unsupported by a bf16 plan" in pkv.last_error()
    p8 = pkv.Params(32, 8, 128, 16, 4096, kv_dtype=pkv.PKV_FP8_E4M3, q_block=1, k_block=16)
    rc = lib.pkv_attn_extend(ctypes.byref(p8), fake, None, fake, fake, fake, 100, fake, 4096, None, fake, fake, 4,
                             64, 0.1, None, None, None, None, fake, 1 << 20, None, 0, None)
    assert rc == pkv.PKV_EINVAL and "needs sfq, sfk and sfv" in pkv.last_error()
    # plan: NULL seq_lens, workspace too small
    rc = lib.pkv_plan_metadata(ctypes.byref(p), pkv.PKV_DECODE, 4, 0, None, None, fake, 1 << 20, None)
    assert rc == pkv.PKV_EINVAL and "seq_lens" in pkv.last_error()
    rc = lib.pkv_plan_metadata(ctypes.byref(p), pkv.PKV_DECODE, 4, 0, fake, None, fake, 4, None)
    assert rc == pkv.PKV_EWORKSPACE
    # kv_store: negative sizes
    rc = lib.pkv_kv_store(ctypes.byref(p), fake, fake, 0, fake, fake, fake, 3, None)
    assert rc == pkv.PKV_EINVAL and "pool_slots" in pkv.last_error()
    # empty batches are no-ops that succeed without touching the device
    rc = lib.pkv_attn_decode(ctypes.byref(p), None, None, None, None, None, 100, None, 4096, None, None, 0,
                             0.1, None, None, None, None, None, 0, None, 0, None)
    assert rc == pkv.PKV_OK and pkv.last_error() == ""


def test_length_bounds(lib):
    rc, _, _ = _ws(lib, pkv.Params(32, 8, 128, 16, (1 << 30) + 1))
    assert rc == pkv.PKV_EUNSUPPORTED and "2^30" in pkv.last_error()
    # a decode batch whose total tiles would not fit the plan's int32 offsets
    p = pkv.Params(32, 8, 128, 16, 1 << 30)
    fake = ctypes.c_void_p(0x1000)
    rc = lib.pkv_plan_metadata(ctypes.byref(p), pkv.PKV_DECODE, 64, 0, fake, None, fake, 1 << 40, None)
    assert rc == pkv.PKV_EUNSUPPORTED and "int32 tile offsets" in pkv.last_error()


def test_block_sparse_table_argument_errors(lib):
    p = pkv.Params(32, 8, 128, 16, 4096)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    call = lambda prm, bs, sfk=None, ssfk=None, nnz=10, stride=4096, batch=4: lib.pkv_block_sparse_table(
        ctypes.byref(prm), batch, fake, fake, stride, None, fake, fake, nnz, bs, sfk, fake, fake, ssfk, None)
    assert call(p, 48) == pkv.PKV_EINVAL and "power of two" in pkv.last_error()
    assert call(p, 64, nnz=-1) == pkv.PKV_EINVAL and "num_indices" in pkv.last_error()
    assert call(p, 64, stride=100) == pkv.PKV_EINVAL and "rtt_stride" in pkv.last_error()
    assert call(p, 64, sfk=fake) == pkv.PKV_EINVAL and "unsupported by a bf16 plan" in pkv.last_error()
    p8 = pkv.Params(32, 8, 128, 16, 4096, kv_dtype=pkv.PKV_FP8_E4M3, q_block=1, k_block=64)
    assert call(p8, 32, sfk=fake, ssfk=fake) == pkv.PKV_EINVAL and "multiple of k_block" in pkv.last_error()
    assert call(p8, 64) == pkv.PKV_EINVAL and "needs sfk and sparse_sfk" in pkv.last_error()
    pn = pkv.Params(32, 8, 128, 16, 4096, decode_q_len=4)
    assert call(pn, 64) == pkv.PKV_EUNSUPPORTED and "one new token" in pkv.last_error()
    assert call(p, 64, batch=0) == pkv.PKV_OK and pkv.last_error() == ""


def test_workspace_does_not_grow_with_square_of_length(lib):
    """O(N) not O(N^2): the plan workspace and decode scratch at 131072 tokens stay
    far below the materialised score matrix of the FlashAttention memory example."""
    p = pkv.Params(64, 8, 128, 64, 131072)
    rc, ws, sc = _ws(lib, p, batch=8)
    assert rc == 0
    scores = oracle.score_matrix_bytes(131072, 2, heads=64, batch=8)
    assert ws + sc < scores / 1000
    p2 = pkv.Params(64, 8, 128, 64, 2 * 131072)
    _, ws2, sc2 = _ws(lib, p2, batch=8)
    assert ws2 + sc2 <= 2 * (ws + sc)


def test_capacity_matches_oracle_formula(lib):
    from oracle.plan import decode_capacity, decode_target_items, extend_capacity
    for (hq, hkv, maxl, chunk, tgt, B, fp8) in [(32, 8, 4097, 0, 4096, 64, False), (64, 8, 131073, 0, 4096, 8, False),
                                                (32, 8, 5000, 64, 0, 37, False), (40, 2, 700, 0, 64, 5, False),
                                                (32, 8, 4097, 0, 100, 64, False), (32, 8, 4097, 0, 100, 64, True),
                                                (32, 8, 300, 0, 40000, 64, True)]:
        extra = dict(kv_dtype=pkv.PKV_FP8_E4M3, k_block=64, q_block=1) if fp8 else {}
        p = pkv.Params(hq, hkv, 128, 16, maxl, kv_chunk=chunk, split_target=tgt, **extra)
        rc, ws, sc = _ws(lib, p, batch=B)
        target = decode_target_items(hkv, hq // hkv, tgt, 1)
        cap = decode_capacity(B, maxl, target, chunk, 64 if fp8 else 32)
        assert sc >= cap * hq * 129 * 4
        assert ws >= (16 + B + 1 + 4 * cap) * 4
    p = pkv.Params(32, 8, 128, 16, 4096)
    rc, ws, _ = _ws(lib, p, mode=pkv.PKV_EXTEND, batch=16, total_q=17000)
    assert ws >= 4 * (16 + 17 + 8 * extend_capacity(16, 17000, 4))


def test_default_split_target_sizes_for_resident_waves(lib):
    """Without a device the library sizes decode plans for 256 CUs x 16 resident
    waves, the same as an explicit split_target of 4096 waves."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only fallback; a device reports its own occupancy")
    for hq, hkv, B in ((32, 8, 64), (64, 8, 8), (40, 2, 5)):
        p0 = pkv.Params(hq, hkv, 128, 16, 131073)
        p1 = pkv.Params(hq, hkv, 128, 16, 131073, split_target=4096)
        assert _ws(lib, p0, batch=B) == _ws(lib, p1, batch=B)


def _shape_params(n=1):
    return pkv.Params(8, 2, 128, 16, max_kv_len=64, decode_q_len=n)


def test_binding_rejects_q_out_lse_shapes():
    """Shapes the kernels would write past: out of [B, Hq, d] with several new
    tokens per request, lse of [B], q with the wrong head count or head_dim."""
    import torch
    from flashattention_paged_kv_amd import binding as bd
    p = _shape_params(n=4)
    q = torch.empty(3 * 4, 8, 128)
    bd._check_q_out_lse(p, q, torch.empty(12, 8, 128), torch.empty(12, 8), 12)  # good
    for q_, out, lse in ((q, torch.empty(3, 8, 128), None),      # out for one token per request
                         (q, None, torch.empty(12)),                 # lse of [rows]
                         (q, None, torch.empty(3, 8)),               # lse for one token per request
                         (torch.empty(12, 4, 128), None, None),      # wrong Hq
                         (torch.empty(12, 8, 64), None, None),       # wrong d
                         (torch.empty(3, 8, 128), None, None)):      # q rows
        with pytest.raises(ValueError):
            bd._check_q_out_lse(p, q_, out, lse, 12)


def test_binding_rejects_short_page_tables():
    import torch
    from flashattention_paged_kv_amd import binding as bd
    p = _shape_params()
    bd._check_page_table(p, torch.empty(4, 64), None, 4)
    bd._check_page_table(p, torch.empty(2, 64), torch.empty(4), 4)  # rows reached through the indirection
    with pytest.raises(ValueError):
        bd._check_page_table(p, torch.empty(3, 64), None, 4)  # a request without a row
    with pytest.raises(ValueError):
        bd._check_page_table(p, torch.empty(4, 64), torch.empty(3), 4)
    with pytest.raises(ValueError):
        bd._check_page_table(p, torch.empty(4, 32), None, 4)  # rows shorter than max_kv_len
