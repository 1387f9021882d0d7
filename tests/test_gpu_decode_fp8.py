"""GPU parity of the 8-bit (OCP E4M3) Sage decode against the fp64 oracle of the
formula, through the C ABI via the ctypes binding."""
import numpy as np
import pytest

import fp8_cases
import full_size
import oracle
from gpu_util import (FP8_REL_L2, FP8_REL_L2_SAME_MAX, check_rel_l2, dev_f32, dev_i32, dev_qk8, dev_u8, host, kv_dtype_of, qk_codes_of, rel_l2,
                      torch_mod)
from workloads import SPECS, Spec, make_device_batch, make_host_batch, pool_before_store

pytestmark = pytest.mark.gpu


def _pkv():
    import flashattention_paged_kv_amd as pkv
    return pkv


def run_fp8(hb, kv_chunk=0, v_mean=None, sm_scale=None, split_target=0, seq_lens=None):
    torch = torch_mod()
    pkv = _pkv()
    lay = hb.layout
    spec = lay.spec
    k_pool = dev_qk8(pool_before_store(hb.k_codes, lay.new_slots, fill=0x7F), spec)
    v_pool = dev_u8(pool_before_store(hb.v_codes, lay.new_slots, fill=0x7F))
    params = pkv.Params(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                        max_kv_len=lay.req_to_token.shape[1], kv_dtype=kv_dtype_of(pkv, spec),
                        q_block=spec.q_block, k_block=spec.k_block, kv_chunk=kv_chunk,
                        split_target=split_target)
    seq = dev_i32(lay.seq_lens if seq_lens is None else seq_lens)
    rtt = dev_i32(lay.req_to_token)
    plan = pkv.plan_metadata(params, pkv.PKV_DECODE, seq)
    pkv.kv_store(params, k_pool, v_pool, dev_qk8(hb.k_new_codes, spec), dev_u8(hb.v_new_codes),
                 dev_i32(lay.new_slots))
    lse = torch.empty((spec.batch, spec.num_q_heads), dtype=torch.float32, device="cuda")
    out = pkv.attn_decode(params, dev_qk8(hb.q_codes, spec), k_pool, v_pool, rtt, seq, plan, lse=lse,
                          sm_scale=sm_scale,
                          sfq=dev_f32(hb.sfq), sfk=dev_f32(hb.sfk), sfv=dev_f32(hb.sfv),
                          v_mean=None if v_mean is None else dev_f32(v_mean))
    torch.cuda.synchronize()
    return host(out), lse.cpu().numpy().astype(np.float64)


def oracle_fp8(hb, v_mean=None, sm_scale=None, seq_lens=None):
    lay = hb.layout
    seq = lay.seq_lens if seq_lens is None else seq_lens
    return oracle.sage_decode(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, seq, hb.sfq, hb.sfk,
                              hb.sfv, lay.spec.k_block, sm_scale=sm_scale, v_mean=v_mean,
                              qk_codes=qk_codes_of(lay.spec))


SMALL = Spec("f8_small", "decode", 6, 32, 8, 128, 16, (0, 700), 1, dtype="fp8", k_block=64)


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("k_block", [64, 16])
def test_fp8_decode_matches_sage_oracle(seed, k_block):
    from dataclasses import replace
    hb = make_host_batch(replace(SMALL, k_block=k_block), seed)
    o, lse = run_fp8(hb)
    ro, rlse = oracle_fp8(hb)
    check_rel_l2(o, ro, f"decode E4M3 seed={seed} k_block={k_block}")
    assert np.abs(lse - rlse).max() <= 1e-3


SMALL_I8 = Spec("i8_small", "decode", 6, 32, 8, 128, 16, (0, 700), 1, dtype="int8", k_block=64)


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("k_block", [64, 16])
def test_int8_decode_matches_sage_oracle(seed, k_block):
    """INT8 Q and K codes (the Sage page's code §3 and §4), E4M3 V."""
    from dataclasses import replace
    hb = make_host_batch(replace(SMALL_I8, k_block=k_block), 40 + seed)
    o, lse = run_fp8(hb)
    ro, rlse = oracle_fp8(hb)
    check_rel_l2(o, ro, f"decode INT8 seed={seed} k_block={k_block}")
    assert np.abs(lse - rlse).max() <= 1e-3


def test_int8_extreme_codes_and_split_merge_with_v_mean():
    """Codes at -128 and 127 in Q and K (int32 dot products up to 2^21) through
    split chunks and the merge, against the oracle."""
    hb = make_host_batch(SMALL_I8, 45)
    rng = np.random.default_rng(46)
    hb.q_codes = rng.choice(np.array([-128, -127, 0, 127], np.int8), size=hb.q_codes.shape)
    ext = rng.random(hb.k_codes.shape) < 0.5
    hb.k_codes = np.where(ext, rng.choice(np.array([-128, 127], np.int8), size=hb.k_codes.shape), hb.k_codes)
    hb.k_new_codes = hb.k_codes[hb.layout.new_slots].copy()
    # keep the scores in a range where softmax is not a one-hot: scale the Q/K steps down
    hb.sfq = (hb.sfq / 64).astype(np.float32)
    vm = rng.uniform(-1, 1, size=hb.sfv.shape).astype(np.float32)
    o1, l1 = run_fp8(hb, kv_chunk=64, v_mean=vm)
    o2, l2 = run_fp8(hb, v_mean=vm)
    ro, rlse = oracle_fp8(hb, v_mean=vm)
    check_rel_l2(o1, ro, "decode INT8 extreme codes, split")
    check_rel_l2(o2, ro, "decode INT8 extreme codes")
    assert np.abs(l1 - rlse).max() <= 1e-3 and np.abs(l2 - rlse).max() <= 1e-3


@pytest.mark.parametrize("n,hq,hkv,kv_chunk,with_vm", [(2, 32, 8, 0, False), (4, 32, 8, 64, True), (3, 16, 2, 0, True)])
def test_int8_several_new_tokens_per_request(n, hq, hkv, kv_chunk, with_vm):
    spec = Spec("i8_multi", "decode", 5, hq, hkv, 128, 16, (0, 900), n, dtype="int8", k_block=64)
    hb = make_host_batch(spec, 50 + n)
    lay = hb.layout
    vm = np.random.default_rng(150 + n).standard_normal((spec.batch, hkv, 128)).astype(np.float32) if with_vm else None
    o, l, sfq_rows = run_fp8_multi(hb, n, v_mean=vm, kv_chunk=kv_chunk)
    ro, rl = oracle.sage_extend(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, lay.seq_lens,
                                lay.cu_seqlens_q, sfq_rows, hb.sfk, hb.sfv, spec.k_block, v_mean=vm, qk_codes="int8")
    check_rel_l2(o, ro, f"decode E4M3 n={n}")
    assert np.abs(l - rl).max() <= 1e-3


def test_fp8_split_merge_and_v_mean():
    hb = make_host_batch(SMALL, 3)
    vm = np.random.default_rng(0).uniform(-1, 1, size=hb.sfv.shape).astype(np.float32)
    o1, l1 = run_fp8(hb, kv_chunk=64, v_mean=vm)
    o2, l2 = run_fp8(hb, kv_chunk=4096, v_mean=vm)
    ro, rlse = oracle_fp8(hb, v_mean=vm)
    check_rel_l2(o1, ro, "decode E4M3 split, v_mean")
    check_rel_l2(o2, ro, "decode E4M3 unsplit, v_mean")
    assert np.abs(l1 - rlse).max() <= 1e-3


def test_fp8_many_segments_and_empty_requests_with_v_mean():
    """Three long chunks over 300 short requests (~100 segments each, so the
    segment records are reloaded mid-stream); every seventh request is empty
    and gets O = v_mean, lse = -inf, as in the oracle's epilogue."""
    spec = Spec("f8_manyseg", "decode", 300, 8, 2, 128, 16, (0, 120), 1, dtype="fp8", k_block=64)
    hb = make_host_batch(spec, 23)
    seq = hb.layout.seq_lens.copy()
    seq[::7] = 0
    vm = np.random.default_rng(1).uniform(-1, 1, size=hb.sfv.shape).astype(np.float32)
    o, lse = run_fp8(hb, v_mean=vm, split_target=6, seq_lens=seq)
    ro, rlse = oracle_fp8(hb, v_mean=vm, seq_lens=seq)
    check_rel_l2(o, ro, "decode E4M3 many segments")
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - rlse[fin]).max() <= 1e-3
    G = spec.num_q_heads // spec.num_kv_heads
    want = np.repeat(vm[::7], G, axis=1)
    np.testing.assert_allclose(o[::7], want, rtol=1e-2, atol=1e-2)


def test_fp8_constant_scores_closed_form():
    """q8 = 0: every p is 1, P8 = 448 exactly, so O = sfV * mean(V8) up to fp32 sums."""
    hb = make_host_batch(SMALL, 4)
    hb.q_codes[:] = 0
    o, lse = run_fp8(hb)
    ro, _ = oracle_fp8(hb)
    lay = hb.layout
    for b in range(SMALL.batch):
        L = int(lay.seq_lens[b])
        np.testing.assert_allclose(lse[b], np.log(L), rtol=0, atol=1e-5)
    check_rel_l2(o, ro, "decode E4M3 constant scores", bound=FP8_REL_L2_SAME_MAX)


@pytest.mark.parametrize("name", ["decode_fp8", "decode_int8"])
def test_full_size_8bit_decode_every_element(name):
    """The full 8-bit decode workloads (E4M3, and INT8 Q/K) in the bench's
    launch configuration; every output element and lse against the oracle."""
    torch = torch_mod()
    pkv = _pkv()
    spec = SPECS[name]
    db = make_device_batch(spec, seed=0, layers=1)
    lay = db.layout
    params = pkv.Params(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                        max_kv_len=lay.req_to_token.shape[1], kv_dtype=kv_dtype_of(pkv, spec),
                        q_block=spec.q_block, k_block=spec.k_block)
    plan = pkv.plan_metadata(params, pkv.PKV_DECODE, db.seq_lens)
    pkv.kv_store(params, db.k_pools[0], db.v_pools[0], db.k_new[0], db.v_new[0], db.new_slots)
    lse = torch.empty((spec.batch, spec.num_q_heads), dtype=torch.float32, device="cuda")
    out = pkv.attn_decode(params, db.q, db.k_pools[0], db.v_pools[0], db.req_to_token, db.seq_lens, plan, lse=lse,
                          sfq=db.sfq, sfk=db.sfk, sfv=db.sfv)
    torch.cuda.synchronize()
    ro, rl = full_size.decode_reference(db, sage=True, qk_codes=qk_codes_of(spec))
    check_rel_l2(host(out), ro, f"{name} every element of {ro.shape}")
    assert np.abs(lse.cpu().numpy() - rl).max() <= 1e-3


def run_fp8_multi(hb, n, v_mean=None, kv_chunk=0, seed=None):
    """n new tokens per request in one 8-bit decode call, with one sfQ per
    new-token row (the request's scale times a per-row factor, so the row
    indexing is exercised).  Returns host (o, lse, the per-row sfQ)."""
    torch = torch_mod()
    pkv = _pkv()
    lay = hb.layout
    spec = lay.spec
    B, hq, hkv = spec.batch, spec.num_q_heads, spec.num_kv_heads
    rng = np.random.default_rng(n if seed is None else seed)
    sfq_rows = (hb.sfq[np.repeat(np.arange(B), n)] * rng.uniform(0.8, 1.25, (B * n, hq))).astype(np.float32)
    k_pool = dev_qk8(pool_before_store(hb.k_codes, lay.new_slots, fill=0x7F), spec)
    v_pool = dev_u8(pool_before_store(hb.v_codes, lay.new_slots, fill=0x7F))
    params = pkv.Params(hq, hkv, 128, spec.page_size, max_kv_len=lay.req_to_token.shape[1],
                        kv_dtype=kv_dtype_of(pkv, spec), q_block=1, k_block=spec.k_block, kv_chunk=kv_chunk,
                        decode_q_len=n)
    seq = dev_i32(lay.seq_lens)
    plan = pkv.plan_metadata(params, pkv.PKV_DECODE, seq)
    pkv.kv_store(params, k_pool, v_pool, dev_qk8(hb.k_new_codes, spec), dev_u8(hb.v_new_codes),
                 dev_i32(lay.new_slots))
    lse = torch.empty((B * n, hq), dtype=torch.float32, device="cuda")
    out = pkv.attn_decode(params, dev_qk8(hb.q_codes, spec), k_pool, v_pool, dev_i32(lay.req_to_token), seq, plan,
                          lse=lse,
                          sfq=dev_f32(sfq_rows), sfk=dev_f32(hb.sfk), sfv=dev_f32(hb.sfv),
                          v_mean=None if v_mean is None else dev_f32(v_mean))
    torch.cuda.synchronize()
    return host(out), lse.cpu().numpy().astype(np.float64), sfq_rows


# (5, 64, 8): 40 columns per kv head, three head groups, 24 units: the
# multi-token instance with plain K/V loads
@pytest.mark.parametrize("n,hq,hkv,kv_chunk,with_vm", [(2, 32, 8, 0, False), (4, 32, 8, 0, True), (8, 8, 8, 0, False),
                                                     (3, 16, 2, 128, True), (16, 8, 1, 0, False), (5, 40, 8, 64, False),
                                                     (5, 64, 8, 0, False)])
def test_fp8_several_new_tokens_per_request(n, hq, hkv, kv_chunk, with_vm):
    """n new tokens per request checked in one 8-bit decode call: new token i
    sees keys 0 .. L - n + i, one sfQ per new-token row; the oracle is the
    8-bit extend formula with n rows per request."""
    spec = Spec("f8_multi", "decode", 5, hq, hkv, 128, 16, (0, 900), n, dtype="fp8", k_block=64)
    hb = make_host_batch(spec, 20 + n)
    lay = hb.layout
    vm = np.random.default_rng(100 + n).standard_normal((spec.batch, hkv, 128)).astype(np.float32) if with_vm else None
    o, l, sfq_rows = run_fp8_multi(hb, n, v_mean=vm, kv_chunk=kv_chunk)
    ro, rl = oracle.sage_extend(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, lay.seq_lens,
                                lay.cu_seqlens_q, sfq_rows, hb.sfk, hb.sfv, spec.k_block, v_mean=vm)
    check_rel_l2(o, ro, f"decode E4M3 n={n}")
    assert np.abs(l - rl).max() <= 1e-3


@pytest.mark.parametrize("dtype", ["fp8", "int8"])
def test_8bit_decode_many_kv_heads(dtype):
    """24 kv heads of one query head each (24 units per token): the kernel
    instances with plain K/V loads, against the Sage oracle."""
    spec = Spec("f8_mha", "decode", 5, 24, 24, 128, 16, (0, 800), 1, dtype=dtype, k_block=64)
    hb = make_host_batch(spec, 31)
    o, lse = run_fp8(hb, split_target=48)
    ro, rlse = oracle_fp8(hb)
    check_rel_l2(o, ro, f"decode {dtype} 24 kv heads")
    assert np.abs(lse - rlse)[np.isfinite(rlse)].max() <= 1e-3
    assert np.array_equal(np.isfinite(lse), np.isfinite(rlse))


# two to eight keys per request: few keys, so each request's E4M3 rounding of
# P does not average out and the quantisation step moves O by about 2%
SHORT = Spec("f8_short", "decode", 64, 32, 8, 128, 16, (1, 7), 1, dtype="fp8", k_block=16)
TIGHT_CASES = {"e4m3_kb64": SMALL, "e4m3_kb16": Spec("f8_small16", "decode", 6, 32, 8, 128, 16, (0, 700), 1,
                                                     dtype="fp8", k_block=16),
               "int8_kb64": SMALL_I8, "e4m3_short": SHORT,
               "int8_short": Spec("i8_short", "decode", 64, 32, 8, 128, 16, (1, 7), 1, dtype="int8", k_block=16)}


@pytest.mark.parametrize("case", sorted(TIGHT_CASES))
def test_8bit_decode_tight_when_the_row_max_is_first(case):
    """Every row's maximum at position 0 and one segment per request: the
    kernel's running max is the oracle's row max from the first tile on, so
    its E4M3 codes of P are the oracle's and the bound is the bf16 rounding of
    O.  (On the short requests, rounding p before scaling by 448 moves the
    oracle's O by about 2% and dividing by the codes' sum by about 0.9%.)"""
    spec = TIGHT_CASES[case]
    hb = make_host_batch(spec, 60)
    gap = fp8_cases.put_row_max_first(hb, qk_codes_of(spec))
    assert gap > 0
    o, lse = run_fp8(hb, kv_chunk=4096, sm_scale=0.03)
    ro, rlse = oracle_fp8(hb, sm_scale=0.03)
    check_rel_l2(o, ro, f"decode {case}, row max first", bound=FP8_REL_L2_SAME_MAX)
    assert np.abs(lse - rlse).max() <= 1e-4


@pytest.mark.parametrize("n", [2, 4])
def test_8bit_multi_token_decode_tight_when_the_row_max_is_first(n):
    """The same bound for several new tokens per request in one call: every
    new row sees position 0."""
    spec = Spec("f8_multi_tight", "decode", 5, 32, 8, 128, 16, (0, 900), n, dtype="fp8", k_block=64)
    hb = make_host_batch(spec, 62 + n)
    lay = hb.layout
    rng = np.random.default_rng(n)
    sfq_rows = (hb.sfq[np.repeat(np.arange(spec.batch), n)] * rng.uniform(0.8, 1.25, (spec.batch * n, 32)))
    hb.sfq = sfq_rows.astype(np.float32)  # one scale per row: the multi-token decode reads [B*n, Hq]
    fp8_cases.put_row_max_first(hb, "e4m3")
    torch = torch_mod()
    pkv = _pkv()
    k_pool = dev_u8(pool_before_store(hb.k_codes, lay.new_slots, fill=0x7F))
    v_pool = dev_u8(pool_before_store(hb.v_codes, lay.new_slots, fill=0x7F))
    params = pkv.Params(32, 8, 128, 16, max_kv_len=lay.req_to_token.shape[1], kv_dtype=pkv.PKV_FP8_E4M3,
                        q_block=1, k_block=64, kv_chunk=4096, decode_q_len=n)
    seq = dev_i32(lay.seq_lens)
    plan = pkv.plan_metadata(params, pkv.PKV_DECODE, seq)
    pkv.kv_store(params, k_pool, v_pool, dev_u8(hb.k_new_codes), dev_u8(hb.v_new_codes), dev_i32(lay.new_slots))
    out = pkv.attn_decode(params, dev_u8(hb.q_codes), k_pool, v_pool, dev_i32(lay.req_to_token), seq, plan,
                          sm_scale=0.03, sfq=dev_f32(hb.sfq), sfk=dev_f32(hb.sfk), sfv=dev_f32(hb.sfv))
    torch.cuda.synchronize()
    ro, _ = oracle.sage_extend(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, lay.seq_lens, lay.cu_seqlens_q,
                               hb.sfq, hb.sfk, hb.sfv, 64, sm_scale=0.03)
    check_rel_l2(host(out), ro, f"decode E4M3 n={n}, row max first", bound=FP8_REL_L2_SAME_MAX)
