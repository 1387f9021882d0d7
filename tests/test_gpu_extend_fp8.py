"""GPU parity of the 8-bit (OCP E4M3) Sage extend against the fp64 oracle of
the formula, through the C ABI via the ctypes binding."""
from dataclasses import replace

import numpy as np
import pytest

import fp8_cases
import full_size
import oracle
from gpu_util import FP8_REL_L2, FP8_REL_L2_SAME_MAX, check_rel_l2, dev_f32, dev_i32, dev_u8, host, rel_l2, torch_mod
from workloads import Spec, make_host_batch, pool_before_store

pytestmark = pytest.mark.gpu


def _pkv():
    import flashattention_paged_kv_amd as pkv
    return pkv


def run_fp8_extend(hb, v_mean=None, sm_scale=None):
    torch = torch_mod()
    pkv = _pkv()
    lay = hb.layout
    spec = lay.spec
    k_pool = dev_u8(pool_before_store(hb.k_codes, lay.new_slots, fill=0x7F))
    v_pool = dev_u8(pool_before_store(hb.v_codes, lay.new_slots, fill=0x7F))
    params = pkv.Params(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                        max_kv_len=lay.req_to_token.shape[1], kv_dtype=pkv.PKV_FP8_E4M3,
                        q_block=1, k_block=spec.k_block)
    seq, cu, rtt = dev_i32(lay.seq_lens), dev_i32(lay.cu_seqlens_q), dev_i32(lay.req_to_token)
    plan = pkv.plan_metadata(params, pkv.PKV_EXTEND, seq, cu, total_q=lay.total_q)
    pkv.kv_store(params, k_pool, v_pool, dev_u8(hb.k_new_codes), dev_u8(hb.v_new_codes), dev_i32(lay.new_slots))
    lse = torch.empty((lay.total_q, spec.num_q_heads), dtype=torch.float32, device="cuda")
    out = pkv.attn_extend(params, dev_u8(hb.q_codes), k_pool, v_pool, rtt, seq, cu, plan, lse=lse,
                          sm_scale=sm_scale, sfq=dev_f32(hb.sfq), sfk=dev_f32(hb.sfk), sfv=dev_f32(hb.sfv),
                          v_mean=None if v_mean is None else dev_f32(v_mean))
    torch.cuda.synchronize()
    return host(out), lse.cpu().numpy().astype(np.float64)


def oracle_fp8_extend(hb, v_mean=None, sm_scale=None):
    lay = hb.layout
    return oracle.sage_extend(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, lay.seq_lens, lay.cu_seqlens_q,
                              hb.sfq, hb.sfk, hb.sfv, lay.spec.k_block, sm_scale=sm_scale, v_mean=v_mean)


SMALL = Spec("f8_ext_small", "extend", 4, 32, 8, 128, 16, (0, 300), (1, 300), dtype="fp8", k_block=16)


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("k_block", [16, 64])
def test_fp8_extend_matches_sage_oracle(seed, k_block):
    hb = make_host_batch(replace(SMALL, k_block=k_block), seed)
    o, lse = run_fp8_extend(hb)
    ro, rlse = oracle_fp8_extend(hb)
    check_rel_l2(o, ro, f"extend 8-bit seed={seed} k_block={k_block}")
    assert np.abs(lse - rlse).max() <= 1e-3


@pytest.mark.parametrize("hq,hkv,page", [(8, 8, 1), (64, 8, 64), (12, 4, 16)])
def test_fp8_extend_head_groupings_and_pages(hq, hkv, page):
    spec = Spec(f"f8_ext_{hq}_{hkv}_{page}", "extend", 3, hq, hkv, 128, page, (0, 200), (1, 150), dtype="fp8",
                k_block=16)
    hb = make_host_batch(spec, 3)
    o, lse = run_fp8_extend(hb)
    ro, rlse = oracle_fp8_extend(hb)
    check_rel_l2(o, ro, f"extend 8-bit hq={hq} hkv={hkv} page={page}")
    assert np.abs(lse - rlse).max() <= 1e-3


def test_fp8_extend_v_mean_and_scale():
    hb = make_host_batch(SMALL, 4)
    vm = np.random.default_rng(0).uniform(-1, 1, size=hb.sfv.shape).astype(np.float32)
    o, lse = run_fp8_extend(hb, v_mean=vm, sm_scale=0.05)
    ro, rlse = oracle_fp8_extend(hb, v_mean=vm, sm_scale=0.05)
    check_rel_l2(o, ro, "extend 8-bit v_mean, sm_scale 0.05")
    assert np.abs(lse - rlse).max() <= 1e-3


def test_fp8_extend_zero_queries_closed_form():
    """q8 = 0: p = 1 for every visible key, P8 = 448 exactly, so O = sfV * mean(V8)
    over each row's visible keys and lse = ln(visible keys)."""
    hb = make_host_batch(SMALL, 5)
    hb.q_codes[:] = 0
    o, lse = run_fp8_extend(hb)
    ro, rlse = oracle_fp8_extend(hb)
    check_rel_l2(o, ro, "extend 8-bit zero queries", bound=1e-2)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-4)


def test_fp8_extend_with_one_new_token_equals_fp8_decode():
    """Same inputs through both 8-bit kernels: n = 1 per request in the extend,
    one decode row per request (sfQ per row = per request)."""
    torch = torch_mod()
    pkv = _pkv()
    spec = Spec("f8_ext_n1", "extend", 6, 32, 8, 128, 16, (0, 900), 1, dtype="fp8", k_block=16)
    hb = make_host_batch(spec, 6)
    lay = hb.layout
    o_ext, l_ext = run_fp8_extend(hb)
    k_pool = dev_u8(pool_before_store(hb.k_codes, lay.new_slots, fill=0x7F))
    v_pool = dev_u8(pool_before_store(hb.v_codes, lay.new_slots, fill=0x7F))
    params = pkv.Params(32, 8, 128, 16, max_kv_len=lay.req_to_token.shape[1], kv_dtype=pkv.PKV_FP8_E4M3,
                        q_block=1, k_block=16)
    seq, rtt = dev_i32(lay.seq_lens), dev_i32(lay.req_to_token)
    plan = pkv.plan_metadata(params, pkv.PKV_DECODE, seq)
    pkv.kv_store(params, k_pool, v_pool, dev_u8(hb.k_new_codes), dev_u8(hb.v_new_codes), dev_i32(lay.new_slots))
    lse = torch.empty((spec.batch, 32), dtype=torch.float32, device="cuda")
    out = pkv.attn_decode(params, dev_u8(hb.q_codes), k_pool, v_pool, rtt, seq, plan, lse=lse, sfq=dev_f32(hb.sfq),
                          sfk=dev_f32(hb.sfk), sfv=dev_f32(hb.sfv))
    torch.cuda.synchronize()
    o_dec = host(out)
    check_rel_l2(o_ext, o_dec, "extend n=1 vs decode, 8-bit")
    assert np.abs(l_ext - lse.cpu().numpy()).max() <= 1e-3


def test_full_size_fp8_extend_longest_request_and_sampled_rows():
    """The full 8-bit extend workload in the bench's launch configuration:
    every row and head of its longest request against the oracle, and 1024
    more (row, head) pairs drawn over the whole batch, each recomputed over
    its visible keys."""
    torch = torch_mod()
    pkv = _pkv()
    from workloads import SPECS, make_device_batch
    spec = SPECS["extend_fp8"]
    db = make_device_batch(spec, seed=0, layers=1)
    lay = db.layout
    params = pkv.Params(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                        max_kv_len=lay.req_to_token.shape[1], kv_dtype=pkv.PKV_FP8_E4M3, q_block=1,
                        k_block=spec.k_block)
    plan = pkv.plan_metadata(params, pkv.PKV_EXTEND, db.seq_lens, db.cu_seqlens_q, total_q=lay.total_q)
    pkv.kv_store(params, db.k_pools[0], db.v_pools[0], db.k_new[0], db.v_new[0], db.new_slots)
    lse = torch.empty((lay.total_q, spec.num_q_heads), dtype=torch.float32, device="cuda")
    out = pkv.attn_extend(params, db.q, db.k_pools[0], db.v_pools[0], db.req_to_token, db.seq_lens,
                          db.cu_seqlens_q, plan, lse=lse, sfq=db.sfq, sfk=db.sfk, sfv=db.sfv)
    torch.cuda.synchronize()
    o = host(out)
    lse_h = lse.cpu().numpy()
    assert np.all(np.isfinite(o))
    b_long = int(np.argmax(lay.new_lens * lay.seq_lens))
    ro, rl = full_size.extend_reference(db, requests=[b_long], sage=True)
    rows = slice(int(lay.cu_seqlens_q[b_long]), int(lay.cu_seqlens_q[b_long + 1]))
    check_rel_l2(o[rows], ro[rows], f"extend_fp8 request {b_long}, all {ro[rows].shape}")
    assert np.abs(lse_h[rows] - rl[rows]).max() <= 1e-3
    sfq, sfk, sfv = db.sfq.cpu().numpy(), db.sfk.cpu().numpy(), db.sfv.cpu().numpy()
    rng = np.random.default_rng(1)
    G = spec.num_q_heads // spec.num_kv_heads
    got, want = [], []
    for _ in range(1024):
        b = int(rng.integers(0, spec.batch))
        n, p = int(lay.new_lens[b]), int(lay.prefix_lens[b])
        i = int(rng.choice([0, n - 1, int(rng.integers(0, n))]))
        h = int(rng.integers(0, spec.num_q_heads))
        g = h // G
        row = int(lay.cu_seqlens_q[b]) + i
        vis = p + i + 1
        slots = db.req_to_token[b, :vis].long()
        K = db.k_pools[0][slots, g:g + 1].cpu().numpy()
        V = db.v_pools[0][slots, g:g + 1].cpu().numpy()
        q8 = db.q[row:row + 1, h:h + 1].cpu().numpy()
        # one decode-shaped request over the row's visible keys (Hq = Hkv = 1)
        r1, l1 = oracle.sage_decode(q8, K, V, np.arange(vis)[None], [vis], sfq[row:row + 1, h:h + 1],
                                    sfk[b:b + 1, g:g + 1], sfv[b:b + 1, g:g + 1], spec.k_block)
        got.append(o[row, h])
        want.append(r1.ravel())
        assert abs(float(lse_h[row, h]) - l1[0, 0]) <= 1e-3
    check_rel_l2(np.concatenate(got), np.concatenate(want), "extend_fp8, 1024 sampled (row, head) pairs")


TIGHT_CASES = {"kb16": SMALL, "kb64": replace(SMALL, k_block=64),
               # one to twelve keys per row: the quantisation step weighs more (in the
               # oracle, rounding p before scaling moves O by about 2%, dividing by the
               # codes' sum by about 0.7%)
               "short": Spec("f8_ext_short", "extend", 16, 32, 8, 128, 16, (0, 6), (1, 6), dtype="fp8", k_block=16)}


@pytest.mark.parametrize("case", sorted(TIGHT_CASES))
def test_fp8_extend_tight_when_the_row_max_is_first(case):
    """Every row's maximum at position 0, the first key the kernel reads.
    The kernel then sets its reference 2 (log2 units) above that max once
    and keeps it, so its codes are E4M3(448·p/4) = E4M3(448·p)/4 exactly
    (a power-of-two shift of a normal E4M3 value; sm_scale 0.03 keeps
    448·p/4 above the subnormal range), and the bound is the bf16 rounding
    of O."""
    hb = make_host_batch(TIGHT_CASES[case], 61)
    gap = fp8_cases.put_row_max_first(hb, "e4m3")
    assert gap > 0
    o, lse = run_fp8_extend(hb, sm_scale=0.03)
    ro, rlse = oracle_fp8_extend(hb, sm_scale=0.03)
    check_rel_l2(o, ro, f"extend E4M3 {case}, row max first", bound=FP8_REL_L2_SAME_MAX)
    assert np.abs(lse - rlse).max() <= 1e-4
