"""GPU parity of the bf16 causal extend (plan + kv_store + attn_extend) against the
fp64 oracle, through the C ABI via the ctypes binding."""
import numpy as np
import pytest

import full_size
import oracle
from gpu_util import assert_bf16_close, assert_lse_close, dev_bf16, dev_i32, host, torch_mod
from workloads import SPECS, Spec, make_device_batch, make_host_batch, permute_pages, pool_before_store, round_bf16

pytestmark = pytest.mark.gpu


def _pkv():
    import flashattention_paged_kv_amd as pkv
    return pkv


def run_extend(hb, sm_scale=None, lse=True):
    torch = torch_mod()
    pkv = _pkv()
    lay = hb.layout
    spec = lay.spec
    q = round_bf16(hb.q)
    k_pool = dev_bf16(pool_before_store(round_bf16(hb.k_pool), lay.new_slots))
    v_pool = dev_bf16(pool_before_store(round_bf16(hb.v_pool), lay.new_slots))
    params = pkv.Params(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                        max_kv_len=max(lay.req_to_token.shape[1], 1))
    seq, cu, rtt = dev_i32(lay.seq_lens), dev_i32(lay.cu_seqlens_q), dev_i32(lay.req_to_token)
    plan = pkv.plan_metadata(params, pkv.PKV_EXTEND, seq, cu, total_q=lay.total_q)
    pkv.kv_store(params, k_pool, v_pool, dev_bf16(round_bf16(hb.k_new)), dev_bf16(round_bf16(hb.v_new)),
                 dev_i32(lay.new_slots))
    lse_t = torch.empty((lay.total_q, spec.num_q_heads), dtype=torch.float32, device="cuda") if lse else None
    out = pkv.attn_extend(params, dev_bf16(q), k_pool, v_pool, rtt, seq, cu, plan, lse=lse_t, sm_scale=sm_scale)
    torch.cuda.synchronize()
    return host(out), (lse_t.cpu().numpy().astype(np.float64) if lse else None), plan


def oracle_extend(hb, sm_scale=None):
    lay = hb.layout
    return oracle.paged_attention(round_bf16(hb.q), round_bf16(hb.k_pool), round_bf16(hb.v_pool),
                                  lay.req_to_token, lay.seq_lens, lay.cu_seqlens_q, sm_scale=sm_scale)


MEDIUM = Spec("ext_med", "extend", 4, 32, 8, 128, 16, (0, 300), (1, 300))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_extend_config(seed):
    hb = make_host_batch(SPECS["tiny_extend"], seed)
    o, lse, _ = run_extend(hb)
    ro, rlse = oracle_extend(hb)
    assert_bf16_close(o, ro, "tiny extend")
    assert_lse_close(lse, rlse, "tiny extend")


@pytest.mark.parametrize("seed", [0, 1])
def test_medium_extend_ragged(seed):
    hb = make_host_batch(MEDIUM, seed)
    o, lse, _ = run_extend(hb)
    ro, rlse = oracle_extend(hb)
    assert_bf16_close(o, ro, "medium extend")
    assert_lse_close(lse, rlse, "medium extend")


@pytest.mark.parametrize("hq,hkv,d,page", [(8, 8, 128, 16), (16, 8, 128, 1), (64, 8, 128, 64), (12, 4, 64, 16),
                                           (32, 2, 128, 16), (6, 6, 64, 2)])
def test_head_groupings_and_pages(hq, hkv, d, page):
    spec = Spec("ext_shape", "extend", 3, hq, hkv, d, page, (0, 200), (1, 160))
    hb = make_host_batch(spec, 4)
    o, lse, _ = run_extend(hb)
    ro, rlse = oracle_extend(hb)
    assert_bf16_close(o, ro, f"extend hq={hq} hkv={hkv} d={d} P={page}")
    assert_lse_close(lse, rlse)


def test_pure_causal_prefill_and_empty_requests():
    spec = Spec("ext_edge", "extend", 5, 8, 2, 128, 16, [0, 0, 37, 5, 0], [70, 0, 0, 1, 129])
    hb = make_host_batch(spec, 5)
    o, lse, _ = run_extend(hb, sm_scale=0.2)
    ro, rlse = oracle_extend(hb, sm_scale=0.2)
    assert_bf16_close(o, ro, "edge extend")
    assert_lse_close(lse, rlse)


def test_decode_equals_extend_with_one_new_token():
    from test_gpu_decode import run_decode
    spec = Spec("ext_one", "extend", 6, 32, 8, 128, 16, (0, 900), 1)
    hb = make_host_batch(spec, 6)
    o_ext, l_ext, _ = run_extend(hb)
    o_dec, l_dec, _, _ = run_decode(hb)
    assert np.abs(o_ext - o_dec).max() <= 2e-2
    assert np.abs(l_ext - l_dec).max() <= 1e-4


def test_page_relabelling_is_bit_invariant_and_deterministic():
    hb = make_host_batch(MEDIUM, 7)
    o1, l1, _ = run_extend(hb)
    o1b, l1b, _ = run_extend(hb)
    assert np.array_equal(o1, o1b) and np.array_equal(l1, l1b)
    lay2, slot_map = permute_pages(hb.layout, np.random.default_rng(2))
    k2 = np.full_like(hb.k_pool, np.nan)
    v2 = np.full_like(hb.v_pool, np.nan)
    k2[slot_map] = hb.k_pool
    v2[slot_map] = hb.v_pool
    hb.layout, hb.k_pool, hb.v_pool = lay2, k2, v2
    o2, l2, _ = run_extend(hb)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_shared_prefix_pages():
    """Every request's page-table row starts with request 0's prefix pages
    (a shared prompt prefix); new tokens stay in each request's own pages."""
    spec = Spec("ext_sharedpfx", "extend", 5, 32, 8, 128, 16, (200, 500), (1, 300))
    hb = make_host_batch(spec, 25)
    lay = hb.layout
    shared = (int(lay.prefix_lens.min()) // 16) * 16
    lay.req_to_token[1:, :shared] = lay.req_to_token[0, :shared]
    o, lse, _ = run_extend(hb)
    ro, rlse = oracle_extend(hb)
    assert_bf16_close(o, ro, "shared prefix")
    assert_lse_close(lse, rlse)


def test_extend_plan_matches_oracle_rederivation():
    torch = torch_mod()
    pkv = _pkv()
    rng = np.random.default_rng(8)
    for G, B in ((4, 16), (1, 3), (8, 40), (3, 7)):
        n = rng.integers(0, 700, size=B).astype(np.int32)
        p = rng.integers(0, 900, size=B).astype(np.int32)
        L = (n + p).astype(np.int32)
        cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        T = int(cu[-1])
        params = pkv.Params(8 * G, 8, 128, 16, max_kv_len=int(L.max()))
        plan = pkv.plan_metadata(params, pkv.PKV_EXTEND, dev_i32(L), dev_i32(cu), total_q=T)
        torch.cuda.synchronize()
        ws = plan.workspace.cpu().numpy().view(np.int32)
        ref = oracle.plan_extend(L, cu, G, int(L.max()), T)
        num = ws[2]
        items_off = -(-(16 + B + 1) // 4) * 4
        items = ws[items_off:items_off + 4 * num].reshape(-1, 4)
        assert num == len(ref["items"]) and ws[3] == ref["capacity"] and ws[4] == ref["block_tokens"]
        assert np.array_equal(items[:, :3], ref["items"])


def test_full_size_extend_every_element():
    """The full extend workload in the bench's launch configuration; every
    output element and lse of every new row is compared with the oracle, run
    per (request, kv head) on host copies of the request's rows."""
    torch = torch_mod()
    pkv = _pkv()
    spec = SPECS["extend_bf16"]
    db = make_device_batch(spec, seed=0, layers=1)
    lay = db.layout
    params = pkv.Params(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                        max_kv_len=lay.req_to_token.shape[1])
    plan = pkv.plan_metadata(params, pkv.PKV_EXTEND, db.seq_lens, db.cu_seqlens_q, total_q=lay.total_q)
    pkv.kv_store(params, db.k_pools[0], db.v_pools[0], db.k_new[0], db.v_new[0], db.new_slots)
    lse = torch.empty((lay.total_q, spec.num_q_heads), dtype=torch.float32, device="cuda")
    out = pkv.attn_extend(params, db.q, db.k_pools[0], db.v_pools[0], db.req_to_token, db.seq_lens,
                          db.cu_seqlens_q, plan, lse=lse)
    torch.cuda.synchronize()
    ro, rl = full_size.extend_reference(db)
    err, rel = assert_bf16_close(host(out), ro, "extend_bf16")
    assert_lse_close(lse.cpu().numpy(), rl, "extend_bf16")
    print(f"extend_bf16: every element of {ro.shape}: max abs {err:.3e}, rel L2 {rel:.3e}", flush=True)
