"""GPU parity of the block-sparse decode (block_sparse_table + plan over the
selected lengths + attn_decode on the compacted table) against the fp64
block-sparse oracles, through the C ABI via the ctypes binding."""
import numpy as np
import pytest

import full_size
import oracle
from gpu_util import (FP8_REL_L2, check_rel_l2, assert_bf16_close, assert_lse_close, dev_bf16, dev_f32, dev_i32, dev_qk8, dev_u8,
                      host, kv_dtype_of, qk_codes_of, rel_l2, torch_mod)
from workloads import SPECS, Spec, block_mask, make_device_batch, make_host_batch, pool_before_store, round_bf16

pytestmark = pytest.mark.gpu


def _pkv():
    import flashattention_paged_kv_amd as pkv
    return pkv


def listed_positions(L, blocks, bs):
    """Logical positions of the listed blocks, in list order (the expected compaction)."""
    n = -(-int(L) // bs)
    return [k * bs + t for k in blocks if 0 <= k < n for t in range(bs) if k * bs + t < L]


def mask_with_edges(lay, bs, density, seed, empty=(), junk=False):
    """A drawn mask; requests in `empty` get no block; with `junk`, every list
    gains a negative number in front and out-of-range numbers behind."""
    indptr, idx = block_mask(lay.seq_lens, bs, density, np.random.default_rng(seed))
    ip, ix = [0], []
    for b in range(len(lay.seq_lens)):
        blocks = [] if b in empty else idx[indptr[b]:indptr[b + 1]].tolist()
        if junk:
            n = -(-int(lay.seq_lens[b]) // bs)
            blocks = [-7] + blocks + [n, n + 3]
        ix.extend(blocks)
        ip.append(len(ix))
    return np.asarray(ip, np.int32), np.asarray(ix, np.int32)


def run_sparse(hb, indptr, idx, bs, v_mean=None, sm_scale=None, rpi=None, rtt_rows=None):
    """Upload a host batch (new rows poisoned until kv_store), build the sparse
    tables, plan over their lengths and decode.  Returns host (o, lse, tables)."""
    torch = torch_mod()
    pkv = _pkv()
    lay = hb.layout
    spec = lay.spec
    fp8 = spec.dtype in ("fp8", "int8")
    rtt_host = lay.req_to_token if rtt_rows is None else rtt_rows
    if fp8:
        kw = dict(kv_dtype=kv_dtype_of(pkv, spec), q_block=spec.q_block, k_block=spec.k_block)
        k_pool = dev_qk8(pool_before_store(hb.k_codes, lay.new_slots, fill=0x7F), spec)
        v_pool = dev_u8(pool_before_store(hb.v_codes, lay.new_slots, fill=0x7F))
        k_new, v_new, q = dev_qk8(hb.k_new_codes, spec), dev_u8(hb.v_new_codes), dev_qk8(hb.q_codes, spec)
        sfk = dev_f32(hb.sfk)
    else:
        kw = {}
        k_pool = dev_bf16(pool_before_store(round_bf16(hb.k_pool), lay.new_slots))
        v_pool = dev_bf16(pool_before_store(round_bf16(hb.v_pool), lay.new_slots))
        k_new, v_new, q = dev_bf16(round_bf16(hb.k_new)), dev_bf16(round_bf16(hb.v_new)), dev_bf16(round_bf16(hb.q))
        sfk = None
    params = pkv.Params(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                        max_kv_len=lay.req_to_token.shape[1], **kw)
    pkv.kv_store(params, k_pool, v_pool, k_new, v_new, dev_i32(lay.new_slots))
    srtt, slens, ssfk = pkv.block_sparse_table(params, dev_i32(lay.seq_lens), dev_i32(rtt_host), dev_i32(indptr),
                                               dev_i32(idx), bs, req_pool_indices=None if rpi is None else dev_i32(rpi),
                                               sfk=sfk)
    plan = pkv.plan_metadata(params, pkv.PKV_DECODE, slens)
    lse = torch.empty((spec.batch, spec.num_q_heads), dtype=torch.float32, device="cuda")
    extra = dict(sfq=dev_f32(hb.sfq), sfk=ssfk, sfv=dev_f32(hb.sfv),
                 v_mean=None if v_mean is None else dev_f32(v_mean)) if fp8 else {}
    out = pkv.attn_decode(params, q, k_pool, v_pool, srtt, slens, plan, lse=lse, sm_scale=sm_scale, **extra)
    torch.cuda.synchronize()
    tables = (srtt.cpu().numpy(), slens.cpu().numpy(), None if ssfk is None else ssfk.cpu().numpy())
    return host(out), lse.cpu().numpy().astype(np.float64), tables


def oracle_sparse(hb, indptr, idx, bs, v_mean=None, sm_scale=None):
    lay = hb.layout
    if lay.spec.dtype in ("fp8", "int8"):
        return oracle.block_sparse_sage_decode(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, lay.seq_lens,
                                               indptr, idx, bs, hb.sfq, hb.sfk, hb.sfv, lay.spec.k_block,
                                               sm_scale=sm_scale, v_mean=v_mean, qk_codes=qk_codes_of(lay.spec))
    return oracle.block_sparse_decode(round_bf16(hb.q), round_bf16(hb.k_pool), round_bf16(hb.v_pool),
                                      lay.req_to_token, lay.seq_lens, indptr, idx, bs, sm_scale=sm_scale)


BF = Spec("bs_bf", "decode", 6, 32, 8, 128, 16, (0, 2000), 1)
F8 = Spec("bs_f8", "decode", 6, 32, 8, 128, 16, (0, 2000), 1, dtype="fp8", k_block=64)


@pytest.mark.parametrize("bs,density,junk", [(16, 0.2, False), (64, 0.1, True), (128, 0.5, False), (1, 0.05, True)])
def test_table_holds_the_listed_positions_in_order(bs, density, junk):
    hb = make_host_batch(BF, 1)
    lay = hb.layout
    indptr, idx = mask_with_edges(lay, bs, density, 2, empty=(3,), junk=junk)
    _, _, (srtt, slens, _) = run_sparse(hb, indptr, idx, bs)
    for b in range(BF.batch):
        pos = listed_positions(lay.seq_lens[b], idx[indptr[b]:indptr[b + 1]].tolist(), bs)
        assert slens[b] == len(pos)
        assert np.array_equal(srtt[b, :len(pos)], lay.req_to_token[b, pos])


@pytest.mark.parametrize("spec,bs,density", [
    (BF, 64, 0.1), (BF, 16, 0.3),
    (Spec("bs_mha", "decode", 4, 8, 8, 128, 16, (0, 1500), 1), 64, 0.25),
    (Spec("bs_d64", "decode", 5, 16, 2, 64, 1, (0, 900), 1), 32, 0.2),
    (Spec("bs_g1p64", "decode", 3, 40, 40, 128, 64, (100, 3000), 1), 128, 0.125),
])
def test_bf16_matches_block_sparse_oracle(spec, bs, density):
    hb = make_host_batch(spec, 3)
    indptr, idx = mask_with_edges(hb.layout, bs, density, 4, empty=(1,), junk=True)
    o, lse, _ = run_sparse(hb, indptr, idx, bs)
    ro, rlse = oracle_sparse(hb, indptr, idx, bs)
    assert_bf16_close(o, ro, f"block-sparse {spec.name} bs={bs}")
    assert_lse_close(lse, rlse, f"block-sparse {spec.name}")


def test_every_block_listed_is_bit_identical_to_dense_decode():
    """All blocks in order: the compacted table is the page table itself, so
    the decode must return exactly the dense result."""
    from test_gpu_decode import run_decode
    hb = make_host_batch(BF, 5)
    lay = hb.layout
    bs = 32
    indptr = np.zeros(BF.batch + 1, np.int32)
    idx = []
    for b in range(BF.batch):
        idx.extend(range(-(-int(lay.seq_lens[b]) // bs)))
        indptr[b + 1] = len(idx)
    o, lse, _ = run_sparse(hb, indptr, np.asarray(idx, np.int32), bs)
    o2, lse2, _, _ = run_decode(hb)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_req_pool_indices_rows():
    hb = make_host_batch(BF, 6)
    lay = hb.layout
    bs = 64
    indptr, idx = mask_with_edges(lay, bs, 0.2, 7)
    rpi = np.random.default_rng(8).permutation(BF.batch + 3)[:BF.batch].astype(np.int32)
    rows = np.full((BF.batch + 3, lay.req_to_token.shape[1]), -1, np.int32)
    rows[rpi] = lay.req_to_token
    o, lse, _ = run_sparse(hb, indptr, idx, bs, rpi=rpi, rtt_rows=rows)
    ro, rlse = oracle_sparse(hb, indptr, idx, bs)
    assert_bf16_close(o, ro, "block-sparse rpi")
    assert_lse_close(lse, rlse)


@pytest.mark.parametrize("bs,density", [(64, 0.1), (128, 0.3), (256, 0.5)])
def test_int8_matches_block_sparse_sage_oracle(bs, density):
    """INT8 Q/K codes (the Sage page's code §3) on the compacted table."""
    spec = Spec("bs_i8", "decode", 6, 32, 8, 128, 16, (0, 2000), 1, dtype="int8", k_block=64)
    hb = make_host_batch(spec, 12)
    indptr, idx = mask_with_edges(hb.layout, bs, density, 13, empty=(4,), junk=True)
    vm = np.random.default_rng(14).standard_normal((spec.batch, spec.num_kv_heads, 128)).astype(np.float32)
    o, lse, _ = run_sparse(hb, indptr, idx, bs, v_mean=vm)
    ro, rlse = oracle_sparse(hb, indptr, idx, bs, v_mean=vm)
    assert np.all(np.isfinite(o))
    check_rel_l2(o, ro, "block-sparse 8-bit")
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - rlse[fin]).max() <= 1e-3


@pytest.mark.parametrize("bs,density", [(64, 0.1), (128, 0.3), (256, 0.5)])
def test_fp8_matches_block_sparse_sage_oracle(bs, density):
    hb = make_host_batch(F8, 9)
    lay = hb.layout
    indptr, idx = mask_with_edges(lay, bs, density, 10, empty=(2,), junk=True)
    vm = np.random.default_rng(11).standard_normal((F8.batch, F8.num_kv_heads, F8.head_dim)).astype(np.float32)
    o, lse, (_, slens, ssfk) = run_sparse(hb, indptr, idx, bs, v_mean=vm)
    ro, rlse = oracle_sparse(hb, indptr, idx, bs, v_mean=vm)
    assert np.all(np.isfinite(o))
    check_rel_l2(o, ro, "block-sparse 8-bit")
    np.testing.assert_array_equal(o[2], np.asarray(round_bf16(np.repeat(vm[2], F8.num_q_heads // F8.num_kv_heads,
                                                                          axis=0)), np.float64))
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - rlse[fin]).max() <= 1e-3
    # the sfK of each virtual k_block is that of its logical k_block
    kb = F8.k_block
    for b in range(F8.batch):
        pos = listed_positions(lay.seq_lens[b], idx[indptr[b]:indptr[b + 1]].tolist(), bs)
        for u in range(-(-len(pos) // kb)):
            np.testing.assert_array_equal(ssfk[b, :, u], hb.sfk[b, :, pos[u * kb] // kb])


def _full_size(name):
    torch = torch_mod()
    pkv = _pkv()
    spec = SPECS[name]
    fp8 = spec.dtype == "fp8"
    db = make_device_batch(spec, seed=0, layers=1)
    lay = db.layout
    kw = dict(kv_dtype=pkv.PKV_FP8_E4M3, q_block=spec.q_block, k_block=spec.k_block) if fp8 else {}
    params = pkv.Params(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                        max_kv_len=lay.req_to_token.shape[1], **kw)
    pkv.kv_store(params, db.k_pools[0], db.v_pools[0], db.k_new[0], db.v_new[0], db.new_slots)
    srtt, slens, ssfk = pkv.block_sparse_table(params, db.seq_lens, db.req_to_token, db.blk_indptr, db.blk_indices,
                                               spec.sparse_block, sfk=db.sfk)
    plan = pkv.plan_metadata(params, pkv.PKV_DECODE, slens)
    lse = torch.empty((spec.batch, spec.num_q_heads), dtype=torch.float32, device="cuda")
    extra = dict(sfq=db.sfq, sfk=ssfk, sfv=db.sfv) if fp8 else {}
    out = pkv.attn_decode(params, db.q, db.k_pools[0], db.v_pools[0], srtt, slens, plan, lse=lse, **extra)
    torch.cuda.synchronize()
    ro, rl = full_size.block_sparse_reference(db, sage=fp8, qk_codes="e4m3")
    if fp8:
        check_rel_l2(host(out), ro, f"{name} every element of {ro.shape}")
        assert np.abs(lse.cpu().numpy() - rl).max() <= 1e-3
    else:
        err, rel = assert_bf16_close(host(out), ro, name)
        assert_lse_close(lse.cpu().numpy(), rl, name)
        print(f"{name}: every element of {ro.shape}: max abs {err:.3e}, rel L2 {rel:.3e}", flush=True)


def test_full_size_sparse_decode_bf16_every_element():
    """The 8-request, 40-head, S in [15360, 75600], density 0.10 workload in the
    bench's launch configuration; every head of every request against the
    oracle over the request's listed keys."""
    _full_size("sparse_decode_bf16")


def test_full_size_sparse_decode_fp8_every_element():
    _full_size("sparse_decode_fp8")
