"""GPU parity of the bf16 split-KV decode (plan + kv_store + attn_decode) against
the fp64 oracle, through the C ABI via the ctypes binding."""
import math

import numpy as np
import pytest

import full_size
import oracle
from gpu_util import (assert_bf16_close, assert_lse_close, dev_bf16, dev_i32, host, torch_mod)
from workloads import SPECS, Spec, make_device_batch, make_host_batch, permute_pages, pool_before_store, round_bf16

pytestmark = pytest.mark.gpu


def _pkv():
    import flashattention_paged_kv_amd as pkv
    return pkv


def run_decode(hb, kv_chunk=0, split_target=0, sm_scale=None, req_pool_indices=None, max_kv_len=None,
               seq_lens_override=None, lse=True, decode_q_len=0):
    """Upload a host batch (new rows poisoned), plan, store, decode; return host (o, lse, plan)."""
    torch = torch_mod()
    pkv = _pkv()
    lay = hb.layout
    spec = lay.spec
    q = round_bf16(hb.q)
    kp = pool_before_store(round_bf16(hb.k_pool), lay.new_slots)
    vp = pool_before_store(round_bf16(hb.v_pool), lay.new_slots)
    k_pool, v_pool = dev_bf16(kp), dev_bf16(vp)
    k_new, v_new = dev_bf16(round_bf16(hb.k_new)), dev_bf16(round_bf16(hb.v_new))
    seq = lay.seq_lens if seq_lens_override is None else seq_lens_override
    params = pkv.Params(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                        max_kv_len=max_kv_len or max(lay.req_to_token.shape[1], 1),
                        kv_chunk=kv_chunk, split_target=split_target, decode_q_len=decode_q_len)
    seq_d = dev_i32(seq)
    rtt = dev_i32(lay.req_to_token)
    plan = pkv.plan_metadata(params, pkv.PKV_DECODE, seq_d)
    pkv.kv_store(params, k_pool, v_pool, k_new, v_new, dev_i32(lay.new_slots))
    lse_t = torch.empty((lay.total_q, spec.num_q_heads), dtype=torch.float32, device="cuda") if lse else None
    rpi = None if req_pool_indices is None else dev_i32(req_pool_indices)
    out = pkv.attn_decode(params, dev_bf16(q), k_pool, v_pool, rtt, seq_d, plan, sm_scale=sm_scale,
                          lse=lse_t, req_pool_indices=rpi)
    torch.cuda.synchronize()
    return host(out), (lse_t.cpu().numpy().astype(np.float64) if lse else None), plan, (k_pool, v_pool)


def oracle_decode(hb, sm_scale=None, seq=None):
    lay = hb.layout
    seq = lay.seq_lens if seq is None else seq
    return oracle.paged_attention(round_bf16(hb.q), round_bf16(hb.k_pool), round_bf16(hb.v_pool),
                                  lay.req_to_token, seq, lay.cu_seqlens_q, sm_scale=sm_scale)


MEDIUM = Spec("dec_med", "decode", 8, 32, 8, 128, 16, (0, 1500), 1)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_decode_config(seed):
    hb = make_host_batch(SPECS["tiny_decode"], seed)
    o, lse, _, _ = run_decode(hb)
    ro, rlse = oracle_decode(hb)
    assert_bf16_close(o, ro, "tiny decode")
    assert_lse_close(lse, rlse, "tiny decode")


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("kv_chunk", [0, 32, 256])
def test_medium_decode_ragged(seed, kv_chunk):
    hb = make_host_batch(MEDIUM, seed)
    o, lse, _, _ = run_decode(hb, kv_chunk=kv_chunk)
    ro, rlse = oracle_decode(hb)
    assert_bf16_close(o, ro, f"medium decode chunk={kv_chunk}")
    assert_lse_close(lse, rlse, "medium decode")


# (24, 24, 64) and (48, 24, 128) have 24 (kv head, head group) units per
# token: the kernel instances with plain (not non-temporal) K/V loads
@pytest.mark.parametrize("hq,hkv,d,page", [(8, 8, 128, 1), (64, 8, 128, 64), (40, 2, 128, 16),
                                           (16, 4, 64, 16), (12, 4, 64, 2), (32, 8, 64, 256),
                                           (24, 24, 64, 16), (48, 24, 128, 16)])
def test_head_layouts_and_pages(hq, hkv, d, page):
    spec = Spec("dec_shape", "decode", 5, hq, hkv, d, page, (0, 700), 1)
    hb = make_host_batch(spec, 3)
    o, lse, _, _ = run_decode(hb, split_target=64)
    ro, rlse = oracle_decode(hb)
    assert_bf16_close(o, ro, f"decode hq={hq} hkv={hkv} d={d} P={page}")
    assert_lse_close(lse, rlse)


def test_custom_scale_and_request_row_indirection():
    hb = make_host_batch(MEDIUM, 4)
    lay = hb.layout
    B = MEDIUM.batch
    perm = np.random.default_rng(0).permutation(B)
    # rows of req_to_token are stored permuted; req_pool_indices maps request b -> its row
    rtt_perm = np.empty_like(lay.req_to_token)
    rtt_perm[perm] = lay.req_to_token
    lay.req_to_token = rtt_perm
    o, lse, _, _ = run_decode(hb, sm_scale=0.05, req_pool_indices=perm)
    lay.req_to_token = rtt_perm[perm]
    ro, rlse = oracle_decode(hb, sm_scale=0.05)
    assert_bf16_close(o, ro, "scale + indirection")
    assert_lse_close(lse, rlse)


def test_forced_split_equals_unsplit_and_runs_are_deterministic():
    hb = make_host_batch(MEDIUM, 5)
    o1, l1, _, _ = run_decode(hb, kv_chunk=32)
    o2, l2, _, _ = run_decode(hb, kv_chunk=32)
    o3, l3, _, _ = run_decode(hb, kv_chunk=4096)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.abs(o1 - o3).max() <= 2e-2
    assert np.abs(l1 - l3).max() <= 1e-4


def test_page_relabelling_is_bit_invariant_on_gpu():
    hb = make_host_batch(MEDIUM, 6)
    o1, l1, _, _ = run_decode(hb)
    lay2, slot_map = permute_pages(hb.layout, np.random.default_rng(1))
    k2 = np.full_like(hb.k_pool, np.nan)
    v2 = np.full_like(hb.v_pool, np.nan)
    k2[slot_map] = hb.k_pool
    v2[slot_map] = hb.v_pool
    hb.layout, hb.k_pool, hb.v_pool = lay2, k2, v2
    o2, l2, _, _ = run_decode(hb)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_one_hot_key_returns_the_value_row_bit_exactly():
    """Indexing probe: one key aligned with q, the rest zero, so every other weight
    underflows in fp32 and O must equal that V row exactly."""
    spec = Spec("onehot", "decode", 4, 8, 2, 128, 16, (40, 300), 1)
    hb = make_host_batch(spec, 7)
    lay = hb.layout
    G = 4
    rng = np.random.default_rng(3)
    targets = []
    for b in range(spec.batch):
        L = int(lay.seq_lens[b])
        slots = lay.req_to_token[b, :L]
        hb.k_pool[slots] = 0.0
        t = int(rng.integers(0, L))
        targets.append(slots[t])
        for g in range(2):
            qh = hb.q[b, g * G]
            hb.q[b, g * G:(g + 1) * G] = qh  # all heads of the group share q
            hb.k_pool[slots[t], g] = qh * (400.0 / float(np.dot(qh, qh)))  # score 400*sm_scale
    hb.q = round_bf16(hb.q)
    hb.k_pool = round_bf16(hb.k_pool)
    hb.v_pool = round_bf16(hb.v_pool)
    hb.k_new = hb.k_pool[lay.new_slots].copy()
    o, _, _, _ = run_decode(hb, sm_scale=1.0, kv_chunk=64)
    for b in range(spec.batch):
        for h in range(spec.num_q_heads):
            want = round_bf16(hb.v_pool[targets[b], h // G])
            assert np.array_equal(o[b, h], want), (b, h)


def test_zero_length_request_gives_zero_and_minus_inf():
    hb = make_host_batch(MEDIUM, 8)
    seq = hb.layout.seq_lens.copy()
    seq[3] = 0
    o, lse, _, _ = run_decode(hb, seq_lens_override=seq, kv_chunk=64)
    assert np.all(o[3] == 0) and np.all(np.isneginf(lse[3]))
    ro, rlse = oracle_decode(hb, seq=seq)
    assert_bf16_close(o, ro, "zero-length row")


def test_chunks_of_more_than_64_segments():
    """Few, long chunks over many short requests: each chunk holds ~100 request
    segments, so the kernels' per-wave segment records are reloaded mid-stream,
    and every seventh request is empty."""
    spec = Spec("manyseg", "decode", 300, 8, 2, 128, 16, (0, 60), 1)
    hb = make_host_batch(spec, 21)
    seq = hb.layout.seq_lens.copy()
    seq[::7] = 0
    # units = 2 (two kv heads, one 16-head group each): 3 chunks
    o, lse, plan, _ = run_decode(hb, split_target=6, seq_lens_override=seq)
    ws = plan.workspace.cpu().numpy().view(np.int32)
    assert ws[6] == 3 and ws[2] > 3 * 64
    ro, rlse = oracle_decode(hb, seq=seq)
    assert_bf16_close(o, ro, "many segments per chunk")
    assert_lse_close(lse, rlse)
    assert np.all(o[::7] == 0) and np.all(np.isneginf(lse[::7]))


def test_long_run_of_empty_requests():
    """150 consecutive empty requests share one global tile offset, so they all
    land in one chunk (with the segments around them)."""
    lens = [3000, 2500, 40] + [0] * 150 + [1800, 33, 700]
    spec = Spec("empties", "decode", len(lens), 32, 8, 128, 16, [max(x - 1, 0) for x in lens], 1)
    hb = make_host_batch(spec, 22)
    seq = np.asarray(lens, dtype=np.int32)
    o, lse, _, _ = run_decode(hb, seq_lens_override=seq)
    ro, rlse = oracle_decode(hb, seq=seq)
    assert_bf16_close(o, ro, "empty run")
    assert_lse_close(lse, rlse)
    assert np.all(o[3:153] == 0) and np.all(np.isneginf(lse[3:153]))


def test_shared_prefix_pages():
    """Requests whose page-table rows point at one request's prefix pages (a
    prefix shared by copy-on-write, as the PagedAttention page describes
    for block sharing): the kernels follow the table, whatever slots repeat."""
    spec = Spec("sharedpfx", "decode", 12, 32, 8, 128, 16, (300, 1500), 1)
    hb = make_host_batch(spec, 24)
    lay = hb.layout
    shared = (int(lay.prefix_lens.min()) // 16) * 16
    lay.req_to_token[1:, :shared] = lay.req_to_token[0, :shared]
    o, lse, _, _ = run_decode(hb)
    ro, rlse = oracle_decode(hb)
    assert_bf16_close(o, ro, "shared prefix")
    assert_lse_close(lse, rlse)


@pytest.mark.parametrize("n,hq,hkv,kv_chunk", [(2, 32, 8, 0), (4, 32, 8, 0), (4, 32, 8, 64), (3, 8, 8, 0),
                                              (8, 16, 2, 0), (5, 64, 8, 0), (16, 8, 8, 96)])
def test_several_new_tokens_per_request(n, hq, hkv, kv_chunk):
    """n new tokens per request in one decode call (a verify step of n drafted
    tokens): token i sees the cached prefix and new tokens 0..i.  Columns of
    the MFMA are (token, head) pairs, n * G of them per kv head."""
    spec = Spec(f"dec_n{n}", "decode", 9, hq, hkv, 128, 16, (0, 900), n)
    hb = make_host_batch(spec, 30 + n)
    o, lse, _, _ = run_decode(hb, decode_q_len=n, kv_chunk=kv_chunk)
    ro, rlse = oracle_decode(hb)
    assert_bf16_close(o, ro, f"n={n}")
    assert_lse_close(lse, rlse)


def _merge_waves(capacity, batch):
    """Waves per merge workgroup the library picks (decode_merge.h)."""
    per = capacity // batch
    return 8 if per >= 64 else (4 if per >= 16 else 1)


@pytest.mark.parametrize("B,lens,hq,hkv,d,n,target,waves", [
    (1, 60000, 16, 2, 128, 1, 512, 8),            # one long request: hundreds of splits
    (1, 20000, 8, 8, 64, 3, 256, 8),              # head_dim 64, three new tokens
    (5, [0, 30000, 2500, 1, 17000], 8, 1, 64, 1, 400, 8),  # one- and two-token requests beside long ones
    (12, (4000, 12000), 32, 8, 128, 1, 256, 4),   # dozens of splits per request
    (12, (4000, 12000), 32, 8, 128, 2, 256, 4),
    (40, (1000, 3000), 32, 8, 128, 1, 256, 1),    # a few splits per request
])
def test_merge_of_many_splits(B, lens, hq, hkv, d, n, target, waves):
    """Requests cut into many splits, so the merge runs its several-wave
    two-pass form (or the one-pass form, last case): against the oracle."""
    spec = Spec(f"merge{B}", "decode", B, hq, hkv, d, 16, lens, n)
    hb = make_host_batch(spec, 70 + B + n)
    units = hkv * -(-(n * (hq // hkv)) // 16)
    o, lse, plan, _ = run_decode(hb, decode_q_len=n, split_target=target * units)
    ws = plan.workspace.cpu().numpy().view(np.int32)
    assert _merge_waves(int(ws[3]), B) == waves, (int(ws[3]), B)
    ro, rlse = oracle_decode(hb)
    assert_bf16_close(o, ro, spec.name)
    assert_lse_close(lse, rlse)


def test_plan_matches_oracle_rederivation_bit_for_bit():
    torch = torch_mod()
    pkv = _pkv()
    rng = np.random.default_rng(11)
    cases = ((0, 0, False), (0, 100, False), (64, 0, False), (0, 50000, False), (0, 0, True), (0, 300, True),
             (96, 0, True))
    # up to 64 requests take the one-wave plan, 150 the workgroup one; the
    # 64-request batch has a run of empty requests; one to three requests
    # have more segments each than the wave has lanes
    modes = set()
    for B, (kv_chunk, target, fp8) in ([(B, c) for B in (37, 150) for c in cases] + [(64, cases[0]), (64, cases[4])] +
                                       [(1, cases[0]), (1, cases[4]), (3, cases[0]), (2, cases[1])]):
        max_kv = 5000
        L = rng.integers(0, max_kv + 1, size=B).astype(np.int32)
        L[min(5, B - 1)] = max_kv + 100  # clamped
        if B == 64:
            L[20:29] = 0
        extra = dict(kv_dtype=pkv.PKV_FP8_E4M3, k_block=64, q_block=1) if fp8 else {}
        params = pkv.Params(32, 8, 128, 16, max_kv_len=max_kv, kv_chunk=kv_chunk, split_target=target, **extra)
        tile = 64 if fp8 else 32
        plan = pkv.plan_metadata(params, pkv.PKV_DECODE, dev_i32(L))
        torch.cuda.synchronize()
        ws = plan.workspace.cpu().numpy().view(np.int32)
        if target:
            assert ws[5] == oracle.decode_target_items(8, 4, target, 0)
        else:
            assert 1 <= ws[5]  # the device's resident items
        ref = oracle.plan_decode(L, max_kv, int(ws[5]), kv_chunk=kv_chunk, tile=tile)
        n = ws[2]
        items_off = -(-(16 + B + 1) // 4) * 4
        items = ws[items_off:items_off + 4 * n].reshape(-1, 4)
        assert n == len(ref["items"]) and ws[3] == ref["capacity"] and ws[4] == ref["chunk_tiles"]
        assert np.array_equal(items, ref["items"])
        assert np.array_equal(ws[16:16 + B + 1], ref["split_off"])
        assert ws[6] == ref["nchunks"]
        if B <= 64 and not kv_chunk:  # the one-wave plan: per-lane or spread segment writing
            modes.add(int(np.diff(ref["split_off"]).max()) > 8)
        if kv_chunk:
            assert ws[7] == 0  # identity: one split per chunk
        else:
            assert np.array_equal(ws[ws[7]:ws[7] + ws[6] + 1], ref["chunk_tab"])
    assert modes == {False, True}  # both ways of writing the segments ran


@pytest.mark.parametrize("hkv,d", [(4, 128), (40, 128), (2, 64), (1, 64)])
def test_kv_store_round_trip_bit_exact(hkv, d):
    torch = torch_mod()
    pkv = _pkv()
    spec = Spec("st", "extend", 6, 2 * hkv, hkv, d, 16, (0, 100), (1, 40))
    hb = make_host_batch(spec, 9)
    lay = hb.layout
    params = pkv.Params(2 * hkv, hkv, d, 16, max_kv_len=lay.max_kv_len)
    kp = dev_bf16(pool_before_store(hb.k_pool, lay.new_slots, fill=7.0))
    vp = dev_bf16(pool_before_store(hb.v_pool, lay.new_slots, fill=7.0))
    before_k = kp.clone()
    pkv.kv_store(params, kp, vp, dev_bf16(hb.k_new), dev_bf16(hb.v_new), dev_i32(lay.new_slots))
    torch.cuda.synchronize()
    k = host(kp)
    v = host(vp)
    assert np.array_equal(k[lay.new_slots], hb.k_new) and np.array_equal(v[lay.new_slots], hb.v_new)
    untouched = np.setdiff1d(np.arange(lay.pool_slots), lay.new_slots)
    idx = dev_i32(untouched).long()
    # compare bit patterns: the untouched rows include NaN poison
    assert torch.equal(kp[idx].view(torch.int16), before_k[idx].view(torch.int16))


def test_kv_store_skips_slots_outside_the_pool():
    torch = torch_mod()
    pkv = _pkv()
    spec = Spec("st2", "extend", 4, 8, 4, 128, 16, (0, 50), (2, 20))
    hb = make_host_batch(spec, 10)
    lay = hb.layout
    params = pkv.Params(8, 4, 128, 16, max_kv_len=lay.max_kv_len)
    kp = dev_bf16(pool_before_store(hb.k_pool, lay.new_slots, fill=7.0))
    vp = dev_bf16(pool_before_store(hb.v_pool, lay.new_slots, fill=7.0))
    slots = lay.new_slots.copy()
    bad = [0, 3, len(slots) - 1]
    slots[bad[0]], slots[bad[1]], slots[bad[2]] = -1, lay.pool_slots, lay.pool_slots + 1000
    pkv.kv_store(params, kp, vp, dev_bf16(hb.k_new), dev_bf16(hb.v_new), dev_i32(slots))
    torch.cuda.synchronize()
    k, v = host(kp), host(vp)
    good = np.setdiff1d(np.arange(len(slots)), bad)
    assert np.array_equal(k[slots[good]], hb.k_new[good]) and np.array_equal(v[slots[good]], hb.v_new[good])
    assert np.all(k[lay.new_slots[bad]] == 7.0) and np.all(v[lay.new_slots[bad]] == 7.0)


def _full_size(name):
    """Full-size workload on the device in the bench's launch configuration;
    every output element and lse is compared with the oracle, run request by
    request on host copies of the rows each request references."""
    torch = torch_mod()
    pkv = _pkv()
    spec = SPECS[name]
    n = int(spec.new) if spec.mode == "decode" else 1
    db = make_device_batch(spec, seed=0, layers=1)
    lay = db.layout
    params = pkv.Params(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                        max_kv_len=lay.req_to_token.shape[1], decode_q_len=n)
    plan = pkv.plan_metadata(params, pkv.PKV_DECODE, db.seq_lens)
    pkv.kv_store(params, db.k_pools[0], db.v_pools[0], db.k_new[0], db.v_new[0], db.new_slots)
    lse = torch.empty((spec.batch * n, spec.num_q_heads), dtype=torch.float32, device="cuda")
    out = pkv.attn_decode(params, db.q, db.k_pools[0], db.v_pools[0], db.req_to_token, db.seq_lens, plan, lse=lse)
    torch.cuda.synchronize()
    ro, rl = full_size.decode_reference(db, q_len=n)
    err, rel = assert_bf16_close(host(out), ro, name)
    assert_lse_close(lse.cpu().numpy(), rl, name)
    print(f"{name}: every element of {ro.shape}: max abs {err:.3e}, rel L2 {rel:.3e}", flush=True)


def test_full_size_decode_bf16_every_element():
    _full_size("decode_bf16")


def test_full_size_long_decode_every_element():
    _full_size("long_decode_bf16")


def test_full_size_single_request_decode_every_element():
    """One 131k-token request: its 256 splits go through the several-wave merge."""
    _full_size("single_decode_bf16")


def test_full_size_decode_n4_every_element():
    """Four new tokens per request checked in one call, at the full batch."""
    _full_size("decode_n4_bf16")


def test_binding_rejects_wrong_output_shapes_before_any_launch():
    """out sized for one token per request when each request checks two, lse
    of [B] instead of [B, Hq], and a page table with fewer rows than requests:
    each raises ValueError in the binding, before the library is called."""
    torch = torch_mod()
    pkv = _pkv()
    spec = Spec("shapes", "decode", 3, 8, 2, 128, 16, (10, 40), 2)
    hb = make_host_batch(spec, 90)
    lay = hb.layout
    params = pkv.Params(8, 2, 128, 16, max_kv_len=lay.req_to_token.shape[1], decode_q_len=2)
    seq = dev_i32(lay.seq_lens)
    plan = pkv.plan_metadata(params, pkv.PKV_DECODE, seq)
    k_pool, v_pool = dev_bf16(round_bf16(hb.k_pool)), dev_bf16(round_bf16(hb.v_pool))
    q, rtt = dev_bf16(round_bf16(hb.q)), dev_i32(lay.req_to_token)
    bad = [dict(out=torch.empty((3, 8, 128), dtype=torch.bfloat16, device="cuda")),
           dict(lse=torch.empty((3,), dtype=torch.float32, device="cuda"))]
    for kw in bad:
        with pytest.raises(ValueError):
            pkv.attn_decode(params, q, k_pool, v_pool, rtt, seq, plan, **kw)
    with pytest.raises(ValueError):
        pkv.attn_decode(params, q, k_pool, v_pool, rtt[:2], seq, plan)
    torch.cuda.synchronize()
