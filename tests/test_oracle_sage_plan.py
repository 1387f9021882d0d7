"""Pins of the 8-bit (Sage) oracle, the scheduling re-derivation, the KV store
and the score-memory helper."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import Spec, make_host_batch, make_layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FP8 = Spec("f8", "decode", 3, 4, 2, 32, 4, (3, 70), 1, dtype="fp8", k_block=16)


def _sage(hb, **kw):
    lay = hb.layout
    return oracle.sage_decode(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, lay.seq_lens,
                              hb.sfq, hb.sfk, hb.sfv, hb.layout.spec.k_block, **kw)


def test_sage_unit_scales_unquantised_p_reduce_to_plain_attention():
    hb = make_host_batch(FP8, 0)
    lay = hb.layout
    hb.sfq[:] = 1.0
    hb.sfk[:] = 1.0
    hb.sfv[:] = 1.0
    o, lse = _sage(hb, quantize_p=False)
    q = oracle.e4m3_decode(hb.q_codes)
    k = oracle.e4m3_decode(hb.k_codes)
    v = oracle.e4m3_decode(hb.v_codes)
    o2, lse2 = oracle.paged_attention(q, k, v, lay.req_to_token, lay.seq_lens, lay.cu_seqlens_q)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-12)


def test_sage_scales_enter_before_softmax():
    """sfQ·sfK multiply the scores: folding them into sm_scale per request is the same."""
    hb = make_host_batch(FP8, 1)
    hb.sfk[:] = 1.25
    hb.sfq[:] = 0.5
    o, lse = _sage(hb)
    hb.sfk[:] = 1.0
    hb.sfq[:] = 1.0
    o2, lse2 = _sage(hb, sm_scale=0.625 / math.sqrt(FP8.head_dim))
    np.testing.assert_allclose(o, o2, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-14, atol=1e-14)


def test_sage_constant_scores_give_scaled_mean():
    hb = make_host_batch(FP8, 2)
    lay = hb.layout
    hb.q_codes[:] = 0  # q = 0: every score is 0, p = 1, P8 = 448 exactly
    o, lse = _sage(hb)
    G = FP8.num_q_heads // FP8.num_kv_heads
    for b in range(FP8.batch):
        L = int(lay.seq_lens[b])
        V = oracle.e4m3_decode(hb.v_codes[lay.req_to_token[b, :L]])
        for h in range(FP8.num_q_heads):
            g = h // G
            np.testing.assert_allclose(o[b, h], hb.sfv[b, g] * V[:, g].mean(axis=0), rtol=1e-14, atol=1e-14)
            assert abs(lse[b, h] - math.log(L)) < 1e-13


def test_sage_power_of_two_sfv_is_exact():
    hb = make_host_batch(FP8, 3)
    o1, _ = _sage(hb)
    hb.sfv *= 4.0
    o2, _ = _sage(hb)
    assert np.array_equal(o2, 4.0 * o1)


def test_sage_two_key_hand_example():
    with open(os.path.join(GOLDEN, "sage_two_keys.json")) as f:
        g = json.load(f)
    q8 = oracle.e4m3_encode(np.array(g["q"]))[None, None, :]
    k8 = oracle.e4m3_encode(np.array(g["k"]))[:, None, :]
    v8 = oracle.e4m3_encode(np.array(g["v"]))[:, None, :]
    assert np.array_equal(oracle.e4m3_decode(k8)[:, 0], np.array(g["k"]))
    rtt = np.array([[0, 1]])
    sfv = np.array(g["sfv"])[None, None, :]
    o, lse = oracle.sage_decode(q8, k8, v8, rtt, [2], np.ones((1, 1)), np.ones((1, 1, 1)), sfv,
                                k_block=64, sm_scale=math.log(2))
    np.testing.assert_allclose(o[0, 0], g["expected_o"], rtol=1e-15, atol=1e-15)
    assert abs(lse[0, 0] - math.log(1.5)) < 1e-15


def test_sage_p_quantisation_changes_little():
    hb = make_host_batch(FP8, 4)
    o_q, _ = _sage(hb)
    o_f, _ = _sage(hb, quantize_p=False)
    rel = np.linalg.norm(o_q - o_f) / np.linalg.norm(o_f)
    assert 0 < rel < 5e-2


# ---------------------------------------------------------------- plan
@pytest.mark.parametrize("kv_chunk,tile", [(0, 32), (0, 64), (32, 32), (96, 32)])
@pytest.mark.parametrize("seed", range(4))
def test_decode_plan_invariants(seed, kv_chunk, tile):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    max_kv = int(rng.integers(1, 5000))
    L = rng.integers(0, max_kv + 1, size=B)
    L[rng.integers(0, B)] = max_kv + 77  # beyond the bound: must be clamped
    Hkv, G = 8, int(rng.choice([1, 4, 8, 20]))
    target = oracle.decode_target_items(Hkv, G, int(rng.integers(1, 9000)), 512)
    plan = oracle.plan_decode(L, max_kv, target, kv_chunk=kv_chunk, tile=tile)
    items = plan["items"]
    assert len(items) <= plan["capacity"]
    Lc = np.minimum(L, max_kv)
    tiles = -(-Lc // tile)
    parts = []
    lengths = items[:, 2] - items[:, 1]
    tab = plan["chunk_tab"]
    assert tab[0] == 0 and tab[-1] == len(items) and np.all(np.diff(tab) >= 1)
    assert len(tab) == plan["nchunks"] + 1
    if kv_chunk and len(items) > target:
        assert np.all(np.diff(lengths) <= 0)  # longest split first
    else:
        assert list(items[:, 0]) == sorted(items[:, 0])  # request order
    if not kv_chunk:
        # balanced chunks: every chunk but the last holds exactly C tiles, the
        # last at most C; C is the smallest size giving <= target chunks
        c, T = plan["chunk_tiles"], int(tiles.sum())
        seg_tiles = -(-lengths // tile)
        per_chunk = [int(seg_tiles[tab[k]:tab[k + 1]].sum()) for k in range(plan["nchunks"])]
        assert sum(per_chunk) == T
        if T:
            assert all(x == c for x in per_chunk[:-1]) and 1 <= per_chunk[-1] <= c
        assert plan["nchunks"] <= target
        if c > 1:
            assert -(-T // (c - 1)) > target
        # a request crosses chunks only at chunk boundaries (global tile offsets)
        starts = np.concatenate([[0], np.cumsum(tiles)])
        for k in range(plan["nchunks"]):
            for i in range(tab[k], tab[k + 1]):
                g0 = starts[items[i, 0]] + items[i, 1] // tile
                if seg_tiles[i]:
                    assert k * c <= g0 and g0 + seg_tiles[i] <= (k + 1) * c
    for b in range(B):
        mine = items[items[:, 0] == b]
        mine = mine[np.argsort(mine[:, 1], kind="stable")]
        assert len(mine) == plan["splits"][b] >= 1
        assert mine[0, 1] == 0 and mine[-1, 2] == Lc[b]
        assert np.all(mine[1:, 1] == mine[:-1, 2])  # contiguous, in order
        assert np.all(mine[:, 1] % tile == 0)
        if Lc[b] > 0:
            assert np.all(mine[:, 2] > mine[:, 1])  # no empty split
        if len(mine) == 1:
            assert mine[0, 3] == -1
        else:
            assert list(mine[:, 3]) == list(range(plan["split_off"][b], plan["split_off"][b + 1]))
            parts += list(mine[:, 3])
        if kv_chunk:
            assert np.all(mine[:, 2] - mine[:, 1] <= kv_chunk)
    assert sorted(parts) == sorted(set(parts))


@pytest.mark.parametrize("seed", range(4))
def test_extend_plan_invariants(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 20))
    n = rng.integers(0, 300, size=B)
    p = rng.integers(0, 300, size=B)
    L = n + p
    cu = np.concatenate([[0], np.cumsum(n)])
    G = int(rng.choice([1, 2, 4, 8, 3]))
    plan = oracle.plan_extend(L, cu, G, int(L.max()) if B else 1, int(cu[-1]))
    bt = plan["block_tokens"]
    items = plan["items"]
    assert len(items) <= plan["capacity"]
    assert np.all(np.diff(items[:, 2]) <= 0)  # longest causal range first
    for b in range(B):
        mine = sorted(items[items[:, 0] == b][:, 1])
        assert mine == list(range(-(-int(n[b]) // bt)))
        for it in items[items[:, 0] == b]:
            assert it[2] == p[b] + min((it[1] + 1) * bt, n[b])


def test_kv_store_round_trip():
    lay, rng = make_layout(Spec("k", "extend", 3, 2, 2, 8, 4, (0, 9), (1, 5)), 0)
    pool = rng.standard_normal((lay.pool_slots, 2, 8))
    new = rng.standard_normal((lay.total_q, 2, 8))
    out = oracle.kv_store(pool, new, lay.new_slots)
    assert np.array_equal(out[lay.new_slots], new)
    untouched = np.setdiff1d(np.arange(lay.pool_slots), lay.new_slots)
    assert np.array_equal(out[untouched], pool[untouched])


def test_score_memory_figures_from_the_flashattention_page():
    with open(os.path.join(GOLDEN, "fa_memory.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        got = oracle.score_matrix_bytes(c["seq_len"], c["elem_bytes"], c["heads"], c["batch"])
        assert got == c["approx_bytes"]


# ---------------------------------------------------------------- 8-bit extend
FP8_EXT = Spec("f8_ext", "extend", 3, 8, 2, 64, 4, (0, 40), (1, 9), dtype="fp8", k_block=16)


def _sage_ext(hb, **kw):
    lay = hb.layout
    return oracle.sage_extend(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, lay.seq_lens,
                              lay.cu_seqlens_q, hb.sfq, hb.sfk, hb.sfv, FP8_EXT.k_block, **kw)


def test_sage_extend_rows_equal_sage_decode_on_the_causal_prefix():
    """Row i of request b is the decode formula over keys 0..p_b+i with that row's sfQ."""
    hb = make_host_batch(FP8_EXT, 0)
    lay = hb.layout
    o, lse = _sage_ext(hb)
    for b in range(FP8_EXT.batch):
        q0, q1 = int(lay.cu_seqlens_q[b]), int(lay.cu_seqlens_q[b + 1])
        p0 = int(lay.seq_lens[b]) - (q1 - q0)
        for t in range(q0, q1):
            od, ld = oracle.sage_decode(hb.q_codes[t:t + 1], hb.k_codes, hb.v_codes, lay.req_to_token[b:b + 1],
                                        [p0 + t - q0 + 1], hb.sfq[t:t + 1], hb.sfk[b:b + 1], hb.sfv[b:b + 1],
                                        FP8_EXT.k_block)
            assert np.array_equal(o[t], od[0]) and np.array_equal(lse[t], ld[0])


def test_sage_extend_unit_scales_unquantised_p_is_plain_causal_attention():
    hb = make_host_batch(FP8_EXT, 1)
    lay = hb.layout
    hb.sfq[:] = 1.0
    hb.sfk[:] = 1.0
    hb.sfv[:] = 1.0
    o, lse = _sage_ext(hb, quantize_p=False)
    q = oracle.e4m3_decode(hb.q_codes)
    k = oracle.e4m3_decode(hb.k_codes)
    v = oracle.e4m3_decode(hb.v_codes)
    ro, rlse = oracle.paged_attention(q, k, v, lay.req_to_token, lay.seq_lens, lay.cu_seqlens_q)
    assert np.abs(o - ro).max() <= 1e-12 and np.abs(lse - rlse).max() <= 1e-12


def test_sage_extend_zero_queries_give_mean_over_visible_keys():
    """q8 = 0: every visible key gets p = 1, P8 = 448 exactly, so O = sfV * mean(V8)
    over keys 0..p_b+i, a different mean for every row."""
    hb = make_host_batch(FP8_EXT, 2)
    lay = hb.layout
    hb.q_codes[:] = 0
    o, lse = _sage_ext(hb)
    v = oracle.e4m3_decode(hb.v_codes)
    G = FP8_EXT.num_q_heads // FP8_EXT.num_kv_heads
    for b in range(FP8_EXT.batch):
        q0, q1 = int(lay.cu_seqlens_q[b]), int(lay.cu_seqlens_q[b + 1])
        p0 = int(lay.seq_lens[b]) - (q1 - q0)
        for t in range(q0, q1):
            vis = p0 + t - q0 + 1
            slots = lay.req_to_token[b, :vis]
            for h in range(FP8_EXT.num_q_heads):
                want = hb.sfv[b, h // G] * v[slots, h // G].mean(axis=0)
                np.testing.assert_allclose(o[t, h], want, rtol=1e-12, atol=1e-12)
                assert abs(lse[t, h] - math.log(vis)) <= 1e-12
