"""Pins of the fp64 paged-attention oracle against things other than itself.

* a library special case: torch's scaled_dot_product_attention (fp64, CPU,
  explicit boolean causal mask) on the gathered contiguous K/V;
* closed forms (Q = 0 gives the mean of the visible V rows and lse = ln n;
  a single non-zero key gives a two-valued softmax);
* invariants (page relabelling, GQA == MHA with repeated kv heads, linearity
  in V, independence of future keys and of other requests, rows of P
  summing to one, decode == last row of extend).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import Spec, make_host_batch, make_layout, permute_pages

SMALL_EXTEND = Spec("t_ext", "extend", 3, 4, 2, 16, 4, (0, 20), (1, 9), dtype="fp32")
SMALL_DECODE = Spec("t_dec", "decode", 4, 6, 2, 16, 4, (0, 30), 1, dtype="fp32")


def _run(hb, **kw):
    lay = hb.layout
    return oracle.paged_attention(hb.q, hb.k_pool, hb.v_pool, lay.req_to_token, lay.seq_lens,
                                  lay.cu_seqlens_q, **kw)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("spec", [SMALL_EXTEND, SMALL_DECODE])
def test_matches_torch_sdpa(spec, seed):
    hb = make_host_batch(spec, seed)
    lay = hb.layout
    sm = 0.37
    o, lse = _run(hb, sm_scale=sm)
    G = spec.num_q_heads // spec.num_kv_heads
    for b in range(spec.batch):
        L, n = int(lay.seq_lens[b]), int(lay.new_lens[b])
        q0 = int(lay.cu_seqlens_q[b])
        slots = lay.req_to_token[b, :L]
        K = torch.from_numpy(hb.k_pool[slots].astype(np.float64)).permute(1, 0, 2)  # [Hkv, L, d]
        V = torch.from_numpy(hb.v_pool[slots].astype(np.float64)).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0).contiguous()
        V = V.repeat_interleave(G, dim=0).contiguous()
        Q = torch.from_numpy(hb.q[q0:q0 + n].astype(np.float64)).permute(1, 0, 2).contiguous()
        i = torch.arange(n)[:, None]
        j = torch.arange(L)[None, :]
        mask = j <= (L - n) + i
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=sm)
        np.testing.assert_allclose(o[q0:q0 + n], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
        # lse against a direct log-sum-exp of the visible scores
        S = sm * torch.einsum("hnd,hld->hnl", Q, K)
        S = S.masked_fill(~mask, -math.inf)
        ref_lse = torch.logsumexp(S, dim=-1).permute(1, 0).numpy()
        np.testing.assert_allclose(lse[q0:q0 + n], ref_lse, rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_visible_rows():
    hb = make_host_batch(SMALL_EXTEND, 5)
    hb.q[:] = 0.0
    lay = hb.layout
    o, lse = _run(hb)
    G = SMALL_EXTEND.num_q_heads // SMALL_EXTEND.num_kv_heads
    for b in range(SMALL_EXTEND.batch):
        L, n = int(lay.seq_lens[b]), int(lay.new_lens[b])
        p, q0 = L - n, int(lay.cu_seqlens_q[b])
        for i in range(n):
            vis = lay.req_to_token[b, :p + i + 1]
            for h in range(SMALL_EXTEND.num_q_heads):
                mean = hb.v_pool[vis, h // G].astype(np.float64).mean(axis=0)
                np.testing.assert_allclose(o[q0 + i, h], mean, rtol=1e-13, atol=1e-13)
                assert abs(lse[q0 + i, h] - math.log(p + i + 1)) < 1e-13


def test_single_nonzero_key_closed_form():
    spec = Spec("one", "decode", 1, 2, 1, 8, 1, 11, 1, dtype="fp32", pool=64)
    hb = make_host_batch(spec, 3)
    lay = hb.layout
    L = int(lay.seq_lens[0])
    target = 4
    slots = lay.req_to_token[0, :L]
    hb.k_pool[slots] = 0.0
    hb.k_pool[slots[target], 0] = 2.0 * hb.q[0, 0]  # only head 0 sees a non-zero score
    sm = 0.5
    o, lse = _run(hb, sm_scale=sm)
    s = sm * 2.0 * float(np.dot(hb.q[0, 0].astype(np.float64), hb.q[0, 0].astype(np.float64)))
    V = hb.v_pool[slots, 0].astype(np.float64)
    w = np.ones(L)
    w[target] = math.exp(s)
    expect = (w[:, None] * V).sum(axis=0) / w.sum()
    np.testing.assert_allclose(o[0, 0], expect, rtol=1e-12, atol=1e-12)
    assert abs(lse[0, 0] - math.log(w.sum())) < 1e-12
    # head 1 sees K = 0 for its own scores (q head 1 also reads kv head 0): s = sm * <q1, 2 q0>
    s1 = sm * 2.0 * float(np.dot(hb.q[0, 1].astype(np.float64), hb.q[0, 0].astype(np.float64)))
    w1 = np.ones(L)
    w1[target] = math.exp(s1)
    np.testing.assert_allclose(o[0, 1], (w1[:, None] * V).sum(axis=0) / w1.sum(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("spec", [SMALL_EXTEND, SMALL_DECODE])
def test_page_relabelling_is_bit_invariant(spec):
    hb = make_host_batch(spec, 7)
    o1, lse1 = _run(hb)
    rng = np.random.default_rng(99)
    lay2, slot_map = permute_pages(hb.layout, rng)
    k2 = np.full_like(hb.k_pool, np.nan)
    v2 = np.full_like(hb.v_pool, np.nan)
    k2[slot_map] = hb.k_pool
    v2[slot_map] = hb.v_pool
    o2, lse2 = oracle.paged_attention(hb.q, k2, v2, lay2.req_to_token, lay2.seq_lens, lay2.cu_seqlens_q)
    assert np.array_equal(o1, o2) and np.array_equal(lse1, lse2)


def test_gqa_equals_mha_with_repeated_heads():
    hb = make_host_batch(SMALL_EXTEND, 11)
    lay = hb.layout
    o1, lse1 = _run(hb)
    G = SMALL_EXTEND.num_q_heads // SMALL_EXTEND.num_kv_heads
    k_rep = np.repeat(hb.k_pool, G, axis=1)
    v_rep = np.repeat(hb.v_pool, G, axis=1)
    o2, lse2 = oracle.paged_attention(hb.q, k_rep, v_rep, lay.req_to_token, lay.seq_lens, lay.cu_seqlens_q)
    assert np.array_equal(o1, o2) and np.array_equal(lse1, lse2)


def test_rows_of_p_sum_to_one_and_respect_the_mask():
    hb = make_host_batch(SMALL_EXTEND, 13)
    lay = hb.layout
    _, _, probs = _run(hb, return_probs=True)
    for b in range(SMALL_EXTEND.batch):
        L, n = int(lay.seq_lens[b]), int(lay.new_lens[b])
        for P in probs[b]:
            assert P.shape == (n, L)
            np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
            i = np.arange(n)[:, None]
            j = np.arange(L)[None, :]
            assert np.all(P[j > (L - n) + i] == 0.0)


def test_power_of_two_v_scaling_is_exact():
    hb = make_host_batch(SMALL_DECODE, 17)
    o1, _ = _run(hb)
    hb.v_pool *= 8.0
    o2, _ = _run(hb)
    assert np.array_equal(o2, 8.0 * o1)


def test_future_keys_and_other_requests_do_not_matter():
    hb = make_host_batch(SMALL_EXTEND, 19)
    lay = hb.layout
    o1, _ = _run(hb)
    # perturb the last new token of request 0: every earlier row of request 0 and
    # every row of the other requests must be bit-identical
    L0, n0 = int(lay.seq_lens[0]), int(lay.new_lens[0])
    last = lay.req_to_token[0, L0 - 1]
    hb.k_pool[last] += 3.0
    hb.v_pool[last] -= 5.0
    o2, _ = _run(hb)
    assert np.array_equal(o1[:n0 - 1], o2[:n0 - 1])
    assert np.array_equal(o1[n0:], o2[n0:])
    assert not np.array_equal(o1[n0 - 1], o2[n0 - 1])


def test_decode_equals_last_row_of_extend():
    spec = SMALL_EXTEND
    hb = make_host_batch(spec, 23)
    lay = hb.layout
    o_ext, lse_ext = _run(hb)
    last_rows = lay.cu_seqlens_q[1:] - 1
    B = spec.batch
    o_dec, lse_dec = oracle.paged_attention(hb.q[last_rows], hb.k_pool, hb.v_pool, lay.req_to_token,
                                            lay.seq_lens, np.arange(B + 1))
    np.testing.assert_allclose(o_dec, o_ext[last_rows], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse_dec, lse_ext[last_rows], rtol=1e-13, atol=1e-13)


def test_empty_decode_row_and_empty_extend_request():
    spec = Spec("e", "extend", 3, 2, 1, 8, 2, [0, 5, 3], [0, 2, 0], dtype="fp32")
    hb = make_host_batch(spec, 1)
    lay = hb.layout
    o, lse = _run(hb)
    assert o.shape[0] == 2
    assert np.all(np.isfinite(o))
    # decode with a zero-length request
    q = np.ones((1, 2, 8))
    o, lse = oracle.paged_attention(q, hb.k_pool, hb.v_pool, lay.req_to_token[:1], np.array([0]),
                                    np.array([0, 1]))
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


def test_reuse_of_slots_across_requests_is_allowed():
    """Two requests sharing prefix pages (copy-on-write style) read the same rows."""
    spec = Spec("s", "decode", 2, 2, 1, 8, 4, [12, 12], 1, dtype="fp32")
    hb = make_host_batch(spec, 2)
    lay = hb.layout
    rtt = lay.req_to_token.copy()
    rtt[1, :8] = rtt[0, :8]  # share the first two pages
    o, _ = oracle.paged_attention(hb.q, hb.k_pool, hb.v_pool, rtt, lay.seq_lens, lay.cu_seqlens_q)
    # request 1's answer equals a request built from the shared rows explicitly
    k = hb.k_pool[rtt[1, :13]][None]
    v = hb.v_pool[rtt[1, :13]][None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(hb.q[1:2].astype(np.float64)).permute(1, 0, 2),
        torch.from_numpy(k[0].astype(np.float64)).permute(1, 0, 2).repeat_interleave(2, 0).contiguous(),
        torch.from_numpy(v[0].astype(np.float64)).permute(1, 0, 2).repeat_interleave(2, 0).contiguous(),
        scale=1 / math.sqrt(8))
    np.testing.assert_allclose(o[1], ref.permute(1, 0, 2).numpy()[0], rtol=1e-12, atol=1e-12)


def _brute_force_row(q, keys, vals, sm_scale):
    """Attention of one query over a list of keys, by explicit loops over plain
    floats ([FA-vs-PA], FlashAttention §1: softmax of the scaled dot products,
    then the weighted sum of the value rows)."""
    scores = []
    for k in keys:
        acc = 0.0
        for c in range(len(q)):
            acc += float(q[c]) * float(k[c])
        scores.append(sm_scale * acc)
    top = max(scores)
    weights = [math.exp(s - top) for s in scores]
    total = sum(weights)
    out = []
    for c in range(len(vals[0])):
        acc = 0.0
        for w, v in zip(weights, vals):
            acc += w * float(v[c])
        out.append(acc / total)
    return out, top + math.log(total)


@pytest.mark.parametrize("seed", [0, 1])
def test_matches_explicit_loop_brute_force(seed):
    """Tiny extend batch (GQA, page size 2, shuffled pool) against attention
    written out as loops: each new token of each request walks its visible
    positions, looks their slots up in the request's page-table row and
    accumulates over plain Python floats."""
    spec = Spec("bf_loops", "extend", 2, 4, 2, 4, 2, (0, 6), (1, 4), dtype="fp32")
    hb = make_host_batch(spec, 70 + seed)
    lay = hb.layout
    sm = 0.61
    o, lse = _run(hb, sm_scale=sm)
    G = spec.num_q_heads // spec.num_kv_heads
    for b in range(spec.batch):
        L = int(lay.seq_lens[b])
        n = int(lay.new_lens[b])
        q0 = int(lay.cu_seqlens_q[b])
        for i in range(n):
            visible = range(L - n + i + 1)
            for h in range(spec.num_q_heads):
                keys = [hb.k_pool[lay.req_to_token[b, j], h // G] for j in visible]
                vals = [hb.v_pool[lay.req_to_token[b, j], h // G] for j in visible]
                want, want_lse = _brute_force_row(hb.q[q0 + i, h], keys, vals, sm)
                np.testing.assert_allclose(o[q0 + i, h], want, rtol=1e-12, atol=1e-13)
                assert abs(lse[q0 + i, h] - want_lse) < 1e-12
