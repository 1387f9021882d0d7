"""Pins of the block-sparse decode oracle (bf16 and 8-bit).

Each pin ties the masked-softmax definition to something other than itself:
the pinned dense oracles (every block listed; a page table cut down by hand
to the selected positions), the log-sum-exp merge identity over a disjoint
split of the selected blocks, and one-hot scores."""
import math

import numpy as np
import pytest

import oracle
from oracle.block_sparse import block_sparse_decode, block_sparse_sage_decode, key_mask
from workloads import Spec, block_mask, make_host_batch

BF = Spec("bs", "decode", 4, 6, 2, 32, 4, (1, 300), 1, dtype="bf16")
F8 = Spec("bs8", "decode", 3, 4, 2, 32, 4, (1, 300), 1, dtype="fp8", k_block=16)


def _q(hb):
    return hb.q  # decode: one row per request, [B, Hq, d]


def _mask(lay, bs, density, seed):
    return block_mask(lay.seq_lens, bs, density, np.random.default_rng(seed))


def _all_blocks(lay, bs, rng):
    indptr, idx = [0], []
    for L in lay.seq_lens:
        n = -(-int(L) // bs)
        idx.extend(rng.permutation(n).tolist())  # every block, in any order
        indptr.append(len(idx))
    return np.asarray(indptr), np.asarray(idx)


def _compacted(lay, indptr, idx, bs):
    """Page table cut down by hand to the listed positions, in position order."""
    B = len(lay.seq_lens)
    rows, lens = [], []
    for b in range(B):
        L = int(lay.seq_lens[b])
        listed = set(int(k) for k in idx[indptr[b]:indptr[b + 1]])
        pos = [j for j in range(L) if j // bs in listed]
        rows.append(lay.req_to_token[b, pos])
        lens.append(len(pos))
    W = max(max(lens), 1)
    rtt = np.full((B, W), -1, np.int64)
    for b in range(B):
        rtt[b, :lens[b]] = rows[b]
    return rtt, np.asarray(lens), [np.asarray([j for j in range(int(lay.seq_lens[b]))
                                               if j // bs in set(int(k) for k in idx[indptr[b]:indptr[b + 1]])])
                                   for b in range(B)]


def test_key_mask_by_hand():
    m = key_mask(10, [0, 2, 9], 4)  # blocks {0..3}, {8, 9}; block 9 lies past L
    assert m.tolist() == [True] * 4 + [False] * 4 + [True] * 2


@pytest.mark.parametrize("bs", [4, 16, 64])
def test_every_block_listed_is_dense_decode(bs):
    hb = make_host_batch(BF, 0)
    lay = hb.layout
    indptr, idx = _all_blocks(lay, bs, np.random.default_rng(1))
    o, lse = block_sparse_decode(_q(hb), hb.k_pool, hb.v_pool, lay.req_to_token, lay.seq_lens, indptr, idx, bs)
    o2, lse2 = oracle.paged_attention(_q(hb), hb.k_pool, hb.v_pool, lay.req_to_token, lay.seq_lens,
                                      lay.cu_seqlens_q)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bs,density", [(4, 0.3), (16, 0.125), (64, 0.5)])
def test_equals_dense_decode_on_the_cut_down_page_table(bs, density):
    """Keys outside the listed blocks are gone: the same as dense decode over a
    page table holding only the listed positions (a partial last block keeps
    only its existing keys)."""
    hb = make_host_batch(BF, 2)
    lay = hb.layout
    indptr, idx = _mask(lay, bs, density, 3)
    o, lse = block_sparse_decode(_q(hb), hb.k_pool, hb.v_pool, lay.req_to_token, lay.seq_lens, indptr, idx, bs)
    rtt, lens, _ = _compacted(lay, indptr, idx, bs)
    cu = np.arange(len(lens) + 1)
    o2, lse2 = oracle.paged_attention(_q(hb), hb.k_pool, hb.v_pool, rtt, lens, cu)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-12)


def test_disjoint_split_merges_by_log_sum_exp():
    hb = make_host_batch(BF, 4)
    lay = hb.layout
    bs = 8
    indptr, idx = _mask(lay, bs, 0.6, 5)
    ia, ib, pa, pb = [], [], [0], [0]
    rng = np.random.default_rng(6)
    for b in range(len(lay.seq_lens)):
        blocks = idx[indptr[b]:indptr[b + 1]]
        side = rng.integers(0, 2, size=len(blocks))
        ia.extend(blocks[side == 0].tolist())
        ib.extend(blocks[side == 1].tolist())
        pa.append(len(ia))
        pb.append(len(ib))
    args = (_q(hb), hb.k_pool, hb.v_pool, lay.req_to_token, lay.seq_lens)
    o, lse = block_sparse_decode(*args, indptr, idx, bs)
    oa, la = block_sparse_decode(*args, np.asarray(pa), np.asarray(ia), bs)
    ob, lb = block_sparse_decode(*args, np.asarray(pb), np.asarray(ib), bs)
    l_ab = np.logaddexp(la, lb)
    np.testing.assert_allclose(lse, l_ab, rtol=0, atol=1e-12)
    wa = np.where(np.isneginf(la), 0.0, np.exp(la - l_ab))[..., None]
    wb = np.where(np.isneginf(lb), 0.0, np.exp(lb - l_ab))[..., None]
    np.testing.assert_allclose(o, wa * oa + wb * ob, rtol=1e-12, atol=1e-12)


def test_out_of_range_blocks_select_nothing_and_empty_selection():
    hb = make_host_batch(BF, 7)
    lay = hb.layout
    bs = 16
    indptr, idx = _mask(lay, bs, 0.3, 8)
    args = (_q(hb), hb.k_pool, hb.v_pool, lay.req_to_token, lay.seq_lens)
    o, lse = block_sparse_decode(*args, indptr, idx, bs)
    # append block numbers past the request's end and negative ones
    ip2, ix2 = [0], []
    for b in range(len(lay.seq_lens)):
        n = -(-int(lay.seq_lens[b]) // bs)
        ix2.extend([-3] + idx[indptr[b]:indptr[b + 1]].tolist() + [n, n + 5])
        ip2.append(len(ix2))
    o2, lse2 = block_sparse_decode(*args, np.asarray(ip2), np.asarray(ix2), bs)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # no block at all: O = 0, lse = -inf
    o3, lse3 = block_sparse_decode(*args, np.zeros(len(lay.seq_lens) + 1, np.int64), np.zeros(0, np.int64), bs)
    assert np.all(o3 == 0) and np.all(np.isneginf(lse3))


def test_one_hot_key_inside_and_outside_the_mask():
    """A key with an overwhelming score decides the output when its block is
    listed and changes nothing when it is not."""
    B, H, d, L, bs = 1, 1, 8, 40, 8
    rng = np.random.default_rng(9)
    q = np.zeros((B, H, d))
    q[0, 0, 0] = 1.0
    k = rng.standard_normal((L, H, d)) * 0.01
    v = rng.standard_normal((L, H, d))
    k[21, 0, 0] = 1e3  # block 2
    rtt = np.arange(L)[None]
    seq = [L]
    listed = block_sparse_decode(q, k, v, rtt, seq, [0, 2], [1, 2], bs, sm_scale=1.0)
    np.testing.assert_allclose(listed[0][0, 0], v[21, 0], rtol=0, atol=1e-12)
    assert abs(listed[1][0, 0] - 1e3) < 1e-9
    unlisted = block_sparse_decode(q, k, v, rtt, seq, [0, 2], [1, 3], bs, sm_scale=1.0)
    keep = [j for j in range(L) if j // bs in (1, 3)]
    s = k[keep, 0] @ q[0, 0]
    p = np.exp(s - s.max())
    np.testing.assert_allclose(unlisted[0][0, 0], p @ v[keep, 0] / p.sum(), rtol=1e-12, atol=1e-12)


def _sage_sparse(hb, indptr, idx, bs, **kw):
    lay = hb.layout
    return block_sparse_sage_decode(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, lay.seq_lens, indptr,
                                    idx, bs, hb.sfq, hb.sfk, hb.sfv, F8.k_block, **kw)


def test_sage_every_block_listed_is_sage_decode():
    hb = make_host_batch(F8, 0)
    lay = hb.layout
    indptr, idx = _all_blocks(lay, 32, np.random.default_rng(2))
    vm = np.random.default_rng(3).standard_normal((F8.batch, F8.num_kv_heads, F8.head_dim))
    o, lse = _sage_sparse(hb, indptr, idx, 32, v_mean=vm)
    o2, lse2 = oracle.sage_decode(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, lay.seq_lens, hb.sfq,
                                  hb.sfk, hb.sfv, F8.k_block, v_mean=vm)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-12)


def test_sage_sfk_follows_the_logical_position():
    """With block_size a multiple of k_block, the result equals sage_decode on
    the cut-down page table whose sfK rows are those of the listed positions'
    logical k_blocks, assembled here by hand."""
    hb = make_host_batch(F8, 1)
    lay = hb.layout
    bs = 2 * F8.k_block
    indptr, idx = _mask(lay, bs, 0.4, 4)
    o, lse = _sage_sparse(hb, indptr, idx, bs)
    rtt, lens, pos = _compacted(lay, indptr, idx, bs)
    nv = max(-(-int(lens.max()) // F8.k_block), 1)
    sfk2 = np.ones((F8.batch, F8.num_kv_heads, nv), np.float32)
    for b in range(F8.batch):
        for u in range(-(-int(lens[b]) // F8.k_block)):
            sfk2[b, :, u] = hb.sfk[b, :, pos[b][u * F8.k_block] // F8.k_block]
    o2, lse2 = oracle.sage_decode(hb.q_codes, hb.k_codes, hb.v_codes, rtt, lens, hb.sfq, sfk2, hb.sfv,
                                  F8.k_block)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-12)


def test_sage_empty_selection_gives_v_mean():
    hb = make_host_batch(F8, 2)
    vm = np.random.default_rng(5).standard_normal((F8.batch, F8.num_kv_heads, F8.head_dim))
    o, lse = _sage_sparse(hb, np.zeros(F8.batch + 1, np.int64), np.zeros(0, np.int64), 32, v_mean=vm)
    G = F8.num_q_heads // F8.num_kv_heads
    for b in range(F8.batch):
        np.testing.assert_array_equal(o[b], np.repeat(vm[b], G, axis=0))
    assert np.all(np.isneginf(lse))


def test_block_mask_generator_shape():
    lens = np.array([0, 1, 64, 65, 1000])
    indptr, idx = block_mask(lens, 64, 0.1, np.random.default_rng(0))
    counts = np.diff(indptr)
    assert counts.tolist() == [0, 1, 1, 1, 2]
    for b, L in enumerate(lens):
        blocks = idx[indptr[b]:indptr[b + 1]]
        assert np.all(np.diff(blocks) > 0)
        if L:
            assert blocks[-1] == (L - 1) // 64
