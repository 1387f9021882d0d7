"""Pins of the INT8 Q/K reading of the 8-bit (Sage) oracle.

[FlashInfer-Sage], code §3 and §4: Q and K may be INT8; their scores
accumulate in 32-bit and enter the softmax as fp32; the formula of the README
block is otherwise unchanged (P8 and V8 stay E4M3)."""
import math

import numpy as np

import oracle
from workloads import Spec, make_host_batch

I8 = Spec("i8", "decode", 3, 4, 2, 32, 4, (3, 70), 1, dtype="int8", k_block=16)


def test_int8_codes_are_twos_complement():
    """All 256 bytes against the definition of two's complement."""
    b = np.arange(256, dtype=np.uint8)
    want = np.where(b < 128, b.astype(np.int64), b.astype(np.int64) - 256).astype(np.float64)
    assert np.array_equal(oracle.qk_values(b, "int8"), want)
    assert np.array_equal(oracle.qk_values(b.view(np.int8), "int8"), want)
    assert oracle.qk_values(np.array([0x80], np.uint8), "int8")[0] == -128.0


def test_int8_two_key_hand_example():
    """d = 4, one head, two keys, unit Q/K scales.

    q = (3, -128, 0, 127), kA = (-2, 1, 0, 0), kB = (5, 0, 0, 1):
    q·kA = -6 - 128 = -134, q·kB = 15 + 127 = 142, a gap of 276.  With
    sm_scale = ln2 / 92 the gap is 3 ln 2, so p_A = 1/8, p_B = 1, 448·p_A = 56
    (an E4M3 value) and l = 9/8.  V (E4M3 values): vA = (1, 2, -0.5, 4),
    vB = (0.25, -1, 3, 8); sfV = (1, 2, 0.5, 1).
    O = sfV·(vA/8 + vB)/(9/8) = (1/3, -4/3, 47/36, 68/9);
    lse = 142·ln2/92 + ln(9/8).
    A byte read unsigned (-128 as 128) or as E4M3 changes the scores."""
    q8 = np.array([3, -128, 0, 127], np.int8)[None, None, :]
    k8 = np.array([[-2, 1, 0, 0], [5, 0, 0, 1]], np.int8)[:, None, :]
    v8 = oracle.e4m3_encode(np.array([[1.0, 2.0, -0.5, 4.0], [0.25, -1.0, 3.0, 8.0]]))[:, None, :]
    sfv = np.array([1.0, 2.0, 0.5, 1.0])[None, None, :]
    o, lse = oracle.sage_decode(q8, k8, v8, np.array([[0, 1]]), [2], np.ones((1, 1)), np.ones((1, 1, 1)), sfv,
                                k_block=64, sm_scale=math.log(2) / 92, qk_codes="int8")
    np.testing.assert_allclose(o[0, 0], [1 / 3, -4 / 3, 47 / 36, 68 / 9], rtol=1e-14, atol=1e-15)
    assert abs(lse[0, 0] - (142 * math.log(2) / 92 + math.log(9 / 8))) < 1e-13


def test_int8_extreme_codes_dot_product_is_exact():
    """q = k = all -128 over d = 128: q·k = 128·16384 = 2^21, exactly.  One
    key, so O = sfV·v and lse = S = sm_scale·sfq·sfk·2^21."""
    d = 128
    q8 = np.full((1, 1, d), -128, np.int8)
    k8 = np.full((1, 1, d), -128, np.int8)
    v8 = oracle.e4m3_encode(np.linspace(-2, 2, d))[None, None, :]
    sfv = np.full((1, 1, d), 0.5)
    o, lse = oracle.sage_decode(q8, k8, v8, np.array([[0]]), [1], np.full((1, 1), 0.25), np.full((1, 1, 1), 2.0 ** -20),
                                sfv, k_block=16, sm_scale=1.0, qk_codes="int8")
    assert lse[0, 0] == 0.25 * 2.0 ** -20 * 2.0 ** 21
    np.testing.assert_array_equal(o[0, 0], 0.5 * oracle.e4m3_decode(v8[0, 0]))


def _as_e4m3(hb):
    """The same batch with its int8 Q/K codes re-encoded as E4M3 (exact for |x| <= 16)."""
    q = oracle.e4m3_encode(hb.q_codes.astype(np.float64))
    k = oracle.e4m3_encode(hb.k_codes.astype(np.float64))
    return q, k


def _small_codes(hb, rng):
    """Replace the int8 codes by integers in [-16, 16], which E4M3 holds exactly."""
    hb.q_codes = rng.integers(-16, 17, size=hb.q_codes.shape).astype(np.int8)
    hb.k_codes = rng.integers(-16, 17, size=hb.k_codes.shape).astype(np.int8)
    return hb


def test_int8_equals_e4m3_reading_where_values_coincide():
    """Every 8-bit function gives the same float64 result for int8 codes and
    for E4M3 codes of the same values: the two readings differ only in how a
    byte maps to a value (the E4M3 path is pinned on its own)."""
    rng = np.random.default_rng(5)
    for seed in (0, 1):
        hb = _small_codes(make_host_batch(I8, seed), rng)
        q_e, k_e = _as_e4m3(hb)
        lay = hb.layout
        args = (lay.req_to_token, lay.seq_lens, hb.sfq, hb.sfk, hb.sfv, I8.k_block)
        o_i, l_i = oracle.sage_decode(hb.q_codes, hb.k_codes, hb.v_codes, *args, qk_codes="int8")
        o_e, l_e = oracle.sage_decode(q_e, k_e, hb.v_codes, *args)
        assert np.array_equal(o_i, o_e) and np.array_equal(l_i, l_e)
        # the multi-row (extend) form on the same batch
        cu = lay.cu_seqlens_q
        o_i, l_i = oracle.sage_extend(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, lay.seq_lens, cu,
                                      hb.sfq, hb.sfk, hb.sfv, I8.k_block, qk_codes="int8")
        o_e, l_e = oracle.sage_extend(q_e, k_e, hb.v_codes, lay.req_to_token, lay.seq_lens, cu,
                                      hb.sfq, hb.sfk, hb.sfv, I8.k_block)
        assert np.array_equal(o_i, o_e) and np.array_equal(l_i, l_e)
        # block-sparse: every other 16-token block listed
        nblk = [(int(L) + 15) // 16 for L in lay.seq_lens]
        idx = [np.arange(0, n, 2) for n in nblk]
        indptr = np.concatenate([[0], np.cumsum([len(i) for i in idx])])
        blocks = np.concatenate(idx)
        o_i, l_i = oracle.block_sparse_sage_decode(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token,
                                                   lay.seq_lens, indptr, blocks, 16, hb.sfq, hb.sfk, hb.sfv,
                                                   I8.k_block, qk_codes="int8")
        o_e, l_e = oracle.block_sparse_sage_decode(q_e, k_e, hb.v_codes, lay.req_to_token, lay.seq_lens, indptr,
                                                   blocks, 16, hb.sfq, hb.sfk, hb.sfv, I8.k_block)
        assert np.array_equal(o_i, o_e) and np.array_equal(l_i, l_e)


def test_int8_scores_match_integer_arithmetic():
    """On a drawn batch, lse with one visible key is that key's score, and the
    score equals sm_scale·sfQ·sfK times the integer dot product computed in
    exact int64 arithmetic."""
    hb = make_host_batch(I8, 3)
    lay = hb.layout
    seq1 = np.ones_like(lay.seq_lens)
    _, lse = oracle.sage_decode(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, seq1, hb.sfq, hb.sfk, hb.sfv,
                                I8.k_block, sm_scale=0.125, qk_codes="int8")
    G = I8.num_q_heads // I8.num_kv_heads
    for b in range(I8.batch):
        slot = int(lay.req_to_token[b, 0])
        for h in range(I8.num_q_heads):
            dot = int(np.dot(hb.q_codes[b, h].astype(np.int64), hb.k_codes[slot, h // G].astype(np.int64)))
            want = 0.125 * float(hb.sfq[b, h]) * float(hb.sfk[b, h // G, 0]) * dot
            assert abs(lse[b, h] - want) <= 1e-12 * max(1.0, abs(want))


def test_int8_batch_codes_cover_the_range():
    """The generated codes are signed and use most of the int8 range."""
    hb = make_host_batch(I8, 0, poison=False)
    used = hb.layout.slot_owner >= 0
    k = hb.k_codes[used]
    assert hb.q_codes.dtype == np.int8 and hb.k_codes.dtype == np.int8
    assert k.min() < -60 and k.max() > 60 and abs(float(k.mean())) < 2.0
