"""Hand-worked pins of the 8-bit (Sage) quantisation step of the oracle.

[FlashInfer-Sage], code §1 and the README "Sage attention" block: the row's
probabilities p = exp(S - m) are kept as E4M3 codes of 448·p, and the sum of
those codes times V8 is divided by 448 times the row sum l of the unquantised
p.  The cases in ``tests/golden/sage_quantisation_cases.json`` use
probabilities that are not powers of two (0.3, 0.01, 0.6, 0.05, 0.7), so

* rounding p first and scaling afterwards (448·E4M3(p)) gives other codes,
* dividing by the sum of the codes instead of 448·l gives another divisor,

and either mistake changes the expected outputs, which are derived by hand in
the file.  One case each for E4M3 Q/K decode, INT8 Q/K decode, block-sparse
decode and the extend rows.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sage_quantisation_cases.json")


def _load():
    with open(GOLDEN) as f:
        return json.load(f)


def _sfk(exprs):
    """The golden file writes the K scales as short expressions of logs."""
    out = []
    for e in exprs:
        if e == "1":
            out.append(1.0)
            continue
        assert e.startswith("ln(")
        inner, _, div = e[3:].partition(")")
        num, _, den = inner.partition("/")
        val = math.log(float(num) / (float(den) if den else 1.0))
        if div:
            assert div.startswith("/")
            val /= float(div[1:])
        out.append(val)
    return np.asarray(out, np.float64)


def _v_rows(g, case):
    rows = []
    for r in case["v_rows"]:
        if isinstance(r, str):
            rows.append([float(r)] * 4)
        else:
            rows.append(g["v"][r])
    return np.asarray(rows, np.float64)


def _codes(vals, qk_codes):
    vals = np.asarray(vals)
    if qk_codes == "int8":
        return vals.astype(np.int8)
    codes = oracle.e4m3_encode(vals)
    assert np.array_equal(oracle.e4m3_decode(codes), vals), "golden Q/K values must be E4M3 values"
    return codes


def _inputs(g, case):
    k = np.asarray(case["k"])
    L = k.shape[0]
    q8 = _codes(np.asarray(case["q"])[None, None, :], case["qk_codes"])
    k8 = _codes(k[:, None, :], case["qk_codes"])
    v = _v_rows(g, case)
    v8 = oracle.e4m3_encode(v)[:, None, :]
    assert np.array_equal(oracle.e4m3_decode(v8[:, 0, :]), v)
    sfk = _sfk(case["sfk_expr"])[None, None, :]
    sfv = np.asarray(g["sfv"], np.float64)[None, None, :]
    rtt = np.arange(L, dtype=np.int32)[None, :]
    return q8, k8, v8, sfk, sfv, rtt, L


def _case(name):
    g = _load()
    for c in g["cases"]:
        if c["name"] == name:
            return g, c
    raise KeyError(name)


def test_golden_codes_are_the_e4m3_rounding_of_448p():
    """The hand-derived P8 of each case is what the codec gives for 448·p,
    and differs from 448·E4M3(p), the other order of the two steps."""
    g = _load()
    for c in g["cases"]:
        if "p8" not in c:
            continue
        p8 = np.asarray(c["p8"])
        assert np.all(oracle.e4m3_decode(oracle.e4m3_encode(p8)) == p8)
        assert abs(p8.sum() - 448 * c["l"]) > 1e-3, c["name"]
        alt = np.asarray(c["mutation_p8_448_times_e4m3_p"])
        assert np.any(alt != p8), c["name"]


@pytest.mark.parametrize("name", ["e4m3_decode_three_keys", "int8_decode_three_keys"])
def test_sage_decode_quantisation_golden(name):
    g, c = _case(name)
    q8, k8, v8, sfk, sfv, rtt, L = _inputs(g, c)
    o, lse = oracle.sage_decode(q8, k8, v8, rtt, [L], np.ones((1, 1)), sfk, sfv, k_block=1, sm_scale=1.0,
                                qk_codes=c["qk_codes"])
    np.testing.assert_allclose(o[0, 0], c["expected_o"], rtol=1e-12, atol=1e-14)
    assert abs(lse[0, 0] - c["expected_lse"]) < 1e-12


def test_block_sparse_sage_decode_quantisation_golden():
    g, c = _case("e4m3_block_sparse_six_keys")
    q8, k8, v8, sfk, sfv, rtt, L = _inputs(g, c)
    blocks = np.asarray(c["blocks"], np.int32)
    o, lse = oracle.block_sparse_sage_decode(q8, k8, v8, rtt, [L], np.array([0, len(blocks)], np.int32), blocks,
                                             c["block_size"], np.ones((1, 1)), sfk, sfv, k_block=1, sm_scale=1.0)
    np.testing.assert_allclose(o[0, 0], c["expected_o"], rtol=1e-12, atol=1e-14)
    assert abs(lse[0, 0] - c["expected_lse"]) < 1e-12


def test_sage_extend_quantisation_golden():
    g, c = _case("e4m3_extend_two_rows")
    q8, k8, v8, sfk, sfv, rtt, L = _inputs(g, c)
    q8 = np.repeat(q8[0], 2, axis=0)[:, None, :]  # two new-token rows, same codes
    o, lse = oracle.sage_extend(q8, k8, v8, rtt, [L], [0, 2], np.ones((2, 1)), sfk, sfv, k_block=1, sm_scale=1.0)
    np.testing.assert_allclose(o[:, 0], c["expected_o_rows"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[:, 0], c["expected_lse_rows"], rtol=0, atol=1e-12)
