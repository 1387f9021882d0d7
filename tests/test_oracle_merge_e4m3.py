"""Pins of the LSE merge and of the E4M3 codec."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import Spec, make_host_batch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("seed", [0, 1])
def test_lse_merge_over_any_partition_equals_unsplit(seed):
    spec = Spec("m", "decode", 3, 4, 2, 16, 1, (5, 60), 1, dtype="fp32", pool=256)
    hb = make_host_batch(spec, seed)
    lay = hb.layout
    o_full, lse_full = oracle.paged_attention(hb.q, hb.k_pool, hb.v_pool, lay.req_to_token,
                                              lay.seq_lens, lay.cu_seqlens_q)
    rng = np.random.default_rng(seed + 100)
    for b in range(spec.batch):
        L = int(lay.seq_lens[b])
        cuts = np.sort(rng.choice(np.arange(1, L), size=min(3, L - 1), replace=False))
        bounds = [0] + list(cuts) + [L, L]  # last piece empty on purpose
        outs, lses = [], []
        for k0, k1 in zip(bounds[:-1], bounds[1:]):
            rtt = lay.req_to_token[b:b + 1, k0:k1] if k1 > k0 else np.zeros((1, 1), np.int32)
            o, l = oracle.paged_attention(hb.q[b:b + 1], hb.k_pool, hb.v_pool, rtt,
                                          np.array([k1 - k0]), np.array([0, 1]))
            outs.append(o[0])
            lses.append(l[0])
        O, lse = oracle.lse_merge(outs, lses)
        np.testing.assert_allclose(O, o_full[b], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, lse_full[b], rtol=1e-12, atol=1e-12)


def test_lse_merge_closed_forms():
    a = np.array([1.0, 2.0])
    b = np.array([3.0, -2.0])
    O, lse = oracle.lse_merge([a, b], [0.5, 0.5])
    np.testing.assert_allclose(O, (a + b) / 2, rtol=0, atol=1e-15)
    assert abs(lse - (0.5 + math.log(2))) < 1e-15
    O, lse = oracle.lse_merge([a, b], [-np.inf, -np.inf])
    assert np.all(O == 0) and np.isneginf(lse)
    O, lse = oracle.lse_merge([a, b], [1.25, -np.inf])
    assert np.array_equal(O, a) and lse == 1.25


def _all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    return v[np.isfinite(v)]


def test_e4m3_encode_matches_torch_float8_e4m3fn_exhaustively():
    v = _all_bf16_values()
    v = v[np.abs(v) <= 464.0]  # torch returns NaN above the rounding range; the oracle saturates
    ours = oracle.e4m3_encode(v.astype(np.float64))
    theirs = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # -0.0 and 0.0 both encode to a zero; compare values for zeros, codes elsewhere
    nz = v != 0
    assert np.array_equal(ours[nz], theirs[nz])
    assert np.all(oracle.e4m3_decode(ours[~nz]) == 0)


def test_e4m3_ties_between_neighbours_round_to_even():
    codes = np.arange(0, 0x7E, dtype=np.uint8)  # consecutive positive finite values
    lo = oracle.e4m3_decode(codes)
    hi = oracle.e4m3_decode(codes + 1)
    mid = (lo + hi) / 2  # exactly representable in float32
    ours = oracle.e4m3_encode(mid)
    theirs = torch.from_numpy(mid.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)
    assert np.all(ours % 2 == 0)  # the even neighbour


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(ours)
    assert np.array_equal(ours[ok], theirs[ok])
    assert np.nanmax(ours) == oracle.E4M3_MAX == 448.0


def test_e4m3_landmarks():
    with open(os.path.join(GOLDEN, "e4m3_landmarks.json")) as f:
        g = json.load(f)
    xs = np.array([x for x, _ in g["encode"]])
    want = np.array([c for _, c in g["encode"]], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(xs), want)
    assert oracle.e4m3_encode(np.array([np.nan]))[0] & 0x7F == 0x7F


def test_e4m3_round_trip_of_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    ok = ~np.isnan(vals)
    back = oracle.e4m3_encode(vals[ok])
    assert np.array_equal(oracle.e4m3_decode(back), vals[ok])
