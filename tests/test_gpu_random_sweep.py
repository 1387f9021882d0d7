"""Seeded random sweeps over the shapes each path accepts (batch, heads,
grouping, head_dim, page size, lengths with empty and tiny requests, block
masks), every case against the fp64 oracle.  They complement the hand-picked
cases with combinations nobody chose; a failure prints the case."""
import os

import numpy as np
import pytest

import oracle
from gpu_util import FP8_REL_L2, assert_bf16_close, check_rel_l2, assert_lse_close, rel_l2
from workloads import Spec, make_host_batch

pytestmark = pytest.mark.gpu

# cases per family; PKV_SWEEP_CASES raises it for a longer run
CASES = int(os.environ.get("PKV_SWEEP_CASES", "16"))


def _draw_shape(rng, d_choices=(64, 128), max_group=16, max_hkv=8, max_batch=9):
    hkv = int(rng.choice([h for h in (1, 2, 3, 4, 8, 12, 24) if h <= max_hkv]))
    group = int(rng.choice([g for g in (1, 2, 3, 4, 5, 8, 16) if g <= max_group]))
    d = int(rng.choice(d_choices))
    page = int(rng.choice([1, 2, 16, 64]))
    batch = int(rng.integers(1, max_batch + 1))
    return batch, group * hkv, hkv, d, page


def _lengths(rng, batch, lo, hi, p_empty=0.15):
    """Uniform lengths with some set to 0; at least one stays positive when lo >= 1."""
    n = rng.integers(lo, hi + 1, size=batch)
    n[rng.random(batch) < p_empty] = 0
    if lo >= 1 and not n.any():
        n[0] = lo
    return [int(x) for x in n]


def test_random_bf16_decode():
    from test_gpu_decode import oracle_decode, run_decode
    rng = np.random.default_rng(2024)
    for case in range(CASES):
        # up to 24 kv heads: layouts with more than 16 units per token take
        # the kernel instances with plain K/V loads
        B, hq, hkv, d, page = _draw_shape(rng, max_group=8, max_hkv=24)
        q_len = int(rng.choice([1, 1, 2, 4]))
        spec = Spec(f"rd{case}", "decode", B, hq, hkv, d, page, _lengths(rng, B, 0, 900), q_len)
        hb = make_host_batch(spec, case)
        kv_chunk = int(rng.choice([0, 0, 64, 160]))
        what = f"case {case}: B={B} hq={hq} hkv={hkv} d={d} page={page} n={q_len} kv_chunk={kv_chunk}"
        o, lse, _, _ = run_decode(hb, kv_chunk=kv_chunk, decode_q_len=q_len)
        ro, rlse = oracle_decode(hb)
        assert_bf16_close(o, ro, what)
        assert_lse_close(lse, rlse, what)


def test_random_bf16_extend():
    from test_gpu_extend import oracle_extend, run_extend
    rng = np.random.default_rng(2025)
    for case in range(CASES):
        B, hq, hkv, d, page = _draw_shape(rng)
        spec = Spec(f"re{case}", "extend", B, hq, hkv, d, page, _lengths(rng, B, 0, 500),
                    _lengths(rng, B, 1, 400, p_empty=0.2))
        hb = make_host_batch(spec, case)
        what = f"case {case}: B={B} hq={hq} hkv={hkv} d={d} page={page}"
        o, lse, _ = run_extend(hb)
        ro, rlse = oracle_extend(hb)
        assert_bf16_close(o, ro, what)
        assert_lse_close(lse, rlse, what)


def test_random_fp8_decode_and_extend():
    from test_gpu_decode_fp8 import oracle_fp8, run_fp8
    from test_gpu_extend_fp8 import oracle_fp8_extend, run_fp8_extend
    rng = np.random.default_rng(2026)
    for case in range(CASES):
        mode = "decode" if case % 2 == 0 else "extend"
        # the 8-bit extend oracle loops over rows and heads: smaller extend cases
        B, hq, hkv, d, page = (_draw_shape(rng, d_choices=(128,)) if mode == "decode" else
                               _draw_shape(rng, d_choices=(128,), max_group=8, max_hkv=4, max_batch=6))
        k_block = int(rng.choice([16, 32, 64]))
        new = 1 if mode == "decode" else _lengths(rng, B, 1, 150, p_empty=0.2)
        spec = Spec(f"r8{case}", mode, B, hq, hkv, d, page, _lengths(rng, B, 0, 600), new, dtype="fp8",
                    k_block=k_block)
        hb = make_host_batch(spec, case)
        vm = rng.standard_normal((B, hkv, d)).astype(np.float32) if case % 3 == 0 else None
        what = f"case {case}: {mode} B={B} hq={hq} hkv={hkv} page={page} k_block={k_block} v_mean={vm is not None}"
        if mode == "decode" and case % 4 == 2:
            # several new tokens per request: the extend formula with n rows each
            from test_gpu_decode_fp8 import run_fp8_multi
            n = int(rng.choice([2, 3, 4]))
            spec = Spec(f"r8m{case}", "decode", B, hq, hkv, d, page, _lengths(rng, B, 0, 600), n, dtype="fp8",
                        k_block=k_block)
            hb = make_host_batch(spec, case)
            what += f" n={n}"
            o, lse, sfq_rows = run_fp8_multi(hb, n, v_mean=vm)
            lay = hb.layout
            ro, rlse = oracle.sage_extend(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, lay.seq_lens,
                                          lay.cu_seqlens_q, sfq_rows, hb.sfk, hb.sfv, k_block, v_mean=vm)
        elif mode == "decode":
            o, lse = run_fp8(hb, v_mean=vm)
            ro, rlse = oracle_fp8(hb, v_mean=vm)
        else:
            o, lse = run_fp8_extend(hb, v_mean=vm)
            ro, rlse = oracle_fp8_extend(hb, v_mean=vm)
        assert np.all(np.isfinite(o)), what
        check_rel_l2(o, ro, str(what))
        fin = np.isfinite(rlse)
        assert np.array_equal(np.isfinite(lse), fin), what
        if fin.any():
            assert np.abs(lse[fin] - rlse[fin]).max() <= 1e-3, what


def test_random_block_sparse_decode():
    from test_gpu_block_sparse import mask_with_edges, oracle_sparse, run_sparse
    rng = np.random.default_rng(2027)
    for case in range(CASES):
        fp8 = case % 2 == 1
        B, hq, hkv, d, page = _draw_shape(rng, d_choices=(128,) if fp8 else (64, 128))
        k_block = 64  # 8-bit: the block sizes below are its multiples
        bs = int(rng.choice([64, 128, 256])) if fp8 else int(rng.choice([1, 16, 32, 64, 128]))
        spec = Spec(f"rs{case}", "decode", B, hq, hkv, d, page, _lengths(rng, B, 0, 1500), 1,
                    dtype="fp8" if fp8 else "bf16", k_block=k_block)
        hb = make_host_batch(spec, case)
        density = float(rng.choice([0.05, 0.2, 0.5, 1.0]))
        empty = tuple(int(x) for x in rng.choice(B, size=min(B, int(rng.integers(0, 2))), replace=False))
        indptr, idx = mask_with_edges(hb.layout, bs, density, case, empty=empty, junk=bool(case % 3 == 0))
        what = f"case {case}: fp8={fp8} B={B} hq={hq} hkv={hkv} d={d} page={page} bs={bs} density={density}"
        o, lse, _ = run_sparse(hb, indptr, idx, bs)
        ro, rlse = oracle_sparse(hb, indptr, idx, bs)
        if fp8:
            assert np.all(np.isfinite(o)), what
            check_rel_l2(o, ro, str(what))
            fin = np.isfinite(rlse)
            assert np.array_equal(np.isfinite(lse), fin), what
            if fin.any():
                assert np.abs(lse[fin] - rlse[fin]).max() <= 1e-3, what
        else:
            assert_bf16_close(o, ro, what)
            assert_lse_close(lse, rlse, what)


def test_random_int8_decode():
    """INT8 Q/K Sage decode: one and several new tokens, dense and block-sparse."""
    from test_gpu_block_sparse import mask_with_edges, oracle_sparse, run_sparse
    from test_gpu_decode_fp8 import oracle_fp8, run_fp8, run_fp8_multi
    rng = np.random.default_rng(2028)
    for case in range(CASES // 2):
        B, hq, hkv, d, page = _draw_shape(rng, d_choices=(128,))
        k_block = int(rng.choice([16, 32, 64]))
        kind = ("one", "multi", "sparse")[case % 3]
        n = int(rng.choice([2, 3, 4])) if kind == "multi" else 1
        spec = Spec(f"ri8{case}", "decode", B, hq, hkv, d, page, _lengths(rng, B, 0, 900), n, dtype="int8",
                    k_block=64 if kind == "sparse" else k_block)
        hb = make_host_batch(spec, 300 + case)
        vm = rng.standard_normal((B, hkv, d)).astype(np.float32) if case % 2 == 0 else None
        what = f"case {case}: {kind} B={B} hq={hq} hkv={hkv} page={page} n={n} k_block={spec.k_block}"
        if kind == "one":
            o, lse = run_fp8(hb, v_mean=vm)
            ro, rlse = oracle_fp8(hb, v_mean=vm)
        elif kind == "multi":
            lay = hb.layout
            o, lse, sfq_rows = run_fp8_multi(hb, n, v_mean=vm)
            ro, rlse = oracle.sage_extend(hb.q_codes, hb.k_codes, hb.v_codes, lay.req_to_token, lay.seq_lens,
                                          lay.cu_seqlens_q, sfq_rows, hb.sfk, hb.sfv, spec.k_block, v_mean=vm,
                                          qk_codes="int8")
        else:
            bs = int(rng.choice([64, 128]))
            indptr, idx = mask_with_edges(hb.layout, bs, float(rng.choice([0.1, 0.5])), case)
            o, lse, _ = run_sparse(hb, indptr, idx, bs, v_mean=vm)
            ro, rlse = oracle_sparse(hb, indptr, idx, bs, v_mean=vm)
        assert np.all(np.isfinite(o)), what
        check_rel_l2(o, ro, str(what))
        fin = np.isfinite(rlse)
        assert np.array_equal(np.isfinite(lse), fin), what
        if fin.any():
            assert np.abs(lse[fin] - rlse[fin]).max() <= 1e-3, what
