"""The allocation-free decode entry point (pkv_attn_decode_noalloc) through
the C ABI: its output equals pkv_attn_decode's bit for bit (same kernels,
same plan) on two calls in a row, the second with a smaller batch, so the
static scratch keeps no state that a later call depends on; and a decode
whose split scratch exceeds the static size is rejected before any launch."""
import numpy as np
import pytest

from gpu_util import dev_f32, dev_i32, dev_u8, torch_mod
from workloads import SPECS, Spec, make_device_batch, make_host_batch, pool_before_store

pytestmark = pytest.mark.gpu


def _pkv():
    import flashattention_paged_kv_amd as pkv
    return pkv


def _both(spec, seed, **extra_params):
    torch = torch_mod()
    pkv = _pkv()
    db = make_device_batch(spec, seed=seed, layers=1)
    lay = db.layout
    params = pkv.Params(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                        max_kv_len=lay.req_to_token.shape[1], **extra_params)
    plan = pkv.plan_metadata(params, pkv.PKV_DECODE, db.seq_lens)
    pkv.kv_store(params, db.k_pools[0], db.v_pools[0], db.k_new[0], db.v_new[0], db.new_slots)
    n = max(params.decode_q_len, 1)
    rows = spec.batch * n
    sc = dict(sfq=db.sfq, sfk=db.sfk, sfv=db.sfv) if db.sfq is not None else {}
    lse_a = torch.empty((rows, spec.num_q_heads), dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    out_a = pkv.attn_decode(params, db.q, db.k_pools[0], db.v_pools[0], db.req_to_token, db.seq_lens, plan,
                            lse=lse_a, **sc)
    out_b = torch.empty_like(out_a)
    pkv.attn_decode_noalloc(params, db.q, db.k_pools[0], db.v_pools[0], db.req_to_token, db.seq_lens, plan,
                            out_b, lse=lse_b, **sc)
    torch.cuda.synchronize()
    print(f"{spec.name}: scratch {plan.scratch_bytes} bytes of {pkv.STATIC_SCRATCH_BYTES}", flush=True)
    assert plan.scratch_bytes <= pkv.STATIC_SCRATCH_BYTES
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), spec.name
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32)), spec.name


def test_noalloc_decode_equals_decode_twice_second_smaller():
    """The full bf16 decode batch, then a smaller one (8 requests) on the same
    static scratch, each bit-identical to the decode with a caller scratch."""
    _both(SPECS["decode_bf16"], 0)
    _both(Spec("noalloc_small", "decode", 8, 32, 8, 128, 16, (100, 1500), 1), 1)


def test_noalloc_8bit_and_multi_token_decode():
    """The 8-bit decode workload (E4M3 Sage) and four tokens per request."""
    _both(SPECS["decode_fp8"], 0, kv_dtype=_pkv().PKV_FP8_E4M3, q_block=1, k_block=64)
    _both(Spec("noalloc_n4", "decode", 16, 32, 8, 128, 16, (200, 3000), 4), 2, decode_q_len=4)


def test_noalloc_rejects_scratch_beyond_the_static_size():
    """A batch whose split partials need more than the static scratch holds is
    rejected with PKV_EWORKSPACE on the host; nothing is launched."""
    torch = torch_mod()
    pkv = _pkv()
    B, hq, hkv, d = 256, 64, 8, 128
    params = pkv.Params(hq, hkv, d, 16, max_kv_len=1024, decode_q_len=16)
    _, scratch = pkv.workspace_size(params, pkv.PKV_DECODE, B)
    assert scratch > pkv.STATIC_SCRATCH_BYTES
    seq = torch.full((B,), 1024, dtype=torch.int32, device="cuda")
    plan = pkv.plan_metadata(params, pkv.PKV_DECODE, seq)
    q = torch.zeros((B * 16, hq, d), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((16, hkv, d), dtype=torch.bfloat16, device="cuda")
    rtt = torch.zeros((B, 1024), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(pkv.PkvError) as ei:
        pkv.attn_decode_noalloc(params, q, pool, pool, rtt, seq, plan, out)
    assert ei.value.code == pkv.PKV_EWORKSPACE and "static scratch" in ei.value.msg
    torch.cuda.synchronize()
