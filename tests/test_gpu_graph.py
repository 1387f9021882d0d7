"""A whole decode step (the plan, every layer's K/V store, every layer's
attention) captured once as a HIP graph and replayed with new sequence
lengths in the same static buffers: the work list is rebuilt on the device
at each replay, and every replay equals the eager run of the same step bit
for bit.  The SGLang basics page names graph capture of the decode forward
(and buffers kept at fixed addresses for it) as part of the backend."""
import numpy as np
import pytest

from gpu_util import FP8_REL_L2, assert_bf16_close, check_rel_l2, host, kv_dtype_of, qk_codes_of, rel_l2, torch_mod
from workloads import Spec, make_device_batch

import oracle

pytestmark = pytest.mark.gpu


def _pkv():
    import flashattention_paged_kv_amd as pkv
    return pkv


def _bits(t):
    torch = torch_mod()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_decode_step_graph_replays_equal_eager_runs():
    torch = torch_mod()
    pkv = _pkv()
    spec = Spec("graph_decode", "decode", 24, 32, 8, 128, 16, (200, 3000), 1)
    layers = 2
    db = make_device_batch(spec, seed=3, layers=layers)
    lay = db.layout
    B, Hq, d = spec.batch, spec.num_q_heads, spec.head_dim
    params = pkv.Params(Hq, spec.num_kv_heads, d, spec.page_size, max_kv_len=lay.req_to_token.shape[1])
    ws_bytes, sc_bytes = pkv.workspace_size(params, pkv.PKV_DECODE, B)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    scratch = torch.empty(max(sc_bytes, 16), dtype=torch.uint8, device="cuda")
    seq = db.seq_lens.clone()  # the static length buffer the graph reads
    outs = [torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    lses = [torch.empty((B, Hq), dtype=torch.float32, device="cuda") for _ in range(layers)]

    def step():
        plan = pkv.plan_metadata(params, pkv.PKV_DECODE, seq, workspace=ws)
        for l in range(layers):
            pkv.kv_store(params, db.k_pools[l], db.v_pools[l], db.k_new[l], db.v_new[l], db.new_slots)
        for l in range(layers):
            pkv.attn_decode(params, db.q, db.k_pools[l], db.v_pools[l], db.req_to_token, seq, plan,
                            scratch=scratch, out=outs[l], lse=lses[l])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # eager warm-up off the capture: library loaded, occupancy cached
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    rng = np.random.default_rng(0)
    full = lay.seq_lens.astype(np.int64)
    for rep in range(4):
        lens = full if rep == 0 else np.maximum(1, full - rng.integers(0, 400, size=B))
        seq.copy_(torch.from_numpy(lens.astype(np.int32)))
        graph.replay()
        torch.cuda.synchronize()
        got = [(o.clone(), s.clone()) for o, s in zip(outs, lses)]
        for o, s in zip(outs, lses):  # poison, so the eager run must rewrite everything
            o.fill_(float("nan"))
            s.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        for l in range(layers):
            assert torch.equal(_bits(got[l][0]), _bits(outs[l])), (rep, l)
            assert torch.equal(_bits(got[l][1]), _bits(lses[l])), (rep, l)
        # and the replay is the attention of those lengths (layer 0, sampled requests)
        if rep == 0:
            k0 = db.k_pools[0].float().cpu().numpy()
            v0 = db.v_pools[0].float().cpu().numpy()
            qh = db.q.float().cpu().numpy()
        for b in (0, B // 2, B - 1):
            ro, _ = oracle.paged_attention(qh[b:b + 1], k0, v0, lay.req_to_token[b:b + 1], lens[b:b + 1],
                                           np.arange(2))
            assert_bf16_close(host(got[0][0])[b:b + 1], ro, f"replay {rep} request {b}")


def _capture(step, torch):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # eager warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = step()
    torch.cuda.synchronize()
    return graph, captured


@pytest.mark.parametrize("dtype", ["fp8", "int8"])
def test_block_sparse_step_graph_replays_equal_eager_runs(dtype):
    """The compacted table, the plan over its lengths and an 8-bit decode
    (E4M3, or INT8 Q/K) captured once; replays with new block lists in the
    same buffers."""
    from workloads import block_mask
    torch = torch_mod()
    pkv = _pkv()
    spec = Spec("graph_sparse", "decode", 6, 16, 4, 128, 16, (300, 4000), 1, dtype=dtype, k_block=64)
    db = make_device_batch(spec, seed=4, layers=1)
    lay = db.layout
    B, Hq, d, bs = spec.batch, spec.num_q_heads, spec.head_dim, 128
    params = pkv.Params(Hq, spec.num_kv_heads, d, spec.page_size, max_kv_len=lay.req_to_token.shape[1],
                        kv_dtype=kv_dtype_of(pkv, spec), q_block=1, k_block=spec.k_block)
    ws_bytes, sc_bytes = pkv.workspace_size(params, pkv.PKV_DECODE, B)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    scratch = torch.empty(max(sc_bytes, 16), dtype=torch.uint8, device="cuda")
    cap = int(sum(-(-int(L) // bs) for L in lay.seq_lens))  # room for every block
    indptr = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    indices = torch.zeros(cap, dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")

    def load_mask(density, seed):
        ip, ix = block_mask(lay.seq_lens, bs, density, np.random.default_rng(seed))
        indptr.copy_(torch.from_numpy(ip))
        indices.zero_()
        indices[:len(ix)].copy_(torch.from_numpy(ix))
        return ip, ix

    def step():
        srtt, slens, ssfk = pkv.block_sparse_table(params, db.seq_lens, db.req_to_token, indptr, indices, bs,
                                                   sfk=db.sfk)
        plan = pkv.plan_metadata(params, pkv.PKV_DECODE, slens, workspace=ws)
        pkv.attn_decode(params, db.q, db.k_pools[0], db.v_pools[0], srtt, slens, plan, scratch=scratch, out=out,
                        lse=lse, sfq=db.sfq, sfk=ssfk, sfv=db.sfv)
        return slens

    load_mask(0.3, 0)
    graph, _ = _capture(step, torch)
    q8, k8, v8 = db.q.cpu().numpy(), db.k_pools[0].cpu().numpy(), db.v_pools[0].cpu().numpy()
    sfq, sfk, sfv = db.sfq.cpu().numpy(), db.sfk.cpu().numpy(), db.sfv.cpu().numpy()
    for rep, density in enumerate((0.3, 0.1, 0.6, 1.0)):
        ip, ix = load_mask(density, rep)
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        assert torch.equal(_bits(got_o), _bits(out)) and torch.equal(_bits(got_l), _bits(lse)), rep
        ro, _ = oracle.block_sparse_sage_decode(q8, k8, v8, lay.req_to_token, lay.seq_lens, ip, ix, bs, sfq, sfk,
                                                sfv, spec.k_block, qk_codes=qk_codes_of(spec))
        check_rel_l2(host(got_o), ro, f"graph replay {rep}")


def test_extend_step_graph_replays_equal_eager_runs():
    """The extend plan, the K/V store and the attention captured once; replays
    with new cached lengths in the same buffers."""
    torch = torch_mod()
    pkv = _pkv()
    spec = Spec("graph_extend", "extend", 5, 16, 4, 128, 16, (100, 900), (20, 300))
    db = make_device_batch(spec, seed=5, layers=1)
    lay = db.layout
    T, Hq, d = lay.total_q, spec.num_q_heads, spec.head_dim
    params = pkv.Params(Hq, spec.num_kv_heads, d, spec.page_size, max_kv_len=lay.req_to_token.shape[1])
    ws_bytes, _ = pkv.workspace_size(params, pkv.PKV_EXTEND, spec.batch, T)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    seq = db.seq_lens.clone()
    out = torch.empty((T, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")

    def step():
        plan = pkv.plan_metadata(params, pkv.PKV_EXTEND, seq, db.cu_seqlens_q, total_q=T, workspace=ws)
        pkv.kv_store(params, db.k_pools[0], db.v_pools[0], db.k_new[0], db.v_new[0], db.new_slots)
        pkv.attn_extend(params, db.q, db.k_pools[0], db.v_pools[0], db.req_to_token, seq, db.cu_seqlens_q, plan,
                        out=out, lse=lse)

    graph, _ = _capture(step, torch)
    rng = np.random.default_rng(1)
    full = lay.seq_lens.astype(np.int64)
    n = lay.new_lens.astype(np.int64)
    k0, v0, qh = (t.float().cpu().numpy() for t in (db.k_pools[0], db.v_pools[0], db.q))
    for rep in range(3):
        # shorter cached prefixes (never below zero): the rows attend to fewer keys
        lens = full if rep == 0 else np.maximum(n, full - rng.integers(0, 100, size=spec.batch))
        seq.copy_(torch.from_numpy(lens.astype(np.int32)))
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        assert torch.equal(_bits(got_o), _bits(out)) and torch.equal(_bits(got_l), _bits(lse)), rep
        ro, _ = oracle.paged_attention(qh, k0, v0, lay.req_to_token, lens, lay.cu_seqlens_q)
        assert_bf16_close(host(got_o), ro, f"extend replay {rep}")
