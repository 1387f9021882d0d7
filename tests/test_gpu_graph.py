"""A whole decode step (the plan, every layer's K/V store, every layer's
attention) captured once as a HIP graph and replayed with new sequence
lengths in the same static buffers: the work list is rebuilt on the device
at each replay, and every replay equals the eager run of the same step bit
for bit.  The SGLang basics page names graph capture of the decode forward
(and buffers kept at fixed addresses for it) as part of the backend."""
import numpy as np
import pytest

from gpu_util import assert_bf16_close, host, torch_mod
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
