"""The three entry points inside a captured hipGraph (torch.cuda.CUDAGraph):
they allocate nothing, set no memory with memset nodes and never synchronize
with the host, so a captured select + forward + backward replays to the same
bits as eager launches.  Each replay runs after eager work on the same
buffers and is checked against the eager results."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lengths,hk", [([700, 300, 1100], 1), ([1500, 260], 2)])
def test_graph_replays_match_eager(gpu_lib, lengths, hk):
    msa = gpu_lib
    p = synth.make_custom_pack(lengths, num_q_heads=16 * hk, num_kv_heads=hk, seed=71)
    dev = torch.device("cuda:0")
    g = lambda t: t.to(dev)
    cu = g(p.cu_seqlens)
    q, k, v, do = g(p.q), g(p.k), g(p.v), g(p.do)
    iq, ik, wq, wk = g(p.idx_q), g(p.idx_k), g(p.w_q), g(p.w_k)
    T, Hq, Hk = p.total, p.num_q_heads, p.num_kv_heads
    dims = msa.make_dims(T, len(p.lengths), p.max_seqlen, Hq, Hk)
    ws = {op: torch.empty(max(msa.msa_workspace_size(dims, op), 1), dtype=torch.uint8, device=dev)
          for op in (msa.MSA_OP_SELECT, msa.MSA_OP_FWD, msa.MSA_OP_BWD)}
    blk = torch.empty(T, Hk, 16, dtype=torch.int32, device=dev)
    o, lse = torch.empty_like(q), torch.empty(T, Hq, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    outs = (blk, o, lse, dq, dk, dv)

    def step():
        msa.msa_index_select(iq, ik, wq, wk, cu, p.max_seqlen, out=blk, workspace=ws[msa.MSA_OP_SELECT])
        msa.msa_attn_fwd(q, k, v, blk, cu, p.max_seqlen, out=o, lse=lse, workspace=ws[msa.MSA_OP_FWD])
        msa.msa_attn_bwd(q, k, v, o, lse, do, blk, cu, p.max_seqlen, dq=dq, dk=dk, dv=dv,
                         workspace=ws[msa.MSA_OP_BWD])

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, name in zip(outs, ref, ("blk", "O", "LSE", "dQ", "dK", "dV")):
            assert torch.equal(got, want), f"replay {rep}: {name}"
        print(f"[graph {lengths} hk={hk}] replay {rep} bitwise equal", flush=True)
        step()  # eager work on the same buffers between replays
        torch.cuda.synchronize()


def test_graph_replays_match_eager_fused_norm(gpu_lib):
    """The fused-norm forward and backward (msa_attn_fwd_qknorm / msa_attn_bwd_qknorm) captured together;
    the backward's outputs are allocated inside the capture, from the graph's pool, and kept alive."""
    msa = gpu_lib
    p = synth.make_custom_pack([1300, 420, 9], num_q_heads=32, num_kv_heads=2, seed=72)
    dev = torch.device("cuda:0")
    g = lambda t: t.to(dev)
    cu = g(p.cu_seqlens)
    q, k, v, do = g(p.q), g(p.k), g(p.v), g(p.do)
    gen = torch.Generator().manual_seed(73)
    wq = g((0.1 * torch.randn(128, generator=gen)).bfloat16())
    wk = g((0.1 * torch.randn(128, generator=gen)).bfloat16())
    iq, ik, iwq, iwk = g(p.idx_q), g(p.idx_k), g(p.w_q), g(p.w_k)
    T, Hq, Hk = p.total, p.num_q_heads, p.num_kv_heads
    dims = msa.make_dims(T, len(p.lengths), p.max_seqlen, Hq, Hk)
    ws = {op: torch.empty(max(msa.msa_workspace_size(dims, op), 1), dtype=torch.uint8, device=dev)
          for op in (msa.MSA_OP_FWD, msa.MSA_OP_BWD_QKNORM)}
    blk = msa.msa_index_select(iq, ik, iwq, iwk, cu, p.max_seqlen)
    o, lse = torch.empty_like(q), torch.empty(T, Hq, dtype=torch.float32, device=dev)

    def step():
        msa.msa_attn_fwd_qknorm(q, k, v, wq, wk, blk, cu, p.max_seqlen, out=o, lse=lse, workspace=ws[msa.MSA_OP_FWD])
        return msa.msa_attn_bwd_qknorm(q, k, v, wq, wk, o, lse, do, blk, cu, p.max_seqlen,
                                       workspace=ws[msa.MSA_OP_BWD_QKNORM])

    ref = [t.clone() for t in (o, lse, *step())]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grads = step()
    torch.cuda.synchronize()
    outs = (o, lse, *grads)
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, name in zip(outs, ref, ("O", "LSE", "dQ", "dK", "dV", "dw_q", "dw_k")):
            assert torch.equal(got, want), f"replay {rep}: {name}"
        print(f"[graph fused norm] replay {rep} bitwise equal", flush=True)
        step()  # eager work on the same inputs between replays
        torch.cuda.synchronize()
