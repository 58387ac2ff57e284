"""The device calls can be captured in a HIP graph: they allocate nothing
and issue no memset, so a captured step (kv_append + decode, and a stream-K
verify call with its merge) replays to the eager call's bits.  Each replay
follows eager work on the same buffers and is checked on its own."""
import pytest
import torch

from paged_kv_cache_98_amd import binding as pkv
from paged_kv_cache_98_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def replay_and_check(step, out, stream, replays=3):
    with torch.cuda.stream(stream):
        for _ in range(3):
            step()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for k in range(replays):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {k}"
        with torch.cuda.stream(stream):  # eager work between the replays
            step()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"eager call after replay {k}"


@pytest.mark.parametrize("batch,lo,hi", [(12, 100, 3000), (64, 512, 4096)])
def test_graph_decode_step(batch, lo, hi):
    """A small batch and the full 8B-shaped one (most sequences shared by
    several workers and merged by the second kernel)."""
    w = W.llama8b_decode(batch=batch, lo=lo, hi=hi, seed=6100)
    print(f"[graph decode] {w.name} batch {batch}", flush=True)
    b = W.materialize(w, device=DEV, poison=True)
    ws = torch.empty(pkv.decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                                w.max_context_len), dtype=torch.uint8, device=DEV)
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), device=DEV)
    s = torch.cuda.Stream()

    def step():
        pkv.kv_append(b.k_new, b.v_new, b.slot_mapping, b.k_cache, b.v_cache, stream=s)
        pkv.paged_decode_attn(b.q, b.k_cache, b.v_cache, b.block_table, b.context_lens, w.scale,
                              max_context_len=w.max_context_len, out=out, workspace=ws, stream=s)

    replay_and_check(step, out, s)


def test_graph_streamk_verify_call():
    cases = [(3000, 6), (2500, 1), (40, 3), (4100, 6), (700, 5)]
    w = W.make_workload("graph_verify", [c for c, _ in cases], [q for _, q in cases],
                        num_q_heads=16, num_kv_heads=4, block_size=16, seed=6200)
    print(f"[graph verify] {w.name}", flush=True)
    b = W.materialize(w, device=DEV, poison=True)
    need = pkv.prefill_workspace_bytes(w.num_seqs, w.total_q, w.max_q_len, w.num_q_heads,
                                       w.num_kv_heads, w.max_context_len)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.empty((w.total_q, w.num_q_heads, w.head_dim), device=DEV)
    s = torch.cuda.Stream()

    def step():
        pkv.paged_prefill_attn(b.q, b.cu_q_lens, b.k_cache, b.v_cache, b.block_table,
                               b.context_lens, w.scale, max_context_len=w.max_context_len,
                               max_q_len=w.max_q_len, causal=True, out=out, workspace=ws,
                               stream=s)

    replay_and_check(step, out, s)
