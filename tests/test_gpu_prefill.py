"""GPU parity of paged_prefill_attn (MFMA chunked prefill, decode rows
allowed in the same call) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_98_amd import binding as pkv
from paged_kv_cache_98_amd import workloads as W
from tests.gpu_common import bf16_parity, oracle_prefill_sample, parity

pytestmark = pytest.mark.gpu

DEV = "cuda"

# (context length, query rows): a whole prompt (positions 0..36), ragged
# chunks at offsets that straddle 64-key tiles, decode rows and an empty one
CHUNKS = [(37, 37), (141, 100), (300, 200), (64, 1), (520, 129), (1000, 64), (77, 0), (700, 1)]


def run_prefill(b, causal=True, out_dtype=torch.float32):
    w = b.workload
    return pkv.paged_prefill_attn(b.q, b.cu_q_lens, b.k_cache, b.v_cache, b.block_table,
                                  b.context_lens, w.scale, max_context_len=w.max_context_len,
                                  max_q_len=w.max_q_len, causal=causal, out_dtype=out_dtype)


def oracle_prefill(bc, causal=True):
    w = bc.workload
    return oracle.paged_attention(bc.q, bc.k_cache, bc.v_cache, bc.block_table, bc.context_lens,
                                  w.scale, cu_q_lens=bc.cu_q_lens, causal=causal)


def chunk_workload(group, bs, hkv=2, seed=3000, chunks=CHUNKS, shared_prefix=0):
    ctx = [c for c, _ in chunks]
    ql = [q for _, q in chunks]
    return W.make_workload(f"chunks_g{group}_bs{bs}", ctx, ql, num_q_heads=hkv * group,
                           num_kv_heads=hkv, block_size=bs, shared_prefix=shared_prefix,
                           seed=seed + 10 * group + bs)


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("group", [1, 2, 4, 8, 16])
def test_prefill_chunks(bs, group):
    w = chunk_workload(group, bs)
    bc = W.materialize(w, logical=True, poison=True)
    out = run_prefill(bc.to(DEV))
    torch.cuda.synchronize()
    parity(out, oracle_prefill(bc), what=w.name)


def test_prefill_non_causal():
    w = chunk_workload(4, 16, seed=3100)
    bc = W.materialize(w, logical=True, poison=True)
    out = run_prefill(bc.to(DEV), causal=False)
    torch.cuda.synchronize()
    parity(out, oracle_prefill(bc, causal=False), what="non-causal")


def test_prefill_bf16_output():
    w = chunk_workload(4, 16, seed=3200)
    bc = W.materialize(w, logical=True, poison=True)
    b = bc.to(DEV)
    out16 = run_prefill(b, out_dtype=torch.bfloat16)
    out32 = run_prefill(b)
    bf16_parity(out16, out32, oracle_prefill(bc), what="prefill bf16 out",
                fp32_err=1e-3, min_within=0.95)


def test_prefill_shared_prefix_mixed_small():
    """Scaled-down mixed batch: 2 chunks + 6 decodes over a shared 160-token
    prefix (every block table maps it to the same physical blocks)."""
    w = W.mixed_prefill(num_chunks=2, chunk=96, num_decodes=6, prefix=160, tail_lo=5,
                        tail_hi=300, seed=3300)
    bc = W.materialize(w, logical=True, poison=True)
    assert torch.equal(bc.block_table[0, :10], bc.block_table[5, :10])
    out = run_prefill(bc.to(DEV))
    torch.cuda.synchronize()
    parity(out, oracle_prefill(bc), what=w.name)


def test_prefill_deterministic_and_permutation_invariant():
    w = chunk_workload(4, 16, seed=3400)
    bc = W.materialize(w, logical=True, poison=True)
    b = bc.to(DEV)
    o1, o2 = run_prefill(b), run_prefill(b)
    op = run_prefill(W.permute_pool(bc, 5).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, op)


def test_prefill_full_size_mixed():
    """The full chunked-prefill + decode batch (4 x 512 queries, 128 decodes,
    shared 800-token prefix) in the launch configuration the benchmark
    times (chunks and decodes in one grid); the oracle checks all 2176 query
    rows and every head, and a second call gives the same bits."""
    w = W.mixed_prefill()
    print(f"[case] {w.describe()}", flush=True)
    b = W.materialize(w, device=DEV, poison=True)
    out = run_prefill(b)
    again = run_prefill(b)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    assert torch.equal(out, again), "mixed call not bitwise deterministic"
    ref, rows = oracle_prefill_sample(b, list(range(w.num_seqs)))
    assert rows.tolist() == list(range(w.total_q))
    parity(out, ref, what=f"mixed full size, all {w.total_q} rows")


@pytest.mark.parametrize("num_seqs,group,hkv", [(280, 4, 2), (130, 8, 1)])
def test_prefill_many_ragged_chunks(num_seqs, group, hkv):
    """Hundreds of ragged chunks (0 to 48 rows, decode rows among them) in
    one grid call small enough that its workgroups take their items in the
    heavy/light pairing order, which ranks every XCD run's items over the
    call's sequences (more of them than a workgroup has threads)."""
    rng = np.random.default_rng(3200 + num_seqs)
    ql = [int(x) for x in rng.integers(0, 49, num_seqs)]
    ql[7] = 48  # max_q_len * G > 128: the grid kernel, not stream-K
    ql[11], ql[12] = 1, 0
    ctx = [q + int(p) for q, p in zip(ql, rng.integers(0, 300, num_seqs))]
    w = W.make_workload(f"many_chunks_{num_seqs}_g{group}", ctx, ql, num_q_heads=hkv * group,
                        num_kv_heads=hkv, block_size=16, seed=3300 + num_seqs)
    P = 128 // group
    per_xcd = -(-(sum(ql) // P + num_seqs) * hkv // 8)
    assert per_xcd <= 4 * 32, "the case is meant to take the pairing order"
    print(f"[many chunks] {w.name} rows {sum(ql)} items per XCD {per_xcd}", flush=True)
    bc = W.materialize(w, logical=True, poison=True)
    out = run_prefill(bc.to(DEV))
    torch.cuda.synchronize()
    parity(out, oracle_prefill(bc), what=w.name)
