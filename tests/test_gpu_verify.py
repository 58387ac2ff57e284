"""GPU parity of speculative-decoding verification: a few causal query rows
per sequence (the last accepted token and the drafts) through
paged_prefill_attn, against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_98_amd import binding as pkv
from paged_kv_cache_98_amd import workloads as W
from tests.gpu_common import oracle_prefill_sample, parity

pytestmark = pytest.mark.gpu

DEV = "cuda"

# (context length including the new rows, new rows): row groups that end at,
# straddle and start tile and block edges, and whole prompts of 2..8 tokens
VERIFY = [(6, 6), (7, 6), (63, 6), (64, 6), (65, 6), (66, 6), (69, 6), (128, 2), (129, 3),
          (130, 8), (1000, 6), (4097, 6), (2, 2), (512, 5), (513, 4), (300, 7)]


def run(b):
    w = b.workload
    return pkv.paged_prefill_attn(b.q, b.cu_q_lens, b.k_cache, b.v_cache, b.block_table,
                                  b.context_lens, w.scale, max_context_len=w.max_context_len,
                                  max_q_len=w.max_q_len, causal=True)


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("group", [1, 4, 8])
def test_verify_rows_around_edges(bs, group):
    hkv = 2
    w = W.make_workload(f"verify_g{group}_bs{bs}", [c for c, _ in VERIFY], [q for _, q in VERIFY],
                        num_q_heads=hkv * group, num_kv_heads=hkv, block_size=bs,
                        seed=4000 + group + bs)
    bc = W.materialize(w, logical=True, poison=True)
    ref = oracle.paged_attention(bc.q, bc.k_cache, bc.v_cache, bc.block_table, bc.context_lens,
                                 w.scale, cu_q_lens=bc.cu_q_lens, causal=True)
    out = run(bc.to(DEV))
    torch.cuda.synchronize()
    parity(out, ref, what=w.name)


def test_verify_full_batch():
    """The 64-sequence verify batch (6 rows each) in the launch configuration
    the benchmark times; every row of every sequence against the oracle."""
    w = W.spec_verify()
    print(f"[case] {w.describe()}", flush=True)
    b = W.materialize(w, device=DEV, poison=True)
    out = run(b)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    ref, rows = oracle_prefill_sample(b, list(range(w.num_seqs)))
    assert rows.tolist() == list(range(w.total_q))
    parity(out, ref, what=f"verify full batch, all {w.total_q} rows")


def test_verify_split_variants():
    """Stream-K chunks on the chunk kernel (items shared between workers,
    merged after it) in every setting they meet: 16 query heads per KV head
    with 8 rows (128 columns, too wide for the rows path), non-causal, bf16
    output, single-row sequences in the same call (whose decode workspace
    sits in front of the stream-K part), and bitwise determinism."""
    from tests.gpu_common import bf16_parity
    cases = [(3000, 8), (2500, 1), (40, 3), (1800, 2), (4100, 8), (700, 1), (129, 4)]
    w = W.make_workload("verify_split_g16", [c for c, _ in cases], [q for _, q in cases],
                        num_q_heads=32, num_kv_heads=2, block_size=16, seed=4100)
    bc = W.materialize(w, logical=True, poison=True)
    b = bc.to(DEV)
    need = pkv.prefill_workspace_bytes(w.num_seqs, w.total_q, w.max_q_len, 32, 2,
                                       w.max_context_len)
    assert need > pkv.decode_workspace_bytes(w.num_seqs, 32, 2, w.max_context_len)
    for causal in (True, False):
        ref = oracle.paged_attention(bc.q, bc.k_cache, bc.v_cache, bc.block_table,
                                     bc.context_lens, w.scale, cu_q_lens=bc.cu_q_lens,
                                     causal=causal)
        call = lambda dt: pkv.paged_prefill_attn(
            b.q, b.cu_q_lens, b.k_cache, b.v_cache, b.block_table, b.context_lens, w.scale,
            max_context_len=w.max_context_len, max_q_len=w.max_q_len, causal=causal,
            out_dtype=dt)
        o32 = call(torch.float32)
        o32b = call(torch.float32)
        o16 = call(torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(o32, o32b)
        parity(o32, ref, what=f"split g16 causal={causal}")
        bf16_parity(o16, o32, ref, what=f"split g16 bf16 causal={causal}",
                    fp32_err=1e-3, min_within=0.95)


@pytest.mark.parametrize("name,hq,hkv,cases", [
    # the widest calls the stream-K path takes: 128 query columns per KV head
    ("sk_g16_r8", 32, 2, [(3000, 8), (50, 8), (900, 1), (2100, 5), (8, 8), (77, 0)]),
    ("sk_g4_r32", 16, 4, [(2000, 32), (32, 32), (700, 1), (4097, 17), (100, 0), (65, 32)]),
    ("sk_g1_r128", 2, 2, [(1500, 128), (128, 128), (3000, 77), (129, 1)]),
    # one long item over every worker: more pieces than the merge's 64 lanes
    # (on the rows path with 24 columns, on the chunk kernel with 96)
    ("sk_one_long", 4, 1, [(100000, 6)]),
    ("sk_one_long_g16", 16, 1, [(100000, 6)]),
])
def test_streamk_widths_and_many_pieces(name, hq, hkv, cases):
    print(f"[stream-K] {name}", flush=True)
    w = W.make_workload(name, [c for c, _ in cases], [q for _, q in cases], num_q_heads=hq,
                        num_kv_heads=hkv, block_size=16, seed=4200 + hq + hkv)
    assert pkv.prefill_workspace_bytes(w.num_seqs, w.total_q, w.max_q_len, hq, hkv,
                                       w.max_context_len) > 0
    bc = W.materialize(w, logical=True, poison=True)
    ref = oracle.paged_attention(bc.q, bc.k_cache, bc.v_cache, bc.block_table, bc.context_lens,
                                 w.scale, cu_q_lens=bc.cu_q_lens, causal=True)
    out = run(bc.to(DEV))
    torch.cuda.synchronize()
    parity(out, ref, what=name)


@pytest.mark.parametrize("group,rows", [(2, 24), (8, 16), (16, 8)])
def test_streamk_merge_query_heads_grouped(group, rows):
    """With at least half as many (sequence, KV head) items as stream-K
    workers, the merge kernel takes several query heads of one KV head per
    wave (2 for G = 2, 4 for G = 8 and 16, so the waves of G = 8 and 16
    start inside a KV head's group of query heads).  64 sequences x 8 KV
    heads, rows and contexts around tile edges, most items cut between two
    workers."""
    rng = np.random.default_rng(4300 + group)
    edges = [63, 64, 65, 127, 128, 129, 511, 512, 513, 1023, 1024, 1025]
    ctx = [int(c) for c in rng.integers(rows, 1300, 64)]
    ctx[:len(edges)] = edges
    ql = [int(q) for q in rng.integers(1, rows + 1, 64)]
    ql[0], ql[1], ql[5] = rows, 1, rows
    w = W.make_workload(f"sk_merge_g{group}", ctx, ql, num_q_heads=8 * group, num_kv_heads=8,
                        block_size=16, seed=4300 + group)
    print(f"[stream-K merge] {w.name} rows {w.total_q}", flush=True)
    bc = W.materialize(w, logical=True, poison=True)
    ref = oracle.paged_attention(bc.q, bc.k_cache, bc.v_cache, bc.block_table, bc.context_lens,
                                 w.scale, cu_q_lens=bc.cu_q_lens, causal=True)
    b = bc.to(DEV)
    o1, o2 = run(b), run(b)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    parity(o1, ref, what=w.name)


def test_streamk_merge_query_heads_grouped_tree():
    """The grouped merge under token-tree masks: 64 sequences x 8 KV heads,
    G = 8, 16-node trees."""
    from oracle import tree
    rng = np.random.default_rng(4400)
    ctx = [int(c) for c in rng.integers(16, 1300, 64)]
    w = W.make_workload("sk_merge_tree_g8", ctx, [16] * 64, num_q_heads=64, num_kv_heads=8,
                        block_size=16, seed=4400)
    bc = W.materialize(w, logical=True, poison=True)
    masks = W.tree_masks(w)
    bits = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    ref = tree.paged_attention_tree(bits(bc.q), bits(bc.k_cache), bits(bc.v_cache),
                                    bc.block_table.numpy(), bc.context_lens.numpy(),
                                    bc.cu_q_lens.numpy(), masks.numpy().view(np.uint64), w.scale)
    b = bc.to(DEV)
    out = pkv.paged_prefill_attn(b.q, b.cu_q_lens, b.k_cache, b.v_cache, b.block_table,
                                 b.context_lens, w.scale, max_context_len=w.max_context_len,
                                 max_q_len=w.max_q_len, tree_mask=masks.to(DEV))
    torch.cuda.synchronize()
    parity(out, ref, what=w.name)


def rows_cases(rows):
    """(context length, rows) for the rows path: full row groups ending at,
    straddling and starting tile (16-key) and block edges, a decode row and
    an empty sequence in the same call, whole prompts."""
    ctx = [rows, rows + 1, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 100, 1000, 4097]
    cases = [(c, rows) for c in ctx if c >= rows]
    return cases + [(500, 1), (70, 0), (129, max(rows - 1, 1)), (2, min(rows, 2))]


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_rows_path_groups_and_edges(bs, group):
    """Chunks of at most 16 rows and 64 (row, head) columns per KV head take
    the decode kernel's matrix-core tile (the rows path): one wave per KV
    head up to 16 columns, two or four sharing the KV head's tiles through
    LDS beyond; 16 rows at one query head per KV head down to 8 at eight,
    causal and not, against the fp64 oracle."""
    rows, hkv = min(16, 64 // group), 2
    cases = rows_cases(rows)
    w = W.make_workload(f"rows_g{group}_bs{bs}", [c for c, _ in cases], [q for _, q in cases],
                        num_q_heads=hkv * group, num_kv_heads=hkv, block_size=bs,
                        seed=4400 + group + bs)
    print(f"[rows path] {w.name}", flush=True)
    bc = W.materialize(w, logical=True, poison=True)
    b = bc.to(DEV)
    for causal in (True, False):
        ref = oracle.paged_attention(bc.q, bc.k_cache, bc.v_cache, bc.block_table,
                                     bc.context_lens, w.scale, cu_q_lens=bc.cu_q_lens,
                                     causal=causal)
        out = pkv.paged_prefill_attn(b.q, b.cu_q_lens, b.k_cache, b.v_cache, b.block_table,
                                     b.context_lens, w.scale, max_context_len=w.max_context_len,
                                     max_q_len=w.max_q_len, causal=causal)
        torch.cuda.synchronize()
        parity(out, ref, what=f"{w.name} causal={causal}")


def test_rows_path_split_bf16_out_and_determinism():
    """The rows path with sequences cut between stream-K workers (few long
    contexts) and 8 KV heads: records per (worker, row, head) merged after
    the tile kernel; bf16 output equals the fp32 output rounded; bitwise
    determinism."""
    from tests.gpu_common import bf16_parity
    cases = [(30000, 4), (2500, 4), (40, 3), (18000, 2), (700, 1), (9000, 4), (5, 4)]
    w = W.make_workload("rows_split_g4", [c for c, _ in cases], [q for _, q in cases],
                        num_q_heads=32, num_kv_heads=8, block_size=16, seed=4500)
    print(f"[rows path split] {w.name}", flush=True)
    bc = W.materialize(w, logical=True, poison=True)
    b = bc.to(DEV)
    ref = oracle.paged_attention(bc.q, bc.k_cache, bc.v_cache, bc.block_table, bc.context_lens,
                                 w.scale, cu_q_lens=bc.cu_q_lens, causal=True)
    call = lambda dt: pkv.paged_prefill_attn(
        b.q, b.cu_q_lens, b.k_cache, b.v_cache, b.block_table, b.context_lens, w.scale,
        max_context_len=w.max_context_len, max_q_len=w.max_q_len, causal=True, out_dtype=dt)
    o32, o32b, o16 = call(torch.float32), call(torch.float32), call(torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o32, o32b)
    parity(o32, ref, what=w.name)
    bf16_parity(o16, o32, ref, what=w.name + " bf16 out", fp32_err=1e-3, min_within=0.95)


@pytest.mark.parametrize("hkv,group,rows", [(16, 1, 16), (16, 4, 4), (3, 2, 8), (5, 8, 2),
                                            (3, 4, 8), (5, 4, 16), (16, 8, 8)])
def test_rows_path_kv_head_layouts(hkv, group, rows):
    """The rows path's workgroups: 16 KV heads in two groups of 8 waves, KV
    head counts that are not powers of two, and the shared-staging
    workgroups (two KV heads of two waves, or one of four) with a last group
    short of a KV head."""
    cases = [(2000, rows), (77, rows), (16, rows), (900, 1)]
    w = W.make_workload(f"rows_hkv{hkv}_g{group}", [c for c, _ in cases], [q for _, q in cases],
                        num_q_heads=hkv * group, num_kv_heads=hkv, block_size=16,
                        seed=4600 + hkv + group)
    print(f"[rows path heads] {w.name}", flush=True)
    bc = W.materialize(w, logical=True, poison=True)
    ref = oracle.paged_attention(bc.q, bc.k_cache, bc.v_cache, bc.block_table, bc.context_lens,
                                 w.scale, cu_q_lens=bc.cu_q_lens, causal=True)
    out = run(bc.to(DEV))
    torch.cuda.synchronize()
    parity(out, ref, what=w.name)
