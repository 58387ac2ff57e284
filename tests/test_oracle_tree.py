"""The token-tree oracle pinned: chain masks reproduce the C oracle's causal
attention, a star tree differs from it exactly where it should, and every
tree node equals a plain
decode of the sequence made of the cached context followed by the node's
own path (laid out contiguously, so the tree machinery plays no part)."""
import numpy as np
import pytest

import oracle
from oracle import tree


def bf16_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def make_case(seed, bs=16, hq=8, hkv=2, ctx=(40, 77, 16, 130), lq=(6, 9, 16, 1)):
    rng = np.random.default_rng(seed)
    d = 128
    nblk = [-(-c // bs) for c in ctx]
    nb = sum(nblk) + 3
    k = bf16_bits(rng.standard_normal((nb, bs, hkv, d)))
    v = bf16_bits(rng.standard_normal((nb, bs, hkv, d)))
    perm = rng.permutation(nb)
    bt = np.full((len(ctx), max(nblk)), -1, np.int32)
    base = 0
    for i, n in enumerate(nblk):
        bt[i, :n] = perm[base:base + n]
        base += n
    cu = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    q = bf16_bits(rng.standard_normal((int(cu[-1]), hq, d)) * 0.5)
    return q, k, v, bt, np.array(ctx, np.int32), cu, rng


def test_pin_chain_masks_are_causal():
    q, k, v, bt, ctx, cu, _ = make_case(1)
    got = tree.paged_attention_tree(q, k, v, bt, ctx, cu, tree.chain_masks(cu), 0.0884)
    ref = oracle.paged_attention(q, k, v, bt, ctx, 0.0884, cu_q_lens=cu, causal=True)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_pin_star_tree_sees_root_and_itself():
    """A star tree (every node a child of node 0) sees the root and itself;
    that is a decode of context + root + node."""
    q, k, v, bt, ctx, cu, _ = make_case(2, ctx=(50,), lq=(7,))
    masks = np.array([1] + [1 | (1 << r) for r in range(1, 7)], dtype=np.uint64)
    got = tree.paged_attention_tree(q, k, v, bt, ctx, cu, masks, 0.1)
    # rows 0 and 1: a star node at position 1 sees the same keys as causal row 1
    ref = oracle.paged_attention(q, k, v, bt, ctx, 0.1, cu_q_lens=cu, causal=True)
    assert np.allclose(got[:2], ref[:2], rtol=1e-12, atol=1e-12)
    assert not np.allclose(got[2:], ref[2:], rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_pin_each_node_is_a_decode_of_its_path(seed):
    bs = 16
    q, k, v, bt, ctx, cu, rng = make_case(seed, bs=bs)
    masks = tree.random_tree_masks(cu, rng)
    got = tree.paged_attention_tree(q, k, v, bt, ctx, cu, masks, 0.0884)
    nb, _, hkv, d = k.shape
    for i in range(len(ctx)):
        n, lq = int(ctx[i]), int(cu[i + 1] - cu[i])
        pos0 = n - lq
        ids = bt[i, :-(-n // bs)]
        rows_k = k[ids].reshape(-1, hkv, d)[:n]
        rows_v = v[ids].reshape(-1, hkv, d)[:n]
        for r in range(lq):
            m = int(masks[cu[i] + r])
            keep = list(range(pos0)) + [pos0 + j for j in range(lq) if (m >> j) & 1]
            # the path as its own contiguous sequence, in fresh blocks
            sk, sv = rows_k[keep], rows_v[keep]
            nk = len(keep)
            nbk = -(-nk // bs)
            pk = np.zeros((nbk, bs, hkv, d), np.uint16)
            pv = np.zeros_like(pk)
            pk.reshape(-1, hkv, d)[:nk] = sk
            pv.reshape(-1, hkv, d)[:nk] = sv
            ref = oracle.paged_attention(q[cu[i] + r:cu[i] + r + 1], pk, pv,
                                         np.arange(nbk, dtype=np.int32)[None, :],
                                         np.array([nk], np.int32), 0.0884)
            assert np.allclose(got[cu[i] + r], ref[0], rtol=1e-12, atol=1e-12), (i, r)


def test_pin_masks_must_name_ancestors_only():
    q, k, v, bt, ctx, cu, _ = make_case(6, ctx=(40,), lq=(3,))
    with pytest.raises(ValueError):
        tree.paged_attention_tree(q, k, v, bt, ctx, cu, np.array([1, 3, 15], np.uint64), 0.1)
