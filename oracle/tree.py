"""Token-tree verification attention -- TEST INFRASTRUCTURE.

What it follows: "让 Agent 跑得快：LLM 推理服务", section 六, "Token Tree
Verification": the draft candidates form a tree (SpecInfer; EAGLE's top-k
expansion), and the target model checks the whole tree in one pass, each
node seeing the cached context and its own path of ancestors.

Readings where the page leaves a step open:
  * A sequence's Lq new tokens are the tree's nodes in topological order
    (every node after its parent), at positions ctx - Lq .. ctx - 1; node r
    carries a mask whose bit j says whether it sees new token j.  It sees
    every cached key before the new tokens.  A linear chain is the mask of
    bits 0 .. r (plain causal attention).
  * Masks only name ancestors and the node itself (bits j <= r), at most
    64 nodes per sequence.

The fp64 reference below gathers each sequence's keys through its block
table and runs the stable three-sweep softmax over the visible ones.
"""
import numpy as np


def _bf16(bits):
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def paged_attention_tree(q_bits, k_bits, v_bits, block_table, context_lens, cu_q_lens,
                         tree_mask, scale):
    """q [sum Lq, Hq, D], pools [NB, bs, Hkv, D] (bf16 bit patterns),
    tree_mask [sum Lq] uint64.  Returns [sum Lq, Hq, D] float64."""
    q = _bf16(q_bits)
    kp, vp = _bf16(k_bits), _bf16(v_bits)
    bt = np.asarray(block_table, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    masks = np.asarray(tree_mask, dtype=np.uint64)
    nb, bs, hkv, d = kp.shape
    hq = q.shape[1]
    g = hq // hkv
    out = np.zeros(q.shape, dtype=np.float64)
    for i in range(ctx.shape[0]):
        n, lq = int(ctx[i]), int(cu[i + 1] - cu[i])
        if lq == 0:
            continue
        if lq > 64 or lq > n:
            raise ValueError(f"sequence {i}: {lq} tree nodes over {n} keys")
        nblk = -(-n // bs)
        ids = bt[i, :nblk]
        k = kp[ids].reshape(nblk * bs, hkv, d)[:n]
        v = vp[ids].reshape(nblk * bs, hkv, d)[:n]
        pos0 = n - lq
        for r in range(lq):
            m = int(masks[cu[i] + r])
            if m >> (r + 1):
                raise ValueError(f"sequence {i}, node {r}: mask names a later node")
            new = [pos0 + j for j in range(lq) if (m >> j) & 1]
            keys = np.array(list(range(pos0)) + new, dtype=np.int64)
            if keys.size == 0:
                continue
            for h in range(hq):
                s = scale * (k[keys, h // g, :] @ q[cu[i] + r, h])
                p = np.exp(s - s.max())
                out[cu[i] + r, h] = (p @ v[keys, h // g, :]) / p.sum()
    return out


def chain_masks(cu_q_lens):
    """Masks of plain causal chunks: node r sees new tokens 0 .. r."""
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    out = []
    for i in range(cu.shape[0] - 1):
        out += [(1 << (r + 1)) - 1 for r in range(int(cu[i + 1] - cu[i]))]
    return np.array(out, dtype=np.uint64)


def random_tree_masks(cu_q_lens, rng):
    """A random tree per sequence: node 0 is the root, node r > 0 hangs under
    a uniformly chosen earlier node; each mask is the node's path to the root."""
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    out = []
    for i in range(cu.shape[0] - 1):
        lq = int(cu[i + 1] - cu[i])
        path = []
        for r in range(lq):
            parent = int(rng.integers(0, r)) if r > 0 else -1
            path.append((path[parent] if parent >= 0 else 0) | (1 << r))
        out += path
    return np.array(out, dtype=np.uint64)
