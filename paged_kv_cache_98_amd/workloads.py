"""Seeded synthetic inputs for paged-KV attention.

This module only builds inputs: context lengths, a shuffled physical block
pool, block tables, slot mappings and N(0, 1) bf16 tensors.  It holds none of
the attention arithmetic, so both the HIP path and the CPU oracle can be fed
from it.

Shapes follow the workloads the pages talk about:
  * Llama-3.1-8B single layer: 32 query heads, 8 KV heads, head_dim 128
    ("让 Agent 跑得快：LLM 推理服务", section 一; "LLM推理工程实战" section 3.1);
  * Llama-2-70B with GQA: 64 query heads over 8 KV heads
    ("LLM 推理优化技术全景", section "KV Cache");
  * 16-token blocks (32 as the alternative the second page reports);
  * chunked prefill in 512-token chunks with decodes riding along
    ("LLM 推理优化技术全景", section "Chunked Prefill");
  * a shared 800-token system prompt ("LLM推理工程实战" section 3.3).

Recipe (fixed, documented next to the design notes):
  * a CPU ``torch.Generator`` seeded per workload draws the context lengths
    and the block permutation;
  * Q, K, V values are fp32 N(0, 1) rounded to bf16 (round-to-nearest-even);
  * physical ids come from ``randperm(num_blocks)`` handed out in order:
    first the shared-prefix blocks, then each sequence's private blocks;
  * block tables are padded with -1;
  * in parity mode every pool slot no sequence owns is NaN, so a stray read
    shows up in the output;
  * FP8 pools (``fp8_pools``) are the bf16 pools divided by a per-cache scale
    (1/64: N(0, 1) values land well inside the E4M3 range of +-448), clamped
    to +-448 and cast with torch's own ``float8_e4m3fn`` conversion, a
    library cast independent of this package's kernels; NaN slots stay NaN
    codes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import torch

HEAD_DIM = 128
SCALE_128 = 1.0 / math.sqrt(128.0)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One batch shape.  ``q_lens[i] == 1`` is a decode row; larger values are
    a chunk of queries whose keys (including the chunk's own) are already in
    the cache.  ``context_lens[i]`` counts every key sequence i can see."""

    name: str
    context_lens: tuple
    q_lens: tuple
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    shared_prefix: int
    seed: int
    scale: float

    @property
    def num_seqs(self) -> int:
        return len(self.context_lens)

    @property
    def is_decode(self) -> bool:
        return all(x == 1 for x in self.q_lens)

    @property
    def max_context_len(self) -> int:
        return max(self.context_lens) if self.context_lens else 0

    @property
    def max_q_len(self) -> int:
        return max(self.q_lens) if self.q_lens else 0

    @property
    def total_q(self) -> int:
        return sum(self.q_lens)

    @property
    def max_blocks_per_seq(self) -> int:
        return max(1, -(-self.max_context_len // self.block_size))

    def kv_token_bytes(self) -> int:
        """Bytes of K plus V per token for one layer (bf16)."""
        return 2 * self.num_kv_heads * self.head_dim * 2

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "num_seqs": self.num_seqs,
            "num_q_heads": self.num_q_heads,
            "num_kv_heads": self.num_kv_heads,
            "head_dim": self.head_dim,
            "block_size": self.block_size,
            "num_blocks": self.num_blocks,
            "sum_context": int(sum(self.context_lens)),
            "max_context": self.max_context_len,
            "sum_q": self.total_q,
            "shared_prefix": self.shared_prefix,
            "seed": self.seed,
        }


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _pool_size(blocks_used: int, headroom: float = 0.10) -> int:
    return int(math.ceil((1.0 + headroom) * blocks_used))


def _private_blocks(ctx: Sequence[int], bs: int, shared_prefix: int) -> List[int]:
    p = shared_prefix // bs
    return [max(0, _ceil_div(c, bs) - p) for c in ctx]


def make_workload(name, context_lens, q_lens=None, *, num_q_heads=32, num_kv_heads=8,
                  head_dim=HEAD_DIM, block_size=16, shared_prefix=0, num_blocks=None,
                  seed=0, scale=None) -> Workload:
    ctx = tuple(int(c) for c in context_lens)
    ql = tuple(int(x) for x in (q_lens if q_lens is not None else [1] * len(ctx)))
    if len(ql) != len(ctx):
        raise ValueError("q_lens and context_lens differ in length")
    if shared_prefix % block_size:
        raise ValueError("the shared prefix must be block aligned")
    if any(c < shared_prefix for c in ctx) and shared_prefix:
        raise ValueError("every sequence must hold the whole shared prefix")
    used = shared_prefix // block_size + sum(_private_blocks(ctx, block_size, shared_prefix))
    nb = _pool_size(used) if num_blocks is None else int(num_blocks)
    if nb < used:
        raise ValueError("pool too small")
    return Workload(name, ctx, ql, num_q_heads, num_kv_heads, head_dim, block_size,
                    max(nb, 1), shared_prefix, seed,
                    SCALE_128 if scale is None else float(scale))


# ---------------------------------------------------------------- the configs

def tiny_decode(seed: int = 1001) -> Workload:
    """4 sequences, ctx 17/33/64/100, bs 16, 8 q heads over 2 KV heads,
    a 64-block pool."""
    return make_workload("tiny_decode", [17, 33, 64, 100], num_q_heads=8, num_kv_heads=2,
                         block_size=16, num_blocks=64, seed=seed)


def llama8b_decode(batch: int = 64, lo: int = 512, hi: int = 4096, block_size: int = 16,
                   seed: int = 1002) -> Workload:
    """Llama-3.1-8B-shaped single-layer decode: ctx ~ U[lo, hi] (integers,
    inclusive), 32 q / 8 KV heads, pool = used blocks + 10 %."""
    g = torch.Generator().manual_seed(seed)
    ctx = torch.randint(lo, hi + 1, (batch,), generator=g).tolist()
    return make_workload(f"llama8b_decode_b{batch}", ctx, block_size=block_size, seed=seed)


def long_context_decode(batch: int = 8, lo: int = 32768, hi: int = 131072,
                        block_size: int = 16, seed: int = 1003) -> Workload:
    """Long-context decode: ctx ~ U[lo, hi], 32 q / 8 KV heads."""
    g = torch.Generator().manual_seed(seed)
    ctx = torch.randint(lo, hi + 1, (batch,), generator=g).tolist()
    return make_workload(f"long_context_decode_b{batch}", ctx, block_size=block_size,
                         seed=seed)


def llama70b_decode(batch: int = 256, block_size: int = 16, median: float = 1024.0,
                    sigma: float = 1.0, lo: int = 16, hi: int = 8192,
                    seed: int = 1004) -> Workload:
    """Llama-2-70B-shaped decode with GQA (64 q / 8 KV heads): ctx =
    round(exp(ln(median) + sigma * z)), z ~ N(0, 1), clipped to [lo, hi]."""
    g = torch.Generator().manual_seed(seed)
    z = torch.randn(batch, generator=g, dtype=torch.float64)
    ctx = torch.round(torch.exp(math.log(median) + sigma * z)).clamp(lo, hi)
    return make_workload(f"llama70b_decode_b{batch}_bs{block_size}",
                         ctx.to(torch.int64).tolist(), num_q_heads=64, num_kv_heads=8,
                         block_size=block_size, seed=seed)


def spec_verify(batch: int = 64, gamma: int = 5, lo: int = 512, hi: int = 4096,
                block_size: int = 16, seed: int = 1006) -> Workload:
    """Speculative-decoding verification ("让 Agent 跑得快：LLM 推理服务",
    section 六: a draft model proposes gamma tokens, typically 5, and the
    target checks them in one parallel prefill): each sequence appends its
    last accepted token and the gamma drafts, gamma + 1 causal query rows at
    the end of a context ~ U[lo, hi] (which includes them); 8B-shaped heads."""
    g = torch.Generator().manual_seed(seed)
    ctx = torch.randint(lo, hi + 1, (batch,), generator=g).tolist()
    return make_workload(f"spec_verify_b{batch}_q{gamma + 1}", ctx, [gamma + 1] * batch,
                         block_size=block_size, seed=seed)


def spec_verify_tree(batch: int = 64, nodes: int = 16, lo: int = 512, hi: int = 4096,
                     block_size: int = 16, seed: int = 1008) -> Workload:
    """Token-tree verification ("让 Agent 跑得快：LLM 推理服务", section 六,
    Token Tree Verification): each sequence appends a tree of `nodes`
    candidate tokens (the last accepted token as its root) at the end of a
    context ~ U[lo, hi]; the masks come from tree_masks().  8B-shaped heads."""
    g = torch.Generator().manual_seed(seed)
    ctx = torch.randint(lo, hi + 1, (batch,), generator=g).tolist()
    return make_workload(f"spec_tree_b{batch}_n{nodes}", ctx, [nodes] * batch,
                         block_size=block_size, seed=seed)


def tree_masks(w: Workload, seed: int = None) -> torch.Tensor:
    """One random tree per sequence over its new tokens, in topological
    order: node 0 is the root and node r > 0 hangs under a uniformly drawn
    earlier node.  Node r's mask has bit j set for every node j on its path
    to the root, itself included.  [total_q] int64 (the uint64 bit
    patterns), on the host."""
    g = torch.Generator().manual_seed(w.seed + 77 if seed is None else seed)
    out = []
    for lq in w.q_lens:
        if lq > 64:
            raise ValueError("a tree has at most 64 nodes")
        paths = []
        for r in range(lq):
            up = paths[int(torch.randint(0, r, (1,), generator=g))] if r else 0
            paths.append(up | (1 << r))
        out += [m - (1 << 64) if m >> 63 else m for m in paths]
    return torch.tensor(out, dtype=torch.int64)


def mixed_prefill(num_chunks: int = 4, chunk: int = 512, num_decodes: int = 128,
                  prefix: int = 800, tail_lo: int = 64, tail_hi: int = 2048,
                  block_size: int = 16, seed: int = 1005) -> Workload:
    """Chunked prefill with decodes riding along, all sharing one prefix.

    Every sequence starts with the same `prefix` tokens (the same physical
    blocks), then a private tail ~ U[tail_lo, tail_hi].  A prefill sequence
    then appends its `chunk` queries (ctx = prefix + tail + chunk, queries at
    positions prefix + tail ...); a decode sequence's ctx is prefix + tail,
    the last of which is its current token.  Prefill rows come first.
    """
    g = torch.Generator().manual_seed(seed)
    tails = torch.randint(tail_lo, tail_hi + 1, (num_chunks + num_decodes,), generator=g).tolist()
    ctx = [prefix + t + chunk for t in tails[:num_chunks]] + [prefix + t for t in tails[num_chunks:]]
    ql = [chunk] * num_chunks + [1] * num_decodes
    return make_workload(f"mixed_prefill_c{num_chunks}x{chunk}_d{num_decodes}", ctx, ql,
                         block_size=block_size, shared_prefix=prefix, seed=seed)


# ------------------------------------------------------------ materialisation

@dataclasses.dataclass
class Batch:
    """Tensors of one workload.  Shapes:
    q [sum Lq, Hq, D] bf16; k_cache, v_cache [NB, bs, Hkv, D] bf16;
    block_table [B, max_blocks] int32 (-1 padded); context_lens [B] int32;
    cu_q_lens [B + 1] int32; k_new, v_new [sum Lq, Hkv, D] bf16 are the K/V
    rows of each sequence's last Lq_i tokens (already present in the pools)
    and slot_mapping [sum Lq] int64 their slots.  k_seq / v_seq, when
    requested, hold each sequence's contiguous [ctx_i, Hkv, D] K/V."""

    workload: Workload
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    context_lens: torch.Tensor
    cu_q_lens: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    slot_mapping: torch.Tensor
    k_seq: Optional[List[torch.Tensor]] = None
    v_seq: Optional[List[torch.Tensor]] = None

    def to(self, device) -> "Batch":
        f = lambda t: t.to(device) if t is not None else None
        return Batch(self.workload, f(self.q), f(self.k_cache), f(self.v_cache),
                     f(self.block_table), f(self.context_lens), f(self.cu_q_lens),
                     f(self.k_new), f(self.v_new), f(self.slot_mapping),
                     self.k_seq, self.v_seq)


def block_assignment(w: Workload) -> torch.Tensor:
    """Block table [B, max_blocks] int32: shared-prefix blocks first, then each
    sequence's private blocks, ids drawn in order from a seeded permutation of
    the pool; -1 pads."""
    g = torch.Generator().manual_seed(w.seed * 7919 + 17)
    perm = torch.randperm(w.num_blocks, generator=g)
    p = w.shared_prefix // w.block_size
    bt = torch.full((w.num_seqs, w.max_blocks_per_seq), -1, dtype=torch.int32)
    nxt = p
    for i, c in enumerate(w.context_lens):
        n = _ceil_div(c, w.block_size)
        if p:
            bt[i, :p] = perm[:p].to(torch.int32)
        k = n - p
        if k > 0:
            bt[i, p:n] = perm[nxt:nxt + k].to(torch.int32)
            nxt += k
    return bt


def slot_of(block_table_row: torch.Tensor, pos: torch.Tensor, block_size: int) -> torch.Tensor:
    """Slot of logical positions `pos` of one sequence: the physical block's
    first slot plus the row inside the block (input construction for
    kv_append)."""
    blk = block_table_row.to(torch.int64)[pos // block_size]
    return blk * block_size + pos % block_size


def _randn_bf16(shape, gen, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def materialize(w: Workload, device="cpu", poison: bool = True, logical: bool = False) -> Batch:
    """Build the tensors of `w` on `device`.

    logical=True (CPU only, small sizes): each sequence's K/V is first drawn
    as a contiguous [ctx, Hkv, D] tensor (the shared prefix once), then
    written block by block into the pool; ``k_seq``/``v_seq`` keep those
    contiguous tensors.  logical=False: every pool slot is drawn directly on
    `device` with a generator seeded from the workload.
    poison=True: slots no sequence owns are NaN; otherwise they stay random.
    """
    device = torch.device(device)
    bs, hkv, d = w.block_size, w.num_kv_heads, w.head_dim
    bt = block_assignment(w)
    ctx_t = torch.tensor(w.context_lens, dtype=torch.int32)
    cu = torch.zeros(w.num_seqs + 1, dtype=torch.int32)
    if w.num_seqs:
        cu[1:] = torch.cumsum(torch.tensor(w.q_lens, dtype=torch.int64), 0).to(torch.int32)
    p = w.shared_prefix // bs

    gcpu = torch.Generator().manual_seed(w.seed)
    k_seq = v_seq = None
    if logical:
        if device.type != "cpu":
            raise ValueError("logical materialisation is CPU only")
        q = _randn_bf16((w.total_q, w.num_q_heads, d), gcpu, "cpu")
        kpre = _randn_bf16((w.shared_prefix, hkv, d), gcpu, "cpu")
        vpre = _randn_bf16((w.shared_prefix, hkv, d), gcpu, "cpu")
        k_seq, v_seq = [], []
        for c in w.context_lens:
            kt = _randn_bf16((c - w.shared_prefix, hkv, d), gcpu, "cpu")
            vt = _randn_bf16((c - w.shared_prefix, hkv, d), gcpu, "cpu")
            k_seq.append(torch.cat([kpre, kt], 0) if w.shared_prefix else kt)
            v_seq.append(torch.cat([vpre, vt], 0) if w.shared_prefix else vt)
        fill = float("nan") if poison else 0.0
        k_cache = torch.full((w.num_blocks, bs, hkv, d), fill, dtype=torch.bfloat16)
        v_cache = torch.full((w.num_blocks, bs, hkv, d), fill, dtype=torch.bfloat16)
        if not poison:
            k_cache.copy_(_randn_bf16(k_cache.shape, gcpu, "cpu"))
            v_cache.copy_(_randn_bf16(v_cache.shape, gcpu, "cpu"))
        for i, c in enumerate(w.context_lens):
            for j in range(_ceil_div(c, bs)):
                if j < p and i > 0:
                    continue  # shared block already written by sequence 0
                rows = min(bs, c - j * bs)
                blk = int(bt[i, j])
                k_cache[blk, :rows] = k_seq[i][j * bs:j * bs + rows]
                v_cache[blk, :rows] = v_seq[i][j * bs:j * bs + rows]
    else:
        gdev = torch.Generator(device=device).manual_seed(w.seed)
        q = _randn_bf16((w.total_q, w.num_q_heads, d), gdev, device)
        k_cache = _randn_bf16((w.num_blocks, bs, hkv, d), gdev, device)
        v_cache = _randn_bf16((w.num_blocks, bs, hkv, d), gdev, device)
        if poison:
            _poison_unused(w, bt, k_cache, v_cache)

    # The rows kv_append writes: each sequence's last Lq_i tokens.
    slots, rows_k, rows_v = [], [], []
    for i, (c, lq) in enumerate(zip(w.context_lens, w.q_lens)):
        if lq == 0:
            continue
        pos = torch.arange(c - lq, c, dtype=torch.int64)
        s = slot_of(bt[i], pos, bs)
        slots.append(s)
        s_dev = s.to(device)
        rows_k.append(k_cache.view(-1, hkv, d)[s_dev])
        rows_v.append(v_cache.view(-1, hkv, d)[s_dev])
    if slots:
        slot_mapping = torch.cat(slots)
        k_new, v_new = torch.cat(rows_k), torch.cat(rows_v)
    else:
        slot_mapping = torch.zeros(0, dtype=torch.int64)
        k_new = torch.zeros((0, hkv, d), dtype=torch.bfloat16, device=device)
        v_new = torch.zeros((0, hkv, d), dtype=torch.bfloat16, device=device)

    return Batch(w, q, k_cache, v_cache, bt.to(device), ctx_t.to(device), cu.to(device),
                 k_new, v_new, slot_mapping.to(device), k_seq, v_seq)


def _poison_unused(w: Workload, bt: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor):
    bs = w.block_size
    owned = torch.zeros(w.num_blocks, dtype=torch.bool)
    valid = bt[bt >= 0].to(torch.int64)
    owned[valid] = True
    unused = torch.nonzero(~owned).flatten().to(k_cache.device)
    k_cache[unused] = float("nan")
    v_cache[unused] = float("nan")
    # rows past the end of each sequence's last block
    for i, c in enumerate(w.context_lens):
        n = _ceil_div(c, bs)
        r = c - (n - 1) * bs
        if n and r < bs:
            last = int(bt[i, n - 1])
            k_cache[last, r:] = float("nan")
            v_cache[last, r:] = float("nan")


FP8_SCALE = 1.0 / 64.0


def fp8_pools(b: Batch, k_scale: float = FP8_SCALE, v_scale: float = FP8_SCALE):
    """(k_codes, v_codes): the batch's pools as uint8 E4M3 codes, same shape
    and device."""
    def cast(pool, scale):
        x = (pool.float() / scale).clamp(-448.0, 448.0)
        return x.to(torch.float8_e4m3fn).view(torch.uint8)
    return cast(b.k_cache, k_scale), cast(b.v_cache, v_scale)


def fp8_block_pools(b: Batch, seed: int, k_spread: float = 2.0, v_spread: float = 1.0):
    """(k_codes, v_codes, k_scales, v_scales): the batch's pools as uint8 E4M3
    codes with one scale per (block, KV head).  Each (block, head) of K is
    first multiplied by 2^u, u uniform in [-k_spread, k_spread] (V likewise
    with v_spread), so blocks and heads differ in magnitude; its scale is
    then its absolute maximum / 448 (1.0 for a block with no finite value),
    and its codes torch's float8 cast of value / scale.  Scales are fp32
    [num_blocks, num_kv_heads] on the pools' device."""
    nb, hkv = b.k_cache.shape[0], b.k_cache.shape[2]
    g = torch.Generator().manual_seed(seed)

    def one(pool, spread):
        f = torch.exp2((torch.rand((nb, hkv), generator=g) * 2 - 1) * spread).to(pool.device)
        x = pool.float() * f[:, None, :, None]
        amax = torch.nan_to_num(x, nan=0.0).abs().amax(dim=(1, 3))
        scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
        codes = (x / scale[:, None, :, None]).clamp(-448.0, 448.0)
        return codes.to(torch.float8_e4m3fn).view(torch.uint8), scale.contiguous()

    kc, ks = one(b.k_cache, k_spread)
    vc, vs = one(b.v_cache, v_spread)
    return kc, vc, ks, vs


def permute_pool(b: Batch, seed: int) -> Batch:
    """The same logical batch with physical ids relabelled by a random
    permutation: block data moved and tables rewritten accordingly."""
    w = b.workload
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(w.num_blocks, generator=g)  # new id of old block x = perm[x]
    dev = b.k_cache.device
    k_new_pool = torch.empty_like(b.k_cache)
    v_new_pool = torch.empty_like(b.v_cache)
    k_new_pool[perm.to(dev)] = b.k_cache
    v_new_pool[perm.to(dev)] = b.v_cache
    bt = b.block_table.cpu().to(torch.int64)
    nbt = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt).to(torch.int32)
    slot = b.slot_mapping.cpu()
    nslot = perm[slot // w.block_size] * w.block_size + slot % w.block_size
    return Batch(w, b.q, k_new_pool, v_new_pool, nbt.to(dev), b.context_lens, b.cu_q_lens,
                 b.k_new, b.v_new, nslot.to(dev), b.k_seq, b.v_seq)
