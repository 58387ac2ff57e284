"""The pages' physical block pool for a paged KV cache -- TEST INFRASTRUCTURE.

A plain model of the bookkeeping the pages describe, used only to check the
library's native block manager (and, through it, block tables and slot
mappings fed to the attention kernels).  Nothing here runs on a GPU.

What it follows:
  * "LLM 推理引擎深度解析：vLLM、SGLang 与 TensorRT-LLM 的核心优化原理",
    section 2.1 "PagedAttention" (its pool sketch): a pool of num_blocks
    fixed-size physical blocks and a free list; allocating a sequence of
    seq_len tokens takes ceil(seq_len / block_size) blocks from the front of
    the free list, not necessarily contiguous, or fails with MemoryError
    when too few are free; freeing puts all of a sequence's blocks back at
    the end of the list, and freeing an id the pool does not know does
    nothing.
  * "让 Agent 跑得快：LLM 推理服务", section 五 (allocation and release
    flow): blocks are taken on demand, one more each time a sequence has
    filled 16 tokens into its last one, so the waste per sequence is at most
    block_size - 1 token slots; a finished sequence's blocks are at once
    usable by others; several block tables may map the same physical block,
    held by a reference count.
  * Same page, section 二, "Copy-on-Write": forked sequences share physical
    blocks with a reference count above 1; only when a sequence must write a
    new token into a shared block is that block copied and its block-table
    entry repointed; a block whose count drops to zero returns to the pool.

Readings where the pages leave a step open:
  * A call that would run out of blocks part-way (an append needing a new
    block and a copy) changes nothing and raises MemoryError.
  * Allocating an id that already exists raises KeyError (the sketch would
    overwrite the entry and lose its blocks).
  * With reference counts, freeing a sequence drops one reference per
    block; a block returns to the list only at count zero.
  * A token that starts a new block never copies: the new block is
    private.  A copy is needed only for the sequence's partly filled last
    block when it is shared.
  * Slots follow the slot-mapping convention of kv_append:
    slot = physical_block * block_size + position % block_size.

Prefix caching ("让 Agent 跑得快", section 七, vLLM's automatic prefix
caching): a full block is identified by its parent block's identity, its
own tokens and an optional extra key (a cache salt); allocation first looks
the prompt's full blocks up in order, takes every hit (reference count + 1,
into the block table) and stops at the first miss, from where the prompt
must be prefilled; released blocks go back to the free queue and stay
matchable until they are reused.  Readings:
  * the identity is the exact chain (parent identity, tokens, salt), kept
    here as nested tuples, so two blocks match only if their whole prefixes
    and salts are equal; the salt enters every block's identity;
  * a prompt's full blocks are registered when it is allocated (their K/V is
    the caller's to compute before another request reads them); partly
    filled blocks and blocks filled later by appends are not registered;
  * taking a block from the free list for new contents (allocation, append,
    copy) drops its registration: the front of the list, the longest-freed
    block, is evicted first; a newer registration of the same identity
    replaces an older one;
  * a hit on a free block takes it out of the free list; the all-or-nothing
    check counts those blocks as no longer free.

Radix-tree prefix sharing ("LLM 推理优化技术全景", section "Prefix Caching 与
RadixAttention"; "让 Agent 跑得快", section 七, RadixAttention): cached
prefixes are matched at token granularity, the longest common prefix with
any cached one, and the matched part's KV is reused; cached prefixes hold
references that keep their KV alive, and when memory runs short the least
recently used ones are dropped.  Readings on a pool of block_size-token
blocks (SGLang's pages hold one token, so there every match is whole pages):
  * an entry is a prompt's tokens up to its last full block, with those
    blocks, registered when the prompt is allocated; it holds one reference
    on each of its blocks.  The partly filled last block stays out: the
    sequence keeps writing into it;
  * a lookup finds L, the longest common prefix of the prompt with any
    entry's tokens; among entries reaching L the most recently used (a
    registration or a hit refreshes an entry) is the donor;
  * the new sequence shares the donor's first L // block_size blocks; when
    L falls inside a block, it gets a fresh block and a copy (the donor's
    block -> the fresh one) to perform before prefill, which starts at
    token L (the copy brings tokens up to L; the caller overwrites the
    rest);
  * the new entry is not registered when its tokens are a prefix of the
    donor's (it would name the donor's blocks again);
  * when fewer blocks are free than the allocation takes, entries are
    dropped in least-recently-used order, never the donor, each releasing
    its references, until enough blocks are free; if even dropping every
    other entry would not free enough, nothing changes (MemoryError);
  * entries and the hash-chain cache above are independent.
"""
from collections import deque


class BlockPool:
    def __init__(self, num_blocks: int, block_size: int = 16):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError("num_blocks >= 0 and block_size > 0 required")
        self.block_size = block_size
        self.num_blocks = num_blocks
        self.free_list = deque(range(num_blocks))
        self.refcount = [0] * num_blocks
        self.tables = {}   # seq_id -> [physical block ids]
        self.lengths = {}  # seq_id -> tokens held
        self.cache = {}    # block identity -> physical block
        self.key_of = [None] * num_blocks
        self.radix = []    # radix entries: {"tokens", "blocks", "stamp"}
        self.clock = 0     # last-use stamps of radix entries

    def num_free(self) -> int:
        return len(self.free_list)

    def _take(self) -> int:
        b = self.free_list.popleft()
        self.refcount[b] = 1
        key = self.key_of[b]
        if key is not None:  # new contents: the registration goes
            if self.cache.get(key) == b:
                del self.cache[key]
            self.key_of[b] = None
        return b

    def _release(self, b: int) -> None:
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free_list.append(b)

    def allocate(self, seq_id: int, seq_len: int) -> list:
        """Blocks for a new sequence of seq_len tokens."""
        if seq_id in self.tables:
            raise KeyError(f"sequence {seq_id} exists")
        if seq_len < 0:
            raise ValueError("seq_len >= 0 required")
        need = -(-seq_len // self.block_size)
        if need > len(self.free_list):
            raise MemoryError("not enough free KV blocks")
        self.tables[seq_id] = [self._take() for _ in range(need)]
        self.lengths[seq_id] = seq_len
        return list(self.tables[seq_id])

    def allocate_cached(self, seq_id, tokens, salt: int = 0):
        """A new sequence holding `tokens`, reusing cached full blocks.

        Returns (blocks, cached_tokens): the block table and the number of
        leading tokens whose K/V the hits already hold (prefill starts there).
        """
        if seq_id in self.tables:
            raise KeyError(f"sequence {seq_id} exists")
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        n = len(tokens)
        keys, key = [], None
        for i in range(n // bs):
            key = (key, tuple(tokens[i * bs:(i + 1) * bs]), int(salt))
            keys.append(key)
        hits = []
        for key in keys:
            b = self.cache.get(key)
            if b is None:
                break
            hits.append(b)
        new = -(-n // bs) - len(hits)
        free_hits = sum(1 for b in hits if self.refcount[b] == 0)
        if new > len(self.free_list) - free_hits:
            raise MemoryError("not enough free KV blocks")
        for b in hits:
            if self.refcount[b] == 0:
                self.free_list.remove(b)
            self.refcount[b] += 1
        blocks = hits + [self._take() for _ in range(new)]
        for i in range(len(hits), len(keys)):
            self.cache[keys[i]] = blocks[i]
            self.key_of[blocks[i]] = keys[i]
        self.tables[seq_id] = blocks
        self.lengths[seq_id] = n
        return list(blocks), len(hits) * bs

    def allocate_radix(self, seq_id, tokens):
        """A new sequence holding `tokens`, reusing the longest cached prefix.

        Returns (blocks, cached_tokens, copies): the block table, the number
        of leading tokens whose K/V the shared and copied blocks hold
        (prefill starts there), and the (source, destination) block copies
        to perform first (at most one).
        """
        if seq_id in self.tables:
            raise KeyError(f"sequence {seq_id} exists")
        tokens = [int(t) for t in tokens]
        bs, n = self.block_size, len(tokens)

        def lcp(a, b):
            k = 0
            while k < len(a) and k < len(b) and a[k] == b[k]:
                k += 1
            return k

        donor, length = None, 0
        for e in self.radix:
            k = lcp(e["tokens"], tokens)
            if k > 0 and (k > length or (k == length and e["stamp"] > donor["stamp"])):
                donor, length = e, k
        shared = donor["blocks"][:length // bs] if donor else []
        partial = donor is not None and length % bs != 0
        fresh = -(-n // bs) - len(shared)
        # what dropping entries in LRU order (never the donor) would free,
        # the new sequence's references on the shared blocks counted first
        count = list(self.refcount)
        for b in shared:
            count[b] += 1
        free, drop = len(self.free_list), []
        for e in sorted((e for e in self.radix if e is not donor), key=lambda e: e["stamp"]):
            if free >= fresh:
                break
            drop.append(e)
            for b in e["blocks"]:
                count[b] -= 1
                free += count[b] == 0
        if free < fresh:
            raise MemoryError("not enough free KV blocks")
        for b in shared:
            self.refcount[b] += 1
        for e in drop:
            self.radix.remove(e)
            for b in e["blocks"]:
                self._release(b)
        blocks = list(shared) + [self._take() for _ in range(fresh)]
        copies = [(donor["blocks"][length // bs], blocks[length // bs])] if partial else []
        if donor is not None:
            self.clock += 1
            donor["stamp"] = self.clock
        full = (n // bs) * bs
        if full > 0 and not (donor is not None and length >= full and
                             donor["tokens"][:full] == tokens[:full]):
            for b in blocks[:n // bs]:
                self.refcount[b] += 1
            self.clock += 1
            self.radix.append({"tokens": tokens[:full], "blocks": blocks[:n // bs],
                               "stamp": self.clock})
        self.tables[seq_id] = blocks
        self.lengths[seq_id] = n
        return list(blocks), length, copies

    def radix_clear(self) -> None:
        """Drop every radix entry, least recently used first, releasing its
        references."""
        for e in sorted(self.radix, key=lambda e: e["stamp"]):
            for b in e["blocks"]:
                self._release(b)
        self.radix = []

    def free(self, seq_id: int) -> None:
        """Drop a sequence; blocks nobody else references go back to the pool.
        An unknown id is ignored."""
        if seq_id not in self.tables:
            return
        for b in self.tables.pop(seq_id):
            self._release(b)
        del self.lengths[seq_id]

    def fork(self, parent: int, child: int) -> None:
        """child starts as a copy of parent's table, sharing every block."""
        if child in self.tables:
            raise KeyError(f"sequence {child} exists")
        blocks = self.tables[parent]
        for b in blocks:
            self.refcount[b] += 1
        self.tables[child] = list(blocks)
        self.lengths[child] = self.lengths[parent]

    def append(self, seq_id: int, num_tokens: int):
        """Room for num_tokens more tokens of seq_id.

        Returns (slots, copies): one slot per new token, in order, and the
        (source, destination) block copies to perform before writing them.
        """
        blocks, length, bs = self.tables[seq_id], self.lengths[seq_id], self.block_size
        if num_tokens < 0:
            raise ValueError("num_tokens >= 0 required")
        if num_tokens == 0:
            return [], []
        # blocks this call needs from the pool: the copy of a shared partly
        # filled last block, then one per block boundary crossed
        last_shared = length % bs != 0 and self.refcount[blocks[-1]] > 1
        new_blocks = -(-(length + num_tokens) // bs) - len(blocks)
        if int(last_shared) + new_blocks > len(self.free_list):
            raise MemoryError("not enough free KV blocks")
        copies = []
        if last_shared:
            old = blocks[-1]
            dst = self._take()
            copies.append((old, dst))
            self._release(old)
            blocks[-1] = dst
        slots = []
        for pos in range(length, length + num_tokens):
            if pos // bs == len(blocks):
                blocks.append(self._take())
            slots.append(blocks[pos // bs] * bs + pos % bs)
        self.lengths[seq_id] = length + num_tokens
        return slots, copies

    def block_table(self, seq_ids, max_blocks: int):
        """[len(seq_ids)][max_blocks] table padded with -1, and the lengths."""
        table = [[-1] * max_blocks for _ in seq_ids]
        lens = []
        for r, s in enumerate(seq_ids):
            blocks = self.tables[s]
            if len(blocks) > max_blocks:
                raise ValueError("max_blocks too small")
            table[r][:len(blocks)] = blocks
            lens.append(self.lengths[s])
        return table, lens

    def check(self) -> None:
        """Pool invariants: every block is free exactly once with count 0, or
        referenced by exactly refcount sequence tables and radix entries."""
        seen = [0] * self.num_blocks
        for blocks in self.tables.values():
            for b in blocks:
                seen[b] += 1
        for e in self.radix:  # radix entries hold references too
            assert len(e["tokens"]) == len(e["blocks"]) * self.block_size
            for b in e["blocks"]:
                seen[b] += 1
        free = set(self.free_list)
        assert len(free) == len(self.free_list), "a block is free twice"
        for b in range(self.num_blocks):
            assert seen[b] == self.refcount[b], (b, seen[b], self.refcount[b])
            assert (b in free) == (self.refcount[b] == 0), b
        for s, blocks in self.tables.items():
            assert len(blocks) == -(-self.lengths[s] // self.block_size), s
        for key, b in self.cache.items():
            assert self.key_of[b] == key, (b, "registration out of step")


def copy_blocks(k_cache, v_cache, pairs):
    """The device half of copy-on-write: every row of block src, K and V,
    lands in block dst ("让 Agent 跑得快", section 二, "Copy-on-Write": the
    shared block is copied before the write).

    k_cache, v_cache: [num_blocks, block_size, Hkv, D] arrays (any dtype;
    bf16 as uint16 bits).  pairs: (src, dst) rows.  A pair naming a block
    outside the pool is skipped.  Returns new arrays; the inputs are kept.
    """
    import numpy as np
    k_src, v_src = np.asarray(k_cache), np.asarray(v_cache)
    k_out, v_out = k_src.copy(), v_src.copy()
    nb = k_src.shape[0]
    for src, dst in pairs:
        src, dst = int(src), int(dst)
        if 0 <= src < nb and 0 <= dst < nb:
            k_out[dst] = k_src[src]
            v_out[dst] = v_src[src]
    return k_out, v_out
