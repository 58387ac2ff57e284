"""The oracle's block pool and whole-block copy pinned to what the pages fix:
block counts and waste, on-demand growth, the pool sketch's order of blocks,
release, sharing under reference counts and copy-on-write."""
import random

import numpy as np
import pytest

import oracle
from oracle.blocks import BlockPool, copy_blocks as oracle_copy_blocks


# ---------------------------------------------------------------- oracle pins

def smallest_blocks(n, bs):
    """Brute force: the fewest bs-token blocks that hold n tokens."""
    k = 0
    while k * bs < n:
        k += 1
    return k


@pytest.mark.parametrize("bs", [16, 32])
def test_pin_blocks_and_waste(bs):
    """A sequence holds the fewest blocks that fit it, and wastes at most
    block_size - 1 slots: 15 for 16-token blocks ("让 Agent 跑得快", sections
    二 and 五)."""
    pool = BlockPool(10_000, bs)
    worst = 0
    for n in range(0, 6 * bs + 3):
        pool.allocate(n, n)
        held = len(pool.tables[n])
        assert held == smallest_blocks(n, bs)
        waste = held * bs - n
        assert 0 <= waste <= bs - 1
        worst = max(worst, waste)
    assert worst == bs - 1
    pool.check()


def test_pin_on_demand_growth():
    """One more block each time 16 tokens have filled the last one
    ("让 Agent 跑得快", section 五, allocation flow)."""
    pool = BlockPool(64, 16)
    pool.allocate("s", 0)
    taken_at = []
    for tok in range(1, 100):
        before = pool.num_free()
        slots, copies = pool.append("s", 1)
        assert copies == []
        if pool.num_free() != before:
            assert before - pool.num_free() == 1
            taken_at.append(tok)
    assert taken_at == [1, 17, 33, 49, 65, 81, 97]
    pool.check()


def test_pin_pool_sketch_worked_example():
    """The pool sketch of "LLM 推理引擎深度解析", section 2.1, run by hand on a
    10-block pool: blocks come off the front of the free list and go back at
    its end; too few free blocks raise MemoryError; freeing an unknown id
    does nothing."""
    pool = BlockPool(10, 16)
    assert pool.allocate("A", 50) == [0, 1, 2, 3]          # ceil(50/16) = 4
    with pytest.raises(MemoryError):
        pool.allocate("B", 100)                            # needs 7, 6 free
    assert list(pool.free_list) == [4, 5, 6, 7, 8, 9]      # nothing taken
    pool.free("A")
    assert list(pool.free_list) == [4, 5, 6, 7, 8, 9, 0, 1, 2, 3]
    assert pool.allocate("B", 100) == [4, 5, 6, 7, 8, 9, 0]
    pool.free("nobody")
    assert list(pool.free_list) == [1, 2, 3]
    pool.check()


def test_pin_freed_blocks_reusable():
    """A finished request's blocks are at once usable by any other request
    ("让 Agent 跑得快", section 五, release flow)."""
    pool = BlockPool(8, 16)
    pool.allocate(1, 8 * 16)
    with pytest.raises(MemoryError):
        pool.allocate(2, 1)
    pool.free(1)
    assert sorted(pool.allocate(2, 8 * 16)) == list(range(8))


def test_pin_shared_system_prompt():
    """50 requests sharing one 5000-token system prompt hold one physical copy
    of it ("让 Agent 跑得快", section 五, shared prefix).  Reading: a shared,
    partly filled last block (5000 = 312 x 16 + 8) is copied on each request's
    first write (section 二, Copy-on-Write), except by the last holder."""
    pool = BlockPool(1000, 16)
    prompt = pool.allocate("prompt", 5000)
    assert len(prompt) == 313
    for r in range(50):
        pool.fork("prompt", r)
    assert pool.num_free() == 1000 - 313                    # one physical copy
    assert all(pool.refcount[b] == 51 for b in prompt)
    pool.free("prompt")
    assert all(pool.refcount[b] == 50 for b in prompt)
    n_copies = 0
    for r in range(50):
        slots, copies = pool.append(r, 1)
        n_copies += len(copies)
        assert pool.tables[r][:312] == prompt[:312]         # full blocks stay shared
        assert slots == [pool.tables[r][312] * 16 + 8]
        if copies:
            assert copies == [(prompt[312], pool.tables[r][312])]
    assert n_copies == 49                                   # the last holder writes in place
    assert pool.tables[49][312] == prompt[312]
    assert pool.num_free() == 1000 - 313 - 49
    pool.check()


def test_pin_copy_on_write_fork():
    """Forked sequences share blocks; the writer gets a private copy, the other
    keeps the original; a full shared last block is never copied: the next
    token opens a fresh block ("让 Agent 跑得快", section 二, Copy-on-Write)."""
    pool = BlockPool(16, 16)
    pool.allocate("p", 20)                                   # blocks 0, 1 (4 tokens in 1)
    pool.fork("p", "c")
    slots, copies = pool.append("c", 3)
    assert copies == [(1, 2)]
    assert pool.tables["c"] == [0, 2] and pool.tables["p"] == [0, 1]
    assert slots == [2 * 16 + 4, 2 * 16 + 5, 2 * 16 + 6]
    assert pool.refcount[:3] == [2, 1, 1]
    # a shared FULL last block: the parent fills block 1, forks, and both write
    pool.append("p", 12)                                     # block 1 now full (32 tokens)
    pool.fork("p", "d")
    s1, c1 = pool.append("d", 1)
    s2, c2 = pool.append("p", 1)
    assert c1 == [] and c2 == []
    assert s1 == [3 * 16] and s2 == [4 * 16]
    assert pool.tables["d"][:2] == pool.tables["p"][:2] == [0, 1]
    pool.check()


def test_pin_all_or_nothing():
    """An append that needs a copy and a new block, with one free block, fails
    and changes nothing (reading: a call that cannot finish changes nothing)."""
    pool = BlockPool(3, 16)
    pool.allocate("p", 20)                                   # blocks 0, 1
    pool.fork("p", "c")
    snap = (list(pool.free_list), list(pool.refcount), {k: list(v) for k, v in pool.tables.items()},
            dict(pool.lengths))
    with pytest.raises(MemoryError):
        pool.append("c", 13)                                 # copy of block 1 + a new block
    assert snap == (list(pool.free_list), list(pool.refcount),
                    {k: list(v) for k, v in pool.tables.items()}, dict(pool.lengths))
    slots, copies = pool.append("c", 12)                     # the copy alone fits
    assert copies == [(1, 2)] and len(slots) == 12
    pool.check()


def test_pin_slots_reach_every_token_once():
    """Slots of all sequences' tokens are distinct, lie in the sequence's own
    blocks at row position % block_size, and agree with the block table."""
    rng = random.Random(5)
    pool = BlockPool(200, 16)
    owner = {}
    for s in range(12):
        pool.allocate(s, 0)
        for _ in range(rng.randrange(1, 6)):
            slots, copies = pool.append(s, rng.randrange(0, 40))
            assert copies == []
            for sl in slots:
                assert sl not in owner
                owner[sl] = s
    for s in range(12):
        n = pool.lengths[s]
        for pos in range(n):
            sl = pool.tables[s][pos // 16] * 16 + pos % 16
            assert owner[sl] == s
    pool.check()


def test_pin_copy_blocks_matches_append():
    """The whole-block copy equals re-appending the source block's rows into
    the destination's slots through the fp64 oracle's own kv_append."""
    rng = np.random.default_rng(7)
    nb, bs, hkv, d = 12, 16, 2, 128
    k = rng.integers(0, 1 << 16, size=(nb, bs, hkv, d), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(nb, bs, hkv, d), dtype=np.uint16)
    pairs = [(3, 7), (0, 11), (5, 2), (-1, 4), (6, 12)]      # the last two name no block
    ko, vo = oracle_copy_blocks(k, v, pairs)
    slots = np.concatenate([dst * bs + np.arange(bs) for _, dst in pairs[:3]]).astype(np.int64)
    k_rows = np.concatenate([k[src] for src, _ in pairs[:3]])
    v_rows = np.concatenate([v[src] for src, _ in pairs[:3]])
    ka, va = oracle.kv_append(k_rows, v_rows, slots, k, v)
    assert np.array_equal(ko, ka) and np.array_equal(vo, va)
    assert np.array_equal(ko[4], k[4]) and np.array_equal(ko[7], k[3])


# ------------------------------------------------------------ prefix cache

def prompt(*parts):
    return [t for p in parts for t in p]


SYS = list(range(1000, 1800))          # an 800-token system prompt: 50 full 16-token blocks


def test_pin_prefix_cache_hit_and_prefill_start():
    """A second request with the same system prompt takes the cached blocks
    (reference count + 1, in its table) and prefills from the first miss
    ("让 Agent 跑得快", section 七, steps 2-3)."""
    pool = BlockPool(200, 16)
    a, cached_a = pool.allocate_cached("a", prompt(SYS, [1, 2, 3]))
    assert cached_a == 0 and len(a) == 51
    b, cached_b = pool.allocate_cached("b", prompt(SYS, [7, 8, 9, 10]))
    assert cached_b == 800                              # prefill starts at token 800
    assert b[:50] == a[:50] and b[50] != a[50]
    assert all(pool.refcount[x] == 2 for x in a[:50]) and pool.refcount[a[50]] == 1
    assert pool.num_free() == 200 - 52
    pool.check()


def test_pin_prefix_cache_only_full_blocks():
    """Only complete blocks are cached; a partly filled block is not
    ("让 Agent 跑得快", section 三: block-granular matching)."""
    pool = BlockPool(20, 16)
    pool.allocate_cached("a", list(range(20)))          # one full block + 4 tokens
    _, cached = pool.allocate_cached("b", list(range(20)))
    assert cached == 16
    assert len(pool.cache) == 1
    _, cached = pool.allocate_cached("c", list(range(15)))
    assert cached == 0                                   # the first block is not full here


def test_pin_prefix_cache_chain_continuity():
    """A block hits only if every block before it hits: the same tokens after
    a different first block miss ("让 Agent 跑得快", section 七, the hash
    chain)."""
    pool = BlockPool(20, 16)
    x, y, z = [1] * 16, [2] * 16, [3] * 16
    pool.allocate_cached("a", prompt(x, y))
    _, cached = pool.allocate_cached("b", prompt(z, y))
    assert cached == 0
    _, cached = pool.allocate_cached("c", prompt(x, z))
    assert cached == 16


def test_pin_prefix_cache_survives_release_until_reused():
    """Released blocks return to the free queue and stay matchable; once the
    free queue hands them out again their registration is gone (section 七,
    step 4)."""
    pool = BlockPool(6, 16)
    toks = list(range(64))                               # 4 full blocks
    blocks, _ = pool.allocate_cached("a", toks)
    pool.free("a")
    assert pool.num_free() == 6 and len(pool.cache) == 4
    again, cached = pool.allocate_cached("b", toks)
    assert cached == 64 and again == blocks and pool.num_free() == 2
    pool.free("b")
    # the free queue is now [4, 5, 0, 1, 2, 3]: three fresh blocks evict block 0
    pool.allocate("c", 48)
    assert pool.tables["c"] == [4, 5, 0]
    assert len(pool.cache) == 3                          # block 0's registration is gone
    pool.free("c")
    _, cached = pool.allocate_cached("d", toks)
    assert cached == 0                                   # the chain broke at block 0
    pool.check()


def test_pin_prefix_cache_salt_isolates():
    """The same tokens under another cache salt never match (section 七,
    cache_salt)."""
    pool = BlockPool(20, 16)
    pool.allocate_cached("a", list(range(32)), salt=1)
    assert pool.allocate_cached("b", list(range(32)), salt=2)[1] == 0
    assert pool.allocate_cached("c", list(range(32)), salt=1)[1] == 32


def test_pin_prefix_cache_hit_rate_depends_on_where_prompts_differ():
    """Fixed system prompt first and the varying question last: every
    request after the first reuses the prompt; a varying token in front
    (a timestamp) makes every block miss (section 七, hit rates)."""
    pool = BlockPool(5000, 16)
    hits_end, hits_front = [], []
    for r in range(10):
        hits_end.append(pool.allocate_cached(("end", r), prompt(SYS, [r] * 40))[1])
        hits_front.append(pool.allocate_cached(("front", r), prompt([r], SYS, [5] * 39))[1])
    assert hits_end == [0] + [800] * 9
    assert hits_front == [0] * 10


def test_pin_prefix_cache_free_hits_count_against_room():
    """A hit on a free block leaves the free list: an allocation that needs
    every free block plus one cached free block fails and changes nothing."""
    pool = BlockPool(4, 16)
    pool.allocate_cached("a", list(range(32)))          # blocks 0, 1 cached
    pool.free("a")
    snap = (list(pool.free_list), list(pool.refcount), dict(pool.cache))
    with pytest.raises(MemoryError):
        pool.allocate_cached("b", list(range(32)) + list(range(100, 148)))  # 2 hits + 3 new
    assert snap == (list(pool.free_list), list(pool.refcount), dict(pool.cache))
    blocks, cached = pool.allocate_cached("b", list(range(32)) + list(range(100, 132)))
    assert cached == 32 and blocks[:2] == [0, 1]
    pool.check()


# ---------------------------------------------------- radix-tree prefix sharing

class KvModel:
    """What the blocks of a pool hold, as token ids per slot (None: never
    written): prefill writes a prompt's tokens, a copy duplicates a block.
    Independent of how the pool decides what to share."""

    def __init__(self, pool):
        self.pool = pool
        self.slots = {}

    def copy(self, src, dst):
        bs = self.pool.block_size
        for o in range(bs):
            self.slots[dst * bs + o] = self.slots.get(src * bs + o)

    def prefill(self, blocks, tokens, start):
        bs = self.pool.block_size
        for p in range(start, len(tokens)):
            self.slots[blocks[p // bs] * bs + p % bs] = tokens[p]

    def holds(self, blocks, tokens, upto):
        bs = self.pool.block_size
        return all(self.slots.get(blocks[p // bs] * bs + p % bs) == tokens[p] for p in range(upto))


def radix_alloc(pool, kv, sid, tokens):
    """allocate_radix, then what the caller does: the copies, the prefill
    from the cached length; checks that the reused blocks held the prefix."""
    blocks, cached, copies = pool.allocate_radix(sid, tokens)
    assert len(copies) <= 1 and len(blocks) == -(-len(tokens) // pool.block_size)
    for src, dst in copies:
        kv.copy(src, dst)
    assert kv.holds(blocks, tokens, cached), (sid, cached)
    kv.prefill(blocks, tokens, cached)
    assert kv.holds(blocks, tokens, len(tokens))
    pool.check()
    return blocks, cached, copies


def test_pin_radix_shares_the_pages_1000_token_prefix():
    """Two requests whose first 1000 tokens agree and then differ ("让 Agent
    跑得快", section 七: the radix tree shares those 1000 tokens where a
    whole-prompt key would miss): with 16-token blocks the second request
    shares 62 full blocks and copies the 63rd (8 tokens of it are the
    prefix), and prefill starts at token 1000; block-level prefix caching
    stops at the last whole block, 992 tokens."""
    common = list(range(1000))
    a, b = common + [5000 + i for i in range(200)], common + [7000 + i for i in range(150)]
    pool = BlockPool(400, 16)
    kv = KvModel(pool)
    blocks_a, cached_a, _ = radix_alloc(pool, kv, "a", a)
    assert cached_a == 0
    blocks_b, cached_b, copies = radix_alloc(pool, kv, "b", b)
    assert cached_b == 1000
    assert blocks_b[:62] == blocks_a[:62] and blocks_b[62] != blocks_a[62]
    assert copies == [(blocks_a[62], blocks_b[62])]
    hc = BlockPool(400, 16)
    hc.allocate_cached("a", a)
    assert hc.allocate_cached("b", b)[1] == 992


def test_pin_radix_equals_block_caching_on_block_aligned_prefixes():
    """A shared system prompt that fills whole blocks: both schemes reuse the
    same blocks and start prefill at the same token ("LLM 推理优化技术全景",
    vLLM APC against SGLang RadixAttention: alike when the prompt divides
    into whole blocks)."""
    sys_prompt = list(range(50, 50 + 800))  # 50 blocks of 16
    rng = random.Random(3)
    radix, hc = BlockPool(2000, 16), BlockPool(2000, 16)
    kv = KvModel(radix)
    for i in range(6):
        p = sys_prompt + [rng.randrange(10_000, 20_000) for _ in range(rng.randrange(1, 300))]
        blocks_r, cached_r, copies = radix_alloc(radix, kv, i, p)
        blocks_h, cached_h = hc.allocate_cached(i, p)
        assert cached_r == cached_h == (0 if i == 0 else 800)
        assert copies == []


def test_pin_radix_longest_prefix_and_most_recent_donor():
    """The longest match wins whichever entry holds it; among entries that
    reach the same length, the most recently used one donates."""
    pool = BlockPool(100, 4)
    kv = KvModel(pool)
    radix_alloc(pool, kv, 1, [1, 2, 3, 4, 5, 6, 7, 8, 9, 10])          # entry: 8 tokens
    radix_alloc(pool, kv, 2, [1, 2, 3, 4, 5, 6, 70, 80, 90, 100, 11])  # shares 6, copies one
    # entries stop at the last full block: 2's holds 8 tokens, so 90 is not matched
    _, cached, copies = radix_alloc(pool, kv, 3, [1, 2, 3, 4, 5, 6, 70, 80, 90, 1])
    assert cached == 8 and copies == [] and pool.tables[3][:2] == pool.tables[2][:2]
    # 1, 2, 3 appears in all three; the last registered or hit (3) donates
    _, cached, copies = radix_alloc(pool, kv, 4, [1, 2, 3, 9, 9])
    assert cached == 3 and copies == [(pool.tables[3][0], pool.tables[4][0])]
    # a prompt that is a prefix of an entry registers nothing new
    entries = len(pool.radix)
    _, cached, copies = radix_alloc(pool, kv, 5, [1, 2, 3, 4, 5, 6, 7, 8])
    assert cached == 8 and copies == [] and len(pool.radix) == entries
    assert pool.tables[5] == pool.tables[1][:2]


def test_pin_radix_lru_eviction_and_all_or_nothing():
    """Entries keep their blocks after the sequences go; when blocks run
    short the least recently used entries go first (a hit refreshes one),
    and a call that cannot be met even by dropping every entry other than
    its donor changes nothing."""
    pool = BlockPool(6, 4)
    kv = KvModel(pool)
    a, b = [1] * 8, [2] * 8
    radix_alloc(pool, kv, "a", a)
    radix_alloc(pool, kv, "b", b)
    pool.free("a")
    pool.free("b")
    assert pool.num_free() == 2 and len(pool.radix) == 2
    _, cached, _ = radix_alloc(pool, kv, "a2", a)       # hit: a's entry refreshed
    assert cached == 8 and pool.num_free() == 2
    pool.free("a2")
    _, cached, _ = radix_alloc(pool, kv, "c", [3] * 12)  # 3 blocks: b's entry goes
    assert cached == 0 and [e["tokens"] for e in pool.radix] == [a, [3] * 12]
    import copy
    snap = copy.deepcopy((pool.free_list, pool.refcount, pool.radix, pool.tables))
    with pytest.raises(MemoryError):
        pool.allocate_radix("d", [1] * 8 + [4] * 20)  # shares 2, needs 5 more: 4 at most
    assert snap == (pool.free_list, pool.refcount, pool.radix, pool.tables)
    pool.radix_clear()
    pool.check()


@pytest.mark.parametrize("seed", range(6))
def test_pin_radix_random_workload_reuses_only_true_prefixes(seed):
    """Random prompts over a few shared stems, appends, forks and frees on a
    tight pool: every reuse hands over exactly the prompt's prefix (the
    KV model), every reference is accounted for, and the reported prefix is
    the longest any live entry offers."""
    rng = random.Random(seed)
    bs = rng.choice([4, 8, 16])
    pool = BlockPool(rng.randrange(30, 90), bs)
    kv = KvModel(pool)
    stems = [[rng.randrange(100) for _ in range(rng.randrange(0, 5 * bs))] for _ in range(4)]
    live, next_id = [], 0
    for _ in range(160):
        op = rng.random()
        if op < 0.55:
            p = rng.choice(stems)[: rng.randrange(0, 5 * bs + 1)]
            p = p + [rng.randrange(100, 200) for _ in range(rng.randrange(1, 3 * bs))]
            best = max((sum(1 for _ in iter_common(e["tokens"], p)) for e in pool.radix), default=0)
            try:
                _, cached, _ = radix_alloc(pool, kv, next_id, p)
            except MemoryError:
                pool.check()
                continue
            assert cached == best
            live.append(next_id)
            next_id += 1
        elif op < 0.75 and live:
            pool.free(live.pop(rng.randrange(len(live))))
            pool.check()
        elif op < 0.9 and live:
            s = rng.choice(live)
            try:
                slots, copies = pool.append(s, rng.randrange(1, 2 * bs))
            except MemoryError:
                continue
            for src, dst in copies:
                kv.copy(src, dst)
            pool.check()
        elif live:
            try:
                pool.fork(rng.choice(live), next_id)
            except MemoryError:
                continue
            live.append(next_id)
            next_id += 1
            pool.check()


def iter_common(a, b):
    for x, y in zip(a, b):
        if x != y:
            return
        yield x
