"""The pages' KV-cache sizing formulas -- TEST INFRASTRUCTURE.

Each is pinned in the tests against numbers the pages print for worked
examples (tests/golden/sizing.json).
"""

def block_memory_bytes(block_size, num_kv_heads, head_size, dtype_size):
    """Bytes of one physical block for one layer: the factor 2 is K plus V.

    "让 Agent 跑得快：LLM 推理服务", section 二 "vLLM：PagedAttention 重新定义
    KV Cache", the block-memory formula.
    """
    return 2 * block_size * num_kv_heads * head_size * dtype_size


def kv_cache_bytes(n_layers, n_kv_heads, d_head, seq_len, batch_size, dtype_bytes):
    """Whole-model KV cache: 2 x layers x kv heads x head dim x tokens x batch
    x dtype bytes.  "LLM 推理优化技术全景", section "KV Cache"; the per-token
    form (seq_len = batch_size = 1) is the one in "让 Agent 跑得快", section 一
    and in "LLM推理工程实战" section 3.1."""
    return 2 * n_layers * n_kv_heads * d_head * seq_len * batch_size * dtype_bytes


def blocks_needed(seq_len, block_size):
    """ceil(seq_len / block_size): the toy allocator's block count
    ("LLM 推理引擎深度解析 ...", section 2.1, PagedKVCache.allocate)."""
    return (seq_len + block_size - 1) // block_size


def internal_waste_tokens(seq_len, block_size):
    """Unused token slots in a request's last block; at most block_size - 1
    ("让 Agent 跑得快", sections 二 and 五: 15 slots for 16-token blocks)."""
    return blocks_needed(seq_len, block_size) * block_size - seq_len

