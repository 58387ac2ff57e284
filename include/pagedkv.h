/*
 * pagedkv.h -- C ABI of libpagedkv.so: attention over a paged KV cache on
 * AMD MI355X (gfx950).
 *
 * What is computed comes from these pages:
 *  - "LLM 推理引擎深度解析：vLLM、SGLang 与 TensorRT-LLM 的核心优化原理"
 *    (jsjson.com), section 2.1 "PagedAttention": the pools are
 *    [num_blocks, block_size, num_heads, head_dim] tensors and a per-sequence
 *    block table maps logical blocks to physical ones;
 *  - "让 Agent 跑得快：LLM 推理服务" (hkg.20260401.xyz agent-book-07),
 *    sections 二 and 五: 16-token blocks allocated on demand, blocks shared
 *    read-only between sequences, only the current token writes;
 *  - "LLM 推理优化技术全景" (docs.ifdog.com inference-optimization): section
 *    "KV Cache" (append, then reuse), "Flash Attention 深度剖析" (attention is
 *    Softmax(Q K^T) V, computed in one pass with a running max m and sum l so
 *    the score matrix is never stored; the rescale is deferred to the end as
 *    in its "Flash Attention v2 的改进"), and "Chunked Prefill" (prompts
 *    processed in equal chunks, decodes batched with them).
 *
 * Conventions shared by every call
 *  - Every array argument is a DEVICE pointer, allocated and owned by the
 *    caller, who keeps it alive until the enqueued work has finished.  The
 *    library allocates nothing, frees nothing and keeps no state between
 *    calls; concurrent calls on different streams are safe when their output
 *    buffers (and workspaces) do not overlap.
 *  - `stream` is a hipStream_t (NULL = the null stream).  All work is
 *    enqueued asynchronously on it; no call synchronises.
 *  - Element types: K/V pools, q, k_new, v_new are bf16; block tables,
 *    context lengths and cu_q_lens are int32; slot mappings are int64.
 *  - Pool layout: k_cache and v_cache are each
 *    [num_blocks][block_size][num_kv_heads][head_dim], row-major, so token
 *    row r of physical block b for KV head h starts at element
 *    ((b * block_size + r) * num_kv_heads + h) * head_dim.
 *  - block_table is [num_seqs][max_blocks_per_seq], row-major: entry (i, j)
 *    is the physical block of sequence i's logical block j (tokens
 *    j*block_size ... j*block_size + block_size - 1).  Entries a sequence
 *    does not use are never read (by convention -1).
 *  - GQA: query head h reads KV head h / (num_q_heads / num_kv_heads).
 *  - Scores are scale * <q, k>; the caller passes the scale (1/sqrt(128)
 *    for the usual softmax temperature).
 *  - Supported: head_dim == 128; block_size 16 or 32;
 *    num_q_heads / num_kv_heads in {1, 2, 4, 8, 16}; num_seqs <= 65535.
 *  - Alignment: q, out, the pools, k_new and v_new must be 16-byte aligned
 *    (the kernels move 128-bit words).
 *  - Errors are detected on the host BEFORE anything is enqueued (so they
 *    can be tested without a GPU): the call returns a negative status and
 *    nothing is launched.  PKV_ERR_LAUNCH reports a HIP error after launch.
 *    Values inside device arrays are not validated: a block id outside the
 *    pool, a slot outside the pool or a context length above
 *    max_blocks_per_seq * block_size is undefined behaviour.  A context
 *    length above `max_context_len` is clamped to it on the device.
 *  - Determinism: results are bitwise reproducible run to run for the same
 *    inputs and arguments (no floating-point atomics).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pkv_status {
    PKV_OK = 0,
    PKV_ERR_NULL = -1,        /* a required pointer is NULL */
    PKV_ERR_SHAPE = -2,       /* inconsistent sizes (negative counts, Hq % Hkv, ...) */
    PKV_ERR_UNSUPPORTED = -3, /* head_dim, block_size, group size or dtype not built */
    PKV_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
    PKV_ERR_LAUNCH = -5,      /* the HIP runtime reported an error at launch */
    PKV_ERR_ALIGN = -6        /* a bf16 array is not 16-byte aligned */
};

enum pkv_out_dtype {
    PKV_OUT_F32 = 0,  /* fp32 output (the default; meets fp32-level accuracy) */
    PKV_OUT_BF16 = 1  /* bf16 output, rounded to nearest even from fp32 */
};

/* Human-readable text for a status code (static storage, never NULL). */
const char *pkv_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int pkv_version(void);

/*
 * kv_append -- write new tokens' K and V rows into their slots.
 * ("LLM 推理优化技术全景", section "KV Cache": each step's new K/V are added to
 * the cache; "让 Agent 跑得快", section 五: only the current token writes.)
 *
 *   k_new, v_new   [num_tokens][num_kv_heads][head_dim] bf16 (read)
 *   slot_mapping   [num_tokens] int64 (read): token t goes to physical block
 *                  slot / block_size, row slot % block_size; slot < 0 skips t.
 *                  Two tokens with the same slot in one call is a caller
 *                  error (which one lands is unspecified).
 *   k_cache, v_cache  pools (written only at the given slots)
 *   num_blocks     pool size in blocks (for the caller's bookkeeping; slots
 *                  are not range-checked on the device)
 * The copy is bit-exact.  num_tokens == 0 is a no-op.
 */
int pkv_kv_append(const void *k_new, const void *v_new, const int64_t *slot_mapping,
                  int64_t num_tokens, void *k_cache, void *v_cache, int64_t num_blocks,
                  int block_size, int num_kv_heads, int head_dim, void *stream);

/*
 * Workspace needed by pkv_paged_decode_attn for these sizes (bytes; 0 only
 * for num_seqs == 0 or inconsistent head counts).  The keys of all
 * sequences are split evenly over the workgroups the GPU holds at once; a
 * sequence shared by several workgroups leaves per-workgroup partial results
 * (running max, running sum, unnormalised accumulator per query head) in the
 * workspace until a log-sum-exp merge combines them.  At most 1024
 * workgroups x 2 records x num_q_heads x 528 bytes, plus the per-sequence
 * tile prefix sums.
 */
size_t pkv_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                  int max_context_len);

/*
 * paged_decode_attn -- one query row per sequence against its cached keys.
 *
 *   out            [num_seqs][num_q_heads][head_dim], fp32 or bf16 (written)
 *   q              [num_seqs][num_q_heads][head_dim] bf16
 *   k_cache, v_cache  pools (read)
 *   block_table    [num_seqs][max_blocks_per_seq] int32
 *   context_lens   [num_seqs] int32: sequence i attends to its keys
 *                  0 ... context_lens[i] - 1 (append the current token first
 *                  if it should see itself); 0 gives an all-zero row
 *   max_context_len  host-side upper bound of context_lens (sizes the split)
 *   workspace      device scratch of at least pkv_decode_workspace_bytes()
 *                  bytes, 16-byte aligned; contents need no initialisation
 *                  and are garbage afterwards
 *   num_seqs       at most 16383 for this call; num_kv_heads 1..8 or 16
 *
 *   out[i, h, :] = sum_t softmax_t(scale * <q[i,h], K_i[t]>) V_i[t]
 * with K_i, V_i the KV head h / G rows of sequence i reached through its
 * block table.  fp32 accumulation throughout.
 */
int pkv_paged_decode_attn(void *out, int out_dtype, const void *q, const void *k_cache,
                          const void *v_cache, const int32_t *block_table,
                          int max_blocks_per_seq, const int32_t *context_lens,
                          int max_context_len, int num_seqs, int num_q_heads,
                          int num_kv_heads, int head_dim, int block_size, float scale,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Workspace needed by pkv_paged_prefill_attn (bytes, >= 0): the decode
 * workspace for the batch's single-row sequences.  A call whose every
 * sequence has exactly max_q_len > 1 rows needs none (workspace may be NULL).
 */
size_t pkv_prefill_workspace_bytes(int num_seqs, int num_q_tokens, int num_q_heads,
                                   int head_dim, int max_context_len);

/*
 * paged_prefill_attn -- a chunk of queries per sequence (causal), decode rows
 * allowed in the same call.  ("LLM 推理优化技术全景", sections "Flash
 * Attention 深度剖析 > 分块算法" and "Chunked Prefill".)
 *
 *   out            [num_q_tokens][num_q_heads][head_dim], fp32 or bf16
 *   q              [num_q_tokens][num_q_heads][head_dim] bf16
 *   cu_q_lens      [num_seqs + 1] int32 device array: prefix sums of the
 *                  per-sequence query counts Lq_i (cu_q_lens[0] = 0,
 *                  cu_q_lens[num_seqs] = num_q_tokens)
 *   context_lens   [num_seqs] int32: keys of sequence i, INCLUDING its
 *                  Lq_i new tokens (already appended).  Query row r of
 *                  sequence i sits at absolute position
 *                  context_lens[i] - Lq_i + r; with causal != 0 it sees keys
 *                  0 ... position, else all context_lens[i] keys.
 *                  Lq_i <= context_lens[i] is required.
 *   max_q_len      host-side upper bound of Lq_i
 *   num_q_tokens   host-side total query rows (= cu_q_lens[num_seqs])
 * Rows with Lq_i == 1 take the bandwidth-bound decode path (the split-KV
 * decode kernels, enqueued after the MFMA chunk kernel on the same stream);
 * longer chunks take the MFMA path.  num_seqs <= 16383 and num_kv_heads in
 * 1..8 or 16 when single-row sequences can be present.  QK^T runs as bf16 x bf16 MFMA with fp32 accumulation;
 * P V runs as fp16 x fp16 MFMA with fp32 accumulation, V converted from bf16
 * to fp16 in registers: exact for |v| in [2^-14, 65504]; smaller magnitudes
 * keep an absolute error below 2^-25, and |v| > 65504 is outside the
 * supported range.
 */
int pkv_paged_prefill_attn(void *out, int out_dtype, const void *q, const int32_t *cu_q_lens,
                           const void *k_cache, const void *v_cache,
                           const int32_t *block_table, int max_blocks_per_seq,
                           const int32_t *context_lens, int max_context_len, int max_q_len,
                           int num_q_tokens, int num_seqs, int num_q_heads, int num_kv_heads,
                           int head_dim, int block_size, float scale, int causal,
                           void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
