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
 * Conventions shared by every device call (the block manager at the end of
 * this header is host-only and has its own)
 *  - Every array argument is a DEVICE pointer, allocated and owned by the
 *    caller, who keeps it alive until the enqueued work has finished.  The
 *    library allocates no device memory, frees nothing and keeps no state
 *    between calls; concurrent calls on different streams are safe when their
 *    output buffers (and workspaces) do not overlap.
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
 *    Values inside device arrays are not validated, apart from the slots of
 *    the append calls and the block ids of pkv_copy_blocks (skipped when
 *    outside the pool): a block-table entry outside the pool or a context
 *    length above max_blocks_per_seq * block_size is undefined behaviour.  A context
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
    PKV_ERR_ALIGN = -6,       /* a bf16 array is not 16-byte aligned */
    PKV_ERR_NO_MEMORY = -7,   /* block manager: too few free blocks; nothing changed */
    PKV_ERR_STATE = -8,       /* block manager: unknown or already existing sequence id */
    PKV_ERR_HOST_ALLOC = -9,  /* block manager: host memory ran out; nothing changed */
    PKV_ERR_VALUE = -10,      /* an FP8 cache scale is not finite and positive */
    PKV_ERR_SCRATCH = -11     /* the call needs more than the library's fixed scratch */
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
 *                  slot / block_size, row slot % block_size; slot < 0 skips t,
 *                  and so does slot >= num_blocks * block_size (a stale
 *                  mapping cannot write outside the pools).  Two tokens with
 *                  the same slot in one call is a caller error (which one
 *                  lands is unspecified).
 *   k_cache, v_cache  pools (written only at the given slots)
 *   num_blocks     pool size in blocks: slots are checked against it on the
 *                  device
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
 * ("LLM 推理优化技术全景", "Flash Attention 深度剖析 > 在线 Softmax": the keys
 * are visited once, block by block, keeping a running maximum m and running
 * sum l and rescaling the partial output by exp(m_old - m_new) when m grows;
 * "Flash Attention v2 的改进": the division by l is deferred to the end and the
 * work is also split along the sequence axis, here into pieces whose partial
 * results are merged by the same rescale; "Prefill vs Decode": decode reads
 * the whole cached K/V for one query row, so it is bound by HBM bandwidth;
 * the gather through the block table is that of "LLM 推理引擎深度解析：vLLM、
 * SGLang 与 TensorRT-LLM 的核心优化原理", section 2.1 "PagedAttention".)
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
 * block table.  fp32 accumulation throughout.  With 8 or 16 query heads per
 * KV head over bf16 pools the tile runs on the matrix cores: q.k as bf16 x
 * bf16 MFMA (exact products), P V as fp16 x fp16 MFMA with V rounded to
 * fp16 (exact for |v| in [2^-14, 65504]; smaller magnitudes keep an
 * absolute error below 2^-25, |v| > 65504 is outside the supported range)
 * and P in fp16 (relative error 2^-11); with 1, 2 or 4 V and P stay fp32.
 */
int pkv_paged_decode_attn(void *out, int out_dtype, const void *q, const void *k_cache,
                          const void *v_cache, const int32_t *block_table,
                          int max_blocks_per_seq, const int32_t *context_lens,
                          int max_context_len, int num_seqs, int num_q_heads,
                          int num_kv_heads, int head_dim, int block_size, float scale,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_decode_attn_noalloc -- pkv_paged_decode_attn for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments and results (the same
 * kernels, bit for bit) without the workspace: its partial results live in
 * a fixed scratch array inside the library, pkv_decode_noalloc_max_bytes()
 * bytes on each GPU, held until the process ends.  The call allocates and
 * frees nothing (no hipMalloc, no library routine that allocates).
 *   PKV_ERR_SCRATCH  pkv_decode_workspace_bytes() of these sizes exceeds
 *                    the scratch (checked on the host, nothing launched)
 *   PKV_ERR_LAUNCH   also when the scratch's device address cannot be found
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (nothing in it needs clearing): calls that overlap on one
 * GPU (different streams, or several threads) race and must be serialised
 * by the caller.
 */
int pkv_paged_decode_attn_noalloc(void *out, int out_dtype, const void *q, const void *k_cache,
                                  const void *v_cache, const int32_t *block_table,
                                  int max_blocks_per_seq, const int32_t *context_lens,
                                  int max_context_len, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int block_size, float scale,
                                  void *stream);

/* Size of the fixed scratch of pkv_paged_decode_attn_noalloc, in bytes. */
size_t pkv_decode_noalloc_max_bytes(void);

/*
 * FP8 KV cache ("让 Agent 跑得快：LLM 推理服务", section 四, FP8 量化: one byte
 * per value, half of bf16, so the bandwidth-bound decode moves half the
 * bytes; "LLM推理工程实战", section 5.3, KV Cache量化: the cache itself stored
 * quantised, as vLLM's kv_cache_dtype=fp8).
 *
 * Format: OCP FP8 E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, subnormals m * 2^-9, no infinities, S.1111.111 = NaN, largest
 * finite 448), one byte per value, in pools laid out exactly like the bf16
 * ones: [num_blocks][block_size][num_kv_heads][head_dim] uint8.  The cache
 * has one scale for K and one for V, chosen by the caller (finite, > 0):
 * the value a code stands for is E4M3(code) * scale.
 */

/*
 * kv_append_fp8 -- quantise new tokens' K and V rows into their slots.
 * Arguments as pkv_kv_append, except that k_cache / v_cache are the FP8
 * pools and k_scale / v_scale their scales.  Each bf16 value x is stored as
 * the E4M3 code nearest to x / scale (one correctly rounded binary32
 * division), clamped to +-448, ties to the even code.  Inputs must be
 * finite.  PKV_ERR_VALUE for a scale that is not finite and positive.
 */
int pkv_kv_append_fp8(const void *k_new, const void *v_new, const int64_t *slot_mapping,
                      int64_t num_tokens, void *k_cache, void *v_cache, int64_t num_blocks,
                      int block_size, int num_kv_heads, int head_dim, float k_scale,
                      float v_scale, void *stream);

/*
 * paged_decode_attn_fp8 -- pkv_paged_decode_attn over FP8 pools:
 *   out[i, h, :] = sum_t softmax_t(scale * <q[i,h], k_scale * Kc_i[t]>) v_scale * Vc_i[t]
 * with Kc, Vc the E4M3 values of the codes.  Same arguments, workspace and
 * limits as pkv_paged_decode_attn, plus the two scales.  The codes are
 * widened in registers, exactly: K to bf16, for q.k as bf16 x bf16 MFMA,
 * and V to fp16, for P V as fp16 x fp16 MFMA with P in fp16 (relative error
 * 2^-11); accumulation is fp32.  Codes of tokens past a sequence's length
 * are never used.
 */
int pkv_paged_decode_attn_fp8(void *out, int out_dtype, const void *q, const void *k_cache,
                              const void *v_cache, float k_scale, float v_scale,
                              const int32_t *block_table, int max_blocks_per_seq,
                              const int32_t *context_lens, int max_context_len, int num_seqs,
                              int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                              float scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * FP8 pools with one scale per (physical block, KV head) for K and one for
 * V, instead of one per cache (the same pages: FP8 quantisation of the KV
 * cache; a finer scale keeps a head or block of large values from pushing
 * the others' codes toward the subnormals).  k_scales / v_scales: device
 * arrays of fp32, [num_blocks][num_kv_heads], 4-byte aligned, owned by the
 * caller; a value stored in block b for KV head h stands for
 * E4M3(code) * scale[b][h].  The caller chooses the scales (for instance
 * from a block's absolute maximum when the block is first written) and
 * keeps them with the block: a block's scale must not change while it holds
 * codes.  Scales must be finite and > 0; other values give unspecified
 * results (never a memory access outside the arrays the caller passes).
 *
 * kv_append_fp8_per_block -- pkv_kv_append_fp8 with the scale of the block
 * each slot lies in (slot / block_size) and of the row's KV head: each
 * value x is stored as the E4M3 code nearest to x / scale[b][h] (one
 * correctly rounded binary32 division), clamped to +-448, ties to the even
 * code.  Slots past num_blocks * block_size, or negative, are skipped.
 * PKV_ERR_NULL if a table is NULL, PKV_ERR_ALIGN if one is not 4-byte
 * aligned; the other errors as pkv_kv_append_fp8.
 */
int pkv_kv_append_fp8_per_block(const void *k_new, const void *v_new,
                                const int64_t *slot_mapping, int64_t num_tokens, void *k_cache,
                                void *v_cache, int64_t num_blocks, int block_size,
                                int num_kv_heads, int head_dim, const float *k_scales,
                                const float *v_scales, void *stream);

/*
 * paged_decode_attn_fp8_per_block -- pkv_paged_decode_attn over FP8 pools
 * with per-(block, KV head) scales:
 *   out[i, h, :] = sum_t softmax_t(scale * <q[i,h], ks(t) * Kc_i[t]>) vs(t) * Vc_i[t]
 * with ks(t), vs(t) the scales of the block holding token t, for KV head
 * h / G.  Same arguments, workspace and limits as pkv_paged_decode_attn,
 * plus the two tables.  Each 16-token tile reads its block's two scales:
 * the K scale joins that tile's score scale, the V scale weights its P V
 * product as the ratio to the largest V scale seen so far (P times that
 * ratio rounds to fp16, relative error 2^-11); the rest as
 * pkv_paged_decode_attn_fp8.
 */
int pkv_paged_decode_attn_fp8_per_block(void *out, int out_dtype, const void *q,
                                        const void *k_cache, const void *v_cache,
                                        const float *k_scales, const float *v_scales,
                                        const int32_t *block_table, int max_blocks_per_seq,
                                        const int32_t *context_lens, int max_context_len,
                                        int num_seqs, int num_q_heads, int num_kv_heads,
                                        int head_dim, int block_size, float scale,
                                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Workspace needed by pkv_paged_prefill_attn and its FP8 and tree variants
 * (bytes, >= 0; 0 for inconsistent sizes), the larger of what the call's
 * path needs over bf16 and over FP8 pools.  With C = max_q_len *
 * (num_q_heads / num_kv_heads) query columns per KV head:
 *  - the rows path (2 <= max_q_len <= 16 and C <= 64, or C <= 32 over FP8
 *    pools; num_seqs <= 16383, num_kv_heads 1..8 or 16): 2 * num_seqs int32,
 *    256-byte aligned, then records of 132 floats for
 *    2 * max_q_len * num_q_heads columns of each of up to
 *    min(ceil(num_seqs * ceil(max_context_len / 16) / 4), 1024,
 *    2048 / num_kv_heads) workers;
 *  - else two parts, either of which may be absent: the decode workspace for
 *    the batch's single-row sequences, and the part of the stream-K chunk
 *    path, which takes calls whose chunks fit one workgroup
 *    (2 <= max_q_len and C <= 128): the (num_seqs + 1) int32 unit prefix
 *    sums, 256-byte aligned, then records of 132 floats for
 *    2 * max_q_len * (num_q_heads / num_kv_heads) columns of each of up to
 *    min(1024, num_seqs * num_kv_heads * ceil(max_context_len / 64))
 *    workers.
 * A call whose every sequence has exactly max_q_len rows, C > 128, needs
 * none (workspace may be NULL).  num_q_tokens is checked for consistency.
 */
size_t pkv_prefill_workspace_bytes(int num_seqs, int num_q_tokens, int max_q_len,
                                   int num_q_heads, int num_kv_heads, int head_dim,
                                   int max_context_len);

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
 * Rows with Lq_i == 1 take the bandwidth-bound decode path and longer
 * chunks the MFMA path.  When the call has both and its chunks do not fit
 * one workgroup, one grid runs them side by side on a 256-CU device (a
 * stream-K decode worker beside a chunk workgroup on every CU), then the
 * decode merge kernel; on another device the decode kernels follow the
 * chunk kernel on the same stream.  Short chunks (speculative-decoding
 * verification; the sizes of the rows path in the workspace comment above)
 * run on the decode kernel's stream-K split and matrix-core tile, a
 * sequence's (row, head) pairs the columns of its S = K Q^T, rows masked on
 * the tiles that reach the chunk, then the decode merge kernel.  Other
 * chunks that fit one workgroup run stream-K on the chunk kernel: all
 * (sequence, KV head, 64-key tile) units cut into equal ranges over the
 * workgroups the GPU holds at once, items shared by two workers merged by a
 * log-sum-exp fold in a second kernel.  num_seqs <= 16383 and num_kv_heads in 1..8 or 16 when
 * single-row sequences can be present; num_seqs <= 16383 for chunks that fit
 * one workgroup (PKV_ERR_UNSUPPORTED otherwise).  QK^T runs as bf16 x bf16 MFMA with fp32 accumulation;
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

/*
 * copy_blocks -- whole-block copies inside the pools, the device half of
 * copy-on-write ("让 Agent 跑得快：LLM 推理服务", section 二, "Copy-on-Write":
 * a shared block is copied only when a sequence must write into it, and that
 * sequence's table entry then points at the copy).
 *
 *   k_cache, v_cache  pools [num_blocks][block_size][num_kv_heads][head_dim]
 *                  bf16 (read at the sources, written at the destinations)
 *   block_mapping  [num_pairs][2] int64 DEVICE array of (source, destination)
 *                  physical block ids, as pkv_bm_append returns them; every
 *                  row of block `source` (all heads, K and V) is copied to
 *                  block `destination`, bit for bit.  A pair with an id
 *                  outside [0, num_blocks) is skipped on the device.
 *                  Destinations must be distinct and no destination may be
 *                  the source of another pair of the same call (the copies
 *                  run in no particular order).
 * num_pairs == 0 is a no-op.  Pools 16-byte aligned.
 */
int pkv_copy_blocks(void *k_cache, void *v_cache, int64_t num_blocks, int block_size,
                    int num_kv_heads, int head_dim, const int64_t *block_mapping,
                    int64_t num_pairs, void *stream);

/*
 * Block manager -- the host-side bookkeeping that produces block tables and
 * slot mappings.  ("LLM 推理引擎深度解析：vLLM、SGLang 与 TensorRT-LLM 的核心
 * 优化原理", section 2.1 "PagedAttention": a pool of fixed-size physical
 * blocks with a free list, a sequence of n tokens holding ceil(n /
 * block_size) not necessarily contiguous blocks, allocation failing when too
 * few are free, freeing returning a sequence's blocks; "让 Agent 跑得快：LLM
 * 推理服务", section 五: blocks taken on demand, one more whenever the last
 * is full, so at most block_size - 1 slots per sequence unused, and block
 * tables sharing physical blocks under a reference count; same page,
 * section 二, "Copy-on-Write": forked sequences share blocks and a shared
 * block is copied before a write.)
 *
 * Conventions of the pkv_bm_* calls
 *  - They run on the host only and touch no GPU; every array argument is a
 *    HOST pointer owned by the caller.  The manager owns its host memory
 *    until pkv_bm_destroy.  One manager must not be used from two threads at
 *    once; different managers are independent.
 *  - Physical block ids are 0 ... num_blocks - 1.  Blocks leave the front of
 *    the free list and return to its back when their count drops to zero.
 *  - Sequence ids are any int64 values chosen by the caller.
 *  - A call that fails returns a negative status and changes nothing
 *    (in particular PKV_ERR_NO_MEMORY leaves every table and count as it was).
 */
typedef struct pkv_block_manager pkv_block_manager;

/* A manager of num_blocks (0 ... 2^31 - 1) blocks of block_size token rows,
 * all free; NULL on bad sizes or when host memory runs out. */
pkv_block_manager *pkv_bm_create(int64_t num_blocks, int block_size);

/* Release the manager (NULL is a no-op). */
void pkv_bm_destroy(pkv_block_manager *bm);

/* Free blocks, or -1 for a NULL manager. */
int64_t pkv_bm_num_free(const pkv_block_manager *bm);

/* New sequence seq_id holding num_tokens (>= 0) tokens: takes
 * ceil(num_tokens / block_size) blocks.  PKV_ERR_STATE if seq_id exists,
 * PKV_ERR_NO_MEMORY if too few blocks are free. */
int pkv_bm_allocate(pkv_block_manager *bm, int64_t seq_id, int64_t num_tokens);

/*
 * Prefix caching ("让 Agent 跑得快：LLM 推理服务", section 七, automatic prefix
 * caching).  A new sequence seq_id holding the prompt tokens[0 .. num_tokens)
 * reuses cached blocks: its full blocks are identified by the chain of
 * (parent block's identity, the block's block_size tokens, salt) and looked
 * up in order; every hit joins the table with one more reference, and the
 * lookup stops at the first miss.  The remaining blocks are taken from the
 * free list and the prompt's new full blocks are registered (their K/V is
 * the caller's to write, from *num_cached_tokens on, before another request
 * reads them).  Released blocks stay matchable until the free list hands
 * them out again for new contents (allocation, append or copy), which drops
 * their registration, the longest-freed first.  Partly filled blocks and
 * blocks filled by later appends are not registered.  A different salt
 * never matches (tenant isolation).  Matching compares the stored tokens,
 * salt and parent hash, so a hash collision gives a miss, never a wrong hit.
 *   num_cached_tokens  (written) leading tokens already held by the hits, a
 *                      multiple of block_size: prefill starts there
 * PKV_ERR_STATE if seq_id exists; PKV_ERR_NO_MEMORY if the new blocks do not
 * fit (free cached hits count as taken); nothing changes on failure.
 */
int pkv_bm_allocate_cached(pkv_block_manager *bm, int64_t seq_id, const int32_t *tokens,
                           int64_t num_tokens, int64_t salt, int64_t *num_cached_tokens);

/* Registered (matchable) blocks, or -1 for a NULL manager. */
int64_t pkv_bm_num_cached(const pkv_block_manager *bm);

/*
 * Radix-tree prefix sharing ("LLM 推理优化技术全景", section "Prefix Caching 与
 * RadixAttention"; "让 Agent 跑得快", section 七, RadixAttention): a new
 * sequence seq_id holding tokens[0 .. num_tokens) reuses the longest prefix
 * it shares, token by token, with any cached prompt.  Cached prompts are the
 * entries of a compressed trie over tokens: each allocation registers its
 * prompt's tokens up to its last full block, with those blocks, and the
 * entry holds one reference on each (so their K/V outlives the sequence;
 * the partly filled last block is not registered).  With L the longest
 * common prefix and the donor the most recently used entry reaching it:
 * the new table shares the donor's first L / block_size blocks, and when L
 * is not a multiple of block_size the next block is a fresh one that the
 * caller fills by copying the donor's (copy_pair, with pkv_copy_blocks)
 * before prefilling tokens L .. num_tokens - 1.  A hit or a registration
 * makes an entry the most recently used.  When fewer blocks are free than
 * the call takes, entries are dropped least recently used first (never the
 * donor), releasing their references.  Independent of
 * pkv_bm_allocate_cached's chain cache.
 *   num_cached_tokens  (written) L: prefill starts there
 *   copy_pair          (written) [2] int64: (source, destination) block of
 *                      the copy, or (-1, -1)
 * PKV_ERR_STATE if seq_id exists; PKV_ERR_NO_MEMORY if the blocks do not fit
 * even with every entry but the donor dropped; nothing changes on failure.
 */
int pkv_bm_allocate_radix(pkv_block_manager *bm, int64_t seq_id, const int32_t *tokens,
                          int64_t num_tokens, int64_t *num_cached_tokens, int64_t *copy_pair);

/* Radix entries held, or -1 for a NULL manager. */
int64_t pkv_bm_radix_num_entries(const pkv_block_manager *bm);

/* Drop every radix entry, least recently used first, releasing its
 * references (blocks that reach zero join the free list in that order). */
int pkv_bm_radix_clear(pkv_block_manager *bm);

/* Drop seq_id; each of its blocks loses one reference and returns to the free
 * list at zero.  An unknown seq_id is ignored (PKV_OK). */
int pkv_bm_free(pkv_block_manager *bm, int64_t seq_id);

/* New sequence child with parent's tokens and blocks, every block gaining a
 * reference (nothing is copied).  PKV_ERR_STATE if parent is unknown or
 * child exists. */
int pkv_bm_fork(pkv_block_manager *bm, int64_t parent, int64_t child);

/*
 * Room for num_tokens (>= 0) more tokens of seq_id.
 *   slots        [num_tokens] int64 (written): the slot of each new token in
 *                order, slot = block * block_size + position % block_size,
 *                ready for pkv_kv_append's slot_mapping
 *   copies       [max_copies][2] int64 (written): (source, destination)
 *                blocks to copy with pkv_copy_blocks BEFORE the new tokens
 *                are written; may be NULL when max_copies is 0
 *   num_copies   (written) copies produced: 0, or 1 when the sequence's
 *                partly filled last block is shared (its count is above 1):
 *                the copy takes a fresh block, the table entry moves to it
 *                and the old block loses a reference.  A token that opens a
 *                new block takes a fresh private block and never copies.
 * PKV_ERR_NO_MEMORY if the copy and the new blocks need more than the free
 * list holds; PKV_ERR_SHAPE if a copy is needed and max_copies < 1.
 */
int pkv_bm_append(pkv_block_manager *bm, int64_t seq_id, int64_t num_tokens, int64_t *slots,
                  int64_t *copies, int64_t max_copies, int64_t *num_copies);

/*
 * pkv_bm_append for a whole batch in one call: sequence seq_ids[i] gets
 * num_tokens[i] (>= 0) more tokens, in order (an id may repeat).
 *   slots        [sum num_tokens] int64 (written): the batch's slots, entry
 *                by entry, each entry's in token order
 *   copies       [max_copies][2] int64 (written): the copies of all entries
 *                in order (at most one per entry, so num_seqs rows always
 *                suffice); may be NULL when max_copies is 0
 *   num_copies   (written) rows of copies used
 * All or nothing: if any entry fails (unknown id PKV_ERR_STATE, too few
 * blocks PKV_ERR_NO_MEMORY, copies full PKV_ERR_SHAPE) the entries before
 * it are undone, the free list included, and nothing has changed.
 */
int pkv_bm_append_batch(pkv_block_manager *bm, const int64_t *seq_ids, const int64_t *num_tokens,
                        int num_seqs, int64_t *slots, int64_t *copies, int64_t max_copies,
                        int64_t *num_copies);

/* Tokens and blocks held by seq_id (PKV_ERR_STATE if unknown). */
int pkv_bm_seq_info(const pkv_block_manager *bm, int64_t seq_id, int64_t *num_tokens,
                    int64_t *num_blocks);

/* Reference count of one block (0 = free); PKV_ERR_SHAPE if out of range. */
int pkv_bm_refcount(const pkv_block_manager *bm, int64_t block, int32_t *count);

/*
 * Block table and context lengths of num_seqs sequences, in the layout the
 * attention calls read.
 *   seq_ids       [num_seqs] int64
 *   table         [num_seqs][max_blocks_per_seq] int32 (written): row i holds
 *                 seq_ids[i]'s blocks in logical order, then -1
 *   context_lens  [num_seqs] int32 (written): tokens held
 * PKV_ERR_STATE for an unknown id, PKV_ERR_SHAPE if a sequence holds more
 * than max_blocks_per_seq blocks; nothing is written then.
 */
int pkv_bm_block_table(const pkv_block_manager *bm, const int64_t *seq_ids, int num_seqs,
                       int32_t *table, int max_blocks_per_seq, int32_t *context_lens);

/*
 * paged_prefill_attn_fp8 -- pkv_paged_prefill_attn over FP8 (E4M3) pools
 * (the format and scales of pkv_paged_decode_attn_fp8): k_cache / v_cache
 * hold one code byte per value, [num_blocks][block_size][num_kv_heads]
 * [head_dim]; keys and values are code value x k_scale / v_scale.  The chunk
 * kernels widen the codes to bf16 (K) and fp16 (V) as they stage a tile, so
 * the tile math is that of the bf16 call; single-row sequences take the FP8
 * decode path.  Workspace as pkv_prefill_workspace_bytes.  Scales must be
 * finite and > 0 (PKV_ERR_VALUE).
 */
int pkv_paged_prefill_attn_fp8(void *out, int out_dtype, const void *q,
                               const int32_t *cu_q_lens, const void *k_cache,
                               const void *v_cache, float k_scale, float v_scale,
                               const int32_t *block_table, int max_blocks_per_seq,
                               const int32_t *context_lens, int max_context_len, int max_q_len,
                               int num_q_tokens, int num_seqs, int num_q_heads, int num_kv_heads,
                               int head_dim, int block_size, float scale, int causal,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_prefill_attn_tree -- token-tree verification ("让 Agent 跑得快：LLM
 * 推理服务", section 六, Token Tree Verification: the draft candidates form a
 * tree, checked by the target model in one pass).  Arguments as
 * pkv_paged_prefill_attn with causal = 1, plus
 *   tree_mask   [num_q_tokens] uint64 device array: the Lq_i new tokens of
 *               sequence i are the nodes of its tree in topological order
 *               (every node after its parent); query row r sees every
 *               cached key before the new tokens and new token j exactly
 *               when bit j of tree_mask[cu_q_lens[i] + r] is set (its path
 *               to the root, itself included).  Bits above r are ignored:
 *               a node never sees a later one.  A mask of bits 0 .. r gives
 *               plain causal attention.
 * Every node must see itself (bit r of its own mask set), so that each row
 * sees at least one key.  tree_mask must be 8-byte aligned (PKV_ERR_ALIGN)
 * and non-NULL when there are rows (PKV_ERR_NULL); max_q_len <= 64
 * (PKV_ERR_UNSUPPORTED otherwise).  Sequences with a single row take the
 * decode path, as in pkv_paged_prefill_attn.
 */
int pkv_paged_prefill_attn_tree(void *out, int out_dtype, const void *q,
                                const int32_t *cu_q_lens, const uint64_t *tree_mask,
                                const void *k_cache, const void *v_cache,
                                const int32_t *block_table, int max_blocks_per_seq,
                                const int32_t *context_lens, int max_context_len, int max_q_len,
                                int num_q_tokens, int num_seqs, int num_q_heads, int num_kv_heads,
                                int head_dim, int block_size, float scale, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * paged_prefill_attn_tree_fp8 -- token-tree verification (as
 * pkv_paged_prefill_attn_tree) over FP8 (E4M3) pools with k_scale / v_scale
 * (as pkv_paged_prefill_attn_fp8).
 */
int pkv_paged_prefill_attn_tree_fp8(void *out, int out_dtype, const void *q,
                                    const int32_t *cu_q_lens, const uint64_t *tree_mask,
                                    const void *k_cache, const void *v_cache, float k_scale,
                                    float v_scale, const int32_t *block_table,
                                    int max_blocks_per_seq, const int32_t *context_lens,
                                    int max_context_len, int max_q_len, int num_q_tokens,
                                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, float scale, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * paged_prefill_attn_fp8_per_block / paged_prefill_attn_tree_fp8_per_block
 * -- pkv_paged_prefill_attn_fp8 and pkv_paged_prefill_attn_tree_fp8 over FP8
 * pools with per-(block, KV head) scales (the tables of
 * pkv_paged_decode_attn_fp8_per_block; same arguments otherwise, and the
 * same workspace, pkv_prefill_workspace_bytes).  Every key's score takes
 * the K scale of its block, and its value the V scale, as a ratio to the
 * largest V scale of the item's tiles so far: on the chunk kernels V is
 * staged as fp16(code x ratio) (the ratio rounded to fp16, the product
 * rounded once more); on the rows path (as over FP8 pools: chunks of at
 * most 16 rows and 32 (row, head) columns per KV head) P is scaled as in
 * the decode.  Chunks and single-row sequences in one call share one grid,
 * as over per-cache pools.
 */
int pkv_paged_prefill_attn_fp8_per_block(void *out, int out_dtype, const void *q,
                                         const int32_t *cu_q_lens, const void *k_cache,
                                         const void *v_cache, const float *k_scales,
                                         const float *v_scales, const int32_t *block_table,
                                         int max_blocks_per_seq, const int32_t *context_lens,
                                         int max_context_len, int max_q_len, int num_q_tokens,
                                         int num_seqs, int num_q_heads, int num_kv_heads,
                                         int head_dim, int block_size, float scale, int causal,
                                         void *workspace, size_t workspace_bytes, void *stream);
int pkv_paged_prefill_attn_tree_fp8_per_block(
    void *out, int out_dtype, const void *q, const int32_t *cu_q_lens, const uint64_t *tree_mask,
    const void *k_cache, const void *v_cache, const float *k_scales, const float *v_scales,
    const int32_t *block_table, int max_blocks_per_seq, const int32_t *context_lens,
    int max_context_len, int max_q_len, int num_q_tokens, int num_seqs, int num_q_heads,
    int num_kv_heads, int head_dim, int block_size, float scale, void *workspace,
    size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
