/*
 * pkv_oracle.c -- plain fp64 CPU reference for attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or helper with the HIP
 * library: it is written from the pages' definitions, deliberately slow and
 * obvious, with one loop per step of the definition.
 *
 * Sources (each function below names the passage it follows):
 *  [KVC]  "LLM 推理优化技术全景" (docs.ifdog.com, inference-optimization),
 *         section "KV Cache": per-layer K and V are kept and reused.
 *  [STD]  same page, "Flash Attention 深度剖析 > 标准注意力的问题": attention is
 *         Softmax(Q K^T) V.
 *  [SMX]  same page, "在线 Softmax": the numerically stable softmax subtracts
 *         the row maximum m and divides by the sum of exp(x - m); done directly
 *         it takes three sweeps (max, sum, divide) -- which is what this
 *         oracle does on purpose.
 *  [PA]   "LLM 推理引擎深度解析：vLLM、SGLang 与 TensorRT-LLM 的核心优化原理"
 *         (jsjson.com), section 2.1 "PagedAttention": the pools are
 *         zeros(num_blocks, block_size, num_heads, head_dim) and a per-sequence
 *         block table maps logical block j to a physical block id.
 *  [PA5]  "让 Agent 跑得快：LLM 推理服务" (hkg.20260401.xyz agent-book-07),
 *         section 五 "PagedAttention 的深度解析": a new physical block per 16
 *         generated tokens; only the current decode token writes; several
 *         block tables may point at the same read-only block.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - scores carry a caller-given scale (the pages write Softmax(QK^T)V bare);
 *  - query head h reads KV head floor(h / (Hq/Hkv)) (contiguous GQA groups);
 *  - the pool's head axis is the KV-head axis;
 *  - sequence i's Lq_i query rows sit at absolute positions
 *    ctx_i - Lq_i ... ctx_i - 1; with `causal` row r sees keys t <= its
 *    position, otherwise all ctx_i keys; decode is Lq_i = 1;
 *  - ctx_i = 0 gives an all-zero output row;
 *  - slot s < 0 in an append means "no write"; slot s >= 0 lands in physical
 *    block s / block_size at row s % block_size.
 *
 * All floating point is fp64.  bf16 inputs are widened exactly (a bf16 value
 * is the top 16 bits of the binary32 with the same value).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_RANGE (-2)
#define ORACLE_ERR_NOMEM (-3)

/* Exact widening of a bf16 bit pattern to double. */
static double widen_bf16(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Reference for kv_append [KVC], [PA5]: for each new token t with slot
 * s = slot_mapping[t] >= 0, copy its Hkv*D K row and V row, byte for byte,
 * to pool row (s / block_size, s % block_size).  Returns ORACLE_ERR_RANGE,
 * before writing anything, if a slot lies outside the pool.
 */
int oracle_kv_append(const uint16_t *k_new, const uint16_t *v_new,
                     const int64_t *slot_mapping, int64_t num_tokens,
                     uint16_t *k_cache, uint16_t *v_cache,
                     int64_t num_blocks, int block_size, int num_kv_heads,
                     int head_dim)
{
    if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache)
        return ORACLE_ERR_ARG;
    if (num_tokens < 0 || num_blocks < 0 || block_size <= 0 ||
        num_kv_heads <= 0 || head_dim <= 0)
        return ORACLE_ERR_ARG;
    for (int64_t t = 0; t < num_tokens; ++t)
        if (slot_mapping[t] >= num_blocks * (int64_t)block_size)
            return ORACLE_ERR_RANGE;

    size_t row = (size_t)num_kv_heads * (size_t)head_dim; /* elements per token */
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t s = slot_mapping[t];
        if (s < 0)
            continue;
        int64_t block = s / block_size;
        int64_t offset = s % block_size;
        size_t dst = ((size_t)block * (size_t)block_size + (size_t)offset) * row;
        memcpy(k_cache + dst, k_new + (size_t)t * row, row * sizeof(uint16_t));
        memcpy(v_cache + dst, v_new + (size_t)t * row, row * sizeof(uint16_t));
    }
    return ORACLE_OK;
}

/*
 * Gather step [PA], [PA5]: the ctx keys/values of one sequence and one KV head
 * copied, widened to fp64, into contiguous [ctx, D] arrays.  Logical token t
 * lives in physical block block_table_row[t / block_size] at row
 * t % block_size.
 */
static int gather_head(double *K, double *V, const uint16_t *k_cache,
                       const uint16_t *v_cache, const int32_t *block_table_row,
                       int64_t num_blocks, int ctx, int block_size,
                       int num_kv_heads, int head_dim, int kv_head)
{
    for (int t = 0; t < ctx; ++t) {
        int32_t phys = block_table_row[t / block_size];
        if (phys < 0 || (int64_t)phys >= num_blocks)
            return ORACLE_ERR_RANGE;
        size_t base = (((size_t)phys * (size_t)block_size + (size_t)(t % block_size)) *
                           (size_t)num_kv_heads + (size_t)kv_head) * (size_t)head_dim;
        for (int d = 0; d < head_dim; ++d) {
            K[(size_t)t * head_dim + d] = widen_bf16(k_cache[base + d]);
            V[(size_t)t * head_dim + d] = widen_bf16(v_cache[base + d]);
        }
    }
    return ORACLE_OK;
}

/*
 * Attention over the paged cache, three-pass softmax [STD], [SMX]:
 *   out[row, h, :] = sum_t exp(s_t - m) V[t, :] / sum_t exp(s_t - m),
 *   s_t = scale * <q[row, h, :], K[t, :]>,  m = max_t s_t,
 * t running over the keys the row may see (all ctx_i keys, or t <= position
 * when causal).  `cu_q_lens` ([num_seqs + 1], prefix sums of Lq_i) may be
 * NULL, meaning one query row per sequence (decode).  q is
 * [sum Lq, Hq, D] bf16; out is [sum Lq, Hq, D] fp64.
 *
 * Work is split over (sequence, KV head) pairs with OpenMP; each pair's
 * arithmetic is independent, so the thread count does not change any result.
 * num_threads <= 0 keeps the OpenMP default.
 */
int oracle_paged_attention(double *out, const uint16_t *q, const int32_t *cu_q_lens,
                           const uint16_t *k_cache, const uint16_t *v_cache,
                           int64_t num_blocks, const int32_t *block_table,
                           int max_blocks_per_seq, const int32_t *context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads,
                           int head_dim, int block_size, double scale, int causal,
                           int num_threads)
{
    if (!out || !q || !k_cache || !v_cache || !block_table || !context_lens)
        return ORACLE_ERR_ARG;
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq < 0 || num_q_heads % num_kv_heads != 0)
        return ORACLE_ERR_ARG;
    for (int i = 0; i < num_seqs; ++i) {
        int ctx = context_lens[i];
        int lq = cu_q_lens ? cu_q_lens[i + 1] - cu_q_lens[i] : 1;
        if (ctx < 0 || lq < 0 || (int64_t)ctx > (int64_t)max_blocks_per_seq * block_size)
            return ORACLE_ERR_RANGE;
        if (lq > ctx && ctx > 0)
            return ORACLE_ERR_RANGE; /* a query position would be negative */
    }
#ifdef _OPENMP
    if (num_threads > 0)
        omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
    const int group = num_q_heads / num_kv_heads;
    const long long pairs = (long long)num_seqs * num_kv_heads;
    int status = ORACLE_OK;

#pragma omp parallel for schedule(dynamic, 1)
    for (long long pair = 0; pair < pairs; ++pair) {
        int i = (int)(pair / num_kv_heads);
        int kvh = (int)(pair % num_kv_heads);
        int ctx = context_lens[i];
        int lq = cu_q_lens ? cu_q_lens[i + 1] - cu_q_lens[i] : 1;
        long long row0 = cu_q_lens ? cu_q_lens[i] : i;

        if (ctx == 0) { /* nothing to attend to: defined as zeros */
            for (int r = 0; r < lq; ++r)
                for (int g = 0; g < group; ++g) {
                    int h = kvh * group + g;
                    double *o = out + ((size_t)(row0 + r) * num_q_heads + h) * head_dim;
                    for (int d = 0; d < head_dim; ++d)
                        o[d] = 0.0;
                }
            continue;
        }

        double *K = malloc(sizeof(double) * (size_t)ctx * head_dim);
        double *V = malloc(sizeof(double) * (size_t)ctx * head_dim);
        double *s = malloc(sizeof(double) * (size_t)ctx);
        double *qd = malloc(sizeof(double) * (size_t)head_dim);
        if (!K || !V || !s || !qd) {
            free(K); free(V); free(s); free(qd);
#pragma omp critical
            status = ORACLE_ERR_NOMEM;
            continue;
        }
        int gs = gather_head(K, V, k_cache, v_cache,
                             block_table + (size_t)i * max_blocks_per_seq, num_blocks,
                             ctx, block_size, num_kv_heads, head_dim, kvh);
        if (gs != ORACLE_OK) {
            free(K); free(V); free(s); free(qd);
#pragma omp critical
            status = gs;
            continue;
        }

        for (int r = 0; r < lq; ++r) {
            int pos = ctx - lq + r;                 /* absolute position of the row */
            int visible = causal ? pos + 1 : ctx;   /* keys t < visible are seen */
            for (int g = 0; g < group; ++g) {
                int h = kvh * group + g;
                const uint16_t *qrow = q + ((size_t)(row0 + r) * num_q_heads + h) * head_dim;
                double *o = out + ((size_t)(row0 + r) * num_q_heads + h) * head_dim;
                for (int d = 0; d < head_dim; ++d)
                    qd[d] = widen_bf16(qrow[d]);

                /* scores */
                for (int t = 0; t < visible; ++t) {
                    double dot = 0.0;
                    for (int d = 0; d < head_dim; ++d)
                        dot += qd[d] * K[(size_t)t * head_dim + d];
                    s[t] = scale * dot;
                }
                /* pass 1: the row maximum */
                double m = -INFINITY;
                for (int t = 0; t < visible; ++t)
                    if (s[t] > m)
                        m = s[t];
                /* pass 2: the sum of exponentials */
                double l = 0.0;
                for (int t = 0; t < visible; ++t)
                    l += exp(s[t] - m);
                /* pass 3: normalised weights times V */
                for (int d = 0; d < head_dim; ++d)
                    o[d] = 0.0;
                for (int t = 0; t < visible; ++t) {
                    double p = exp(s[t] - m) / l;
                    for (int d = 0; d < head_dim; ++d)
                        o[d] += p * V[(size_t)t * head_dim + d];
                }
            }
        }
        free(K); free(V); free(s); free(qd);
    }
    return status;
}

/* Threads the OpenMP runtime would use by default (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
