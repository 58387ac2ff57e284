// api.hip -- the C ABI of libpagedkv.so (declared in include/pagedkv.h):
// argument validation on the host, then the launch on the caller's stream.
// Every check runs before anything is enqueued, so all error statuses can be
// exercised without a GPU.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "pagedkv.h"
#include "pkv_device.h"
#include "pkv_launch.h"

namespace {

constexpr int kVersion = 200;  // 0.2.0
// Decode keeps the per-sequence tile prefix sums in LDS: (num_seqs + 1) int32
// must fit the 64 KB a workgroup may allocate.
constexpr int kMaxDecodeSeqs = 16383;
// A decode workgroup serves up to 8 KV heads, one wave each; 16 heads run as
// two groups of 8.
constexpr int kMaxDecodeKvHeads = 16;
// A token-tree mask is one 64-bit word per node.
constexpr int kMaxTreeNodes = 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A cache scale: finite and positive.
bool valid_scale(float s) { return s > 0.0f && s <= 3.402823466e38f; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Shape checks shared by decode and prefill.
int check_attention_shape(int max_blocks_per_seq, int max_context_len, int num_seqs,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int out_dtype) {
    if (out_dtype != PKV_OUT_F32 && out_dtype != PKV_OUT_BF16) return PKV_ERR_UNSUPPORTED;
    if (head_dim != pkv::kHeadDim) return PKV_ERR_UNSUPPORTED;
    if (block_size != 16 && block_size != 32) return PKV_ERR_UNSUPPORTED;
    if (num_seqs < 0 || num_seqs > 65535 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        max_blocks_per_seq < 0 || max_context_len < 0)
        return PKV_ERR_SHAPE;
    if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
    if (!supported_group(num_q_heads / num_kv_heads)) return PKV_ERR_UNSUPPORTED;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PKV_ERR_SHAPE;
    return PKV_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH; }

// The fixed scratch of pkv_paged_decode_attn_noalloc: the decode workspace
// of calls that may not allocate, in the library's own device memory.  Each
// GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in: its device address is
// fetched once per device (hipGetSymbolAddress, that device current) and
// only that address is passed on.
constexpr size_t kScratchBytes = (size_t)80 << 20;
__device__ __attribute__((aligned(256))) static char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch, or NULL (with *err set).
void* scratch_address(hipError_t* err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

// Calls whose chunks have at most 16 rows and 64 (row, head) columns per KV
// head, 32 over FP8 pools (speculative-decoding verification, token trees),
// run whole on the decode kernel's matrix-core tile, every sequence's rows
// as columns of its S = K Q^T; wider ones on the chunk kernels.
constexpr int kRowsPathMaxRows = 16;
bool rows_path(int num_seqs, int max_q_len, int num_q_heads, int num_kv_heads, bool kv_fp8) {
    const int cols = max_q_len * (num_q_heads / num_kv_heads);
    return max_q_len >= 2 && max_q_len <= kRowsPathMaxRows && cols <= (kv_fp8 ? 32 : 64) &&
           num_seqs <= kMaxDecodeSeqs && (num_kv_heads <= 8 || num_kv_heads == kMaxDecodeKvHeads);
}

// The chunk kernels' workspace: the decode kernels' part for single-row
// sequences, then, when the call's chunks fit one workgroup (stream-K), that
// kernel's prefix sums and records at *chunk_offset.
size_t chunk_workspace(int num_seqs, int max_q_len, int num_q_heads, int num_kv_heads,
                       int head_dim, int max_context_len, size_t* chunk_offset) {
    // decode records are per query head, so the KV head count does not matter here
    const size_t dec = pkv::decode_workspace_bytes(num_seqs, num_q_heads, 1, head_dim,
                                                   max_context_len);
    if (chunk_offset) *chunk_offset = 0;
    const int group = num_q_heads / num_kv_heads;
    if (!pkv::prefill_streamk(max_q_len, group)) return dec;
    const size_t off = align_up(dec, 256);
    if (chunk_offset) *chunk_offset = off;
    return off + pkv::prefill_streamk_bytes(num_seqs, max_q_len, group, num_kv_heads,
                                            max_context_len);
}

// The rows path's workspace: the decode kernels' for max_q_len rows.
size_t rows_workspace(int num_seqs, int max_q_len, int num_q_heads, int num_kv_heads,
                      int head_dim, int max_context_len) {
    return pkv::decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       max_context_len, max_q_len);
}

// What a prefill call of these sizes needs over either pool type (the rows
// path takes more columns over bf16 pools than over FP8 ones).
size_t prefill_workspace(int num_seqs, int max_q_len, int num_q_heads, int num_kv_heads,
                         int head_dim, int max_context_len) {
    size_t n = 0;
    for (const bool fp8 : {false, true}) {
        const size_t c =
            rows_path(num_seqs, max_q_len, num_q_heads, num_kv_heads, fp8)
                ? rows_workspace(num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim,
                                 max_context_len)
                : chunk_workspace(num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim,
                                  max_context_len, nullptr);
        n = c > n ? c : n;
    }
    return n;
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
    switch (status) {
        case PKV_OK: return "ok";
        case PKV_ERR_NULL: return "a required pointer is NULL";
        case PKV_ERR_SHAPE: return "inconsistent sizes";
        case PKV_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, group size or dtype";
        case PKV_ERR_WORKSPACE: return "workspace missing or too small";
        case PKV_ERR_LAUNCH: return "HIP launch error";
        case PKV_ERR_ALIGN: return "a bf16 or output array is not 16-byte aligned";
        case PKV_ERR_NO_MEMORY: return "not enough free KV blocks";
        case PKV_ERR_STATE: return "unknown or already existing sequence id";
        case PKV_ERR_HOST_ALLOC: return "host memory allocation failed";
        case PKV_ERR_VALUE: return "a scale is not finite and positive";
        case PKV_ERR_SCRATCH: return "the call needs more than the library's fixed scratch";
        default: return "unknown status";
    }
}

int pkv_version(void) { return kVersion; }

int pkv_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                  int64_t num_tokens, void* k_cache, void* v_cache, int64_t num_blocks,
                  int block_size, int num_kv_heads, int head_dim, void* stream) {
    if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0) return PKV_ERR_SHAPE;
    if (head_dim != pkv::kHeadDim) return PKV_ERR_UNSUPPORTED;
    if (block_size != 16 && block_size != 32) return PKV_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PKV_OK;
    if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_ERR_ALIGN;
    pkv::AppendArgs a;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.k_cache = static_cast<uint16_t*>(k_cache);
    a.v_cache = static_cast<uint16_t*>(v_cache);
    a.row_elems = num_kv_heads * head_dim;
    a.num_slots = num_blocks * block_size;
    return to_status(pkv::launch_kv_append(a, static_cast<hipStream_t>(stream)));
}

int pkv_copy_blocks(void* k_cache, void* v_cache, int64_t num_blocks, int block_size,
                    int num_kv_heads, int head_dim, const int64_t* block_mapping,
                    int64_t num_pairs, void* stream) {
    if (num_pairs < 0 || num_blocks < 0 || num_kv_heads <= 0) return PKV_ERR_SHAPE;
    if (head_dim != pkv::kHeadDim) return PKV_ERR_UNSUPPORTED;
    if (block_size != 16 && block_size != 32) return PKV_ERR_UNSUPPORTED;
    if (num_pairs == 0) return PKV_OK;
    if (!k_cache || !v_cache || !block_mapping) return PKV_ERR_NULL;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_ALIGN;
    pkv::CopyBlocksArgs a;
    a.k_cache = static_cast<uint16_t*>(k_cache);
    a.v_cache = static_cast<uint16_t*>(v_cache);
    a.block_mapping = block_mapping;
    a.num_pairs = num_pairs;
    a.num_blocks = num_blocks;
    a.block_elems = (int64_t)block_size * num_kv_heads * head_dim;
    return to_status(pkv::launch_copy_blocks(a, static_cast<hipStream_t>(stream)));
}

size_t pkv_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                  int max_context_len) {
    if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0) return 0;
    return pkv::decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       max_context_len);
}

}  // extern "C"

namespace {

// Validation and launch shared by the bf16 and FP8 decode calls.
int decode_call(void* out, int out_dtype, const void* q, const void* k_cache, const void* v_cache,
                bool kv_fp8, float k_scale, float v_scale, const int32_t* block_table,
                int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                float scale, void* workspace, size_t workspace_bytes, void* stream,
                bool fixed_scratch = false, const float* k_scales = nullptr,
                const float* v_scales = nullptr) {
    int st = check_attention_shape(max_blocks_per_seq, max_context_len, num_seqs, num_q_heads,
                                   num_kv_heads, head_dim, block_size, out_dtype);
    if (st != PKV_OK) return st;
    if (num_seqs > kMaxDecodeSeqs) return PKV_ERR_UNSUPPORTED;
    if (num_kv_heads > 8 && num_kv_heads != kMaxDecodeKvHeads) return PKV_ERR_UNSUPPORTED;
    if (kv_fp8 && !(valid_scale(k_scale) && valid_scale(v_scale))) return PKV_ERR_VALUE;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_cache || !v_cache || !block_table || !context_lens) return PKV_ERR_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_ERR_ALIGN;
    if (kv_fp8 && (k_scales != nullptr || v_scales != nullptr)) {
        if (!k_scales || !v_scales) return PKV_ERR_NULL;
        if (!aligned4(k_scales) || !aligned4(v_scales)) return PKV_ERR_ALIGN;
    }
    const size_t need = pkv::decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                    max_context_len);
    if (fixed_scratch) {
        if (need > kScratchBytes) return PKV_ERR_SCRATCH;
        hipError_t e = hipSuccess;
        workspace = scratch_address(&e);
        if (!workspace) return PKV_ERR_LAUNCH;
        workspace_bytes = kScratchBytes;
    }
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PKV_ERR_ALIGN;

    pkv::DecodeArgs a;
    a.out = out;
    a.out_bf16 = out_dtype == PKV_OUT_BF16;
    a.q = static_cast<const uint16_t*>(q);
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.kv_fp8 = kv_fp8;
    a.out_scale = kv_fp8 ? v_scale : 1.0f;
    a.block_table = block_table;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.max_context_len = max_context_len;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.scale_log2 = scale * 1.4426950408889634f;
    if (kv_fp8) a.scale_log2 *= k_scale;
    if (kv_fp8 && k_scales) {
        a.k_scales = k_scales;
        a.v_scales = v_scales;
    }
    a.seq_workers = static_cast<int32_t*>(workspace);
    a.records = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         align_up((size_t)2 * num_seqs * sizeof(int32_t), 256));
    a.max_workers = pkv::decode_max_workers(num_seqs, max_context_len);
    a.cu_q_lens = nullptr;
    return to_status(pkv::launch_decode(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int pkv_paged_decode_attn(void* out, int out_dtype, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* block_table,
                          int max_blocks_per_seq, const int32_t* context_lens,
                          int max_context_len, int num_seqs, int num_q_heads, int num_kv_heads,
                          int head_dim, int block_size, float scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
    return decode_call(out, out_dtype, q, k_cache, v_cache, false, 1.0f, 1.0f, block_table,
                       max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, block_size, scale, workspace, workspace_bytes,
                       stream);
}

int pkv_paged_decode_attn_noalloc(void* out, int out_dtype, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  int max_blocks_per_seq, const int32_t* context_lens,
                                  int max_context_len, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int block_size, float scale,
                                  void* stream) {
    return decode_call(out, out_dtype, q, k_cache, v_cache, false, 1.0f, 1.0f, block_table,
                       max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, block_size, scale, nullptr, 0, stream, true);
}

size_t pkv_decode_noalloc_max_bytes(void) { return kScratchBytes; }

int pkv_paged_decode_attn_fp8(void* out, int out_dtype, const void* q, const void* k_cache,
                              const void* v_cache, float k_scale, float v_scale,
                              const int32_t* block_table, int max_blocks_per_seq,
                              const int32_t* context_lens, int max_context_len, int num_seqs,
                              int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                              float scale, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_call(out, out_dtype, q, k_cache, v_cache, true, k_scale, v_scale, block_table,
                       max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, block_size, scale, workspace, workspace_bytes,
                       stream);
}

int pkv_paged_decode_attn_fp8_per_block(void* out, int out_dtype, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const float* k_scales, const float* v_scales,
                                        const int32_t* block_table, int max_blocks_per_seq,
                                        const int32_t* context_lens, int max_context_len,
                                        int num_seqs, int num_q_heads, int num_kv_heads,
                                        int head_dim, int block_size, float scale,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    if (num_seqs > 0 && (!k_scales || !v_scales)) return PKV_ERR_NULL;
    return decode_call(out, out_dtype, q, k_cache, v_cache, true, 1.0f, 1.0f, block_table,
                       max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, block_size, scale, workspace, workspace_bytes,
                       stream, false, k_scales, v_scales);
}

}  // extern "C"

namespace {

int append_fp8_call(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                    int64_t num_tokens, void* k_cache, void* v_cache, int64_t num_blocks,
                    int block_size, int num_kv_heads, int head_dim, float k_scale, float v_scale,
                    const float* k_scales, const float* v_scales, void* stream) {
    if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0) return PKV_ERR_SHAPE;
    if (head_dim != pkv::kHeadDim) return PKV_ERR_UNSUPPORTED;
    if (block_size != 16 && block_size != 32) return PKV_ERR_UNSUPPORTED;
    if (!(valid_scale(k_scale) && valid_scale(v_scale))) return PKV_ERR_VALUE;
    if (num_tokens == 0) return PKV_OK;
    if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_ERR_ALIGN;
    if (k_scales || v_scales) {
        if (!k_scales || !v_scales) return PKV_ERR_NULL;
        if (!aligned4(k_scales) || !aligned4(v_scales)) return PKV_ERR_ALIGN;
    }
    pkv::AppendFp8Args a;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.k_cache = static_cast<uint8_t*>(k_cache);
    a.v_cache = static_cast<uint8_t*>(v_cache);
    a.row_elems = num_kv_heads * head_dim;
    a.num_slots = num_blocks * block_size;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    a.block_size = block_size;
    return to_status(pkv::launch_kv_append_fp8(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int pkv_kv_append_fp8(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                      int64_t num_tokens, void* k_cache, void* v_cache, int64_t num_blocks,
                      int block_size, int num_kv_heads, int head_dim, float k_scale,
                      float v_scale, void* stream) {
    return append_fp8_call(k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache, num_blocks,
                           block_size, num_kv_heads, head_dim, k_scale, v_scale, nullptr,
                           nullptr, stream);
}

int pkv_kv_append_fp8_per_block(const void* k_new, const void* v_new,
                                const int64_t* slot_mapping, int64_t num_tokens, void* k_cache,
                                void* v_cache, int64_t num_blocks, int block_size,
                                int num_kv_heads, int head_dim, const float* k_scales,
                                const float* v_scales, void* stream) {
    if (num_tokens > 0 && (!k_scales || !v_scales)) return PKV_ERR_NULL;
    return append_fp8_call(k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache, num_blocks,
                           block_size, num_kv_heads, head_dim, 1.0f, 1.0f, k_scales, v_scales,
                           stream);
}

size_t pkv_prefill_workspace_bytes(int num_seqs, int num_q_tokens, int max_q_len,
                                   int num_q_heads, int num_kv_heads, int head_dim,
                                   int max_context_len) {
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        num_q_tokens < 0 || max_q_len < 0 || num_q_heads % num_kv_heads != 0)
        return 0;
    return prefill_workspace(num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim,
                             max_context_len);
}

}  // extern "C"

namespace {

int prefill_call(void* out, int out_dtype, const void* q, const int32_t* cu_q_lens,
                 const void* k_cache, const void* v_cache, bool kv_fp8, float k_scale,
                 float v_scale, const int32_t* block_table,
                 int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                 int max_q_len, int num_q_tokens, int num_seqs, int num_q_heads,
                 int num_kv_heads, int head_dim, int block_size, float scale, int causal,
                 const uint64_t* tree_mask, void* workspace, size_t workspace_bytes,
                 void* stream, const float* k_scales = nullptr, const float* v_scales = nullptr) {
    int st = check_attention_shape(max_blocks_per_seq, max_context_len, num_seqs, num_q_heads,
                                   num_kv_heads, head_dim, block_size, out_dtype);
    if (st != PKV_OK) return st;
    if (max_q_len < 0 || num_q_tokens < 0) return PKV_ERR_SHAPE;
    if (max_q_len > max_context_len) return PKV_ERR_SHAPE;
    if (kv_fp8 && !(valid_scale(k_scale) && valid_scale(v_scale))) return PKV_ERR_VALUE;
    if ((int64_t)num_q_tokens > (int64_t)num_seqs * max_q_len) return PKV_ERR_SHAPE;
    if (num_seqs == 0 || num_q_tokens == 0) return PKV_OK;
    if (!out || !q || !cu_q_lens || !k_cache || !v_cache || !block_table || !context_lens)
        return PKV_ERR_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_ERR_ALIGN;
    const bool block_scales = kv_fp8 && (k_scales != nullptr || v_scales != nullptr);
    if (block_scales) {
        if (!k_scales || !v_scales) return PKV_ERR_NULL;
        if (!aligned4(k_scales) || !aligned4(v_scales)) return PKV_ERR_ALIGN;
    }
    // Rows of sequences with a single query go to the bandwidth-bound decode
    // kernels; they can exist unless every sequence has max_q_len > 1 rows.
    const bool uniform_chunks = max_q_len > 1 && (int64_t)num_q_tokens == (int64_t)num_seqs * max_q_len;
    const bool any_decode_rows = !uniform_chunks;
    const bool decode_limits_ok = num_seqs <= kMaxDecodeSeqs &&
                                  (num_kv_heads <= 8 || num_kv_heads == kMaxDecodeKvHeads);
    const bool rows = rows_path(num_seqs, max_q_len, num_q_heads, num_kv_heads, kv_fp8);
    const bool streamk = !rows && pkv::prefill_streamk(max_q_len, num_q_heads / num_kv_heads);
    if (any_decode_rows && !decode_limits_ok) return PKV_ERR_UNSUPPORTED;
    // the stream-K chunk kernel keeps the sequences' unit prefix sums in LDS
    // beside its two tile buffers
    if (streamk && num_seqs > kMaxDecodeSeqs) return PKV_ERR_UNSUPPORTED;
    size_t chunk_off = 0;
    if (any_decode_rows || streamk || rows) {
        const size_t need =
            rows ? rows_workspace(num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim,
                                  max_context_len)
                 : chunk_workspace(num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim,
                                   max_context_len, &chunk_off);
        if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return PKV_ERR_ALIGN;
    }

    pkv::PrefillArgs a;
    a.out = out;
    a.out_bf16 = out_dtype == PKV_OUT_BF16;
    a.q = static_cast<const uint16_t*>(q);
    a.cu_q_lens = cu_q_lens;
    a.k_cache = static_cast<const uint16_t*>(k_cache);
    a.v_cache = static_cast<const uint16_t*>(v_cache);
    a.block_table = block_table;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.max_context_len = max_context_len;
    a.max_q_len = max_q_len;
    a.num_q_tokens = num_q_tokens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.scale_log2 = scale * 1.4426950408889634f;
    if (kv_fp8) a.scale_log2 *= k_scale;
    a.kv_fp8 = kv_fp8;
    a.out_scale = kv_fp8 ? v_scale : 1.0f;
    a.causal = causal != 0;
    a.decode_rows_elsewhere = any_decode_rows;
    a.streamk = streamk;
    if (streamk) {
        char* base = static_cast<char*>(workspace) + chunk_off;
        a.cum = reinterpret_cast<int32_t*>(base);
        a.records = reinterpret_cast<float*>(
            base + align_up((size_t)(num_seqs + 1) * sizeof(int32_t), 256));
        a.max_workers = pkv::prefill_streamk_max_workers(num_seqs, num_kv_heads, max_context_len);
    }
    a.tree_mask = tree_mask;
    if (block_scales) {
        a.k_scales = k_scales;
        a.v_scales = v_scales;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!any_decode_rows && !rows) return to_status(pkv::launch_prefill(a, s));

    pkv::DecodeArgs d;
    d.out = out;
    d.out_bf16 = a.out_bf16;
    d.q = a.q;
    d.k_cache = a.k_cache;
    d.v_cache = a.v_cache;
    d.block_table = block_table;
    d.max_blocks_per_seq = max_blocks_per_seq;
    d.context_lens = context_lens;
    d.max_context_len = max_context_len;
    d.num_seqs = num_seqs;
    d.num_q_heads = num_q_heads;
    d.num_kv_heads = num_kv_heads;
    d.block_size = block_size;
    d.scale_log2 = a.scale_log2;
    d.kv_fp8 = kv_fp8;
    d.out_scale = a.out_scale;
    d.seq_workers = static_cast<int32_t*>(workspace);
    d.records = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         align_up((size_t)2 * num_seqs * sizeof(int32_t), 256));
    d.max_workers = pkv::decode_max_workers(num_seqs, max_context_len);
    d.cu_q_lens = cu_q_lens;
    d.k_scales = a.k_scales;
    d.v_scales = a.v_scales;
    if (rows) {
        d.rows = max_q_len;
        d.causal = causal != 0;
        d.tree_mask = tree_mask;
        d.max_workers = pkv::decode_max_workers(num_seqs, max_context_len, max_q_len, num_kv_heads);
        return to_status(pkv::launch_decode(d, s));
    }
    if (max_q_len > 1 && !streamk) {
        // chunks and decode rows in one grid, sharing the CUs
        const hipError_t e = pkv::launch_mixed(a, d, s);
        if (e != hipErrorNotSupported) return to_status(e);
    }
    if (max_q_len > 1) {
        st = to_status(pkv::launch_prefill(a, s));
        if (st != PKV_OK) return st;
    }
    return to_status(pkv::launch_decode(d, s));
}

}  // namespace

extern "C" {

int pkv_paged_prefill_attn(void* out, int out_dtype, const void* q, const int32_t* cu_q_lens,
                           const void* k_cache, const void* v_cache, const int32_t* block_table,
                           int max_blocks_per_seq, const int32_t* context_lens,
                           int max_context_len, int max_q_len, int num_q_tokens, int num_seqs,
                           int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                           float scale, int causal, void* workspace, size_t workspace_bytes,
                           void* stream) {
    return prefill_call(out, out_dtype, q, cu_q_lens, k_cache, v_cache, false, 1.0f, 1.0f,
                        block_table, max_blocks_per_seq, context_lens, max_context_len, max_q_len,
                        num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                        scale, causal, nullptr, workspace, workspace_bytes, stream);
}

int pkv_paged_prefill_attn_fp8(void* out, int out_dtype, const void* q, const int32_t* cu_q_lens,
                               const void* k_cache, const void* v_cache, float k_scale,
                               float v_scale, const int32_t* block_table, int max_blocks_per_seq,
                               const int32_t* context_lens, int max_context_len, int max_q_len,
                               int num_q_tokens, int num_seqs, int num_q_heads, int num_kv_heads,
                               int head_dim, int block_size, float scale, int causal,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_call(out, out_dtype, q, cu_q_lens, k_cache, v_cache, true, k_scale, v_scale,
                        block_table, max_blocks_per_seq, context_lens, max_context_len, max_q_len,
                        num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                        scale, causal, nullptr, workspace, workspace_bytes, stream);
}

int pkv_paged_prefill_attn_tree(void* out, int out_dtype, const void* q,
                                const int32_t* cu_q_lens, const uint64_t* tree_mask,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_table, int max_blocks_per_seq,
                                const int32_t* context_lens, int max_context_len, int max_q_len,
                                int num_q_tokens, int num_seqs, int num_q_heads, int num_kv_heads,
                                int head_dim, int block_size, float scale, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (max_q_len > kMaxTreeNodes) return PKV_ERR_UNSUPPORTED;
    if (num_seqs > 0 && num_q_tokens > 0 && !tree_mask) return PKV_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(tree_mask) & 7) return PKV_ERR_ALIGN;
    return prefill_call(out, out_dtype, q, cu_q_lens, k_cache, v_cache, false, 1.0f, 1.0f,
                        block_table, max_blocks_per_seq, context_lens, max_context_len, max_q_len,
                        num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                        scale, 1, tree_mask, workspace, workspace_bytes, stream);
}

int pkv_paged_prefill_attn_tree_fp8(void* out, int out_dtype, const void* q,
                                    const int32_t* cu_q_lens, const uint64_t* tree_mask,
                                    const void* k_cache, const void* v_cache, float k_scale,
                                    float v_scale, const int32_t* block_table,
                                    int max_blocks_per_seq, const int32_t* context_lens,
                                    int max_context_len, int max_q_len, int num_q_tokens,
                                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    if (max_q_len > kMaxTreeNodes) return PKV_ERR_UNSUPPORTED;
    if (num_seqs > 0 && num_q_tokens > 0 && !tree_mask) return PKV_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(tree_mask) & 7) return PKV_ERR_ALIGN;
    return prefill_call(out, out_dtype, q, cu_q_lens, k_cache, v_cache, true, k_scale, v_scale,
                        block_table, max_blocks_per_seq, context_lens, max_context_len, max_q_len,
                        num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                        scale, 1, tree_mask, workspace, workspace_bytes, stream);
}

int pkv_paged_prefill_attn_fp8_per_block(void* out, int out_dtype, const void* q,
                                         const int32_t* cu_q_lens, const void* k_cache,
                                         const void* v_cache, const float* k_scales,
                                         const float* v_scales, const int32_t* block_table,
                                         int max_blocks_per_seq, const int32_t* context_lens,
                                         int max_context_len, int max_q_len, int num_q_tokens,
                                         int num_seqs, int num_q_heads, int num_kv_heads,
                                         int head_dim, int block_size, float scale, int causal,
                                         void* workspace, size_t workspace_bytes, void* stream) {
    if (num_seqs > 0 && num_q_tokens > 0 && (!k_scales || !v_scales)) return PKV_ERR_NULL;
    return prefill_call(out, out_dtype, q, cu_q_lens, k_cache, v_cache, true, 1.0f, 1.0f,
                        block_table, max_blocks_per_seq, context_lens, max_context_len, max_q_len,
                        num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                        scale, causal, nullptr, workspace, workspace_bytes, stream, k_scales,
                        v_scales);
}

int pkv_paged_prefill_attn_tree_fp8_per_block(
    void* out, int out_dtype, const void* q, const int32_t* cu_q_lens, const uint64_t* tree_mask,
    const void* k_cache, const void* v_cache, const float* k_scales, const float* v_scales,
    const int32_t* block_table, int max_blocks_per_seq, const int32_t* context_lens,
    int max_context_len, int max_q_len, int num_q_tokens, int num_seqs, int num_q_heads,
    int num_kv_heads, int head_dim, int block_size, float scale, void* workspace,
    size_t workspace_bytes, void* stream) {
    if (max_q_len > kMaxTreeNodes) return PKV_ERR_UNSUPPORTED;
    if (num_seqs > 0 && num_q_tokens > 0 && !tree_mask) return PKV_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(tree_mask) & 7) return PKV_ERR_ALIGN;
    if (num_seqs > 0 && num_q_tokens > 0 && (!k_scales || !v_scales)) return PKV_ERR_NULL;
    return prefill_call(out, out_dtype, q, cu_q_lens, k_cache, v_cache, true, 1.0f, 1.0f,
                        block_table, max_blocks_per_seq, context_lens, max_context_len, max_q_len,
                        num_q_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                        scale, 1, tree_mask, workspace, workspace_bytes, stream, k_scales,
                        v_scales);
}

}  // extern "C"
