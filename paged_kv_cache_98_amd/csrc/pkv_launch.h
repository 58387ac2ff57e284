// pkv_launch.h -- internal interface between the C-ABI entry points
// (api.hip) and the kernel launchers.  Arguments arrive here already
// validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

struct AppendArgs {
    const uint16_t* k_new;
    const uint16_t* v_new;
    const int64_t* slot_mapping;
    int64_t num_tokens;
    uint16_t* k_cache;
    uint16_t* v_cache;
    int row_elems;  // num_kv_heads * head_dim
    int64_t num_slots;  // num_blocks * block_size: slots at or past it are skipped
};

struct AppendFp8Args {
    const uint16_t* k_new;  // bf16
    const uint16_t* v_new;
    const int64_t* slot_mapping;
    int64_t num_tokens;
    uint8_t* k_cache;  // E4M3 codes
    uint8_t* v_cache;
    int row_elems;  // num_kv_heads * head_dim
    int64_t num_slots;  // num_blocks * block_size: slots at or past it are skipped
    float k_scale;
    float v_scale;
    // or one scale per (block, KV head): [num_blocks][num_kv_heads] fp32
    const float* k_scales = nullptr;
    const float* v_scales = nullptr;
    int block_size = 16;
};

struct CopyBlocksArgs {
    uint16_t* k_cache;
    uint16_t* v_cache;
    const int64_t* block_mapping;  // [num_pairs][2] (source, destination)
    int64_t num_pairs;
    int64_t num_blocks;
    int64_t block_elems;  // block_size * num_kv_heads * head_dim
};

struct DecodeArgs {
    void* out;
    bool out_bf16;
    const uint16_t* q;
    const void* k_cache;  // bf16, or FP8 (E4M3) codes when kv_fp8
    const void* v_cache;
    bool kv_fp8 = false;
    float out_scale = 1.0f;  // multiplies the output (the FP8 cache's v_scale)
    const int32_t* block_table;
    int max_blocks_per_seq;
    const int32_t* context_lens;
    int max_context_len;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int block_size;
    float scale_log2;     // scale * log2(e) (times k_scale for an FP8 cache)
    int32_t* seq_workers; // workspace: [2][num_seqs] workers holding each sequence's first / last tile
    float* records;       // workspace: [max_workers][2][num_q_heads][head_dim + 4] partials
    int64_t max_workers;  // workers whose records fit the workspace
    // NULL for a plain decode batch.  Set for the decode rows of a mixed
    // prefill batch: only sequences with one query row are handled, reading
    // and writing row cu_q_lens[i].
    const int32_t* cu_q_lens;
    // With rows > 1 (and cu_q_lens) every sequence of 1 .. rows query rows,
    // rows cu_q_lens[i] ..: causal, or under one 64-bit key mask per row
    // over the chunk's keys (tree_mask, [num_q_tokens]).
    int rows = 1;
    bool causal = true;
    const uint64_t* tree_mask = nullptr;
    // FP8 pools with one scale per (block, KV head): [num_blocks][num_kv_heads]
    // fp32 tables for K and V (then scale_log2 and out_scale carry none)
    const float* k_scales = nullptr;
    const float* v_scales = nullptr;
};

struct PrefillArgs {
    void* out;
    bool out_bf16;
    const uint16_t* q;
    const int32_t* cu_q_lens;
    const void* k_cache;  // bf16, or FP8 (E4M3) codes when kv_fp8
    const void* v_cache;
    bool kv_fp8 = false;
    float out_scale = 1.0f;  // multiplies the output (the FP8 cache's v_scale)
    const int32_t* block_table;
    int max_blocks_per_seq;
    const int32_t* context_lens;
    int max_context_len;
    int max_q_len;
    int num_q_tokens;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int block_size;
    float scale_log2;
    bool causal;
    bool decode_rows_elsewhere;  // skip sequences with one query row
    // chunks that fit one workgroup run stream-K (prefill_streamk)
    bool streamk = false;
    int32_t* cum = nullptr;      // workspace: [num_seqs + 1] unit prefix sums
    float* records = nullptr;    // workspace: [max_workers][2][max_q_len * group][132]
    int64_t max_workers = 0;     // workers whose records fit the workspace
    const uint64_t* tree_mask = nullptr;  // [num_q_tokens] token-tree masks, or none
    // FP8 pools with one scale per (block, KV head): [num_blocks][num_kv_heads]
    // fp32 tables (then scale_log2 and out_scale carry none)
    const float* k_scales = nullptr;
    const float* v_scales = nullptr;
};

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_kv_append_fp8(const AppendFp8Args& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// The log-sum-exp merge of the decode rows shared by several workers (the
// second kernel of launch_decode, on its own after launch_mixed).
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream);
// A mixed batch in one grid: the chunks' MFMA items and the decode rows'
// stream-K workers co-resident on the CUs, then the decode merge.  Returns
// hipErrorNotSupported (nothing launched) for calls it does not take.
hipError_t launch_mixed(const PrefillArgs& a, const DecodeArgs& d, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// A prefill call whose chunks fit one workgroup (2 <= max_q_len and
// max_q_len * group <= 128 query columns) runs stream-K over its key tiles;
// its workspace part is a prefix-sum array and up to
// prefill_streamk_max_workers workers' records (prefill_streamk_bytes).
bool prefill_streamk(int max_q_len, int group);
int64_t prefill_streamk_max_workers(int num_seqs, int num_kv_heads, int max_context_len);
size_t prefill_streamk_bytes(int num_seqs, int max_q_len, int group, int num_kv_heads,
                             int max_context_len);

// Workgroups of `kern` the device holds at once with this block size and
// dynamic LDS (all CUs; cached per kernel and device).
hipError_t resident_workgroups(const void* kern, int threads, size_t lds, int* out);

// Decode workspace: which workers hold each sequence's first and last tiles,
// then the partial-result records ([workers][2][rows][num_q_heads] of them;
// rows > 1 for sequences of several query rows).
size_t decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                              int max_context_len, int rows = 1);
int64_t decode_max_workers(int num_seqs, int max_context_len, int rows = 1, int num_kv_heads = 1);

}  // namespace pkv
