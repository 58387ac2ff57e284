// kv_append.hip -- writes into the pools: new tokens' K/V rows scattered to
// their slots, and whole-block copies for copy-on-write.
//
// "LLM 推理优化技术全景", section "KV Cache": each step's new K and V join the
// cache; "让 Agent 跑得快", section 五: only the current token writes.  With the
// pool laid out [num_blocks][block_size][Hkv][D], slot s = block * block_size
// + row starts at element s * Hkv * D, so the copy needs only the slot.
// Each thread moves one 16-byte word of K and the same word of V; a token row
// of Hkv * D bf16 is Hkv * D / 8 words, so consecutive threads write
// consecutive words of one row (coalesced).  Negative slots are skipped, and
// so is a slot past the pool's last row, so a stale slot mapping cannot write
// outside the pools.
//
// The FP8 variant ("让 Agent 跑得快", section 四: one byte per value, half
// the bytes of bf16; "LLM推理工程实战", section 5.3: the KV cache stored
// quantised) writes OCP E4M3 codes: each value x becomes the E4M3 value
// nearest to x / scale (one correctly rounded binary32 division, clamped to
// +-448 first, since the hardware conversion rounds to nearest even but
// turns magnitudes past 464 into NaN), with the cache's own scale for K and
// for V.  A thread turns one 16-byte word (eight bf16) into one 8-byte word
// of codes.
//
// Copy-on-write ("让 Agent 跑得快", section 二, "Copy-on-Write"): before a
// sequence writes into a block it shares, the block is copied whole (every
// row and head of K and V) to a fresh block; block b is the contiguous
// block_size * Hkv * D elements starting at b * block_size * Hkv * D.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

__global__ void __launch_bounds__(256)
kv_append_kernel(const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
                 const int64_t* __restrict__ slot_mapping, int64_t num_words,
                 uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int words_per_row,
                 int64_t num_slots) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < num_words; w += stride) {
        const int64_t t = w / words_per_row;
        const int64_t c = w - t * words_per_row;
        const int64_t s = slot_mapping[t];
        if (s < 0 || s >= num_slots) continue;
        const int64_t dst = s * words_per_row + c;
        k_cache[dst] = k_new[w];
        v_cache[dst] = v_new[w];
    }
}

constexpr float kE4m3Max = 448.0f;

// Eight bf16 values -> eight E4M3 codes (byte i = value i).
__device__ __forceinline__ uint2 quantise8(uint4 x, float scale) {
    float y[8] = {bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y),
                  bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w)};
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(y[i] / scale, -kE4m3Max), kE4m3Max);
    uint2 r;
    r.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    r.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)r.x, true);
    r.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    r.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], (int)r.y, true);
    return r;
}

// With BLOCK_SCALES the scales are per (block, KV head): [num_blocks]
// [num_kv_heads] fp32 tables, read for the block slot s lies in (s / bs)
// and the word's KV head (kHeadDim / 8 words per head).
template <bool BLOCK_SCALES>
__global__ void __launch_bounds__(256)
kv_append_fp8_kernel(const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
                     const int64_t* __restrict__ slot_mapping, int64_t num_words,
                     uint2* __restrict__ k_cache, uint2* __restrict__ v_cache, int words_per_row,
                     float k_scale, float v_scale, int64_t num_slots,
                     const float* __restrict__ k_scales, const float* __restrict__ v_scales,
                     int block_size) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < num_words; w += stride) {
        const int64_t t = w / words_per_row;
        const int64_t c = w - t * words_per_row;
        const int64_t s = slot_mapping[t];
        if (s < 0 || s >= num_slots) continue;
        const int64_t dst = s * words_per_row + c;
        float ks = k_scale, vs = v_scale;
        if constexpr (BLOCK_SCALES) {
            const int64_t e = (s / block_size) * (words_per_row / (kHeadDim / 8)) + c / (kHeadDim / 8);
            ks = k_scales[e];
            vs = v_scales[e];
        }
        k_cache[dst] = quantise8(k_new[w], ks);
        v_cache[dst] = quantise8(v_new[w], vs);
    }
}

// Whole-block copies for copy-on-write.  The grid-stride loop runs over
// units of one 512-word slice (256 threads x 2 words) of one tensor: all K
// units, then all V units.  A block of block_size * Hkv * D bf16 is
// block_size * Hkv * 16 words, a whole number of 256-word rows, so a slice
// is either entirely inside its block (the usual case: both words loaded
// before either is stored, with no per-word test) or holds the block's last
// row.  The stores are non-temporal: the copy is not read back soon, and
// keeping it out of the caches lets the writes stream (about 1.35x faster
// than ordinary stores on MI355X).  A pair naming a block outside the pool
// is skipped, so a bad id cannot write outside it.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kCopyWordsPerThread = 2;
constexpr int kCopyThreads = 256;
constexpr int kCopySlice = kCopyWordsPerThread * kCopyThreads;

__global__ void __launch_bounds__(kCopyThreads)
copy_blocks_kernel(u32x4_t* __restrict__ k_cache, u32x4_t* __restrict__ v_cache,
                   const int64_t* __restrict__ block_mapping, int64_t num_pairs, int slices,
                   int64_t num_blocks, int64_t block_words) {
    const int64_t units_per_tensor = num_pairs * slices;
    for (int64_t u = blockIdx.x; u < 2 * units_per_tensor; u += gridDim.x) {
        const bool is_v = u >= units_per_tensor;
        const int64_t r = is_v ? u - units_per_tensor : u;
        const int64_t pair = r / slices;
        const int64_t slice = r - pair * slices;
        const int64_t src = block_mapping[2 * pair];
        const int64_t dst = block_mapping[2 * pair + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
        u32x4_t* pool = is_v ? v_cache : k_cache;
        const int64_t first = slice * kCopySlice;
        const u32x4_t* from = pool + src * block_words + first + threadIdx.x;
        u32x4_t* to = pool + dst * block_words + first + threadIdx.x;
        const int64_t rows = (block_words - first) / kCopyThreads;
        if (rows >= kCopyWordsPerThread) {
            u32x4_t x[kCopyWordsPerThread];
#pragma unroll
            for (int i = 0; i < kCopyWordsPerThread; ++i) x[i] = from[i * kCopyThreads];
#pragma unroll
            for (int i = 0; i < kCopyWordsPerThread; ++i)
                __builtin_nontemporal_store(x[i], to + i * kCopyThreads);
        } else {
            for (int64_t i = 0; i < rows; ++i)
                __builtin_nontemporal_store(from[i * kCopyThreads], to + i * kCopyThreads);
        }
    }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
    const int64_t block_words = a.block_elems / 8;  // a multiple of kCopyThreads
    const int slices = (int)((block_words + kCopySlice - 1) / kCopySlice);
    const int64_t num_units = 2 * a.num_pairs * slices;
    const int blocks = (int)(num_units < 65536 ? num_units : 65536);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(blocks), dim3(kCopyThreads), 0, stream,
                       reinterpret_cast<u32x4_t*>(a.k_cache), reinterpret_cast<u32x4_t*>(a.v_cache),
                       a.block_mapping, a.num_pairs, slices, a.num_blocks, block_words);
    return hipGetLastError();
}

hipError_t launch_kv_append_fp8(const AppendFp8Args& a, hipStream_t stream) {
    const int words_per_row = a.row_elems / 8;  // 16-byte words of bf16 in, 8-byte words out
    const int64_t num_words = a.num_tokens * words_per_row;
    if (num_words == 0) return hipSuccess;
    const int64_t want = (num_words + 255) / 256;
    const int blocks = (int)(want < 65536 ? want : 65536);
    if (a.k_scales != nullptr)
        hipLaunchKernelGGL(kv_append_fp8_kernel<true>, dim3(blocks), dim3(256), 0, stream,
                           reinterpret_cast<const uint4*>(a.k_new), reinterpret_cast<const uint4*>(a.v_new),
                           a.slot_mapping, num_words, reinterpret_cast<uint2*>(a.k_cache),
                           reinterpret_cast<uint2*>(a.v_cache), words_per_row, 1.0f, 1.0f,
                           a.num_slots, a.k_scales, a.v_scales, a.block_size);
    else
        hipLaunchKernelGGL(kv_append_fp8_kernel<false>, dim3(blocks), dim3(256), 0, stream,
                           reinterpret_cast<const uint4*>(a.k_new), reinterpret_cast<const uint4*>(a.v_new),
                           a.slot_mapping, num_words, reinterpret_cast<uint2*>(a.k_cache),
                           reinterpret_cast<uint2*>(a.v_cache), words_per_row, a.k_scale, a.v_scale,
                           a.num_slots, nullptr, nullptr, a.block_size);
    return hipGetLastError();
}

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
    const int words_per_row = a.row_elems / 8;
    const int64_t num_words = a.num_tokens * words_per_row;
    if (num_words == 0) return hipSuccess;
    const int64_t want = (num_words + 255) / 256;
    const int blocks = (int)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(kv_append_kernel, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(a.k_new), reinterpret_cast<const uint4*>(a.v_new),
                       a.slot_mapping, num_words, reinterpret_cast<uint4*>(a.k_cache),
                       reinterpret_cast<uint4*>(a.v_cache), words_per_row, a.num_slots);
    return hipGetLastError();
}

}  // namespace pkv
