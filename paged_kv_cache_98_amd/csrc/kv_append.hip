// kv_append.hip -- scatter new tokens' K/V rows into their pool slots.
//
// "LLM 推理优化技术全景", section "KV Cache": each step's new K and V join the
// cache; "让 Agent 跑得快", section 五: only the current token writes.  With the
// pool laid out [num_blocks][block_size][Hkv][D], slot s = block * block_size
// + row starts at element s * Hkv * D, so the copy needs only the slot.
// Each thread moves one 16-byte word of K and the same word of V; a token row
// of Hkv * D bf16 is Hkv * D / 8 words, so consecutive threads write
// consecutive words of one row (coalesced).  Negative slots are skipped.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

__global__ void __launch_bounds__(256)
kv_append_kernel(const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
                 const int64_t* __restrict__ slot_mapping, int64_t num_words,
                 uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int words_per_row) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < num_words; w += stride) {
        const int64_t t = w / words_per_row;
        const int64_t c = w - t * words_per_row;
        const int64_t s = slot_mapping[t];
        if (s < 0) continue;
        const int64_t dst = s * words_per_row + c;
        k_cache[dst] = k_new[w];
        v_cache[dst] = v_new[w];
    }
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
    const int words_per_row = a.row_elems / 8;
    const int64_t num_words = a.num_tokens * words_per_row;
    if (num_words == 0) return hipSuccess;
    const int64_t want = (num_words + 255) / 256;
    const int blocks = (int)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(kv_append_kernel, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(a.k_new), reinterpret_cast<const uint4*>(a.v_new),
                       a.slot_mapping, num_words, reinterpret_cast<uint4*>(a.k_cache),
                       reinterpret_cast<uint4*>(a.v_cache), words_per_row);
    return hipGetLastError();
}

}  // namespace pkv
