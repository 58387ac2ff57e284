// prefill.hip -- chunked-prefill attention over the paged cache on gfx950
// matrix cores (MFMA), causal, GQA-packed.
//
// What it computes ("LLM 推理优化技术全景", "Flash Attention 深度剖析 >
// 分块算法" and "在线 Softmax"; "Chunked Prefill"): for query row r of
// sequence i, at absolute position p = ctx_i - Lq_i + r, and query head h,
//     out[row, h, :] = sum_{t <= p} exp(s_t - m) V[t, :] / sum_{t <= p} exp(s_t - m),
//     s_t = scale * <q[row, h, :], K[t, :]>,
// (all ctx_i keys when not causal).  Keys come from 16- or 32-token physical
// blocks through the block table.  The page's outer loop over query blocks
// is the grid; its inner loop over key/value blocks runs in each workgroup,
// with S = Q K^T and O += P V on the matrix cores and the running max m /
// sum l kept per query, so S never leaves the chip.
//
// Tiling (one workgroup = 4 waves, 128 "query columns"):
//   * a workgroup owns one KV head and 128 / G consecutive query positions
//     of one sequence; its 128 columns are (position, head) pairs, column
//     c = (c / G)-th position, query head kvh * G + c % G, so every K/V tile
//     staged in LDS serves all G query heads (GQA);
//   * wave w owns columns 32w .. 32w + 31; with v_mfma_f32_32x32x16 the
//     query index is the MFMA's N index (lane % 32) in both products:
//       S^T[64 keys x 32 cols]  = K (A, from LDS) . Q^T (B, registers)
//       O^T[128 dims x 32 cols] += V^T (A, from LDS) . P^T (B, registers)
//     so each lane holds the scores of exactly one query column: the row max
//     and sum are lane-local (plus one exchange with lane ^ 32), the rescale
//     of O^T by exp(m_old - m_new) is lane-local, and P^T's accumulator
//     layout is already the B operand of the second MFMA (the 16 keys of a
//     k-step are taken in the order the accumulator holds them, and V^T is
//     read from LDS in that same order);
//   * QK^T runs on bf16 inputs (exact products, fp32 accumulate); P V runs on
//     fp16: P in [0, 1] rounds with 2^-11 relative error (bf16 would give
//     2^-8), and bf16 V converts to fp16 exactly for |v| in [2^-14, 65504];
//   * K and V tiles of 64 keys are double-buffered in LDS: K as [key][dim]
//     bf16, V transposed to [dim][key] fp16 while it is staged; the next
//     tile's global loads are in flight while the current tile is computed.
//
// Token trees ("让 Agent 跑得快", section 六, Token Tree Verification): with
// a mask per query row, a verify chunk's rows are the nodes of a draft tree
// in topological order, and row r sees the cached context plus the chunk's
// tokens j whose bit is set in its mask (its path to the root); the masks
// are applied, with the causal limit, in the tiles that hold chunk keys.
//
// Stream-K for chunks that fit one workgroup (every sequence's rows in one
// slot, as in speculative-decoding verification): such a call reads every
// key once per KV head for a few queries, so it is bandwidth-bound, and one
// workgroup per item would last as long as the longest context.  Instead
// the items' key tiles are laid end to end and cut into equal ranges, one
// per resident workgroup; items split between workers leave their
// unnormalised O, reference maximum m and sum l per column in the
// workspace, and prefill_streamk_merge_kernel combines them:
// M = max m_k, L = sum l_k 2^(m_k - M), out = sum O_k 2^(m_k - M) / L (the
// sequence-axis parallelism of "Flash Attention v2 的改进").
#include <type_traits>

#include "decode_core.h"
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int D = kHeadDim;
constexpr int kKT = 64;          // keys per K/V tile
constexpr int kCols = 128;       // query columns per workgroup
constexpr int kThreads = 256;    // 4 waves
constexpr int kKsStride = D + 8;      // bf16 elements per K row in LDS (272 B)
// V^T rows in LDS: 64 keys + 16 fp16 of padding (160 B).  A row's keys sit
// in eight 16-byte units of 8 keys: unit u = 4 kb + 2 ks + h holds keys
// 32 kb + 16 ks + 4 h .. + 3 and then 32 kb + 16 ks + 8 + 4 h .. + 3 -- the
// eight keys, in the order the S accumulator hands them to P^T, that MFMA
// lane half h reads for k-step ks of half tile kb, so each A operand is one
// 16-byte read.  Unit u of row d is stored at slot u ^ vt_swizzle(d).  The
// pitch and the swizzle were chosen by measuring the LDS bank-conflict
// counter for the exact access patterns of the operand reads and the
// staging stores (the 64 four-byte banks do not serve the lanes of a wave
// in any simple grouping): with a 160-byte pitch and a swizzle constant
// over 16 rows the operand reads run at the conflict-free rate and the
// 8-byte staging stores at half of it; a 144-byte pitch halves the reads'
// rate too, a 192-byte one is conflict-free for both but does not leave
// room for two workgroups per CU.
constexpr int kVtStride = kKT + 16;
__device__ __forceinline__ int vt_swizzle(int d) { return (d >> 4) & 7; }
// element index of key k (0 .. 63) of dim d in a V^T tile
__device__ __forceinline__ int vt_index(int d, int k) {
    const int u = 4 * (k >> 5) + 2 * ((k >> 4) & 1) + ((k >> 2) & 1);
    return d * kVtStride + 8 * (u ^ vt_swizzle(d)) + 4 * ((k >> 3) & 1) + (k & 3);
}
constexpr int kKsElems = kKT * kKsStride;
constexpr int kVtElems = D * kVtStride;

struct PrefillIds {
    const int32_t* row;
    int nblk;
    int base;
    int cur;
    int nxt;
    // window starting at block `first`
    __device__ __forceinline__ void init(const int32_t* r, int n, int first, int lane) {
        row = r;
        nblk = n;
        base = first;
        cur = first + lane < n ? r[first + lane] : 0;
        nxt = first + 64 + lane < n ? r[first + 64 + lane] : 0;
    }
    // id of block `blk` (wave-uniform, non-decreasing between calls)
    __device__ __forceinline__ int get(int blk, int lane) {
        while (blk >= base + 64) {
            cur = nxt;
            base += 64;
            nxt = base + 64 + lane < nblk ? row[base + 64 + lane] : 0;
        }
        return __builtin_amdgcn_readlane(cur, blk - base);
    }
    // ids of the four 16-key groups of the 64-key tile at k0.  The window
    // starts at the block of a tile's first key and moves by 64 blocks, so a
    // tile's 4 (or 2) blocks never straddle it and one move check serves
    // all four (tiles are visited in increasing order).
    template <int BS>
    __device__ __forceinline__ void tile(int k0, int lane, int (&id)[4]) {
        const int blk0 = k0 / BS;
        while (blk0 >= base + 64) {
            cur = nxt;
            base += 64;
            nxt = base + 64 + lane < nblk ? row[base + 64 + lane] : 0;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) id[i] = __builtin_amdgcn_readlane(cur, (k0 + 16 * i) / BS - base);
    }
};

// Global -> register staging of one 64-key tile: K chunks (4 x 16 B) and V
// chunks (4 consecutive keys, 8 dims each) per thread.
struct Stage {
    uint4 k[4];
    uint4 v[4];
};

// The V part of a thread's staging: 8 dims 8 vc .. 8 vc + 7 of the four
// consecutive keys vkey .. vkey + 3, all inside the wave's 16-key group
// (vkey = 16 wave + 8 vhalf + 4 vh).  The lane bits are dealt so that the
// 16 lanes of each quarter wave store 16 different 8-byte slots of the
// banks: lane bits 0-2 and 4 give vc, bit 3 gives vhalf, bit 5 vh.
struct VStageMap {
    int vc, vhalf, vh;
    __device__ __forceinline__ explicit VStageMap(int lane)
        : vc((lane & 7) | (((lane >> 4) & 1) << 3)), vhalf((lane >> 3) & 1), vh((lane >> 5) & 1) {}
    __device__ __forceinline__ int key(int wave) const { return 16 * wave + 8 * vhalf + 4 * vh; }
};

// This thread's byte offsets inside a block for its staging loads: row
// within the block times the row pitch, plus its 16-byte chunk of the head's
// 256 bytes.  K load i carries key k0 + kq + 16 i, V load i key
// k0 + vkey + i; k0 is a multiple of 64, hence of the block size, so the
// offsets are the same for every tile.
template <int BS>
__device__ __forceinline__ void stage_offsets(uint32_t (&koff)[4], uint32_t (&voff)[4],
                                              uint32_t row_bytes, int tid) {
    const int col = tid & 15;
    const int kq = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) koff[i] = (uint32_t)((kq + 16 * i) % BS) * row_bytes + col * 16;
    const VStageMap vm(tid & 63);
    const int vkey = vm.key(tid >> 6);
#pragma unroll
    for (int i = 0; i < 4; ++i) voff[i] = (uint32_t)((vkey + i) % BS) * row_bytes + vm.vc * 16;
}

// Loads one 64-key tile into registers.  Every load of a wave reads one
// physical block: K load i lies in the tile's 16-key group i, and all V
// loads of wave w in group w.  So the block's address is a scalar buffer
// base and the lane offsets are the fixed ones above; keys past kv_end read
// zeros without a memory access.  kbase / vbase point at this KV head's
// slice of block 0 of the pools.
template <int BS, bool CHECK>
__device__ __forceinline__ void stage_load(Stage& sg, PrefillIds& ids, const char* kbase,
                                           const char* vbase, int k0, int kv_end,
                                           size_t block_bytes, const uint32_t (&koff)[4],
                                           const uint32_t (&voff)[4], int tid, int lane) {
    const int kq = tid >> 4;
    // ids of the tile's four 16-key groups, fetched in increasing order (the
    // window only moves forward)
    int id[4];
    ids.tile<BS>(k0, lane, id);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __amdgpu_buffer_rsrc_t r = buffer_rsrc(kbase + (size_t)id[i] * block_bytes);
        const uint32_t o = !CHECK || k0 + kq + 16 * i < kv_end ? koff[i] : kBufferOob;
        sg.k[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
    }
    // the wave's V group id, chosen with a wave-uniform index so that the
    // resource stays in scalar registers (no waterfall loop)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int vid = wave == 0 ? id[0] : wave == 1 ? id[1] : wave == 2 ? id[2] : id[3];
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(vbase + (size_t)vid * block_bytes);
    const int vkey = k0 + VStageMap(lane).key(wave);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t o = !CHECK || vkey + i < kv_end ? voff[i] : kBufferOob;
        sg.v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
    }
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    f16x2_t h;
    h[0] = (_Float16)a;
    h[1] = (_Float16)b;
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ void stage_store(const Stage& sg, uint16_t* __restrict__ ks,
                                            uint16_t* __restrict__ vt, int tid) {
    const int col = tid & 15;
    const int kq = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(ks + (kq + 16 * i) * kKsStride + col * 8) = sg.k[i];
    // V^T[dim][key] in fp16: dim 8 vc + w gets this thread's four keys as
    // one 8-byte store, at the same slot of each of its 8 rows (their
    // swizzle is vc / 2)
    const int lane = tid & 63;
    const VStageMap vm(lane);
    const int vkey = vm.key(tid >> 6);
    uint16_t* vrow = vt + vt_index(8 * vm.vc, vkey);
    const uint32_t w0[4] = {sg.v[0].x, sg.v[0].y, sg.v[0].z, sg.v[0].w};
    const uint32_t w1[4] = {sg.v[1].x, sg.v[1].y, sg.v[1].z, sg.v[1].w};
    const uint32_t w2[4] = {sg.v[2].x, sg.v[2].y, sg.v[2].z, sg.v[2].w};
    const uint32_t w3[4] = {sg.v[3].x, sg.v[3].y, sg.v[3].z, sg.v[3].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        *reinterpret_cast<uint2*>(vrow + (2 * w) * kVtStride) =
            make_uint2(pack_f16x2(bf16_lo(w0[w]), bf16_lo(w1[w])),
                       pack_f16x2(bf16_lo(w2[w]), bf16_lo(w3[w])));
        *reinterpret_cast<uint2*>(vrow + (2 * w + 1) * kVtStride) =
            make_uint2(pack_f16x2(bf16_hi(w0[w]), bf16_hi(w1[w])),
                       pack_f16x2(bf16_hi(w2[w]), bf16_hi(w3[w])));
    }
}

// FP8 (E4M3) pools: a 64-key tile of one KV head is 8 KB of K codes and 8 KB
// of V codes.  Thread t stages K rows t / 8 and t / 8 + 32 and V rows
// 2 (t / 8) and 2 (t / 8) + 1, bytes (dims) 16 (t % 8) .. + 15 of each; in
// LDS the tile takes the layouts of the bf16 path, K widened to bf16 and V
// to fp16 (both exact for E4M3 values), so the tile math is the same.  The
// scales are applied outside: k_scale in the score scale, v_scale in the
// final division.
struct StageFp8 {
    uint4 k[2];
    uint4 v[2];
};

// FP8 pools with one scale per (block, KV head): lane l also carries the K
// and V scales of the tile's 16-key group l % 4 (their blocks' scales), so
// a wave has all four at hand through readlane.  A thread's two V rows are
// adjacent keys of 16-key group `wave` (one block), so one V ratio serves
// all its V values: they are staged as fp16(code x ratio), the ratio being
// the group's V scale over the tile's reference (the largest V scale of the
// item's tiles so far).  The K scales go to LDS beside the tile and
// multiply its scores.
struct StageFp8Bs : StageFp8 {
    float ks;
    float vs;
};

template <int BS>
__device__ __forceinline__ void stage_offsets_fp8(uint32_t (&koff)[4], uint32_t (&voff)[4],
                                                  uint32_t row_bytes, int tid) {
    const int col = tid & 7;
    const int kq = tid >> 3;
#pragma unroll
    for (int i = 0; i < 2; ++i) koff[i] = (uint32_t)((kq + 32 * i) % BS) * row_bytes + col * 16;
#pragma unroll
    for (int p = 0; p < 2; ++p) voff[p] = (uint32_t)((2 * kq + p) % BS) * row_bytes + col * 16;
    koff[2] = koff[3] = voff[2] = voff[3] = 0;
}

// A wave's K load i lies in the tile's 16-key group wave / 2 + 2 i and its V
// loads in group `wave` (t / 8 = 8 wave + lane / 8), one physical block each.
template <int BS, bool CHECK>
__device__ __forceinline__ void stage_load_fp8(StageFp8& sg, PrefillIds& ids, const char* kbase,
                                               const char* vbase, int k0, int kv_end,
                                               size_t block_bytes, const uint32_t (&koff)[4],
                                               const uint32_t (&voff)[4], int tid, int lane) {
    const int kq = tid >> 3;
    const int wave = tid >> 6;
    int id[4];
    ids.tile<BS>(k0, lane, id);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int kid = __builtin_amdgcn_readfirstlane(id[(wave >> 1) + 2 * i]);
        const __amdgpu_buffer_rsrc_t r = buffer_rsrc(kbase + (size_t)kid * block_bytes);
        const uint32_t o = !CHECK || k0 + kq + 32 * i < kv_end ? koff[i] : kBufferOob;
        sg.k[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
    }
    const int vid = __builtin_amdgcn_readfirstlane(id[wave]);
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(vbase + (size_t)vid * block_bytes);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const uint32_t o = !CHECK || k0 + 2 * kq + p < kv_end ? voff[p] : kBufferOob;
        sg.v[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
    }
}

template <bool RATIO = false>
__device__ __forceinline__ void stage_store_fp8(const StageFp8& sg, uint16_t* __restrict__ ks,
                                                uint16_t* __restrict__ vt, int tid,
                                                float vratio = 1.0f) {
    const int col = tid & 7;
    const int kq = tid >> 3;
    // K: 16 codes -> 16 bf16 in row kq + 32 i, elements 16 col .. + 15
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t w[4] = {sg.k[i].x, sg.k[i].y, sg.k[i].z, sg.k[i].w};
        uint32_t b[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            b[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[j], 1.0f, false));
            b[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[j], 1.0f, true));
        }
        uint16_t* row = ks + (kq + 32 * i) * kKsStride + 16 * col;
        *reinterpret_cast<uint4*>(row) = make_uint4(b[0], b[1], b[2], b[3]);
        *reinterpret_cast<uint4*>(row + 8) = make_uint4(b[4], b[5], b[6], b[7]);
    }
    // V^T: dim d = 16 col + 4 j + e takes the fp16 pair (key 2 kq,
    // key 2 kq + 1), adjacent in the row's layout
    const uint32_t a[4] = {sg.v[0].x, sg.v[0].y, sg.v[0].z, sg.v[0].w};
    const uint32_t c[4] = {sg.v[1].x, sg.v[1].y, sg.v[1].z, sg.v[1].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // bytes (a.k, c.k, a.k+1, c.k+1) of the two rows' words, k = 0 and 2
        const uint32_t w0 = __builtin_amdgcn_perm(c[j], a[j], 0x05010400u);
        const uint32_t w1 = __builtin_amdgcn_perm(c[j], a[j], 0x07030602u);
        f16x2_t vp[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w0, 1.0f, false),
                         __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w0, 1.0f, true),
                         __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w1, 1.0f, false),
                         __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w1, 1.0f, true)};
        if constexpr (RATIO) {
            // code x ratio (<= 1) in fp16: the exact code value times the
            // ratio rounded to fp16, rounded once more
            const _Float16 r16 = (_Float16)vratio;
            const f16x2_t rr = {r16, r16};
#pragma unroll
            for (int e = 0; e < 4; ++e) vp[e] = vp[e] * rr;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int d = 16 * col + 4 * j + e;
            *reinterpret_cast<uint32_t*>(vt + vt_index(d, 2 * kq)) = __builtin_bit_cast(uint32_t, vp[e]);
        }
    }
}

// Online-softmax step for one 32-key half tile of this lane's query column:
// raw scores s (element e is key kb0 + 8 (e / 4) + 4 h + e % 4) -> P^T
// fragments (fp16, k-steps of 16 keys) and the updated running max / sum,
// with O rescaled.  MASK (diagonal or last tile only) drops keys after the
// column's position or past the context.
constexpr float kLazyMax = 8.0f;  // p < 2^8 between rescales

// TWO: elements 0 .. 7 (the half's first 16 keys) take the score scale cl2
// and elements 8 .. 15 cl2b (per-block K scales folded into each 16-key
// group's scale; the scales are >= 0, so a group's maximum scales with it).
template <bool MASK, bool TWO = false>
__device__ __forceinline__ void softmax_half(f32x16_t& s, f16x8_t (&pf)[2], f32x16_t (&o)[4],
                                             float& m_run, float& l_run, float cl2, int kb0, int h,
                                             int pos, int ctx, bool diag, uint64_t tmask,
                                             int tbase, float cl2b = 0.0f) {
    // four independent partial maxima / sums, so neither is one long
    // dependent chain
    float mt4[4] = {-3.402823466e38f, -3.402823466e38f, -3.402823466e38f, -3.402823466e38f};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        if (MASK) {
            const int key = kb0 + 8 * (e >> 2) + 4 * h + (e & 3);
            // a token-tree node also drops the chunk's keys off its path
            // (key - tbase < 64 wherever the mask is read)
            const bool ok = (!diag || key <= pos) && key < ctx &&
                            (key < tbase || ((tmask >> ((key - tbase) & 63)) & 1));
            s[e] = ok ? s[e] : -3.402823466e38f;
        }
        if constexpr (TWO) {
            // partial maxima 0, 1 over elements 0 .. 7, 2, 3 over 8 .. 15
            const int k = 2 * (e >> 3) + (e & 1);
            mt4[k] = fmaxf(mt4[k], s[e]);
        } else {
            mt4[e & 3] = fmaxf(mt4[e & 3], s[e]);
        }
    }
    float mt;
    if constexpr (TWO) {
        mt = fmaxf(fmaxf(mt4[0], mt4[1]) * cl2, fmaxf(mt4[2], mt4[3]) * cl2b);
        mt = max_lane_halves(mt);
    } else {
        mt = fmaxf(fmaxf(mt4[0], mt4[1]), fmaxf(mt4[2], mt4[3]));
        mt = max_lane_halves(mt) * cl2;
    }
    // Lazy reference maximum: m_run moves only when a score exceeds it by
    // more than kLazyMax (log2 units), so p = 2^(s - m_run) stays below
    // 2^kLazyMax (far inside fp16) and O and l are rescaled only on those
    // rare jumps; softmax does not depend on which reference is used.
    float alpha = 1.0f;
    if (__any(mt > m_run + kLazyMax)) {
        const float mn = mt > m_run + kLazyMax ? mt : m_run;
        alpha = fast_exp2(m_run - mn);
        m_run = mn;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[mb][e] *= alpha;
    }
    const float mn = m_run;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        float p = fast_exp2(fmaf(s[e], TWO && e >= 8 ? cl2b : cl2, -mn));
        // a dropped key must give 0 even for a zero scale
        if (MASK) p = s[e] == -3.402823466e38f ? 0.0f : p;
        pf[e >> 3][e & 7] = (_Float16)p;
    }
    // the sum of the fp16 weights P V uses (so the normalised weights are
    // those weights exactly): fp32 dot products of their pairs with (1, 1)
    const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    float ls2[2] = {0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
            const f16x2_t pr = {pf[k][2 * q2], pf[k][2 * q2 + 1]};
            ls2[q2 & 1] = __builtin_amdgcn_fdot2(pr, one, ls2[q2 & 1], false);
        }
    l_run = fmaf(l_run, alpha, ls2[0] + ls2[1]);
}

constexpr int kRecStride = D + 4;  // floats per partial record: O[128], m, l, 2 pad
constexpr int64_t kMaxChunkWorkers = 1024;  // stream-K workgroups, at most

// Key tiles [t0, t1) of one item -- a sequence's KV head kvh and its query
// rows r0 .. r0 + P - 1, P = 128 / G, of a chunk of lq rows ending at
// position ctx - 1 -- on the calling workgroup.  Every wave of the
// workgroup calls it with the same arguments (rec_col aside) and meets the
// same barriers, and the tile buffers are free again when it returns.
// rec_col is this lane's column record, or NULL for the final output: with
// a record the unnormalised O^T, the reference maximum m and the sum l are
// stored instead of O / l.
// BSC: FP8 pools with per-(block, KV head) scales (k_scales / v_scales,
// [num_blocks][num_kv_heads]; s_sc: 2 x 8 floats of LDS, a tile buffer's
// four K scales and its V reference).
template <int BS, int G, bool OUT_BF16, bool FP8, bool BSC = false>
__device__ __forceinline__ void chunk_item(
    uint16_t (&s_ks)[2][kKsElems], uint16_t (&s_vt)[2][kVtElems], void* __restrict__ out,
    const uint16_t* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ bt_row, int num_q_heads,
    int num_kv_heads, float scale_log2, float out_scale, int causal,
    const uint64_t* __restrict__ tree_mask, int q_begin, int lq, int ctx, int kvh, int r0, int t0,
    int t1, float* rec_col, const float* __restrict__ k_scales = nullptr,
    const float* __restrict__ v_scales = nullptr, float* __restrict__ s_sc = nullptr) {
    static_assert(!BSC || FP8, "per-block scales are an FP8 pool format");
    constexpr int P = kCols / G;  // query positions per workgroup
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int pos0 = ctx - lq;  // position of the chunk's first query row

    // ---- this lane's query column
    const int h = lane >> 5;              // half of the wave
    const int c = wave * 32 + (lane & 31);
    const int r = r0 + c / G;             // row inside the chunk
    const int g = c % G;
    const bool col_valid = r < lq;
    const int pos = pos0 + r;
    const int r_last = (r0 + P < lq ? r0 + P : lq) - 1;
    const int kv_end = causal ? (pos0 + r_last + 1 < ctx ? pos0 + r_last + 1 : ctx) : ctx;
    const int ntiles = (kv_end + kKT - 1) / kKT;

    // Q^T fragments: k-step kk covers dims 16 kk + 8 h .. + 7 of this column;
    // a negative scale moves into q's sign so maxima work on raw scores.
    const uint32_t neg = scale_log2 < 0.0f ? 0x80008000u : 0u;
    const float cl2 = fabsf(scale_log2);
    bf16x8_t qf[8];
    {
        const size_t qrow = ((size_t)(q_begin + (col_valid ? r : 0)) * num_q_heads +
                             (size_t)kvh * G + g) * D;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            uint4 w = col_valid ? *reinterpret_cast<const uint4*>(q + qrow + 16 * kk + 8 * h)
                                : make_uint4(0, 0, 0, 0);
            w.x ^= neg; w.y ^= neg; w.z ^= neg; w.w ^= neg;
            qf[kk] = __builtin_bit_cast(bf16x8_t, w);
        }
    }

    f32x16_t o[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[mb][e] = 0.0f;
    float m_run = kNegBig;
    float l_run = 0.0f;

    constexpr int kElem = FP8 ? 1 : 2;  // bytes per cached value
    const uint32_t row_bytes = (uint32_t)num_kv_heads * D * kElem;
    const size_t block_bytes = (size_t)BS * row_bytes;
    const char* kbase = reinterpret_cast<const char*>(k_cache) + (size_t)kvh * D * kElem;
    const char* vbase = reinterpret_cast<const char*>(v_cache) + (size_t)kvh * D * kElem;
    uint32_t koff[4], voff[4];
    if constexpr (FP8)
        stage_offsets_fp8<BS>(koff, voff, row_bytes, tid);
    else
        stage_offsets<BS>(koff, voff, row_bytes, tid);
    PrefillIds ids;
    ids.init(bt_row, (ctx + BS - 1) / BS, t0 * kKT / BS, lane);
    using StageT = std::conditional_t<FP8, std::conditional_t<BSC, StageFp8Bs, StageFp8>, Stage>;
    // check_c: whether keys of the tile may lie at or past kv_end
    auto load_next = [&](StageT& x, int k0n, auto check_c) {
        constexpr bool CHECK = decltype(check_c)::value;
        if constexpr (FP8)
            stage_load_fp8<BS, CHECK>(x, ids, kbase, vbase, k0n, kv_end, block_bytes, koff, voff, tid, lane);
        else
            stage_load<BS, CHECK>(x, ids, kbase, vbase, k0n, kv_end, block_bytes, koff, voff, tid, lane);
        if constexpr (BSC) {
            // the scales of 16-key group lane % 4 (blocks past the context
            // read as block 0: their keys are masked)
            int id[4];
            ids.tile<BS>(k0n, lane, id);
            const int gq = lane & 3;
            const int idg = gq == 0 ? id[0] : (gq == 1 ? id[1] : (gq == 2 ? id[2] : id[3]));
            const size_t e = (size_t)idg * num_kv_heads + kvh;
            x.ks = k_scales[e];
            x.vs = v_scales[e];
        }
    };
    float vref_st = 0.0f;  // V reference of the last staged tile (BSC)
    auto store_tile = [&](const StageT& x, int b) {
        if constexpr (BSC) {
            float vg[4];
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
                vg[gq] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x.vs), gq));
            const float vnew = fmaxf(fmaxf(vref_st, fmaxf(vg[0], vg[1])), fmaxf(vg[2], vg[3]));
            vref_st = vnew;
            stage_store_fp8<true>(x, s_ks[b], s_vt[b], tid, vg[tid >> 6] / vnew);
            if (tid < 4) s_sc[8 * b + tid] = x.ks;
            if (tid == 0) s_sc[8 * b + 4] = vnew;
        } else if constexpr (FP8) {
            stage_store_fp8(x, s_ks[b], s_vt[b], tid);
        } else {
            stage_store(x, s_ks[b], s_vt[b], tid);
        }
    };
    StageT sg;
    if (t1 > t0) {
        load_next(sg, t0 * kKT, std::true_type{});
        store_tile(sg, t0 & 1);
    }
    __syncthreads();

    // this lane's part of its V^T operand addresses (see the PV loop): row
    // L = lane % 32 of the 32-row block mb, unit 4 kb + 2 ks + h at slot
    // (4 kb + 2 ks + h) ^ (2 mb + L / 16): bit 0 of the slot is h ^ L / 16,
    // the lane's part; bits 1 and 2 are constants
    const int vt_lane = (lane & 31) * kVtStride + 8 * (h ^ ((lane & 31) >> 4));
    // One 64-key tile: load the next tile (NEXT), the tile in two 32-key
    // halves -- each S^T = K . Q^T (the first k-step adds to an inline zero),
    // online softmax, then O^T += V^T . P^T with A = V^T rows (dims) and the
    // keys in accumulator order -- then stage the next tile in LDS.
    const bool diag = causal != 0;
    // this column's token-tree mask over the chunk's keys (none: all seen)
    const int tbase = tree_mask ? pos0 : 0x7fffffff;
    const uint64_t tmask = tree_mask && col_valid ? tree_mask[q_begin + r] : ~0ull;
    float vref_o = 0.0f;  // units of O (BSC): the V reference of the last tile computed
    auto run_tile = [&](int j, auto mask_c, bool next, auto check_c) {
        constexpr bool MASK = decltype(mask_c)::value;
        const int k0 = j * kKT;
        const int buf = j & 1;
        if constexpr (BSC) {
            // this tile's V values are in units of its reference, which only
            // grows: bring O to it first
            const float vb = s_sc[8 * buf + 4];
            if (vb > vref_o) {
                const float f = vref_o / vb;
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[mb][e] *= f;
                vref_o = vb;
            }
        }
        if (next)
            load_next(sg, k0 + kKT, check_c);
        // S for both halves first, so that each half's softmax (VALU) has
        // matrix-core work in flight beside it: the second half's S during
        // the first softmax, the first half's P V during the second
        f32x16_t sc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const uint16_t* krow = s_ks[buf] + (32 * kb + (lane & 31)) * kKsStride + 8 * h;
            const f32x16_t zero = {};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(krow + 16 * kk));
                sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], kk == 0 ? zero : sc[kb], 0, 0, 0);
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            // the half's eight V^T operands, read before its softmax so the
            // LDS latency hides behind it: keys 16 ks + 4 h .. + 3 and
            // 16 ks + 8 + 4 h .. + 3 of the half, unit 4 kb + 2 ks + h of
            // row d = 32 mb + L
            f16x8_t va[2][4];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const uint16_t* vrow = s_vt[buf] + 32 * mb * kVtStride + 32 * (kb ^ (mb >> 1)) +
                                           16 * (ks ^ (mb & 1));
                    va[ks][mb] = *reinterpret_cast<const f16x8_t*>(vrow + vt_lane);
                }
            f16x8_t pf[2];  // P^T fragments, keys 16 ks .. 16 ks + 15 of the half
            if constexpr (BSC) {
                // the half's keys 0 .. 15 (elements 0 .. 7) lie in 16-key
                // group 2 kb, keys 16 .. 31 in group 2 kb + 1: each group's
                // K scale joins its score scale
                const float ka = cl2 * s_sc[8 * buf + 2 * kb], kz = cl2 * s_sc[8 * buf + 2 * kb + 1];
                softmax_half<MASK, true>(sc[kb], pf, o, m_run, l_run, ka, k0 + 32 * kb, h, pos, ctx,
                                         diag, tmask, tbase, kz);
            } else {
                softmax_half<MASK>(sc[kb], pf, o, m_run, l_run, cl2, k0 + 32 * kb, h, pos, ctx,
                                   diag, tmask, tbase);
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
                    o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[ks][mb], pf[ks], o[mb], 0, 0, 0);
        }
        if (next) store_tile(sg, buf ^ 1);
        __syncthreads();
    };
    // Only tiles that reach the causal diagonal (k0 + 63 > pos0 + r0) or the
    // context's end (k0 + 64 > ctx) need masks; they are the last ones.  The
    // tiles before them, all with a next tile, run in a loop of their own with
    // no branch in its body.  (A segment's last tile always takes the masked
    // path; its masks then drop nothing.)
    // A wave none of whose columns is a real query row (short chunks: a verify
    // chunk of 6 rows x 4 heads fills 24 of the 128 columns) only stages its
    // share of every tile for the others and meets them at each tile's
    // barrier; its results would be discarded.  It leaves after the last
    // barrier, when no wave reads the tile buffers any more.
    if (r0 + (wave * 32) / G >= lq) {
        for (int jj = t0; jj < t1; ++jj) {
            if (jj + 1 < t1) {
                load_next(sg, (jj + 1) * kKT, std::true_type{});
                store_tile(sg, (jj + 1) & 1);
            }
            __syncthreads();
        }
        return;
    }
    // with token-tree masks every key of the chunk may be dropped, so masks
    // start at the chunk's first position
    const int first_pos = tree_mask ? pos0 : pos0 + r0;
    const int j_diag = causal ? (first_pos >= kKT - 1 ? (first_pos - (kKT - 1)) / kKT + 1 : 0) : ntiles;
    const int j_tail = ctx >= kKT ? (ctx - kKT) / kKT + 1 : 0;
    int j_plain = j_diag < j_tail ? j_diag : j_tail;
    j_plain = j_plain < t1 - 1 ? j_plain : t1 - 1;
    // A tile before j_plain lies wholly before kv_end (it ends before the
    // first query position and the context's end), so while the next tile
    // is one of those its loads need no bounds check.
    int j = t0;
    for (; j < j_plain - 1; ++j) run_tile(j, std::false_type{}, true, std::false_type{});
    for (; j < j_plain; ++j) run_tile(j, std::false_type{}, true, std::true_type{});
    for (; j < t1; ++j) run_tile(j, std::true_type{}, j + 1 < t1, std::true_type{});

    // ---- finish: total l over both halves, then out = O / l
    const float lt = sum_lane_halves(l_run);
    if (!col_valid) return;
    if constexpr (BSC) {
        // O in absolute units
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[mb][e] *= vref_o;
    }
    if (rec_col) {  // part of the item's keys: the record of this column
        float* rp = rec_col;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                *reinterpret_cast<float4*>(rp + 32 * mb + 8 * e4 + 4 * h) =
                    make_float4(o[mb][4 * e4], o[mb][4 * e4 + 1], o[mb][4 * e4 + 2], o[mb][4 * e4 + 3]);
        if (h == 0) {
            rp[D] = m_run;
            rp[D + 1] = lt;
        }
        return;
    }
    const float inv = ntiles > 0 ? out_scale / lt : 0.0f;
    const size_t orow = ((size_t)(q_begin + r) * num_q_heads + (size_t)kvh * G + g) * D;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const int d0 = 32 * mb + 8 * e4 + 4 * h;
            const float x0 = o[mb][4 * e4 + 0] * inv, x1 = o[mb][4 * e4 + 1] * inv;
            const float x2 = o[mb][4 * e4 + 2] * inv, x3 = o[mb][4 * e4 + 3] * inv;
            if (OUT_BF16) {
                uint2 w;
                w.x = (uint32_t)f32_to_bf16_rne(x0) | ((uint32_t)f32_to_bf16_rne(x1) << 16);
                w.y = (uint32_t)f32_to_bf16_rne(x2) | ((uint32_t)f32_to_bf16_rne(x3) << 16);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow + d0) = w;
            } else {
                *reinterpret_cast<float4*>(static_cast<float*>(out) + orow + d0) =
                    make_float4(x0, x1, x2, x3);
            }
        }
}


// Query slot `slot` of KV head kvh in a grid of num_q_tokens / P + num_seqs
// slots per KV head, P = 128 / G query positions each: slot y belongs to
// sequence i with T(i) <= y < T(i + 1), T(i) = cu_q_lens[i] / P + i (T never
// skips a needed slot), and holds its rows (y - T(i)) P onwards; runs all
// its key tiles, or nothing for a slot past its chunk's rows or (with the
// decode rows taken elsewhere) of a single-row sequence.
// The sequence and rows of query slot `slot` (P positions per slot): false
// for a slot with nothing to do.  Wave-uniform; every wave of the block
// takes the same decision.
struct SlotRows {
    int seq, q_begin, lq, r0, ctx, ntiles;
};
template <int P>
__device__ __forceinline__ bool slot_rows(SlotRows& sr, const int32_t* __restrict__ cu_q_lens,
                                          const int32_t* __restrict__ context_lens,
                                          int max_context_len, int num_seqs, int causal,
                                          int decode_rows_elsewhere, int slot) {
    const int lane = threadIdx.x & 63;
    // ---- which sequence owns this slot: 64-way search over T(i)
    int lo = 0, hi = num_seqs;  // T(lo) <= slot < T(hi), T(num_seqs) = grid size
    while (hi - lo > 1) {
        const int step = (hi - lo + 63) / 64;
        const int idx = lo + lane * step;
        const bool ok = idx < hi && (cu_q_lens[idx] / P + idx) <= slot;
        const unsigned long long m = __ballot(ok);  // low bits set, lane 0 always
        const int last = 63 - __builtin_clzll(m);
        lo = lo + last * step;
        const int nh = lo + step;
        hi = nh < hi ? nh : hi;
    }
    sr.seq = lo;
    sr.q_begin = cu_q_lens[lo];
    sr.lq = cu_q_lens[lo + 1] - sr.q_begin;
    sr.r0 = (slot - (sr.q_begin / P + lo)) * P;
    if (sr.r0 >= sr.lq) return false;
    if (decode_rows_elsewhere && sr.lq == 1) return false;
    int ctx = context_lens[lo];
    sr.ctx = ctx < 0 ? 0 : (ctx > max_context_len ? max_context_len : ctx);
    const int pos0 = sr.ctx - sr.lq;
    const int r_last = (sr.r0 + P < sr.lq ? sr.r0 + P : sr.lq) - 1;
    const int kv_end = causal ? (pos0 + r_last + 1 < sr.ctx ? pos0 + r_last + 1 : sr.ctx) : sr.ctx;
    sr.ntiles = (kv_end + kKT - 1) / kKT;
    return true;
}

template <int BS, int G, bool OUT_BF16, bool FP8, bool BSC = false>
__device__ __forceinline__ void run_slot(
    uint16_t (&s_ks)[2][kKsElems], uint16_t (&s_vt)[2][kVtElems], void* __restrict__ out,
    const uint16_t* __restrict__ q, const int32_t* __restrict__ cu_q_lens,
    const void* __restrict__ k_cache, const void* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, int max_blocks_per_seq,
    const int32_t* __restrict__ context_lens, int max_context_len, int num_seqs,
    int num_q_heads, int num_kv_heads, float scale_log2, float out_scale, int causal,
    int decode_rows_elsewhere, const uint64_t* __restrict__ tree_mask, int kvh, int slot,
    const float* __restrict__ k_scales = nullptr, const float* __restrict__ v_scales = nullptr,
    float* __restrict__ s_sc = nullptr) {
    SlotRows sr;
    if (!slot_rows<kCols / G>(sr, cu_q_lens, context_lens, max_context_len, num_seqs, causal,
                              decode_rows_elsewhere, slot))
        return;
    chunk_item<BS, G, OUT_BF16, FP8, BSC>(s_ks, s_vt, out, q, k_cache, v_cache,
                                          block_table + (size_t)sr.seq * max_blocks_per_seq,
                                          num_q_heads, num_kv_heads, scale_log2, out_scale, causal,
                                          tree_mask, sr.q_begin, sr.lq, sr.ctx, kvh, sr.r0, 0,
                                          sr.ntiles, nullptr, k_scales, v_scales, s_sc);
}

// The position, inside an XCD's run of (KV head, slot) items
// [run0, run0 + cnt) of a (slots, KV heads) grid, of the item whose rank by
// key tiles (descending, ties by position) is `want`.  LDS scratch:
// 2 num_seqs + 2 + cnt ints; every thread of the block calls it, and the
// scratch is free again when it returns.
template <int P, int NT>
__device__ __forceinline__ int ranked_item(int* scratch, const int32_t* __restrict__ cu_q_lens,
                                           const int32_t* __restrict__ context_lens,
                                           int max_context_len, int num_seqs, int causal,
                                           int decode_rows_elsewhere, int run0, int cnt, int want) {
    const int tid = threadIdx.x;
    int* s_cu = scratch;  // cu_q_lens, context_lens, works, pick
    int* s_ctx = s_cu + num_seqs + 1;
    int* s_w = s_ctx + num_seqs;
    int* s_pick = s_w + cnt;
    for (int i = tid; i <= num_seqs; i += NT) {
        s_cu[i] = cu_q_lens[i];
        if (i < num_seqs) s_ctx[i] = context_lens[i];
    }
    __syncthreads();
    for (int t = tid; t < cnt; t += NT) {
        const int sl = (run0 + t) % (int)gridDim.x;
        int lo = 0, hi = num_seqs;  // the last i with T(i) = cu_q_lens[i] / P + i <= sl
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_cu[mid] / P + mid <= sl) lo = mid; else hi = mid;
        }
        const int lq = s_cu[lo + 1] - s_cu[lo];
        const int r0 = (sl - (s_cu[lo] / P + lo)) * P;
        int work = 0;
        if (r0 < lq && !(decode_rows_elsewhere && lq == 1)) {
            int ctx = s_ctx[lo];
            ctx = ctx < 0 ? 0 : (ctx > max_context_len ? max_context_len : ctx);
            const int r_last = (r0 + P < lq ? r0 + P : lq) - 1;
            const int kv_end = causal ? (ctx - lq + r_last + 1 < ctx ? ctx - lq + r_last + 1 : ctx)
                                      : ctx;
            work = (kv_end + kKT - 1) / kKT;
        }
        s_w[t] = work;
    }
    __syncthreads();
    for (int t = tid; t < cnt; t += NT) {
        const int wt = s_w[t];
        int rank = 0;
        for (int u = 0; u < cnt; ++u) {
            const int wu = s_w[u];
            rank += (wu > wt || (wu == wt && u < t)) ? 1 : 0;
        }
        if (rank == want) *s_pick = t;
    }
    __syncthreads();
    const int pick = *s_pick;
    __syncthreads();  // the scratch goes back to its owner
    return pick;
}

// Grid: (num_q_tokens / P + num_seqs, num_kv_heads), P = 128 / G query
// positions per workgroup, remapped XCD by XCD; block 256.  Slot y of
// sequence i is y - T(i),
// T(i) = cu_q_lens[i] / P + i; T never skips a needed slot.  Each
// workgroup runs all key tiles of its (slot, KV head) item.
template <int BS, int G, bool OUT_BF16, bool FP8, bool BSC = false>
__global__ void __launch_bounds__(kThreads, 2)
prefill_mfma_kernel(void* __restrict__ out, const uint16_t* __restrict__ q,
                    const int32_t* __restrict__ cu_q_lens, const void* __restrict__ k_cache,
                    const void* __restrict__ v_cache, const int32_t* __restrict__ block_table,
                    int max_blocks_per_seq, const int32_t* __restrict__ context_lens,
                    int max_context_len, int num_seqs, int num_q_heads, int num_kv_heads,
                    float scale_log2, float out_scale, int causal, int decode_rows_elsewhere,
                    const uint64_t* __restrict__ tree_mask, int pair_cus,
                    const float* __restrict__ k_scales, const float* __restrict__ v_scales) {
    constexpr int P = kCols / G;
    __shared__ __attribute__((aligned(16))) uint16_t s_ks[2][kKsElems];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kVtElems];
    __shared__ float s_sc[BSC ? 16 : 1];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // The dispatcher deals workgroups to the 8 XCDs in turn, each with its
    // own L2: give each XCD a contiguous run of (KV head, slot) items, so the
    // query slots that read the same keys share one L2 (a bijection of the
    // grid onto itself).
    const int nwg = gridDim.x * gridDim.y;
    const int lin = blockIdx.y * gridDim.x + blockIdx.x;
    const int per = nwg / 8, rem = nwg % 8, xcd = lin % 8;
    const int run0 = xcd * per + (xcd < rem ? xcd : rem);
    int item = run0 + lin / 8;
    if (pair_cus > 0) {
        // Within an XCD the dispatcher hands workgroups to its pair_cus CUs
        // in turn, two per CU, so run positions p and p + pair_cus share a
        // CU, and the one left alone when its partner ends runs faster.
        // Causal slots differ in key tiles (up to 1.3x the mean for 512-row
        // chunks), so the run is taken in order of work: positions
        // 0 .. pair_cus - 1 get the heaviest items and the next pair_cus
        // positions the lighter half of the first 2 pair_cus in reverse, so
        // each CU holds a heavy and a light item; the rest follow in order.
        // A permutation of the run (ties by position), so still a bijection.
        const int cnt = per + (xcd < rem ? 1 : 0);
        const int p = lin / 8;
        const int m = cnt < 2 * pair_cus ? cnt : 2 * pair_cus;
        const int want = p < pair_cus ? p : (p < m ? m + pair_cus - 1 - p : p);
        item = run0 + ranked_item<P, kThreads>(reinterpret_cast<int*>(&s_ks[0][0]), cu_q_lens,
                                               context_lens, max_context_len, num_seqs, causal,
                                               decode_rows_elsewhere, run0, cnt, want);
    }
    const int kvh = item / gridDim.x;
    const int slot = item - kvh * gridDim.x;
    run_slot<BS, G, OUT_BF16, FP8, BSC>(s_ks, s_vt, out, q, cu_q_lens, k_cache, v_cache,
                                        block_table, max_blocks_per_seq, context_lens,
                                        max_context_len, num_seqs, num_q_heads, num_kv_heads,
                                        scale_log2, out_scale, causal, decode_rows_elsewhere,
                                        tree_mask, kvh, slot, k_scales, v_scales, s_sc);
}

// A mixed batch in one grid ("LLM 推理优化技术全景", Chunked Prefill,
// decode-maximal batching: the compute-bound chunk and the bandwidth-bound
// decodes share the machine).  The dispatcher deals workgroups to the 8 XCDs
// in turn and, inside an XCD, to its CUs in turn, two per CU; so the first
// dec_per_xcd workgroups of each XCD's run are decode workers (stream-K
// ranges over the decode rows' keys, one head group of up to 4 KV heads
// each) and take a slot on every CU and the second slot of half of them,
// and the rest are the chunks' query slots, an XCD-contiguous run each (as
// prefill_mfma_kernel deals them), which take the remaining slots and every
// slot freed later.  The decode workers' partial results are merged by the
// decode merge kernel afterwards.
// LDS: the chunk path's K / V^T tile buffers; a decode worker keeps its tile
// prefix sums, its waves' V tiles and their partial sums in them instead.
template <int BS, int G, bool OUT_BF16, bool FP8, bool BSC = false>
__global__ void __launch_bounds__(kThreads, 2)
mixed_kernel(void* __restrict__ out, const uint16_t* __restrict__ q,
             const int32_t* __restrict__ cu_q_lens, const void* __restrict__ k_cache,
             const void* __restrict__ v_cache, const int32_t* __restrict__ block_table,
             int max_blocks_per_seq, const int32_t* __restrict__ context_lens,
             int max_context_len, int num_seqs, int num_q_heads, int num_kv_heads,
             float scale_log2, float out_scale, int causal, float* __restrict__ dec_rec,
             int32_t* __restrict__ dec_seq_workers, int dec_workers, int dec_groups,
             int dec_per_xcd, int num_slots, int chunk_per_xcd,
             const uint64_t* __restrict__ tree_mask, const float* __restrict__ k_scales,
             const float* __restrict__ v_scales) {
    __shared__ __attribute__((aligned(16))) uint16_t s_ks[2][kKsElems];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kVtElems];
    __shared__ float s_sc[BSC ? 16 : 1];
    const int b = blockIdx.x;
    const int xcd = b % 8;
    const int k = b / 8;
    if (k < dec_per_xcd) {
        const int d = xcd * dec_per_xcd + k;
        if (d >= dec_workers * dec_groups) return;
        // the tile policies of the decode call (dispatched in decode.hip);
        // the waves' V tiles of the matrix-core ones, then the wave partials
        using KV8 = std::conditional_t<BSC, std::conditional_t<(G >= 4), dec::KvFp8MfmaBh, dec::KvFp8WideBh>,
                                       std::conditional_t<(G >= 4), dec::KvFp8Mfma, dec::KvFp8Wide>>;
        using KV = std::conditional_t<FP8, KV8, std::conditional_t<(G >= 8), dec::KvBf16Mfma, dec::KvBf16>>;
        constexpr int kVxElems = (kThreads / 64) * dec::kVxWaveElems;
        static_assert(2 * kVxElems + 4 * (kThreads / 64) <= (int)sizeof(s_vt), "decode LDS");
        int32_t* s_cum = reinterpret_cast<int32_t*>(&s_ks[0][0]);
        uint16_t* s_vx = &s_vt[0][0];
        int32_t* s_part = reinterpret_cast<int32_t*>(s_vx + kVxElems);
        dec::decode_worker<KV, BS, G, OUT_BF16, kThreads / 64>(
            out, dec_rec, dec_seq_workers, q, k_cache, v_cache, block_table, max_blocks_per_seq,
            context_lens, max_context_len, num_seqs, num_q_heads, num_kv_heads, scale_log2,
            out_scale, dec_workers, cu_q_lens, s_cum, s_part, d % dec_workers, d / dec_workers,
            s_vx, 1, 1, nullptr, nullptr, nullptr, k_scales, v_scales);
        return;
    }
    const int item = xcd * chunk_per_xcd + (k - dec_per_xcd);
    if (k - dec_per_xcd >= chunk_per_xcd || item >= num_slots * num_kv_heads) return;
    const int kvh = item / num_slots;
    run_slot<BS, G, OUT_BF16, FP8, BSC>(s_ks, s_vt, out, q, cu_q_lens, k_cache, v_cache,
                                        block_table, max_blocks_per_seq, context_lens,
                                        max_context_len, num_seqs, num_q_heads, num_kv_heads,
                                        scale_log2, out_scale, causal, 1, tree_mask, kvh,
                                        item - kvh * num_slots, k_scales, v_scales, s_sc);
}

// Stream-K units of sequence i in a call of chunks that fit one workgroup
// (Lq <= max_q_len <= P): one per (KV head, 64-key tile) when its rows are
// ours.  A sequence with more rows than max_q_len breaks the call's
// contract; it gets no units (its columns would fall outside the records).
__device__ __forceinline__ int streamk_units(const int32_t* __restrict__ cu_q_lens,
                                             const int32_t* __restrict__ context_lens, int i,
                                             int max_context_len, int max_q_len, int num_kv_heads,
                                             int decode_rows_elsewhere) {
    const int lq = cu_q_lens[i + 1] - cu_q_lens[i];
    if (lq <= 0 || lq > max_q_len || (decode_rows_elsewhere && lq == 1)) return 0;
    int ctx = context_lens[i];
    ctx = ctx < 0 ? 0 : (ctx > max_context_len ? max_context_len : ctx);
    return num_kv_heads * ((ctx + kKT - 1) / kKT);
}

// Chunks that fit one workgroup (every sequence's rows are one slot, as in
// speculative-decoding verification) read each key once per KV head for a
// few queries: bandwidth-bound, with items of very different lengths.  A
// grid of one workgroup per item lasts as long as its longest context, so
// here the items' key tiles are laid end to end -- sequence-major, then KV
// head, then tile -- and cut into num_workers equal contiguous ranges, one
// per resident workgroup (as the decode kernel does).  A worker runs the
// items of its range in order; an item it covers whole finishes in place,
// a partial one (at most the first and the last of its range) leaves per
// column records in slot 0 or 1 of the worker, which
// prefill_streamk_merge_kernel folds in worker order.
// Grid: (num_workers); block 256; dynamic LDS (num_seqs + 1) int32 for the
// unit prefix sums, which workgroup 0 also stores in cum_out.
// Records: [num_workers][2][max_q_len * G][kRecStride] floats, column
// c = r G + g.
template <int BS, int G, bool OUT_BF16, bool FP8, bool BSC = false>
__global__ void __launch_bounds__(kThreads, 2)
prefill_streamk_kernel(void* __restrict__ out, float* __restrict__ rec,
                       int32_t* __restrict__ cum_out, const uint16_t* __restrict__ q,
                       const int32_t* __restrict__ cu_q_lens, const void* __restrict__ k_cache,
                       const void* __restrict__ v_cache, const int32_t* __restrict__ block_table,
                       int max_blocks_per_seq, const int32_t* __restrict__ context_lens,
                       int max_context_len, int num_seqs, int num_q_heads, int num_kv_heads,
                       float scale_log2, float out_scale, int causal, int decode_rows_elsewhere,
                       int num_workers, int max_q_len, const uint64_t* __restrict__ tree_mask,
                       const float* __restrict__ k_scales, const float* __restrict__ v_scales) {
    const int rec_cols = max_q_len * G;  // columns per record slot
    __shared__ __attribute__((aligned(16))) uint16_t s_ks[2][kKsElems];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kVtElems];
    __shared__ float s_sc[BSC ? 16 : 1];
    __shared__ int32_t s_part[kThreads / 64];
    extern __shared__ int32_t s_cum[];  // s_cum[i] = units of sequences < i
    const int tid = threadIdx.x;
    const int lane = tid & 63;

    // ---- prefix sums of per-sequence units: each thread sums `per`
    // consecutive sequences, each wave scans its 64 sums with lane shuffles,
    // one barrier passes the waves' totals around
    const int per = (num_seqs + kThreads - 1) / kThreads;
    int local = 0;
    for (int k = 0; k < per; ++k) {
        const int i = tid * per + k;
        if (i < num_seqs)
            local += streamk_units(cu_q_lens, context_lens, i, max_context_len, max_q_len,
                                   num_kv_heads, decode_rows_elsewhere);
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) s_part[tid >> 6] = incl;
    __syncthreads();
    int run = incl - local, total = 0;
#pragma unroll
    for (int k = 0; k < kThreads / 64; ++k) {
        const int t = s_part[k];
        run += k < (tid >> 6) ? t : 0;
        total += t;
    }
    for (int k = 0; k < per; ++k) {
        const int i = tid * per + k;
        if (i < num_seqs) {
            s_cum[i] = run;
            run += streamk_units(cu_q_lens, context_lens, i, max_context_len, max_q_len,
                                 num_kv_heads, decode_rows_elsewhere);
        }
    }
    if (tid == 0) s_cum[num_seqs] = total;
    __syncthreads();
    if (blockIdx.x == 0)
        for (int i = tid; i <= num_seqs; i += kThreads) cum_out[i] = s_cum[i];

    const int64_t U = s_cum[num_seqs];
    // never more workers than units, so every worker's range is non-empty
    const int64_t W = num_workers < U ? num_workers : U;
    const int64_t w = blockIdx.x;
    if (w >= W) return;  // the whole workgroup
    int64_t t = worker_start(w, U, W);
    const int64_t t_end = worker_start(w + 1, U, W);
    const int col = (tid >> 6) * 32 + (lane & 31);  // this lane's query column
    int slot = 0;
    while (t < t_end) {
        // sequence holding unit t: the last i with s_cum[i] <= t
        int lo = 0, hi = num_seqs;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_cum[mid] <= t) lo = mid; else hi = mid;
        }
        const int seq = lo;
        const int q_begin = cu_q_lens[seq];
        const int lq = cu_q_lens[seq + 1] - q_begin;
        int ctx = context_lens[seq];
        ctx = ctx < 0 ? 0 : (ctx > max_context_len ? max_context_len : ctx);
        const int n = (ctx + kKT - 1) / kKT;  // tiles per KV head, >= 1 here
        const int64_t u = t - s_cum[seq];
        const int kvh = (int)(u / n);
        const int tile0 = (int)(u - (int64_t)kvh * n);
        const int64_t item_end = t + (n - tile0);
        const int64_t seg_end = t_end < item_end ? t_end : item_end;
        const int t1 = tile0 + (int)(seg_end - t);
        // columns past the chunk's rows never write, so their record
        // address (beyond rec_cols) is never used
        float* rc = (tile0 != 0 || t1 != n)
                        ? rec + ((size_t)(w * 2 + slot) * rec_cols + col) * kRecStride
                        : nullptr;
        chunk_item<BS, G, OUT_BF16, FP8, BSC>(s_ks, s_vt, out, q, k_cache, v_cache,
                                              block_table + (size_t)seq * max_blocks_per_seq,
                                              num_q_heads, num_kv_heads, scale_log2, out_scale,
                                              causal, tree_mask, q_begin, lq, ctx, kvh, 0, tile0,
                                              t1, rc, k_scales, v_scales, s_sc);
        slot = 1;
        t = seg_end;
    }
}

// Finishes the rows of prefill_streamk_kernel's items that several workers
// shared, folding their records in worker order:
// M = max_k m_k, L = sum_k l_k 2^(m_k - M), out = sum_k O_k 2^(m_k - M) / L
// (the sequence-axis parallelism of "Flash Attention v2 的改进"); rows of a
// sequence with no key get zeros.
// Grid: (num_seqs, ceil(max_q_len * num_q_heads / CG / 4)); block: 4 waves,
// one (row, CG consecutive query heads of one KV head) each: their columns
// share one set of pieces, so a wave issues the (m, l) and the first A O rows
// of all CG columns before it waits for any.  Lane k holds piece k's m and l,
// and dims 2 lane, 2 lane + 1 of the output.
template <int G, int CG, bool OUT_BF16>
__global__ void __launch_bounds__(256)
prefill_streamk_merge_kernel(void* __restrict__ out, const float* __restrict__ rec,
                             const int32_t* __restrict__ cum, const int32_t* __restrict__ cu_q_lens,
                             int num_seqs, int num_q_heads, int num_kv_heads, int num_workers,
                             int rec_cols, int decode_rows_elsewhere, float out_scale) {
    static_assert(G % CG == 0, "a wave's columns belong to one KV head");
    constexpr int A = CG == 1 ? 8 : 4;  // O rows loaded together per column
    const int lane = threadIdx.x & 63;
    const int seq = blockIdx.x;
    const int item = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int q_begin = cu_q_lens[seq];
    const int lq = cu_q_lens[seq + 1] - q_begin;
    const int per_row = num_q_heads / CG;
    const int r = item / per_row;
    const int h0 = (item - r * per_row) * CG;  // first query head of the wave
    const int kvh = h0 / G;
    if (r >= lq) return;
    if (decode_rows_elsewhere && lq == 1) return;  // a decode row: not ours
    // element (head h0 + c, dims 2 lane, 2 lane + 1) of the row
    const size_t e0 = ((size_t)(q_begin + r) * num_q_heads + h0) * D + 2 * lane;
    auto store2 = [&](int c, float x0, float x1) {
        const size_t e = e0 + (size_t)c * D;
        if (OUT_BF16) {
            const uint32_t v = (uint32_t)f32_to_bf16_rne(x0) | ((uint32_t)f32_to_bf16_rne(x1) << 16);
            *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + e) = v;
        } else {
            *reinterpret_cast<float2*>(static_cast<float*>(out) + e) = make_float2(x0, x1);
        }
    };
    const int64_t units = cum[seq + 1] - cum[seq];
    if (units == 0) {  // no key to attend to
#pragma unroll
        for (int c = 0; c < CG; ++c) store2(c, 0.0f, 0.0f);
        return;
    }
    const int64_t n = units / num_kv_heads;
    const int64_t start = cum[seq] + (int64_t)kvh * n;
    const int64_t U = cum[num_seqs];
    const int64_t W = num_workers < U ? num_workers : U;
    const int64_t wf = worker_of(start, U, W);
    const int64_t wl = worker_of(start + n - 1, U, W);
    if (wf == wl) return;  // finished in place by its only worker
    const int slot_f = worker_start(wf, U, W) < start ? 1 : 0;
    // record column of query head h0 + c: r G + (h0 + c) % G
    auto rec_of = [&](int64_t w, int c) {
        const int slot = w == wf ? slot_f : 0;
        return rec + ((size_t)(w * 2 + slot) * rec_cols + r * G + h0 % G + c) * kRecStride;
    };
    // (m, l) of the first 64 pieces, one per lane, and the first A pieces'
    // O rows, for each column
    float2 ml0[CG];
    float2 av0[CG][A];
#pragma unroll
    for (int c = 0; c < CG; ++c) {
        ml0[c] = wf + lane <= wl ? *reinterpret_cast<const float2*>(rec_of(wf + lane, c) + D)
                                 : make_float2(-INFINITY, 0.0f);
#pragma unroll
        for (int u = 0; u < A; ++u)
            av0[c][u] = wf + u <= wl
                            ? *reinterpret_cast<const float2*>(rec_of(wf + u, c) + 2 * lane)
                            : make_float2(0.0f, 0.0f);
    }
#pragma unroll
    for (int c = 0; c < CG; ++c) {
        float mx = ml0[c].x;
        for (int64_t w = wf + 64 + lane; w <= wl; w += 64) mx = fmaxf(mx, rec_of(w, c)[D]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        // the pieces in worker order, 64 at a time: lane k holds the
        // scale exp2(m - mx) and the sum l of piece base + k; past the
        // first A, the O rows are loaded A pieces at a time
        float L = 0.0f, a0 = 0.0f, a1 = 0.0f;
        for (int64_t base = wf; base <= wl; base += 64) {
            const int cnt = wl - base + 1 < 64 ? (int)(wl - base + 1) : 64;
            float2 ml = ml0[c];
            if (base != wf)
                ml = lane < cnt ? *reinterpret_cast<const float2*>(rec_of(base + lane, c) + D)
                                : make_float2(-INFINITY, 0.0f);
            const float fk = lane < cnt ? fast_exp2(ml.x - mx) : 0.0f;
            const float lk = ml.y;
            for (int k = 0; k < cnt; k += A) {
                float2 av[A];
                if (base == wf && k == 0) {
#pragma unroll
                    for (int u = 0; u < A; ++u) av[u] = av0[c][u];
                } else {
#pragma unroll
                    for (int u = 0; u < A; ++u)
                        av[u] = k + u < cnt
                                    ? *reinterpret_cast<const float2*>(rec_of(base + k + u, c) + 2 * lane)
                                    : make_float2(0.0f, 0.0f);
                }
#pragma unroll
                for (int u = 0; u < A; ++u) {
                    if (k + u >= cnt) break;
                    const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fk), k + u));
                    L = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(lk), k + u)), f, L);
                    a0 = fmaf(av[u].x, f, a0);
                    a1 = fmaf(av[u].y, f, a1);
                }
            }
        }
        const float inv = out_scale / L;
        store2(c, a0 * inv, a1 * inv);
    }
}

template <int BS, int G, bool OUT_BF16, bool FP8, bool BSC = false>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
    constexpr int P = kCols / G;
    if (a.streamk) {
        auto kern = prefill_streamk_kernel<BS, G, OUT_BF16, FP8, BSC>;
        const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int32_t);
        int resident = 0;
        hipError_t e = resident_workgroups(reinterpret_cast<const void*>(kern), kThreads, lds,
                                           &resident);
        if (e != hipSuccess) return e;
        // as many workers as the chip holds at once, never more than the
        // records in the workspace allow
        int64_t workers = resident < a.max_workers ? resident : a.max_workers;
        if (workers < 1) workers = 1;
        hipLaunchKernelGGL(kern, dim3((int)workers), dim3(kThreads), lds, stream, a.out,
                           a.records, a.cum, a.q, a.cu_q_lens, a.k_cache, a.v_cache,
                           a.block_table, a.max_blocks_per_seq, a.context_lens,
                           a.max_context_len, a.num_seqs, a.num_q_heads, a.num_kv_heads,
                           a.scale_log2, a.out_scale, a.causal ? 1 : 0,
                           a.decode_rows_elsewhere ? 1 : 0, (int)workers, a.max_q_len,
                           a.tree_mask, a.k_scales, a.v_scales);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        // With about as many items (sequence, KV head) as workers, an item
        // is cut into two pieces or so and a merge wave takes the query heads
        // of one KV head together (4 columns' loads in flight: the 16-node
        // tree batch 176.5 -> 171.0 us per call, the 6-row verify batch
        // 130.8 -> 129.3); with many pieces per item one column per wave
        // gives more waves to the longer folds (8 long sequences: 440.5
        // against 448.1 us with 4 columns).
        constexpr int CG = G < 4 ? G : 4;
        const int64_t items = (int64_t)a.num_seqs * a.num_kv_heads;
        const int cols = 2 * items >= workers ? CG : 1;
        dim3 mgrid(a.num_seqs, (a.max_q_len * (a.num_q_heads / cols) + 3) / 4);
        auto merge = cols == 1 ? prefill_streamk_merge_kernel<G, 1, OUT_BF16>
                               : prefill_streamk_merge_kernel<G, CG, OUT_BF16>;
        hipLaunchKernelGGL(merge, mgrid, dim3(256), 0, stream, a.out, a.records, a.cum,
                           a.cu_q_lens, a.num_seqs, a.num_q_heads, a.num_kv_heads, (int)workers,
                           a.max_q_len * G, a.decode_rows_elsewhere ? 1 : 0, a.out_scale);
        return hipGetLastError();
    }
    const int slots = a.num_q_tokens / P + a.num_seqs;
    // Pair heavy and light slots on each CU when the whole grid is at most
    // about two rounds of the chip (the order is ranked in each workgroup,
    // in LDS the K tiles take later).
    auto kern = prefill_mfma_kernel<BS, G, OUT_BF16, FP8, BSC>;
    int pair_cus = 0;
    {
        int resident = 0, cus = 0, dev = 0;
        hipError_t e = resident_workgroups(reinterpret_cast<const void*>(kern), kThreads, 0,
                                           &resident);
        if (e == hipSuccess) e = hipGetDevice(&dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        const int64_t per = ((int64_t)slots * a.num_kv_heads + 7) / 8;
        const int h = cus / 8;
        if (cus % 8 == 0 && resident == 2 * cus && per <= 4 * h && a.num_seqs <= 4096 &&
            2 * (int64_t)a.num_seqs + 2 + per <= (int64_t)(kKsElems * 2 * sizeof(uint16_t) / sizeof(int)))
            pair_cus = h;
    }
    hipLaunchKernelGGL(kern, dim3(slots, a.num_kv_heads),
                       dim3(kThreads), 0, stream, a.out, a.q, a.cu_q_lens, a.k_cache, a.v_cache,
                       a.block_table, a.max_blocks_per_seq, a.context_lens, a.max_context_len,
                       a.num_seqs, a.num_q_heads, a.num_kv_heads, a.scale_log2, a.out_scale,
                       a.causal ? 1 : 0, a.decode_rows_elsewhere ? 1 : 0, a.tree_mask, pair_cus,
                       a.k_scales, a.v_scales);
    return hipGetLastError();
}

template <int BS, int G>
hipError_t launch_prefill_g(const PrefillArgs& a, hipStream_t s) {
    if (a.kv_fp8 && a.k_scales != nullptr)
        return a.out_bf16 ? launch_prefill_t<BS, G, true, true, true>(a, s)
                          : launch_prefill_t<BS, G, false, true, true>(a, s);
    if (a.kv_fp8)
        return a.out_bf16 ? launch_prefill_t<BS, G, true, true>(a, s)
                          : launch_prefill_t<BS, G, false, true>(a, s);
    return a.out_bf16 ? launch_prefill_t<BS, G, true, false>(a, s)
                      : launch_prefill_t<BS, G, false, false>(a, s);
}

template <int BS>
hipError_t launch_prefill_bs(const PrefillArgs& a, hipStream_t s) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_prefill_g<BS, 1>(a, s);
        case 2: return launch_prefill_g<BS, 2>(a, s);
        case 4: return launch_prefill_g<BS, 4>(a, s);
        case 8: return launch_prefill_g<BS, 8>(a, s);
        case 16: return launch_prefill_g<BS, 16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

// Workgroups of the mixed grid's decode role on each XCD of 32 CUs: every
// CU holds one and half the CUs a second (for 4 x 512 chunks + 128 decodes:
// 219 us per call against 228 with one per CU, 223 with 40 and 226 with 56).
constexpr int kMixedCusPerXcd = 32;
constexpr int kMixedDecodePerXcd = 48;

template <int BS, int G, bool OUT_BF16, bool FP8, bool BSC = false>
hipError_t launch_mixed_t(const PrefillArgs& a, const DecodeArgs& d, hipStream_t stream) {
    constexpr int P = kCols / G;
    auto kern = mixed_kernel<BS, G, OUT_BF16, FP8, BSC>;
    int resident = 0, cus = 0, dev = 0;
    hipError_t e = resident_workgroups(reinterpret_cast<const void*>(kern), kThreads, 0,
                                       &resident);
    if (e == hipSuccess) e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // the layout the role split assumes: 8 XCDs of kMixedCusPerXcd CUs
    // holding two workgroups each, and the decode's prefix sums in the tile
    // buffers
    if (cus != 8 * kMixedCusPerXcd || resident != 2 * cus ||
        (int64_t)(a.num_seqs + 1) * (int64_t)sizeof(int32_t) > (int64_t)sizeof(uint16_t) * 2 * kKsElems)
        return hipErrorNotSupported;
    const int dec_groups = (a.num_kv_heads + 3) / 4;
    int64_t dec_workers = (8 * kMixedDecodePerXcd) / dec_groups;
    if (dec_workers > d.max_workers) dec_workers = d.max_workers;
    if (dec_workers < 1) dec_workers = 1;
    const int dec_per_xcd = (int)((dec_workers * dec_groups + 7) / 8);
    const int num_slots = a.num_q_tokens / P + a.num_seqs;
    const int chunk_per_xcd = (num_slots * a.num_kv_heads + 7) / 8;
    hipLaunchKernelGGL(kern, dim3(8 * (dec_per_xcd + chunk_per_xcd)), dim3(kThreads), 0, stream,
                       a.out, a.q, a.cu_q_lens, a.k_cache, a.v_cache, a.block_table,
                       a.max_blocks_per_seq, a.context_lens, a.max_context_len, a.num_seqs,
                       a.num_q_heads, a.num_kv_heads, a.scale_log2, a.out_scale, a.causal ? 1 : 0,
                       d.records, d.seq_workers, (int)dec_workers, dec_groups, dec_per_xcd,
                       num_slots, chunk_per_xcd, a.tree_mask, a.k_scales, a.v_scales);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode_merge(d, stream);
}

template <int BS, int G>
hipError_t launch_mixed_g(const PrefillArgs& a, const DecodeArgs& d, hipStream_t s) {
    if (a.kv_fp8 && a.k_scales != nullptr)
        return a.out_bf16 ? launch_mixed_t<BS, G, true, true, true>(a, d, s)
                          : launch_mixed_t<BS, G, false, true, true>(a, d, s);
    if (a.kv_fp8)
        return a.out_bf16 ? launch_mixed_t<BS, G, true, true>(a, d, s)
                          : launch_mixed_t<BS, G, false, true>(a, d, s);
    return a.out_bf16 ? launch_mixed_t<BS, G, true, false>(a, d, s)
                      : launch_mixed_t<BS, G, false, false>(a, d, s);
}

template <int BS>
hipError_t launch_mixed_bs(const PrefillArgs& a, const DecodeArgs& d, hipStream_t s) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_mixed_g<BS, 1>(a, d, s);
        case 2: return launch_mixed_g<BS, 2>(a, d, s);
        case 4: return launch_mixed_g<BS, 4>(a, d, s);
        case 8: return launch_mixed_g<BS, 8>(a, d, s);
        case 16: return launch_mixed_g<BS, 16>(a, d, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool prefill_streamk(int max_q_len, int group) {
    return max_q_len >= 2 && max_q_len * group <= kCols;
}

int64_t prefill_streamk_max_workers(int num_seqs, int num_kv_heads, int max_context_len) {
    const int64_t units =
        (int64_t)num_seqs * num_kv_heads * ((max_context_len + kKT - 1) / kKT);
    const int64_t w = units < kMaxChunkWorkers ? units : kMaxChunkWorkers;
    return w < 1 ? 1 : w;
}

size_t prefill_streamk_bytes(int num_seqs, int max_q_len, int group, int num_kv_heads,
                             int max_context_len) {
    const size_t cum = ((size_t)(num_seqs + 1) * sizeof(int32_t) + 255) / 256 * 256;
    return cum + (size_t)prefill_streamk_max_workers(num_seqs, num_kv_heads, max_context_len) *
                     2 * max_q_len * group * kRecStride * sizeof(float);
}

hipError_t launch_mixed(const PrefillArgs& a, const DecodeArgs& d, hipStream_t stream) {
    return a.block_size == 16 ? launch_mixed_bs<16>(a, d, stream) : launch_mixed_bs<32>(a, d, stream);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    return a.block_size == 16 ? launch_prefill_bs<16>(a, stream) : launch_prefill_bs<32>(a, stream);
}

}  // namespace pkv
