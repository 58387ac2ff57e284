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
// Key split (chunks of a few rows, as in speculative-decoding verification:
// at most 64 of the 128 columns used): such a call reads every key once
// per KV head for a handful of queries, so it is bandwidth-bound.  When its
// (slot, KV head) items are too few to fill the chip (a few long contexts),
// a workgroup takes one piece of at most split_tiles key tiles of its item
// instead of the whole item; an item of one piece finishes in place,
// the pieces of a longer one leave their unnormalised O, reference maximum
// m and sum l per real column in the workspace, and prefill_merge_kernel
// combines them: M = max m_k, L = sum l_k 2^(m_k - M),
// out = sum O_k 2^(m_k - M) / L (the sequence-axis parallelism of "Flash
// Attention v2 的改进").
#include <type_traits>

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
// V^T rows in LDS: 64 keys + 8 fp16 of padding (144 B), with the sixteen
// 4-key groups of row d stored at group index g ^ vt_swizzle(d).  With
// both, the staging stores (four bytes, two keys of one dim per lane) and
// the MFMA operand reads (eight bytes, four keys per lane) each touch every
// bank equally often.
constexpr int kVtStride = kKT + 8;
__device__ __forceinline__ int vt_swizzle(int d) { return (d >> 3) & 15; }
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
};

// Global -> register staging of one 64-key tile: K chunks (4 x 16 B) and V
// chunks (2 key pairs x 2 halves of the tile, 4 x 16 B) per thread.
struct Stage {
    uint4 k[4];
    uint4 v[4];
};

// This thread's byte offsets inside a block for its staging loads: row
// within the block times the row pitch, plus its 16-byte chunk of the head's
// 256 bytes.  K load i carries key k0 + kq + 16 i, V load 2 j + p key
// k0 + 2 kq + p + 32 j; k0 is a multiple of 64, hence of the block size, so
// the offsets are the same for every tile.
template <int BS>
__device__ __forceinline__ void stage_offsets(uint32_t (&koff)[4], uint32_t (&voff)[4],
                                              uint32_t row_bytes, int tid) {
    const int col = tid & 15;
    const int kq = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) koff[i] = (uint32_t)((kq + 16 * i) % BS) * row_bytes + col * 16;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int p = 0; p < 2; ++p)
            voff[2 * j + p] = (uint32_t)((2 * kq + p + 32 * j) % BS) * row_bytes + col * 16;
}

// Loads one 64-key tile into registers.  Every load of a wave reads one
// physical block: K load i lies in the tile's 16-key group i, V load 2 j + p
// in group 2 j + (kq >= 8), and kq = 4 wave + lane / 16 is at least 8 for
// waves 2 and 3 only.  So the block's address is a scalar buffer base and
// the lane offsets are the fixed ones above; keys past kv_end read zeros
// without a memory access.  kbase / vbase point at this KV head's slice of
// block 0 of the pools.
template <int BS>
__device__ __forceinline__ void stage_load(Stage& sg, PrefillIds& ids, const char* kbase,
                                           const char* vbase, int k0, int kv_end,
                                           size_t block_bytes, const uint32_t (&koff)[4],
                                           const uint32_t (&voff)[4], int tid, int lane) {
    const int kq = tid >> 4;
    const bool upper = (tid >> 6) >= 2;  // wave-uniform: kq >= 8
    // ids of the tile's four 16-key groups, fetched in increasing order (the
    // window only moves forward)
    int id[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) id[i] = ids.get((k0 + 16 * i) / BS, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __amdgpu_buffer_rsrc_t r = buffer_rsrc(kbase + (size_t)id[i] * block_bytes);
        const uint32_t o = k0 + kq + 16 * i < kv_end ? koff[i] : kBufferOob;
        sg.k[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const __amdgpu_buffer_rsrc_t r =
            buffer_rsrc(vbase + (size_t)(upper ? id[2 * j + 1] : id[2 * j]) * block_bytes);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const uint32_t o = k0 + 2 * kq + p + 32 * j < kv_end ? voff[2 * j + p] : kBufferOob;
            sg.v[2 * j + p] =
                __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
        }
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
    // V^T[dim][key] as fp16 pairs of adjacent keys: keys 2 kq + 32 j and
    // the next one are in group kq / 2 + 8 j at offset 2 (kq % 2); this
    // thread's dims 8 col .. 8 col + 7 all have swizzle col, so the group
    // lands at (kq / 2 ^ col) ^ 8 j
    uint16_t* vcol = vt + col * 8 * kVtStride + 4 * ((kq / 2) ^ col) + 2 * (kq % 2);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint4 a = sg.v[2 * j];
        const uint4 b = sg.v[2 * j + 1];
        const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
        const uint32_t wb[4] = {b.x, b.y, b.z, b.w};
        // XOR with 8 j flips bit 3 of the group index: +-32 fp16
        uint16_t* vj = vcol + (j == 0 ? 0 : (((kq / 2) ^ col) & 8 ? -32 : 32));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            *reinterpret_cast<uint32_t*>(vj + (2 * w) * kVtStride) = pack_f16x2(bf16_lo(wa[w]), bf16_lo(wb[w]));
            *reinterpret_cast<uint32_t*>(vj + (2 * w + 1) * kVtStride) = pack_f16x2(bf16_hi(wa[w]), bf16_hi(wb[w]));
        }
    }
}

// Online-softmax step for one 32-key half tile of this lane's query column:
// raw scores s (element e is key kb0 + 8 (e / 4) + 4 h + e % 4) -> P^T
// fragments (fp16, k-steps of 16 keys) and the updated running max / sum,
// with O rescaled.  MASK (diagonal or last tile only) drops keys after the
// column's position or past the context.
constexpr float kLazyMax = 8.0f;  // p < 2^8 between rescales

template <bool MASK>
__device__ __forceinline__ void softmax_half(f32x16_t& s, f16x8_t (&pf)[2], f32x16_t (&o)[4],
                                             float& m_run, float& l_run, float cl2, int kb0, int h,
                                             int pos, int ctx, bool diag, uint64_t tmask,
                                             int tbase) {
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
        mt4[e & 3] = fmaxf(mt4[e & 3], s[e]);
    }
    float mt = fmaxf(fmaxf(mt4[0], mt4[1]), fmaxf(mt4[2], mt4[3]));
    mt = fmaxf(mt, xor_lane(mt, 32)) * cl2;
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
    float ls4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        float p = fast_exp2(fmaf(s[e], cl2, -mn));
        // a dropped key must give 0 even for a zero scale
        if (MASK) p = s[e] == -3.402823466e38f ? 0.0f : p;
        ls4[e & 3] += p;
        pf[e >> 3][e & 7] = (_Float16)p;
    }
    l_run = fmaf(l_run, alpha, (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]));
}

constexpr int kRecStride = D + 4;  // floats per split record: O[128], m, l, 2 pad
constexpr int kMinSplitTiles = 8;  // a piece streams at least 512 keys ...
constexpr int kMaxPieces = 32;     // ... and an item has at most 32 pieces
constexpr int64_t kSplitBelowItems = 256;
constexpr int64_t kSplitTargetGroups = 2048;

// Key tiles of the (slot, KV head) item that holds query row r of a
// sequence with lq rows and context ctx (the slot's last row decides).
template <int G>
__device__ __forceinline__ int item_tiles(int r, int lq, int ctx, int causal) {
    constexpr int P = kCols / G;
    const int r0 = r / P * P;
    const int r_last = (r0 + P < lq ? r0 + P : lq) - 1;
    const int pos0 = ctx - lq;
    const int kv_end = causal ? (pos0 + r_last + 1 < ctx ? pos0 + r_last + 1 : ctx) : ctx;
    return (kv_end + kKT - 1) / kKT;
}

// Grid: ((num_q_tokens / (128 / G) + num_seqs) * max_pieces, num_kv_heads);
// block 256.  x / max_pieces is the slot, x % max_pieces the piece (always 0
// without a key split).  Slot y of sequence i is y - T(i),
// T(i) = cu_q_lens[i] / P + i with P = 128 / G positions per workgroup; T
// never skips a needed slot.
template <int BS, int G, bool OUT_BF16>
__global__ void __launch_bounds__(kThreads, 2)
prefill_mfma_kernel(void* __restrict__ out, const uint16_t* __restrict__ q,
                    const int32_t* __restrict__ cu_q_lens, const uint16_t* __restrict__ k_cache,
                    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
                    int max_blocks_per_seq, const int32_t* __restrict__ context_lens,
                    int max_context_len, int num_seqs, int num_q_heads, int num_kv_heads,
                    float scale_log2, int causal, int decode_rows_elsewhere, int split_tiles,
                    int max_pieces, float* __restrict__ rec, int num_q_tokens,
                    const uint64_t* __restrict__ tree_mask) {
    constexpr int P = kCols / G;  // query positions per workgroup
    __shared__ __attribute__((aligned(16))) uint16_t s_ks[2][kKsElems];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kVtElems];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kvh = blockIdx.y;
    const int slot = blockIdx.x / max_pieces;
    const int piece = blockIdx.x - slot * max_pieces;

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
    const int seq = lo;
    const int q_begin = cu_q_lens[seq];
    const int lq = cu_q_lens[seq + 1] - q_begin;
    const int tile = slot - (q_begin / P + seq);
    const int r0 = tile * P;
    if (r0 >= lq) return;
    if (decode_rows_elsewhere && lq == 1) return;
    int ctx = context_lens[seq];
    ctx = ctx < 0 ? 0 : (ctx > max_context_len ? max_context_len : ctx);
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
    // this workgroup's key tiles [t0, t1) and the item's piece count
    int t0 = 0, t1 = ntiles, npieces = 1;
    if (split_tiles > 0) {
        t0 = piece * split_tiles;
        if (piece > 0 && t0 >= ntiles) return;  // piece 0 also covers ntiles == 0
        t1 = t0 + split_tiles < ntiles ? t0 + split_tiles : ntiles;
        npieces = (ntiles + split_tiles - 1) / split_tiles;
        npieces = npieces > 1 ? npieces : 1;
    }

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

    const uint32_t row_bytes = (uint32_t)num_kv_heads * D * sizeof(uint16_t);
    const size_t block_bytes = (size_t)BS * row_bytes;
    const char* kbase = reinterpret_cast<const char*>(k_cache) + (size_t)kvh * D * sizeof(uint16_t);
    const char* vbase = reinterpret_cast<const char*>(v_cache) + (size_t)kvh * D * sizeof(uint16_t);
    uint32_t koff[4], voff[4];
    stage_offsets<BS>(koff, voff, row_bytes, tid);
    PrefillIds ids;
    ids.init(block_table + (size_t)seq * max_blocks_per_seq, (ctx + BS - 1) / BS,
             t0 * kKT / BS, lane);

    Stage sg;
    if (t1 > t0) {
        stage_load<BS>(sg, ids, kbase, vbase, t0 * kKT, kv_end, block_bytes, koff, voff, tid,
                       lane);
        stage_store(sg, s_ks[t0 & 1], s_vt[t0 & 1], tid);
    }
    __syncthreads();

    // this lane's part of its V^T operand addresses (see the PV loop)
    const int vt_lo = (lane & 31) * kVtStride + 4 * (h ^ ((lane & 31) >> 3));
    const int vt_hi = (lane & 31) * kVtStride + 4 * ((h ^ ((lane & 31) >> 3)) ^ 2);
    // One 64-key tile: load the next tile (NEXT), the tile in two 32-key
    // halves -- each S^T = K . Q^T (the first k-step adds to an inline zero),
    // online softmax, then O^T += V^T . P^T with A = V^T rows (dims) and the
    // keys in accumulator order -- then stage the next tile in LDS.
    const bool diag = causal != 0;
    // this column's token-tree mask over the chunk's keys (none: all seen)
    const int tbase = tree_mask ? pos0 : 0x7fffffff;
    const uint64_t tmask = tree_mask && col_valid ? tree_mask[q_begin + r] : ~0ull;
    auto run_tile = [&](int j, auto mask_c, bool next) {
        constexpr bool MASK = decltype(mask_c)::value;
        const int k0 = j * kKT;
        const int buf = j & 1;
        if (next)
            stage_load<BS>(sg, ids, kbase, vbase, k0 + kKT, kv_end, block_bytes, koff, voff, tid,
                           lane);
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
            f16x8_t pf[2];  // P^T fragments, keys 16 ks .. 16 ks + 15 of the half
            softmax_half<MASK>(sc[kb], pf, o, m_run, l_run, cl2, k0 + 32 * kb, h, pos, ctx, diag,
                               tmask, tbase);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    // keys 16 ks + 4 h .. + 3 and 16 ks + 8 + 4 h .. + 3 of the
                    // half are groups g = 8 kb + 4 ks + h and g + 2 of row
                    // d = 32 mb + L, swizzle 4 mb + L / 8: the lane's part
                    // (h ^ L / 8, and that ^ 2) is in vt_lo / vt_hi, the rest
                    // is a constant offset
                    const int cg = 4 * ((2 * kb + ks) ^ mb);
                    const uint16_t* vrow = s_vt[buf] + 32 * mb * kVtStride + 4 * cg;
                    const uint2 lo4 = *reinterpret_cast<const uint2*>(vrow + vt_lo);
                    const uint2 hi4 = *reinterpret_cast<const uint2*>(vrow + vt_hi);
                    const f16x8_t a = __builtin_bit_cast(f16x8_t, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
                    o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[ks], o[mb], 0, 0, 0);
                }
            }
        }
        if (next) stage_store(sg, s_ks[buf ^ 1], s_vt[buf ^ 1], tid);
        __syncthreads();
    };
    // Only tiles that reach the causal diagonal (k0 + 63 > pos0 + r0) or the
    // context's end (k0 + 64 > ctx) need masks; they are the last ones.  The
    // tiles before them, all with a next tile, run in a loop of their own with
    // no branch in its body.  (A piece's last tile always takes the masked
    // path; its masks then drop nothing.)
    // A wave none of whose columns is a real query row (short chunks: a verify
    // chunk of 6 rows x 4 heads fills 24 of the 128 columns) only stages its
    // share of every tile for the others and meets them at each tile's
    // barrier; its results would be discarded.
    if (r0 + (wave * 32) / G >= lq) {
        for (int jj = t0; jj < t1; ++jj) {
            if (jj + 1 < t1) {
                stage_load<BS>(sg, ids, kbase, vbase, (jj + 1) * kKT, kv_end, block_bytes, koff,
                               voff, tid, lane);
                stage_store(sg, s_ks[(jj + 1) & 1], s_vt[(jj + 1) & 1], tid);
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
    int j = t0;
    for (; j < j_plain; ++j) run_tile(j, std::false_type{}, true);
    for (; j < t1; ++j) run_tile(j, std::true_type{}, j + 1 < t1);

    // ---- finish: total l over both halves, then out = O / l
    const float lt = l_run + xor_lane(l_run, 32);
    if (!col_valid) return;
    if (npieces > 1) {  // one piece of several: the record of this column
        float* rp = rec + (((size_t)piece * num_q_tokens + (size_t)(q_begin + r)) * num_q_heads +
                           (size_t)kvh * G + g) * kRecStride;
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
    const float inv = ntiles > 0 ? 1.0f / lt : 0.0f;
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

// Combines the pieces of split items.  Grid: (num_seqs, ceil(max_q_len *
// num_q_heads / 4)); block: 4 waves, one (row, query head) each; lane k
// holds piece k's m and l, and dims 2 lane, 2 lane + 1 of the output.
template <int G, bool OUT_BF16>
__global__ void __launch_bounds__(256)
prefill_merge_kernel(void* __restrict__ out, const float* __restrict__ rec,
                     const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ context_lens,
                     int max_context_len, int num_q_heads, int num_q_tokens, int causal,
                     int decode_rows_elsewhere, int split_tiles) {
    const int lane = threadIdx.x & 63;
    const int seq = blockIdx.x;
    const int item = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int q_begin = cu_q_lens[seq];
    const int lq = cu_q_lens[seq + 1] - q_begin;
    const int r = item / num_q_heads;
    const int head = item - r * num_q_heads;
    if (r >= lq) return;
    if (decode_rows_elsewhere && lq == 1) return;
    int ctx = context_lens[seq];
    ctx = ctx < 0 ? 0 : (ctx > max_context_len ? max_context_len : ctx);
    const int npieces = (item_tiles<G>(r, lq, ctx, causal) + split_tiles - 1) / split_tiles;
    if (npieces <= 1) return;  // finished in place
    auto rec_of = [&](int k) {
        return rec + (((size_t)k * num_q_tokens + (size_t)(q_begin + r)) * num_q_heads + head) *
                         kRecStride;
    };
    float2 ml = make_float2(-INFINITY, 0.0f);
    if (lane < npieces) ml = *reinterpret_cast<const float2*>(rec_of(lane) + D);
    float mx = ml.x;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float fk = lane < npieces ? fast_exp2(ml.x - mx) : 0.0f;
    float lsum = ml.y * fk;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lsum += __shfl_xor(lsum, o);
    // eight pieces' rows in flight at a time
    float a0 = 0.0f, a1 = 0.0f;
    for (int k = 0; k < npieces; k += 8) {
        float2 av[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            av[u] = k + u < npieces ? *reinterpret_cast<const float2*>(rec_of(k + u) + 2 * lane)
                                    : make_float2(0.0f, 0.0f);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int kk = k + u < 63 ? k + u : 63;
            const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fk), kk));
            a0 = fmaf(av[u].x, f, a0);
            a1 = fmaf(av[u].y, f, a1);
        }
    }
    const float inv = 1.0f / lsum;
    const size_t e = ((size_t)(q_begin + r) * num_q_heads + head) * D + 2 * lane;
    if (OUT_BF16) {
        const uint32_t w = (uint32_t)f32_to_bf16_rne(a0 * inv) |
                           ((uint32_t)f32_to_bf16_rne(a1 * inv) << 16);
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + e) = w;
    } else {
        *reinterpret_cast<float2*>(static_cast<float*>(out) + e) = make_float2(a0 * inv, a1 * inv);
    }
}

template <int BS, int G, bool OUT_BF16>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
    constexpr int P = kCols / G;
    const int slots = a.num_q_tokens / P + a.num_seqs;
    const int pieces = a.split_tiles > 0 ? a.max_pieces : 1;
    dim3 grid(slots * pieces, a.num_kv_heads);
    hipLaunchKernelGGL((prefill_mfma_kernel<BS, G, OUT_BF16>), grid, dim3(kThreads), 0, stream,
                       a.out, a.q, a.cu_q_lens, a.k_cache, a.v_cache, a.block_table,
                       a.max_blocks_per_seq, a.context_lens, a.max_context_len, a.num_seqs,
                       a.num_q_heads, a.num_kv_heads, a.scale_log2, a.causal ? 1 : 0,
                       a.decode_rows_elsewhere ? 1 : 0, a.split_tiles, pieces, a.records,
                       a.num_q_tokens, a.tree_mask);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.split_tiles == 0) return e;
    dim3 mgrid(a.num_seqs, (a.max_q_len * a.num_q_heads + 3) / 4);
    hipLaunchKernelGGL((prefill_merge_kernel<G, OUT_BF16>), mgrid, dim3(256), 0, stream, a.out,
                       a.records, a.cu_q_lens, a.context_lens, a.max_context_len, a.num_q_heads,
                       a.num_q_tokens, a.causal ? 1 : 0, a.decode_rows_elsewhere ? 1 : 0,
                       a.split_tiles);
    return hipGetLastError();
}

template <int BS, int G>
hipError_t launch_prefill_g(const PrefillArgs& a, hipStream_t s) {
    return a.out_bf16 ? launch_prefill_t<BS, G, true>(a, s) : launch_prefill_t<BS, G, false>(a, s);
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

}  // namespace

void prefill_split_plan(int max_q_len, int group, int max_context_len, int num_seqs,
                        int num_kv_heads, int* split_tiles, int* max_pieces) {
    *split_tiles = 0;
    *max_pieces = 1;
    // only chunks with few query columns per workgroup stream keys ...
    if (max_q_len < 2 || max_q_len * group > kCols / 2) return;
    // ... and only when their items leave most of the chip idle: below half
    // of the 512 workgroups an MI355X runs at once (two per CU), the pieces
    // aim at about 2048 workgroups
    const int64_t items = (int64_t)num_seqs * num_kv_heads *
                          ((max_q_len + kCols / group - 1) / (kCols / group));
    if (items >= kSplitBelowItems) return;
    const int64_t want = (kSplitTargetGroups + items - 1) / items;
    const int pieces_goal = (int)(want < kMaxPieces ? want : kMaxPieces);
    const int tiles = (max_context_len + kKT - 1) / kKT;
    int s = (tiles + pieces_goal - 1) / pieces_goal;
    s = s > kMinSplitTiles ? s : kMinSplitTiles;
    const int pieces = (tiles + s - 1) / s;
    if (pieces < 2) return;
    *split_tiles = s;
    *max_pieces = pieces;
}

size_t prefill_record_bytes(int num_q_tokens, int num_q_heads, int max_pieces) {
    return (size_t)max_pieces * num_q_tokens * num_q_heads * kRecStride * sizeof(float);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    return a.block_size == 16 ? launch_prefill_bs<16>(a, stream) : launch_prefill_bs<32>(a, stream);
}

}  // namespace pkv
