// decode_core.h -- the decode worker of libpagedkv, shared by the decode
// kernels and the one-grid mixed prefill + decode kernel.
//
// softmax and a stream-K split of the keys over persistent waves.
//
// What it computes ("LLM 推理优化技术全景", "Flash Attention 深度剖析"): for
// every sequence i and query head h,
//     out[i,h,:] = sum_t exp(s_t - m) V[t,:] / sum_t exp(s_t - m),
//     s_t = scale * <q[i,h,:], K[t,:]>,
// over the sequence's context_lens[i] keys, which live in 16- or 32-token
// physical blocks found through the block table ("LLM 推理引擎深度解析 ...",
// section 2.1; "让 Agent 跑得快", section 五).  The keys are visited once, a
// 16-token tile at a time, keeping a running maximum m and running sum l and
// rescaling the accumulator by exp(m_old - m_new) whenever m grows (the
// page's "在线 Softmax"); the division by l is deferred to the very end as in
// its "Flash Attention v2 的改进".
//
// Split of the work (the sequence-axis parallelism of that section, taken
// to its balanced limit):
//   * a worker is a workgroup with one wave per KV head; the G = Hq/Hkv
//     query heads of a KV head ride along in its wave, so each K/V byte is
//     read from HBM once per KV head (GQA grouping), and the waves of a
//     worker read each physical block's rows of all heads together
//     (contiguous bs * Hkv * D bf16 of K, the same of V);
//   * all sequences' 16-token tiles are laid end to end and cut into W
//     equal contiguous ranges, one per persistent worker (W = what the chip
//     holds at once).  A worker walks its range sequence by sequence: a
//     sequence it covers whole is finalised in place; a piece of a sequence
//     shared with other workers leaves (m, l, unnormalised acc) per query
//     head in the workspace, and the merge kernel combines the pieces with
//     the same exp(m_k - M) rescale (a log-sum-exp merge);
//   * so every worker streams the same number of bytes, no workgroup is
//     launched without work, and long contexts split across many workers.
// Inside a wave (64 lanes = 4 rows of 16): a tile of one head is 4 KB of K
// and 4 KB of V, four 128-bit loads per lane each; lane (row r, col c) holds
// dims 8c..8c+7 of tokens 4i + r, i = 0..3; the 16-lane row reduces the QK
// partial sums with DPP adds; each row is its own online-softmax stream
// (tokens = r mod 4) merged with the other rows at the end of a piece; the
// next tile's loads are issued before the current tile's math.  An FP8
// cache (one byte per value) uses the same layout with 64-bit loads, or,
// for up to 4 query heads per KV head, 8 rows of 8 lanes holding 16 dims of
// 2 tokens each (see the storage policies below).  Scores are
// in the log2 domain (scale * log2 e folded in), exponentials are v_exp_f32.
#pragma once

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace dec {


// How the pools store a value, and the lane layout that goes with it.  A
// wave sees a 16-token tile of one KV head as rows of kRowLanes lanes: lane
// (row r, col c) holds dims kDims c .. kDims c + kDims - 1 of the tile's
// tokens kRows i + r, i = 0 .. kLoads - 1, one word per token, and the
// kRowLanes lanes of a row reduce their partial dot products with DPP.
//   * K comes out as bf16 pairs for the dot2 instructions (E4M3 to bf16 is
//     exact: every E4M3 value is a bf16 value);
//   * V comes out as floats, or, for FP8, as fp16 pairs over two tokens.
// The FP8 cache's two scales are applied outside the tile loop: k_scale
// inside the score scale, v_scale on the finished output.  Pools with one
// scale per (block, KV head) (kBlockScales) take them per tile instead.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// bf16 pools: 8 dims (16 bytes) per lane and token, rows of 16 lanes.
struct KvBf16 {
    static constexpr int kElemBytes = 2;
    static constexpr int kDims = 8;
    static constexpr bool kPairedPV = false;
    static constexpr bool kMfma = false;
    static constexpr bool kBlockScales = false;
    using Word = uint4;
    static __device__ __forceinline__ Word load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
    static __device__ __forceinline__ void k_pairs(const Word& w, uint32_t (&kp)[4]) {
        kp[0] = w.x; kp[1] = w.y; kp[2] = w.z; kp[3] = w.w;
    }
    static __device__ __forceinline__ void v_floats(const Word& w, float (&v)[8]) {
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
        v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
        v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    }
};

// bf16 pools on the matrix cores, for 8 or 16 query heads per KV head: the
// layout above repeats the G heads' dot products, their row sums and the
// softmax in every lane of a row, which makes the VALU work the bound from
// 8 heads on.  A tile of 16 tokens:
//   S[16 tokens][16 cols] = K Q^T: four v_mfma_f32_16x16x32_bf16, K straight
//     from HBM in the operand layout (lane l: token l % 16, dims
//     32 kb + 8 (l / 16) .. + 7), Q^T in registers (column l % 16 is query
//     head l % 16; columns past G are zero);
//   lane l then holds the scores of tokens 4 (l / 16) .. + 3 of head l % 16,
//     so the softmax takes 4 exponentials per lane, and the head's running
//     max is shared by its 4 lanes (a max over lanes l ^ 16, l ^ 32);
//   O[16 rows][128 dims] += P V: eight v_mfma_f32_16x16x16_f16 (one per 16
//     dims), P in fp16 straight from the score accumulator's layout, V
//     rounded to fp16 (exact for |v| in [2^-14, 65504]) and passed through a
//     16 x 128 tile of LDS that each wave owns, to read it back as 4 tokens
//     of one dim per lane.
// Lane l holds O rows (heads) 4 (l / 16) .. + 3, dim 16 nb + l % 16.
struct KvBf16Mfma : KvBf16 {
    static constexpr bool kMfma = true;
    // loads per lane and token for a tile's K (and V): 16 bytes each, load j
    // holding the 8 dims of k-block j, dims 32 j + 8 q4 .. + 7 for the lanes
    // of quarter q4 (64 contiguous bytes of a token per load)
    static constexpr int kMfmaLoads = 4;
    static __device__ __forceinline__ int mfma_dim(int kb, int q4) { return 32 * kb + 8 * q4; }
    static __device__ __forceinline__ uint32_t mfma_byte(int j, int q4) { return 2 * mfma_dim(j, q4); }
    // k-block kb of a token as 8 bf16 (the MFMA operand) and as 8 fp16 (the
    // V tile's format)
    static __device__ __forceinline__ uint4 k_bf16x8(const Word (&w)[4], int kb) { return w[kb]; }
    static __device__ __forceinline__ uint4 v_f16x8(const Word (&w)[4], int kb) {
        const uint32_t wd[4] = {w[kb].x, w[kb].y, w[kb].z, w[kb].w};
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f16x2_t hp = {(_Float16)bf16_lo(wd[e]), (_Float16)bf16_hi(wd[e])};
            h[e] = __builtin_bit_cast(uint32_t, hp);
        }
        return make_uint4(h[0], h[1], h[2], h[3]);
    }
};
constexpr int kVxStride = kHeadDim + 8;         // fp16 per token row of a wave's V tile
constexpr int kVxWaveElems = kTileTokens * kVxStride;

// FP8 codes in the OCP E4M3 format, decoded by the hardware conversions.
// Their P V runs on fp16 dot products over token pairs: a lane's tokens i
// and i + 1 give, for every dim, the pair (v_i, v_i+1) (a byte permute puts
// the two codes side by side, one conversion widens them to fp16 exactly)
// and (p_i, p_i+1) rounds to fp16 once per query head, so one
// v_dot2_f32_f16 does the work of two fp32 FMAs.  P is in [0, 1] and rounds
// with 2^-11 relative error, as in the chunked-prefill kernel.
template <int NWORDS>  // 32-bit words of codes per lane and token
struct KvFp8Base {
    static constexpr int kElemBytes = 1;
    static constexpr int kDims = 4 * NWORDS;
    static constexpr bool kPairedPV = true;
    static constexpr bool kMfma = false;
    static constexpr bool kBlockScales = false;
    template <bool HIGH>  // codes 2, 3 of the word instead of 0, 1
    static __device__ __forceinline__ uint32_t bf16_pair(uint32_t codes) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                                (int)codes, 1.0f, HIGH));
    }
    static __device__ __forceinline__ void k_pairs_of(const uint32_t (&w)[NWORDS],
                                                      uint32_t (&kp)[2 * NWORDS]) {
#pragma unroll
        for (int j = 0; j < NWORDS; ++j) {
            kp[2 * j] = bf16_pair<false>(w[j]);
            kp[2 * j + 1] = bf16_pair<true>(w[j]);
        }
    }
    static __device__ __forceinline__ void v_floats_of(const uint32_t (&w)[NWORDS],
                                                       float (&v)[4 * NWORDS]) {
#pragma unroll
        for (int j = 0; j < NWORDS; ++j) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[j], false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[j], true);
            v[4 * j] = lo[0]; v[4 * j + 1] = lo[1]; v[4 * j + 2] = hi[0]; v[4 * j + 3] = hi[1];
        }
    }
    // vp[e] = (value of token a, value of token b) at dim 4 j + e: word j of
    // each token holds dims 4 j .. 4 j + 3
    static __device__ __forceinline__ void pairs4(uint32_t a, uint32_t b, f16x2_t (&vp)[4]) {
        // bytes (a.k, b.k, a.k+1, b.k+1) of the two words, k = 0 and 2
        const uint32_t w0 = __builtin_amdgcn_perm(b, a, 0x05010400u);
        const uint32_t w1 = __builtin_amdgcn_perm(b, a, 0x07030602u);
        vp[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w0, 1.0f, false);
        vp[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w0, 1.0f, true);
        vp[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w1, 1.0f, false);
        vp[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w1, 1.0f, true);
    }
};

// FP8 pools, 16 dims (16 bytes) per lane and token, rows of 8 lanes: half
// the lanes share a token, so the row sums take three DPP steps instead of
// four and each softmax value is computed by 8 lanes instead of 16 (up to 4
// query heads per KV head).
struct KvFp8Wide : KvFp8Base<4> {
    using Word = uint4;
    static __device__ __forceinline__ Word load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
    static __device__ __forceinline__ void k_pairs(const Word& w, uint32_t (&kp)[8]) {
        k_pairs_of({w.x, w.y, w.z, w.w}, kp);
    }
    static __device__ __forceinline__ void v_floats(const Word& w, float (&v)[16]) {
        v_floats_of({w.x, w.y, w.z, w.w}, v);
    }
    static __device__ __forceinline__ void v_pairs4(const Word& a, const Word& b, int j,
                                                    f16x2_t (&vp)[4]) {
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
        pairs4(aw[j], bw[j], vp);
    }
};

// FP8 pools on the matrix cores: the tile of KvBf16Mfma, codes widened by
// the hardware conversions to bf16 for K and fp16 for V (both exact for
// E4M3), so the results differ from the VALU tiles' by rounding only (P in
// fp16 there too).  A lane loads 16 codes per load, two loads per token:
// load j of quarter q4 holds dims 64 j + 16 q4 .. + 15, and k-block kb takes
// half kb & 1 of load kb >> 1.  The dot product does not care which dims a
// k-block holds as long as the Q operand holds the same ones.
struct KvFp8Mfma : KvFp8Wide {
    static constexpr bool kMfma = true;
    static constexpr int kMfmaLoads = 2;
    static __device__ __forceinline__ int mfma_dim(int kb, int q4) {
        return 64 * (kb >> 1) + 16 * q4 + 8 * (kb & 1);
    }
    static __device__ __forceinline__ uint32_t mfma_byte(int j, int q4) { return 64 * j + 16 * q4; }
    static __device__ __forceinline__ uint2 half_of(const Word (&w)[2], int kb) {
        const Word& x = w[kb >> 1];
        return (kb & 1) ? make_uint2(x.z, x.w) : make_uint2(x.x, x.y);
    }
    static __device__ __forceinline__ uint4 k_bf16x8(const Word (&w)[2], int kb) {
        const uint2 c = half_of(w, kb);
        return make_uint4(bf16_pair<false>(c.x), bf16_pair<true>(c.x), bf16_pair<false>(c.y),
                          bf16_pair<true>(c.y));
    }
    static __device__ __forceinline__ uint4 v_f16x8(const Word (&w)[2], int kb) {
        const uint2 c = half_of(w, kb);
        const f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)c.x, 1.0f, false);
        const f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)c.x, 1.0f, true);
        const f16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)c.y, 1.0f, false);
        const f16x2_t e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)c.y, 1.0f, true);
        return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                          __builtin_bit_cast(uint32_t, d), __builtin_bit_cast(uint32_t, e));
    }
};

// FP8 pools with one scale per (physical block, KV head) for K and one for
// V, read per tile (a 16-token tile lies in one block): the K scale joins
// the score scale of that tile; the V scale enters P V as the ratio
// vs / vref <= 1 to a reference that only grows (the largest V scale the
// piece has met; the accumulator is rescaled by vref_old / vref_new when
// it moves, as for a running maximum), so P * ratio stays in [0, 1] for its
// fp16 rounding, and the piece's result is multiplied by vref at its end.
// The running sum l takes the unscaled weights.
struct KvFp8WideBh : KvFp8Wide {
    static constexpr bool kBlockScales = true;
};
struct KvFp8MfmaBh : KvFp8Mfma {
    static constexpr bool kBlockScales = true;
};

// A tile's two scales, from the [num_blocks][num_kv_heads] fp32 tables:
// lane-uniform buffer loads, issued with the tile's own loads (vector
// memory, so they complete in order with them).  Scalar loads measured no
// fewer vector registers and more spills on the two-block rows tile.
__device__ __forceinline__ void load_block_scales(const float* k_scales, const float* v_scales,
                                                  int phys, int num_kv_heads, int kvh, float& ks,
                                                  float& vs) {
    // the block's row of the table as the (wave-uniform) buffer base, the
    // head as the offset: a per-lane base would put a loop around each load
    const size_t b = (size_t)phys * num_kv_heads;
    const uint32_t off = (uint32_t)kvh * (uint32_t)sizeof(float);
    ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(k_scales + b), off, 0, 0));
    vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(v_scales + b), off, 0, 0));
}

template <typename KV>
struct Layout {
    static constexpr int kDims = KV::kDims;                  // per lane and token
    static constexpr int kRowLanes = kHeadDim / kDims;       // lanes sharing a token
    static constexpr int kRows = 64 / kRowLanes;             // tokens per load
    static constexpr int kLoads = kTileTokens / kRows;       // loads per lane per tile
};

template <int LANES, int N>
__device__ __forceinline__ void row_sums(float (&x)[N]) {
    if constexpr (LANES == 16) row_sums16(x);
    else row_sums8(x);
}

template <typename KV>
struct Tile {
    typename KV::Word k[Layout<KV>::kLoads];
    typename KV::Word v[Layout<KV>::kLoads];
    float ks, vs;  // the block's scales (kBlockScales)
};

// Loads one tile: `kt` / `vt` address the tile's first row for this KV head
// in the K / V pool, `voff[i]` is this lane's byte offset of load group i
// (tokens kRows i + row, its dims): buffer loads with a scalar base and a
// 32-bit lane offset, so no per-lane 64-bit addresses are kept.
template <typename KV>
__device__ __forceinline__ void load_tile(Tile<KV>& t, const char* kt, const char* vt,
                                          const uint32_t (&voff)[Layout<KV>::kLoads]) {
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kt);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vt);
#pragma unroll
    for (int i = 0; i < Layout<KV>::kLoads; ++i) t.k[i] = KV::load(rk, voff[i]);
#pragma unroll
    for (int i = 0; i < Layout<KV>::kLoads; ++i) t.v[i] = KV::load(rv, voff[i]);
}

template <int G, int ND>
struct State {
    float m[G];        // running max (log2 domain), uniform across the row
    float l[G];        // running sum, uniform across the row
    float acc[G][ND];  // unnormalised output, this lane's dims
    float alpha[G];    // last rescale factor exp2(m_old - m_new) (bf16 pools)
};

// One 16-token tile: QK, online-softmax update, PV.  `ntok_left` is the
// number of valid tokens from the start of this tile (>= 16 for a full one).
// Raw scores are maximised unscaled (the scale is >= 0 after the sign of q
// absorbed a negative one) and scaled inside the exponent's FMA.
template <typename KV, int G, bool PARTIAL>
__device__ __forceinline__ void process_tile(State<G, KV::kDims>& st, const Tile<KV>& t,
                                             const uint32_t (&qv)[G][KV::kDims / 2], float c,
                                             int row, int ntok_left, float vr = 1.0f) {
    constexpr int kLoads = Layout<KV>::kLoads;
    constexpr int kRows = Layout<KV>::kRows;
    constexpr int ND = KV::kDims;
    static_assert(G <= 4, "8 and 16 query heads per KV head run the matrix-core tile");
    // partial dot products of every (token, head), then their row sums
    // together (a step across all of them before the next, so no DPP read
    // waits on the instruction just before it)
    float sf[kLoads * G];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        uint32_t k[ND / 2];
        KV::k_pairs(t.k[i], k);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float d = dot2_bf16(k[0], qv[g][0], 0.0f);
#pragma unroll
            for (int j = 1; j < ND / 2; ++j) d = dot2_bf16(k[j], qv[g][j], d);
            sf[i * G + g] = d;
        }
    }
    row_sums<Layout<KV>::kRowLanes>(sf);
    float s[kLoads][G];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
#pragma unroll
        for (int g = 0; g < G; ++g) s[i][g] = sf[i * G + g];
        if (PARTIAL) {
            // Tokens past the end may hold anything: they must not raise the
            // maximum (lowest finite value, so that a zero scale stays finite)
            // and get p = 0 below.
            const bool valid = (kRows * i + row) < ntok_left;
#pragma unroll
            for (int g = 0; g < G; ++g) s[i][g] = valid ? s[i][g] : -3.402823466e38f;
        }
    }
    float p[kLoads][G];
    if constexpr (KV::kPairedPV) {
        float m_old[G], sum[G];
        bool grew = false;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float bm = kLoads == 4 ? fmaxf(fmaxf(s[0][g], s[1][g]), fmaxf(s[2][g], s[3][g]))
                                   : fmaxf(s[0][g], s[1][g]);
            bm *= c;
            const float mn = fmaxf(st.m[g], bm);
            grew |= mn > st.m[g];
            m_old[g] = st.m[g];
            st.m[g] = mn;
            sum[g] = 0.0f;
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
                p[i][g] = fast_exp2(fmaf(s[i][g], c, -mn));
                if (PARTIAL) p[i][g] = (kRows * i + row) < ntok_left ? p[i][g] : 0.0f;
                sum[g] += p[i][g];
            }
        }
        // The exp(m_old - m_new) rescale of l and the accumulator is needed only
        // when some running maximum moved; after the first tiles that is rare
        // (an unmoved maximum gives exactly 1 either way).
        float alpha[G];
#pragma unroll
        for (int g = 0; g < G; ++g) alpha[g] = 1.0f;
        if (__any(grew)) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                alpha[g] = fast_exp2(m_old[g] - st.m[g]);
#pragma unroll
                for (int d = 0; d < ND; ++d) st.acc[g][d] *= alpha[g];
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) st.l[g] = fmaf(st.l[g], alpha[g], sum[g]);
    } else {
        bool grew = false;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float bm = kLoads == 4 ? fmaxf(fmaxf(s[0][g], s[1][g]), fmaxf(s[2][g], s[3][g]))
                                   : fmaxf(s[0][g], s[1][g]);
            bm *= c;
            const float mn = fmaxf(st.m[g], bm);
            grew |= mn > st.m[g];
            const float alpha = fast_exp2(st.m[g] - mn);
            st.m[g] = mn;
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
                p[i][g] = fast_exp2(fmaf(s[i][g], c, -mn));
                if (PARTIAL) p[i][g] = (kRows * i + row) < ntok_left ? p[i][g] : 0.0f;
                sum += p[i][g];
            }
            st.l[g] = fmaf(st.l[g], alpha, sum);
            st.alpha[g] = alpha;
        }
        // The accumulator needs the exp(m_old - m_new) rescale only when some
        // running maximum moved; after the first tiles that is rare.
        if (__any(grew)) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int d = 0; d < ND; ++d) st.acc[g][d] *= st.alpha[g];
        }
    }
    if constexpr (KV::kPairedPV && !PARTIAL) {
#pragma unroll
        for (int i = 0; i < kLoads; i += 2) {
            f16x2_t pp[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if constexpr (KV::kBlockScales)
                    pp[g] = f16x2_t{(_Float16)(p[i][g] * vr), (_Float16)(p[i + 1][g] * vr)};
                else
                    pp[g] = f16x2_t{(_Float16)p[i][g], (_Float16)p[i + 1][g]};
            }
            // four dims at a time, so few pairs are live at once
#pragma unroll
            for (int j = 0; j < ND / 4; ++j) {
                f16x2_t vp[4];
                KV::v_pairs4(t.v[i], t.v[i + 1], j, vp);
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        st.acc[g][4 * j + e] =
                            __builtin_amdgcn_fdot2(vp[e], pp[g], st.acc[g][4 * j + e], false);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            float v[ND];
            KV::v_floats(t.v[i], v);
            if (PARTIAL) {
                // A masked token has p = 0, but its pool slot may hold anything
                // (NaN included): zero the value so 0 * v stays 0.
                const bool valid = (kRows * i + row) < ntok_left;
#pragma unroll
                for (int d = 0; d < ND; ++d) v[d] = valid ? v[d] : 0.0f;
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float pw = KV::kBlockScales ? p[i][g] * vr : p[i][g];
#pragma unroll
                for (int d = 0; d < ND; ++d) st.acc[g][d] = fmaf(pw, v[d], st.acc[g][d]);
            }
        }
    }
}

template <bool OUT_BF16>
__device__ __forceinline__ void store8(void* out, size_t elem, const float (&x)[8]) {
    if (OUT_BF16) {
        uint4 w;
        w.x = (uint32_t)f32_to_bf16_rne(x[0]) | ((uint32_t)f32_to_bf16_rne(x[1]) << 16);
        w.y = (uint32_t)f32_to_bf16_rne(x[2]) | ((uint32_t)f32_to_bf16_rne(x[3]) << 16);
        w.z = (uint32_t)f32_to_bf16_rne(x[4]) | ((uint32_t)f32_to_bf16_rne(x[5]) << 16);
        w.w = (uint32_t)f32_to_bf16_rne(x[6]) | ((uint32_t)f32_to_bf16_rne(x[7]) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + elem) = w;
    } else {
        float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + elem);
        o[0] = make_float4(x[0], x[1], x[2], x[3]);
        o[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
}

template <bool OUT_BF16>
__device__ __forceinline__ void store1(void* out, size_t elem, float x) {
    if (OUT_BF16) static_cast<uint16_t*>(out)[elem] = f32_to_bf16_rne(x);
    else static_cast<float*>(out)[elem] = x;
}

constexpr int kRecStride = kHeadDim + 4;  // floats per record: acc[128], m, l, 2 pad
constexpr int kMinTilesPerWorker = 4;   // fewer waves for tiny batches
// KV heads (one wave each) served by one workgroup: every tile fits a wave
// in 256 registers, two waves per SIMD.
constexpr int kMaxWavesPerWorker = 8;
constexpr int64_t kMaxWorkers = 1024;    // workgroups of 8 waves an MI355X holds at most
constexpr int64_t kRowsMaxWaves = 2048;  // waves an MI355X holds at two per SIMD
// Cost of a sequence boundary inside a worker's range, in quarter tiles:
// single-row decodes, and the rows path (several query rows per sequence,
// whose boundary also reloads the column blocks' queries and, with shared
// staging, refills the LDS pipeline).  Rows path, in A/Bs against 6:
// 6-row verify 127.1 -> 126.3 us, token trees 169.9 -> 168.7, FP8 verify
// 73.0 -> 70.9 (16 measured between the two).
constexpr int64_t kSeqCost = 6;
constexpr int64_t kSeqCostRows = 32;

__device__ __forceinline__ int clamp_ctx(int ctx, int max_context_len) {
    return ctx < 0 ? 0 : (ctx > max_context_len ? max_context_len : ctx);
}

// With cu_q_lens (a mixed prefill batch) only sequences with exactly one
// query row are decoded here, and their q / out row is cu_q_lens[i]; without
// it every sequence is one row, row i.
__device__ __forceinline__ bool is_decode_row(const int32_t* __restrict__ cu_q_lens, int i) {
    return cu_q_lens == nullptr || cu_q_lens[i + 1] - cu_q_lens[i] == 1;
}
__device__ __forceinline__ int row_of(const int32_t* __restrict__ cu_q_lens, int i) {
    return cu_q_lens == nullptr ? i : cu_q_lens[i];
}
// Query rows of sequence i this path handles: with max_rows == 1 the
// single-row sequences (1), else any sequence of 1 .. max_rows rows (its
// row count); 0 for the rest.
__device__ __forceinline__ int rows_of(const int32_t* __restrict__ cu_q_lens, int i, int max_rows) {
    if (cu_q_lens == nullptr) return 1;
    const int lq = cu_q_lens[i + 1] - cu_q_lens[i];
    if (max_rows == 1) return lq == 1 ? 1 : 0;
    return lq >= 1 && lq <= max_rows ? lq : 0;
}
__device__ __forceinline__ int tiles_of(const int32_t* __restrict__ context_lens,
                                        const int32_t* __restrict__ cu_q_lens, int i,
                                        int max_context_len, int max_rows) {
    if (rows_of(cu_q_lens, i, max_rows) == 0) return 0;
    return (clamp_ctx(context_lens[i], max_context_len) + kTileTokens - 1) / kTileTokens;
}

// Sliding window over a block-table row: lane j of `cur` holds the id of
// block base + j, lane j of `nxt` that of base + 64 + j.  Tiles are visited
// in increasing order, so the window only ever moves forward by 64.
struct IdWindow {
    const int32_t* row;
    int nblk;
    int base;
    int cur;
    int nxt;
    __device__ __forceinline__ void init(const int32_t* r, int n, int first, int lane) {
        row = r;
        nblk = n;
        base = first;
        cur = first + lane < n ? r[first + lane] : 0;
        nxt = first + 64 + lane < n ? r[first + 64 + lane] : 0;
    }
    __device__ __forceinline__ int get(int blk, int lane) {
        if (blk >= base + 64) {
            cur = nxt;
            base += 64;
            // clamped rather than masked: the load lands straight in `nxt`
            // and nothing waits for it until the window moves again
            const int k = base + 64 + lane;
            nxt = row[k < nblk ? k : nblk - 1];
        }
        return __builtin_amdgcn_readlane(cur, blk - base);
    }
};

// Physical block (wave-uniform) holding a tile, and the byte offset of the
// tile's first token row in a pool.
template <int BS>
__device__ __forceinline__ int tile_block(IdWindow& ids, int tile, int lane) {
    return ids.get(tile * kTileTokens / BS, lane);
}
template <int BS>
__device__ __forceinline__ size_t tile_offset(int phys, int tile, size_t row_bytes) {
    return ((size_t)phys * BS + (tile * kTileTokens) % BS) * row_bytes;
}
template <int BS>
__device__ __forceinline__ size_t tile_bytes(IdWindow& ids, int tile, size_t row_bytes, int lane) {
    return tile_offset<BS>(tile_block<BS>(ids, tile, lane), tile, row_bytes);
}

// One decode worker: the workgroup's waves (at most NWAVES, one per KV head
// of head group `group`; waves past the last KV head leave after the scan)
// walk worker w's range of (sequence, 16-token tile) units together, so each
// physical block's K rows of all heads of the group (contiguous) are fetched
// at the same time.  s_cum: (num_seqs + 1) int32 of LDS for the tile prefix
// sums (s_cum[i] = tiles per KV head of sequences < i), s_part: NWAVES int32.
// Records: [W][2][max_rows][num_q_heads][kRecStride] floats.
template <typename KV, int BS, int G, bool OUT_BF16, int NWAVES, int NCB = 1, int CSPLIT = 1>
__device__ __forceinline__ void decode_worker(
    void* __restrict__ out, float* __restrict__ rec, int32_t* __restrict__ seq_workers,
    const uint16_t* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    int max_blocks_per_seq, const int32_t* __restrict__ context_lens, int max_context_len,
    int num_seqs, int num_q_heads, int num_kv_heads, float scale_log2, float out_scale,
    int num_workers, const int32_t* __restrict__ cu_q_lens, int32_t* __restrict__ s_cum,
    int32_t* __restrict__ s_part, int worker, int group, uint16_t* __restrict__ s_vx = nullptr,
    int max_rows = 1, int causal = 1, const uint64_t* __restrict__ tree_mask = nullptr,
    uint4* __restrict__ s_q = nullptr, uint16_t* __restrict__ s_st = nullptr,
    const float* __restrict__ k_scales = nullptr, const float* __restrict__ v_scales = nullptr) {
    static_assert(NCB == 1 || KV::kMfma, "two column blocks need the matrix-core tile");
    static_assert(CSPLIT == 1 || (KV::kMfma && NCB == 1 && KV::kElemBytes == 2),
                  "shared staging: the bf16 matrix-core tile, one block per wave");
    constexpr int D = kHeadDim;
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;  // at most NWAVES waves

    // ---- prefix sums of per-sequence tile counts: each thread sums `per`
    // consecutive sequences, each wave scans its 64 sums with lane
    // shuffles, and one barrier passes the waves' totals around
    const int per = (num_seqs + nthr - 1) / nthr;
    int local = 0;
    for (int k = 0; k < per; ++k) {
        const int i = tid * per + k;
        if (i < num_seqs)
            local += tiles_of(context_lens, cu_q_lens, i, max_context_len, max_rows);
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if ((tid & 63) >= off) incl += y;
    }
    if ((tid & 63) == 63) s_part[tid >> 6] = incl;
    __syncthreads();
    int run = incl - local, total = 0;
    for (int k = 0; k < nthr / 64; ++k) {
        const int t = s_part[k];
        run += k < (tid >> 6) ? t : 0;
        total += t;
    }
    for (int k = 0; k < per; ++k) {
        const int i = tid * per + k;
        if (i < num_seqs) {
            s_cum[i] = run;
            run += tiles_of(context_lens, cu_q_lens, i, max_context_len, max_rows);
        }
    }
    if (tid == 0) s_cum[num_seqs] = total;
    __syncthreads();

    const int64_t U = s_cum[num_seqs];
    // never more workers than tiles, so every worker's range is non-empty
    const int64_t W = num_workers < U ? num_workers : U;
    using L = Layout<KV>;
    constexpr int ND = KV::kDims;
    const int lane = tid & 63;
    // CSPLIT waves per KV head (sub = which of them), each on its own 16
    // columns, sharing the KV head's tiles through LDS
    const int kvh = group * ((nthr >> 6) / CSPLIT) + (tid >> 6) / CSPLIT;
    const int sub = __builtin_amdgcn_readfirstlane((tid >> 6) % CSPLIT);  // wave-uniform
    if (kvh >= num_kv_heads) return;  // a wave with no head: nothing below waits for it
    const int row = lane / L::kRowLanes;
    const int col = lane % L::kRowLanes;
    const int64_t w = worker;
    // Ranges of equal cost, not equal tiles: a tile costs 4 units and every
    // sequence boundary kSeqC more (a worker that starts a new sequence
    // restarts its load pipeline and loads another query and block-id
    // window), so workers that cross more boundaries get fewer tiles.
    // Worker wi starts at the first tile t with cost(t) >= wi * total / W,
    // cost(t) = 4 t + kSeqC * seq(t); the sequence is found among the
    // costs of the sequences' first tiles.
    const int64_t kSeqC = max_rows > 1 ? kSeqCostRows : kSeqCost;
    const int64_t cost_total = 4 * U + kSeqC * (int64_t)(num_seqs - 1);
    auto range_start = [&](int64_t wi) -> int64_t {
        if (wi >= W) return U;
        const int64_t target = wi * cost_total / W;
        int lo = 0, hi = num_seqs;  // largest i with 4 cum[i] + kSeqC i <= target
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (4 * (int64_t)s_cum[mid] + kSeqC * (int64_t)mid <= target) lo = mid; else hi = mid;
        }
        int64_t tt = (target - kSeqC * (int64_t)lo + 3) / 4;
        tt = tt < s_cum[lo] ? s_cum[lo] : tt;
        return tt > s_cum[lo + 1] ? s_cum[lo + 1] : tt;
    };
    int64_t t = w < W ? range_start(w) : 0;
    const int64_t t_end = w < W ? range_start(w + 1) : 0;

    const uint32_t neg = scale_log2 < 0.0f ? 0x80008000u : 0u;
    const float c = fabsf(scale_log2);
    const size_t row_bytes = (size_t)num_kv_heads * D * KV::kElemBytes;
    uint32_t voff[L::kLoads];
#pragma unroll
    for (int i = 0; i < L::kLoads; ++i)
        voff[i] = (uint32_t)((L::kRows * i + row) * row_bytes +
                             ((size_t)kvh * D + col * ND) * KV::kElemBytes);
    const char* kbase = reinterpret_cast<const char*>(k_cache);
    const char* vbase = reinterpret_cast<const char*>(v_cache);
    bool first_piece = true;

    while (t < t_end) {
        // sequence holding tile t: the last i with cum[i] <= t
        int lo = 0, hi = num_seqs;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_cum[mid] <= t) lo = mid; else hi = mid;
        }
        const int seq = lo;
        const int64_t seg_t0 = s_cum[seq];
        const int64_t seg_t1 = s_cum[seq + 1];  // > t
        const int tile0 = (int)(t - seg_t0);
        const int64_t piece_end = t_end < seg_t1 ? t_end : seg_t1;
        const int ntile = (int)(piece_end - t);
        const int ctx = clamp_ctx(context_lens[seq], max_context_len);
        const int row0 = row_of(cu_q_lens, seq);  // the sequence's first q / out row
        const size_t head_row = ((size_t)row0 * num_q_heads + (size_t)kvh * G) * D;
        const bool whole = (t == seg_t0) && (piece_end == seg_t1);
        const int slot = first_piece ? 0 : 1;
        // which workers hold a sequence's first and last tiles (and the
        // record slot of the first), for the merge kernel
        if (tid == 0 && group == 0) {
            if (t == seg_t0) seq_workers[seq] = (int32_t)w | (slot << 30);
            if (piece_end == seg_t1) seq_workers[num_seqs + seq] = (int32_t)w;
        }
        const int n = ntile;
        const bool tail = piece_end == seg_t1 && (ctx % kTileTokens) != 0;
        IdWindow ids;
        ids.init(block_table + (size_t)seq * max_blocks_per_seq, (ctx + BS - 1) / BS,
                 (tile0 * kTileTokens) / BS, lane);

      if constexpr (CSPLIT > 1) {
        typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
        typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        typedef short v4i16_t __attribute__((ext_vector_type(4)));
        const int r16 = lane & 15, q4 = lane >> 4;
        // column cbase + r16: query row (cbase + r16) / G, head
        // kvh G + (cbase + r16) % G
        const int cbase = 16 * sub;
        const int lq = rows_of(cu_q_lens, seq, max_rows);
        const int cpos = ctx - lq;
        const int mask_from = tree_mask != nullptr ? cpos : (causal ? cpos + 1 : ctx);
        const int cr = (cbase + r16) / G;
        bf16x8_t qb[4];
        {
            const size_t qrow =
                ((size_t)(row0 + cr) * num_q_heads + (size_t)kvh * G + (cbase + r16) % G) * D;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                uint4 x = make_uint4(0, 0, 0, 0);
                if (cr < lq) {
                    x = *reinterpret_cast<const uint4*>(q + qrow + 32 * kb + 8 * q4);
                    x.x ^= neg; x.y ^= neg; x.z ^= neg; x.w ^= neg;
                }
                qb[kb] = __builtin_bit_cast(bf16x8_t, x);
            }
        }
        f32x4_t o[8];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) o[nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        float m = kNegBig, l = 0.0f;
        // The KV head's LDS: two buffers of a 32-token tile, K (bf16) then V
        // (fp16), rows of kStRow elements.  A 32-token tile is 16 loads of
        // 16 bytes per lane (8 of K, 8 of V, load i carrying tokens
        // 4 i + lane / 16, bytes 16 (lane % 16) of the head's row); the
        // KV head's waves take 16 / CSPLIT of them each.
        constexpr int kStRow = kHeadDim + 8;
        constexpr int kStTile = 32 * kStRow;
        constexpr int NLD = 16 / CSPLIT;
        uint16_t* const st = s_st + (size_t)((tid >> 6) / CSPLIT) * (4 * kStTile);
        const int n2 = (n + 1) / 2;  // 32-token tiles of the piece
        struct Part { uint4 w[NLD]; };
        auto st_load = [&](Part& x, int jj) {
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int ii = sub * NLD + i;       // 0 .. 7 K, 8 .. 15 V
                const int tok = 4 * (ii & 7) + (lane >> 4);  // 0 .. 31
                // 16-token tile of the piece: tok / 16, which is the same in
                // every lane of load i, so the tile's block id and buffer
                // base stay wave-uniform (no per-lane loop around the load)
                const int j = 2 * jj + ((ii & 7) >> 2);
                const bool valid = j < n && (tile0 + j) * kTileTokens + (tok & 15) < ctx;
                const size_t o0 = tile_bytes<BS>(ids, tile0 + (j < n ? j : n - 1), row_bytes, lane);
                const __amdgpu_buffer_rsrc_t r = buffer_rsrc((ii < 8 ? kbase : vbase) + o0);
                const uint32_t off = valid ? (uint32_t)((tok & 15) * row_bytes +
                                                        (size_t)kvh * D * 2 + 16 * (lane & 15))
                                           : kBufferOob;
                x.w[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
            }
        };
        auto st_store = [&](const Part& x, int jj) {
            uint16_t* const b = st + (jj & 1) * (2 * kStTile);
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int ii = sub * NLD + i;
                const int tok = 4 * (ii & 7) + (lane >> 4);
                uint4 wv = x.w[i];
                if (ii >= 8) {  // V as fp16
                    const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
                    uint32_t hh[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const f16x2_t hp = {(_Float16)bf16_lo(wd[e]), (_Float16)bf16_hi(wd[e])};
                        hh[e] = __builtin_bit_cast(uint32_t, hp);
                    }
                    wv = make_uint4(hh[0], hh[1], hh[2], hh[3]);
                }
                *reinterpret_cast<uint4*>(b + (ii >= 8 ? kStTile : 0) + tok * kStRow + 8 * (lane & 15)) = wv;
            }
        };
        // one 16-token tile (half s of 32-token tile jj) from LDS
        auto st_compute = [&](int jj, int s2) {
            const int j = 2 * jj + s2;
            if (j >= n) return;
            const bool masked = (tile0 + j + 1) * kTileTokens > mask_from;
            const uint16_t* const kt = st + (jj & 1) * (2 * kStTile) + 16 * s2 * kStRow;
            const uint16_t* const vt = kt + kStTile;
            f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kt + r16 * kStRow + 32 * kb + 8 * q4)),
                    qb[kb], sc, 0, 0, 0);
            const int tok0 = (tile0 + j) * kTileTokens + 4 * q4;
            bool vis[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vis[i] = true;
                if (masked) {
                    const int tok = tok0 + i;
                    vis[i] = tok <= (causal ? cpos + cr : ctx - 1);
                    if (tree_mask != nullptr && lq > 1) {
                        const int sh = tok - cpos;  // <= cr < 16 where tok <= the limit
                        const uint64_t bits = cr < lq ? tree_mask[row0 + cr] : 0;
                        vis[i] = vis[i] && (sh < 0 || ((bits >> (sh & 63)) & 1));
                    }
                }
            }
            float sv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[i] = vis[i] ? sc[i] : -3.402823466e38f;
            float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            mt = max_lane_quads(mt) * c;
            const float mn = fmaxf(m, mt);
            const bool grew = mn > m;
            const float alpha = fast_exp2(m - mn);
            m = mn;
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = vis[i] ? fast_exp2(fmaf(sv[i], c, -mn)) : 0.0f;
            l = fmaf(l, alpha, (p[0] + p[1]) + (p[2] + p[3]));
            if (__any(grew)) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __shfl(alpha, 4 * q4 + i);
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb) o[nb][i] *= ai;
                }
            }
            const f16x4_t pa = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
            const uint16_t* const vrow = vt + (4 * q4 + (r16 >> 2)) * kStRow + 4 * (r16 & 3);
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const f16x4_t vb = __builtin_bit_cast(f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16_t*)(vrow + 16 * nb)));
                o[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vb, o[nb], 0, 0, 0);
            }
        };
        // two register sets, roles alternating over pairs of 32-token tiles:
        // tile jj + 1 is in flight in one while jj is computed, and is stored
        // to LDS at the end of jj, behind the workgroup's barrier
        Part ra, rb;
        st_load(ra, 0);
        if (n2 > 1) st_load(rb, 1);
        st_store(ra, 0);
        __syncthreads();
        for (int jj = 0; jj < n2; jj += 2) {
            if (jj + 2 < n2) st_load(ra, jj + 2);
            st_compute(jj, 0);
            st_compute(jj, 1);
            if (jj + 1 < n2) st_store(rb, jj + 1);
            __syncthreads();
            if (jj + 1 >= n2) break;
            if (jj + 3 < n2) st_load(rb, jj + 3);
            st_compute(jj + 1, 0);
            st_compute(jj + 1, 1);
            if (jj + 2 < n2) st_store(ra, jj + 2);
            __syncthreads();
        }
        const float lt = sum_lane_quads(l);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = cbase + 4 * q4 + i;
            const float mh = __shfl(m, 4 * q4 + i);
            const float lh = __shfl(lt, 4 * q4 + i);
            const int r = cc / G;
            if (r >= lq) continue;
            const size_t qh = (size_t)kvh * G + cc % G;
            if (whole) {
                const float inv = out_scale / lh;
                const size_t e = ((size_t)(row0 + r) * num_q_heads + qh) * D;
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) store1<OUT_BF16>(out, e + 16 * nb + r16, o[nb][i] * inv);
            } else {
                float* rr = rec + (((size_t)(w * 2 + slot) * max_rows + r) * num_q_heads + qh) * kRecStride;
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) rr[16 * nb + r16] = o[nb][i];
                if (r16 == 0) {
                    rr[D] = mh;
                    rr[D + 1] = lh;
                }
            }
        }
      } else if constexpr (KV::kMfma) {
        typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
        typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        typedef short v4i16_t __attribute__((ext_vector_type(4)));
        const int r16 = lane & 15, q4 = lane >> 4;
        // The columns of the S = K Q^T product: column cc = 16 cb + r16 of
        // block cb is query row cc / G of the sequence, head kvh G + cc % G;
        // with one row per sequence (decode) simply head r16.
        const int lq = rows_of(cu_q_lens, seq, max_rows);
        // keys a row may see: causal rows up to their own position
        // ctx - lq + r; the rows of a token tree of those only the keys
        // before the chunk and the chunk keys their mask selects (a
        // single-row sequence sees all its keys, as on the decode path);
        // else all ctx keys
        const int cpos = ctx - lq;
        const int mask_from = tree_mask != nullptr ? cpos : (causal ? cpos + 1 : ctx);
        // Q^T operands (rows = the 8 dims of k-block kb): in registers for
        // one block, in the wave's LDS for two (the registers hold the
        // second block's O instead)
        bf16x8_t qreg[NCB == 1 ? 4 : 1];
        uint4* const sq = s_q + (size_t)(tid >> 6) * (NCB * 4 * 64);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int cc = 16 * cb + r16;
            const int r = cc / G;
            const size_t qrow = ((size_t)(row0 + r) * num_q_heads + (size_t)kvh * G + cc % G) * D;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                uint4 x = make_uint4(0, 0, 0, 0);
                if (r < lq) {
                    x = *reinterpret_cast<const uint4*>(q + qrow + KV::mfma_dim(kb, q4));
                    x.x ^= neg; x.y ^= neg; x.z ^= neg; x.w ^= neg;
                }
                if constexpr (NCB == 1) qreg[kb] = __builtin_bit_cast(bf16x8_t, x);
                else sq[(cb * 4 + kb) * 64 + lane] = x;
            }
        }
        auto qop = [&](int cb, int kb) -> bf16x8_t {
            if constexpr (NCB == 1) {
                return qreg[kb];
            } else {
                // read per use: an offset the compiler cannot see through
                // keeps it from hoisting the loop-invariant reads back into
                // registers
                int idx = (cb * 4 + kb) * 64 + lane;
                asm volatile("" : "+v"(idx));
                return __builtin_bit_cast(bf16x8_t, sq[idx]);
            }
        };
        f32x4_t o[NCB][8];
        float m[NCB], l[NCB];  // column r16's running max (the same in its 4 lanes) and sum
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) o[cb][nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            m[cb] = kNegBig;
            l[cb] = 0.0f;
        }
        // byte offsets of token r16's loads in a tile
        constexpr int NL = KV::kMfmaLoads;
        uint32_t koff[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j)
            koff[j] = (uint32_t)(r16 * row_bytes + (size_t)kvh * D * KV::kElemBytes + KV::mfma_byte(j, q4));
        uint16_t* const vx = s_vx + (tid >> 6) * kVxWaveElems;  // this wave's V tile
        struct MTile { typename KV::Word k[NL]; typename KV::Word v[NL]; float ks, vs; };
        float vref = 0.0f;  // the piece's V reference scale (kBlockScales)
        // tiles that reach the keys some row may not see take the mask
        auto masked_of = [&](int j) { return (tile0 + j + 1) * kTileTokens > mask_from; };
        auto fetch = [&](MTile& x, int j) {
            const int phys = tile_block<BS>(ids, tile0 + j, lane);
            if constexpr (KV::kBlockScales)
                load_block_scales(k_scales, v_scales, phys, num_kv_heads, kvh, x.ks, x.vs);
            const size_t o0 = tile_offset<BS>(phys, tile0 + j, row_bytes);
            const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kbase + o0);
            const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vbase + o0);
            // tokens past the end read zeros
            const bool valid = (tile0 + j) * kTileTokens + r16 < ctx;
#pragma unroll
            for (int jj = 0; jj < NL; ++jj) {
                const uint32_t off = valid ? koff[jj] : kBufferOob;
                x.k[jj] = KV::load(rk, off);
                x.v[jj] = KV::load(rv, off);
            }
        };
        auto process = [&](const MTile& x, int j, bool masked) {
            // V as fp16 into the wave's LDS tile, token r16, k-block kb's dims
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                *reinterpret_cast<uint4*>(vx + r16 * kVxStride + KV::mfma_dim(kb, q4)) = KV::v_f16x8(x.v, kb);
            const int tok0 = (tile0 + j) * kTileTokens + 4 * q4;  // this lane's first token
            float ct = c, vr = 1.0f;  // this tile's score scale and V ratio
            if constexpr (KV::kBlockScales) {
                ct = c * x.ks;
                if (x.vs > vref) {
                    const float f = vref / x.vs;
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                        for (int nb = 0; nb < 8; ++nb) o[cb][nb] *= f;
                    vref = x.vs;
                }
                vr = x.vs / vref;
            }
            f16x4_t pa[NCB];
            float alpha[NCB];
            bool grew = false;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                // S = K Q^T: lane holds tokens 4 q4 .. + 3 of column 16 cb + r16
                f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, KV::k_bf16x8(x.k, kb)), qop(cb, kb), sc, 0, 0, 0);
                bool vis[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vis[i] = true;
                    if (masked) {
                        // the column's limits, taken again here: masked tiles are rare
                        const int r = (16 * cb + r16) / G;
                        const int tok = tok0 + i;
                        vis[i] = tok <= (causal ? cpos + r : ctx - 1);
                        if (tree_mask != nullptr && lq > 1) {
                            const int sh = tok - cpos;  // <= r < 16 where tok <= the limit
                            const uint64_t bits = r < lq ? tree_mask[row0 + r] : 0;
                            vis[i] = vis[i] && (sh < 0 || ((bits >> (sh & 63)) & 1));
                        }
                    }
                }
                float sv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[i] = vis[i] ? sc[i] : -3.402823466e38f;
                float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
                mt = max_lane_quads(mt) * ct;
                const float mn = fmaxf(m[cb], mt);
                grew |= mn > m[cb];
                alpha[cb] = fast_exp2(m[cb] - mn);
                m[cb] = mn;
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) p[i] = vis[i] ? fast_exp2(fmaf(sv[i], ct, -mn)) : 0.0f;
                l[cb] = fmaf(l[cb], alpha[cb], (p[0] + p[1]) + (p[2] + p[3]));
                if constexpr (KV::kBlockScales)
                    pa[cb] = f16x4_t{(_Float16)(p[0] * vr), (_Float16)(p[1] * vr),
                                     (_Float16)(p[2] * vr), (_Float16)(p[3] * vr)};
                else
                    pa[cb] = f16x4_t{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
            }
            if (__any(grew)) {
                // O row 4 q4 + i is column 4 q4 + i, whose alpha lane 4 q4 + i holds
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float ai = __shfl(alpha[cb], 4 * q4 + i);
#pragma unroll
                        for (int nb = 0; nb < 8; ++nb) o[cb][nb][i] *= ai;
                    }
            }
            // V operand: tokens 4 q4 .. + 3 of dim 16 nb + r16, by one
            // transposing read (ds_read_b64_tr_b16: within each 16 lanes,
            // lane i gets element i % 4 of the 8-byte chunks that lanes
            // 4 k + i / 4 address, k = 0 .. 3; so lane (r16, q4) addresses
            // token 4 q4 + r16 / 4, dims 16 nb + 4 (r16 % 4) .. + 3).  The
            // wave's own stores above are done: its LDS operations run in
            // order.
            const uint16_t* const vrow = vx + (4 * q4 + (r16 >> 2)) * kVxStride + 4 * (r16 & 3);
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const f16x4_t vb = __builtin_bit_cast(f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16_t*)(vrow + 16 * nb)));
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    o[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa[cb], vb, o[cb][nb], 0, 0, 0);
            }
        };
        // Only a sequence's last two tiles can need the mask (rows <= 16).
        MTile a, b;
        fetch(a, 0);
        if (n == 1) {
            process(a, 0, masked_of(0));
        } else {
            fetch(b, 1);
            int j = 0;
            for (; j + 3 < n; j += 2) {  // tiles j, j + 1 are neither of the last two
                process(a, j, false);
                fetch(a, j + 2);
                process(b, j + 1, false);
                fetch(b, j + 3);
                if (NWAVES == 8) __syncthreads();
            }
            process(a, j, masked_of(j));
            if (n - j == 3) {
                fetch(a, j + 2);
                process(b, j + 1, masked_of(j + 1));
                process(a, j + 2, masked_of(j + 2));
            } else {
                process(b, j + 1, masked_of(j + 1));
            }
        }
        // ---- the piece's result: l over the column's 4 lanes; a lane's O
        // rows are columns 4 q4 .. + 3 of each block, whose (m, l) lanes
        // 4 q4 .. + 3 hold
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const float lt = sum_lane_quads(l[cb]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int cc = 16 * cb + 4 * q4 + i;
                const float mh = __shfl(m[cb], 4 * q4 + i);
                const float lh = __shfl(lt, 4 * q4 + i);
                const int r = cc / G;
                if (r >= lq) continue;
                const size_t qh = (size_t)kvh * G + cc % G;
                // O in absolute units: times the V reference scale
                const float ou = KV::kBlockScales ? out_scale * vref : out_scale;
                const float vu = KV::kBlockScales ? vref : 1.0f;
                if (whole) {
                    const float inv = ou / lh;
                    const size_t e = ((size_t)(row0 + r) * num_q_heads + qh) * D;
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb)
                        store1<OUT_BF16>(out, e + 16 * nb + r16, o[cb][nb][i] * inv);
                } else {
                    float* rr = rec + (((size_t)(w * 2 + slot) * max_rows + r) * num_q_heads + qh) * kRecStride;
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb)
                        rr[16 * nb + r16] = KV::kBlockScales ? o[cb][nb][i] * vu : o[cb][nb][i];
                    if (r16 == 0) {
                        rr[D] = mh;
                        rr[D + 1] = lh;
                    }
                }
            }
        }
      } else {
        uint32_t qv[G][ND / 2];  // this lane's dims of each query head, bf16 pairs
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int w8 = 0; w8 < ND / 8; ++w8) {
                const uint4 x = *reinterpret_cast<const uint4*>(q + head_row + (size_t)g * D +
                                                                col * ND + 8 * w8);
                qv[g][4 * w8] = x.x ^ neg; qv[g][4 * w8 + 1] = x.y ^ neg;
                qv[g][4 * w8 + 2] = x.z ^ neg; qv[g][4 * w8 + 3] = x.w ^ neg;
            }
        State<G, ND> st;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            st.m[g] = kNegBig;
            st.l[g] = 0.0f;
#pragma unroll
            for (int d = 0; d < ND; ++d) st.acc[g][d] = 0.0f;
        }

        // Two-deep load pipeline over the piece's tiles 0 .. n-1 (buffers a
        // and b alternate).  The steady-state loop issues both of its loads
        // unconditionally, so while one buffer is processed the other's
        // eight loads stay in flight (a load issued on some paths only would
        // force the wait counters to drain it).  Only the sequence's last
        // tile can be partial, and it is never inside the loop.
        auto fetch = [&](Tile<KV>& x, int j) {
            const int phys = tile_block<BS>(ids, tile0 + j, lane);
            if constexpr (KV::kBlockScales)
                load_block_scales(k_scales, v_scales, phys, num_kv_heads, kvh, x.ks, x.vs);
            const size_t o = tile_offset<BS>(phys, tile0 + j, row_bytes);
            load_tile(x, kbase + o, vbase + o, voff);
        };
        // a tile's score scale and V ratio; with per-(block, head) scales the
        // V reference moves first (the same in every lane: one block and
        // one KV head per tile and wave)
        float vref = 0.0f;
        auto scales_of = [&](const Tile<KV>& x, float& ct, float& vr) {
            ct = c;
            vr = 1.0f;
            if constexpr (KV::kBlockScales) {
                ct = c * x.ks;
                if (x.vs > vref) {
                    const float f = vref / x.vs;
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int d = 0; d < ND; ++d) st.acc[g][d] *= f;
                    vref = x.vs;
                }
                vr = x.vs / vref;
            }
        };
        auto full = [&](const Tile<KV>& x) {
            float ct, vr;
            scales_of(x, ct, vr);
            process_tile<KV, G, false>(st, x, qv, ct, row, kTileTokens, vr);
        };
        auto finish = [&](const Tile<KV>& x, int j) {
            float ct, vr;
            scales_of(x, ct, vr);
            if (tail && j == n - 1)
                process_tile<KV, G, true>(st, x, qv, ct, row, ctx - (tile0 + j) * kTileTokens, vr);
            else
                process_tile<KV, G, false>(st, x, qv, ct, row, kTileTokens, vr);
        };
        Tile<KV> a, b;
        fetch(a, 0);
        if (n == 1) {
            finish(a, 0);
        } else {
            fetch(b, 1);
            int j = 0;
            for (; j + 3 < n; j += 2) {  // tiles j + 2 and j + 3 exist and are full
                full(a);
                fetch(a, j + 2);
                full(b);
                fetch(b, j + 3);
                // Eight waves stream their heads with nothing else tying them
                // together, and two share each SIMD: left alone they drift
                // tens of microseconds apart and the last ones finish alone,
                // at half the loads in flight.  A barrier per tile pair keeps
                // them in step (it waits for no load).  Four waves per
                // workgroup, whose math is the tighter limit, do better
                // without it.
                if (NWAVES == 8) __syncthreads();
            }
            // two or three tiles left: j (in a), j + 1 (in b), maybe j + 2
            full(a);
            if (n - j == 3) {
                fetch(a, j + 2);
                full(b);
                finish(a, j + 2);
            } else {
                finish(b, j + 1);
            }
        }

        // Merge the row streams: M = max m_r, l = sum l_r 2^(m_r - M),
        // acc = sum acc_r 2^(m_r - M).  A row that saw no token has
        // m = kNegBig, l = 0, acc = 0 and drops out.
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float mx = st.m[g];
#pragma unroll
            for (int o = L::kRowLanes; o < 64; o <<= 1) mx = fmaxf(mx, xor_lane(mx, o));
            const float f = fast_exp2(st.m[g] - mx);
            float lt = st.l[g] * f;
#pragma unroll
            for (int o = L::kRowLanes; o < 64; o <<= 1) lt += xor_lane(lt, o);
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                float x = st.acc[g][d] * f;
#pragma unroll
                for (int o = L::kRowLanes; o < 64; o <<= 1) x += xor_lane(x, o);
                st.acc[g][d] = x;
            }
            st.m[g] = mx;
            st.l[g] = lt;
        }

        // Row r stores heads g = r, r + kRows, ...
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g % L::kRows != row) continue;
            if (whole) {
                // with per-(block, head) scales the accumulator is in units of vref
                const float inv = (KV::kBlockScales ? out_scale * vref : out_scale) / st.l[g];
#pragma unroll
                for (int w8 = 0; w8 < ND / 8; ++w8) {
                    float o[8];
#pragma unroll
                    for (int d = 0; d < 8; ++d) o[d] = st.acc[g][8 * w8 + d] * inv;
                    store8<OUT_BF16>(out, head_row + (size_t)g * D + col * ND + 8 * w8, o);
                }
            } else {
                float* r = rec + ((size_t)(w * 2 + slot) * num_q_heads + (size_t)kvh * G + g) * kRecStride;
                float4* pa = reinterpret_cast<float4*>(r + col * ND);
                const float vu = KV::kBlockScales ? vref : 1.0f;
#pragma unroll
                for (int w4 = 0; w4 < ND / 4; ++w4) {
                    if constexpr (KV::kBlockScales)
                        pa[w4] = make_float4(st.acc[g][4 * w4] * vu, st.acc[g][4 * w4 + 1] * vu,
                                             st.acc[g][4 * w4 + 2] * vu, st.acc[g][4 * w4 + 3] * vu);
                    else
                        pa[w4] = make_float4(st.acc[g][4 * w4], st.acc[g][4 * w4 + 1],
                                             st.acc[g][4 * w4 + 2], st.acc[g][4 * w4 + 3]);
                }
                if (col == 0) {
                    r[D] = st.m[g];
                    r[D + 1] = st.l[g];
                }
            }
        }
      }
        first_piece = false;
        t = piece_end;
    }
}

}  // namespace dec
}  // namespace pkv
