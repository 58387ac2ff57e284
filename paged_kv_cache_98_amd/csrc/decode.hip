// decode.hip -- paged decode attention for gfx950: split-KV partitions with
// a single-pass online softmax, then a log-sum-exp merge.
//
// What it computes ("LLM 推理优化技术全景", "Flash Attention 深度剖析"): for
// every sequence i and query head h,
//     out[i,h,:] = sum_t exp(s_t - m) V[t,:] / sum_t exp(s_t - m),
//     s_t = scale * <q[i,h,:], K[t,:]>,
// over the sequence's context_lens[i] keys, which live in 16- or 32-token
// physical blocks found through the block table ("LLM 推理引擎深度解析 ...",
// section 2.1; "让 Agent 跑得快", section 五).  The keys are visited once, a
// tile at a time, keeping a running maximum m and running sum l and
// rescaling the accumulator by exp(m_old - m_new) whenever m grows (the
// page's "在线 Softmax"); the division by l is deferred to the very end as in
// its "Flash Attention v2 的改进".  Long contexts are cut into 512-token
// partitions processed in parallel (the sequence-axis parallelism of the
// same section); each partition leaves (m, l, unnormalised acc) and a merge
// kernel combines them with the same exp(m_k - M) rescale.
//
// Work decomposition (one wavefront = 64 lanes = 4 rows of 16 lanes):
//   * one wave per (sequence, KV head, partition); a workgroup holds the
//     waves of 1, 2 or 4 consecutive KV heads of the same (sequence,
//     partition), so the workgroup reads whole 2 KB token rows of the pool;
//   * the G = Hq/Hkv query heads of the KV head are handled by the same wave,
//     so each K/V byte is read from HBM once per KV head (GQA grouping);
//   * a 16-token tile of one head is 4 KB of K and 4 KB of V: every lane
//     moves 4 x 16 B of each.  Lane (row r, col c) holds dims 8c..8c+7 of
//     tokens 4i + r, i = 0..3; its 16-lane row reduces the QK partial sums
//     with DPP adds;
//   * each 16-lane row is its own online-softmax stream (tokens = r mod 4)
//     with its own m, l, acc; the four rows are merged at the end of the
//     partition, so no cross-row traffic happens inside the loop;
//   * the next tile's K/V loads are issued before the current tile's math.
// Scores are kept in the log2 domain: s * scale * log2(e), exponentials are
// v_exp_f32 (2^x).
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

constexpr int kLoads = kTileTokens / 4;  // 128-bit loads per lane per tile (K or V)

struct Tile {
    uint4 k[kLoads];
    uint4 v[kLoads];
};

// Element offset of physical tile `tile` (16 tokens) of the partition.
template <int BS>
__device__ __forceinline__ size_t tile_base(int ids_reg, int tile, size_t row_elems) {
    const int phys = __builtin_amdgcn_readlane(ids_reg, (tile * kTileTokens) / BS);
    const int row0 = (tile * kTileTokens) % BS;
    return ((size_t)phys * BS + row0) * row_elems;
}

__device__ __forceinline__ void load_tile(Tile& t, const uint16_t* __restrict__ kc,
                                          const uint16_t* __restrict__ vc, size_t base,
                                          uint32_t lane_off, uint32_t four_rows) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        t.k[i] = *reinterpret_cast<const uint4*>(kc + base + lane_off + i * four_rows);
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        t.v[i] = *reinterpret_cast<const uint4*>(vc + base + lane_off + i * four_rows);
    }
}

template <int G>
struct State {
    float m[G];       // running max (log2 domain), uniform across the row
    float l[G];       // running sum, uniform across the row
    float acc[G][8];  // unnormalised output, dims 8c..8c+7 of this lane
};

// One 16-token tile: QK, online-softmax update, PV.  `ntok_left` is the
// number of valid tokens from the start of this tile (>= 16 for a full one).
template <int G, bool PARTIAL>
__device__ __forceinline__ void process_tile(State<G>& st, const Tile& t, const uint4 (&qv)[G],
                                             float scale_log2, int row, int ntok_left) {
    float s[kLoads][G];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float d = dot2_bf16(t.k[i].x, qv[g].x, 0.0f);
            d = dot2_bf16(t.k[i].y, qv[g].y, d);
            d = dot2_bf16(t.k[i].z, qv[g].z, d);
            d = dot2_bf16(t.k[i].w, qv[g].w, d);
            d = row_sum16(d);
            s[i][g] = d * scale_log2;
        }
        if (PARTIAL) {
            const bool valid = (4 * i + row) < ntok_left;
#pragma unroll
            for (int g = 0; g < G; ++g) s[i][g] = valid ? s[i][g] : -INFINITY;
        }
    }
    float p[kLoads][G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float bm = fmaxf(fmaxf(s[0][g], s[1][g]), fmaxf(s[2][g], s[3][g]));
        const float mn = fmaxf(st.m[g], bm);
        const float alpha = fast_exp2(st.m[g] - mn);
        st.m[g] = mn;
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            p[i][g] = fast_exp2(s[i][g] - mn);
            sum += p[i][g];
        }
        st.l[g] = st.l[g] * alpha + sum;
#pragma unroll
        for (int d = 0; d < 8; ++d) st.acc[g][d] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        float v[8];
        v[0] = bf16_lo(t.v[i].x); v[1] = bf16_hi(t.v[i].x);
        v[2] = bf16_lo(t.v[i].y); v[3] = bf16_hi(t.v[i].y);
        v[4] = bf16_lo(t.v[i].z); v[5] = bf16_hi(t.v[i].z);
        v[6] = bf16_lo(t.v[i].w); v[7] = bf16_hi(t.v[i].w);
        if (PARTIAL) {
            // A masked token has p = 0, but its pool slot may hold anything
            // (NaN included): zero the value so 0 * v stays 0.
            const bool valid = (4 * i + row) < ntok_left;
#pragma unroll
            for (int d = 0; d < 8; ++d) v[d] = valid ? v[d] : 0.0f;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int d = 0; d < 8; ++d) st.acc[g][d] = fmaf(p[i][g], v[d], st.acc[g][d]);
        }
    }
}

template <int G>
__device__ __forceinline__ void process_any(State<G>& st, const Tile& t, const uint4 (&qv)[G],
                                            float scale_log2, int row, int ntok_left) {
    if (ntok_left >= kTileTokens)
        process_tile<G, false>(st, t, qv, scale_log2, row, ntok_left);
    else
        process_tile<G, true>(st, t, qv, scale_log2, row, ntok_left);
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

// Grid: (max_partitions, num_kv_heads / waves_per_group, num_seqs); block:
// 64 * waves_per_group threads.
template <int BS, int G, bool OUT_BF16>
__global__ void __launch_bounds__(256)
decode_partition_kernel(void* __restrict__ out, float2* __restrict__ part_ml,
                        float* __restrict__ part_acc, const uint16_t* __restrict__ q,
                        const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
                        const int32_t* __restrict__ block_table, int max_blocks_per_seq,
                        const int32_t* __restrict__ context_lens, int max_context_len,
                        int num_q_heads, int num_kv_heads, float scale_log2, int max_parts) {
    constexpr int D = kHeadDim;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int waves = blockDim.x >> 6;
    const int part = blockIdx.x;
    const int kvh = blockIdx.y * waves + wave;
    const int seq = blockIdx.z;
    const int row = lane >> 4;
    const int col = lane & 15;

    int ctx = context_lens[seq];
    ctx = ctx < 0 ? 0 : (ctx > max_context_len ? max_context_len : ctx);
    const int nparts = (ctx + kPartitionTokens - 1) / kPartitionTokens;
    const size_t head_row = ((size_t)seq * num_q_heads + (size_t)kvh * G) * D;

    if (ctx == 0) {
        if (part == 0) {  // nothing to attend to: a defined all-zero row
            for (int e = lane; e < G * D; e += 64) {
                if (OUT_BF16) static_cast<uint16_t*>(out)[head_row + e] = 0;
                else static_cast<float*>(out)[head_row + e] = 0.0f;
            }
        }
        return;
    }
    if (part >= nparts) return;

    const int tok0 = part * kPartitionTokens;
    const int ntok = min(kPartitionTokens, ctx - tok0);
    const int ntiles = (ntok + kTileTokens - 1) / kTileTokens;
    const int nblk = (ntok + BS - 1) / BS;

    // Physical ids of this partition's blocks: lane j holds the j-th.
    const int32_t* bt_row = block_table + (size_t)seq * max_blocks_per_seq + tok0 / BS;
    const int ids = lane < nblk ? bt_row[lane] : 0;

    uint4 qv[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        qv[g] = *reinterpret_cast<const uint4*>(q + head_row + (size_t)g * D + col * 8);

    State<G> st;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        st.m[g] = kNegBig;
        st.l[g] = 0.0f;
#pragma unroll
        for (int d = 0; d < 8; ++d) st.acc[g][d] = 0.0f;
    }

    const size_t row_elems = (size_t)num_kv_heads * D;  // elements between token rows
    const uint32_t lane_off = (uint32_t)(row * row_elems + (size_t)kvh * D + col * 8);
    const uint32_t four_rows = (uint32_t)(4 * row_elems);

    Tile a, b;
    load_tile(a, k_cache, v_cache, tile_base<BS>(ids, 0, row_elems), lane_off, four_rows);
    for (int j = 0; j < ntiles; j += 2) {
        if (j + 1 < ntiles)
            load_tile(b, k_cache, v_cache, tile_base<BS>(ids, j + 1, row_elems), lane_off, four_rows);
        process_any<G>(st, a, qv, scale_log2, row, ntok - j * kTileTokens);
        if (j + 1 >= ntiles) break;
        if (j + 2 < ntiles)
            load_tile(a, k_cache, v_cache, tile_base<BS>(ids, j + 2, row_elems), lane_off, four_rows);
        process_any<G>(st, b, qv, scale_log2, row, ntok - (j + 1) * kTileTokens);
    }

    // Merge the four row streams: M = max m_r, l = sum l_r 2^(m_r - M),
    // acc = sum acc_r 2^(m_r - M).  Row 0 always saw a valid token.
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float mx = fmaxf(st.m[g], xor_lane(st.m[g], 16));
        mx = fmaxf(mx, xor_lane(mx, 32));
        const float f = fast_exp2(st.m[g] - mx);
        float lt = st.l[g] * f;
        lt += xor_lane(lt, 16);
        lt += xor_lane(lt, 32);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            float x = st.acc[g][d] * f;
            x += xor_lane(x, 16);
            x += xor_lane(x, 32);
            st.acc[g][d] = x;
        }
        st.m[g] = mx;
        st.l[g] = lt;
    }

    // Row r stores heads g = r, r + 4, ...
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if ((g & 3) != row) continue;
        if (nparts == 1) {
            const float inv = 1.0f / st.l[g];
            float o[8];
#pragma unroll
            for (int d = 0; d < 8; ++d) o[d] = st.acc[g][d] * inv;
            store8<OUT_BF16>(out, head_row + (size_t)g * D + col * 8, o);
        } else {
            const size_t slot = ((size_t)seq * num_q_heads + (size_t)kvh * G + g) * max_parts + part;
            float4* pa = reinterpret_cast<float4*>(part_acc + slot * D + col * 8);
            pa[0] = make_float4(st.acc[g][0], st.acc[g][1], st.acc[g][2], st.acc[g][3]);
            pa[1] = make_float4(st.acc[g][4], st.acc[g][5], st.acc[g][6], st.acc[g][7]);
            if (col == 0) part_ml[slot] = make_float2(st.m[g], st.l[g]);
        }
    }
}

// Log-sum-exp merge of the partitions of one (sequence, query head) per
// wave: M = max_k m_k, L = sum_k l_k 2^(m_k - M), out = sum_k acc_k 2^(m_k - M) / L.
// Grid: (ceil(num_q_heads / 4), num_seqs); block: 256 (4 waves, one head each).
template <bool OUT_BF16>
__global__ void __launch_bounds__(256)
decode_merge_kernel(void* __restrict__ out, const float2* __restrict__ part_ml,
                    const float* __restrict__ part_acc, const int32_t* __restrict__ context_lens,
                    int max_context_len, int num_q_heads, int max_parts) {
    constexpr int D = kHeadDim;
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int seq = blockIdx.y;
    if (h >= num_q_heads) return;
    int ctx = context_lens[seq];
    ctx = ctx < 0 ? 0 : (ctx > max_context_len ? max_context_len : ctx);
    const int nparts = (ctx + kPartitionTokens - 1) / kPartitionTokens;
    if (nparts <= 1) return;  // written directly by the partition kernel

    const size_t slot0 = ((size_t)seq * num_q_heads + h) * max_parts;
    float mx = -INFINITY;
    for (int p = lane; p < nparts; p += 64) mx = fmaxf(mx, part_ml[slot0 + p].x);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));

    float L = 0.0f, a0 = 0.0f, a1 = 0.0f;
    const float2* acc2 = reinterpret_cast<const float2*>(part_acc);
    for (int p = 0; p < nparts; ++p) {
        const float2 ml = part_ml[slot0 + p];
        const float w = fast_exp2(ml.x - mx);
        L = fmaf(ml.y, w, L);
        const float2 a = acc2[(slot0 + p) * (D / 2) + lane];
        a0 = fmaf(a.x, w, a0);
        a1 = fmaf(a.y, w, a1);
    }
    const float inv = 1.0f / L;
    const size_t e = ((size_t)seq * num_q_heads + h) * D + 2 * lane;
    if (OUT_BF16) {
        const uint32_t w = (uint32_t)f32_to_bf16_rne(a0 * inv) |
                           ((uint32_t)f32_to_bf16_rne(a1 * inv) << 16);
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + e) = w;
    } else {
        *reinterpret_cast<float2*>(static_cast<float*>(out) + e) = make_float2(a0 * inv, a1 * inv);
    }
}

template <int BS, int G, bool OUT_BF16>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    const int waves = (a.num_kv_heads % 4 == 0) ? 4 : (a.num_kv_heads % 2 == 0 ? 2 : 1);
    dim3 grid(a.max_parts, a.num_kv_heads / waves, a.num_seqs);
    dim3 block(64 * waves);
    hipLaunchKernelGGL((decode_partition_kernel<BS, G, OUT_BF16>), grid, block, 0, stream, a.out,
                       a.part_ml, a.part_acc, a.q, a.k_cache, a.v_cache, a.block_table,
                       a.max_blocks_per_seq, a.context_lens, a.max_context_len, a.num_q_heads,
                       a.num_kv_heads, a.scale_log2, a.max_parts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_parts <= 1) return e;
    dim3 mgrid((a.num_q_heads + 3) / 4, a.num_seqs);
    hipLaunchKernelGGL((decode_merge_kernel<OUT_BF16>), mgrid, dim3(256), 0, stream, a.out,
                       a.part_ml, a.part_acc, a.context_lens, a.max_context_len, a.num_q_heads,
                       a.max_parts);
    return hipGetLastError();
}

template <int BS, int G>
hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s) {
    return a.out_bf16 ? launch_decode_t<BS, G, true>(a, s) : launch_decode_t<BS, G, false>(a, s);
}

template <int BS>
hipError_t launch_decode_bs(const DecodeArgs& a, hipStream_t s) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_decode_g<BS, 1>(a, s);
        case 2: return launch_decode_g<BS, 2>(a, s);
        case 4: return launch_decode_g<BS, 4>(a, s);
        case 8: return launch_decode_g<BS, 8>(a, s);
        case 16: return launch_decode_g<BS, 16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    return a.block_size == 16 ? launch_decode_bs<16>(a, stream) : launch_decode_bs<32>(a, stream);
}

}  // namespace pkv
