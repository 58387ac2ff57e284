// decode.hip -- paged decode attention for gfx950: the stream-K decode
// kernel (the worker of decode_core.h over a grid of persistent workgroups),
// the log-sum-exp merge of sequences shared by several workers, and the
// launchers.
#include "decode_core.h"

namespace pkv {

namespace {

using namespace dec;

// Grid: (num_workers, head groups); a workgroup has one wave per KV head of
// its group (all KV heads when there are at most 8, else groups of 8);
// dynamic LDS (num_seqs + 1) int32 for the tile prefix sums.  With
// max_rows > 1 (short chunks, as in speculative-decoding verification) every
// sequence of up to max_rows rows, causal or under per-row tree masks, its
// (row, head) pairs the columns of the matrix-core tile: NCB blocks of 16
// per KV head (the Q operands of two blocks in LDS).
// Shared staging: workgroups of 8 waves (four KV heads of two waves) for
// CSPLIT = 2, of 4 waves (one KV head of four) for CSPLIT = 4.  In A/Bs
// against 4 waves for both: long-context verify 429.4 -> 406.7 us, the
// 6-row verify unchanged (126.7 / 126.3); token trees (CSPLIT = 4) went
// 169.0 -> 178.7 with 8, so they keep 4.
template <int CSPLIT>
constexpr int cs_waves() { return CSPLIT == 2 ? 8 : 4; }

template <typename KV, int BS, int G, bool OUT_BF16, int NCB, int CSPLIT>
__global__ void __launch_bounds__(64 * kMaxWavesPerWorker)
decode_streamk_kernel(void* __restrict__ out, float* __restrict__ rec, int32_t* __restrict__ seq_workers,
                      const uint16_t* __restrict__ q, const void* __restrict__ k_cache,
                      const void* __restrict__ v_cache, const int32_t* __restrict__ block_table,
                      int max_blocks_per_seq, const int32_t* __restrict__ context_lens,
                      int max_context_len, int num_seqs, int num_q_heads, int num_kv_heads,
                      float scale_log2, float out_scale, int num_workers,
                      const int32_t* __restrict__ cu_q_lens, int max_rows, int causal,
                      const uint64_t* __restrict__ tree_mask, const float* __restrict__ k_scales,
                      const float* __restrict__ v_scales) {
    constexpr int kWaves = kMaxWavesPerWorker;
    extern __shared__ int32_t s_cum[];
    __shared__ int32_t s_part[kWaves];
    // the matrix-core tile's per-wave V staging (one element otherwise)
    __shared__ __attribute__((aligned(16))) uint16_t s_vx[KV::kMfma && CSPLIT == 1 ? kWaves * kVxWaveElems : 8];
    __shared__ uint4 s_q[NCB > 1 ? kWaves * NCB * 4 * 64 : 1];
    // shared staging (cs_waves waves): two 32-token K and V tiles per KV head
    __shared__ __attribute__((aligned(16))) uint16_t s_st[CSPLIT > 1 ? (cs_waves<CSPLIT>() / CSPLIT) * 4 * 32 * (kHeadDim + 8) : 8];
    decode_worker<KV, BS, G, OUT_BF16, kWaves, NCB, CSPLIT>(
        out, rec, seq_workers, q, k_cache, v_cache, block_table, max_blocks_per_seq,
        context_lens, max_context_len, num_seqs, num_q_heads, num_kv_heads, scale_log2, out_scale,
        num_workers, cu_q_lens, s_cum, s_part, blockIdx.x, blockIdx.y, s_vx, max_rows, causal,
        tree_mask, s_q, s_st, k_scales, v_scales);
}

// Finishes every (sequence, query row, query head): zero rows for empty
// contexts, and the log-sum-exp merge of a sequence's pieces when several
// workers shared it: M = max_k m_k, L = sum_k l_k 2^(m_k - M),
// out = sum_k acc_k 2^(m_k - M) / L.
// Grid: (ceil(num_q_heads / 4), num_seqs, max_rows); block: 4 waves, one
// query head each.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256)
decode_merge_kernel(void* __restrict__ out, const float* __restrict__ rec,
                    const int32_t* __restrict__ seq_workers, const int32_t* __restrict__ context_lens,
                    int max_context_len, int num_seqs, int num_q_heads,
                    float out_scale, const int32_t* __restrict__ cu_q_lens, int max_rows) {
    constexpr int D = kHeadDim;
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int seq = blockIdx.y;
    const int r = blockIdx.z;
    if (h >= num_q_heads) return;
    // the row count, the context length and the workers holding the
    // sequence's first and last tiles are independent loads: all four are
    // issued before any of them is needed (the worker ids are read even
    // where the sequence turns out to have no tiles; they are in bounds)
    const int rows = rows_of(cu_q_lens, seq, max_rows);
    const int ctx_raw = context_lens[seq];
    const int32_t first = seq_workers[seq];
    const int64_t wl = seq_workers[num_seqs + seq];
    if (r >= rows) return;  // not a row of ours
    const size_t e = ((size_t)(row_of(cu_q_lens, seq) + r) * num_q_heads + h) * D + 2 * lane;
    if (clamp_ctx(ctx_raw, max_context_len) == 0) {  // nothing to attend to: a defined all-zero row
        store1<OUT_BF16>(out, e, 0.0f);
        store1<OUT_BF16>(out, e + 1, 0.0f);
        return;
    }
    const int64_t wf = first & 0x3fffffff;
    if (wf == wl) return;  // finalised by its only worker
    const int slot_f = (first >> 30) & 1;

    auto rec_of = [&](int64_t w) {
        const int slot = w == wf ? slot_f : 0;
        return rec + (((size_t)(w * 2 + slot) * max_rows + r) * num_q_heads + h) * kRecStride;
    };
    // accumulator rows of pieces p .. p + 7 (those that exist), loaded
    // eight pieces ahead of their use; the first eight go out together
    // with the pieces' (m, l)
    float2 av[8];
    auto load8 = [&](int64_t p) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
            av[u] = p + u <= wl ? *reinterpret_cast<const float2*>(rec_of(p + u) + 2 * lane)
                                : make_float2(0.0f, 0.0f);
    };
    load8(wf);
    // maximum over the pieces' running maxima, one piece per lane; the
    // first 64 pieces' (m, l) stay in their lanes
    float2 ml0 = make_float2(-INFINITY, 0.0f);
    if (wf + lane <= wl) ml0 = *reinterpret_cast<const float2*>(rec_of(wf + lane) + D);
    float mx = ml0.x;
    for (int64_t w = wf + 64 + lane; w <= wl; w += 64) mx = fmaxf(mx, rec_of(w)[D]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    // then the pieces in worker order, 64 at a time: lane k holds the scale
    // exp2(m - mx) and the sum l of piece base + k
    float L = 0.0f, a0 = 0.0f, a1 = 0.0f;
    for (int64_t base = wf; base <= wl; base += 64) {
        const int cnt = wl - base + 1 < 64 ? (int)(wl - base + 1) : 64;
        float2 ml = ml0;
        if (base != wf)
            ml = lane < cnt ? *reinterpret_cast<const float2*>(rec_of(base + lane) + D)
                            : make_float2(-INFINITY, 0.0f);
        const float fk = lane < cnt ? fast_exp2(ml.x - mx) : 0.0f;
        const float lk = ml.y;
        for (int k = 0; k < cnt; k += 8) {
            float2 cur[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) cur[u] = av[u];
            if (base + k + 8 <= wl) load8(base + k + 8);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (k + u >= cnt) break;
                const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fk), k + u));
                L = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(lk), k + u)), f, L);
                a0 = fmaf(cur[u].x, f, a0);
                a1 = fmaf(cur[u].y, f, a1);
            }
        }
    }
    const float inv = out_scale / L;
    store1<OUT_BF16>(out, e, a0 * inv);
    store1<OUT_BF16>(out, e + 1, a1 * inv);
}

template <typename KV, int BS, int G, bool OUT_BF16, int NCB, int CSPLIT>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    auto kern = decode_streamk_kernel<KV, BS, G, OUT_BF16, NCB, CSPLIT>;
    constexpr int kMax = kMaxWavesPerWorker;
    // head groups of kMax waves; the API admits 1..8 and 16 KV heads.  With
    // shared staging: workgroups of cs_waves waves, cs_waves / CSPLIT KV
    // heads each (the last group's missing heads leave at once; a wave that
    // has ended no longer holds back the others' barriers).
    const int hpg = cs_waves<CSPLIT>() / CSPLIT;
    const int waves = CSPLIT > 1 ? cs_waves<CSPLIT>()
                      : (a.num_kv_heads <= kMax ? a.num_kv_heads
                                                : (a.num_kv_heads % kMax == 0 ? kMax : 1));
    const int groups = CSPLIT > 1 ? (a.num_kv_heads + hpg - 1) / hpg : a.num_kv_heads / waves;
    const int threads = 64 * waves;
    const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int32_t);
    int resident = 0;
    hipError_t e = resident_workgroups(reinterpret_cast<const void*>(kern), threads, lds,
                                          &resident);
    if (e != hipSuccess) return e;
    // as many workers as the chip holds at once, never more than the records
    // in the workspace allow
    int64_t workers = resident / groups;
    if (workers > a.max_workers) workers = a.max_workers;
    if (workers < 1) workers = 1;
    hipLaunchKernelGGL(kern, dim3((int)workers, groups),
                       dim3(threads), lds, stream, a.out, a.records, a.seq_workers, a.q, a.k_cache,
                       a.v_cache, a.block_table, a.max_blocks_per_seq, a.context_lens,
                       a.max_context_len, a.num_seqs, a.num_q_heads, a.num_kv_heads, a.scale_log2,
                       a.out_scale, (int)workers, a.cu_q_lens, a.rows, a.causal ? 1 : 0,
                       a.tree_mask, a.k_scales, a.v_scales);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode_merge(a, stream);
}

template <typename KV, int BS, int G, int NCB = 1, int CSPLIT = 1>
hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s) {
    return a.out_bf16 ? launch_decode_t<KV, BS, G, true, NCB, CSPLIT>(a, s)
                      : launch_decode_t<KV, BS, G, false, NCB, CSPLIT>(a, s);
}

// Sequences of up to a.rows > 1 query rows: the matrix-core tile over their
// (row, head) pairs as columns, one block of 16 per KV head, or two for FP8
// pools (whose 16 VGPRs per tile in flight leave room for the second block's
// accumulators; a bf16 tile's 32 do not, and spilled, it lost to the
// stream-K chunk kernel).  The host admits rows <= 16 and rows x G <= 16,
// or <= 32 over FP8 pools.
template <typename KV, int BS, int G>
hipError_t launch_rows_g(const DecodeArgs& a, hipStream_t s) {
    if (a.rows * G <= 16) return launch_decode_g<KV, BS, G, 1>(a, s);
    if constexpr (G >= 2 && KV::kElemBytes == 1) {
        if (a.rows * G <= 32) return launch_decode_g<KV, BS, G, 2>(a, s);
    }
    if constexpr (G >= 2 && KV::kElemBytes == 2) {
        if (a.rows * G <= 32) return launch_decode_g<KV, BS, G, 1, 2>(a, s);
        if (a.rows * G <= 64) return launch_decode_g<KV, BS, G, 1, 4>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename KV, int BS>
hipError_t launch_rows_bs(const DecodeArgs& a, hipStream_t s) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_rows_g<KV, BS, 1>(a, s);
        case 2: return launch_rows_g<KV, BS, 2>(a, s);
        case 4: return launch_rows_g<KV, BS, 4>(a, s);
        case 8: return launch_rows_g<KV, BS, 8>(a, s);
        case 16: return launch_rows_g<KV, BS, 16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

// bf16 pools: the tile math on the matrix cores for 8 and 16 query heads
// per KV head, where the VALU layout is bound by its own arithmetic
// (70B-shaped batch, 8 heads: 334 -> 308 us per call against fp16 dot
// products on the VALU).  Up to 4 heads the VALU tile keeps P and V in fp32
// (errors near 1e-6 against the fp64 oracle); the matrix-core tile, with P
// and V in fp16 (errors near 1e-4), was 2.5 % faster on the 8B-shaped batch
// (4 heads), which did not buy that loss.
template <int BS>
hipError_t launch_decode_bf16_bs(const DecodeArgs& a, hipStream_t s) {
    if (a.rows > 1) return launch_rows_bs<KvBf16Mfma, BS>(a, s);
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_decode_g<KvBf16, BS, 1>(a, s);
        case 2: return launch_decode_g<KvBf16, BS, 2>(a, s);
        case 4: return launch_decode_g<KvBf16, BS, 4>(a, s);
        case 8: return launch_decode_g<KvBf16Mfma, BS, 8>(a, s);
        case 16: return launch_decode_g<KvBf16Mfma, BS, 16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

// FP8 pools: the matrix-core tile from 4 query heads per KV head, whose
// heads fill 4 of the MFMA's 16 columns or more.  Its P V is fp16 as on the
// VALU tiles, so it costs no accuracy; measured against them: 70B-shaped
// batch (8 heads) 303 -> 171 us, 8B-shaped batch (4 heads) 74.6 -> 59.7 us.
// With 1 or 2 heads the columns are mostly padding and the gain was 2-3 %,
// so those keep the VALU tile (16 dims per lane).
// FP8 pools with per-(block, KV head) scales, the rows path included (its
// two-block tile spills 32-76 bytes with the scales' registers and still
// beats the stream-K chunk kernel: 6-row verify 77.9 against 99.8 us).
template <int BS>
hipError_t launch_decode_fp8_bh_bs(const DecodeArgs& a, hipStream_t s) {
    if (a.rows > 1) return launch_rows_bs<KvFp8MfmaBh, BS>(a, s);
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_decode_g<KvFp8WideBh, BS, 1>(a, s);
        case 2: return launch_decode_g<KvFp8WideBh, BS, 2>(a, s);
        case 4: return launch_decode_g<KvFp8MfmaBh, BS, 4>(a, s);
        case 8: return launch_decode_g<KvFp8MfmaBh, BS, 8>(a, s);
        case 16: return launch_decode_g<KvFp8MfmaBh, BS, 16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <int BS>
hipError_t launch_decode_fp8_bs(const DecodeArgs& a, hipStream_t s) {
    // per-(block, KV head) scales: the same tiles reading them per tile
    if (a.k_scales != nullptr) return launch_decode_fp8_bh_bs<BS>(a, s);
    if (a.rows > 1) return launch_rows_bs<KvFp8Mfma, BS>(a, s);
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_decode_g<KvFp8Wide, BS, 1>(a, s);
        case 2: return launch_decode_g<KvFp8Wide, BS, 2>(a, s);
        case 4: return launch_decode_g<KvFp8Mfma, BS, 4>(a, s);
        case 8: return launch_decode_g<KvFp8Mfma, BS, 8>(a, s);
        case 16: return launch_decode_g<KvFp8Mfma, BS, 16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Workgroups of `kern` the device holds at once, for this much dynamic LDS
// (a pure function of the kernel and the device, cached per thread).
hipError_t resident_workgroups(const void* kern, int threads, size_t lds, int* out) {
    struct Entry { const void* kern; int threads; size_t lds; int dev; int blocks; };
    static thread_local Entry cache[16];
    static thread_local int next = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const size_t lds_key = (lds + 4095) / 4096 * 4096;
    for (const Entry& c : cache)
        if (c.kern == kern && c.threads == threads && c.lds == lds_key && c.dev == dev) {
            *out = c.blocks;
            return hipSuccess;
        }
    int n = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, lds_key);
    if (e != hipSuccess) return e;
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    *out = (n < 1 ? 1 : n) * cus;
    cache[next] = Entry{kern, threads, lds_key, dev, *out};
    next = (next + 1) % 16;
    return hipSuccess;
}

int64_t decode_max_workers(int num_seqs, int max_context_len, int rows, int num_kv_heads) {
    const int64_t tiles = (int64_t)num_seqs * ((max_context_len + kTileTokens - 1) / kTileTokens);
    int64_t w = (tiles + kMinTilesPerWorker - 1) / kMinTilesPerWorker;
    if (w > kMaxWorkers) w = kMaxWorkers;
    // several rows per sequence: records grow with the rows, so no more
    // workers than a 256-CU device holds at once (8 waves per CU, one per
    // KV head)
    if (rows > 1) {
        const int64_t cap = kRowsMaxWaves / (num_kv_heads < 1 ? 1 : num_kv_heads);
        if (w > cap) w = cap;
    }
    return w < 1 ? 1 : w;
}

size_t decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                              int max_context_len, int rows) {
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || rows < 1)
        return 0;
    const size_t cum = ((size_t)2 * num_seqs * sizeof(int32_t) + 255) / 256 * 256;
    return cum + (size_t)decode_max_workers(num_seqs, max_context_len, rows, num_kv_heads) * 2 *
                     rows * num_q_heads * kRecStride * sizeof(float);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream) {
    dim3 mgrid((a.num_q_heads + 3) / 4, a.num_seqs, a.rows);
    if (a.out_bf16)
        hipLaunchKernelGGL((decode_merge_kernel<true>), mgrid, dim3(256), 0, stream, a.out,
                           a.records, a.seq_workers, a.context_lens, a.max_context_len,
                           a.num_seqs, a.num_q_heads, a.out_scale, a.cu_q_lens, a.rows);
    else
        hipLaunchKernelGGL((decode_merge_kernel<false>), mgrid, dim3(256), 0, stream, a.out,
                           a.records, a.seq_workers, a.context_lens, a.max_context_len,
                           a.num_seqs, a.num_q_heads, a.out_scale, a.cu_q_lens, a.rows);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.kv_fp8)
        return a.block_size == 16 ? launch_decode_fp8_bs<16>(a, stream)
                                  : launch_decode_fp8_bs<32>(a, stream);
    return a.block_size == 16 ? launch_decode_bf16_bs<16>(a, stream)
                              : launch_decode_bf16_bs<32>(a, stream);
}

}  // namespace pkv
