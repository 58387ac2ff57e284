// pkv_device.h -- device-side helpers shared by the gfx950 kernels of
// libpagedkv: bf16 unpacking, the bf16 dot2 instruction, and 16-lane row
// reductions built from DPP moves (a CDNA wave is 64 lanes = 4 rows of 16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kHeadDim = 128;
// Split-KV partition length in tokens.  A multiple of every supported block
// size, so partitions start on block boundaries.
constexpr int kPartitionTokens = 512;
// Tokens per inner tile of the decode loop: 16 tokens = 4 KB of K (or V) for
// one KV head, moved by one wave as four 128-bit loads per lane.
constexpr int kTileTokens = 16;
// A finite "minus infinity" for running maxima, so that a row that has seen
// no key yet never produces exp2(-inf - -inf).
constexpr float kNegBig = -1.0e30f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Raw buffer resource over `base` (wave-uniform, so it lives in scalar
// registers) spanning 2^31 - 1 bytes; word 3 is the gfx9-family raw-buffer
// format.  A lane offset at or past kBufferOob reads zeros without touching
// memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                             0x00020000);
}
constexpr uint32_t kBufferOob = 0x80000000u;

// fp32 value of the low / high bf16 of a packed pair (exact: a bf16 is the
// top half of the fp32 with the same value).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// c + a.lo * b.lo + a.hi * b.hi with bf16 pairs, fp32 accumulate
// (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}

// DPP controls: quad permutations and mirrors inside a 16-lane row.
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i in each half row
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15 - i in the row

// Sum over the 16 lanes of each row; every lane of the row receives the
// same bits.  Each step adds two partners that hold equal values within
// their groups (pairs, quads, half rows), so both sides compute A + B and
// B + A, which round alike; rotations would pair lanes asymmetrically and
// leave quads with differently rounded totals.
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp_mov<kDppQuadXor1>(x);
    x += dpp_mov<kDppQuadXor2>(x);
    x += dpp_mov<kDppRowHalfMirror>(x);
    x += dpp_mov<kDppRowMirror>(x);
    return x;
}

// row_sum16 of N independent values, one butterfly step across all of them
// before the next: a DPP read of a register written by the VALU instruction
// just before it needs hazard wait states, and N independent chains keep
// the producer of each step N instructions back.
template <int N>
__device__ __forceinline__ void row_sums16(float (&x)[N]) {
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] += dpp_mov<kDppQuadXor1>(x[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] += dpp_mov<kDppQuadXor2>(x[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] += dpp_mov<kDppRowHalfMirror>(x[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] += dpp_mov<kDppRowMirror>(x[n]);
}

// The same over each half row of 8 lanes (a wave seen as 8 rows of 8).
__device__ __forceinline__ float row_sum8(float x) {
    x += dpp_mov<kDppQuadXor1>(x);
    x += dpp_mov<kDppQuadXor2>(x);
    x += dpp_mov<kDppRowHalfMirror>(x);
    return x;
}
template <int N>
__device__ __forceinline__ void row_sums8(float (&x)[N]) {
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] += dpp_mov<kDppQuadXor1>(x[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] += dpp_mov<kDppQuadXor2>(x[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] += dpp_mov<kDppRowHalfMirror>(x[n]);
}

// Exchange across rows: value of lane ^ 16 / lane ^ 32 (LDS-crossbar permute).
__device__ __forceinline__ float xor_lane(float x, int mask) {
    int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

// Max / sum of x over lanes l and l ^ 32, with gfx950's 32-lane swap (a
// VALU exchange; the LDS crossbar is not involved).  Each lane ends up with
// both halves' values, so the symmetric reductions need no lane select.
__device__ __forceinline__ float max_lane_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_lane_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max / sum of x over lanes l, l ^ 16, l ^ 32, l ^ 48 (the same position in
// the four 16-lane rows), with gfx950's 16- and 32-lane swaps.
__device__ __forceinline__ float max_lane_quads(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max_lane_halves(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float sum_lane_quads(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return sum_lane_halves(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Stream-K ranges: U work units laid end to end, cut into W equal contiguous
// ranges.  Worker w owns units [worker_start(w), worker_start(w + 1)).
__device__ __forceinline__ int64_t worker_start(int64_t w, int64_t U, int64_t W) {
    return (w * U) / W;
}
// The worker whose range holds unit t.
__device__ __forceinline__ int64_t worker_of(int64_t t, int64_t U, int64_t W) {
    return ((t + 1) * W - 1) / U;
}

}  // namespace pkv
