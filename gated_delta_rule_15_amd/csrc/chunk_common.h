// chunk_common.h -- device helpers shared by the chunked-forward kernels (gfx950).
//
// MFMA 16x16x32 f16 conventions (l = lane, j = l & 15, g = l >> 4):
//   accumulator register r of lane l holds element (row 4g + r, column j);
//   an operand fragment of lane l is row/column j with the 8 reduction indices
//   {32kb + 4g + r} U {32kb + 16 + 4g + r}, r = 0..3.
// Matrices used as operands from LDS store their reduction index permuted within each
// 32-block (pperm below), so one fragment is one 16-byte read.
#pragma once
#include "gdr_device.h"

namespace gdr {

// The chunk's triangular matrices are stored without their all-zero 32x32 block: A^T (row m
// holds A[l][m], nonzero for l >= m) keeps rows 0..31 at full width and rows 32..63 at columns
// 32..63; T (lower triangular) keeps rows 0..31 at columns 0..31 and rows 32..63 at full width.
// Each is 384 pieces of 8 halfs (3072 halfs), stored in piece order.
constexpr int kTriHalfs = 3 * kChunk * kChunk / 4;
constexpr int kTriPieces = kTriHalfs / 8;
__device__ __forceinline__ void at_piece(int idx, int& row, int& col) {
    if (idx < 256) {
        row = idx >> 3;
        col = (idx & 7) * 8;
    } else {
        row = 32 + ((idx - 256) >> 2);
        col = 32 + ((idx - 256) & 3) * 8;
    }
}
__device__ __forceinline__ void t_piece(int idx, int& row, int& col) {
    if (idx < 128) {
        row = idx >> 2;
        col = (idx & 3) * 8;
    } else {
        row = 32 + ((idx - 128) >> 3);
        col = ((idx - 128) & 7) * 8;
    }
}

// Workspace of the per-channel-gate two-kernel path, per (sequence, chunk), in halfs:
// A^T and T (compact, T's columns pperm'd), K e^G [C][DK], Q e^G [C][DK], K e^{G_C - G} [C][DK]
// (fp16), then e^{G_C} [DK] (fp32, natural channel order).
template <int DK>
constexpr int kda_ws_stride() { return 2 * kTriHalfs + 3 * kChunk * DK + 2 * DK; }

// position of logical index m inside its row under the 32-block permutation
__device__ __forceinline__ int pperm(int m) {
    return (m & ~31) | (((m >> 2) & 3) << 3) | (((m >> 4) & 1) << 2) | (m & 3);
}

__device__ __forceinline__ void mma16(float4v& acc, const half8& a, const half8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ half8 ld8(const _Float16* p) { return *reinterpret_cast<const half8*>(p); }
__device__ __forceinline__ half4 ldtr(const _Float16* p) {
    typedef short short4v __attribute__((ext_vector_type(4)));
    const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p));
    return __builtin_bit_cast(half4, v);
}
__device__ __forceinline__ half8 cat8(const half4& lo, const half4& hi) {
    return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ half8 pack8(const float4v& lo, const float4v& hi) {
    half8 h;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        h[r] = (_Float16)lo[r];
        h[4 + r] = (_Float16)hi[r];
    }
    return h;
}
__device__ __forceinline__ float4v zero4() { return float4v{0.0f, 0.0f, 0.0f, 0.0f}; }
__device__ __forceinline__ float4v ld4f(const float* p) { return *reinterpret_cast<const float4v*>(p); }
// Wave-local ordering of LDS writes before later LDS reads of the same wave.
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Workgroup barrier for LDS traffic only.  Unlike __syncthreads() it does not wait for the
// wave's outstanding global loads, so prefetches stay in flight across phases; no global
// memory is exchanged between waves.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 8 bf16 (one uint4, element order preserved) -> 8 fp16.
__device__ __forceinline__ half8 bf16x8_to_half8(const uint4& u) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    half8 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[2 * e] = (_Float16)__uint_as_float(w[e] << 16);
        h[2 * e + 1] = (_Float16)__uint_as_float(w[e] & 0xffff0000u);
    }
    return h;
}
// One 16-byte piece (8 bf16) of a row of DK values whose DK / 8 pieces sit in consecutive
// lanes of one 16-lane DPP row: the row's inverse L2 norm 1 / max(||x||, 1e-6) (returned in
// inv, the same in every lane of the row) and the piece divided by the norm, in fp16.
// quad_perm xor 1 and xor 2, row_half_mirror (and row_mirror for 16 lanes) leave the row's
// sum of squares in every lane.  Every lane of the wave must take part.
template <int DK>
__device__ __forceinline__ half8 unit_rows(const uint4& u, float& inv) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float x[8], ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0xB1, 0xf, 0xf, false));
    ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x4E, 0xf, 0xf, false));
    ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x141, 0xf, 0xf, false));
    if constexpr (DK == 128)
        ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x140, 0xf, 0xf, false));
    inv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-12f));
    half8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (_Float16)(x[e] * inv);
    return h;
}
// 8 bf16 (one uint4) -> 8 fp16 written as two 4-element groups at permuted positions.
__device__ __forceinline__ void stage8(_Float16* row, int m0, const uint4& u) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    half4 a, b;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        a[2 * e] = (_Float16)__uint_as_float(w[e] << 16);
        a[2 * e + 1] = (_Float16)__uint_as_float(w[e] & 0xffff0000u);
        b[2 * e] = (_Float16)__uint_as_float(w[2 + e] << 16);
        b[2 * e + 1] = (_Float16)__uint_as_float(w[2 + e] & 0xffff0000u);
    }
    *reinterpret_cast<half4*>(row + pperm(m0)) = a;
    *reinterpret_cast<half4*>(row + pperm(m0 + 4)) = b;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves (no LDS traffic):
// shifts by 1, 2, 4, 8 within each 16-lane row, then the row totals are broadcast into the
// following rows.  Lanes whose source falls outside the row receive 0.
__device__ __forceinline__ float dpp_add(float x, int y_bits) { return x + __int_as_float(y_bits); }
__device__ __forceinline__ float wave_inclusive_scan(float x) {
    int b = __float_as_int(x);
    x = dpp_add(x, __builtin_amdgcn_update_dpp(0, b, 0x111, 0xf, 0xf, false));  // row_shr:1
    b = __float_as_int(x);
    x = dpp_add(x, __builtin_amdgcn_update_dpp(0, b, 0x112, 0xf, 0xf, false));  // row_shr:2
    b = __float_as_int(x);
    x = dpp_add(x, __builtin_amdgcn_update_dpp(0, b, 0x114, 0xf, 0xf, false));  // row_shr:4
    b = __float_as_int(x);
    x = dpp_add(x, __builtin_amdgcn_update_dpp(0, b, 0x118, 0xf, 0xf, false));  // row_shr:8
    b = __float_as_int(x);
    x = dpp_add(x, __builtin_amdgcn_update_dpp(0, b, 0x142, 0xa, 0xf, false));  // row_bcast:15
    b = __float_as_int(x);
    x = dpp_add(x, __builtin_amdgcn_update_dpp(0, b, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return x;
}
// Largest |x| over a lane's registers (NaN entries are ignored by max).
template <int N>
__device__ __forceinline__ float max_abs(const float4v (&x)[N]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(x[i][r]));
    return m;
}
// Largest value over the 64 lanes, the same in every lane: a DPP reduction inside each 16-lane
// row (quad_perm xor 1 and xor 2, row_half_mirror, row_mirror), then the four row results.
__device__ __forceinline__ float wave_max_abs(float m) {
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xf, 0xf, false)));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xf, 0xf, false)));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x141, 0xf, 0xf, false)));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x140, 0xf, 0xf, false)));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float lane_value(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Buffer resources: a load past the resource's byte range returns zeros and a store past it
// is dropped, which pads the ragged last chunk with identity tokens (k = q = v = 0,
// g = beta = 0) and clips its output rows without any branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return uint4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ float bld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void bst16(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint4& u) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{u.x, u.y, u.z, u.w}, r, off, 0, 0);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float float2v __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{lo, hi}, bf16x2));  // one RNE cvt_pk
}

}  // namespace gdr
