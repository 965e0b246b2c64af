// gdr_device.h -- device helpers shared by the libgdr kernels (gfx950 / CDNA4 only).
//
// MFMA conventions used throughout (64-lane wavefront, l = lane id, g = l / 32):
//   32x32 tile, operand fragment: lane (i = l % 32, g) holds 8 consecutive reduction
//   indices k = 8g .. 8g+7 of row i (A operand) or column i (B operand).  Because the
//   instruction pairs A's and B's reduction slots identically, any consistent placement of
//   the logical k across (g, element) is a valid product; the fp32 emulation below relies
//   on that.
//   32x32 accumulator (16 floats): register r of lane l is element
//       row = 8 * (r / 4) + 4 * g + (r % 4),   col = l % 32.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace gdr {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;   // chunk length C
constexpr int kWave = 64;    // CDNA wavefront

// ---------------------------------------------------------------- host-side launch helpers
// Dynamic LDS beyond the default limit is enabled per kernel and device
// (hipFuncAttributeMaxDynamicSharedMemorySize).  `done` holds one bit per device id below 64,
// so a launcher makes the call once per device; concurrent first calls only repeat it.
template <typename Kern>
inline hipError_t enable_dynamic_lds(Kern kern, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
    if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

// Compute units of the current device, cached per device id (below 64).
inline hipError_t device_cu_count(int& ncu) {
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool slot = dev >= 0 && dev < 64;
    if (slot && (ncu = cache[dev].load(std::memory_order_relaxed)) > 0) return hipSuccess;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (ncu < 1) ncu = 1;
    if (slot) cache[dev].store(ncu, std::memory_order_relaxed);
    return hipSuccess;
}

// ---------------------------------------------------------------- scalar conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16 with round-to-nearest-even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// I/O element access for the two supported dtypes.
template <typename IOT> struct IO;
template <> struct IO<uint16_t> {  // bf16 stored as raw bits
    static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float x) { p[i] = f32_to_bf16_bits(x); }
};
template <> struct IO<float> {
    static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, int64_t i, float x) { p[i] = x; }
};

// ---------------------------------------------------------------- MFMA operand fragments
// Frag<OpT>: the 8 reduction-slot values one lane contributes to a 32x32x16 product.
template <typename OpT> struct Frag;
template <> struct Frag<_Float16> { half8 v; };
template <> struct Frag<float> { float8v v; };

template <typename OpT>
__device__ __forceinline__ Frag<OpT> load_frag(const OpT* p);  // 8 consecutive elements
template <>
__device__ __forceinline__ Frag<_Float16> load_frag<_Float16>(const _Float16* p) {
    Frag<_Float16> f;
    f.v = *reinterpret_cast<const half8*>(p);
    return f;
}
template <>
__device__ __forceinline__ Frag<float> load_frag<float>(const float* p) {
    Frag<float> f;
    f.v = *reinterpret_cast<const float8v*>(p);
    return f;
}

// 8 elements at a stride (transposed gather from a row-major LDS matrix).
template <typename OpT>
__device__ __forceinline__ Frag<OpT> gather_frag(const OpT* p, int stride) {
    Frag<OpT> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = p[e * stride];
    return f;
}

// acc += A * B on a 32x32 tile with a 16-deep reduction.
__device__ __forceinline__ void mma32(float16v& acc, const Frag<_Float16>& a, const Frag<_Float16>& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.v, b.v, acc, 0, 0, 0);
}
// fp32 operands: eight 32x32x2 products; instruction e pairs slot e of every lane, so the
// 16 reduction indices are covered once each, in the same order for A and B.
__device__ __forceinline__ void mma32(float16v& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// Accumulator register r of lane l -> (row, col) of the 32x32 tile.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

// Store the 4 consecutive-row accumulator values r = 4j..4j+3 of one lane (rows
// 8j + 4g .. 8j + 4g + 3 of column col) into a [col][row] matrix with row stride `ld`.
template <typename OpT>
__device__ __forceinline__ void store4_transposed(OpT* base, int ld, int col, int row0, float a, float b,
                                                  float c, float d) {
    OpT* p = base + col * ld + row0;
    if constexpr (sizeof(OpT) == 2) {
        half4 h = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
        *reinterpret_cast<half4*>(p) = h;
    } else {
        float4v f = {a, b, c, d};
        *reinterpret_cast<float4v*>(p) = f;
    }
}

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

// Workgroups are dispatched round-robin over the 8 XCDs; renumber them so that consecutive
// logical indices (the d_v tiles of one sequence, which read the same q/k chunks) land on
// the same XCD and share its L2.  A bijection of [0, nwg) for any nwg.
__device__ __forceinline__ int xcd_major_index(int wg, int nwg) {
    const int xcd = wg & 7, slot = wg >> 3;
    const int q8 = nwg >> 3, r8 = nwg & 7;
    return xcd * q8 + (xcd < r8 ? xcd : r8) + slot;
}

}  // namespace gdr
