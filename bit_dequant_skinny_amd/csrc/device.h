// Device helpers for the gfx950 kernels of the q4skinny library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// A bf16 value is the upper half of an fp32 pattern, so widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest with ties to even.  Adding 0x7fff plus
// the lowest kept bit carries into the kept half exactly when the discarded
// half is above one half, or equal to it with an odd kept half.  NaN inputs
// keep their sign and upper payload and get the quiet bit.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Codebook lookup through the cross-lane permute unit.  Every lane of the
// wave holds codebook[lane % 16] in `table`; ds_bpermute returns the `table`
// register of the lane whose byte address is given, so the 16-entry table is
// read with no LDS allocation and no bank conflicts.  All 64 lanes must be
// active when this runs.
__device__ __forceinline__ float cb_lookup(int table, uint32_t code) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((int)((code & 15u) << 2), table));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Element types of the C ABI (the Q4_DTYPE_* codes).
enum : int { kBf16 = 0, kF32 = 1, kF16 = 2 };

// IEEE binary16 <-> fp32.  Widening is exact; narrowing rounds to nearest
// even (v_cvt_f16_f32 in the default rounding mode, fp16 denormals kept).
__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}
__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// A pair of fp16 values as two pairs of bf16 values, hi and lo, with
// hi + lo equal to each fp16 value exactly: hi is the nearest bf16 and the
// remainder has at most 3 significant bits, well inside bf16's precision and
// range.
__device__ __forceinline__ uint2 f16x2_to_bf16_hilo(uint32_t d) {
    const float f0 = f16_to_f32(d & 0xffffu), f1 = f16_to_f32(d >> 16);
    const uint32_t h0 = f32_to_bf16_rne(f0), h1 = f32_to_bf16_rne(f1);
    const uint32_t l0 = f32_to_bf16_rne(f0 - bf16_lo(h0)), l1 = f32_to_bf16_rne(f1 - bf16_lo(h1));
    return make_uint2(h0 | (h1 << 16), l0 | (l1 << 16));
}

// Element i of a vector of type dt (bf16, fp16 or fp32), widened to fp32.
__device__ __forceinline__ float load_elem(const void *p, size_t i, int dt) {
    if (dt == kF32) return reinterpret_cast<const float *>(p)[i];
    const uint32_t b = reinterpret_cast<const uint16_t *>(p)[i];
    return dt == kF16 ? f16_to_f32(b) : bf16_lo(b);
}

// Rounds v to type dt (nearest even) and stores it as element i.
__device__ __forceinline__ void store_elem(void *p, size_t i, float v, int dt) {
    if (dt == kF32) reinterpret_cast<float *>(p)[i] = v;
    else if (dt == kF16) reinterpret_cast<uint16_t *>(p)[i] = (uint16_t)f32_to_f16_rne(v);
    else reinterpret_cast<uint16_t *>(p)[i] = (uint16_t)f32_to_bf16_rne(v);
}

// Packed-byte decode table of the matrix-core kernels.  Entry e (a packed
// byte, low nibble = even k) holds x = (hi(cb[e & 15]), hi(cb[e >> 4])) and
// y = (lo(cb[e & 15]), lo(cb[e >> 4])) in bf16, where hi = bf16(cb) and
// lo = bf16(cb - hi): hi + lo equals the fp32 codebook value to within 2^-16
// relative (two roundings to 8 significant bits), and exactly when the value
// has at most 16 significant bits.  Two entries back to back, [x0 y0 x1 y1],
// form the operand [hi(c0) hi(c1) lo(c0) lo(c1) hi(c2) hi(c3) lo(c2) lo(c3)] of
// v_mfma_f32_16x16x32_bf16, which against the activations [a0 a1 a0 a1 a2 a3
// a2 a3] forms a*hi + a*lo exactly in the fp32 accumulator.
__device__ __forceinline__ uint2 pair_table_entry(float c0, float c1) {
    const uint32_t h0 = f32_to_bf16_rne(c0), h1 = f32_to_bf16_rne(c1);
    const uint32_t l0 = f32_to_bf16_rne(c0 - __uint_as_float(h0 << 16));
    const uint32_t l1 = f32_to_bf16_rne(c1 - __uint_as_float(h1 << 16));
    return make_uint2(h0 | (h1 << 16), l0 | (l1 << 16));
}

// A lane of group g = lane / 16 loads 16 packed bytes (32 codes) at byte
// 16*g of a 128-wide segment of one weight row.  One v_permlane32_swap of
// dwords (0, 2) and one of (1, 3) leave lanes 0-31 with their own dwords 0,1
// and dwords 0,1 of the lane 32 above, and lanes 32-63 with dwords 2,3 of the
// lane 32 below and their own dwords 2,3, so that dwords 0,1 of every lane
// hold codes of the segment's first 64 k and dwords 2,3 codes of the second.
// This is the k offset, within the segment, of the 8 codes in dword t.
__device__ __forceinline__ uint32_t swapped_k_offset(int g, int t) {
    return 32 * (g & 1) + 16 * (g >> 1) + 8 * (t & 1) + 64 * (t >> 1);
}

__device__ __forceinline__ void permlane32_swap_dwords(uint4 &w) {
    const auto s02 = __builtin_amdgcn_permlane32_swap(w.x, w.z, false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(w.y, w.w, false, false);
    w.x = s02[0];
    w.z = s02[1];
    w.y = s13[0];
    w.w = s13[1];
}

__device__ __forceinline__ floatx4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 128-bit global load that bypasses nothing but keeps the access a single
// global_load_dwordx4.
__device__ __forceinline__ uint4 ld128(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// Sum across the 64 lanes of a wave (every lane gets the total).  The order
// of additions is fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace q4
