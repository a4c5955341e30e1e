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
