// plx_device.hpp -- gfx950 device helpers shared by the Parallax kernels.
//
// Vector types for the bf16 matrix-core builtins, buffer-resource loads (out-of-range
// reads return zero, so ragged tails and masked cache rows need no extra predicates),
// RNE packing to bf16 and wave-level shuffles. CDNA4 only: 64-wide wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// ----------------------------------------------------------------------------- buffers
// Raw buffer resource over [base, base + bytes). Dword 3 selects 32-bit data format with
// no swizzle (the gfx9-family raw-buffer setting).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 16-byte load at byte offset `off`; returns zeros when off + 16 > bytes of the resource.
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Same, marked non-temporal (streamed once; do not keep in the caches).
__device__ __forceinline__ u32x4 load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}

// ----------------------------------------------------------------------------- bf16
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }


__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// ----------------------------------------------------------------------------- math
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ----------------------------------------------------------------------------- shuffles
__device__ __forceinline__ float shfl_xor(float x, int mask) {
    const int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

// Swap values between adjacent lanes (0<->1, 2<->3, ...): DPP quad permutation [1,0,3,2].
__device__ __forceinline__ float swap_adjacent(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}

// max(x, x of the lane 32 away): v_permlane32_swap hands each half-wave the other half's
// value (entry 1 holds the upper half's x in lanes 0..31, entry 0 the lower half's x in
// lanes 32..63), a VALU exchange instead of an LDS round trip.
__device__ __forceinline__ float max_with_other_half(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false,
                                                    false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

// max(a, b, c): the NaN-propagating maximum, which gfx950 executes as one v_maximum3_f32. The
// fmaxf chain would first canonicalize every operand that comes from a matrix instruction (a
// v_max x, x per element under IEEE mode); for non-NaN inputs both give the same value.
__device__ __forceinline__ float max3(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

__device__ __forceinline__ float wave_max(float x) {
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, shfl_xor(x, m));
    return x;
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

}  // namespace plx
