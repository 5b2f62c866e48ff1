// Device helpers shared by the gfx950 kernels of the MXFP8 library.
//
// Formats: BF16 in, OCP E4M3 (or E5M2) payload bytes and E8M0 scale bytes
// out (one scale per 32 elements, or per 32x32 weight tile).  The scale
// exponent is the smallest e with amax <= 448 * 2^e ("rceil"; 57344 for
// E5M2), clamped to [-127, 127];
// on BF16 bits that is e = E - 135 + [mantissa > 96] for a normal amax
// (448 = 1.75 * 2^8 and 1.75 = 1 + 96/128), and -127 for zero or subnormal
// amax.  A block holding NaN or Inf gets scale 0xFF and payload 0x7F.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Largest BF16 magnitude pattern of the two halves of a packed pair.
__device__ __forceinline__ uint32_t pair_absmax(uint32_t w) {
  uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
  return lo > hi ? lo : hi;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 16-byte streaming load (read once, no reuse expected).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Max over 8 packed BF16 (one 16-byte chunk) of the magnitude bits.
__device__ __forceinline__ uint32_t chunk_absmax(uint4 v) {
  return umax(umax(pair_absmax(v.x), pair_absmax(v.y)), umax(pair_absmax(v.z), pair_absmax(v.w)));
}

// Butterfly max across lanes l ^ 1 and l ^ 2 (the four lanes of a quad),
// through DPP quad permutations.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  uint32_t t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  v = umax(v, t);
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  return umax(v, t);
}

__device__ __forceinline__ uint32_t xor_max(uint32_t v, int mask) {
  return umax(v, (uint32_t)__shfl_xor((int)v, mask, 64));
}

// Payload element types: OCP E4M3 (largest finite 448) and E5M2 (largest
// finite 57344 = 1.75 * 2^15).
enum Elem { ELEM_E4M3 = 0, ELEM_E5M2 = 1 };

// E8M0 scale byte for a block whose largest magnitude has BF16 bits `amax`:
// e = E - 135 + [m > 96] for E4M3 (448 = 1.75 * 2^8) and E - 142 + [m > 96]
// for E5M2 (57344 = 1.75 * 2^15), at least -127.
template <int EL>
__device__ __forceinline__ uint32_t scale_byte_t(uint32_t amax) {
  if (amax >= 0x7F80u) return 0xFFu;  // Inf or NaN in the block
  constexpr int off = EL == ELEM_E5M2 ? 142 : 135;
  int e = (int)(amax >> 7) - off + ((amax & 0x7Fu) > 96u ? 1 : 0);
  e = e < -127 ? -127 : e;
  return (uint32_t)(e + 127);
}
__device__ __forceinline__ uint32_t scale_byte(uint32_t amax) { return scale_byte_t<ELEM_E4M3>(amax); }

// The scale operand of v_cvt_scalef32_pk_{fp8,bf8}_bf16: a float whose value
// is 2^(byte - 127); byte 0 is the subnormal float 2^-127.
__device__ __forceinline__ float cvt_scale(uint32_t byte) {
  return __uint_as_float(byte ? (byte << 23) : 0x00400000u);
}

// Four BF16 (two packed words) -> four payload bytes of one dword, dividing
// by the block scale with round-to-nearest-even (v_cvt_scalef32_pk_fp8_bf16
// for E4M3, v_cvt_scalef32_pk_bf8_bf16 for E5M2).
template <int EL>
__device__ __forceinline__ uint32_t cvt4_t(uint32_t w0, uint32_t w1, float scale) {
  v2s acc = {0, 0};
  if (EL == ELEM_E5M2) {
    acc = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(acc, __builtin_bit_cast(v2bf, w0), scale, false);
    acc = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(acc, __builtin_bit_cast(v2bf, w1), scale, true);
  } else {
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(acc, __builtin_bit_cast(v2bf, w0), scale, false);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(acc, __builtin_bit_cast(v2bf, w1), scale, true);
  }
  return __builtin_bit_cast(uint32_t, acc);
}
__device__ __forceinline__ uint32_t cvt4(uint32_t w0, uint32_t w1, float scale) {
  return cvt4_t<ELEM_E4M3>(w0, w1, scale);
}

// Eight BF16 of a chunk -> eight payload bytes.  A non-finite block (scale
// byte 0xFF) gives all-NaN payload bytes (0x7F is NaN in both formats).
template <int EL>
__device__ __forceinline__ uint2 cvt8_t(uint4 v, uint32_t sbyte) {
  if (sbyte == 0xFFu) return make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
  float sc = cvt_scale(sbyte);
  return make_uint2(cvt4_t<EL>(v.x, v.y, sc), cvt4_t<EL>(v.z, v.w, sc));
}
__device__ __forceinline__ uint2 cvt8(uint4 v, uint32_t sbyte) { return cvt8_t<ELEM_E4M3>(v, sbyte); }

// BF16 pairs built from the same half of two packed words: (lo of a, lo of
// b) and (hi of a, hi of b).  Used to pair two rows of one column.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return (a & 0xFFFFu) | (b << 16);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xFFFF0000u);
}

// Two FP32 values -> two BF16 in one dword (a in the low half), rounded to
// nearest even, with gfx950's v_cvt_pk_bf16_f32.  Checked on the device
// against integer round-to-nearest-even on all 2^32 FP32 bit patterns (NaN
// inputs give NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

}  // namespace mx
