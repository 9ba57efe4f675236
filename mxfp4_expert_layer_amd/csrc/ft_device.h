// Device helpers shared by libft's HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include "ft_internal.h"

namespace ft {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

// Direct global -> LDS copies: lane l's 16 (or 4) bytes land at lds + 16 l (4 l); the wait
// for them is the vector-memory count (checked on gfx950: per-lane sources may be scattered).
__device__ __forceinline__ void dma16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds, 4, 0, 0);
}
// The same copies through a buffer resource: the address is the resource's base + voff (per
// lane) + soff (wave-uniform); a lane whose offset lies past the resource's size reads zeros.
constexpr int kBufFlags = 0x00020000;   // raw buffer, 32-bit data format (gfx9 word 3)
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                       void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void bdma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                      void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, soff, 0, 0);
}
// s_waitcnt with vmcnt = n and no wait on the other counters (gfx9 field layout)
#define FT_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

// E8M0 code -> fp32 scale 2^(e - 127): e = 0 is 2^-127 (an fp32 subnormal), e = 255 NaN.
// The scaled FP4 converts below use only the exponent field of this value, which for every
// code but 255 is exactly the E8M0 exponent (measured on gfx950: a scale of 0.75 acts as 2^-1,
// and the subnormal 2^-127 acts as 2^-127).
__device__ __forceinline__ float e8m0_f32(uint32_t e) {
  uint32_t bits = (e == 0u) ? 0x00400000u : ((e == 255u) ? 0x7fc00000u : (e << 23));
  return __uint_as_float(bits);
}

// Eight E2M1 codes (one dword, element 0 in the low nibble) times a power-of-two scale ->
// eight bf16 (exact: an E2M1 value has at most 2 significant bits).
__device__ __forceinline__ bf16x8 fp4x8_bf16(uint32_t w, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  auto lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  auto hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Eight E2M1 codes times an arbitrary fp32 scale s -> eight bf16, for NVFP4 (s = an E4M3
// value): each code is converted to fp32 exactly (unit scale), multiplied by s in fp32 and
// truncated to its upper 16 bits.  E2M1 x E4M3 has at most 6 significant bits and lies within
// [2^-10, 2688], so the product and its truncation are exact (a NaN s gives NaN).
__device__ __forceinline__ bf16x8 fp4x8_bf16_mul(uint32_t w, float s) {
#define FT_FP4PAIR(b)                                                                      \
  [&] {                                                                                     \
    const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, b);                   \
    return __builtin_amdgcn_perm(__float_as_uint(f[1] * s), __float_as_uint(f[0] * s),     \
                                 0x07060302u);                                              \
  }()
  const uint4 d = make_uint4(FT_FP4PAIR(0), FT_FP4PAIR(1), FT_FP4PAIR(2), FT_FP4PAIR(3));
#undef FT_FP4PAIR
  return __builtin_bit_cast(bf16x8, d);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }
// silu with the hardware exp and reciprocal (v_exp_f32, v_rcp_f32: a few ulp), for the
// prefill epilogues, where h is then quantised to FP4 or rounded to bf16: either decision
// moves only for values within a few fp32 ulp of its boundary.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// v of lane (lane ^ J), with the VALU's own lane exchanges instead of the LDS crossbar
// (checked on gfx950): DPP quad permutes for 1 and 2, row rotates for 4 and 8 (row_ror:n
// gives lane i the value of lane i - n within its row of 16), and the gfx950 permlane swaps
// for 16 and 32.  Lane-dependent choices use constant lane masks (one v_cndmask).
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  if (J == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false);
  if (J == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, false);
  if (J == 4) {
    const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x12C, 0xf, 0xf, false);
    const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xf, 0xf, false);
    return __builtin_amdgcn_inverse_ballot_w64(0xF0F0F0F0F0F0F0F0ull) ? dn : up;
  }
  if (J == 8) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xf, 0xf, false);
  if (J == 16) {
    const auto sw = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return __builtin_amdgcn_inverse_ballot_w64(0xFFFF0000FFFF0000ull) ? sw[0] : sw[1];
  }
  const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __builtin_amdgcn_inverse_ballot_w64(0xFFFFFFFF00000000ull) ? sw[0] : sw[1];
}

// Sum over the 64 lanes by a butterfly of lane exchanges: every lane gets the same value.
__device__ __forceinline__ float wave_sum(float v) {
  v += __uint_as_float(xor_lane<1>(__float_as_uint(v)));
  v += __uint_as_float(xor_lane<2>(__float_as_uint(v)));
  v += __uint_as_float(xor_lane<4>(__float_as_uint(v)));
  v += __uint_as_float(xor_lane<8>(__float_as_uint(v)));
  v += __uint_as_float(xor_lane<16>(__float_as_uint(v)));
  v += __uint_as_float(xor_lane<32>(__float_as_uint(v)));
  return v;
}

// E2M1 value table and E4M3 decode in plain fp32 (NVFP4 paths and the debug dequant).
__device__ __forceinline__ float e2m1_f32(uint32_t c) {
  const float m = (c & 4) ? ((c & 2) ? ((c & 1) ? 6.f : 4.f) : ((c & 1) ? 3.f : 2.f))
                          : ((c & 2) ? ((c & 1) ? 1.5f : 1.f) : ((c & 1) ? 0.5f : 0.f));
  return (c & 8) ? -m : m;
}
// The same E4M3 decode by bit assembly: a normal code's fp32 exponent field is e + 120 with
// its 3 mantissa bits on top of the fp32 mantissa; a subnormal is m x 2^-9.
// The magnitude bits eeeemmm placed at fp32 bit 20 read as 2^(e - 127) (1 + m/8) for e > 0 and
// as the fp32 subnormal m 2^-129 for e = 0; one multiply by 2^120 turns both into the E4M3
// value (2^(e - 7) (1 + m/8), or m 2^-9), exactly.  No branch and no select but the NaN code's.
// Needs fp32 denormal inputs kept (the kernels' default float mode, which does not flush).
__device__ __forceinline__ float e4m3_f32_fast(uint32_t c) {
  const float mag = __uint_as_float((c & 0x7fu) << 20) * 0x1p120f;
  const float v = (c & 0x7fu) == 0x7fu ? __uint_as_float(0x7fc00000u) : mag;
  return __uint_as_float(__float_as_uint(v) | ((c & 0x80u) << 24));
}
__device__ __forceinline__ float e4m3_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15, m = c & 7;
  float v;
  if (e == 15 && m == 7) v = __uint_as_float(0x7fc00000u);
  else if (e == 0) v = ldexpf((float)m * 0.125f, -6);
  else v = ldexpf(1.f + (float)m * 0.125f, (int)e - 7);
  return (c & 0x80) ? -v : v;
}

// ---- 24-bit floats (fp32 with the low 8 mantissa bits rounded away, to nearest even) ----
// Four values in 12 bytes, value i in bits 24 i .. 24 i + 23.  Infinities stay infinite, a
// NaN stays a NaN, finite values keep their exponent range (a value may round up to inf only
// from within 2^-16 of the fp32 maximum); the relative rounding error is at most 2^-16.
// fp32 bits rounded at bit 8, to nearest even (the value sits in bytes 1..3); a NaN becomes
// the quiet NaN of its sign
__device__ __forceinline__ uint32_t f32_round24(float f) {
  const uint32_t b = __float_as_uint(f);
  const uint32_t r = b + 0x7fu + ((b >> 8) & 1u);
  return f != f ? ((b & 0x80000000u) | 0x7fc00000u) : r;
}
__device__ __forceinline__ uint3 pack_f24x4(float v0, float v1, float v2, float v3) {
  const uint32_t r0 = f32_round24(v0), r1 = f32_round24(v1), r2 = f32_round24(v2),
                 r3 = f32_round24(v3);
  // bytes 1..3 of each, in order: [r0.1 r0.2 r0.3 r1.1] [r1.2 r1.3 r2.1 r2.2] [r2.3 r3.1 r3.2 r3.3]
  return make_uint3(__builtin_amdgcn_perm(r1, r0, 0x05030201u),
                    __builtin_amdgcn_perm(r2, r1, 0x06050302u),
                    __builtin_amdgcn_perm(r3, r2, 0x07060503u));
}
__device__ __forceinline__ float4 unpack_f24x4(uint3 w) {
  return make_float4(__uint_as_float(w.x << 8),
                     __uint_as_float(((w.x >> 24) | (w.y << 8)) << 8),
                     __uint_as_float(((w.y >> 16) | (w.z << 16)) << 8),
                     __uint_as_float(w.z & 0xffffff00u));
}

// ---- OCP MX quantiser (32-value blocks, E8M0 scale, E2M1 codes) -----------------------------
// Block scale 2^(floor(log2 amax) - 2) (2 is E2M1's largest exponent) with the exponent
// clamped to [-127, 127]: for a finite fp32 amax with biased exponent field f that is the E8M0
// code max(f - 2, 0) (zero and subnormal blocks get 0).  A non-finite amax gives the NaN code.
__device__ __forceinline__ uint32_t mx_scale_code(float amax) {
  const uint32_t f = (__float_as_uint(amax) >> 23) & 0xffu;
  return f == 0xffu ? 0xffu : (f > 2u ? f - 2u : 0u);
}
// 1 / scale = 2^(127 - code), a normal fp32 for codes 0..252 (NaN for 255).
__device__ __forceinline__ float mx_inv_scale(uint32_t code) {
  return code == 0xffu ? __uint_as_float(0x7fc00000u) : __uint_as_float((254u - code) << 23);
}
// E2M1 code of v / scale: r = |v| / scale (exact, a power-of-two product) rounded to the
// nearest of 0, .5, 1, 1.5, 2, 3, 4, 6 with ties to the even code, saturating at 6; the code's
// sign bit is v's sign bit.
__device__ __forceinline__ uint32_t mx_code(float v, float inv) {
  const float r = fabsf(v) * inv;
  const uint32_t c = (uint32_t)(r > 0.25f) + (uint32_t)(r >= 0.75f) + (uint32_t)(r > 1.25f) +
                     (uint32_t)(r >= 1.75f) + (uint32_t)(r > 2.5f) + (uint32_t)(r >= 3.5f) +
                     (uint32_t)(r > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

}  // namespace ft
