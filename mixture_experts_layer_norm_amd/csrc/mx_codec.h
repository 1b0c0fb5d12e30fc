// OCP Microscaling v1.0 encoding on the device (E4M3 elements, E8M0 block scale, blocks of 32):
// the MXFP8 format the sparsenotes page "Mixture-of-Kittens: MoE Megakernel for NVL72s" names in
// "The production details". Shared by the dispatch quantiser, the MXFP8 GEMM's SwiGLU epilogue
// and the MXFP8 backward kernels.
#pragma once
#include "common.h"

namespace moe {

// Values already divided by the block scale -> E4M3 codes, round to nearest even (subnormals
// included), saturating at +-448: the clamp (v_med3) then gfx950's packed conversion to OCP E4M3
// (v_cvt_pk_fp8_f32), 2.5 instructions per value where a software encoder took about 15. Four
// values packed little-endian (value i in byte i). A NaN input gives an unspecified code.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const float lo = -448.0f, hi = 448.0f;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, lo, hi), __builtin_amdgcn_fmed3f(b, lo, hi), 0,
                                          false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, lo, hi), __builtin_amdgcn_fmed3f(d, lo, hi), w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const float c = __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false) & 0xffu;
}

// Block scale exponent for a block whose largest magnitude is amax (> 0):
// floor(log2 amax) - 8, clamped to [-127, 127]. fp32 subnormals clamp to -127.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  int eb = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  int se = eb - 127 - 8;
  return se < -127 ? -127 : (se > 127 ? 127 : se);
}

// Quantise 32 fp32 values (one block) into 32 codes packed in 8 words; returns the E8M0 byte.
__device__ __forceinline__ uint32_t mx_block(const float* v, uint32_t* packed) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  if (amax == 0.f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) packed[i] = 0u;
    return 127u;
  }
  const int se = mx_shared_exp(amax);
  const float inv = __uint_as_float((uint32_t)(127 - se) << 23);   // 2^-se, exact
#pragma unroll
  for (int i = 0; i < 8; ++i)
    packed[i] = e4m3_pack4(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv);
  return (uint32_t)(se + 127);
}

// E4M3 code -> value (no NaN codes are produced by the encoder above).
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  const uint32_t e = (code >> 3) & 15u, m = code & 7u;
  const float mag = e == 0 ? (float)m * 0.001953125f                      // m * 2^-9
                           : __uint_as_float(((e + 120u) << 23) | (m << 20));   // (1 + m/8) 2^(e-7)
  return (code & 0x80u) ? -mag : mag;
}

// 2^(byte - 127) for an E8M0 scale byte in [0, 254] (byte 0 is the fp32 subnormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t byte) { return __uint_as_float(byte ? byte << 23 : 0x00400000u); }

}  // namespace moe
