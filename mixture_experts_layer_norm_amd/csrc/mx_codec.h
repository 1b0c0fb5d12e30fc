// OCP Microscaling v1.0 encoding on the device (E4M3 elements, E8M0 block scale, blocks of 32):
// the MXFP8 format the sparsenotes page "Mixture-of-Kittens: MoE Megakernel for NVL72s" names in
// "The production details". Shared by the dispatch quantiser, the MXFP8 GEMM's SwiGLU epilogue
// and the MXFP8 backward kernels.
#pragma once
#include "common.h"

namespace moe {

// |v| already divided by the block scale -> E4M3 code, round to nearest even, saturate at 448
// (NaN and infinities saturate too). Branch-free: both candidate codes are formed and one is
// selected, so a wavefront quantising a block takes no divergent branches.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  const uint32_t ua = __float_as_uint(a);
  // normal range (a >= 2^-6): keep 3 mantissa bits, round to nearest even, rebias 127 -> 7, cap
  // at 0x7e (448); a >= 2^-6 gives r >= 121 << 3, so the subtraction does not wrap there
  const uint32_t r = (ua + 0x7ffffu + ((ua >> 20) & 1u)) >> 20;
  const uint32_t cn = min(r - ((127u - 7u) << 3), 0x7eu);
  // below 2^-6: multiples of 2^-9 (8, i.e. 2^-6 itself, is also the first normal code)
  const uint32_t cs = (uint32_t)rintf(fminf(a, 0.015625f) * 512.0f);
  const uint32_t c = a < 0.015625f ? cs : cn;
  return sign | (a < 448.0f ? c : 0x7eu);
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
  for (int i = 0; i < 8; ++i) {
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) w |= e4m3_code(v[4 * i + b] * inv) << (8 * b);
    packed[i] = w;
  }
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
