// MXFP8 element and scale encoding shared by the quantisers and the GEMM
// epilogues that quantise their own outputs (OCP Microscaling v1.0 rules:
// shared exponent floor(log2 amax) - 8, clamped to [-127, 127], -127 for an
// all-zero block; elements rounded to nearest-even E4M3, saturating at 448).
#pragma once
#include "moe_common.h"

// Shared exponent of a block with largest magnitude amax (bits of a float).
MOE_DEV int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  int X = ilogbf(amax) - 8;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// E4M3 codes of v0, v1 * 2^-X (exact scaling), packed into bytes 0-1 of the
// result.  v_cvt_pk_fp8_f32 rounds to nearest even into the OCP E4M3 format;
// clamping to +-448 first gives the saturating rule (values >= 464 would
// otherwise round past the largest finite code).  Checked against the rule on
// every finite bf16 input.
MOE_DEV uint32_t e4m3_pair(float v0, float v1, float inv_scale) {
  const float a = fminf(fmaxf(v0 * inv_scale, -448.0f), 448.0f);
  const float b = fminf(fmaxf(v1 * inv_scale, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}
MOE_DEV float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }   // 2^e, -126 <= e <= 127

// 8 values (one 16-byte bf16 chunk) -> 8 codes
MOE_DEV uint2 e4m3_8(const float* v, float inv) {
  return uint2{e4m3_pair(v[0], v[1], inv) | (e4m3_pair(v[2], v[3], inv) << 16),
               e4m3_pair(v[4], v[5], inv) | (e4m3_pair(v[6], v[7], inv) << 16)};
}

// Block maximum over the four lanes of an aligned quad (each holding 8 of the
// block's 32 values).  Call from uniform control flow.
MOE_DEV float quad_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1, 64));
  return fmaxf(v, __shfl_xor(v, 2, 64));
}
