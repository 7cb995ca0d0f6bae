// MXFP8 quantiser (OCP Microscaling v1.0 rules; the pages only name the MXFP8
// format -- Olmo-core 3 article, "three splits" section).
//
// Block = 32 consecutive values of a row.  Shared exponent X = floor(log2 amax)
// - 8 (8 = largest E4M3 exponent), clamped to [-127, 127]; -127 for an all-zero
// block.  Scale byte = X + 127.  Element = v * 2^-X rounded to nearest-even E4M3
// (bias 7, 3 mantissa bits, subnormal quantum 2^-9, largest 448), saturating;
// the element byte keeps the sign bit of v.  All steps are exact in fp32, so
// the codes do not depend on evaluation order.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

MOE_DEV uint32_t e4m3_code(float v, int X) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
  float s = ldexpf(fabsf(v), -X);
  float r;
  if (s >= 0.015625f) {                       // 2^-6: normal range
    int e = ilogbf(s);
    float q = ldexpf(1.0f, e - 3);
    r = rintf(s / q) * q;
  } else {
    r = rintf(s * 512.0f) * (1.0f / 512.0f);  // subnormal quantum 2^-9
  }
  r = fminf(r, 448.0f);
  uint32_t code;
  if (r == 0.0f) code = 0;
  else if (r < 0.015625f) code = (uint32_t)(r * 512.0f);
  else {
    int e = ilogbf(r);
    uint32_t m = (uint32_t)((ldexpf(r, -e) - 1.0f) * 8.0f);
    code = ((uint32_t)(e + 7) << 3) | m;
  }
  return sign | code;
}

MOE_DEV int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  int X = ilogbf(amax) - 8;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

namespace {

// One thread per 32-value block of a row-major [rows, cols] bf16 matrix.
__global__ __launch_bounds__(256) void quantize_rows_kernel(const bf16_t* __restrict__ src, int64_t rows, int64_t cols,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t nb = cols / 32;
  const int64_t total = rows * nb;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < total; b += (int64_t)gridDim.x * 256) {
    const int64_t r = b / nb, c = b - r * nb;
    const bf16_t* p = src + r * cols + c * 32;
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ldg16(p + 8 * i);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        amax = fmaxf(amax, fabsf(__uint_as_float(v[i][j] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(v[i][j] & 0xffff0000u)));
      }
    const int X = mx_exponent(amax);
    uint32_t ow[8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; j += 2) {               // two dwords of source -> one dword of codes
        uint32_t c0 = e4m3_code(__uint_as_float(v[i][j] << 16), X);
        uint32_t c1 = e4m3_code(__uint_as_float(v[i][j] & 0xffff0000u), X);
        uint32_t c2 = e4m3_code(__uint_as_float(v[i][j + 1] << 16), X);
        uint32_t c3 = e4m3_code(__uint_as_float(v[i][j + 1] & 0xffff0000u), X);
        ow[i * 2 + j / 2] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
      }
    uint8_t* cp = codes + r * cols + c * 32;
    stg16(cp, u32x4{ow[0], ow[1], ow[2], ow[3]});
    stg16(cp + 16, u32x4{ow[4], ow[5], ow[6], ow[7]});
    scales[r * nb + c] = (uint8_t)(X + 127);
  }
}

}  // namespace

hipError_t launch_quantize_rows(const void* src, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                hipStream_t st) {
  const int64_t blocks = rows * (cols / 32);
  int64_t g = (blocks + 255) / 256;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)g), dim3(256), 0, st, (const bf16_t*)src, rows, cols, codes,
                     scales);
  return hipGetLastError();
}

}  // namespace moe
