// MXFP8 quantisers (OCP Microscaling v1.0 rules; the pages only name the MXFP8
// format -- Olmo-core 3 article, "three splits" section, and the SonicMoE
// article's closing section).
//
// Block = 32 consecutive values along the GEMM's reduction axis.  Shared
// exponent X = floor(log2 amax) - 8 (8 = largest E4M3 exponent), clamped to
// [-127, 127]; -127 for an all-zero block.  Scale byte = X + 127.  Element =
// v * 2^-X rounded to nearest-even E4M3 (bias 7, 3 mantissa bits, subnormal
// quantum 2^-9, largest 448), saturating; the element byte keeps the sign bit of
// v.  Every step is exact in fp32, so codes do not depend on evaluation order.
//
// Layouts produced for the MX grouped GEMMs (every operand K-contiguous):
//  * codes [rows][K] (u8), K = the reduction axis;
//  * "stage-major" scales [K/64][srows][2]: the two block scales of 64
//    consecutive K values of one row are adjacent, and one 64-wide K step of
//    consecutive rows is contiguous (one DMA per GEMM stage).
// Three producers: rows (reduction along a row), columns (reduction along the
// first axis of [G][R][C] matrices, written transposed: weights for the
// backward GEMMs), and tokens (reduction along the token axis of each expert's
// row segment, written transposed [C][padded tokens] with every segment
// starting at a multiple of 64 and zero-padded: the weight-gradient GEMMs).
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

// quantise 32 floats (one block) into 8 dwords of codes; returns the scale byte
MOE_DEV uint32_t mx_block(const float* v, uint32_t* ow) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int X = mx_exponent(amax);
#pragma unroll
  for (int w = 0; w < 8; ++w)
    ow[w] = e4m3_code(v[4 * w], X) | (e4m3_code(v[4 * w + 1], X) << 8) | (e4m3_code(v[4 * w + 2], X) << 16) |
            (e4m3_code(v[4 * w + 3], X) << 24);
  return (uint32_t)(X + 127);
}

namespace {

// (1) along rows: one thread per 32-block of a row-major [rows, K] bf16 matrix.
// Scale layouts: plain [rows][K/32] (staged == 0, the test hook) or stage-major.
// With `offsets` the source is a permuted activation: only its offsets[E] rows
// in use are read, and row r of expert e lands at row r - offsets[e] + pad_off[e].
__global__ __launch_bounds__(256) void quantize_rows_kernel(const bf16_t* __restrict__ src, int64_t rows, int64_t K,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                           int64_t srows, int staged,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ expert_of_row,
                                                           const int32_t* __restrict__ pad_off, int E) {
  const int64_t nb = K / 32;
  const int64_t nr = offsets ? (int64_t)offsets[E] : rows;
  const int64_t total = nr * nb;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < total; b += (int64_t)gridDim.x * 256) {
    const int64_t r = b / nb, c = b - r * nb;
    const bf16_t* p = src + r * K + c * 32;
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 q = ldg16(p + 8 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(q[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(q[j] & 0xffff0000u);
      }
    }
    uint32_t ow[8];
    const uint32_t sc = mx_block(v, ow);
    int64_t dr = r;
    if (offsets) {
      const int e = expert_of_row[r];
      dr = r - offsets[e] + pad_off[e];
    }
    uint8_t* cp = codes + dr * K + c * 32;
    stg16(cp, u32x4{ow[0], ow[1], ow[2], ow[3]});
    stg16(cp + 16, u32x4{ow[4], ow[5], ow[6], ow[7]});
    if (staged) scales[((c >> 1) * srows + dr) * 2 + (c & 1)] = (uint8_t)sc;
    else scales[dr * nb + c] = (uint8_t)sc;
  }
}

// (2)/(3) along the first axis, written transposed.  One block = 64 positions of
// the reduction axis x 64 columns, staged through LDS.
//   columns mode (tok_off == nullptr): src [G][R][C]; position p of group g is
//     row p of matrix g; out codes [G][C][R], scales [R/64][G*C][2].
//   tokens mode: src [rows][C] (expert segments given by seg_off), positions are
//     padded tokens: segment e occupies [pad_off[e], pad_off[e+1]) with
//     pad_off[e] a multiple of 64; position p maps to source row
//     seg_off[e] + (p - pad_off[e]) when that is inside the segment, else 0.
//     out codes [C][P], scales [P/64][C][2], P = the padded capacity.
__global__ __launch_bounds__(128) void quantize_t_kernel(const bf16_t* __restrict__ src, int G, int R, int C,
                                                        const int32_t* __restrict__ seg_off,
                                                        const int32_t* __restrict__ pad_off, int E,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                        int64_t P) {
  __shared__ float tile[64][65];
  const int ct = blockIdx.x;            // column tile
  const int pt = blockIdx.y;            // position tile (64 positions)
  const int g = blockIdx.z;
  const int c0 = ct * 64;
  const int64_t p0 = (int64_t)pt * 64;
  int e = 0;
  int64_t src_base = 0, valid = 64;
  if (seg_off) {
    if (p0 >= pad_off[E]) return;
    int lo = 0, hi = E;                 // segment holding p0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pad_off[mid] <= p0) lo = mid; else hi = mid;
    }
    e = lo;
    const int64_t into = p0 - pad_off[e];
    src_base = seg_off[e] + into;
    valid = (int64_t)(seg_off[e + 1] - seg_off[e]) - into;
  } else {
    src_base = (int64_t)g * R + p0;
  }
  // load 64 rows x 64 columns (bf16) into LDS as floats
  for (int i = threadIdx.x; i < 64 * 8; i += 128) {
    const int rr = i >> 3, ch = i & 7;
    float v[8];
    if (rr < valid) {
      u32x4 q = ldg16(src + (src_base + rr) * C + c0 + ch * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(q[j] << 16);
        v[2 * j + 1] = __uint_as_float(q[j] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[rr][ch * 8 + j] = v[j];
  }
  __syncthreads();
  const int c = threadIdx.x & 63, b = threadIdx.x >> 6;   // column, 32-block inside the 64 positions
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = tile[b * 32 + i][c];
  uint32_t ow[8];
  const uint32_t sc = mx_block(v, ow);
  int64_t crow, srows;
  if (seg_off) { crow = c0 + c; srows = C; }
  else { crow = (int64_t)g * C + c0 + c; srows = (int64_t)G * C; }
  const int64_t len = seg_off ? P : (int64_t)R;
  uint8_t* cp = codes + crow * len + p0 + b * 32;
  stg16(cp, u32x4{ow[0], ow[1], ow[2], ow[3]});
  stg16(cp + 16, u32x4{ow[4], ow[5], ow[6], ow[7]});
  scales[((p0 >> 6) * srows + crow) * 2 + b] = (uint8_t)sc;
}

// pad_off[e] = sum over experts j < e of count_j rounded up to 64 (E <= 256)
__global__ __launch_bounds__(256) void pad_offsets_kernel(const int32_t* __restrict__ offsets, int E,
                                                         int32_t* __restrict__ pad_off) {
  __shared__ int32_t buf[256];
  const int i = threadIdx.x;
  const int v = i < E ? (offsets[i + 1] - offsets[i] + 63) / 64 * 64 : 0;
  buf[i] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int add = i >= o ? buf[i - o] : 0;
    __syncthreads();
    buf[i] += add;
    __syncthreads();
  }
  if (i < E) pad_off[i + 1] = buf[i];
  if (i == 0) pad_off[0] = 0;
}

int qgrid(int64_t blocks) {
  int64_t g = (blocks + 255) / 256;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

hipError_t launch_quantize_rows(const void* src, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                hipStream_t st) {
  hipLaunchKernelGGL(quantize_rows_kernel, dim3(qgrid(rows * (cols / 32))), dim3(256), 0, st, (const bf16_t*)src,
                     rows, cols, codes, scales, (int64_t)0, 0, (const int32_t*)nullptr, (const int32_t*)nullptr,
                     (const int32_t*)nullptr, 0);
  return hipGetLastError();
}

hipError_t mx_quantize_rows_staged(const void* src, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                                   int64_t srows, hipStream_t st) {
  hipLaunchKernelGGL(quantize_rows_kernel, dim3(qgrid(rows * (K / 32))), dim3(256), 0, st, (const bf16_t*)src, rows,
                     K, codes, scales, srows, 1, (const int32_t*)nullptr, (const int32_t*)nullptr,
                     (const int32_t*)nullptr, 0);
  return hipGetLastError();
}

hipError_t mx_quantize_rows_padded(const void* src, int64_t rows, int64_t K, const int32_t* offsets,
                                   const int32_t* expert_of_row, const int32_t* pad_off, int E, uint8_t* codes,
                                   uint8_t* scales, int64_t srows, hipStream_t st) {
  hipLaunchKernelGGL(quantize_rows_kernel, dim3(qgrid(rows * (K / 32))), dim3(256), 0, st, (const bf16_t*)src, rows,
                     K, codes, scales, srows, 1, offsets, expert_of_row, pad_off, E);
  return hipGetLastError();
}

hipError_t mx_quantize_cols(const void* src, int G, int R, int C, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  hipLaunchKernelGGL(quantize_t_kernel, dim3(C / 64, R / 64, G), dim3(128), 0, st, (const bf16_t*)src, G, R, C,
                     (const int32_t*)nullptr, (const int32_t*)nullptr, 0, codes, scales, (int64_t)0);
  return hipGetLastError();
}

hipError_t mx_quantize_tokens(const void* src, int C, const int32_t* seg_off, const int32_t* pad_off, int E,
                              int64_t P, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  hipLaunchKernelGGL(quantize_t_kernel, dim3(C / 64, (unsigned)(P / 64), 1), dim3(128), 0, st, (const bf16_t*)src, 1,
                     0, C, seg_off, pad_off, E, codes, scales, P);
  return hipGetLastError();
}

hipError_t mx_pad_offsets(const int32_t* offsets, int E, int32_t* pad_off, hipStream_t st) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(256), 0, st, offsets, E, pad_off);
  return hipGetLastError();
}

}  // namespace moe
