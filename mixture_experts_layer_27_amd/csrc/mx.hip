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
// Elements are converted with v_cvt_pk_fp8_f32 after exact scaling by 2^-X
// (see e4m3_pair).
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
// A fused pass produces the row codes together with the column or token codes
// from one read of the source (weights and permuted activations, which are
// operands along both of their axes).
#include "moe_common.h"
#include "moe_internal.h"
#include "mx_codes.h"

namespace moe {

MOE_DEV void unpack8(u32x4 q, float* v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(q[j] << 16);
    v[2 * j + 1] = __uint_as_float(q[j] & 0xffff0000u);
  }
}

namespace {

// (1) along rows.  One tile = 32 rows x 128 values (four 32-blocks of each
// row); its 512 16-byte chunks are loaded two per thread, all loads first.  Four
// consecutive lanes hold one block: its maximum is reduced across the quad and
// every lane writes its 8 codes.  The tile's scale bytes are gathered in LDS and
// written per row (2 bytes per 64-value step of a row, or 4 bytes per row in the
// plain layout), not one byte per quad.  Scale layouts: plain [rows][K/32]
// (staged == 0, the test hook) or stage-major [K/64][srows][2].  With `offsets`
// the source is a permuted activation: only its offsets[E] rows in use are read,
// and row r of expert e lands at row r - offsets[e] + pad_off[e].
__global__ __launch_bounds__(256) void quantize_rows_kernel(const bf16_t* __restrict__ src, int64_t rows, int64_t K,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                           int64_t srows, int staged,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ expert_of_row,
                                                           const int32_t* __restrict__ pad_off, int E) {
  __shared__ uint8_t sc[32][4];    // [tile row][block of the tile]
  __shared__ int64_t drow[32];     // destination row of each tile row (-1: none)
  const int64_t nr = offsets ? (int64_t)offsets[E] : rows;
  const int64_t ktiles = (K + 127) / 128;
  const int64_t ntiles = ((nr + 31) / 32) * ktiles;
  const int t = threadIdx.x;
  for (int64_t tl = blockIdx.x; tl < ntiles; tl += gridDim.x) {
    const int64_t r0 = (tl / ktiles) * 32, k0 = (tl % ktiles) * 128;
    if (t < 32) {
      const int64_t r = r0 + t;
      int64_t dr = -1;
      if (r < nr) {
        dr = r;
        if (offsets) {
          const int e = expert_of_row[r];
          dr = r - offsets[e] + pad_off[e];
        }
      }
      drow[t] = dr;
    }
    u32x4 raw[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = t + 256 * u;            // row i >> 4, 8-value chunk i & 15
      const int64_t r = r0 + (i >> 4), kk = k0 + (i & 15) * 8;
      raw[u] = (r < nr && kk < K) ? ldg16_nt(src + r * K + kk) : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();                          // drow visible
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = t + 256 * u;
      const int rl = i >> 4, ch = i & 15;
      const int64_t kk = k0 + ch * 8;
      float v[8];
      unpack8(raw[u], v);
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      const int X = mx_exponent(amax);
      const int64_t dr = drow[rl];
      if (dr >= 0 && kk < K) {               // uniform over the quad (K % 32 == 0)
        *reinterpret_cast<uint2*>(codes + dr * K + kk) = e4m3_8(v, pow2f(-X));
        if ((ch & 3) == 0) sc[rl][ch >> 2] = (uint8_t)(X + 127);
      }
    }
    __syncthreads();                          // sc complete
    if (t < 64) {                             // one thread per (row, 64-value step)
      const int rl = t >> 1, s = t & 1;
      const int64_t dr = drow[rl], kb = k0 + 64 * s;   // first value of the step
      if (dr >= 0 && kb < K) {
        const int nb = K - kb >= 64 ? 2 : 1;   // blocks of this step inside K
        if (staged) {
          uint8_t* dst = scales + ((kb >> 6) * srows + dr) * 2;
          if (nb == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(sc[rl][2 * s] | (sc[rl][2 * s + 1] << 8));
          else dst[0] = sc[rl][2 * s];
        } else {
          uint8_t* dst = scales + dr * (K / 32) + (kb >> 5);
          dst[0] = sc[rl][2 * s];
          if (nb == 2) dst[1] = sc[rl][2 * s + 1];
        }
      }
    }
    __syncthreads();                          // sc and drow reused by the next tile
  }
}

// (2)/(3) along the first axis, written transposed.  One block = 128 positions
// of the reduction axis x 64 columns: loaded with 16-byte row reads, staged in
// LDS, and each thread quantises one column over one 32-position block.
//   columns mode (seg_off == nullptr): src [G][R][C]; position p of group g is
//     row p of matrix g; out codes [G][C][R], scales [R/64][G*C][2].
//   tokens mode: src [rows][C] (expert segments given by seg_off), positions are
//     padded tokens: segment e occupies [pad_off[e], pad_off[e+1]) with
//     pad_off[e] a multiple of 64; position p maps to source row
//     seg_off[e] + (p - pad_off[e]) when that is inside the segment, else 0.
//     out codes [C][P], scales [P/64][C][2], P = the padded capacity.
// plain_scales (columns mode, test hook): scales [G*C][R/32] instead.
__global__ __launch_bounds__(256) void quantize_t_kernel(const bf16_t* __restrict__ src, int G, int R, int C,
                                                        const int32_t* __restrict__ seg_off,
                                                        const int32_t* __restrict__ pad_off, int E,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                        int64_t P, int plain_scales,
                                                        const int32_t* __restrict__ gather) {
  __shared__ float tile[128][65];
  const int c0 = blockIdx.x * 64;
  const int64_t p0 = (int64_t)blockIdx.y * 128;
  const int g = blockIdx.z;
  const int64_t len = seg_off ? P : (int64_t)R;
  if (p0 >= (seg_off ? (int64_t)pad_off[E] : (int64_t)R)) return;
  // source row and valid count of each 64-position half
  int64_t base[2], valid[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int64_t ph = p0 + 64 * hh;
    base[hh] = 0;
    valid[hh] = 0;
    if (seg_off) {
      if (ph < pad_off[E]) {
        int lo = 0, hi = E;   // segment holding ph: pad_off[lo] <= ph < pad_off[lo+1]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (pad_off[mid] <= ph) lo = mid; else hi = mid;
        }
        const int64_t into = ph - pad_off[lo];
        base[hh] = seg_off[lo] + into;
        valid[hh] = (int64_t)(seg_off[lo + 1] - seg_off[lo]) - into;
      }
    } else if (ph < R) {
      base[hh] = (int64_t)g * R + ph;
      valid[hh] = 64;
    }
  }
  // 128 rows x 64 columns: 8 threads per row, 16 bytes each; all four loads of a
  // thread are issued before any of them is used
  u32x4 raw[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = threadIdx.x + 256 * u;
    const int rr = i >> 3, ch = i & 7;
    const int hh = rr >> 6, rl = rr & 63;
    const int64_t sr = gather && rl < valid[hh] ? (int64_t)gather[base[hh] + rl] : base[hh] + rl;   // tokens mode
    raw[u] = rl < valid[hh] ? (gather ? ldg16(src + sr * C + c0 + ch * 8) : ldg16_nt(src + sr * C + c0 + ch * 8))
                            : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = threadIdx.x + 256 * u;
    const int rr = i >> 3, ch = i & 7;
    float v[8];
    unpack8(raw[u], v);
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[rr][ch * 8 + j] = v[j];
  }
  __syncthreads();
  // thread -> (column c, 32-position block b); lanes pair up blocks 2m, 2m+1 of one
  // column so the two scale bytes of a 64-position step are written together
  const int t = threadIdx.x;
  const int b = ((t >> 7) << 1) | (t & 1);   // 0..3
  const int c = (t >> 1) & 63;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = tile[b * 32 + i][c];
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const int X = mx_exponent(amax);
  const float inv = pow2f(-X);
  int64_t crow, srows;
  if (seg_off) { crow = c0 + c; srows = C; }
  else { crow = (int64_t)g * C + c0 + c; srows = (int64_t)G * C; }
  const int64_t pb = p0 + b * 32;
  if (pb >= len) return;
  uint8_t* cp = codes + crow * len + pb;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint2 lo = e4m3_8(v + 16 * h, inv), hi2 = e4m3_8(v + 16 * h + 8, inv);
    *reinterpret_cast<u32x4*>(cp + 16 * h) = u32x4{lo.x, lo.y, hi2.x, hi2.y};
  }
  if (plain_scales) scales[crow * (len / 32) + (pb >> 5)] = (uint8_t)(X + 127);
  else scales[((pb >> 6) * srows + crow) * 2 + ((pb >> 5) & 1)] = (uint8_t)(X + 127);
}

// (4) both directions from one read of the source.  A tile of 128 positions x 128
// columns is quantised along its rows (blocks of 32 columns) and along its
// positions (blocks of 32 positions).  Positions as in quantize_t_kernel
// (columns mode: the R rows of each of the G matrices [R][C]; tokens mode: the
// padded tokens of the expert segments, zero past each segment's end).
//   row codes [G*R][C] (columns mode) or [P][C] (tokens mode: row = padded
//     position, padding rows included), stage-major scales [C/64][rsrows][2];
//   position codes [G][C][len], len = R or P, scales [len/64][G*C][2].
// C and the position extent (R, or pad_off[E]) are multiples of 64.  The
// position codes are transposed through LDS so that each store instruction
// writes whole 128-byte lines of the [C][len] layout.
// WIDE: each lane quantises 16 columns of a row and stores their codes in one
// 16-byte store (faster for the activation passes; the weight passes keep
// 8 columns per lane, which measured faster for them).
template <bool WIDE>
__global__ __launch_bounds__(256) void quantize_dual_kernel(const bf16_t* __restrict__ src, int G, int R, int C,
                                                           const int32_t* __restrict__ seg_off,
                                                           const int32_t* __restrict__ pad_off, int E, int64_t P,
                                                           uint8_t* __restrict__ rcodes, uint8_t* __restrict__ rscales,
                                                           int64_t rsrows, uint8_t* __restrict__ tcodes,
                                                           uint8_t* __restrict__ tscales,
                                                           const int32_t* __restrict__ gather) {
  constexpr int VS = 136;   // value tile row stride (bf16 elements; rows stay 16-byte aligned)
  constexpr int CS = 144;   // code tile row stride (bytes): 16 consecutive columns hit distinct banks
  // the code tile takes the value tile's place once every column has been read:
  // 35 KB of LDS per block, four blocks per CU
  __shared__ __attribute__((aligned(16))) uint16_t vt[128 * VS];
  uint8_t* const ct = reinterpret_cast<uint8_t*>(vt);
  static_assert(128 * CS <= 128 * VS * 2, "code tile fits in the value tile");
  __shared__ uint8_t sc[128][4];
  const int t = threadIdx.x;
  const int c0 = blockIdx.x * 128;
  const int64_t p0 = (int64_t)blockIdx.y * 128;
  const int g = blockIdx.z;
  const int64_t len = seg_off ? P : (int64_t)R;
  const int64_t plim = seg_off ? (int64_t)pad_off[E] : (int64_t)R;   // positions in use
  if (p0 >= plim) return;
  int64_t base[2], valid[2];   // source row of each 64-position half, and how many of its rows are real
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int64_t ph = p0 + 64 * hh;
    base[hh] = 0;
    valid[hh] = 0;
    if (ph < plim) {
      if (seg_off) {
        int lo = 0, hi = E;   // segment holding ph: pad_off[lo] <= ph < pad_off[lo+1]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (pad_off[mid] <= ph) lo = mid; else hi = mid;
        }
        const int64_t into = ph - pad_off[lo];
        base[hh] = seg_off[lo] + into;
        valid[hh] = (int64_t)(seg_off[lo + 1] - seg_off[lo]) - into;
      } else {
        base[hh] = (int64_t)g * R + ph;
        valid[hh] = 64;
      }
    }
  }
  if constexpr (WIDE) {
    // 128 rows x 8 pairs of 8-value chunks (32 contiguous bytes per lane), eight
    // 16-byte loads per thread, all issued first
    u32x4 raw[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = t + 256 * v;
      const int rr = i >> 3, cp = i & 7, hh = rr >> 6, rl = rr & 63;
      const int64_t sr = gather && rl < valid[hh] ? (int64_t)gather[base[hh] + rl] : base[hh] + rl;   // tokens mode
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col = c0 + cp * 16 + q * 8;
        const bool ok = rl < valid[hh] && col < C;
        raw[2 * v + q] = ok ? (gather ? ldg16(src + sr * C + col) : ldg16_nt(src + sr * C + col)) : u32x4{0u, 0u, 0u, 0u};
      }
    }
    // along rows: two consecutive lanes hold one 32-column block, each lane 16
    // columns whose codes leave in one 16-byte store
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = t + 256 * v;
      const int rr = i >> 3, cp = i & 7;
      const int col = c0 + cp * 16;
      const int64_t p = p0 + rr;
      *reinterpret_cast<u32x4*>(vt + rr * VS + cp * 16) = raw[2 * v];
      *reinterpret_cast<u32x4*>(vt + rr * VS + cp * 16 + 8) = raw[2 * v + 1];
      float x[16];
      unpack8(raw[2 * v], x);
      unpack8(raw[2 * v + 1], x + 8);
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(x[j]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      const int X = mx_exponent(amax);
      if (p < plim && col < C) {               // uniform over the pair (C is a multiple of 32)
        const int64_t drow = seg_off ? p : (int64_t)g * R + p;
        const float inv = pow2f(-X);
        const uint2 lo = e4m3_8(x, inv), hi = e4m3_8(x + 8, inv);
        *reinterpret_cast<u32x4*>(rcodes + drow * C + col) = u32x4{lo.x, lo.y, hi.x, hi.y};
        if ((cp & 1) == 0) sc[rr][cp >> 1] = (uint8_t)(X + 127);
      }
    }
  } else {
    // 128 rows x 16 chunks of 8 values, eight 16-byte loads per thread, all issued first
    u32x4 raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = t + 256 * u;
      const int rr = i >> 4, ch = i & 15, hh = rr >> 6, rl = rr & 63;
      const int col = c0 + ch * 8;
      const bool ok = rl < valid[hh] && col < C;
      const int64_t sr = gather && ok ? (int64_t)gather[base[hh] + rl] : base[hh] + rl;   // tokens mode
      raw[u] = ok ? (gather ? ldg16(src + sr * C + col) : ldg16_nt(src + sr * C + col)) : u32x4{0u, 0u, 0u, 0u};
    }
    // along rows: four consecutive lanes hold one 32-column block
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = t + 256 * u;
      const int rr = i >> 4, ch = i & 15;
      const int col = c0 + ch * 8;
      const int64_t p = p0 + rr;
      *reinterpret_cast<u32x4*>(vt + rr * VS + ch * 8) = raw[u];
      float v[8];
      unpack8(raw[u], v);
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      const int X = mx_exponent(amax);
      if (p < plim && col < C) {               // uniform over the quad
        const int64_t drow = seg_off ? p : (int64_t)g * R + p;
        *reinterpret_cast<uint2*>(rcodes + drow * C + col) = e4m3_8(v, pow2f(-X));
        if ((ch & 3) == 0) sc[rr][ch >> 2] = (uint8_t)(X + 127);
      }
    }
  }
  __syncthreads();
  {   // row scales: one thread per (row, 64-column step)
    const int rr = t >> 1, s = t & 1;
    const int64_t p = p0 + rr;
    const int kb = c0 + 64 * s;
    if (p < plim && kb < C) {
      const int64_t drow = seg_off ? p : (int64_t)g * R + p;
      *reinterpret_cast<uint16_t*>(rscales + ((int64_t)(kb >> 6) * rsrows + drow) * 2) =
          (uint16_t)(sc[rr][2 * s] | (sc[rr][2 * s + 1] << 8));
    }
  }
  {   // along positions: column c, positions [64h, 64h + 64) = two blocks
    const int c = t & 127, h = t >> 7;
    int Xb[2];
    float v[2][32];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 32; ++i) v[b][i] = __uint_as_float((uint32_t)vt[(64 * h + 32 * b + i) * VS + c] << 16);
    __syncthreads();   // all values are in registers: the code tile may overwrite them
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[b][i]));
      const int X = mx_exponent(amax);
      const float inv = pow2f(-X);
      uint8_t* cp = ct + c * CS + 64 * h + 32 * b;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint2 lo = e4m3_8(v[b] + 16 * q, inv), hi2 = e4m3_8(v[b] + 16 * q + 8, inv);
        *reinterpret_cast<u32x4*>(cp + 16 * q) = u32x4{lo.x, lo.y, hi2.x, hi2.y};
      }
      Xb[b] = X;
    }
    const int64_t pb = p0 + 64 * h;
    const int col = c0 + c;
    if (pb < plim && col < C) {
      const int64_t crow = seg_off ? col : (int64_t)g * C + col;
      const int64_t srows = seg_off ? C : (int64_t)G * C;
      *reinterpret_cast<uint16_t*>(tscales + ((pb >> 6) * srows + crow) * 2) =
          (uint16_t)((Xb[0] + 127) | ((Xb[1] + 127) << 8));
    }
  }
  __syncthreads();
  // position codes out: 8 lanes per column, 16 bytes each
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = t + 256 * u;
    const int c = i >> 3, ch = i & 7;
    const int col = c0 + c;
    const int64_t p = p0 + ch * 16;
    if (col < C && p < plim) {
      const int64_t crow = seg_off ? col : (int64_t)g * C + col;
      *reinterpret_cast<u32x4*>(tcodes + crow * len + p) = *reinterpret_cast<const u32x4*>(ct + c * CS + ch * 16);
    }
  }
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

int qgrid(int64_t threads) {
  int64_t g = (threads + 255) / 256;
  if (g > 16384) g = 16384;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

// one block per 32-row x 128-value tile (grid-strided past 16384 tiles)
int rows_grid(int64_t rows, int64_t K) { return qgrid(((rows + 31) / 32) * ((K + 127) / 128) * 256); }

hipError_t launch_quantize_rows(const void* src, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                hipStream_t st) {
  hipLaunchKernelGGL(quantize_rows_kernel, dim3(rows_grid(rows, cols)), dim3(256), 0, st, (const bf16_t*)src,
                     rows, cols, codes, scales, (int64_t)0, 0, (const int32_t*)nullptr, (const int32_t*)nullptr,
                     (const int32_t*)nullptr, 0);
  return hipGetLastError();
}

hipError_t mx_quantize_rows_staged(const void* src, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                                   int64_t srows, hipStream_t st) {
  hipLaunchKernelGGL(quantize_rows_kernel, dim3(rows_grid(rows, K)), dim3(256), 0, st, (const bf16_t*)src, rows,
                     K, codes, scales, srows, 1, (const int32_t*)nullptr, (const int32_t*)nullptr,
                     (const int32_t*)nullptr, 0);
  return hipGetLastError();
}

hipError_t mx_quantize_rows_padded(const void* src, int64_t rows, int64_t K, const int32_t* offsets,
                                   const int32_t* expert_of_row, const int32_t* pad_off, int E, uint8_t* codes,
                                   uint8_t* scales, int64_t srows, hipStream_t st) {
  hipLaunchKernelGGL(quantize_rows_kernel, dim3(rows_grid(rows, K)), dim3(256), 0, st, (const bf16_t*)src, rows,
                     K, codes, scales, srows, 1, offsets, expert_of_row, pad_off, E);
  return hipGetLastError();
}

hipError_t mx_quantize_cols(const void* src, int G, int R, int C, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  hipLaunchKernelGGL(quantize_t_kernel, dim3(C / 64, (R + 127) / 128, G), dim3(256), 0, st, (const bf16_t*)src, G, R, C,
                     (const int32_t*)nullptr, (const int32_t*)nullptr, 0, codes, scales, (int64_t)0, 0,
                     (const int32_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_quantize_cols_plain(const void* src, int R, int C, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  hipLaunchKernelGGL(quantize_t_kernel, dim3(C / 64, (R + 127) / 128, 1), dim3(256), 0, st, (const bf16_t*)src, 1, R,
                     C, (const int32_t*)nullptr, (const int32_t*)nullptr, 0, codes, scales, (int64_t)0, 1,
                     (const int32_t*)nullptr);
  return hipGetLastError();
}

hipError_t mx_quantize_tokens(const void* src, int C, const int32_t* seg_off, const int32_t* pad_off, int E,
                              int64_t P, uint8_t* codes, uint8_t* scales, hipStream_t st, const int32_t* gather) {
  hipLaunchKernelGGL(quantize_t_kernel, dim3(C / 64, (unsigned)((P + 127) / 128), 1), dim3(256), 0, st, (const bf16_t*)src, 1,
                     0, C, seg_off, pad_off, E, codes, scales, P, 0, gather);
  return hipGetLastError();
}

hipError_t mx_quantize_dual(const void* src, int G, int R, int C, const int32_t* seg_off, const int32_t* pad_off,
                            int E, int64_t P, const MxOperand& rows, const MxOperand& pos, hipStream_t st,
                            const int32_t* gather) {
  const int64_t len = seg_off ? P : (int64_t)R;
  auto kern = seg_off ? quantize_dual_kernel<true> : quantize_dual_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((C + 127) / 128, (unsigned)((len + 127) / 128), G), dim3(256), 0, st,
                     (const bf16_t*)src, G, R, C, seg_off, pad_off, E, P, rows.codes, rows.scales, rows.srows,
                     pos.codes, pos.scales, gather);
  return hipGetLastError();
}

hipError_t mx_pad_offsets(const int32_t* offsets, int E, int32_t* pad_off, hipStream_t st) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(256), 0, st, offsets, E, pad_off);
  return hipGetLastError();
}

}  // namespace moe
