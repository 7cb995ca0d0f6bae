// MXFP8 grouped GEMM for gfx950: v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3,
// one E8M0 scale per 32 K values of every row/column, fp32 accumulation).
//
// Operands are pre-quantised and K-contiguous (see mx.hip); the pipeline is the
// one of gemm_dma.h with 64 fp8 of K per stage (one MFMA K step), 64-byte tile
// rows with the same swizzle, and a 1 KiB scale block per stage:
//   [0, 2*BM)            A scales, tile row r -> bytes 2r (K block 0), 2r+1 (block 1)
//   [2*BM, 2*BM + 2*BN)  B scales
// fetched by one DMA instruction of wave 0 from the stage-major scale arrays.
//
// Operand lane layout of the instruction (measured with an in-bounds probe):
// lane l = r + 32 g holds row/column r; its bytes 0-15 are K values 16 g..16 g+15
// of the step (first 32-block) and bytes 16-31 are K values 32+16 g..47+16 g
// (second block); its scale operand is the scale of block g of row/column r.
// So lane l reads 16-byte chunks g and 2+g of its row and scale byte g.
// Scale rows are fetched in 16-byte chunks (eight rows of one 64-wide K step),
// which must start on 16-byte boundaries: every scale array has a multiple of 8
// rows and every tile's first scale row is a multiple of 8.
#pragma once
#include "gemm_dma.h"

namespace moe_gemm {

struct MxArgs {
  const uint8_t* a_scale;   // [K/64][a_srows][2], a_srows >= 8
  int64_t a_srows;
  // grouped-M GEMMs: the A operand holds the segment of expert e from row
  // a_pad[e] (a multiple of 64) instead of offsets[e], so that the scale rows of
  // a tile start on a 16-byte boundary
  const int32_t* a_pad;
  const uint8_t* b_scale;   // [K/64][b_srows][2]; scale row of B row j of expert e = e * b_erows + j
  int64_t b_srows;
  int64_t b_erows;
};

// DMA sources of one fp8 operand tile (ROWS rows x 64 bytes).
template <int ROWS, int NW>
struct DmaBytes {
  static constexpr int Q = ROWS / 16 / NW;
  static_assert(Q >= 1 && (ROWS / 16) % NW == 0, "tile rows must split over the waves");
  const uint8_t* src[Q];
  int q0;
  template <class RowFn>
  MOE_DEV void init(RowFn rowfn, int wave, int lane) {
    q0 = wave * Q;
#pragma unroll
    for (int u = 0; u < Q; ++u) {
      const int row = (q0 + u) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ kc_h(row);
      src[u] = rowfn(row) + c * 16;
    }
  }
  MOE_DEV void issue(char* tile, int64_t k0) const {
#pragma unroll
    for (int u = 0; u < Q; ++u) dma16(src[u] + k0, tile + (q0 + u) * 1024);
  }
};

template <int BM, int BN, int WM, int WN, int GROUP, int EPI, int S>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_mx(Args args, MxArgs mx) {
  constexpr int NW = WM * WN;
  constexpr int BK = 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int ASZ = BM * 64, BSZ = BN * 64, SCZ = 1024, STAGE = ASZ + BSZ + SCZ;
  static_assert(2 * (BM + BN) <= SCZ && BM % 8 == 0 && BN % 8 == 0, "scale block");
  static_assert(S >= 2 && S <= 4, "ring depth");
  static_assert(GROUP != GROUP_NONE, "grouped GEMMs only");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  TileCtx ctx;
  if (!decode_tile<BM, BN, BK, GROUP>(args, ctx)) return;
  const int e = ctx.e, nt = ctx.nt;
  const int row_begin = ctx.row_begin, row_end = ctx.row_end;
  const int k_begin = ctx.k_begin, k_end = ctx.k_end;
  const int m0 = ctx.m0, n0 = ctx.n0;
  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(args.A) + (int64_t)e * args.a_estride;
  const uint8_t* Bb = reinterpret_cast<const uint8_t*>(args.B) + (int64_t)e * args.b_estride;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // A operand row of output row g (grouped M): g + a_shift
  int64_t a_shift = 0;
  if constexpr (GROUP == GROUP_M) a_shift = (int64_t)mx.a_pad[e] - args.offsets[e];
  // row (of the operand array) of A tile row `row`
  auto a_grow = [&](int row) -> int64_t {
    if constexpr (GROUP == GROUP_M) {
      int g = row_begin + row;
      return (g < row_end ? g : row_end - 1) + a_shift;   // rows past the segment only feed unstored outputs
    } else {
      int g = m0 + row;
      return g < args.M ? g : args.M - 1;
    }
  };
  auto b_jrow = [&](int row) -> int64_t {   // row inside this expert's B matrix
    if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_MX) {
      const int w = row / WTN, jj = row % WTN;
      const int g = nt * (BN / 2) + w * (WTN / 2) + (jj % (WTN / 2));
      return (jj < WTN / 2) ? g : (args.f + g);
    } else {
      const int j = n0 + row;
      return j < args.N ? j : args.N - 1;
    }
  };
  DmaBytes<BM, NW> da;
  DmaBytes<BN, NW> db;
  da.init([&](int row) { return Ab + a_grow(row) * args.lda; }, wave, lane);
  db.init([&](int row) { return Bb + b_jrow(row) * args.ldb; }, wave, lane);

  // scale DMA (wave 0): lane i < BM/8 fetches the scales of A tile rows 8i..8i+7,
  // the next BN/8 lanes those of B, the rest a zero block.  Eight consecutive tile
  // rows always map to eight consecutive operand rows (runs are >= 32 rows); a
  // chunk that starts past the last row is moved back inside the array, since
  // such rows only feed outputs that are never stored.
  const uint8_t* sc_src = reinterpret_cast<const uint8_t*>(g_dma_zero);
  int64_t sc_srows = 0;
  if (lane < BM / 8) {
    int64_t r = (GROUP == GROUP_M ? row_begin + a_shift : (int64_t)m0) + lane * 8;
    if (r > mx.a_srows - 8) r = mx.a_srows - 8;
    sc_src = mx.a_scale + r * 2;
    sc_srows = mx.a_srows;
  } else if (lane < BM / 8 + BN / 8) {
    const int row = (lane - BM / 8) * 8;
    int64_t j;
    if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_MX) {
      j = b_jrow(row);
    } else {
      j = n0 + row;
      if (j > args.N - 8) j = args.N - 8;
    }
    sc_src = mx.b_scale + ((int64_t)e * mx.b_erows + j) * 2;
    sc_srows = mx.b_srows;
  }

  auto issue = [&](int kt) {
    char* st = smem + (kt % S) * STAGE;
    const int64_t k0 = k_begin + (int64_t)kt * BK;
    da.issue(st, k0);
    db.issue(st + ASZ, k0);
    if (wave == 0) {
      const void* g = sc_srows ? (const void*)(sc_src + (k0 / 64) * sc_srows * 2) : (const void*)sc_src;
      dma16(g, st + ASZ + BSZ);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  constexpr int LPS = DmaBytes<BM, NW>::Q + DmaBytes<BN, NW>::Q;
  const int nk = (k_end > k_begin) ? (k_end - k_begin + BK - 1) / BK : 0;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s);

  const int g = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int ahead = min(S - 2, nk - 1 - kt);
    if (wave == 0) {
      if (S >= 4 && ahead >= 2) wait_vm_lgkm0<2 * (LPS + 1)>();
      else if (S >= 3 && ahead >= 1) wait_vm_lgkm0<LPS + 1>();
      else wait_vm_lgkm0<0>();
    } else {
      if (S >= 4 && ahead >= 2) wait_vm_lgkm0<2 * LPS>();
      else if (S >= 3 && ahead >= 1) wait_vm_lgkm0<LPS>();
      else wait_vm_lgkm0<0>();
    }
    cta_barrier();
    if (kt + S - 1 < nk) issue(kt + S - 1);
    const char* as = smem + (kt % S) * STAGE;
    const char* bs = as + ASZ;
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(bs + BSZ);
    i32x8 af[TM], bfr[TN];
    int sa[TM], sb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * WTM + i * 32 + (lane & 31);
      const u32x4 lo = *reinterpret_cast<const u32x4*>(as + kc_off(row, g));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(as + kc_off(row, 2 + g));
      af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      sa[i] = sc[row * 2 + g];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = wn * WTN + j * 32 + (lane & 31);
      const u32x4 lo = *reinterpret_cast<const u32x4*>(bs + kc_off(row, g));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(bs + kc_off(row, 2 + g));
      bfr[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      sb[j] = sc[2 * BM + row * 2 + g];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
  }
  __syncthreads();
  wave_epilogue<BM, BN, WM, WN, GROUP, EPI>(args, ctx, acc, smem);
}

template <int BM, int BN, int WM, int WN, int S>
constexpr size_t mx_lds_bytes() {
  constexpr size_t ring = (size_t)S * ((BM + BN) * 64 + 1024);
  constexpr size_t epi = (size_t)WM * WN * 32 * (BN / WN + 8) * 4;
  return ring > epi ? ring : epi;
}

}  // namespace moe_gemm
