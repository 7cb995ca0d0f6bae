// MXFP8 version of the register-staged 256 x 256 grouped GEMM (gemm_big.h):
// the same eight waves of 128 x 64, tile kinds, decode, LDS double buffer and
// epilogues, with E4M3 operands and one E8M0 scale per 32 K values.
//
// A stage holds 128 bytes of K per tile row, i.e. 128 fp8 values = two steps of
// v_mfma_scale_f32_32x32x64_f8f6f4, so the operand bytes per stage and the LDS
// layout (128-byte rows, chunk c of row r at slot c ^ ((r >> 1) & 7)) are those
// of the bf16 kernel while each stage carries twice the flops.  For MFMA step s
// of a stage, lane r + 32 g of a fragment holds row r: 16-byte chunks 4 s + g
// and 4 s + 2 + g of the stage, and the scale of 32-block g of that step (the
// instruction's lane layout, see gemm_mx.h).
//
// Scales are not staged in LDS (a 128 x 512 tile already fills it): every lane
// loads the scale bytes of its own fragment rows straight from the stage-major
// arrays [K/64][srows][2] -- per stage and MFMA step one byte per fragment; the
// 32 rows x 2 blocks of one fragment are 64 consecutive bytes, one segment per
// load instruction.  They are fetched one stage ahead.
//
// K extents are multiples of 64 (activation widths, and 64-aligned token
// segments for the weight gradients); when a tile's K holds an odd number of
// 64-steps the second step of its last stage is skipped, so bytes past the
// extent (the next row or the next expert's tokens) never reach an MFMA.
#pragma once
#include "gemm_big.h"
#include "gemm_mx.h"

namespace moe_gemm {

template <int BM, int BN, int WM, int WN, int GROUP, int EPI>
MOE_DEV void mx_big_tile(const Args& args, const MxArgs& mx, const TileCtx& ctx, char* smem) {
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int NT = WM * WN * 64;
  static_assert(NT == kBigThreads && WTM == 128 && WTN == 64, "eight waves of 128 x 64");
  constexpr int SB = 128;                          // K bytes (fp8 values) per stage
  constexpr int ASZ = BM * SB, BSZ = BN * SB, STAGE = ASZ + BSZ;
  const int e = ctx.e, nt = ctx.nt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 5;
  const char* Ab = reinterpret_cast<const char*>(args.A) + (int64_t)e * args.a_estride;
  const char* Bb = reinterpret_cast<const char*>(args.B) + (int64_t)e * args.b_estride;

  // operand row of A tile row r, and how many tile rows are valid
  int64_t a_row0 = 0;
  int a_rows = 0;
  if constexpr (GROUP == GROUP_M) {
    a_row0 = ctx.row_begin + (int64_t)mx.a_pad[e] - args.offsets[e];   // expert-padded rows
    a_rows = min(BM, ctx.row_end - ctx.row_begin);
  } else {
    a_row0 = ctx.m0;
    a_rows = min(BM, args.M - ctx.m0);
  }
  // row of B (inside this expert's matrix) of tile column row; -1 when absent
  auto b_row = [&](int row) -> int {
    int j = ctx.n0 + row;
    if constexpr (EPI == EPI_SWIGLU_MX) {
      const int w = row / WTN, jj = row % WTN;
      const int gg = nt * (BN / 2) + w * (WTN / 2) + (jj % (WTN / 2));
      j = gg >= args.f ? -1 : (jj < WTN / 2) ? gg : (args.f + gg);
    }
    return j < args.N ? j : -1;
  };
  const int64_t k0 = (GROUP == GROUP_K) ? ctx.k_begin : 0;   // first K byte of the tile
  const int kext = (GROUP == GROUP_M) ? args.K : (ctx.k_end - ctx.k_begin);
  const int nsteps = kext > 0 ? (kext + 63) / 64 : 0;        // MFMA steps
  const int nk = (nsteps + 1) / 2;                           // stages

  RegOperand<BM, true, NT> ra;
  RegOperand<BN, true, NT> rb;
  {
    const int64_t rowb = args.lda;
    ra.base = Ab + a_row0 * rowb + k0;
    ra.step = SB;
    ra.num0 = (int64_t)a_rows * rowb - k0;    // rows >= a_rows start past it
    ra.init_kc([&](int r) -> int64_t { return (int64_t)r * rowb; });
  }
  {
    const int64_t rowb = args.ldb;
    rb.base = Bb + k0;
    rb.step = SB;
    rb.num0 = (int64_t)args.N * rowb - k0;
    rb.init_kc([&](int row) -> int64_t {
      const int j = b_row(row);
      return (int64_t)(j < 0 ? args.N : j) * rowb;   // absent rows lie past num0
    });
  }

  // scale bytes: per fragment one byte per MFMA step, fetched a stage ahead.
  // args.K is the full K extent of the scale arrays (the token capacity P for
  // the weight gradients); each step's [srows][2] block is its own buffer, empty
  // for steps past the extent.
  const int64_t step0 = k0 / 64;                  // global 64-step index of the tile's first step
  const int64_t ksteps = args.K / 64;
  uint32_t soa[TM], sob[TN];                      // byte offset of (fragment row, block g) in a step's block
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = wm * WTM + i * 32 + (lane & 31);
    const int64_t row = a_row0 + (r < a_rows ? r : 0);
    soa[i] = (uint32_t)(row * 2 + g);
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int jr = b_row(wn * WTN + j * 32 + (lane & 31));
    const int64_t row = (int64_t)e * mx.b_erows + (jr < 0 ? 0 : jr);
    sob[j] = (uint32_t)(row * 2 + g);
  }
  auto load_scales = [&](int kt, int (&sa)[2][TM], int (&sb)[2][TN]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t st = step0 + 2 * kt + s;
      const bool in = st < ksteps;
      const __amdgpu_buffer_rsrc_t ra_s =
          make_rsrc(mx.a_scale + (in ? st : 0) * mx.a_srows * 2, in ? (uint32_t)(mx.a_srows * 2) : 0u);
      const __amdgpu_buffer_rsrc_t rb_s =
          make_rsrc(mx.b_scale + (in ? st : 0) * mx.b_srows * 2, in ? (uint32_t)(mx.b_srows * 2) : 0u);
#pragma unroll
      for (int i = 0; i < TM; ++i) sa[s][i] = __builtin_amdgcn_raw_buffer_load_b8(ra_s, (int)soa[i], 0, 0);
#pragma unroll
      for (int j = 0; j < TN; ++j) sb[s][j] = __builtin_amdgcn_raw_buffer_load_b8(rb_s, (int)sob[j], 0, 0);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  auto frag = [&](const char* base, int row, int s) -> i32x8 {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + kc_offk<64>(row, 4 * s + g));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + kc_offk<64>(row, 4 * s + 2 + g));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  // TMV: the wave's 32-row sub-tiles that hold rows of the segment; the others
  // skip their fragment reads and MFMAs (zero accumulators, never stored).
  auto run_loop = [&](auto tmv_c) {
  constexpr int TMV = decltype(tmv_c)::value;
  auto step = [&](const char* as, int s, const int (&sa)[TM], const int (&sb)[TN]) {
    const char* bs = as + ASZ;
    i32x8 af[TM], bf[TN];
#pragma unroll
    for (int i = 0; i < TMV; ++i) af[i] = frag(as, wm * WTM + i * 32 + (lane & 31), s);
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = frag(bs, wn * WTN + j * 32 + (lane & 31), s);
#pragma unroll
    for (int i = 0; i < TMV; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
  };

  int sa[2][TM], sb[2][TN], na[2][TM], nb[2][TN];
  if (nk > 0) {
    ra.load(0); rb.load(0);
    load_scales(0, sa, sb);
    ra.store(smem); rb.store(smem + ASZ);
    ra.load(1); rb.load(1);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    cta_barrier();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const char* as = smem + (kt & 1) * STAGE;
    char* an = smem + ((kt + 1) & 1) * STAGE;   // the next stage, written during this one
    load_scales(kt + 1, na, nb);                // past the extent: out of range, zero
    ra.store(an); rb.store(an + ASZ);
    ra.load(kt + 2); rb.load(kt + 2);
    step(as, 0, sa[0], sb[0]);
    if (2 * kt + 1 < nsteps) step(as, 1, sa[1], sb[1]);
    __builtin_amdgcn_s_waitcnt(0xc07f);          // this wave's fragment reads and stage writes are done
    cta_barrier();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < TM; ++i) sa[s][i] = na[s][i];
#pragma unroll
      for (int j = 0; j < TN; ++j) sb[s][j] = nb[s][j];
    }
  }
  };
  if constexpr (GROUP == GROUP_M && EPI != EPI_DSWIGLU_MX) {   // (the dA' epilogue leaves no registers for it)
    const int valid = a_rows - wm * WTM;   // >= 1 by the tile decode
    if (valid > 96) run_loop(std::integral_constant<int, 4>{});
    else if (valid > 64) run_loop(std::integral_constant<int, 3>{});
    else if (valid > 32) run_loop(std::integral_constant<int, 2>{});
    else run_loop(std::integral_constant<int, 1>{});
  } else {
    run_loop(std::integral_constant<int, TM>{});
  }
  wave_epilogue<BM, BN, WM, WN, GROUP, EPI>(args, ctx, acc, smem);
}

// Row-segment (GROUP_M) GEMMs; the tile body also supports GROUP_K (A and B
// rows over token positions, args.K = the token capacity of the scale arrays).
template <int GROUP, int EPI>
__global__ __launch_bounds__(kBigThreads) void grouped_gemm_mx_big(Args args, MxArgs mx) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  static_assert(GROUP == GROUP_M || GROUP == GROUP_K, "grouped GEMMs only");
  TileCtx ctx;
  if constexpr (GROUP == GROUP_K) {
    if (!decode_tile<256, 256, kBigBK, GROUP_K>(args, ctx)) return;
    mx_big_tile<256, 256, 2, 4, GROUP, EPI>(args, mx, ctx, smem);
  } else {
    bool wide = false;
    if (!big_decode_m(args, blockIdx.x, ctx, &wide)) return;
    if (wide) mx_big_tile<128, 512, 1, 8, GROUP, EPI>(args, mx, ctx, smem);
    else mx_big_tile<256, 256, 2, 4, GROUP, EPI>(args, mx, ctx, smem);
  }
}

}  // namespace moe_gemm
