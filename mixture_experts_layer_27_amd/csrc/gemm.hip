// Launchers of the grouped GEMMs of the MoE layer (forward, backward, router).
//
// Expert FFN = SwiGLU without biases (h = W1_e x with W1_e = [W_gate; W_up],
// a = silu(h_gate) * h_up, y = W2_e a).  The per-expert loop of the "Beam"
// blog's MoELayer (section 5.3) becomes one grouped launch per GEMM ("grouped
// GEMM" of the Olmo-core 3 article, "three splits" section): tiles are
// scheduled per expert segment from device-resident offsets, so no routing
// metadata ever returns to the host.
//
// Backward (SonicMoE article, section 1): dA' = dO_perm W2_e is never stored;
// its epilogue recomputes A from the saved H, reduces dS = <dA', A> per row,
// and emits dH (SwiGLU backward) and gA = g * A for the W2 gradient.
#include <atomic>

#include "gemm_big.h"
#include "gemm_dma.h"
#include "gemm_engine.h"
#include "moe_internal.h"

namespace moe {
using namespace moe_gemm;

namespace {

template <typename T, int BM, int BN, int WM, int WN, bool AKC, bool BKC, int GROUP, int EPI>
hipError_t run(const Args& a, int64_t logical_tiles, hipStream_t st) {
  auto kern = grouped_gemm<T, BM, BN, WM, WN, AKC, BKC, GROUP, EPI>;
  constexpr size_t lds = lds_bytes<T, BM, BN, WM, WN>();
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = 8 * ((logical_tiles + 7) / 8);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WM * WN * 64), lds, st, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, bool AKC, bool BKC, int GROUP, int EPI, int S = 4>
hipError_t run_dma(const Args& a, int64_t logical_tiles, hipStream_t st) {
  auto kern = grouped_gemm_dma<BM, BN, WM, WN, AKC, BKC, GROUP, EPI, S>;
  constexpr size_t lds = dma_lds_bytes<BM, BN, WM, WN, S>();
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = 8 * ((logical_tiles + 7) / 8);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WM * WN * 64), lds, st, a);
  return hipGetLastError();
}

template <bool AKC, bool BKC, int GROUP, int EPI, int GATHER = 0>
hipError_t run_big(const Args& a, int64_t logical_tiles, hipStream_t st) {
  auto kern = grouped_gemm_big<AKC, BKC, GROUP, EPI, GATHER>;
  const size_t lds = big_lds_bytes(GROUP == GROUP_M);   // GROUP_M may run 128 x 512 tiles
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t grid = 8 * ((logical_tiles + 7) / 8);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBigThreads), lds, st, a);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Persistent weight-gradient launch: one block per CU (its LDS admits no second),
// a multiple of 8 so every block stays on its XCD's chunks.
template <bool AKC, bool BKC, int EPI, int GATHER = 0>
hipError_t run_wgrad_big(const Args& a, int64_t logical_tiles, hipStream_t st) {
  auto kern = grouped_wgrad_big<AKC, BKC, EPI, GATHER>;
  constexpr size_t lds = big_wgrad_lds_bytes();
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t need = 8 * ((logical_tiles + 7) / 8);
  const int64_t cap = 8 * (int64_t)(device_cus() / 8 > 0 ? device_cus() / 8 : 1);
  const int64_t grid = need < cap ? need : cap;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBigThreads), lds, st, a);
  return hipGetLastError();
}

// Persistent row-segment launch (bf16 output): one block per CU, as above.  It
// pays once a CU has many tiles to walk (sparse_e256: 72 logical tiles per CU,
// down 1573 -> 1516 us, dX 2296 -> 2264 us); with about 10 per CU (fine_e128)
// the static walk cannot even out tiles of unequal length and it loses 2-5%.
bool use_rows_walk(int64_t logical_tiles) { return logical_tiles >= 32 * (int64_t)device_cus(); }
template <bool AKC, bool BKC, int EPI, int GATHER = 0>
hipError_t run_rows_big(const Args& a, int64_t logical_tiles, hipStream_t st) {
  auto kern = grouped_rows_big<AKC, BKC, EPI, GATHER>;
  constexpr size_t lds = big_rows_lds_bytes();
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t need = 8 * ((logical_tiles + 7) / 8);
  const int64_t cap = 8 * (int64_t)(device_cus() / 8 > 0 ? device_cus() / 8 : 1);
  const int64_t grid = need < cap ? need : cap;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBigThreads), lds, st, a);
  return hipGetLastError();
}

// The 256 x 256 register-staged kernel pays a longer unoverlapped epilogue per
// tile (one block per CU); it wins when the reduction is deep enough (from
// K = 512: GEMM2 at d_ff = 512 takes 1618 instead of 1750 us).
bool use_big(int K) { return K >= 512; }

Args base_args() {
  Args a{};
  a.ksplit = 1;
  return a;
}

int64_t grouped_m_tiles(const moe_shape& s, int bm) { return (max_rows(s) + bm - 1) / bm + s.E; }

}  // namespace

// ---------------------------------------------------------------- forward

// x_rows = x_perm, or (gather != nullptr) x [T, d] read through gather = token_of_row
hipError_t gemm_up_swiglu(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const void* x_rows,
                          const int32_t* gather, const void* w1, void* h, void* act, hipStream_t st) {
  Args a = base_args();
  a.A = x_rows; a.lda = s.d;
  a.a_gather = gather; a.gather_rows = s.T;
  a.B = w1; a.ldb = s.d; a.b_estride = (int64_t)2 * s.d_ff * s.d;
  a.C = h; a.ldc = 2 * s.d_ff;
  a.C2 = act; a.ldc2 = s.d_ff;
  a.offsets = p.offsets;
  a.N = 2 * s.d_ff; a.K = s.d; a.E = s.E; a.f = s.d_ff;
  if (s.act == MOE_BF16) {
    a.tile_prefix = pi.prefix128; a.tile_expert = pi.tile_e128;
    if (use_big(a.K)) {
      const int64_t tiles = grouped_m_tiles(s, 128) * ceil_div(a.N, 512);
      return gather ? run_big<true, true, GROUP_M, EPI_SWIGLU, 1>(a, tiles, st)
                    : run_big<true, true, GROUP_M, EPI_SWIGLU>(a, tiles, st);
    }
    a.tilesN = a.N / 256;
    return run_dma<128, 256, 2, 4, true, true, GROUP_M, EPI_SWIGLU, 3>(a, grouped_m_tiles(s, 128) * a.tilesN, st);
  }
  a.tile_prefix = pi.prefix128; a.tile_expert = pi.tile_e128; a.tilesN = a.N / 128;
  return run<float, 128, 128, 2, 2, true, true, GROUP_M, EPI_SWIGLU>(a, grouped_m_tiles(s, 128) * a.tilesN, st);
}

hipError_t gemm_down(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const void* act,
                     const void* w2, void* y, hipStream_t st) {
  Args a = base_args();
  a.A = act; a.lda = s.d_ff;
  a.B = w2; a.ldb = s.d_ff; a.b_estride = (int64_t)s.d * s.d_ff;
  a.C = y; a.ldc = s.d;
  a.offsets = p.offsets;
  a.N = s.d; a.K = s.d_ff; a.E = s.E; a.f = s.d_ff;
  if (s.act == MOE_BF16) {
    a.tile_prefix = pi.prefix128; a.tile_expert = pi.tile_e128;
    if (use_big(a.K)) {
      const int64_t tiles = grouped_m_tiles(s, 128) * ceil_div(a.N, 512);
      return use_rows_walk(tiles) ? run_rows_big<true, true, EPI_ACT>(a, tiles, st)
                                  : run_big<true, true, GROUP_M, EPI_ACT>(a, tiles, st);
    }
    a.tilesN = ceil_div(a.N, 256);
    return run_dma<128, 256, 2, 4, true, true, GROUP_M, EPI_ACT, 3>(a, grouped_m_tiles(s, 128) * a.tilesN, st);
  }
  a.tile_prefix = pi.prefix128; a.tile_expert = pi.tile_e128; a.tilesN = ceil_div(a.N, 128);
  return run<float, 128, 128, 2, 2, true, true, GROUP_M, EPI_ACT>(a, grouped_m_tiles(s, 128) * a.tilesN, st);
}

// GEMM2 with the combine's first half in its epilogue (bf16): row r of A W2^T is
// scaled by its gate and stored at row pos[r] of yg (the token-ordered rows of
// the plan's tok_rows), so the rows a token sums are contiguous.
hipError_t gemm_down_gate_scatter(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const void* act,
                                  const void* w2, const int32_t* pos, void* yg, hipStream_t st) {
  Args a = base_args();
  a.A = act; a.lda = s.d_ff;
  a.B = w2; a.ldb = s.d_ff; a.b_estride = (int64_t)s.d * s.d_ff;
  a.C = yg; a.ldc = s.d; a.c_rows = pos;
  a.row_gate = p.gate_of_row;
  a.offsets = p.offsets;
  a.N = s.d; a.K = s.d_ff; a.E = s.E; a.f = s.d_ff;
  a.tile_prefix = pi.prefix128; a.tile_expert = pi.tile_e128;
  if (use_big(a.K)) {
    const int64_t tiles = grouped_m_tiles(s, 128) * ceil_div(a.N, 512);
    return use_rows_walk(tiles) ? run_rows_big<true, true, EPI_GATE_SCATTER>(a, tiles, st)
                                : run_big<true, true, GROUP_M, EPI_GATE_SCATTER>(a, tiles, st);
  }
  a.tilesN = ceil_div(a.N, 256);
  return run_dma<128, 256, 2, 4, true, true, GROUP_M, EPI_GATE_SCATTER, 3>(a, grouped_m_tiles(s, 128) * a.tilesN, st);
}

// ---------------------------------------------------------------- backward

// dS partial sums per row: one per (column tile, wave column) on the bf16 path,
// one per column tile on the fp32 path
int gemm_dact_parts(const moe_shape& s) {
  if (s.act != MOE_BF16) return ceil_div(s.d_ff, 128);
  // 64-column wave tiles: over ceil(f / 512) 512-column quanta (the 256 x 256
  // kernels: bf16 with deep K, MXFP8 always), or over 256-column tiles (bf16
  // with shallow K)
  if (s.gemm == MOE_MXFP8 || use_big(s.d)) return ceil_div(s.d_ff, 512) * 8;
  return ceil_div(s.d_ff, 256) * 4;
}

hipError_t gemm_dact(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const void* do_rows,
                     const int32_t* gather, const void* w2, const void* h, void* dh, void* ga, float* ds_part,
                     hipStream_t st) {
  Args a = base_args();
  a.A = do_rows; a.lda = s.d;
  a.a_gather = gather; a.gather_rows = s.T;
  a.B = w2; a.ldb = s.d_ff; a.b_estride = (int64_t)s.d * s.d_ff;   // W2_e read as [K = d, N = f]
  a.C = dh; a.ldc = 2 * s.d_ff;
  a.C2 = ga; a.ldc2 = s.d_ff;
  a.C3 = ds_part; a.ldc3 = max_rows(s);
  a.aux = h; a.ld_aux = 2 * s.d_ff;
  a.row_gate = p.gate_of_row;
  a.offsets = p.offsets;
  a.N = s.d_ff; a.K = s.d; a.E = s.E; a.f = s.d_ff;
  if (s.act == MOE_BF16) {
    a.tile_prefix = pi.prefix128; a.tile_expert = pi.tile_e128;
    if (use_big(a.K)) {
      const int64_t tiles = grouped_m_tiles(s, 128) * ceil_div(a.N, 512);
      return gather ? run_big<true, false, GROUP_M, EPI_DSWIGLU, 1>(a, tiles, st)
                    : run_big<true, false, GROUP_M, EPI_DSWIGLU>(a, tiles, st);
    }
    a.tilesN = ceil_div(a.N, 256);
    return run_dma<128, 256, 2, 4, true, false, GROUP_M, EPI_DSWIGLU, 3>(a, grouped_m_tiles(s, 128) * a.tilesN, st);
  }
  a.tile_prefix = pi.prefix128; a.tile_expert = pi.tile_e128; a.tilesN = ceil_div(a.N, 128);
  return run<float, 128, 128, 2, 2, true, false, GROUP_M, EPI_DSWIGLU>(a, grouped_m_tiles(s, 128) * a.tilesN, st);
}

hipError_t gemm_dx_perm(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const void* dh,
                        const void* w1, void* dx_perm, hipStream_t st) {
  Args a = base_args();
  a.A = dh; a.lda = 2 * s.d_ff;
  a.B = w1; a.ldb = s.d; a.b_estride = (int64_t)2 * s.d_ff * s.d;    // W1_e read as [K = 2f, N = d]
  a.C = dx_perm; a.ldc = s.d;
  a.offsets = p.offsets;
  a.N = s.d; a.K = 2 * s.d_ff; a.E = s.E; a.f = s.d_ff;
  if (s.act == MOE_BF16) {
    a.tile_prefix = pi.prefix128; a.tile_expert = pi.tile_e128;
    if (use_big(a.K)) {
      const int64_t tiles = grouped_m_tiles(s, 128) * ceil_div(a.N, 512);
      return use_rows_walk(tiles) ? run_rows_big<true, false, EPI_ACT>(a, tiles, st)
                                  : run_big<true, false, GROUP_M, EPI_ACT>(a, tiles, st);
    }
    a.tilesN = ceil_div(a.N, 256);
    return run_dma<128, 256, 2, 4, true, false, GROUP_M, EPI_ACT, 3>(a, grouped_m_tiles(s, 128) * a.tilesN, st);
  }
  a.tile_prefix = pi.prefix128; a.tile_expert = pi.tile_e128; a.tilesN = ceil_div(a.N, 128);
  return run<float, 128, 128, 2, 2, true, false, GROUP_M, EPI_ACT>(a, grouped_m_tiles(s, 128) * a.tilesN, st);
}

// dW1_e [2f, d] = dH_e^T X_perm_e and dW2_e [d, f] = dO_perm_e^T gA_e: the
// reduction runs over the expert's rows (variable K, cut into chunks of at most
// w.kch rows), fp32 outputs; chunks past an expert's first land in partial
// slots that launch_wgrad_reduce adds afterwards.
namespace {
hipError_t run_wgrad(const moe_shape& s, const WgradChunks& w, Args& a, hipStream_t st) {
  a.chunks = w.chunks; a.nchunks = w.nchunks; a.Cpart = w.part;
  if (s.act == MOE_BF16) {
    a.tilesM = ceil_div(a.M, 256); a.tilesN = ceil_div(a.N, 256);
    const int64_t tiles = 8 * (int64_t)ceil_div(w.max_chunks, 8) * a.tilesM * a.tilesN;
    if (a.a_gather) return run_wgrad_big<false, false, EPI_F32, 1>(a, tiles, st);
    if (a.b_gather) return run_wgrad_big<false, false, EPI_F32, 2>(a, tiles, st);
    return run_wgrad_big<false, false, EPI_F32>(a, tiles, st);
  }
  if (a.a_gather || a.b_gather) return hipErrorNotSupported;   // gathered k rows: bf16 kernels only
  a.tilesM = ceil_div(a.M, 128); a.tilesN = ceil_div(a.N, 128);
  const int64_t tiles = 8 * (int64_t)ceil_div(w.max_chunks, 8) * a.tilesM * a.tilesN;
  return run<float, 128, 128, 2, 2, false, false, GROUP_K, EPI_F32>(a, tiles, st);
}
}  // namespace

hipError_t gemm_dw1(const moe_shape& s, const WgradChunks& w, const void* dh, const void* x_rows, const int32_t* gather,
                    float* dw1, hipStream_t st) {
  Args a = base_args();
  a.A = dh; a.lda = 2 * s.d_ff;          // [K = rows, M = 2f]
  a.B = x_rows; a.ldb = s.d;             // [K = rows, N = d]: x_perm, or x read through gather
  a.b_gather = gather; a.gather_rows = s.T;
  a.C = dw1; a.ldc = s.d; a.c_estride = (int64_t)2 * s.d_ff * s.d;
  a.M = 2 * s.d_ff; a.N = s.d; a.E = s.E;
  return run_wgrad(s, w, a, st);
}

hipError_t gemm_dw2(const moe_shape& s, const WgradChunks& w, const void* do_rows, const int32_t* gather,
                    const void* ga, float* dw2, hipStream_t st) {
  Args a = base_args();
  a.A = do_rows; a.lda = s.d;            // [K = rows, M = d]: dO_perm, or dout read through gather
  a.a_gather = gather; a.gather_rows = s.T;
  a.B = ga; a.ldb = s.d_ff;              // [K = rows, N = f]
  a.C = dw2; a.ldc = s.d_ff; a.c_estride = (int64_t)s.d * s.d_ff;
  a.M = s.d; a.N = s.d_ff; a.E = s.E;
  return run_wgrad(s, w, a, st);
}

// ---------------------------------------------------------------- router

hipError_t gemm_router_logits(const moe_shape& s, const void* x, const void* wg, const float* bias,
                              const float* noise, float* logits, hipStream_t st) {
  Args a = base_args();
  a.A = x; a.lda = s.d;
  a.B = wg; a.ldb = s.d;
  a.C = logits; a.ldc = s.E;
  a.bias = bias;
  a.aux = noise; a.ld_aux = s.E;         // routing noise [T, E] or nullptr
  a.M = s.T; a.N = s.E; a.K = s.d;
  // 32-row tiles: T/32 blocks keep every CU busy with two of them (the K loop is
  // latency-bound at this width); all E columns in one tile read each x row once.
  a.tilesM = ceil_div(s.T, 32);
  if (s.act == MOE_BF16 && s.E % 256 == 0 && s.d % 32 == 0 &&
      (int64_t)ceil_div(s.T, 128) * (s.E / 256) >= device_cus()) {
    // 128 x 256 tiles on the DMA main loop: a quarter of the operand bytes per
    // flop of 32 x 128 tiles, worth it once every CU gets a tile (sparse_e256:
    // 104 instead of 196 us); with fewer tiles the 32-row tiles fill the chip
    a.tilesM = ceil_div(s.T, 128);
    a.tilesN = s.E / 256;
    a.total_static = a.tilesM * a.tilesN;
    return run_dma<128, 256, 2, 4, true, true, GROUP_NONE, EPI_LOGITS, 3>(a, a.total_static, st);
  }
  if (s.act == MOE_BF16) {
    if (s.E > 64) {
      a.tilesN = ceil_div(s.E, 128);
      a.total_static = a.tilesM * a.tilesN;
      return run<bf16_t, 32, 128, 1, 4, true, true, GROUP_NONE, EPI_LOGITS>(a, a.total_static, st);
    }
    a.tilesN = 1;
    a.total_static = a.tilesM;
    return run<bf16_t, 32, 64, 1, 2, true, true, GROUP_NONE, EPI_LOGITS>(a, a.total_static, st);
  }
  a.tilesM = ceil_div(s.T, 128); a.tilesN = ceil_div(s.E, 64);
  a.total_static = a.tilesM * a.tilesN;
  return run<float, 128, 64, 4, 1, true, true, GROUP_NONE, EPI_LOGITS>(a, a.total_static, st);
}

// Dense router term of the input gradient: dxr = dzq W, K = the dz columns (with
// bf16 activations dz and its residual against W_g twice, so dxr = dz W_g to
// 16 significant bits of dz).
hipError_t gemm_router_dx_dense(const moe_shape& s, const void* dzq, const void* wg, float* dxr, hipStream_t st) {
  Args a = base_args();
  a.A = dzq; a.lda = router_dz_ld(s);    // [T, K]
  a.B = wg; a.ldb = s.d;                 // [K, N = d]
  a.C = dxr; a.ldc = s.d;
  a.M = s.T; a.N = s.d; a.K = router_dz_rows(s);
  a.tilesM = ceil_div(s.T, 128); a.tilesN = ceil_div(s.d, 128);
  a.total_static = a.tilesM * a.tilesN;
  if (s.act == MOE_BF16) return run<bf16_t, 128, 128, 2, 2, true, false, GROUP_NONE, EPI_F32>(a, a.total_static, st);
  return run<float, 128, 128, 2, 2, true, false, GROUP_NONE, EPI_F32>(a, a.total_static, st);
}

// dW_g on the persistent 256 x 256 weight-gradient kernel: both operands are
// token-major like the expert weight gradients.  Used when the tiles of the
// chunks fill the 256 CUs with chunks of at least 1024 token rows
// (sparse_e256: 2 x 16 tiles x 8 chunks of 4096 rows); otherwise 128 x 128
// split-K tiles.
namespace {
int router_dwg_big_splits(const moe_shape& s) {
  const int M = router_dz_rows(s);
  if (s.act != MOE_BF16 || M % 256 != 0 || s.d % 256 != 0) return 0;
  const int pe = (M / 256) * (s.d / 256);
  const int sp = ceil_div(256, pe);
  if ((int64_t)sp * 1024 > s.T) return 0;
  return sp;
}
}  // namespace

int gemm_router_dwg_splits(const moe_shape& s) {
  if (const int big = router_dwg_big_splits(s)) return big;
  const int tiles = ceil_div(router_dz_rows(s), 128) * ceil_div(s.d, 128);
  int sp = ceil_div(512, tiles);
  const int maxsp = ceil_div(s.T, 256);
  if (sp > maxsp) sp = maxsp;
  if (sp < 1) sp = 1;
  return sp;
}

// dW_g partials: part[split] [router_dz_rows, d] = dzq[K-slice]^T x[K-slice]; the
// reduction adds the dz rows and (bf16) their residual rows
hipError_t gemm_router_dwg(const moe_shape& s, const void* dzq, const void* x, float* part, hipStream_t st) {
  Args a = base_args();
  a.A = dzq; a.lda = router_dz_ld(s);    // [K = T, M]
  a.B = x; a.ldb = s.d;                  // [K = T, N = d]
  a.M = router_dz_rows(s); a.N = s.d; a.K = s.T;
  a.C = part; a.ldc = s.d; a.c_kstride = (int64_t)a.M * s.d;
  a.ksplit = gemm_router_dwg_splits(s);
  if (router_dwg_big_splits(s)) {
    a.tilesM = a.M / 256; a.tilesN = s.d / 256;
    a.Cpart = part + a.c_kstride; a.c_estride = a.c_kstride;   // chunk q > 0: slot q - 1 = part[q]
    return run_wgrad_big<false, false, EPI_F32>(a, 8 * (int64_t)ceil_div(a.ksplit, 8) * a.tilesM * a.tilesN, st);
  }
  a.tilesM = ceil_div(a.M, 128); a.tilesN = ceil_div(s.d, 128);
  a.total_static = a.tilesM * a.tilesN * a.ksplit;
  if (s.act == MOE_BF16) return run<bf16_t, 128, 128, 2, 2, false, false, GROUP_NONE, EPI_F32>(a, a.total_static, st);
  return run<float, 128, 128, 2, 2, false, false, GROUP_NONE, EPI_F32>(a, a.total_static, st);
}

}  // namespace moe
