// Launchers of the MXFP8 expert GEMMs (the three splits of the Olmo-core 3
// article, "three splits" section, with their operands in MXFP8).
//
// Every operand is quantised along the reduction axis of its GEMM (mx.hip):
//   forward   H  = X_perm W1_e^T   : X_perm rows along d,   W1_e rows along d
//             Y  = A W2_e^T        : A rows along f,        W2_e rows along f
//   backward  dA'= dO_perm W2_e    : dO_perm rows along d,  W2_e columns along d
//             dX_perm = dH W1_e    : dH rows along 2f,      W1_e columns along 2f
//             dW1_e = dH^T X_perm  : both along the expert's tokens
//             dW2_e = dO^T gA      : both along the expert's tokens
// The epilogues (SwiGLU, its backward with dS, plain stores) are the bf16 ones.
#include "gemm_mx_big.h"
#include "moe_internal.h"

namespace moe {
using namespace moe_gemm;

namespace {

// Row-segment GEMMs: 256 x 256 register-staged tiles (128 x 512 for odd
// segment tails), eight waves.  Weight gradients: the 128 x 256 LDS-DMA kernel,
// whose two blocks per CU overlap one tile's fp32 stores with the other's MFMAs
// (716 us vs 619 us for dW1 at fine_e128 on the 256 x 256 kernel).
template <int GROUP, int EPI>
hipError_t run_mx(const Args& a, const MxArgs& m, int64_t logical_tiles, hipStream_t st) {
  auto kern = grouped_gemm_mx_big<GROUP, EPI>;
  const size_t lds = big_lds_bytes(GROUP == GROUP_M);
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t grid = 8 * ((logical_tiles + 7) / 8);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBigThreads), lds, st, a, m);
  return hipGetLastError();
}

template <int GROUP, int EPI, int S = 3>
hipError_t run_mx_dma(const Args& a, const MxArgs& m, int64_t logical_tiles, hipStream_t st) {
  auto kern = grouped_gemm_mx<128, 256, 2, 4, GROUP, EPI, S>;
  constexpr size_t lds = mx_lds_bytes<128, 256, 2, 4, S>();
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = 8 * ((logical_tiles + 7) / 8);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, st, a, m);
  return hipGetLastError();
}

Args base_args() {
  Args a{};
  a.ksplit = 1;
  return a;
}

int64_t m_tiles(const moe_shape& s) { return (max_rows(s) + 127) / 128 + s.E; }   // 128-row units

}  // namespace

hipError_t gemm_mx_up_swiglu(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const MxOperand& x,
                             const MxOperand& w1, void* h, const MxOperand& act, hipStream_t st) {
  Args a = base_args();
  a.A = x.codes; a.lda = s.d;
  a.B = w1.codes; a.ldb = s.d; a.b_estride = (int64_t)2 * s.d_ff * s.d;
  a.C = h; a.ldc = 2 * s.d_ff;
  // A is only needed as the down GEMM's operand: the epilogue writes it in MXFP8
  a.q_codes = act.codes; a.q_scales = act.scales; a.q_ld = s.d_ff; a.q_srows = act.srows; a.q_pad = act.pad;
  a.offsets = p.offsets;
  a.N = 2 * s.d_ff; a.K = s.d; a.E = s.E; a.f = s.d_ff;
  a.tile_prefix = pi.prefix128; a.tile_expert = pi.tile_e128;
  MxArgs m{x.scales, x.srows, x.pad, w1.scales, w1.srows, 2 * (int64_t)s.d_ff};
  return run_mx<GROUP_M, EPI_SWIGLU_MX>(a, m, m_tiles(s) * ceil_div(a.N, 512), st);
}

hipError_t gemm_mx_down(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const MxOperand& act,
                        const MxOperand& w2, void* y, hipStream_t st) {
  Args a = base_args();
  a.A = act.codes; a.lda = s.d_ff;
  a.B = w2.codes; a.ldb = s.d_ff; a.b_estride = (int64_t)s.d * s.d_ff;
  a.C = y; a.ldc = s.d;
  a.offsets = p.offsets;
  a.N = s.d; a.K = s.d_ff; a.E = s.E; a.f = s.d_ff;
  a.tile_prefix = pi.prefix128; a.tile_expert = pi.tile_e128;
  MxArgs m{act.scales, act.srows, act.pad, w2.scales, w2.srows, (int64_t)s.d};
  return run_mx<GROUP_M, EPI_ACT>(a, m, m_tiles(s) * ceil_div(a.N, 512), st);
}

// w2t: W2 quantised along d, stored [E][f][d]
hipError_t gemm_mx_dact(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const MxOperand& dout,
                        const MxOperand& w2t, const void* h, const MxOperand& dhq, const MxOperand& dh_t,
                        const MxOperand& ga_t, int64_t P, float* ds_part, hipStream_t st) {
  Args a = base_args();
  a.A = dout.codes; a.lda = s.d;
  a.B = w2t.codes; a.ldb = s.d; a.b_estride = (int64_t)s.d_ff * s.d;
  a.ldc = 2 * s.d_ff; a.ldc2 = s.d_ff;   // dH and gA exist only as codes (no bf16 copies)
  a.C3 = ds_part; a.ldc3 = max_rows(s);
  a.aux = h; a.ld_aux = 2 * s.d_ff;
  a.row_gate = p.gate_of_row;
  a.offsets = p.offsets;
  a.N = s.d_ff; a.K = s.d; a.E = s.E; a.f = s.d_ff;
  a.tile_prefix = pi.prefix128; a.tile_expert = pi.tile_e128;
  // dH in MXFP8 along 2f for the dX_perm GEMM, dH and gA along tokens for the weight gradients
  a.q_codes = dhq.codes; a.q_scales = dhq.scales; a.q_ld = 2 * s.d_ff; a.q_srows = dhq.srows; a.q_pad = dhq.pad;
  a.t_codes = dh_t.codes; a.t_scales = dh_t.scales; a.t2_codes = ga_t.codes; a.t2_scales = ga_t.scales;
  a.t_len = P;
  MxArgs m{dout.scales, dout.srows, dout.pad, w2t.scales, w2t.srows, (int64_t)s.d_ff};
  return run_mx<GROUP_M, EPI_DSWIGLU_MX>(a, m, m_tiles(s) * ceil_div(a.N, 512), st);
}

// w1t: W1 quantised along 2f, stored [E][d][2f]
hipError_t gemm_mx_dx_perm(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const MxOperand& dh,
                           const MxOperand& w1t, void* dx_perm, hipStream_t st) {
  Args a = base_args();
  a.A = dh.codes; a.lda = 2 * s.d_ff;
  a.B = w1t.codes; a.ldb = 2 * s.d_ff; a.b_estride = (int64_t)s.d * 2 * s.d_ff;
  a.C = dx_perm; a.ldc = s.d;
  a.offsets = p.offsets;
  a.N = s.d; a.K = 2 * s.d_ff; a.E = s.E; a.f = s.d_ff;
  a.tile_prefix = pi.prefix128; a.tile_expert = pi.tile_e128;
  MxArgs m{dh.scales, dh.srows, dh.pad, w1t.scales, w1t.srows, (int64_t)s.d};
  return run_mx<GROUP_M, EPI_ACT>(a, m, m_tiles(s) * ceil_div(a.N, 512), st);
}

// dW_e [M, N] = sum over the expert's (64-padded) token positions of lhs x rhs;
// lhs codes [M][P], rhs codes [N][P], both quantised along the token axis.  The
// positions are cut into chunks (w, built from the padded offsets) as in the
// bf16 weight gradients.
hipError_t gemm_mx_wgrad(const moe_shape& s, const WgradChunks& w, int64_t P, const MxOperand& lhs, int M,
                         const MxOperand& rhs, int N, float* dw, hipStream_t st) {
  Args a = base_args();
  a.A = lhs.codes; a.lda = P;
  a.B = rhs.codes; a.ldb = P;
  a.C = dw; a.ldc = N; a.c_estride = (int64_t)M * N;
  a.chunks = w.chunks; a.nchunks = w.nchunks; a.Cpart = w.part;
  a.M = M; a.N = N; a.E = s.E;
  a.tilesM = ceil_div(M, 128); a.tilesN = ceil_div(N, 256);
  const int64_t tiles = 8 * (int64_t)ceil_div(w.max_chunks, 8) * a.tilesM * a.tilesN;
  MxArgs m{lhs.scales, lhs.srows, nullptr, rhs.scales, rhs.srows, 0};
  return run_mx_dma<GROUP_K, EPI_F32>(a, m, tiles, st);
}

}  // namespace moe
