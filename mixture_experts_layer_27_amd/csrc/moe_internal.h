// Internal declarations shared by the host-side translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kPlanBlock = 256;     // tokens per block in the plan kernels
constexpr int kLossTokens = 64;     // tokens per block of the router-loss partial sums
constexpr int kBmSmall = 128;       // m-tile of the fp32 grouped GEMMs
constexpr int kBmLarge = 256;       // m-tile of the bf16 grouped GEMMs

// Internal region of the plan blob (plan.sched points at its start):
//   [0, E+1)            m-tile prefix for BM = 128
//   tile_e [max_rows/128 + E]  expert of each 128-row m-tile
//   hist [E * nblk]     per-(expert, token block) counts, then bases after the scan
//   blk_tok [nblk + 1]  rows per token block, then its exclusive scan
//   sel_t [E * ceil(T/32)] (rounding only) bit t of row e: token t selected expert e
struct PlanInternal {
  int32_t* prefix128;
  int32_t* tile_e128;
  int32_t* hist;
  int32_t* blk_tok;
  uint32_t* sel_t;
  float* loss_part;   // [ceil(T/kLossTokens)][E+1] router-loss partial sums
  int nblk;
  int words;   // ceil(E/32)
};
PlanInternal plan_internal(const moe_shape& s, const moe_plan& p);
int64_t max_rows(const moe_shape& s);
inline int64_t max_mtiles128(const moe_shape& s) { return (max_rows(s) + 127) / 128 + s.E; }
inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// ---- routing (route.hip)
hipError_t launch_topk(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, bool rounding,
                       hipStream_t st);
hipError_t launch_plan_build(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, bool raw,
                             bool with_prob_gates, hipStream_t st);
hipError_t launch_round_select(const moe_shape& s, const moe_plan& p, const PlanInternal& pi,
                               hipStream_t st);
// capacity factor: clear the keep bits of each expert's rows past its capacity
hipError_t launch_capacity_drop(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, hipStream_t st);
// load-balance and z-loss values into plan.aux
hipError_t launch_router_losses(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, hipStream_t st);
// dz is nonzero beyond each token's selected experts
inline bool dense_router_grad(const moe_shape& s) {
  return s.gate_mode == MOE_GATE_ALL || s.lb_coef != 0.0f || s.z_coef != 0.0f;
}

// The router gradient dz as a GEMM operand dzq [T][router_dz_ld]: columns [0, ldz)
// hold dz in the act dtype (zero past E); with bf16 activations columns
// [ldz, 2 ldz) hold its bf16 rounding residual, and the router GEMMs treat the
// two halves as one operand of router_dz_rows columns (W_g doubled to match).
inline int router_ldz(const moe_shape& s) { return (s.E + 7) / 8 * 8; }
inline bool router_dz_split(const moe_shape& s) { return s.act == MOE_BF16; }
inline int router_dz_ld(const moe_shape& s) { return router_ldz(s) * (router_dz_split(s) ? 2 : 1); }
inline int router_dz_rows(const moe_shape& s) { return router_dz_split(s) ? router_ldz(s) + s.E : s.E; }

// Weight-gradient K chunks (see wgrad_chunks_kernel): tables in the backward
// workspace, partial outputs for chunks past each expert's first.
struct WgradChunks {
  int4* chunks;          // [max_chunks]
  int32_t* nchunks;      // [1]
  int2* slot_range;      // [E]
  float* part;           // [max_extra][largest weight gradient]
  int kch;               // rows per chunk (a multiple of 64)
  int max_chunks, max_extra;
};

// ---- elementwise (elementwise.hip)
// dst[r] = src[token_of_row[r]] for every routed row r
hipError_t launch_permute_rows(const moe_shape& s, const void* src, const moe_plan& p, void* dst, hipStream_t st);
hipError_t launch_combine(const moe_shape& s, const void* y, const moe_plan& p, void* out,
                          hipStream_t st);
// pos[tok_rows[q]] = q for the plan's rows (the token-order position of each row)
hipError_t launch_row_positions(const moe_shape& s, const moe_plan& p, int32_t* pos, hipStream_t st);
// out[t] = sum of rows tok_ptr[t] .. tok_ptr[t+1]-1 of yg, ascending, in fp32 (bf16 act)
hipError_t launch_segment_sum(const moe_shape& s, const void* yg, const moe_plan& p, void* out, hipStream_t st);
// dxr: the dense router term dz W_g (fp32 [T,d]) or nullptr (then gathered from W_g)
hipError_t launch_router_dx(const moe_shape& s, const moe_plan& p, const void* dx_perm, const float* dz,
                            const void* wg, const float* dxr, void* dx, hipStream_t st);
hipError_t launch_router_bwd(const moe_shape& s, const moe_plan& p, const float* ds_part, int nparts,
                             float* ds_out, float* dlogits, void* dzq, hipStream_t st);
hipError_t launch_splitk_reduce(const float* part, int nsplit, int64_t n, float* out, hipStream_t st);
// dW_g [E, d] = sum over splits of rows [0, E) (+ rows [lo_row, lo_row + E) when lo_row >= 0)
// of the partials part[q] (stride pstride floats)
hipError_t launch_router_dwg_reduce(const float* part, int nsplit, int64_t pstride, int E, int d, int lo_row,
                                    float* out, hipStream_t st);
// W_g doubled for the split dzq: [2 ldz, d] bf16, rows [0, E) and [ldz, ldz + E) = W_g, others 0
hipError_t launch_router_wg2(const void* wg, int E, int ldz, int d, void* wg2, hipStream_t st);
hipError_t launch_wgrad_chunks(const int32_t* offsets, int E, int kch, const WgradChunks& w, hipStream_t st);
hipError_t launch_wgrad_reduce(const WgradChunks& w, int E, int64_t mn, float* dw, hipStream_t st);

// ---- grouped GEMMs (gemm.hip)
struct GemmPlanView {
  const int32_t* offsets;
  const int32_t* prefix;   // m-tile prefix matching the kernel's BM
  int64_t n_max;
};
// Row operands taken "through gather": the GEMM reads row r of the permuted
// operand as row gather[r] of the unpermuted tensor ([T, ...]); nullptr = the
// operand is already permuted.
hipError_t gemm_up_swiglu(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const void* x_rows,
                          const int32_t* gather, const void* w1, void* h, void* a, hipStream_t st);
hipError_t gemm_down(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const void* a,
                     const void* w2, void* y, hipStream_t st);
// GEMM2 whose epilogue applies each row's gate and stores it at row pos[r] (bf16 only)
hipError_t gemm_down_gate_scatter(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const void* act,
                                  const void* w2, const int32_t* pos, void* yg, hipStream_t st);
hipError_t gemm_dact(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const void* do_rows,
                     const int32_t* gather, const void* w2, const void* h, void* dh, void* ga, float* ds_part,
                     hipStream_t st);
int gemm_dact_parts(const moe_shape& s);
hipError_t gemm_dx_perm(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const void* dh,
                        const void* w1, void* dx_perm, hipStream_t st);
// x_rows: x_perm, or x read through `gather` (token_of_row; bf16 only)
hipError_t gemm_dw1(const moe_shape& s, const WgradChunks& w, const void* dh, const void* x_rows, const int32_t* gather,
                    float* dw1, hipStream_t st);
hipError_t gemm_dw2(const moe_shape& s, const WgradChunks& w, const void* do_rows, const int32_t* gather,
                    const void* ga, float* dw2, hipStream_t st);
hipError_t gemm_router_logits(const moe_shape& s, const void* x, const void* wg, const float* bias,
                              const float* noise, float* logits, hipStream_t st);
// dxr [T,d] fp32 = dzq W (dense router gradients): K = router_dz_rows columns of dzq,
// wg = W_g [E, d] (fp32) or the doubled W_g of launch_router_wg2 (bf16)
hipError_t gemm_router_dx_dense(const moe_shape& s, const void* dzq, const void* wg, float* dxr, hipStream_t st);
int gemm_router_dwg_splits(const moe_shape& s);
// split-K partials part[q] [router_dz_rows, d] = dzq[K-slice]^T x[K-slice]
hipError_t gemm_router_dwg(const moe_shape& s, const void* dzq, const void* x, float* part, hipStream_t st);

// ---- MXFP8 (mx.hip, gemm_mx.hip)
// A quantised GEMM operand: codes [rows][K] (E4M3 bytes, K-contiguous) and
// stage-major scales [K/64][srows][2] (E8M0 bytes).
// Row-quantised activations of the grouped-M GEMMs are stored expert-padded:
// the segment of expert e starts at row pad[e] (a multiple of 64).
struct MxOperand {
  uint8_t* codes;
  uint8_t* scales;
  int64_t srows;
  const int32_t* pad;   // expert-padded row layout, or nullptr
};
hipError_t launch_quantize_rows(const void* src, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                hipStream_t st);
hipError_t mx_quantize_rows_staged(const void* src, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                                   int64_t srows, hipStream_t st);
// rows of a permuted activation [offsets[E], K] into the expert-padded layout
hipError_t mx_quantize_rows_padded(const void* src, int64_t rows, int64_t K, const int32_t* offsets,
                                   const int32_t* expert_of_row, const int32_t* pad_off, int E, uint8_t* codes,
                                   uint8_t* scales, int64_t srows, hipStream_t st);
hipError_t mx_quantize_cols(const void* src, int G, int R, int C, uint8_t* codes, uint8_t* scales, hipStream_t st);
// the same with plain scales [C][R/32] (test hook)
hipError_t launch_quantize_cols_plain(const void* src, int R, int C, uint8_t* codes, uint8_t* scales, hipStream_t st);
hipError_t mx_quantize_tokens(const void* src, int C, const int32_t* seg_off, const int32_t* pad_off, int E,
                              int64_t P, uint8_t* codes, uint8_t* scales, hipStream_t st,
                              const int32_t* gather = nullptr);
hipError_t mx_pad_offsets(const int32_t* offsets, int E, int32_t* pad_off, hipStream_t st);
// rows and columns (seg_off == nullptr: G matrices [R][C]) or rows and tokens
// (seg_off, pad_off, P as for mx_quantize_tokens) in one pass
hipError_t mx_quantize_dual(const void* src, int G, int R, int C, const int32_t* seg_off, const int32_t* pad_off,
                            int E, int64_t P, const MxOperand& rows, const MxOperand& pos, hipStream_t st,
                            const int32_t* gather = nullptr);
hipError_t gemm_mx_up_swiglu(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const MxOperand& x,
                             const MxOperand& w1, void* h, const MxOperand& act, hipStream_t st);
hipError_t gemm_mx_down(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const MxOperand& act,
                        const MxOperand& w2, void* y, hipStream_t st);
hipError_t gemm_mx_dact(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const MxOperand& dout,
                        const MxOperand& w2t, const void* h, const MxOperand& dhq, const MxOperand& dh_t,
                        const MxOperand& ga_t, int64_t P, float* ds_part, hipStream_t st);
hipError_t gemm_mx_dx_perm(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, const MxOperand& dh,
                           const MxOperand& w1t, void* dx_perm, hipStream_t st);
hipError_t gemm_mx_wgrad(const moe_shape& s, const WgradChunks& w, int64_t P, const MxOperand& lhs, int M,
                         const MxOperand& rhs, int N, float* dw, hipStream_t st);

}  // namespace moe
