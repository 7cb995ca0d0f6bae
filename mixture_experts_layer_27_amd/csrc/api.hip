// C ABI of the MoE layer: validation, plan/workspace carving and launch order.
// Every call only enqueues on the caller's stream; nothing is launched when a
// check fails; no device-to-host copy or synchronisation happens anywhere.
#include <string.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {

int64_t max_rows(const moe_shape& s) {
  return (int64_t)s.T * s.k + (s.round_tile ? (int64_t)s.E * (s.round_tile / 2) : 0);
}

namespace {

constexpr size_t kAlign = 256;
size_t al(size_t b) { return (b + kAlign - 1) / kAlign * kAlign; }

int words_of(const moe_shape& s) { return (s.E + 31) / 32; }
int nblk_of(const moe_shape& s) { return (s.T + kPlanBlock - 1) / kPlanBlock; }
size_t esz(const moe_shape& s) { return s.act == MOE_BF16 ? 2 : 4; }

// Carves the plan blob in a fixed order; with base == nullptr it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  template <typename P>
  P* take(size_t bytes) {
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += al(bytes);
    return p;
  }
};

void carve_plan(const moe_shape& s, char* base, moe_plan* p, size_t* total) {
  Carver c{base};
  const int64_t T = s.T, E = s.E, k = s.k, N = max_rows(s);
  moe_plan q{};
  q.logits = c.take<float>(T * E * 4);
  q.probs_t = s.round_tile ? c.take<float>(E * T * 4) : nullptr;
  q.topk_idx = c.take<int32_t>(T * k * 4);
  q.topk_gate = c.take<float>(T * k * 4);
  q.counts_raw = c.take<int32_t>(E * 4);
  q.counts = c.take<int32_t>(E * 4);
  q.offsets = c.take<int32_t>((E + 1) * 4);
  q.token_of_row = c.take<int32_t>(N * 4);
  q.expert_of_row = c.take<int32_t>(N * 4);
  q.gate_of_row = c.take<float>(N * 4);
  q.row_of_slot = c.take<int32_t>(T * k * 4);
  q.tok_ptr = c.take<int32_t>((T + 1) * 4);
  q.tok_rows = c.take<int32_t>(N * 4);
  q.keep_bits = c.take<uint32_t>(T * words_of(s) * 4);
  q.aux = c.take<float>((4 + E) * 4);
  // internal region
  q.sched = c.take<int32_t>((E + 1) * 4);
  c.take<int32_t>(max_mtiles128(s) * 4);
  c.take<int32_t>(E * nblk_of(s) * 4);
  c.take<int32_t>((nblk_of(s) + 1) * 4);
  if (s.round_tile) c.take<uint32_t>(E * ((T + 31) / 32) * 4);
  c.take<float>((size_t)((T + kLossTokens - 1) / kLossTokens) * (E + 1) * 4);   // router-loss partials
  if (p) *p = q;
  if (total) *total = c.off;
}

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_EINVAL;
  if (s->T <= 0 || s->d <= 0 || s->E <= 0 || s->k <= 0 || s->d_ff <= 0) return MOE_EINVAL;
  if (s->k > s->E) return MOE_EINVAL;
  if (s->act != MOE_F32 && s->act != MOE_BF16) return MOE_EINVAL;
  if (s->gemm == MOE_F32 && s->act != MOE_F32) return MOE_EINVAL;
  if ((s->gemm == MOE_BF16 || s->gemm == MOE_MXFP8) && s->act != MOE_BF16) return MOE_EINVAL;
  if (s->gemm != MOE_F32 && s->gemm != MOE_BF16 && s->gemm != MOE_MXFP8) return MOE_EINVAL;
  if (s->round_tile < 0 || (s->round_tile & 1)) return MOE_EINVAL;
  if (s->gate_mode != MOE_GATE_TOPK && s->gate_mode != MOE_GATE_ALL) return MOE_EINVAL;
  for (float v : {s->capacity_factor, s->lb_coef, s->z_coef})
    if (!(v >= 0.0f) || !(v <= 3.0e38f)) return MOE_EINVAL;   // negative, NaN or infinite
  if (s->capacity_factor > 0.0f && s->round_tile) return MOE_ENOTSUP;
  if (s->k > 8 || s->E > 256) return MOE_ENOTSUP;
  if (s->d % 64 || s->d_ff % 64) return MOE_ENOTSUP;
  if (s->act == MOE_BF16 && s->d_ff % 128) return MOE_ENOTSUP;
  if (s->d > 16384 || s->d_ff > 16384) return MOE_ENOTSUP;
  if (s->T > (1 << 20)) return MOE_ENOTSUP;
  if (s->round_tile > 4096) return MOE_ENOTSUP;
  if (max_rows(*s) >= ((int64_t)1 << 31)) return MOE_ENOTSUP;
  return MOE_OK;
}

bool aligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Row gathers fused into the GEMM / quantiser loads: bf16 activations (the fp32
// weight-gradient kernel has no gathered loads) whose [T, d] tensors fit the
// 32-bit offsets of one buffer resource.
bool gather_ok(const moe_shape& s) {
  return s.act == MOE_BF16 && (int64_t)s.T * s.d * 2 < ((int64_t)1 << 31);
}
bool aligned_or_null(const void* p) { return !p || (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

moe_status check_plan(const moe_shape& s, const moe_plan* p) {
  if (!p) return MOE_EINVAL;
  const void* ptrs[] = {p->logits, p->topk_idx, p->topk_gate, p->counts_raw, p->counts, p->offsets,
                        p->token_of_row, p->expert_of_row, p->gate_of_row, p->row_of_slot, p->tok_ptr,
                        p->tok_rows, p->keep_bits, p->sched};
  for (const void* q : ptrs)
    if (!aligned(q)) return MOE_EINVAL;
  if (s.round_tile && !aligned(p->probs_t)) return MOE_EINVAL;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// A call's launch sequence: each step runs only while every earlier one succeeded,
// and with a trace the caller's next event is recorded after it (names[i] = the
// kernel between events[i] and events[i + 1]).
struct Seq {
  hipStream_t st;
  moe_trace* tr;
  hipError_t e = hipSuccess;
  Seq(hipStream_t s, moe_trace* t) : st(s), tr(t) {
    if (tr) {
      tr->count = 0;
      record(nullptr);
    }
  }
  void record(const char* name) {
    if (tr->count >= tr->capacity || tr->count > MOE_TRACE_MAX_KERNELS) return;
    if (tr->count > 0) tr->names[tr->count - 1] = name;
    e = hipEventRecord(reinterpret_cast<hipEvent_t>(tr->events[tr->count]), st);
    if (e == hipSuccess) tr->count++;
  }
  template <class F>
  void operator()(const char* name, F&& launch) {
    if (e != hipSuccess) return;
    e = launch();
    if (e == hipSuccess && tr) record(name);
  }
  moe_status status() const { return e == hipSuccess ? MOE_OK : MOE_EHIP; }
};

bool trace_ok(const moe_trace* t) {
  if (!t) return true;
  if (t->capacity < 0 || (t->capacity > 0 && !t->events)) return false;
  for (int i = 0; i < t->capacity; ++i)
    if (!t->events[i]) return false;
  return true;
}

// token capacity of the expert-padded layout of the MX weight-gradient operands
int64_t tok_cap(const moe_shape& s) { return (max_rows(s) + 64 * (int64_t)s.E + 63) / 64 * 64; }

MxOperand take_mx(Carver& c, int64_t rows, int64_t K, int64_t srows, const int32_t* pad = nullptr) {
  MxOperand o;
  o.codes = c.take<uint8_t>((size_t)rows * K);
  o.scales = c.take<uint8_t>((size_t)(K / 64) * srows * 2);
  o.srows = srows;
  o.pad = pad;
  return o;
}

// rows per weight-gradient chunk: at most 32 chunks past the experts' first, and
// a chunk's rows of either operand span less than 2 GiB (one buffer resource
// of the bf16 kernel addresses them)
int wgrad_kch(const moe_shape& s, int64_t ncap) {
  int64_t k = (ncap + 31) / 32;
  k = (k + 63) / 64 * 64;
  if (k < 1024) k = 1024;
  const int64_t row_bytes = (int64_t)2 * (2 * s.d_ff > s.d ? 2 * s.d_ff : s.d);
  const int64_t cap = ((int64_t)1 << 31) / row_bytes / 64 * 64;
  return (int)(k < cap ? k : cap);
}
int64_t wgrad_cap(const moe_shape& s) { return s.gemm == MOE_MXFP8 ? tok_cap(s) : max_rows(s); }

struct BwdWs {
  void *do_perm, *dh, *ga, *xbuf, *dzq, *wg2;
  float *ds_part, *dlogits, *dwg_part;
  float* dxr;   // dense router term dz W_g [T, d] (routing variants only)
  WgradChunks wg;
  // MXFP8 only
  MxOperand doq, w2t, dhq, w1t, dh_t, x_t, do_t, ga_t;
  int32_t* pad_off;
};

size_t carve_bwd(const moe_shape& s, char* base, BwdWs* w) {
  Carver c{base};
  const int64_t N = max_rows(s);
  BwdWs q{};
  q.do_perm = gather_ok(s) ? nullptr : c.take<char>(N * s.d * esz(s));   // dO is gathered inside the loads
  // MXFP8 keeps dH and gA only as codes (written by the dA' epilogue)
  q.dh = s.gemm == MOE_MXFP8 ? nullptr : c.take<char>(N * 2 * s.d_ff * esz(s));
  q.ga = s.gemm == MOE_MXFP8 ? nullptr : c.take<char>(N * s.d_ff * esz(s));
  q.xbuf = c.take<char>(N * s.d * esz(s));
  q.ds_part = c.take<float>((size_t)gemm_dact_parts(s) * N * 4);
  q.dlogits = c.take<float>((size_t)s.T * s.E * 4);
  q.dzq = c.take<char>((size_t)s.T * router_dz_ld(s) * esz(s));
  q.dwg_part = c.take<float>((size_t)gemm_router_dwg_splits(s) * router_dz_rows(s) * s.d * 4);
  q.dxr = dense_router_grad(s) ? c.take<float>((size_t)s.T * s.d * 4) : nullptr;
  q.wg2 = dense_router_grad(s) && router_dz_split(s) ? c.take<char>((size_t)2 * router_ldz(s) * s.d * 2) : nullptr;
  {
    const int64_t ncap = wgrad_cap(s);
    WgradChunks& g = q.wg;
    g.kch = wgrad_kch(s, ncap);
    g.max_extra = (int)(ncap / g.kch);
    g.max_chunks = s.E + g.max_extra;
    g.chunks = c.take<int4>((size_t)g.max_chunks * 16);
    g.nchunks = c.take<int32_t>(4);
    g.slot_range = c.take<int2>((size_t)s.E * 8);
    const int64_t mn = (int64_t)2 * s.d_ff * s.d;   // the larger of dW1_e, dW2_e
    g.part = c.take<float>((size_t)g.max_extra * mn * 4);
  }
  if (s.gemm == MOE_MXFP8) {
    const int64_t E = s.E, d = s.d, f = s.d_ff, P = tok_cap(s);
    q.pad_off = c.take<int32_t>((E + 1) * 4);
    q.doq = take_mx(c, P, d, P, q.pad_off);
    q.w2t = take_mx(c, E * f, d, E * f);
    q.dhq = take_mx(c, P, 2 * f, P, q.pad_off);
    q.w1t = take_mx(c, E * d, 2 * f, E * d);
    q.dh_t = take_mx(c, 2 * f, P, 2 * f);
    q.x_t = take_mx(c, d, P, d);
    q.do_t = take_mx(c, d, P, d);
    q.ga_t = take_mx(c, f, P, f);
  }
  if (w) *w = q;
  return c.off;
}

struct FwdWs {
  void* act;              // A [N_max, f]
  int32_t* pad_off;       // MXFP8 only: expert-padded row offsets, quantised operands
  MxOperand x, w1, a, w2;
  MxOperand w1t, w2t, x_t;   // MXFP8: the backward's orientation of W1, W2 and x_perm
};

// MXFP8: the weight codes come first, so where they sit depends only on E, d
// and d_ff (moe_quantize_weights_mx fills them once for micro-batches of any T).
size_t carve_fwd(const moe_shape& s, char* base, FwdWs* w) {
  Carver c{base};
  const int64_t N = max_rows(s);
  FwdWs q{};
  if (s.gemm != MOE_MXFP8) q.act = c.take<char>((size_t)N * s.d_ff * esz(s));   // MXFP8: A only as codes
  if (s.gemm == MOE_MXFP8) {
    const int64_t E = s.E, d = s.d, f = s.d_ff, P = tok_cap(s);
    q.w1 = take_mx(c, E * 2 * f, d, E * 2 * f);
    q.w2 = take_mx(c, E * d, f, E * d);
    q.w1t = take_mx(c, E * d, 2 * f, E * d);
    q.w2t = take_mx(c, E * f, d, E * f);
    q.pad_off = c.take<int32_t>((E + 1) * 4);
    q.x = take_mx(c, P, d, P, q.pad_off);
    q.a = take_mx(c, P, f, P, q.pad_off);
    q.x_t = take_mx(c, d, P, d);
  }
  if (w) *w = q;
  return c.off;
}

size_t experts_ws(const moe_shape& s) { return carve_fwd(s, nullptr, nullptr); }

// The expert FFN with the combine in GEMM2's epilogue: the expert workspace,
// then the gated rows in token order [N_max, d] and each row's position [N_max].
struct CombineWs {
  FwdWs f;
  void* yg;
  int32_t* pos;
};
size_t carve_combine(const moe_shape& s, char* base, CombineWs* w) {
  const size_t fb = al(experts_ws(s));
  Carver c{base ? base + fb : nullptr};
  CombineWs q{};
  if (base) carve_fwd(s, base, &q.f);
  q.yg = c.take<char>((size_t)max_rows(s) * s.d * esz(s));
  q.pos = c.take<int32_t>((size_t)max_rows(s) * 4);
  if (w) *w = q;
  return fb + c.off;
}
size_t combine_ws(const moe_shape& s) { return carve_combine(s, nullptr, nullptr); }

}  // namespace

PlanInternal plan_internal(const moe_shape& s, const moe_plan& p) {
  PlanInternal pi{};
  pi.nblk = nblk_of(s);
  pi.words = words_of(s);
  char* b = reinterpret_cast<char*>(p.sched);
  pi.prefix128 = reinterpret_cast<int32_t*>(b);
  b += al((size_t)(s.E + 1) * 4);
  pi.tile_e128 = reinterpret_cast<int32_t*>(b);
  b += al((size_t)max_mtiles128(s) * 4);
  pi.hist = reinterpret_cast<int32_t*>(b);
  b += al((size_t)s.E * pi.nblk * 4);
  pi.blk_tok = reinterpret_cast<int32_t*>(b);
  b += al((size_t)(pi.nblk + 1) * 4);
  pi.sel_t = s.round_tile ? reinterpret_cast<uint32_t*>(b) : nullptr;
  if (s.round_tile) b += al((size_t)s.E * ((s.T + 31) / 32) * 4);
  pi.loss_part = reinterpret_cast<float*>(b);
  return pi;
}

}  // namespace moe

using namespace moe;

extern "C" {

int64_t moe_max_rows(const moe_shape* s) { return (check_shape(s) == MOE_OK) ? max_rows(*s) : -1; }

size_t moe_plan_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  size_t total = 0;
  carve_plan(*s, nullptr, nullptr, &total);
  return total;
}

moe_status moe_plan_init(const moe_shape* s, void* blob, size_t blob_bytes, moe_plan* plan) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!aligned(blob) || !plan) return MOE_EINVAL;
  if ((reinterpret_cast<uintptr_t>(blob) & (kAlign - 1)) != 0) return MOE_EINVAL;
  size_t total = 0;
  carve_plan(*s, nullptr, nullptr, &total);
  if (blob_bytes < total) return MOE_EWORKSPACE;
  carve_plan(*s, reinterpret_cast<char*>(blob), plan, nullptr);
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_shape* s, int which) {
  if (check_shape(s) != MOE_OK) return 0;
  switch (which) {
    case MOE_WS_ROUTE: return 0;
    case MOE_WS_ROUND: return 0;
    case MOE_WS_EXPERTS: return experts_ws(*s);
    case MOE_WS_EXPERTS_COMBINE: return combine_ws(*s);
    case MOE_WS_BACKWARD: return carve_bwd(*s, nullptr, nullptr);
    default: return 0;
  }
}

moe_status moe_route(const moe_shape* s, const void* x, const void* w_gate, const float* bias, const float* noise,
                     moe_plan* plan, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!aligned(x) || !aligned(w_gate) || (bias && (reinterpret_cast<uintptr_t>(bias) & 3)) ||
      (noise && (reinterpret_cast<uintptr_t>(noise) & 3)))
    return MOE_EINVAL;
  if ((st = check_plan(*s, plan)) != MOE_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  PlanInternal pi = plan_internal(*s, *plan);
  hipError_t e = gemm_router_logits(*s, x, w_gate, bias, noise, plan->logits, hs);
  if (e == hipSuccess) e = launch_topk(*s, *plan, pi, s->round_tile != 0, hs);
  if (e == hipSuccess) e = launch_plan_build(*s, *plan, pi, true, false, hs);
  if (s->capacity_factor > 0.0f) {
    if (e == hipSuccess) e = launch_capacity_drop(*s, *plan, pi, hs);
    if (e == hipSuccess) e = launch_plan_build(*s, *plan, pi, false, false, hs);
  }
  if (e == hipSuccess && (s->lb_coef != 0.0f || s->z_coef != 0.0f)) e = launch_router_losses(*s, *plan, pi, hs);
  return hip_status(e);
}

moe_status moe_round_tokens(const moe_shape* s, moe_plan* plan, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->round_tile == 0) return MOE_EINVAL;
  if ((st = check_plan(*s, plan)) != MOE_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  PlanInternal pi = plan_internal(*s, *plan);
  hipError_t e = launch_round_select(*s, *plan, pi, hs);
  if (e == hipSuccess) e = launch_plan_build(*s, *plan, pi, false, true, hs);
  return hip_status(e);
}

moe_status moe_permute(const moe_shape* s, const void* src, const moe_plan* plan, void* dst, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!aligned(src) || !aligned(dst)) return MOE_EINVAL;
  if ((st = check_plan(*s, plan)) != MOE_OK) return st;
  return hip_status(launch_permute_rows(*s, src, *plan, dst, reinterpret_cast<hipStream_t>(stream)));
}

namespace {
// The expert FFN of the forward.  rows = x_perm (gather == nullptr) or x read
// through gather = token_of_row (the permutation fused into the operand loads).
// wcodes (MXFP8): the weight codes are already in ws (moe_quantize_weights_mx),
// w1 and w2 are not read.
moe_status experts_forward(const moe_shape* s, const void* rows, const int32_t* gather, const void* w1,
                           const void* w2, const moe_plan* plan, void* h_saved, void* y, void* ws, size_t ws_bytes,
                           void* stream, moe_trace* trace, bool wcodes = false) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (wcodes && s->gemm != MOE_MXFP8) return MOE_ENOTSUP;
  if (!aligned(rows) || !aligned(h_saved) || !aligned(y)) return MOE_EINVAL;
  if (!wcodes && (!aligned(w1) || !aligned(w2))) return MOE_EINVAL;
  if ((st = check_plan(*s, plan)) != MOE_OK) return st;
  if (!aligned(ws) || ws_bytes < experts_ws(*s)) return MOE_EWORKSPACE;
  if (!trace_ok(trace)) return MOE_EINVAL;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  PlanInternal pi = plan_internal(*s, *plan);
  FwdWs w;
  carve_fwd(*s, reinterpret_cast<char*>(ws), &w);
  Seq seq(hs, trace);
  if (s->gemm == MOE_MXFP8) {
    // x_perm and the weights are quantised along both of their axes in one pass
    // each: this call's GEMMs use the rows, the backward the other orientation
    const int64_t P = tok_cap(*s);
    const int E = s->E, d = s->d, f = s->d_ff;
    const int32_t* off = plan->offsets;
    seq("mx_pad_offsets", [&] { return mx_pad_offsets(off, E, w.pad_off, hs); });
    seq("mx_quantize_x", [&] { return mx_quantize_dual(rows, 1, 0, d, off, w.pad_off, E, P, w.x, w.x_t, hs, gather); });
    if (!wcodes)
      seq("mx_quantize_w1", [&] { return mx_quantize_dual(w1, E, 2 * f, d, nullptr, nullptr, 0, 0, w.w1, w.w1t, hs); });
    seq("mx_up_swiglu", [&] { return gemm_mx_up_swiglu(*s, *plan, pi, w.x, w.w1, h_saved, w.a, hs); });
    if (!wcodes)
      seq("mx_quantize_w2", [&] { return mx_quantize_dual(w2, E, d, f, nullptr, nullptr, 0, 0, w.w2, w.w2t, hs); });
    seq("mx_down", [&] { return gemm_mx_down(*s, *plan, pi, w.a, w.w2, y, hs); });
    return seq.status();
  }
  seq("up_swiglu", [&] { return gemm_up_swiglu(*s, *plan, pi, rows, gather, w1, h_saved, w.act, hs); });
  seq("down", [&] { return gemm_down(*s, *plan, pi, w.act, w2, y, hs); });
  return seq.status();
}
}  // namespace

moe_status moe_grouped_gemm_swiglu(const moe_shape* s, const void* x_perm, const void* w1, const void* w2,
                                   const moe_plan* plan, void* h_saved, void* y, void* ws, size_t ws_bytes,
                                   void* stream) {
  return experts_forward(s, x_perm, nullptr, w1, w2, plan, h_saved, y, ws, ws_bytes, stream, nullptr);
}

moe_status moe_grouped_gemm_swiglu_traced(const moe_shape* s, const void* x_perm, const void* w1, const void* w2,
                                          const moe_plan* plan, void* h_saved, void* y, void* ws, size_t ws_bytes,
                                          void* stream, moe_trace* trace) {
  return experts_forward(s, x_perm, nullptr, w1, w2, plan, h_saved, y, ws, ws_bytes, stream, trace);
}

moe_status moe_grouped_gemm_swiglu_gather_traced(const moe_shape* s, const void* x, const void* w1, const void* w2,
                                                 const moe_plan* plan, void* h_saved, void* y, void* ws,
                                                 size_t ws_bytes, void* stream, moe_trace* trace) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!gather_ok(*s)) return MOE_ENOTSUP;
  if ((st = check_plan(*s, plan)) != MOE_OK) return st;
  return experts_forward(s, x, plan->token_of_row, w1, w2, plan, h_saved, y, ws, ws_bytes, stream, trace);
}

moe_status moe_grouped_gemm_swiglu_gather(const moe_shape* s, const void* x, const void* w1, const void* w2,
                                          const moe_plan* plan, void* h_saved, void* y, void* ws, size_t ws_bytes,
                                          void* stream) {
  return moe_grouped_gemm_swiglu_gather_traced(s, x, w1, w2, plan, h_saved, y, ws, ws_bytes, stream, nullptr);
}

moe_status moe_grouped_gemm_swiglu_combine(const moe_shape* s, const void* x, int x_gathered, const void* w1,
                                           const void* w2, const moe_plan* plan, void* h_saved, void* out, void* ws,
                                           size_t ws_bytes, void* stream, moe_trace* trace) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->act != MOE_BF16 || s->gemm != MOE_BF16) return MOE_ENOTSUP;
  if (x_gathered != 0 && x_gathered != 1) return MOE_EINVAL;
  if (x_gathered && !gather_ok(*s)) return MOE_ENOTSUP;
  if (!aligned(x) || !aligned(w1) || !aligned(w2) || !aligned(h_saved) || !aligned(out)) return MOE_EINVAL;
  if ((st = check_plan(*s, plan)) != MOE_OK) return st;
  if (!aligned(ws) || ws_bytes < combine_ws(*s)) return MOE_EWORKSPACE;
  if (!trace_ok(trace)) return MOE_EINVAL;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  PlanInternal pi = plan_internal(*s, *plan);
  CombineWs w;
  carve_combine(*s, reinterpret_cast<char*>(ws), &w);
  const int32_t* gather = x_gathered ? plan->token_of_row : nullptr;
  Seq seq(hs, trace);
  seq("up_swiglu", [&] { return gemm_up_swiglu(*s, *plan, pi, x, gather, w1, h_saved, w.f.act, hs); });
  seq("row_positions", [&] { return launch_row_positions(*s, *plan, w.pos, hs); });
  seq("down_gate_scatter", [&] { return gemm_down_gate_scatter(*s, *plan, pi, w.f.act, w2, w.pos, w.yg, hs); });
  seq("segment_sum", [&] { return launch_segment_sum(*s, w.yg, *plan, out, hs); });
  return seq.status();
}

moe_status moe_quantize_weights_mx(const moe_shape* s, const void* w1, const void* w2, void* ws, size_t ws_bytes,
                                   void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->gemm != MOE_MXFP8) return MOE_ENOTSUP;
  if (!aligned(w1) || !aligned(w2)) return MOE_EINVAL;
  if (!aligned(ws) || ws_bytes < experts_ws(*s)) return MOE_EWORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  FwdWs w;
  carve_fwd(*s, reinterpret_cast<char*>(ws), &w);
  const int E = s->E, d = s->d, f = s->d_ff;
  hipError_t e = mx_quantize_dual(w1, E, 2 * f, d, nullptr, nullptr, 0, 0, w.w1, w.w1t, hs);
  if (e == hipSuccess) e = mx_quantize_dual(w2, E, d, f, nullptr, nullptr, 0, 0, w.w2, w.w2t, hs);
  return hip_status(e);
}

moe_status moe_grouped_gemm_swiglu_wcodes(const moe_shape* s, const void* x, int x_gathered, const moe_plan* plan,
                                          void* h_saved, void* y, void* ws, size_t ws_bytes, void* stream,
                                          moe_trace* trace) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->gemm != MOE_MXFP8) return MOE_ENOTSUP;
  if (x_gathered != 0 && x_gathered != 1) return MOE_EINVAL;
  if (x_gathered && !gather_ok(*s)) return MOE_ENOTSUP;
  if ((st = check_plan(*s, plan)) != MOE_OK) return st;
  return experts_forward(s, x, x_gathered ? plan->token_of_row : nullptr, nullptr, nullptr, plan, h_saved, y, ws,
                         ws_bytes, stream, trace, true);
}

}  // extern "C"

// ---- the expert FFN without any allocation: its workspace is this file's
// device array.  Each GPU the library runs on holds its own copy of the array
// until the process ends; host code uses only the address hipGetSymbolAddress
// returns for the current device (the array's name is a host-side stand-in).
namespace {
constexpr size_t kNoAllocScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

hipError_t scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

moe_status moe_grouped_gemm_swiglu_noalloc(const moe_shape* s, const void* x_perm, const void* w1, const void* w2,
                                           const moe_plan* plan, void* h_saved, void* y, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!aligned(x_perm) || !aligned(w1) || !aligned(w2) || !aligned(h_saved) || !aligned(y)) return MOE_EINVAL;
  if ((st = check_plan(*s, plan)) != MOE_OK) return st;
  if (experts_ws(*s) > kNoAllocScratchBytes) return MOE_EWORKSPACE;
  void* ws = nullptr;
  if (scratch_of_current_device(&ws) != hipSuccess) return MOE_EHIP;
  return experts_forward(s, x_perm, nullptr, w1, w2, plan, h_saved, y, ws, kNoAllocScratchBytes, stream, nullptr);
}

moe_status moe_unpermute_combine(const moe_shape* s, const void* y, const moe_plan* plan, void* out, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!aligned(y) || !aligned(out)) return MOE_EINVAL;
  if ((st = check_plan(*s, plan)) != MOE_OK) return st;
  return hip_status(launch_combine(*s, y, *plan, out, reinterpret_cast<hipStream_t>(stream)));
}

namespace {
moe_status backward_impl(const moe_shape* s, const void* x, const void* w_gate, const void* w1, const void* w2,
                         const moe_plan* plan, const void* h_saved, const void* x_perm, const void* fwd_ws,
                         const void* dout, void* dx, float* dw_gate, float* dw1, float* dw2, float* dlogits, float* ds,
                         void* ws, size_t ws_bytes, void* stream, moe_trace* trace) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!aligned(x) || !aligned(w_gate) || !aligned(w1) || !aligned(w2) || !aligned(h_saved) || !aligned(dout) ||
      !aligned(dx) || !aligned(dw_gate) || !aligned(dw1) || !aligned(dw2) || !aligned_or_null(dlogits) ||
      !aligned_or_null(x_perm) || !aligned_or_null(fwd_ws) ||
      (ds && (reinterpret_cast<uintptr_t>(ds) & 3)))
    return MOE_EINVAL;
  if ((st = check_plan(*s, plan)) != MOE_OK) return st;
  if (!aligned(ws) || ws_bytes < carve_bwd(*s, nullptr, nullptr)) return MOE_EWORKSPACE;
  if (!trace_ok(trace)) return MOE_EINVAL;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  PlanInternal pi = plan_internal(*s, *plan);
  BwdWs w;
  carve_bwd(*s, reinterpret_cast<char*>(ws), &w);
  float* dz = dlogits ? dlogits : w.dlogits;
  // dO reaches the GEMMs through token_of_row inside their operand loads when the
  // kernels allow it (as fast as a permuted copy here, and no copy is stored),
  // else as a permuted copy.  x without x_perm is read the same way by dW1.
  const bool fused = gather_ok(*s);
  const int32_t* tor = plan->token_of_row;
  Seq seq(hs, trace);
  if (!fused) seq("permute_dout", [&] { return launch_permute_rows(*s, dout, *plan, w.do_perm, hs); });
  const void* dO = fused ? dout : w.do_perm;
  const int32_t* dOg = fused ? tor : nullptr;
  if (s->gemm == MOE_MXFP8) {
    const int64_t P = tok_cap(*s);
    const int E = s->E, d = s->d, f = s->d_ff;
    const int32_t* off = plan->offsets;
    // the forward's workspace already holds W1, W2 along their first axes and
    // x_perm along tokens, quantised from the same inputs
    FwdWs fw{};
    if (fwd_ws) carve_fwd(*s, reinterpret_cast<char*>(const_cast<void*>(fwd_ws)), &fw);
    const MxOperand& w1t = fwd_ws ? fw.w1t : w.w1t;
    const MxOperand& w2t = fwd_ws ? fw.w2t : w.w2t;
    const MxOperand& x_t = fwd_ws ? fw.x_t : w.x_t;
    seq("mx_pad_offsets", [&] { return mx_pad_offsets(off, E, w.pad_off, hs); });
    seq("mx_quantize_dout", [&] { return mx_quantize_dual(dO, 1, 0, d, off, w.pad_off, E, P, w.doq, w.do_t, hs, dOg); });
    if (!fwd_ws) seq("mx_quantize_w2t", [&] { return mx_quantize_cols(w2, E, d, f, w.w2t.codes, w.w2t.scales, hs); });
    seq("mx_dact", [&] {
      return gemm_mx_dact(*s, *plan, pi, w.doq, w2t, h_saved, w.dhq, w.dh_t, w.ga_t, P, w.ds_part, hs);
    });
    if (!fwd_ws) seq("mx_quantize_w1t", [&] { return mx_quantize_cols(w1, E, 2 * f, d, w.w1t.codes, w.w1t.scales, hs); });
    // the token-axis quantiser reads x through the plan (a memory-bound pass: gathering is free)
    const void* xp = x_perm ? x_perm : fused ? x : w.xbuf;
    const int32_t* xg = (!x_perm && fused) ? tor : nullptr;
    if (!x_perm && !fwd_ws && !fused) seq("permute_x", [&] { return launch_permute_rows(*s, x, *plan, w.xbuf, hs); });
    if (!fwd_ws)
      seq("mx_quantize_x_tokens", [&] {
        return mx_quantize_tokens(xp, d, plan->offsets, w.pad_off, E, P, w.x_t.codes, w.x_t.scales, hs, xg);
      });
    seq("wgrad_chunks", [&] { return launch_wgrad_chunks(w.pad_off, E, w.wg.kch, w.wg, hs); });
    seq("mx_dw1", [&] { return gemm_mx_wgrad(*s, w.wg, P, w.dh_t, 2 * f, x_t, d, dw1, hs); });
    seq("dw1_reduce", [&] { return launch_wgrad_reduce(w.wg, E, (int64_t)2 * f * d, dw1, hs); });
    seq("mx_dw2", [&] { return gemm_mx_wgrad(*s, w.wg, P, w.do_t, d, w.ga_t, f, dw2, hs); });
    seq("dw2_reduce", [&] { return launch_wgrad_reduce(w.wg, E, (int64_t)d * f, dw2, hs); });
    // dx_perm (x_perm no longer needed)
    seq("mx_dx_perm", [&] { return gemm_mx_dx_perm(*s, *plan, pi, w.dhq, w1t, w.xbuf, hs); });
  } else {
    seq("dact", [&] { return gemm_dact(*s, *plan, pi, dO, dOg, w2, h_saved, w.dh, w.ga, w.ds_part, hs); });
    // without x_perm, dW1 reads x through the plan (no permuted copy)
    const bool gx = !x_perm && fused;
    if (!x_perm && !gx) seq("permute_x", [&] { return launch_permute_rows(*s, x, *plan, w.xbuf, hs); });
    const void* xp = x_perm ? x_perm : gx ? x : w.xbuf;
    seq("wgrad_chunks", [&] { return launch_wgrad_chunks(plan->offsets, s->E, w.wg.kch, w.wg, hs); });
    seq("dw1", [&] { return gemm_dw1(*s, w.wg, w.dh, xp, gx ? tor : nullptr, dw1, hs); });
    seq("dw1_reduce", [&] { return launch_wgrad_reduce(w.wg, s->E, (int64_t)2 * s->d_ff * s->d, dw1, hs); });
    seq("dw2", [&] { return gemm_dw2(*s, w.wg, dO, dOg, w.ga, dw2, hs); });
    seq("dw2_reduce", [&] { return launch_wgrad_reduce(w.wg, s->E, (int64_t)s->d * s->d_ff, dw2, hs); });
    // dx_perm (x_perm no longer needed)
    seq("dx_perm", [&] { return gemm_dx_perm(*s, *plan, pi, w.dh, w1, w.xbuf, hs); });
  }
  seq("router_bwd", [&] { return launch_router_bwd(*s, *plan, w.ds_part, gemm_dact_parts(*s), ds, dz, w.dzq, hs); });
  if (w.wg2) seq("router_wg2", [&] { return launch_router_wg2(w_gate, s->E, router_ldz(*s), s->d, w.wg2, hs); });
  if (w.dxr) seq("router_dx_dense", [&] { return gemm_router_dx_dense(*s, w.dzq, w.wg2 ? w.wg2 : w_gate, w.dxr, hs); });
  seq("router_dx", [&] { return launch_router_dx(*s, *plan, w.xbuf, dz, w_gate, w.dxr, dx, hs); });
  seq("router_dwg", [&] { return gemm_router_dwg(*s, w.dzq, x, w.dwg_part, hs); });
  seq("router_dwg_reduce", [&] {
    return launch_router_dwg_reduce(w.dwg_part, gemm_router_dwg_splits(*s), (int64_t)router_dz_rows(*s) * s->d,
                                    s->E, s->d, router_dz_split(*s) ? router_ldz(*s) : -1, dw_gate, hs);
  });
  return seq.status();
}
}  // namespace

moe_status moe_backward(const moe_shape* s, const void* x, const void* w_gate, const void* w1, const void* w2,
                        const moe_plan* plan, const void* h_saved, const void* x_perm, const void* fwd_ws,
                        const void* dout, void* dx, float* dw_gate, float* dw1, float* dw2, float* dlogits, float* ds,
                        void* ws, size_t ws_bytes, void* stream) {
  return backward_impl(s, x, w_gate, w1, w2, plan, h_saved, x_perm, fwd_ws, dout, dx, dw_gate, dw1, dw2, dlogits, ds,
                       ws, ws_bytes, stream, nullptr);
}

moe_status moe_backward_traced(const moe_shape* s, const void* x, const void* w_gate, const void* w1, const void* w2,
                               const moe_plan* plan, const void* h_saved, const void* x_perm, const void* fwd_ws,
                               const void* dout, void* dx, float* dw_gate, float* dw1, float* dw2, float* dlogits,
                               float* ds, void* ws, size_t ws_bytes, void* stream, moe_trace* trace) {
  return backward_impl(s, x, w_gate, w1, w2, plan, h_saved, x_perm, fwd_ws, dout, dx, dw_gate, dw1, dw2, dlogits, ds,
                       ws, ws_bytes, stream, trace);
}

moe_status moe_quantize_mx(const void* src_bf16, int64_t rows, int64_t cols, int k_axis, uint8_t* codes,
                           uint8_t* scales, void* stream) {
  if (!aligned(src_bf16) || !aligned(codes) || !scales) return MOE_EINVAL;
  if (rows <= 0 || cols <= 0 || (k_axis != 0 && k_axis != 1)) return MOE_EINVAL;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (k_axis == 1) {
    if (cols % 32) return MOE_EINVAL;
    return hip_status(launch_quantize_rows(src_bf16, rows, cols, codes, scales, hs));
  }
  if (rows % 64 || cols % 64 || rows > (1 << 30) || cols > (1 << 30)) return MOE_EINVAL;
  return hip_status(launch_quantize_cols_plain(src_bf16, (int)rows, (int)cols, codes, scales, hs));
}

const char* moe_status_str(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ENOTSUP: return "shape not supported";
    case MOE_EWORKSPACE: return "workspace or plan blob too small";
    case MOE_EHIP: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
