// HBM-bound kernels of the layer: the permutation gather (tokens into contiguous
// per-expert rows, the "row-wise" expert buffers of the Olmo-core 3 article,
// "three splits" section), the gate-weighted combine ("Beam" blog section 2.2:
// the output is the gate-weighted sum of the chosen experts' outputs), the
// router backward, and the split-K reduction.
//
// Rows are moved as 16-byte vectors; consecutive threads take consecutive
// vectors of one row, so every wave reads and writes whole spans.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

// dst[r] = src[t] for every row r of token t (the token's rows are
// tok_rows[tok_ptr[t] .. tok_ptr[t+1])), i.e. dst[r] = src[token_of_row[r]].
// Written as a scatter: each source vector is read once and stored to each of
// its rows, so the source streams from HBM once instead of once per row.
// vec = 16-byte vectors per row; each thread moves U vectors of one token.
template <int U>
__global__ __launch_bounds__(256) void scatter_rows_kernel(const char* __restrict__ src,
                                                          const int32_t* __restrict__ tok_ptr,
                                                          const int32_t* __restrict__ tok_rows, int T_, int vec,
                                                          char* __restrict__ dst) {
  const int per_tok = vec / U;   // threads per token
  const int64_t total = (int64_t)T_ * per_tok;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int t = (int)(i / per_tok);
    const int c0 = (int)(i - (int64_t)t * per_tok);
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ldg16_nt(src + ((int64_t)t * vec + c0 + u * per_tok) * 16);
    const int p0 = tok_ptr[t], p1 = tok_ptr[t + 1];
    for (int p = p0; p < p1; ++p) {
      char* drow = dst + (int64_t)tok_rows[p] * vec * 16;
#pragma unroll
      for (int u = 0; u < U; ++u) stg16(drow + (int64_t)(c0 + u * per_tok) * 16, v[u]);
    }
  }
}

// out[t] = sum over the rows of t (ascending) of gate[r] * y[r], fp32 accumulation.
// One wave per token: each lane owns CL 16-byte column chunks per pass and
// issues the loads of up to RU rows before adding them (in ascending row order),
// so RU * CL row vectors are in flight per lane.  The rows are read once:
// non-temporal loads.  SEG: y holds the gated rows in token order already (row
// q of y = the q-th entry of tok_rows, gate applied), so t sums rows
// tok_ptr[t] .. tok_ptr[t+1]-1 as they are.
template <typename T, int RU, bool SEG = false>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y, const int32_t* __restrict__ tok_ptr,
                                                     const int32_t* __restrict__ tok_rows,
                                                     const float* __restrict__ gate, int T_, int d,
                                                     T* __restrict__ out) {
  constexpr int EV = 16 / sizeof(T);   // elements per vector
  constexpr int CL = 4;                // column chunks per lane per pass
  const int vec = d / EV;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  const int p0 = tok_ptr[t], p1 = tok_ptr[t + 1];
  for (int cb = 0; cb < vec; cb += 64 * CL) {
    float acc[CL][EV];
#pragma unroll
    for (int j = 0; j < CL; ++j)
#pragma unroll
      for (int q = 0; q < EV; ++q) acc[j][q] = 0.0f;
    for (int p = p0; p < p1; p += RU) {
      int r[RU];
      float g[RU];
      u32x4 v[RU][CL];
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        if constexpr (SEG) {
          r[u] = p + u < p1 ? p + u : -1;
          g[u] = 1.0f;
        } else {
          r[u] = p + u < p1 ? tok_rows[p + u] : -1;
          g[u] = r[u] >= 0 ? gate[r[u]] : 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int j = 0; j < CL; ++j) {
          const int c = cb + lane + 64 * j;
          v[u][j] = (r[u] >= 0 && c < vec) ? ldg16_nt(y + (int64_t)r[u] * d + c * EV) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        if (r[u] < 0) break;
#pragma unroll
        for (int j = 0; j < CL; ++j) {
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              acc[j][2 * q] += g[u] * __uint_as_float(v[u][j][q] << 16);
              acc[j][2 * q + 1] += g[u] * __uint_as_float(v[u][j][q] & 0xffff0000u);
            }
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[j][q] += g[u] * __uint_as_float(v[u][j][q]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < CL; ++j) {
      const int c = cb + lane + 64 * j;
      if (c >= vec) continue;
      u32x4 o;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf2(acc[j][2 * q], acc[j][2 * q + 1]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[j][q]);
      }
      stg16(out + (int64_t)t * d + c * EV, o);
    }
  }
}

// pos[tok_rows[q]] = q for the q < tok_ptr[T] rows in use: where each row of the
// expert-ordered layout sits in token order (a permutation of [0, N)).
__global__ __launch_bounds__(256) void row_positions_kernel(const int32_t* __restrict__ tok_rows,
                                                           const int32_t* __restrict__ tok_ptr, int T_, int64_t n_max,
                                                           int32_t* __restrict__ pos) {
  const int64_t n = tok_ptr[T_];
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n && q < n_max;
       q += (int64_t)gridDim.x * blockDim.x)
    pos[tok_rows[q]] = (int32_t)q;
}

// Input gradient: dx[t] = sum over the rows r of t (ascending) of dx_perm[r]
//                        + sum over the experts e of dz[t, e] * W_g[e]   (router term)
// in fp32.  dz[t] is nonzero only at the experts of t's rows and at its top-k
// experts (router backward below), so the router term is a gather of a few W_g
// rows (L2-resident) rather than a GEMM; a top-k expert is visited here only when
// t has no row at it (token rounding dropped the pair).
// One wave per token: each lane owns four 16-byte column chunks per pass and
// issues the loads of up to RU rows (and their W_g rows) before adding them in
// ascending row order.  dX_perm rows are read once (non-temporal loads), W_g
// rows are shared by every token (ordinary loads, L2-resident).  When dz is dense (routing variants) the
// router term comes precomputed as dxr = dz W_g (fp32 [T, d], a GEMM) instead.
template <typename T, int RU>
__global__ __launch_bounds__(256) void router_dx_kernel(const T* __restrict__ dx_perm, const int32_t* __restrict__ tok_ptr,
                                                       const int32_t* __restrict__ tok_rows,
                                                       const int32_t* __restrict__ expert_of_row,
                                                       const int32_t* __restrict__ topk_idx,
                                                       const uint32_t* __restrict__ keep_bits, int words,
                                                       const float* __restrict__ dz, const T* __restrict__ wg,
                                                       const float* __restrict__ dxr,
                                                       int T_, int E, int d, int k, T* __restrict__ out) {
  constexpr int EV = 16 / sizeof(T);
  constexpr int CL = 4;                       // column chunks per lane per pass
  const int vec = d / EV;
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));   // wave-uniform
  if (t >= T_) return;
  auto add = [&](float* acc, const u32x4& v, float w) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += w * __uint_as_float(v[q] << 16);
        acc[2 * q + 1] += w * __uint_as_float(v[q] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += w * __uint_as_float(v[q]);
    }
  };
  const float* dzt = dz + (int64_t)t * E;
  const int p0 = tok_ptr[t], p1 = tok_ptr[t + 1];
  for (int cb = 0; cb < vec; cb += 64 * CL) {
    float acc[CL][EV];
#pragma unroll
    for (int j = 0; j < CL; ++j)
#pragma unroll
      for (int q = 0; q < EV; ++q) acc[j][q] = 0.0f;
    for (int p = p0; p < p1; p += RU) {       // rows in ascending order, RU with their loads in flight
      int r[RU], erow[RU];
      float z[RU];
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        r[u] = p + u < p1 ? tok_rows[p + u] : -1;
        erow[u] = r[u] >= 0 ? expert_of_row[r[u]] : 0;
        z[u] = (dxr || r[u] < 0) ? 0.0f : dzt[erow[u]];
      }
      u32x4 v[RU][CL], w[RU][CL];
#pragma unroll
      for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int j = 0; j < CL; ++j) {
          const int c = cb + lane + 64 * j;
          const bool ok = r[u] >= 0 && c < vec;
          v[u][j] = ok ? ldg16_nt(dx_perm + (int64_t)r[u] * d + c * EV) : u32x4{0u, 0u, 0u, 0u};
          w[u][j] = (ok && !dxr) ? ldg16(wg + (int64_t)erow[u] * d + c * EV) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        if (r[u] < 0) break;
#pragma unroll
        for (int j = 0; j < CL; ++j) {
          add(acc[j], v[u][j], 1.0f);
          add(acc[j], w[u][j], z[u]);
        }
      }
    }
    if (dxr) {
#pragma unroll
      for (int j = 0; j < CL; ++j) {
        const int c = cb + lane + 64 * j;
        if (c >= vec) continue;
        const float* src = dxr + (int64_t)t * d + c * EV;
#pragma unroll
        for (int q = 0; q < EV; ++q) acc[j][q] += src[q];
      }
    }
    for (int i = 0; i < k && !dxr; ++i) {
      const int e = topk_idx[(int64_t)t * k + i];
      if ((keep_bits[(int64_t)t * words + (e >> 5)] >> (e & 31)) & 1u) continue;
      const float z = dzt[e];
#pragma unroll
      for (int j = 0; j < CL; ++j) {
        const int c = cb + lane + 64 * j;
        if (c < vec) add(acc[j], ldg16(wg + (int64_t)e * d + c * EV), z);
      }
    }
#pragma unroll
    for (int j = 0; j < CL; ++j) {
      const int c = cb + lane + 64 * j;
      if (c >= vec) continue;
      u32x4 o;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf2(acc[j][2 * q], acc[j][2 * q + 1]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[j][q]);
      }
      stg16(out + (int64_t)t * d + c * EV, o);
    }
  }
}

// Router backward, one wave per token.  dS of every row is a fixed-order sum of
// the per-column-tile partials.  For token t with top-k set K (gates S) and rows
// A (gates g):  dz_e = [e in A] g_e dS_e - [e in K] S_e * sum_{A} g dS.
// Routing variants ("Beam" blog sections 2.2/2.3, distributed-MoE article,
// challenge 1) make dz dense over all E: with full-softmax gates the second
// term is -P_e * sum_A g dS (P = softmax of the token's logits); the
// load-balance loss lb_coef * CV(Pbar)^2 adds P_e (h_e - <h, P>) with
// h_e = (lb_coef / T) (2 (Pbar_e - m) / (E m^2) - 2 var / (E m^3)), m and var
// the mean and population variance of Pbar (from the forward, aux[4..]); the
// z-loss adds (2 z_coef / T) lse P_e.
// Writes dlogits (fp32) and the GEMM operand dzq, row stride ld: columns [0, ldz)
// hold dz (zero padded past E) in the act dtype; with bf16 activations columns
// [ldz, 2 ldz) hold the rounding residual bf16(dz - bf16(dz)), so the two router
// GEMMs see dz as the sum of two bf16 values (16 significant bits).
template <typename T>
__global__ __launch_bounds__(256) void router_bwd_kernel(const int32_t* __restrict__ tok_ptr,
                                                        const int32_t* __restrict__ tok_rows,
                                                        const int32_t* __restrict__ expert_of_row,
                                                        const float* __restrict__ gate_of_row,
                                                        const int32_t* __restrict__ topk_idx,
                                                        const float* __restrict__ topk_gate,
                                                        const float* __restrict__ ds_part, int nparts,
                                                        int64_t part_stride, int T_, int E, int k,
                                                        float* __restrict__ ds_out, float* __restrict__ dlogits,
                                                        T* __restrict__ dzq, int ldz, int ld, int gate_all,
                                                        const float* __restrict__ logits,
                                                        const float* __restrict__ aux, float lb_coef, float z_coef) {
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));   // wave-uniform
  if (t >= T_) return;
  const int p0 = tok_ptr[t], p1 = tok_ptr[t + 1], n = p1 - p0;
  float vals[4] = {0.f, 0.f, 0.f, 0.f};   // experts lane, lane+64, lane+128, lane+192
  float acc = 0.0f;
  // the partials of a row are summed by a group of np2 lanes (all loads in flight
  // at once, then a fixed shuffle tree); 64 / np2 rows per pass
  int np2 = 1;
  while (np2 < nparts && np2 < 64) np2 <<= 1;
  const int rpp = 64 / np2;
  for (int pb = 0; pb < n; pb += rpp) {
    const int pi = pb + lane / np2, q0 = lane % np2;
    float v = 0.0f, gr = 0.0f;
    int r = 0, er = 0;
    if (pi < n) {   // the row's gate and expert load alongside its partials
      r = tok_rows[p0 + pi];
      gr = gate_of_row[r];
      er = expert_of_row[r];
      for (int q = q0; q < nparts; q += np2) v += ds_part[q * part_stride + r];
    }
    for (int o = 1; o < np2; o <<= 1) v += __shfl_xor(v, o, 64);
    for (int u = 0; u < rpp && pb + u < n; ++u) {   // rows in ascending order
      const float ds = __shfl(v, u * np2, 64);
      const int rr = __shfl(r, u * np2, 64);
      if (ds_out && lane == 0) ds_out[rr] = ds;
      const float gds = __shfl(gr, u * np2, 64) * ds;
      acc += gds;
      const int e = __shfl(er, u * np2, 64);
      if ((e & 63) == lane) vals[e >> 6] += gds;
    }
  }
  const bool dense = gate_all || lb_coef != 0.0f || z_coef != 0.0f;   // uniform over the grid
  if (!gate_all) {
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[(int64_t)t * k + j];
      if ((e & 63) == lane) vals[e >> 6] -= topk_gate[(int64_t)t * k + j] * acc;
    }
  }
  if (dense) {
    // the token's full softmax P and log-sum-exp from its logits
    float z[4], P[4];
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = lane + 64 * v;
      z[v] = e < E ? logits[(int64_t)t * E + e] : -INFINITY;
      m = fmaxf(m, z[v]);
    }
    m = wave_max(m);
    float sl = 0.0f;
#pragma unroll
    for (int v = 0; v < 4; ++v) sl += (lane + 64 * v < E) ? expf(z[v] - m) : 0.0f;
    const float se = wave_sum(sl);
#pragma unroll
    for (int v = 0; v < 4; ++v) P[v] = (lane + 64 * v < E) ? expf(z[v] - m) / se : 0.0f;
    if (gate_all) {
#pragma unroll
      for (int v = 0; v < 4; ++v) vals[v] -= P[v] * acc;
    }
    if (lb_coef != 0.0f) {
      float pb[4], sp = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pb[v] = (lane + 64 * v < E) ? aux[4 + lane + 64 * v] : 0.0f;
        sp += pb[v];
      }
      const float mean = wave_sum(sp) / (float)E;
      float sv = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) sv += (lane + 64 * v < E) ? (pb[v] - mean) * (pb[v] - mean) : 0.0f;
      const float var = wave_sum(sv) / (float)E;
      float h[4], sh = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        h[v] = (lane + 64 * v < E)
                   ? (lb_coef / (float)T_) * (2.0f * (pb[v] - mean) / ((float)E * mean * mean) -
                                              2.0f * var / ((float)E * mean * mean * mean))
                   : 0.0f;
        sh += h[v] * P[v];
      }
      const float hp = wave_sum(sh);
#pragma unroll
      for (int v = 0; v < 4; ++v) vals[v] += P[v] * (h[v] - hp);
    }
    if (z_coef != 0.0f) {
      const float c = 2.0f * z_coef / (float)T_ * (m + logf(se));
#pragma unroll
      for (int v = 0; v < 4; ++v) vals[v] += c * P[v];
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int e = lane + 64 * v;
    if (e < E) dlogits[(int64_t)t * E + e] = vals[v];
    if (e < ldz) {
      const float z = e < E ? vals[v] : 0.0f;
      if constexpr (sizeof(T) == 2) {
        const bf16_t hi = f2bf(z);
        dzq[(int64_t)t * ld + e] = hi;
        dzq[(int64_t)t * ld + ldz + e] = f2bf(z - bf2f(hi));   // exact difference in fp32
      } else {
        dzq[(int64_t)t * ld + e] = z;
      }
    }
  }
}

// dW_g from the split-K partials of the router-weight GEMM: part[q] holds rows
// [0, E) (the dz columns) and, when lo_row >= 0, rows [lo_row, lo_row + E) (their
// bf16 residuals); out[e] = sum_q part[q][e] + sum_q part[q][lo_row + e], each sum
// in split order.
__global__ __launch_bounds__(256) void router_dwg_reduce_kernel(const float* __restrict__ part, int nsplit,
                                                               int64_t pstride, int64_t n, int64_t lo_off,
                                                               float* __restrict__ out) {
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += (int64_t)gridDim.x * 256 * 4) {
    f32x4 hi = {0.f, 0.f, 0.f, 0.f}, lo = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < nsplit; ++q) {
      const f32x4 a = ldf4_nt(part + q * pstride + i);
      f32x4 b = {0.f, 0.f, 0.f, 0.f};
      if (lo_off >= 0) b = ldf4_nt(part + q * pstride + lo_off + i);
      hi += a;
      lo += b;
    }
    *reinterpret_cast<f32x4*>(out + i) = hi + lo;
  }
}

// B operand of the dense router term with split dz: rows [0, E) and [ldz, ldz + E)
// are W_g, the rows between and after are zero ([2 ldz, d] bf16).
__global__ __launch_bounds__(256) void router_wg2_kernel(const bf16_t* __restrict__ wg, int E, int ldz, int d,
                                                        bf16_t* __restrict__ wg2) {
  const int64_t n = (int64_t)2 * ldz * d / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t el = i * 8;
    const int r = (int)(el / d), c = (int)(el % d);
    const int src = r < ldz ? r : r - ldz;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (src < E) v = ldg16(wg + (int64_t)src * d + c);
    stg16(wg2 + el, v);
  }
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int nsplit, int64_t n,
                                                           float* __restrict__ out) {
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += (int64_t)gridDim.x * 256 * 4) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    int q = 0;
    for (; q + 8 <= nsplit; q += 8) {   // eight partials' loads in flight, added in split order
      f32x4 p[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) p[u] = ldf4_nt(part + (q + u) * n + i);
#pragma unroll
      for (int u = 0; u < 8; ++u) s += p[u];
    }
    for (; q < nsplit; ++q) s += ldf4_nt(part + q * n + i);
    *reinterpret_cast<f32x4*>(out + i) = s;
  }
}

// Weight-gradient chunks: expert e's reduction rows [off[e], off[e+1]) are cut
// into ch_e = max(1, ceil(n_e / kch)) pieces of at most kch rows.  Chunk c of
// expert e is (e, k0, k1, slot): slot -1 for c = 0 (written to the expert's
// own gradient), else one of the expert's consecutive partial slots
// slot_range[e] = [first, last + 1).  One block, E <= 256.
__global__ __launch_bounds__(256) void wgrad_chunks_kernel(const int32_t* __restrict__ off, int E, int kch,
                                                          int4* __restrict__ chunks, int32_t* __restrict__ nchunks,
                                                          int2* __restrict__ slot_range) {
  __shared__ int sq[256], ss[256];
  const int e = threadIdx.x;
  int n = 0, ch = 0;
  if (e < E) {
    n = off[e + 1] - off[e];
    ch = n > 0 ? (n + kch - 1) / kch : 1;
  }
  sq[e] = ch;
  ss[e] = ch > 0 ? ch - 1 : 0;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {   // inclusive scans
    const int a = e >= o ? sq[e - o] : 0, b = e >= o ? ss[e - o] : 0;
    __syncthreads();
    sq[e] += a;
    ss[e] += b;
    __syncthreads();
  }
  if (e >= E) return;
  const int q0 = sq[e] - ch, s0 = ss[e] - (ch - 1);
  for (int c = 0; c < ch; ++c) {
    const int k0 = off[e] + c * kch;
    chunks[q0 + c] = int4{e, k0, min(off[e + 1], k0 + kch), c == 0 ? -1 : s0 + c - 1};
  }
  slot_range[e] = int2{s0, s0 + ch - 1};
  if (e == E - 1) *nchunks = sq[e];
}

// dW[e] += partial slots of e, in slot order (fixed order: deterministic).
// Every block walks all experts (those without partial slots are skipped at
// once), so a heavily loaded expert's partials are spread over the whole grid.
// The experts that have partial slots are listed in LDS first (E <= 256, one
// thread each; the list order does not matter, each expert's sum is its own).
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(float* __restrict__ dw, const float* __restrict__ part,
                                                          const int2* __restrict__ slot_range, int E, int64_t mn) {
  __shared__ int2 srs[256];
  __shared__ int act[256];
  __shared__ int nact;
  if (threadIdx.x == 0) nact = 0;
  __syncthreads();
  if ((int)threadIdx.x < E) {
    const int2 sr = slot_range[threadIdx.x];
    if (sr.y > sr.x) {
      const int i = atomicAdd(&nact, 1);
      act[i] = threadIdx.x;
      srs[i] = sr;
    }
  }
  __syncthreads();
  for (int a = 0; a < nact; ++a) {
    const int e = act[a];
    const int2 sr = srs[a];
    float* out = dw + (int64_t)e * mn;
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < mn; i += (int64_t)gridDim.x * 256 * 4) {
      f32x4 a = *reinterpret_cast<const f32x4*>(out + i);
      for (int s = sr.x; s < sr.y; ++s) a += ldf4_nt(part + (int64_t)s * mn + i);
      *reinterpret_cast<f32x4*>(out + i) = a;
    }
  }
}

int grid_for(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g > 256 * 32) g = 256 * 32;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

hipError_t launch_permute_rows(const moe_shape& s, const void* src, const moe_plan& p, void* dst, hipStream_t st) {
  const int esz = s.act == MOE_BF16 ? 2 : 4;
  const int vec = s.d * esz / 16;
  if (vec % 4 == 0) {
    const int64_t work = (int64_t)s.T * (vec / 4);
    hipLaunchKernelGGL(scatter_rows_kernel<4>, dim3(grid_for(work, 256)), dim3(256), 0, st, (const char*)src,
                       p.tok_ptr, p.tok_rows, s.T, vec, (char*)dst);
  } else {
    const int64_t work = (int64_t)s.T * vec;
    hipLaunchKernelGGL(scatter_rows_kernel<1>, dim3(grid_for(work, 256)), dim3(256), 0, st, (const char*)src,
                       p.tok_ptr, p.tok_rows, s.T, vec, (char*)dst);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const moe_shape& s, const void* y, const moe_plan& p, void* out, hipStream_t st) {
  if (s.act == MOE_BF16)
    hipLaunchKernelGGL((combine_kernel<bf16_t, 1>), dim3(ceil_div(s.T, 4)), dim3(256), 0, st, (const bf16_t*)y,
                       p.tok_ptr, p.tok_rows, p.gate_of_row, s.T, s.d, (bf16_t*)out);
  else
    hipLaunchKernelGGL((combine_kernel<float, 1>), dim3(ceil_div(s.T, 4)), dim3(256), 0, st, (const float*)y,
                       p.tok_ptr, p.tok_rows, p.gate_of_row, s.T, s.d, (float*)out);
  return hipGetLastError();
}

hipError_t launch_segment_sum(const moe_shape& s, const void* yg, const moe_plan& p, void* out, hipStream_t st) {
  if (s.act != MOE_BF16) return hipErrorInvalidValue;
  hipLaunchKernelGGL((combine_kernel<bf16_t, 1, true>), dim3(ceil_div(s.T, 4)), dim3(256), 0, st,
                     (const bf16_t*)yg, p.tok_ptr, p.tok_rows, p.gate_of_row, s.T, s.d, (bf16_t*)out);
  return hipGetLastError();
}

hipError_t launch_row_positions(const moe_shape& s, const moe_plan& p, int32_t* pos, hipStream_t st) {
  const int64_t n = max_rows(s);
  hipLaunchKernelGGL(row_positions_kernel, dim3(grid_for(n, 256)), dim3(256), 0, st, p.tok_rows, p.tok_ptr, s.T, n,
                     pos);
  return hipGetLastError();
}

hipError_t launch_router_dx(const moe_shape& s, const moe_plan& p, const void* dx_perm, const float* dz,
                            const void* wg, const float* dxr, void* dx, hipStream_t st) {
  const int words = (s.E + 31) / 32;
  if (s.act == MOE_BF16) {
    hipLaunchKernelGGL((router_dx_kernel<bf16_t, 1>), dim3(ceil_div(s.T, 4)), dim3(256), 0, st, (const bf16_t*)dx_perm,
                       p.tok_ptr, p.tok_rows, p.expert_of_row, p.topk_idx, p.keep_bits, words, dz,
                       (const bf16_t*)wg, dxr, s.T, s.E, s.d, s.k, (bf16_t*)dx);
  } else {
    hipLaunchKernelGGL((router_dx_kernel<float, 1>), dim3(ceil_div(s.T, 4)), dim3(256), 0, st, (const float*)dx_perm,
                       p.tok_ptr, p.tok_rows, p.expert_of_row, p.topk_idx, p.keep_bits, words, dz,
                       (const float*)wg, dxr, s.T, s.E, s.d, s.k, (float*)dx);
  }
  return hipGetLastError();
}

hipError_t launch_router_bwd(const moe_shape& s, const moe_plan& p, const float* ds_part, int nparts,
                             float* ds_out, float* dlogits, void* dzq, hipStream_t st) {
  const int ldz = router_ldz(s), ld = router_dz_ld(s);
  const int grid = ceil_div(s.T, 4);
  const int64_t pstride = max_rows(s);
  if (s.act == MOE_BF16)
    hipLaunchKernelGGL(router_bwd_kernel<bf16_t>, dim3(grid), dim3(256), 0, st, p.tok_ptr, p.tok_rows,
                       p.expert_of_row, p.gate_of_row, p.topk_idx, p.topk_gate, ds_part, nparts, pstride, s.T, s.E,
                       s.k, ds_out, dlogits, (bf16_t*)dzq, ldz, ld, (int)(s.gate_mode == MOE_GATE_ALL), p.logits,
                       p.aux, s.lb_coef, s.z_coef);
  else
    hipLaunchKernelGGL(router_bwd_kernel<float>, dim3(grid), dim3(256), 0, st, p.tok_ptr, p.tok_rows,
                       p.expert_of_row, p.gate_of_row, p.topk_idx, p.topk_gate, ds_part, nparts, pstride, s.T, s.E,
                       s.k, ds_out, dlogits, (float*)dzq, ldz, ld, (int)(s.gate_mode == MOE_GATE_ALL), p.logits,
                       p.aux, s.lb_coef, s.z_coef);
  return hipGetLastError();
}

hipError_t launch_wgrad_chunks(const int32_t* offsets, int E, int kch, const WgradChunks& w, hipStream_t st) {
  hipLaunchKernelGGL(wgrad_chunks_kernel, dim3(1), dim3(256), 0, st, offsets, E, kch, w.chunks, w.nchunks,
                     w.slot_range);
  return hipGetLastError();
}

hipError_t launch_wgrad_reduce(const WgradChunks& w, int E, int64_t mn, float* dw, hipStream_t st) {
  if (w.max_extra == 0) return hipSuccess;
  hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(1024), dim3(256), 0, st, dw, w.part, w.slot_range, E, mn);
  return hipGetLastError();
}

hipError_t launch_router_dwg_reduce(const float* part, int nsplit, int64_t pstride, int E, int d, int lo_row,
                                    float* out, hipStream_t st) {
  const int64_t n = (int64_t)E * d;
  hipLaunchKernelGGL(router_dwg_reduce_kernel, dim3(grid_for(n / 4, 256)), dim3(256), 0, st, part, nsplit, pstride,
                     n, lo_row >= 0 ? (int64_t)lo_row * d : (int64_t)-1, out);
  return hipGetLastError();
}

hipError_t launch_router_wg2(const void* wg, int E, int ldz, int d, void* wg2, hipStream_t st) {
  hipLaunchKernelGGL(router_wg2_kernel, dim3(grid_for((int64_t)2 * ldz * d / 8, 256)), dim3(256), 0, st,
                     (const bf16_t*)wg, E, ldz, d, (bf16_t*)wg2);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* part, int nsplit, int64_t n, float* out, hipStream_t st) {
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid_for(n / 4, 256)), dim3(256), 0, st, part, nsplit, n, out);
  return hipGetLastError();
}

}  // namespace moe
