// Routing kernels: wave64 top-k with softmax over the selected logits, the
// deterministic plan build (histogram -> prefix scan -> stable scatter by token)
// and token rounding.
//
// Top-k follows the "Beam" blog (section 5.3) and the "Trinity Large" commentary
// (code example 1): experts are ranked by logit, the k best are kept and their
// gates are a softmax over those k logits.  Ties go to the lower expert index.
// With MOE_GATE_ALL the gates are the full softmax at the selected experts,
// not renormalised (the blog's section 2.2 formula; its section 3.3 names the
// choice).  Routing variants of its section 2.3 and of the distributed-MoE
// article (challenge 1): a per-expert capacity that drops the pairs past it in
// token order, and the load-balance loss CV(Pbar)^2 and z-loss, reduced here
// in a fixed order.
// The plan lays the token-expert pairs out as contiguous per-expert row
// segments ("row-wise" expert buffers of the Olmo-core 3 article, "three splits"
// section), tokens ascending inside a segment; everything stays on the device.
// Token rounding follows the SonicMoE article, section 3.
#include <climits>
#include <cmath>
#include <cstdint>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxTopK = 8;   // the library's limit on k (checked on the host)

// Logits as order-preserving integers for the selection: a larger key is a
// larger value, -0 maps to +0 (they tie), and INT_MIN lies below every key of a
// number (the slot of a taken or absent expert).
MOE_DEV int order_key(float v) {
  const int b = v == 0.0f ? 0 : __float_as_int(v);
  return b ^ ((b >> 31) & 0x7fffffff);
}
MOE_DEV float key_float(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7fffffff)); }

// Wave-wide maximum of an int (uniform result): DPP maxima inside each 16-lane
// row, then rows 0-1 and 2-3 (row_bcast:15), then all four (row_bcast:31), which
// leaves it in lane 63.
template <int CTRL, int ROWS>
MOE_DEV int dpp_imax(int v) {
  // lanes outside ROWS read INT_MIN, the identity of max
  return max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, CTRL, ROWS, 0xf, false));
}
MOE_DEV int wave_max_i32(int v) {
  v = dpp_imax<0xB1, 0xf>(v);    // quad_perm [1,0,3,2]
  v = dpp_imax<0x4E, 0xf>(v);    // quad_perm [2,3,0,1]
  v = dpp_imax<0x141, 0xf>(v);   // row_half_mirror
  v = dpp_imax<0x140, 0xf>(v);   // row_mirror: every lane holds its row's maximum
  v = dpp_imax<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_imax<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}

// One wave per token; a wave takes TPW tokens in turn (NT/64*TPW per block).  Lane
// l holds experts l, l+64, ...  With ROUND (64 tokens per block: sixteen waves of
// four) the block also writes the full softmax expert-major (probs_t) and the
// selection bitmap expert-major (sel_t), transposed through LDS.
template <int V, bool ROUND, int TPW, int NT>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
                                                  uint32_t* __restrict__ keep_bits, int words,
                                                  float* __restrict__ probs_t, uint32_t* __restrict__ sel_t,
                                                  int wordsT, int gate_all) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* pt = reinterpret_cast<float*>(smem);                       // [E][65]: a wave's writes (one expert
                                                                    // per lane) fall in distinct banks
  uint32_t* sel = reinterpret_cast<uint32_t*>(smem + (size_t)E * 65 * 4);  // [E][2]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  static_assert(!ROUND || (NT / 64) * TPW == 64, "the transposed writes assume 64 tokens per block");
  const int t0 = blockIdx.x * (NT / 64) * TPW;
  if constexpr (ROUND) {
    for (int i = threadIdx.x; i < E * 2; i += NT) sel[i] = 0u;
    __syncthreads();
  }
  for (int it = 0; it < TPW; ++it) {
    const int tl = wave * TPW + it;
    const int t = t0 + tl;
    if (t >= T) break;
    float z[V];
    int ks[V];   // selection keys of the candidates (INT_MIN once taken, or absent)
#pragma unroll
    for (int v = 0; v < V; ++v) {
      int e = lane + 64 * v;
      z[v] = (e < E) ? logits[(int64_t)t * E + e] : -INFINITY;
      ks[v] = (e < E) ? order_key(z[v]) : INT_MIN;
    }
    // Round j: the largest candidate key, then the lowest expert index holding
    // it (expert lane + 64 v: the first slot v with a match, its lowest lane).
    // k <= E leaves a candidate in every round.  The loops over the k selections
    // run to kMaxTopK with a uniform j < k test, so sel_e / sel_z are indexed by
    // constants (a runtime index costs a select chain over all 8 per access).
    int sel_e[kMaxTopK];
    float sel_z[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= k) break;
      int m = ks[0];
#pragma unroll
      for (int v = 1; v < V; ++v) m = max(m, ks[v]);
      const int bk = wave_max_i32(m);
      int be = -1;
#pragma unroll
      for (int v = V - 1; v >= 0; --v) {
        const uint64_t hit = __builtin_amdgcn_ballot_w64(ks[v] == bk);
        if (hit) be = 64 * v + (int)__builtin_ctzll(hit);
      }
      sel_e[j] = be;
      sel_z[j] = key_float(bk);
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (lane + 64 * v == be) ks[v] = INT_MIN;
    }
    // softmax over the k selected logits (the first is the largest), or the
    // full softmax's denominator (gate_all, uniform over the wave)
    float den = 0.0f;
    if (gate_all) {
      float sa = 0.0f;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (lane + 64 * v < E) sa += expf(z[v] - sel_z[0]);
      den = wave_sum(sa);
    } else {
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (j < k) den += expf(sel_z[j] - sel_z[0]);
    }
    if (lane < k) {
      float zj = sel_z[0];
      int ej = sel_e[0];
#pragma unroll
      for (int j = 1; j < kMaxTopK; ++j)
        if (j < k && lane == j) { zj = sel_z[j]; ej = sel_e[j]; }
      topk_idx[(int64_t)t * k + lane] = ej;
      topk_gate[(int64_t)t * k + lane] = expf(zj - sel_z[0]) / den;
    }
    if (lane < words) {
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (j < k && (sel_e[j] >> 5) == lane) w |= 1u << (sel_e[j] & 31);
      keep_bits[(int64_t)t * words + lane] = w;
    }
    if constexpr (ROUND) {
      float s = 0.0f;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (lane + 64 * v < E) s += expf(z[v] - sel_z[0]);
      s = wave_sum(s);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        int e = lane + 64 * v;
        if (e < E) pt[e * 65 + tl] = expf(z[v] - sel_z[0]) / s;
      }
      if (lane < k) {
        int ej = sel_e[0];
#pragma unroll
        for (int j = 1; j < kMaxTopK; ++j)
          if (j < k && lane == j) ej = sel_e[j];
        atomicOr(&sel[ej * 2 + (tl >> 5)], 1u << (tl & 31));
      }
    }
  }
  if constexpr (ROUND) {
    __syncthreads();
    for (int i = threadIdx.x; i < E * 64; i += NT) {
      int e = i >> 6, tl = i & 63;
      if (t0 + tl < T) probs_t[(int64_t)e * T + t0 + tl] = pt[e * 65 + tl];
    }
    for (int i = threadIdx.x; i < E * 2; i += NT) {
      int e = i >> 1, h = i & 1;
      int wi = blockIdx.x * 2 + h;
      if (wi < wordsT) sel_t[(int64_t)e * wordsT + wi] = sel[i];
    }
  }
}

// Per-(wave, expert) 64-bit masks of the tokens of a 256-token block that keep
// the expert: bit l of mask[w][e] = token (block, w, l) has a row at e.
struct BlockMasks {
  uint32_t* m;  // [4][E][2]
  int E;
  MOE_DEV uint32_t& at(int w, int e, int h) { return m[(w * E + e) * 2 + h]; }
};

MOE_DEV void build_masks(BlockMasks bm, const uint32_t* keep_bits, int words, int t, bool valid,
                         int* tok_count) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * bm.E * 2; i += 256) bm.m[i] = 0u;
  __syncthreads();
  int cnt = 0;
  if (valid) {
    for (int w = 0; w < words; ++w) {
      uint32_t bits = keep_bits[(int64_t)t * words + w];
      cnt += __popc(bits);
      while (bits) {
        int b = __ffs(bits) - 1;
        bits &= bits - 1;
        atomicOr(&bm.at(wave, w * 32 + b, lane >> 5), 1u << (lane & 31));
      }
    }
  }
  *tok_count = cnt;
  __syncthreads();
}

__global__ __launch_bounds__(256) void plan_count_kernel(const uint32_t* __restrict__ keep_bits, int T, int E,
                                                        int words, int nblk, int32_t* __restrict__ hist,
                                                        int32_t* __restrict__ blk_tok) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  BlockMasks bm{reinterpret_cast<uint32_t*>(smem), E};
  __shared__ int red[256];
  const int t = blockIdx.x * 256 + threadIdx.x;
  int cnt;
  build_masks(bm, keep_bits, words, t, t < T, &cnt);
  for (int e = threadIdx.x; e < E; e += 256) {
    int h = 0;
    for (int w = 0; w < 4; ++w) h += __popc(bm.at(w, e, 0)) + __popc(bm.at(w, e, 1));
    hist[(int64_t)e * nblk + blockIdx.x] = h;
  }
  red[threadIdx.x] = cnt;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) blk_tok[blockIdx.x] = red[0];
}

// Inclusive prefix sum across the 64 lanes of a wave.
MOE_DEV int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive scan of one int per thread over a 1024-thread block (sh: >= 17
// ints); returns the thread's exclusive prefix, *total the block's sum.
MOE_DEV int block_excl_scan_1024(int x, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < 16 ? sh[lane] : 0;
    const int wi = wave_incl_scan(w);
    if (lane < 16) sh[lane] = wi - w;
    if (lane == 15) sh[16] = wi;
  }
  __syncthreads();
  const int r = sh[wave] + incl - x;
  *total = sh[16];
  __syncthreads();
  return r;
}

// Exclusive scan of n ints in place by one 1024-thread block; returns the total.
// Batches of 16 chunks of 1024 elements: each thread loads one element of every
// chunk (coalesced, all 16 loads in flight), every chunk is scanned across the
// waves with lane shuffles, then one pass over the 16 x 16 wave totals.
MOE_DEV int block_scan_inplace(int32_t* a, int64_t n, int* sh /* >= 272 ints */) {
  constexpr int B = 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int64_t base = 0; base < n; base += (int64_t)B * 1024) {
    int v[B], incl[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int64_t i = base + (int64_t)j * 1024 + tid;
      v[j] = i < n ? a[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < B; ++j) incl[j] = wave_incl_scan(v[j]);
    if (lane == 63) {
#pragma unroll
      for (int j = 0; j < B; ++j) sh[j * 16 + wave] = incl[j];
    }
    __syncthreads();
    if (wave == 0) {   // exclusive scan of the 256 wave totals in (chunk, wave) order, 4 per lane
      int q[4], sum = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) { q[u] = sh[4 * lane + u]; sum += q[u]; }
      int run = wave_incl_scan(sum) - sum;
#pragma unroll
      for (int u = 0; u < 4; ++u) { sh[4 * lane + u] = run; run += q[u]; }
      if (lane == 63) sh[256] = run;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int64_t i = base + (int64_t)j * 1024 + tid;
      if (i < n) a[i] = carry + sh[j * 16 + wave] + incl[j] - v[j];
    }
    carry += sh[256];
    __syncthreads();
  }
  return carry;
}

__global__ __launch_bounds__(1024) void plan_scan_kernel(int E, int nblk, int32_t* __restrict__ hist,
                                                        int32_t* __restrict__ blk_tok, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ counts_raw, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ pre128, int32_t* __restrict__ tile_e,
                                                        float* __restrict__ aux) {
  __shared__ int sh[1024];
  __shared__ double red[1024];
  const int total = block_scan_inplace(hist, (int64_t)E * nblk, sh);
  const int toks = block_scan_inplace(blk_tok, nblk, sh);
  if (threadIdx.x == 0) blk_tok[nblk] = toks;
  // one thread per expert (E <= 256 < 1024)
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
    const int o = hist[(int64_t)e * nblk];
    const int o1 = (e + 1 < E) ? hist[(int64_t)(e + 1) * nblk] : total;
    cnt = o1 - o;
    offsets[e] = o;
    counts[e] = cnt;
    if (counts_raw) counts_raw[e] = cnt;
  }
  if (e == 0) offsets[E] = total;
  if (aux) {   // count monitor (Trinity Large example 2): mean_e (c_e - mean c)^2, fixed-order tree sums
    red[e] = (double)cnt;
    __syncthreads();
    for (int o = 512; o > 0; o >>= 1) {
      if (e < o) red[e] += red[e + o];
      __syncthreads();
    }
    const double mean = red[0] / E;
    __syncthreads();
    red[e] = e < E ? ((double)cnt - mean) * ((double)cnt - mean) : 0.0;
    __syncthreads();
    for (int o = 512; o > 0; o >>= 1) {
      if (e < o) red[e] += red[e + o];
      __syncthreads();
    }
    if (e == 0) aux[2] = (float)(red[0] / E);
  }
  // 128-row m-tile prefix over the experts (block scan), then each expert's tiles
  const int tiles = (cnt + 127) / 128;
  int all_tiles;
  const int p0 = block_excl_scan_1024(tiles, sh, &all_tiles);
  if (e < E) {
    pre128[e] = p0;
    if (e == E - 1) pre128[E] = p0 + tiles;
    for (int j = 0; j < tiles; ++j) tile_e[p0 + j] = e;
  }
}

__global__ __launch_bounds__(256) void plan_scatter_kernel(
    const uint32_t* __restrict__ keep_bits, int T, int E, int k, int words, int nblk,
    const int32_t* __restrict__ hist, const int32_t* __restrict__ blk_tok, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_gate, const float* __restrict__ probs_t, bool prob_gates, bool gate_all,
    int32_t* __restrict__ token_of_row, int32_t* __restrict__ expert_of_row, float* __restrict__ gate_of_row,
    int32_t* __restrict__ row_of_slot, int32_t* __restrict__ tok_ptr, int32_t* __restrict__ tok_rows) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  BlockMasks bm{reinterpret_cast<uint32_t*>(smem), E};
  int* hb = reinterpret_cast<int*>(smem + (size_t)4 * E * 2 * 4);   // [E] this block's first row per expert
  __shared__ int sc[256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const bool valid = t < T;
  for (int e = threadIdx.x; e < E; e += 256) hb[e] = hist[(int64_t)e * nblk + blockIdx.x];
  int cnt;
  build_masks(bm, keep_bits, words, t, valid, &cnt);   // (its barriers also publish hb)
  // token -> first row slot in tok_rows (block base + exclusive scan of counts)
  sc[threadIdx.x] = cnt;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    int v = (threadIdx.x >= o) ? sc[threadIdx.x - o] : 0;
    __syncthreads();
    sc[threadIdx.x] += v;
    __syncthreads();
  }
  const int tbase = blk_tok[blockIdx.x] + sc[threadIdx.x] - cnt;
  if (blockIdx.x == 0 && threadIdx.x == 0) tok_ptr[T] = blk_tok[nblk];
  if (!valid) return;
  tok_ptr[t] = tbase;
  const uint32_t ltmask = (1u << (lane & 31)) - 1u;
  auto row_of = [&](int e) -> int {
    int r = hb[e];
    for (int w = 0; w < wave; ++w) r += __popc(bm.at(w, e, 0)) + __popc(bm.at(w, e, 1));
    if (lane >= 32) r += __popc(bm.at(wave, e, 0));
    r += __popc(bm.at(wave, e, lane >> 5) & ltmask);
    return r;
  };
  float ptop = 0.0f;
  if (prob_gates && !gate_all)
    for (int j = 0; j < k; ++j) ptop += probs_t[(int64_t)topk_idx[(int64_t)t * k + j] * T + t];
  int tk[8];   // k <= 8
#pragma unroll
  for (int j = 0; j < 8; ++j) tk[j] = j < k ? topk_idx[(int64_t)t * k + j] : -1;
  for (int j = 0; j < k; ++j) row_of_slot[(int64_t)t * k + j] = -1;
  int n = 0;
  for (int w = 0; w < words; ++w) {
    uint32_t bits = keep_bits[(int64_t)t * words + w];
    while (bits) {
      int b = __ffs(bits) - 1;
      bits &= bits - 1;
      int e = w * 32 + b;
      int r = row_of(e);
      int slot = -1;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (tk[j] == e) slot = j;
      float g;
      if (slot >= 0) {
        g = topk_gate[(int64_t)t * k + slot];
        row_of_slot[(int64_t)t * k + slot] = r;
      } else {
        g = probs_t[(int64_t)e * T + t];          // pair added by token rounding
        if (!gate_all) g /= ptop;
      }
      token_of_row[r] = t;
      expert_of_row[r] = e;
      gate_of_row[r] = g;
      tok_rows[tbase + n] = r;
      ++n;
    }
  }
}

// Token rounding, one 1024-thread block per expert: radix-select the cut among
// the candidates (selected pairs when dropping, unselected tokens when adding)
// and flip their keep bits.  Thread i owns a contiguous run of tokens (the tie
// rule needs token order); the column sits in LDS with one pad word per 32
// tokens, so the runs of consecutive threads fall in different banks.
MOE_DEV int rs_pad(int t) { return t + (t >> 5); }

__global__ __launch_bounds__(1024) void round_select_kernel(const float* __restrict__ probs_t,
                                                           const uint32_t* __restrict__ sel_t, int wordsT,
                                                           const int32_t* __restrict__ counts_raw, int T, int tile,
                                                           uint32_t* __restrict__ keep_bits, int words,
                                                           bool col_in_lds) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int hist[256];
  __shared__ int sh[32];
  __shared__ int bc[2];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = counts_raw[e];
  int target = ((n + tile / 2) / tile) * tile;
  if (target > T) target = (n / tile) * tile;
  if (target == n) return;
  const bool drop = target < n;
  int c = drop ? n - target : target - n;
  const uint32_t* selrow = sel_t + (int64_t)e * wordsT;
  const float* col = probs_t + (int64_t)e * T;
  float* lc = reinterpret_cast<float*>(smem);
  if (col_in_lds) {
    for (int i = tid; i < T; i += 1024) lc[rs_pad(i)] = col[i];
    __syncthreads();
  }
  auto is_cand = [&](int t) -> bool {
    bool s = (selrow[t >> 5] >> (t & 31)) & 1u;
    return drop ? s : !s;
  };
  auto key_of = [&](int t) -> uint32_t {
    uint32_t b = __float_as_uint(col_in_lds ? lc[rs_pad(t)] : col[t]);   // P >= 0: bit order = value order
    return drop ? b : ~b;                   // ascending key = order of removal / addition
  };
  const int per = (T + 1023) / 1024;
  const int lo = min(tid * per, T), hi = min(lo + per, T);
  uint32_t prefix = 0u, mask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int t = lo; t < hi; ++t) {
      if (!is_cand(t)) continue;
      uint32_t kk = key_of(t);
      if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & 255], 1);
    }
    __syncthreads();
    if (wave == 0) {   // the digit where the running count reaches c: four digits per lane
      int h[4], sum = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) { h[u] = hist[4 * lane + u]; sum += h[u]; }
      int cum = wave_incl_scan(sum) - sum;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (cum < c && cum + h[u] >= c) { bc[0] = 4 * lane + u; bc[1] = c - cum; }
        cum += h[u];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)bc[0] << shift;
    mask |= 255u << shift;
    c = bc[1];
    __syncthreads();
  }
  // c = number of candidates with key == prefix to take; ties go by token
  int ties = 0;
  for (int t = lo; t < hi; ++t)
    if (is_cand(t) && key_of(t) == prefix) ++ties;
  int total_ties;
  int rank = block_excl_scan_1024(ties, sh, &total_ties);
  const uint32_t bit = 1u << (e & 31);
  for (int t = lo; t < hi; ++t) {
    if (!is_cand(t)) continue;
    uint32_t kk = key_of(t);
    bool take = kk < prefix;
    if (kk == prefix) {
      // dropping removes the larger tokens first, adding takes the smaller first
      take = drop ? (rank >= total_ties - c) : (rank < c);
      ++rank;
    }
    if (!take) continue;
    uint32_t* w = keep_bits + (int64_t)t * words + (e >> 5);
    if (drop) atomicAnd(w, ~bit);
    else atomicOr(w, bit);
  }
}

// Capacity: rows of expert e past its first C (rows are in token order) lose
// their keep bit; the plan is rebuilt from the remaining bits.
__global__ __launch_bounds__(256) void capacity_drop_kernel(const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ token_of_row,
                                                           const int32_t* __restrict__ expert_of_row, int E,
                                                           int64_t nmax, int64_t C, uint32_t* __restrict__ keep_bits,
                                                           int words) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= nmax || r >= offsets[E]) return;
  const int e = expert_of_row[r];
  if (r - offsets[e] < C) return;
  atomicAnd(keep_bits + (int64_t)token_of_row[r] * words + (e >> 5), ~(1u << (e & 31)));
}

// Router losses, pass 1: block b sums the full softmax P_t and lse_t^2 of its
// kLossTokens tokens (wave w: 16 consecutive tokens in order; then the four
// waves in order) into part[b][0..E) and part[b][E].
template <int V>
__global__ __launch_bounds__(256) void router_loss_partial_kernel(const float* __restrict__ logits, int T, int E,
                                                                 float* __restrict__ part) {
  __shared__ float wp[4][257];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float ps[V];
#pragma unroll
  for (int v = 0; v < V; ++v) ps[v] = 0.0f;
  float zs = 0.0f;
  for (int i = 0; i < kLossTokens / 4; ++i) {
    const int t = blockIdx.x * kLossTokens + wave * (kLossTokens / 4) + i;
    if (t >= T) break;
    float z[V];
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = lane + 64 * v;
      z[v] = e < E ? logits[(int64_t)t * E + e] : -INFINITY;
      m = fmaxf(m, z[v]);
    }
    m = wave_max(m);
    float sl = 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v) sl += (lane + 64 * v < E) ? expf(z[v] - m) : 0.0f;
    const float s = wave_sum(sl);
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (lane + 64 * v < E) ps[v] += expf(z[v] - m) / s;
    const float lse = m + logf(s);
    zs += lse * lse;
  }
#pragma unroll
  for (int v = 0; v < V; ++v)
    if (lane + 64 * v < E) wp[wave][lane + 64 * v] = ps[v];
  if (lane == 0) wp[wave][256] = zs;
  __syncthreads();
  const int e = threadIdx.x;
  if (e < E) part[(int64_t)blockIdx.x * (E + 1) + e] = ((wp[0][e] + wp[1][e]) + wp[2][e]) + wp[3][e];
  if (e == 0)
    part[(int64_t)blockIdx.x * (E + 1) + E] = ((wp[0][256] + wp[1][256]) + wp[2][256]) + wp[3][256];
}

// Pass 2 (one block of 1024): Pbar, CV^2 = var / mean^2 (population variance
// over the E entries), lb = lb_coef * CV^2, z-loss = z_coef * sum lse^2 / T.
// Column e (E = the lse^2 column) is summed by four threads over the blocks
// b = q mod 4, then the four sums in order: a fixed order.
__global__ __launch_bounds__(1024) void router_loss_final_kernel(const float* __restrict__ part, int nb, int T, int E,
                                                                float lb_coef, float z_coef,
                                                                float* __restrict__ aux) {
  __shared__ float q4[4][257];
  __shared__ float red[256];
  {
    const int c = threadIdx.x & 255, q = threadIdx.x >> 8;
    float acc = 0.0f;
    if (c <= E) {
#pragma unroll 8
      for (int b = q; b < nb; b += 4) acc += part[(int64_t)b * (E + 1) + c];
    }
    q4[q][c] = acc;
    if (c == 255 && E == 256) {   // the lse^2 column of E = 256 sits at c = 256
      float az = 0.0f;
      for (int b = q; b < nb; b += 4) az += part[(int64_t)b * (E + 1) + 256];
      q4[q][256] = az;
    }
  }
  __syncthreads();
  if (threadIdx.x >= 256) return;
  const int e = threadIdx.x;
  float pb = 0.0f;
  if (e < E) {
    pb = (((q4[0][e] + q4[1][e]) + q4[2][e]) + q4[3][e]) / (float)T;
    aux[4 + e] = pb;
  }
  red[e] = e < E ? pb : 0.0f;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (e < o) red[e] += red[e + o];
    __syncthreads();
  }
  const float m = red[0] / (float)E;
  __syncthreads();
  red[e] = e < E ? (pb - m) * (pb - m) : 0.0f;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (e < o) red[e] += red[e + o];
    __syncthreads();
  }
  if (e == 0) {
    const float cv2 = (red[0] / (float)E) / (m * m);
    const float zs = ((q4[0][E] + q4[1][E]) + q4[2][E]) + q4[3][E];
    aux[0] = lb_coef * cv2;
    aux[1] = z_coef * zs / (float)T;
    aux[3] = cv2;
  }
}

}  // namespace

hipError_t launch_topk(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, bool rounding,
                       hipStream_t st) {
  const int grid = rounding ? ceil_div(s.T, 64) : ceil_div(s.T, 4);
  const int wordsT = ceil_div(s.T, 32);
  size_t lds = rounding ? (size_t)s.E * 65 * 4 + (size_t)s.E * 8 : 0;
#define MOE_TOPK(V, R)                                                                                  \
  do {                                                                                                 \
    auto kern = topk_kernel<V, R, R ? 4 : 1, R ? 1024 : 256>;                                                      \
    if (lds > 65536) hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
    hipLaunchKernelGGL(kern, dim3(grid), dim3(R ? 1024 : 256), lds, st, p.logits, s.T, s.E, s.k, p.topk_idx, \
                       p.topk_gate, p.keep_bits, pi.words, p.probs_t, pi.sel_t, wordsT,                \
                       (int)(s.gate_mode == MOE_GATE_ALL));                                             \
  } while (0)
  if (s.E <= 64) { if (rounding) MOE_TOPK(1, true); else MOE_TOPK(1, false); }
  else if (s.E <= 128) { if (rounding) MOE_TOPK(2, true); else MOE_TOPK(2, false); }
  else { if (rounding) MOE_TOPK(4, true); else MOE_TOPK(4, false); }
#undef MOE_TOPK
  return hipGetLastError();
}

hipError_t launch_plan_build(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, bool raw,
                             bool with_prob_gates, hipStream_t st) {
  const size_t lds = (size_t)4 * s.E * 2 * 4;
  hipLaunchKernelGGL(plan_count_kernel, dim3(pi.nblk), dim3(256), lds, st, p.keep_bits, s.T, s.E, pi.words,
                     pi.nblk, pi.hist, pi.blk_tok);
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), 0, st, s.E, pi.nblk, pi.hist, pi.blk_tok, p.counts,
                     raw ? p.counts_raw : nullptr, p.offsets, pi.prefix128, pi.tile_e128, raw ? p.aux : nullptr);
  hipLaunchKernelGGL(plan_scatter_kernel, dim3(pi.nblk), dim3(256), lds + (size_t)s.E * 4, st, p.keep_bits, s.T, s.E, s.k,
                     pi.words, pi.nblk, pi.hist, pi.blk_tok, p.topk_idx, p.topk_gate, p.probs_t,
                     with_prob_gates, s.gate_mode == MOE_GATE_ALL, p.token_of_row, p.expert_of_row, p.gate_of_row, p.row_of_slot, p.tok_ptr,
                     p.tok_rows);
  return hipGetLastError();
}

hipError_t launch_capacity_drop(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, hipStream_t st) {
  const int64_t nmax = max_rows(s);
  const double c = std::ceil((double)s.capacity_factor * (double)s.T * (double)s.k / (double)s.E);
  const int64_t C = c > 9.0e18 ? INT64_MAX : (int64_t)c;
  hipLaunchKernelGGL(capacity_drop_kernel, dim3(ceil_div(nmax, 256)), dim3(256), 0, st, p.offsets, p.token_of_row,
                     p.expert_of_row, s.E, nmax, C, p.keep_bits, pi.words);
  return hipGetLastError();
}

hipError_t launch_router_losses(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, hipStream_t st) {
  const int nb = ceil_div(s.T, kLossTokens);
  if (s.E <= 64)
    hipLaunchKernelGGL(router_loss_partial_kernel<1>, dim3(nb), dim3(256), 0, st, p.logits, s.T, s.E, pi.loss_part);
  else if (s.E <= 128)
    hipLaunchKernelGGL(router_loss_partial_kernel<2>, dim3(nb), dim3(256), 0, st, p.logits, s.T, s.E, pi.loss_part);
  else
    hipLaunchKernelGGL(router_loss_partial_kernel<4>, dim3(nb), dim3(256), 0, st, p.logits, s.T, s.E, pi.loss_part);
  hipLaunchKernelGGL(router_loss_final_kernel, dim3(1), dim3(1024), 0, st, pi.loss_part, nb, s.T, s.E, s.lb_coef,
                     s.z_coef, p.aux);
  return hipGetLastError();
}

hipError_t launch_round_select(const moe_shape& s, const moe_plan& p, const PlanInternal& pi, hipStream_t st) {
  const size_t col = (size_t)(s.T + s.T / 32 + 1) * 4;   // padded column
  const bool in_lds = col <= 144 * 1024;
  const size_t lds = in_lds ? col : 0;
  if (lds > 65536)
    hipFuncSetAttribute((const void*)round_select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(round_select_kernel, dim3(s.E), dim3(1024), lds, st, p.probs_t, pi.sel_t,
                     ceil_div(s.T, 32), p.counts_raw, s.T, s.round_tile, p.keep_bits, pi.words, in_lds);
  return hipGetLastError();
}

}  // namespace moe
