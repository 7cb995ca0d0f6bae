// Pipelined bf16 main loop for the grouped expert GEMMs on gfx950.
//
// Operand tiles go global -> LDS with global_load_lds_dwordx4 (no VGPR staging)
// into a ring of S stages of BK = 32; the loads for stage k+S-1 are issued while
// stage k is multiplied, so up to S-1 stages of memory latency are covered.  One
// barrier per stage; each wave waits only for its own loads of the stage it is
// about to read (s_waitcnt vmcnt(n)) before the barrier.
//
// LDS layouts (both 64 B of K per tile row, i.e. 32 bf16).  The gfx950 LDS has
// 64 banks: a 16-byte read serves 16 lanes (256 B) per cycle, so 16 consecutive
// fragment rows must land in 16 different 16 B bank groups.
//  * K-contiguous operand: [rows][32] bf16, 16 B chunk c of row r stored at slot
//    c ^ h(r), h(r) = ((r >> 1) ^ (r >> 3)) & 1 | ((r >> 2) & 1) << 1: rows r..r+15
//    of one chunk (an MFMA fragment read) then cover all 64 banks, and any 8
//    consecutive rows cover 32.
//  * M/N-contiguous operand: [32 k][rows] bf16, 32 B slot s of k-row k stored at
//    s ^ ((k & 3) << 1).  Fragments are read with ds_read_b64_tr_b16: within each group
//    of 16 lanes, lane i receives element i % 4 of the 8-byte words read by lanes
//    4j + i/4 (j = 0..3).  Lanes reading k-rows kb..kb+3 at columns n0 + 4*(i%4)
//    therefore hand lane i the four k values of column n0 + i -- two such reads
//    build the 8-k MFMA operand from a tile stored in its natural layout.
// The DMA write of one wave instruction covers 1 KiB of LDS contiguously
// (lane i -> byte 16 i), so each lane fetches the global chunk that the layout
// places there; masked lanes (rows past a segment) fetch a zero block.
#pragma once
#include "gemm_engine.h"
#include "mx_codes.h"

namespace moe_gemm {

static __device__ __attribute__((aligned(16))) uint32_t g_dma_zero[4];   // source of masked DMA lanes

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// global_load_lds_dwordx4 written out: the compiler, which cannot tell the DMA's
// LDS bytes from those a later ds_read_b64_tr_b16 reads, would otherwise wait for
// every DMA in flight (vmcnt(0)) before each stage's first transposed fragment
// read, and the ring would hide no latency.  The kernels order the DMA with
// explicit s_waitcnt vmcnt(n) + barrier before any read of the stage.  No
// register is written by the instruction (the data goes to LDS only).
MOE_DEV void dma16(const void* g, char* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)lds_wave_base);
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(m0) : "memory");
}

MOE_DEV u32x4 lds_tr_frag(const char* p0, const char* p1) {
  s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p0);
  s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p1);
  uint2 x = __builtin_bit_cast(uint2, a), y = __builtin_bit_cast(uint2, b);
  return u32x4{x.x, x.y, y.x, y.y};
}

// compiler-only fence: the slab is accessed under different types (fp32 staging,
// bf16 / packed stores); keeps the compiler from reordering those LDS accesses
MOE_DEV void lds_fence() { asm volatile("" ::: "memory"); }

// barrier without the compiler's implicit wait on every outstanding memory op;
// the asm fences keep the compiler from moving LDS accesses across it
MOE_DEV void cta_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14])
template <int N>
MOE_DEV void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | (((N >> 4) & 3) << 14));
}

MOE_DEV int kc_h(int row) { return (((row >> 1) ^ (row >> 3)) & 1) | (((row >> 2) & 1) << 1); }
MOE_DEV int kc_off(int row, int chunk) { return row * 64 + ((chunk ^ kc_h(row)) << 4); }
// 128-byte rows (BK = 64): chunk c of row r at slot c ^ ((r >> 1) & 7); rows r..r+15
// of one chunk land in 16 different 16 B bank groups
MOE_DEV int kc8_h(int row) { return (row >> 1) & 7; }
template <int BK>
MOE_DEV int kc_offk(int row, int chunk) {
  if constexpr (BK == 32) return kc_off(row, chunk);
  else return row * 128 + ((chunk ^ kc8_h(row)) << 4);
}
MOE_DEV int mn_x(int k) { return (k & 3) << 1; }
template <int ROWS>
MOE_DEV int mn_off(int k, int byte) {
  static_assert(ROWS >= 128, "the k-row swizzle needs 8 slots of 32 B");
  return k * (ROWS * 2) + ((((byte >> 5) ^ mn_x(k)) << 5) | (byte & 31));
}

// DMA sources of one operand tile (ROWS rows x BK k) for the lanes of this wave.
template <int ROWS, int NW, bool KC, int BK = 32>
struct DmaOperand {
  static_assert(BK == 32 || BK == 64, "stage depth");
  static constexpr int RPI = 1024 / (BK * 2);   // KC: tile rows per 1 KiB instruction
  static constexpr int LPR = BK * 2 / 16;       // KC: lanes per tile row
  static constexpr int Q = ROWS * BK * 2 / 1024 / NW;   // 1 KiB instructions per wave per stage
  static_assert(Q >= 1 && (ROWS * BK * 2 / 1024) % NW == 0, "tile rows must split over the waves");
  const bf16_t* src[Q];   // KC: element pointer of (row, chunk) at k = 0; MN: unused
  int kl[Q], mn[Q];       // MN: local k row and column of the lane's 16 bytes
  int q0;

  template <class RowFn>
  MOE_DEV void init_kc(RowFn rowfn, int wave, int lane) {
    q0 = wave * Q;
#pragma unroll
    for (int u = 0; u < Q; ++u) {
      const int row = (q0 + u) * RPI + lane / LPR;
      const int c = (lane % LPR) ^ (BK == 32 ? kc_h(row) : kc8_h(row));
      src[u] = rowfn(row) + c * 8;
    }
  }
  MOE_DEV void init_mn(int wave, int lane) {
    q0 = wave * Q;
#pragma unroll
    for (int u = 0; u < Q; ++u) {
      const int b = (q0 + u) * 1024 + lane * 16;
      const int k = b / (ROWS * 2), within = b % (ROWS * 2);
      const int s = (within >> 5) ^ mn_x(k);
      kl[u] = k;
      mn[u] = s * 16 + ((within >> 4) & 1) * 8;
    }
  }
  // KC: k0 = first K element of the stage (no K tail on these operands)
  MOE_DEV void issue_kc(char* tile, int k0) const {
#pragma unroll
    for (int u = 0; u < Q; ++u) dma16(src[u] + k0, tile + (q0 + u) * 1024);
  }
  // MN: base = element (k = 0, row = 0) of the operand; rows [k0, k_end) valid,
  // columns [0, rvalid) valid relative to base's column
  MOE_DEV void issue_mn(char* tile, const bf16_t* base, int64_t ld, int k0, int k_end, int rvalid) const {
#pragma unroll
    for (int u = 0; u < Q; ++u) {
      const int k = k0 + kl[u];
      const void* g = (k < k_end && mn[u] < rvalid) ? (const void*)(base + (int64_t)k * ld + mn[u])
                                                    : (const void*)g_dma_zero;
      dma16(g, tile + (q0 + u) * 1024);
    }
  }
};

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>), in order
template <int N, class F>
MOE_DEV void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

MOE_DEV float fast_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

constexpr uint32_t kBufferFlags = 0x00020000;   // gfx9 raw buffer: 32-bit dwords, no swizzle
constexpr int kCachePolicyNT = 2;                 // buffer store cache policy: non-temporal (nt)

MOE_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, (int)kBufferFlags);
}

// threadIdx.x through an opaque move: values derived from it are computed where
// they are used and not hoisted out of a persistent kernel's tile loop (where they
// would stay live across the main loop and spill).
MOE_DEV int opaque_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

struct NoEpilogueHook {
  template <class I>
  MOE_DEV void operator()(I) const {}
};

// Wave-private epilogue: each wave stages its (BM/WM) x (BN/WN) accumulators in
// its own LDS slab, 32 rows at a time, and reads them back as 8-column vectors --
// no block-wide barrier.  Slab row stride WTN + 8 floats keeps the two 32-lane
// halves of each staging store in different bank halves.
// SwiGLU: the wave's columns [0, WTN/2) are gate columns, [WTN/2, WTN) the
// matching up columns.  dS partials go to C3[(nt * WN + wn) * ldc3 + row].
// Latency: every sub-tile first issues all its global loads (the saved H and the
// gates of the SwiGLU backward) and all its slab reads, then computes and
// stores, so a wave waits once per sub-tile rather than once per row chunk.
// PERSIST (a kernel that walks several tiles): the thread index is taken through
// opaque_tid, the weight gradients are written with raw buffer stores (below),
// and after(integral_constant<int, i>) runs once sub-tile i is stored and its
// slab rows are read back (the kernel starts its next tile there).
template <int BM, int BN, int WM, int WN, int GROUP, int EPI, bool PERSIST = false, class After = NoEpilogueHook>
MOE_DEV void wave_epilogue(const Args& args, const TileCtx& ctx, f32x16 (&acc)[BM / WM / 32][BN / WN / 32],
                           char* smem, After after = After{}) {
  using T = bf16_t;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int SS = WTN + 8;              // slab row stride (floats)
  constexpr int CPR = WTN / 8;             // 8-column chunks per wave row
  const int tid = PERSIST ? opaque_tid() : (int)threadIdx.x;
  const int lane = tid & 63, wave = PERSIST ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  float* slab = reinterpret_cast<float*>(smem) + wave * 32 * SS;
  const int rbase = ctx.row_begin + wm * WTM;     // GROUP_M: first row of this wave's tile
  const int mbase = ctx.m0 + wm * WTM;            // GROUP_K: first output row
  const int cbase = ctx.n0 + wn * WTN;            // first output column
  // SwiGLU backward: the sub-tile's H (gate and up) and gates.  The bf16 kernel
  // loads sub-tile i + 1's while it works on sub-tile i (two register sets, one
  // per parity); the MXFP8 one, whose epilogue holds more registers, loads each
  // sub-tile's at its start.
  constexpr int IT_H = (EPI == EPI_DSWIGLU || EPI == EPI_DSWIGLU_MX) ? 32 * CPR / 64 : 1;
  constexpr bool H_AHEAD = EPI == EPI_DSWIGLU;
  u32x4 hgv2[H_AHEAD ? 2 : 1][IT_H], huv2[H_AHEAD ? 2 : 1][IT_H];
  float gv2[H_AHEAD ? 2 : 1][IT_H];
  auto load_h = [&](auto sc, auto bc) {
    constexpr int si = decltype(sc)::value, b = decltype(bc)::value;
    const T* Hs = reinterpret_cast<const T*>(args.aux);
#pragma unroll
    for (int it = 0; it < IT_H; ++it) {
      const int u = lane + 64 * it;
      const int rr = u / CPR, ch = u % CPR;
      const int grow = rbase + si * 32 + rr;
      const int col = cbase + ch * 8;
      if (grow < ctx.row_end && col < args.N) {
        const T* hrow = Hs + (int64_t)grow * args.ld_aux;
        hgv2[b][it] = ldg16(hrow + col);
        huv2[b][it] = ldg16(hrow + args.f + col);
        gv2[b][it] = args.row_gate[grow];
      } else {
        hgv2[b][it] = huv2[b][it] = u32x4{0u, 0u, 0u, 0u};
        gv2[b][it] = 0.0f;
      }
    }
  };
  if constexpr (H_AHEAD) load_h(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
  // one 32-row sub-tile at a time; the sub-tile index is a compile-time constant
  // so the accumulators stay in registers however large the per-row work is
  static_for<TM>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (EPI == EPI_DSWIGLU || EPI == EPI_DSWIGLU_MX) {
      static_assert(CPR <= 64 && (32 * CPR) % 64 == 0, "row reduction inside one wave");
      static_assert(EPI != EPI_DSWIGLU_MX || CPR % 4 == 0, "lane quads hold 32-column blocks");
      constexpr int IT = IT_H;
      constexpr int B = H_AHEAD ? (i & 1) : 0;
      if constexpr (H_AHEAD) {
        if constexpr (i + 1 < TM) load_h(std::integral_constant<int, i + 1>{}, std::integral_constant<int, B ^ 1>{});
      } else {
        load_h(std::integral_constant<int, i>{}, std::integral_constant<int, 0>{});   // overlaps the staging below
      }
      auto& hgv = hgv2[B];
      auto& huv = huv2[B];
      auto& gv = gv2[B];
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q)
          slab[(8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)) * SS + j * 32 + (lane & 31)] = acc[i][j][q];
      __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): the slab is written (one wave, in order)
      float dap[IT][8];
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int u = lane + 64 * it;
        const float* src = slab + (u / CPR) * SS + (u % CPR) * 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) dap[it][c] = src[c];
      }
      lds_fence();                                 // the dA' reads above stay before the staging below
      T* dH = reinterpret_cast<T*>(args.C);
      T* gA = reinterpret_cast<T*>(args.C2);
      // MXFP8: the sub-tile's dH (bf16, as stored) is staged in the slab (rows of
      // 128 gate+up columns, pitch PB) for the token-axis pass below, gA kept packed
      constexpr int PB = 2 * WTN + 8;
      uint16_t* stage = reinterpret_cast<uint16_t*>(slab);
      u32x4 gaq[IT];
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int u = lane + 64 * it;
        const int rr = u / CPR, ch = u % CPR;
        const int grow = rbase + i * 32 + rr;
        const int col = cbase + ch * 8;
        float part = 0.0f;
        const bool ok = grow < ctx.row_end && col < args.N;   // uniform over each lane quad
        float dhg[8], dhu[8], ga[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) dhg[c] = dhu[c] = ga[c] = 0.0f;
        if (ok) {
          const float g = gv[it];
          float hg[8], hu[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            hg[2 * q] = __uint_as_float(hgv[it][q] << 16);
            hg[2 * q + 1] = __uint_as_float(hgv[it][q] & 0xffff0000u);
            hu[2 * q] = __uint_as_float(huv[it][q] << 16);
            hu[2 * q + 1] = __uint_as_float(huv[it][q] & 0xffff0000u);
          }
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float sg = fast_sigmoid(hg[c]);
            const float sl = hg[c] * sg;
            const float a = Vec8<T>::rnd(sl * hu[c]);      // A as stored in the forward
            part += dap[it][c] * a;
            const float da = g * dap[it][c];
            dhg[c] = da * hu[c] * (sg * (1.0f + hg[c] * (1.0f - sg)));
            dhu[c] = da * sl;
            ga[c] = g * a;
          }
          if constexpr (EPI == EPI_DSWIGLU) {   // MXFP8 keeps dH and gA only as codes
            T* drow = dH + (int64_t)grow * args.ldc;
            Vec8<T>::store(drow + col, dhg);
            Vec8<T>::store(drow + args.f + col, dhu);
            Vec8<T>::store(gA + (int64_t)grow * args.ldc2 + col, ga);
          }
        }
        if constexpr (EPI == EPI_DSWIGLU_MX) {
          // dH as stored (bf16), quantised along 2f: gate columns col.. and up
          // columns f + col.., each lane quad one 32-column block of each
          float mg = 0.0f, mu = 0.0f;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            dhg[c] = Vec8<T>::rnd(dhg[c]);
            dhu[c] = Vec8<T>::rnd(dhu[c]);
            mg = fmaxf(mg, fabsf(dhg[c]));
            mu = fmaxf(mu, fabsf(dhu[c]));
          }
          mg = quad_max(mg);
          mu = quad_max(mu);
          if (ok) {
            const int Xg = mx_exponent(mg), Xu = mx_exponent(mu);
            const int64_t prow = grow + (int64_t)args.q_pad[ctx.e] - args.offsets[ctx.e];
            uint8_t* crow = args.q_codes + prow * args.q_ld;
            *reinterpret_cast<uint2*>(crow + col) = e4m3_8(dhg, pow2f(-Xg));
            *reinterpret_cast<uint2*>(crow + args.f + col) = e4m3_8(dhu, pow2f(-Xu));
            if ((ch & 3) == 0) {
              const int kg = col, ku = args.f + col;
              args.q_scales[((kg >> 6) * args.q_srows + prow) * 2 + ((kg >> 5) & 1)] = (uint8_t)(Xg + 127);
              args.q_scales[((ku >> 6) * args.q_srows + prow) * 2 + ((ku >> 5) & 1)] = (uint8_t)(Xu + 127);
            }
          }
          // stage dH (bf16) for the token-axis pass (the dA' values were read from
          // the slab before this loop; one wave, in-order LDS), keep gA (bf16)
          u32x4 pg, pu;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            pg[q] = pack_bf2(dhg[2 * q], dhg[2 * q + 1]);
            pu[q] = pack_bf2(dhu[2 * q], dhu[2 * q + 1]);
            gaq[it][q] = pack_bf2(ga[2 * q], ga[2 * q + 1]);
          }
          *reinterpret_cast<u32x4*>(stage + rr * PB + ch * 8) = pg;
          *reinterpret_cast<u32x4*>(stage + rr * PB + WTN + ch * 8) = pu;
        }
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) part += __shfl_xor(part, o, 64);
        if (ch == 0 && grow < ctx.row_end) args.C3[(int64_t)(ctx.nt * WN + wn) * args.ldc3 + grow] = part;
      }
      if constexpr (EPI == EPI_DSWIGLU_MX) {
        // along tokens: the sub-tile's 32 rows are one 32-position block of the
        // expert-padded token axis (segments start at multiples of 64 and this
        // block starts 32-aligned inside its segment); lane l quantises column l
        // of each 64-column group from its 32 staged values.  Rows past the
        // segment hold zeros; blocks past the padded segment are not written.
        static_assert(WTN == 64 && CPR == 8, "one column per lane");
        const int e = ctx.e;
        const int rel = rbase + i * 32 - args.offsets[e];
        const bool blk = rel < args.q_pad[e + 1] - args.q_pad[e];
        const int64_t p0 = (int64_t)args.q_pad[e] + rel;
        auto column = [&](const uint16_t* src, int pitch, uint8_t* codes, uint8_t* scales, int64_t srows,
                          int64_t crow) {
          float v[32];
          float amax = 0.0f;
#pragma unroll
          for (int r = 0; r < 32; ++r) {
            v[r] = __uint_as_float((uint32_t)src[r * pitch] << 16);
            amax = fmaxf(amax, fabsf(v[r]));
          }
          const int X = mx_exponent(amax);
          const float inv = pow2f(-X);
          uint8_t* cp = codes + crow * args.t_len + p0;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint2 lo = e4m3_8(v + 16 * q, inv), hi2 = e4m3_8(v + 16 * q + 8, inv);
            *reinterpret_cast<u32x4*>(cp + 16 * q) = u32x4{lo.x, lo.y, hi2.x, hi2.y};
          }
          scales[((p0 >> 6) * srows + crow) * 2 + ((p0 >> 5) & 1)] = (uint8_t)(X + 127);
        };
        const int gc = cbase + lane;   // this lane's column of the gate (and gA) group
        lds_fence();
        __builtin_amdgcn_s_waitcnt(0xc07f);        // the staged dH is in the slab
        if (blk && gc < args.N) {
          column(stage + lane, PB, args.t_codes, args.t_scales, 2 * (int64_t)args.f, gc);
          column(stage + WTN + lane, PB, args.t_codes, args.t_scales, 2 * (int64_t)args.f, args.f + gc);
        }
        lds_fence();
        __builtin_amdgcn_s_waitcnt(0xc07f);        // dH read back before gA overwrites the slab
        constexpr int PA = WTN + 8;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          const int u = lane + 64 * it;
          *reinterpret_cast<u32x4*>(stage + (u / CPR) * PA + (u % CPR) * 8) = gaq[it];
        }
        lds_fence();
        __builtin_amdgcn_s_waitcnt(0xc07f);
        if (blk && gc < args.N) column(stage + lane, PA, args.t2_codes, args.t2_scales, (int64_t)args.f, gc);
        lds_fence();                               // read back before the next sub-tile's fp32 staging
      }
    } else {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q)
          slab[(8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)) * SS + j * 32 + (lane & 31)] = acc[i][j][q];
      __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): the slab is written (one wave, in order)
      if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_MX) {
        constexpr int HC = CPR / 2;
        constexpr int IT = 32 * HC / 64;
        static_assert(EPI != EPI_SWIGLU_MX || HC == 4, "one 32-column block of A per wave row");
        T* H = reinterpret_cast<T*>(args.C);
        T* Aout = reinterpret_cast<T*>(args.C2);
        float hg[IT][8], hu[IT][8];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          const int u = lane + 64 * it;
          const float* src = slab + (u / HC) * SS + (u % HC) * 8;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            hg[it][c] = Vec8<T>::rnd(src[c]);
            hu[it][c] = Vec8<T>::rnd(src[WTN / 2 + c]);
          }
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          const int u = lane + 64 * it;
          const int rr = u / HC, ch = u % HC;
          const int grow = rbase + i * 32 + rr;
          const int gcol = ctx.nt * (BN / 2) + wn * (WTN / 2) + ch * 8;
          // uniform over each lane quad (a 32-column block never straddles f, f % 128 == 0)
          const bool ok = grow < ctx.row_end && gcol < args.f;
          float a[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) a[c] = hg[it][c] * fast_sigmoid(hg[it][c]) * hu[it][c];
          if (ok) {
            T* hrow = H + (int64_t)grow * args.ldc;
            Vec8<T>::store(hrow + gcol, hg[it]);
            Vec8<T>::store(hrow + args.f + gcol, hu[it]);
          }
          if constexpr (EPI == EPI_SWIGLU_MX) {
            // A as the forward stores it (bf16), quantised along f: this row's 32
            // columns of the wave are one block held by a lane quad
            float amax = 0.0f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              a[c] = Vec8<T>::rnd(a[c]);
              amax = fmaxf(amax, fabsf(a[c]));
            }
            amax = quad_max(amax);
            if (ok) {
              const int X = mx_exponent(amax);
              const int64_t prow = grow + (int64_t)args.q_pad[ctx.e] - args.offsets[ctx.e];
              *reinterpret_cast<uint2*>(args.q_codes + prow * args.q_ld + gcol) = e4m3_8(a, pow2f(-X));
              if (ch == 0)
                args.q_scales[((gcol >> 6) * args.q_srows + prow) * 2 + ((gcol >> 5) & 1)] = (uint8_t)(X + 127);
            }
          } else {
            if (ok) Vec8<T>::store(Aout + (int64_t)grow * args.ldc2 + gcol, a);
          }
        }
      } else {
        // act dtype (EPI_ACT) or fp32 (weight-gradient slabs, split-K partials).
        // Every lane stores one 16-byte vector and consecutive lanes hold
        // consecutive columns, so each store instruction writes whole 128-byte
        // lines (fp32 rows written as two interleaved halves cost ~10% of the
        // weight-gradient time).
        using OT = typename std::conditional<EPI == EPI_ACT || EPI == EPI_GATE_SCATTER, T, float>::type;
        constexpr int VW = 16 / (int)sizeof(OT);   // values per 16-byte store
        constexpr int CU = WTN / VW;               // 16-byte units per wave row
        constexpr int IT = 32 * CU / 64;
        OT* C = reinterpret_cast<OT*>(args.C);
        if constexpr (GROUP == GROUP_K) C = wgrad_out<OT>(args, ctx);
        // Weight gradients are written once and not read again in the step: their
        // stores carry the non-temporal hint, so gigabytes of fp32 rows stream out
        // instead of filling the caches with dirty lines that later kernels would
        // pay to write back (and that would push out the GEMM's operand tiles).
        // Persistent weight gradients: raw buffer stores from the sub-tile's first
        // row, a lane outside the output given an offset past the record count (it
        // writes nothing), so no branch surrounds the stores and the compiler can
        // count them (the next tile's loads, issued before them, are then waited
        // for without waiting for the stores).  Offsets < 32 * ldc * 4 < 2^31.
        // The same branch-free stores for a persistent kernel's bf16 rows (EPI_ACT;
        // those are read by the next kernel and keep the default cache policy).
        constexpr bool BUF = PERSIST && ((GROUP == GROUP_K && EPI == EPI_F32) || (GROUP == GROUP_M && EPI == EPI_ACT));
        constexpr int BUF_POLICY = GROUP == GROUP_K ? kCachePolicyNT : 0;
        constexpr uint32_t kNoStore = 0x7ffffff0u;
        const int brow = (GROUP == GROUP_K ? mbase : rbase) + i * 32;
        const __amdgpu_buffer_rsrc_t crs = make_rsrc(BUF ? C + (int64_t)brow * args.ldc : C, kNoStore);
        float v[IT][VW];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          const int u = lane + 64 * it;
          const float* src = slab + (u / CU) * SS + (u % CU) * VW;
          if constexpr (VW == 8) {
            // lanes of odd rows read their second 16 bytes first: with the slab's
            // row stride (8 banks past a multiple of 64) the 16 lanes of each
            // read then cover all 64 banks once instead of half of them twice
            const int h = ((u / CU) & 1) * 4;
            const f32x4 a = *reinterpret_cast<const f32x4*>(src + h);
            const f32x4 b = *reinterpret_cast<const f32x4*>(src + (4 - h));
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              v[it][c] = h ? b[c] : a[c];
              v[it][4 + c] = h ? a[c] : b[c];
            }
          } else {
#pragma unroll
            for (int c = 0; c < VW; ++c) v[it][c] = src[c];
          }
        }
        if constexpr (EPI == EPI_LOGITS) {
          // router logits: (z + bias) + noise, in that order; the launcher keeps
          // N a multiple of the tile width (no partial column vectors)
          static_assert(GROUP == GROUP_NONE && VW == 4, "logits: fp32 rows of x W_g^T");
          const float* nz = reinterpret_cast<const float*>(args.aux);   // routing noise [M, N] or null
#pragma unroll
          for (int it = 0; it < IT; ++it) {
            const int u = lane + 64 * it;
            const int grow = mbase + i * 32 + u / CU, col = cbase + (u % CU) * VW;
            if (grow < args.M && col < args.N) {
#pragma unroll
              for (int c = 0; c < VW; ++c)
                v[it][c] = (v[it][c] + (args.bias ? args.bias[col + c] : 0.0f)) +
                           (nz ? nz[(int64_t)grow * args.ld_aux + col + c] : 0.0f);
            }
          }
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
          const int u = lane + 64 * it;
          const int rr = u / CU, ch = u % CU;
          int grow;
          bool ok;
          if constexpr (GROUP == GROUP_M) { grow = rbase + i * 32 + rr; ok = grow < ctx.row_end; }
          else { grow = mbase + i * 32 + rr; ok = grow < args.M; }
          const int col = cbase + ch * VW;
          if constexpr (BUF) {
            u32x4 q;
            if constexpr (VW == 8) {
#pragma unroll
              for (int h = 0; h < 4; ++h) q[h] = pack_bf2(v[it][2 * h], v[it][2 * h + 1]);
            } else {
              q = u32x4{__float_as_uint(v[it][0]), __float_as_uint(v[it][1]), __float_as_uint(v[it][2]),
                        __float_as_uint(v[it][3])};
            }
            const uint32_t off = (ok && col < args.N) ? (uint32_t)(rr * args.ldc + col) * (uint32_t)sizeof(OT) : kNoStore;
            __builtin_amdgcn_raw_buffer_store_b128(q, crs, (int)off, 0, BUF_POLICY);
          } else if (ok && col < args.N) {
            if constexpr (EPI == EPI_GATE_SCATTER) {
              // the combine's gate, applied before the row is rounded to the act
              // dtype; the row goes to its token-order position
              const float g = args.row_gate[grow];
#pragma unroll
              for (int c = 0; c < VW; ++c) v[it][c] *= g;
              Vec8<OT>::store(C + (int64_t)args.c_rows[grow] * args.ldc + col, v[it]);
            } else if constexpr (VW == 8) {
              Vec8<OT>::store(C + (int64_t)grow * args.ldc + col, v[it]);
            } else {
              const u32x4 q{__float_as_uint(v[it][0]), __float_as_uint(v[it][1]), __float_as_uint(v[it][2]),
                            __float_as_uint(v[it][3])};
              u32x4* dst = reinterpret_cast<u32x4*>(C + (int64_t)grow * args.ldc + col);
              if constexpr (GROUP == GROUP_K) __builtin_nontemporal_store(q, dst);
              else *dst = q;
            }
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);          // slab reads done before the next sub-tile overwrites it
    after(ic);
  });
}

template <int BM, int BN, int WM, int WN, bool AKC, bool BKC, int GROUP, int EPI, int S, int BK = 32>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_dma(Args args) {
  using T = bf16_t;
  constexpr int NW = WM * WN;
  static_assert(S >= 2 && S <= 5, "ring depth");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int ASZ = BM * BK * 2, BSZ = BN * BK * 2, STAGE = ASZ + BSZ;
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold a 32x32 MFMA tile");
  static_assert(GROUP != GROUP_NONE || (AKC && EPI == EPI_LOGITS), "GROUP_NONE: the router logits (x rows)");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  TileCtx ctx;
  if (!decode_tile<BM, BN, BK, GROUP>(args, ctx)) return;
  const int e = ctx.e, nt = ctx.nt;
  const int row_begin = ctx.row_begin, row_end = ctx.row_end;
  const int k_begin = ctx.k_begin, k_end = ctx.k_end;
  const int m0 = ctx.m0, n0 = ctx.n0;
  const T* Ab = reinterpret_cast<const T*>(args.A) + (int64_t)e * args.a_estride;
  const T* Bb = reinterpret_cast<const T*>(args.B) + (int64_t)e * args.b_estride;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;

  DmaOperand<BM, NW, AKC, BK> da;
  DmaOperand<BN, NW, BKC, BK> db;
  if constexpr (AKC) {
    da.init_kc([&](int row) -> const T* {
      if constexpr (GROUP == GROUP_NONE) {   // rows m0.. of A; past M only feed unstored outputs
        const int g = min(m0 + row, args.M - 1);
        return Ab + (int64_t)g * args.lda;
      }
      int g = row_begin + row;
      if (g >= row_end) g = row_end - 1;     // rows past the segment only feed unstored outputs
      const int src = args.a_gather ? args.a_gather[g] : g;
      return Ab + (int64_t)src * args.lda;
    }, wave, lane);
  } else {
    da.init_mn(wave, lane);
  }
  if constexpr (BKC) {
    db.init_kc([&](int row) -> const T* {
      int j = n0 + row;
      if constexpr (EPI == EPI_SWIGLU) {
        // wave wn's columns: first half gate rows, second half the matching up rows
        const int w = row / WTN, jj = row % WTN;
        const int g = nt * (BN / 2) + w * (WTN / 2) + (jj % (WTN / 2));
        j = (jj < WTN / 2) ? g : (args.f + g);
      } else {
        if (j >= args.N) j = args.N - 1;
      }
      return Bb + (int64_t)j * args.ldb;
    }, wave, lane);
  } else {
    db.init_mn(wave, lane);
  }

  auto issue = [&](int kt) {
    char* st = smem + (kt % S) * STAGE;
    const int k0 = k_begin + kt * BK;
    if constexpr (AKC) da.issue_kc(st, k0);
    else da.issue_mn(st, Ab + m0, args.lda, k0, k_end, args.M - m0);
    if constexpr (BKC) db.issue_kc(st + ASZ, k0);
    else db.issue_mn(st + ASZ, Bb + n0, args.ldb, k0, k_end, args.N - n0);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  constexpr int LPS = DmaOperand<BM, NW, AKC, BK>::Q + DmaOperand<BN, NW, BKC, BK>::Q;   // loads per stage
  constexpr int KS = BK / 16;                   // 16-deep MFMA steps per stage
  static_assert(KS % 2 == 0, "fragment double buffer alternates over the steps of a stage");
  const int nk = (k_end > k_begin) ? (k_end - k_begin + BK - 1) / BK : 0;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s);

  auto frags = [&](const char* as, int ks, u32x4 (&af)[TM], u32x4 (&bfr)[TN]) {
    const char* bs = as + ASZ;
    const int kb = ks * 16 + (lane >> 5) * 8 + ((lane & 15) >> 2);   // MN: first k row of the lane
    const int cb = (((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2;   // MN: byte column of the lane
    if constexpr (AKC) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(as + kc_offk<BK>(wm * WTM + i * 32 + (lane & 31), ks * 2 + (lane >> 5)));
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int byte = (wm * WTM + i * 32) * 2 + cb;
        af[i] = lds_tr_frag(as + mn_off<BM>(kb, byte), as + mn_off<BM>(kb + 4, byte));
      }
    }
    if constexpr (BKC) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const u32x4*>(bs + kc_offk<BK>(wn * WTN + j * 32 + (lane & 31), ks * 2 + (lane >> 5)));
    } else {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int byte = (wn * WTN + j * 32) * 2 + cb;
        bfr[j] = lds_tr_frag(bs + mn_off<BN>(kb, byte), bs + mn_off<BN>(kb + 4, byte));
      }
    }
  };
  auto mma = [&](const u32x4 (&af)[TM], const u32x4 (&bfr)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) Mma<T>::run(acc[i][j], af[i], bfr[j]);
  };
  // Fragments alternate between two register sets.  The last step of stage kt
  // is multiplied after the next barrier, so its MFMAs cover the first fragment
  // reads of stage kt + 1 (a stage's reads can only start after its barrier).
  u32x4 fa[2][TM], fb[2][TN];
  for (int kt = 0; kt < nk; ++kt) {
    const int ahead = min(S - 2, nk - 1 - kt);   // stages already issued after this one
    if (S >= 5 && ahead >= 3) wait_vm_lgkm0<3 * LPS>();
    else if (S >= 4 && ahead >= 2) wait_vm_lgkm0<2 * LPS>();
    else if (S >= 3 && ahead >= 1) wait_vm_lgkm0<LPS>();
    else wait_vm_lgkm0<0>();
    cta_barrier();                               // stage kt landed for every wave; slot (kt - 1) % S is free
    if (kt + S - 1 < nk) issue(kt + S - 1);
    const char* as = smem + (kt % S) * STAGE;
    frags(as, 0, fa[0], fb[0]);
    if (kt > 0) mma(fa[1], fb[1]);               // stage kt - 1, last step
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) {
      frags(as, ks, fa[ks & 1], fb[ks & 1]);
      mma(fa[(ks - 1) & 1], fb[(ks - 1) & 1]);
    }
  }
  if (nk > 0) mma(fa[1], fb[1]);
  __syncthreads();
  wave_epilogue<BM, BN, WM, WN, GROUP, EPI>(args, ctx, acc, smem);
}

template <int BM, int BN, int WM, int WN, int S, int BK = 32>
constexpr size_t dma_lds_bytes() {
  constexpr size_t ring = (size_t)S * (BM + BN) * BK * 2;
  constexpr size_t epi = (size_t)WM * WN * 32 * (BN / WN + 8) * 4;
  return ring > epi ? ring : epi;
}

}  // namespace moe_gemm
