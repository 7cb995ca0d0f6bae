// Register-staged bf16 main loop for the grouped expert GEMMs on gfx950:
// 8 waves per block (two per SIMD), each wave a 128 x 64 output tile (4 x 2 MFMA
// 32x32x16 sub-tiles, 128 accumulator registers), K in stages of 64.
//
// Why this shape: a CU is fed about 35-40 GB/s of operand data from L2 in
// these GEMMs, so output area per byte fetched decides the MFMA rate.  A
// 256 x 256 block tile fetches 64 KiB per 64-deep stage for 8.4 MFLOP, half
// again more work per byte than a 128 x 256 tile, and one such block fills a
// CU's LDS.  Two waves per SIMD let one wave's MFMAs cover the other's waits
// (barrier, fragment reads, load arrivals); that beats four 128 x 128 waves,
// which read fewer fragment bytes from LDS but stall alone.  Within a wave,
// global loads for stage k+2 are in flight in registers while stage k is
// multiplied and stage k+1 is written to LDS, and every group of MFMAs runs
// with the fragments of the next group already being read.
//
// Stage pipeline per iteration k (LDS double buffer, one barrier):
//   MFMA block 1 (k16 step 0)  + LDS reads of step 1
//   MFMA block 2 (step 1)      + LDS writes of stage k+1 from registers, each followed by the
//                                buffer load of stage k+2 into the register it freed; reads of step 2
//   MFMA block 3 (step 2)      + reads of step 3
//   barrier
//   MFMA block 4 (step 3)      + reads of step 0 of stage k+1
// so a load has one full iteration to arrive.
// The body has no branches: past the last stage the LDS writes land in the idle
// buffer and the buffer loads are out of range (they return zero, no access).
// Scheduling-group barriers place one LDS/global instruction after each MFMA.
//
// Global loads are raw buffer loads: the tile's operand rows are one buffer
// whose record count ends at the last valid row, so rows past an expert segment
// or a K chunk read as zero without per-lane masks.
//
// Tile shapes.  GROUP_K (weight gradients): 256 x 256 tiles.  GROUP_M (row
// segments of experts): segments are covered in units of 128 rows; each pair of
// units is a 256 x 256 ("tall", 2 x 4 waves) tile, an odd last unit a 128 x 512
// ("wide", 1 x 8 waves) tile, so a segment's padding is at most 127 rows, as
// with 128-row tiles.  A
// tall tile pair of n-tiles and a wide tile cover the same area, so logical
// tile L = unit * ceil(N / 512) + c indexes both with the plan's 128-row unit
// tables.
//
// LDS layouts are those of the DMA main loop with 128-byte K rows (BK = 64):
// K-contiguous operands [rows][64] with chunk c of row r at slot c ^ ((r >> 1) & 7);
// M/N-contiguous operands [64 k][rows] with 32 B slots XOR-swizzled by k.
#pragma once
#include "gemm_dma.h"

namespace moe_gemm {

constexpr int kBigBK = 64;
constexpr int kBigThreads = 512;

// One operand tile (ROWS rows x 64 k, bf16) staged through registers by NT
// threads, ROWS * 8 / NT 16-byte loads each.  Load i of a thread lands NT * 16
// bytes after load i - 1 in LDS for both layouts (NT / 8 K-contiguous rows, or
// NT * 8 / ROWS k rows, a multiple of 4 so the k-row swizzle repeats).
template <int ROWS, bool KC, int NT>
struct RegOperand {
  static constexpr int L = ROWS * 8 / NT;
  static constexpr int STEP = NT * 16;
  static_assert(L >= 1 && (NT * 8 / ROWS) % 4 == 0, "block shape");
  uint32_t voff[L];         // byte offset of each load from the stage's base
  int lds0;                 // LDS byte offset of load 0
  u32x4 v[L];
  const char* base;         // operand bytes of stage 0
  int64_t step;             // bytes per stage along K
  int64_t num0;             // valid bytes from base at stage 0

  // K-contiguous rows: row_off(r) = byte offset of tile row r from base; an absent
  // row gives an offset past the valid range, so its loads return zero
  template <class RowOff>
  MOE_DEV void init_kc(RowOff row_off) {
    const int t = threadIdx.x, c = t & 7, r0 = t >> 3;
    lds0 = r0 * 128 + ((c ^ kc8_h(r0)) << 4);
#pragma unroll
    for (int i = 0; i < L; ++i) voff[i] = (uint32_t)(row_off(r0 + (NT / 8) * i) + c * 16);
  }
  // M/N-contiguous: k rows ld elements apart, the tile's columns contiguous
  MOE_DEV void init_mn(int64_t ld) {
    constexpr int CPK = ROWS / 8;          // 16-byte chunks per k row
    constexpr int KPP = NT / CPK;          // k rows per pass of the block
    const int t = threadIdx.x, cc = t % CPK, k0 = t / CPK;
    lds0 = mn_off<ROWS>(k0, cc * 16);
#pragma unroll
    for (int i = 0; i < L; ++i) voff[i] = (uint32_t)((int64_t)(k0 + KPP * i) * ld * 2 + cc * 16);
  }
  // M/N-contiguous with gathered k rows: k row r of the chunk [k_begin, k_end)
  // is row gidx[r] of the source (a permutation fused into the loads).  A wave
  // covers RPW consecutive k rows per pass, so it needs L * RPW source rows per
  // stage: that many lanes load them one stage ahead (fetch_rows, one load
  // instruction) and each load reads its row from them with lane reads.
  // Offsets are 32-bit (the source holds fewer than 2^31 bytes).
  static constexpr int RPW = 64 / (ROWS / 8);   // k rows per wave and pass
  const int32_t* gidx;
  int gk, gkend, kl;
  uint32_t gld, gcol;
  int32_t idxv;
  MOE_DEV void init_mn_gather(int64_t ld, const int32_t* g, int k_begin, int k_end, int64_t col_bytes,
                              int64_t src_rows) {
    constexpr int CPK = ROWS / 8;
    const int t = threadIdx.x, cc = t % CPK, k0 = t / CPK;
    lds0 = mn_off<ROWS>(k0, cc * 16);
    gidx = g; gk = k_begin; gkend = k_end; kl = k0;
    gld = (uint32_t)(ld * 2);
    gcol = (uint32_t)(col_bytes + cc * 16);
    step = 0;
    num0 = src_rows * (int64_t)gld;
    fetch_rows();
  }
  MOE_DEV void fetch_rows() {
    constexpr int KPP = NT / (ROWS / 8);
    static_assert(RPW == 1 || RPW == 2, "one or two k rows per wave and pass");
    const int lane = threadIdx.x & 63;
    const int kw = (int)(threadIdx.x & ~63u) / (ROWS / 8);   // the wave's first k row of a pass
    int src = -1;
    if (lane < L * RPW) {
      const int k = gk + kw + lane % RPW + KPP * (lane / RPW);
      if (k < gkend) src = gidx[k];
    }
    idxv = src;
    gk += KPP * L;
  }
  MOE_DEV void load_gather() {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, (uint32_t)num0);
    const bool upper = RPW == 2 && (threadIdx.x & 63) >= 32;   // the wave's second k row
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int n0 = __builtin_amdgcn_readlane(idxv, RPW * i);
      const int n1 = RPW == 2 ? __builtin_amdgcn_readlane(idxv, RPW * i + RPW - 1) : n0;
      const int n = upper ? n1 : n0;
      const uint32_t off = n >= 0 ? (uint32_t)n * gld + gcol : 0xfffffff0u;   // absent: past num0
      v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    }
    fetch_rows();
  }
  MOE_DEV void load(int kt) {
    const int64_t n = num0 - kt * step;   // <= 0 past the operand: every load returns zero
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + kt * step, (uint32_t)(n > 0 ? n : 0));
#pragma unroll
    for (int i = 0; i < L; ++i)
      v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff[i], 0, 0));
  }
  MOE_DEV void store(char* stage) const {
#pragma unroll
    for (int i = 0; i < L; ++i) *reinterpret_cast<u32x4*>(stage + lds0 + STEP * i) = v[i];
  }
};

template <int BM, int BN>
constexpr size_t big_ring_bytes() { return (size_t)2 * (BM + BN) * kBigBK * 2; }
constexpr size_t big_lds_bytes(bool wide) {
  return wide ? big_ring_bytes<128, 512>() : big_ring_bytes<256, 256>();
}

// The main loop of one BM x BN tile with WM x WN waves of 128 x 64.  GATHER bit
// 1: the rows of A (GROUP_M) or the k rows of A (GROUP_K) are read through
// args.a_gather; bit 2: the k rows of B (GROUP_K) through args.b_gather; either
// from a source of args.gather_rows rows: the permutation of the rows is fused
// into the operand loads (no permuted copy is written).
// PERSIST: lane values come from opaque_tid (see the persistent kernel below).
template <int BM, int BN, int WM, int WN, bool AKC, bool BKC, int GROUP, int EPI, int GATHER, bool PERSIST = false>
struct BigPipe {
  using T = bf16_t;
  static constexpr int BK = kBigBK;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int NT = WM * WN * 64;
  static_assert(NT == kBigThreads && WTM == 128 && WTN == 64, "eight waves of 128 x 64");
  static constexpr int ASZ = BM * BK * 2, BSZ = BN * BK * 2, STAGE = ASZ + BSZ;
  RegOperand<BM, AKC, NT> ra;
  RegOperand<BN, BKC, NT> rb;
  int lane, wm, wn;

  MOE_DEV BigPipe() { lanes(); }
  MOE_DEV void lanes() {
    const int tid = PERSIST ? opaque_tid() : (int)threadIdx.x;
    const int wave = PERSIST ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
    lane = tid & 63;
    wm = wave / WN;
    wn = wave % WN;
  }

  // Point the operand loads at tile ctx (a gathered operand fetches the source
  // rows of its first stage).
  MOE_DEV void setup(const Args& args, const TileCtx& ctx) {
    const int e = ctx.e, nt = ctx.nt;
    const char* Ab = reinterpret_cast<const char*>(args.A) + (int64_t)e * args.a_estride * 2;
    const char* Bb = reinterpret_cast<const char*>(args.B) + (int64_t)e * args.b_estride * 2;
    if constexpr (AKC && (GATHER & 1)) {   // GROUP_M, rows gathered: row r of the tile is source row a_gather[..]
      const int nrows = min(BM, ctx.row_end - ctx.row_begin);
      const int64_t rowb = args.lda * 2;
      ra.base = Ab;
      ra.step = BK * 2;
      ra.num0 = args.gather_rows * rowb;
      ra.init_kc([&](int r) -> int64_t {
        return (r < nrows ? (int64_t)args.a_gather[ctx.row_begin + r] : args.gather_rows) * rowb;   // absent: past num0
      });
    } else if constexpr (AKC) {   // GROUP_M: rows row_begin.. of the segment, K contiguous
      const int nrows = min(BM, ctx.row_end - ctx.row_begin);
      const int64_t rowb = args.lda * 2;
      ra.base = Ab + (int64_t)ctx.row_begin * rowb;
      ra.step = BK * 2;
      ra.num0 = (int64_t)nrows * rowb;     // rows >= nrows start past it
      ra.init_kc([&](int r) -> int64_t { return (int64_t)r * rowb; });
    } else if constexpr (GATHER & 1) {    // GROUP_K, k rows gathered
      ra.base = Ab;
      ra.init_mn_gather(args.lda, args.a_gather, ctx.k_begin, ctx.k_end, (int64_t)ctx.m0 * 2, args.gather_rows);
    } else {               // GROUP_K: k rows k_begin..k_end of the chunk, columns m0.. contiguous
      ra.base = Ab + ((int64_t)ctx.k_begin * args.lda + ctx.m0) * 2;
      ra.step = (int64_t)BK * args.lda * 2;
      ra.num0 = (int64_t)(ctx.k_end - ctx.k_begin) * args.lda * 2 - (int64_t)ctx.m0 * 2;
      ra.init_mn(args.lda);
    }
    if constexpr (BKC) {   // weights [N][K]
      const int64_t rowb = args.ldb * 2;
      rb.base = Bb;
      rb.step = BK * 2;
      rb.num0 = (int64_t)args.N * rowb;
      rb.init_kc([&](int row) -> int64_t {
        int j = ctx.n0 + row;
        if constexpr (EPI == EPI_SWIGLU) {
          // wave wn's columns: first half gate rows, second half the matching up rows
          const int w = row / WTN, jj = row % WTN;
          const int g = nt * (BN / 2) + w * (WTN / 2) + (jj % (WTN / 2));
          j = g >= args.f ? args.N : (jj < WTN / 2) ? g : (args.f + g);   // past f: absent
        }
        return (int64_t)j * rowb;         // j >= N lies past num0
      });
    } else if constexpr (GATHER & 2) {    // GROUP_K, k rows of B gathered
      rb.base = Bb;
      rb.init_mn_gather(args.ldb, args.b_gather, ctx.k_begin, ctx.k_end, (int64_t)ctx.n0 * 2, args.gather_rows);
    } else {               // [K][N]: k rows, columns n0.. contiguous
      const int kb = (GROUP == GROUP_K) ? ctx.k_begin : 0;
      const int kend = (GROUP == GROUP_K) ? ctx.k_end : args.K;
      rb.base = Bb + ((int64_t)kb * args.ldb + ctx.n0) * 2;
      rb.step = (int64_t)BK * args.ldb * 2;
      rb.num0 = (int64_t)(kend - kb) * args.ldb * 2 - (int64_t)ctx.n0 * 2;
      rb.init_mn(args.ldb);
    }
  }

  // stage loads, in stage order (the gathered operands fetch their rows one stage ahead)
  MOE_DEV void load_a(int kt) {
    if constexpr (!AKC && (GATHER & 1)) ra.load_gather(); else ra.load(kt);
  }
  MOE_DEV void load_b(int kt) {
    if constexpr (!BKC && (GATHER & 2)) rb.load_gather(); else rb.load(kt);
  }
  // A gathered operand's loads go first: its next-stage row-index load is then
  // followed by the other operand's loads, which the stage waits for anyway, so
  // waiting for the index costs nothing extra (issued last, it cost dW1 5%).
  MOE_DEV void load_ab(int kt) {
    if constexpr (!BKC && (GATHER & 2)) { load_b(kt); load_a(kt); } else { load_a(kt); load_b(kt); }
  }
  MOE_DEV void store(char* stage) const { ra.store(stage); rb.store(stage + ASZ); }
  // stage 0 written to LDS and visible to the block, stage 1 loading into registers
  MOE_DEV void prologue(char* smem) {
    load_ab(0);
    store(smem);
    load_ab(1);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    cta_barrier();
  }

  template <int TMV>
  MOE_DEV void frags(const char* as, int ks, u32x4 (&af)[TM], u32x4 (&bfr)[TN]) const {
    const char* bs = as + ASZ;
    const int kb = ks * 16 + (lane >> 5) * 8 + ((lane & 15) >> 2);       // MN: first k row of the lane
    const int cb = (((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2;       // MN: byte column of the lane
    if constexpr (AKC) {
#pragma unroll
      for (int i = 0; i < TMV; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(as + kc_offk<64>(wm * WTM + i * 32 + (lane & 31), ks * 2 + (lane >> 5)));
    } else {
#pragma unroll
      for (int i = 0; i < TMV; ++i) {
        const int byte = (wm * WTM + i * 32) * 2 + cb;
        af[i] = lds_tr_frag(as + mn_off<BM>(kb, byte), as + mn_off<BM>(kb + 4, byte));
      }
    }
    if constexpr (BKC) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const u32x4*>(bs + kc_offk<64>(wn * WTN + j * 32 + (lane & 31), ks * 2 + (lane >> 5)));
    } else {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int byte = (wn * WTN + j * 32) * 2 + cb;
        bfr[j] = lds_tr_frag(bs + mn_off<BN>(kb, byte), bs + mn_off<BN>(kb + 4, byte));
      }
    }
  }
  template <int TMV>
  MOE_DEV static void mma(f32x16 (&acc)[TM][TN], const u32x4 (&af)[TM], const u32x4 (&bfr)[TN]) {
#pragma unroll
    for (int i = 0; i < TMV; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) Mma<T>::run(acc[i][j], af[i], bfr[j]);
  }

  // nk stages into acc.  On entry stage 0 is in LDS (prologue) and stage 1 is
  // loading into the registers (or PRO: the prologue is the first step).  TMV: how many of the wave's four 32-row
  // sub-tiles hold rows of the segment; sub-tiles wholly past the segment's last
  // row skip their fragment reads and MFMAs (their accumulators stay zero and are
  // never stored); the operand loads, LDS writes and barriers are the same for
  // every wave.  PEEL: the first iteration is code of its own, so its wait for
  // stage 1 does not take in memory operations issued after those loads (they
  // complete in issue order).
  template <int TMV, bool PEEL, bool PRO = false>
  MOE_DEV void run(int nk, char* smem, f32x16 (&acc)[TM][TN]) {
    constexpr int NR = (AKC ? TMV : 2 * TMV) + (BKC ? TN : 2 * TN);   // LDS reads per k16 step
    u32x4 a0[TM], b0[TN], a1[TM], b1[TN];
    if constexpr (PERSIST) lanes();   // fragment offsets computed per tile (opaque_tid)
    if (nk > 0) {
      if constexpr (PRO) prologue(smem);   // PRO: the prologue runs here first
      frags<TMV>(smem, 0, a0, b0);
    }
    auto iter = [&](int kt) __attribute__((always_inline)) {
      const char* as = smem + (kt & 1) * STAGE;
      char* an = smem + ((kt + 1) & 1) * STAGE;   // the next stage, written during this one
      frags<TMV>(as, 1, a1, b1);
      mma<TMV>(acc, a0, b0);
      frags<TMV>(as, 2, a0, b0);
      store(an);
      load_ab(kt + 2);
      mma<TMV>(acc, a1, b1);
      frags<TMV>(as, 3, a1, b1);
      mma<TMV>(acc, a0, b0);
#pragma unroll
      for (int i = 0; i < TMV * TN; ++i) {          // block 1: MFMA + fragment read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < TMV * TN; ++i) {          // block 2: MFMA + LDS write + the load that refills
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // its registers (+ fragment read)
        if (i < ra.L + rb.L) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        if (i < ra.L + rb.L) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < TMV * TN; ++i) {          // block 3: MFMA + fragment read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);          // this wave's fragment reads and stage writes are done
      cta_barrier();
      frags<TMV>(an, 0, a0, b0);
      mma<TMV>(acc, a1, b1);
#pragma unroll
      for (int i = 0; i < TMV * TN; ++i) {          // block 4: MFMA + the next stage's first fragments
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      }
    };
    int kt = 0;
    if constexpr (PEEL) {
      if (nk > 0) iter(0);
      kt = 1;
    }
    for (; kt < nk; ++kt) iter(kt);
  }
};

template <int TM, int TN>
MOE_DEV void zero_acc(f32x16 (&acc)[TM][TN]) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
}

// One output tile: BM x BN with WM x WN waves of 128 x 64.  PERSIST: inside a
// persistent kernel's tile walk (lane values through opaque_tid, the epilogue's
// branch-free stores).
template <int BM, int BN, int WM, int WN, bool AKC, bool BKC, int GROUP, int EPI, int GATHER = 0, bool PERSIST = false>
MOE_DEV void big_tile(const Args& args, const TileCtx& ctx, char* smem) {
  using P = BigPipe<BM, BN, WM, WN, AKC, BKC, GROUP, EPI, GATHER, PERSIST>;
  P p;
  p.setup(args, ctx);
  f32x16 acc[P::TM][P::TN];
  zero_acc(acc);
  const int kext = (GROUP == GROUP_M) ? args.K : (ctx.k_end - ctx.k_begin);
  const int nk = kext > 0 ? (kext + P::BK - 1) / P::BK : 0;
  if constexpr (GROUP == GROUP_M) {
    const int valid = min(BM, ctx.row_end - ctx.row_begin) - p.wm * P::WTM;   // >= 1 by the tile decode
    if (valid > 96) p.template run<4, false, true>(nk, smem, acc);
    else if (valid > 64) p.template run<3, false, true>(nk, smem, acc);
    else if (valid > 32) p.template run<2, false, true>(nk, smem, acc);
    else p.template run<1, false, true>(nk, smem, acc);
  } else {
    p.template run<P::TM, false, true>(nk, smem, acc);
  }
  wave_epilogue<BM, BN, WM, WN, GROUP, EPI, PERSIST>(args, ctx, acc, smem);
}

// Weight gradients (GROUP_K), persistent: a block per CU walks the logical
// blocks b, b + gridDim.x, ... (gridDim.x a multiple of 8, so a block keeps to
// its XCD's chunks and every CU of an XCD gets the same share of each chunk).
// A wave that ends waits for its stores to be acknowledged, and a new block then
// waits for its first stages; here the next tile's first stages are fetched
// while this tile's fp32 rows are stored, in the gaps of the epilogue: the
// gathered operand's row indices before sub-tile 0, stage 0 after it, stage 0
// written to LDS and stage 1 fetched after sub-tile 1.  Loads complete in issue
// order, so waiting for them does not wait for the stores issued after them, and
// the stores drain under the next tile's first stages.  The epilogue's row slabs
// sit above stage 0 of the ring (in stage 1, idle until the next tile's first
// iteration, which follows a barrier).
template <bool AKC, bool BKC, int EPI, int GATHER>
MOE_DEV void big_wgrad_tiles(const Args& args, char* smem) {
  using P = BigPipe<256, 256, 2, 4, AKC, BKC, GROUP_K, EPI, GATHER, true>;
  auto stages = [](const TileCtx& c) {
    const int kext = c.k_end - c.k_begin;
    return kext > 0 ? (kext + P::BK - 1) / P::BK : 0;
  };
  P p;
  int b = blockIdx.x;
  TileCtx ctx;
  if (!decode_k_block<256, 256, kBigBK>(args, b, ctx)) return;
  f32x16 acc[P::TM][P::TN];
  zero_acc(acc);
  p.setup(args, ctx);
  p.prologue(smem);
  p.template run<P::TM, false>(stages(ctx), smem, acc);
  for (;;) {
    const int nb = b + (int)gridDim.x;
    TileCtx nx;
    const bool more = decode_k_block<256, 256, kBigBK>(args, nb, nx);
    if (more) p.setup(args, nx);
    // after the last stage's barrier no wave reads this tile's stages any more
    wave_epilogue<256, 256, 2, 4, GROUP_K, EPI, true>(args, ctx, acc, smem + P::STAGE, [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i == 0) {
        if (more) p.load_ab(0);
      } else if constexpr (i == 1) {
        if (more) {
          p.store(smem);
          p.load_ab(1);
        }
      }
    });
    if (!more) return;
    __builtin_amdgcn_s_waitcnt(0xc07f);   // stage 0 written, slab rows read back
    cta_barrier();
    ctx = nx;
    b = nb;
    zero_acc(acc);
    // reached only from here: its wait for stage 1 leaves out the stores above
    p.template run<P::TM, true>(stages(ctx), smem, acc);
  }
}

// GROUP_M decode over 128-row units (see the header comment): returns false when
// the block has no tile; *wide tells the shape.  Inside an expert, the tall
// tiles go in groups of kGroupM unit pairs with the n-tile outer and the pair
// inner, so consecutive tiles (one XCD) share weight columns in L2.
MOE_DEV bool big_decode_m(const Args& args, int b, TileCtx& c, bool* wide) {
  const int nW = (args.N + 511) / 512;
  const int total = args.tile_prefix[args.E] * nW;
  const int per = (total + 7) >> 3;
  if ((b >> 3) >= per) return false;
  const int L = (b & 7) * per + (b >> 3);
  if (L >= total) return false;
  const int e = args.tile_expert[L / nW];
  const int p0 = args.tile_prefix[e], ue = args.tile_prefix[e + 1] - p0;
  const int q = L - p0 * nW;                 // tile index inside the expert
  const int pairs = ue >> 1, ntall = 2 * nW;
  c.e = e; c.split = 0; c.slot = -1;
  c.row_end = args.offsets[e + 1];
  c.k_begin = 0; c.k_end = args.K;
  if (q < pairs * ntall) {      // tall: unit pair `pair`, n-tile nt
    const int g = q / (kGroupM * ntall);
    const int gsize = min(kGroupM, pairs - g * kGroupM);
    const int within = q - g * kGroupM * ntall;
    const int nt = within / gsize;
    const int pair = g * kGroupM + (within - nt * gsize);
    *wide = false;
    c.mt = pair; c.nt = nt;
    c.row_begin = args.offsets[e] + pair * 256;
    c.m0 = pair * 256; c.n0 = nt * 256;
  } else {                      // wide: the odd last unit
    const int cq = q - pairs * ntall;
    *wide = true;
    c.mt = ue - 1; c.nt = cq;
    c.row_begin = args.offsets[e] + (ue - 1) * 128;
    c.m0 = (ue - 1) * 128; c.n0 = cq * 512;
  }
  return true;
}

// Row-segment GEMMs with a bf16 output (GROUP_M, EPI_ACT: down, dX_perm),
// persistent: a block per CU takes the logical blocks b, b + gridDim.x, ... of
// big_decode_m (gridDim.x a multiple of 8: the block keeps to its XCD's range),
// in two passes.  First its tall tiles, each started inside the previous one's
// epilogue as the weight gradients do (big_wgrad_tiles); each wave still skips
// the sub-tiles of its rows that lie past the segment (one main-loop copy per
// count, chosen per tile).  Then its wide tiles (an expert's odd last unit) as
// in the one-tile kernel: in one pass the wide tiles' code would hold the tall
// chain's values live across it and spill.
template <bool AKC, bool BKC, int EPI, int GATHER>
MOE_DEV void big_rows_tiles(const Args& args, char* smem) {
  using P = BigPipe<256, 256, 2, 4, AKC, BKC, GROUP_M, EPI, GATHER, true>;
  const int nk = (args.K + P::BK - 1) / P::BK;
  const int G = (int)gridDim.x;
  // the first tall tile at block index bb or later (bb advanced to it); false past the end
  auto next_tall = [&](int& bb, TileCtx& c) __attribute__((always_inline)) {
    for (;; bb += G) {
      bool w = false;
      if (!big_decode_m(args, bb, c, &w)) return false;
      if (!w) return true;
    }
  };
  int b = blockIdx.x;
  TileCtx ctx;
  if (next_tall(b, ctx)) {
    P p;
    f32x16 acc[P::TM][P::TN];
    // the main loop with this wave's count of sub-tiles holding rows of the
    // segment (>= 1 by the tile decode); PEEL: reached from a prefetch, else
    // the prologue runs first
    auto main_loop = [&](auto peel_c) __attribute__((always_inline)) {
      constexpr bool PEEL = decltype(peel_c)::value;
      const int valid = min(256, ctx.row_end - ctx.row_begin) - p.wm * P::WTM;
      if (valid > 96) p.template run<4, PEEL, !PEEL>(nk, smem, acc);
      else if (valid > 64) p.template run<3, PEEL, !PEEL>(nk, smem, acc);
      else if (valid > 32) p.template run<2, PEEL, !PEEL>(nk, smem, acc);
      else p.template run<1, PEEL, !PEEL>(nk, smem, acc);
    };
    p.setup(args, ctx);
    zero_acc(acc);
    main_loop(std::false_type{});
    for (;;) {
      int nb = b + G;
      TileCtx nx;
      const bool pre = next_tall(nb, nx);
      if (pre) p.setup(args, nx);
      // after the last stage's barrier no wave reads this tile's stages any more
      wave_epilogue<256, 256, 2, 4, GROUP_M, EPI, true>(args, ctx, acc, smem + P::STAGE,
                                                        [&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i == 0) {
          if (pre) p.load_ab(0);
        } else if constexpr (i == 1) {
          if (pre) {
            p.store(smem);
            p.load_ab(1);
          }
        }
      });
      if (!pre) break;
      __builtin_amdgcn_s_waitcnt(0xc07f);   // stage 0 written, slab rows read back
      cta_barrier();
      b = nb;
      ctx = nx;
      zero_acc(acc);
      main_loop(std::true_type{});
    }
  }
  for (int bb = blockIdx.x;; bb += G) {
    TileCtx c;
    bool w = false;
    if (!big_decode_m(args, bb, c, &w)) return;
    if (!w) continue;
    __builtin_amdgcn_s_waitcnt(0xc07f);     // the previous tile's LDS reads done
    cta_barrier();                          // before this tile writes its ring
    big_tile<128, 512, 1, 8, AKC, BKC, GROUP_M, EPI, GATHER, true>(args, c, smem);
  }
}

// LDS of the persistent row-segment kernel: the wide tiles' ring (the whole LDS)
constexpr size_t big_rows_lds_bytes() { return big_ring_bytes<128, 512>(); }

// LDS of the persistent weight-gradient kernel: stage 0, then the larger of
// stage 1 and the epilogue's row slabs (eight waves x 32 rows x 72 floats)
constexpr size_t big_wgrad_lds_bytes() {
  constexpr size_t stage = (size_t)(256 + 256) * kBigBK * 2, slabs = (size_t)8 * 32 * (64 + 8) * 4;
  return stage + (slabs > stage ? slabs : stage);
}

template <bool AKC, bool BKC, int EPI, int GATHER>
__global__ __launch_bounds__(kBigThreads) void grouped_wgrad_big(Args args) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  big_wgrad_tiles<AKC, BKC, EPI, GATHER>(args, smem);
}

template <bool AKC, bool BKC, int EPI, int GATHER>
__global__ __launch_bounds__(kBigThreads) void grouped_rows_big(Args args) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  big_rows_tiles<AKC, BKC, EPI, GATHER>(args, smem);
}

template <bool AKC, bool BKC, int GROUP, int EPI, int GATHER = 0>
__global__ __launch_bounds__(kBigThreads) void grouped_gemm_big(Args args) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  static_assert(GROUP == GROUP_M || GROUP == GROUP_K, "grouped GEMMs only");
  TileCtx ctx;
  if constexpr (GROUP == GROUP_K) {
    if (!decode_tile<256, 256, kBigBK, GROUP_K>(args, ctx)) return;
    big_tile<256, 256, 2, 4, AKC, BKC, GROUP, EPI, GATHER>(args, ctx, smem);
  } else {
    bool wide = false;
    if (!big_decode_m(args, blockIdx.x, ctx, &wide)) return;
    if (wide) big_tile<128, 512, 1, 8, AKC, BKC, GROUP, EPI, GATHER>(args, ctx, smem);
    else big_tile<256, 256, 2, 4, AKC, BKC, GROUP, EPI, GATHER>(args, ctx, smem);
  }
}

}  // namespace moe_gemm
