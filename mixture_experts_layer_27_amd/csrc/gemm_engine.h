// Grouped GEMM engine for gfx950 (CDNA4): one template covers every expert GEMM
// of the MoE layer and the two router GEMMs.
//
//   D[m, n] = sum_k A[m, k] * B[n, k]        (B given as [N,K] or as [K,N])
//
// * Element type: bf16 (v_mfma_f32_32x32x16_bf16) or fp32 (v_mfma_f32_32x32x2_f32);
//   fp32 accumulation either way.
// * Operand layouts: "KC" = K contiguous ([rows, K] row-major), or "MN" = M/N
//   contiguous ([K, rows]); MN operands are transposed in registers while they
//   are staged into LDS, so the LDS tile is always [rows][K] and the MFMA loop
//   is the same for every variant.
// * Grouping: GROUP_M -- rows of A are split into per-expert segments given by
//   device offsets (forward GEMMs, dA', dX); GROUP_K -- the reduction runs over
//   one expert's segment of rows (weight gradients, variable K); GROUP_NONE --
//   one plain problem (router GEMMs), optionally split along K.
// * Tiles: BM x BN block tile, BK = 128 bytes of K per stage, WM x WN waves,
//   each wave owns (BM/WM) x (BN/WN) as 32x32 MFMA sub-tiles.  Two LDS stages,
//   register-staged global loads for stage k+1 overlap the MFMAs of stage k.
//   LDS rows are 128 B; 16-byte chunks are XOR-swizzled by (row ^ row>>3) & 7 so
//   the MFMA fragment reads (32 consecutive rows, one chunk) and the transposed
//   stores (rows 8 apart) are both free of bank conflicts.
// * Block -> tile order is XCD-aware: hardware block b runs on XCD b % 8, so
//   consecutive logical tiles (same expert and weight tile) go to one XCD and
//   share its L2.
#pragma once
#include <type_traits>
#include "moe_common.h"

namespace moe_gemm {

enum { GROUP_M = 0, GROUP_K = 1, GROUP_NONE = 2 };
enum { EPI_ACT = 0, EPI_F32 = 1, EPI_SWIGLU = 2, EPI_DSWIGLU = 3, EPI_LOGITS = 4,
       EPI_SWIGLU_MX = 6, EPI_DSWIGLU_MX = 7,   // *_MX: also emit an MXFP8 copy of A / dH
       EPI_GATE_SCATTER = 8 };   // act dtype: row r scaled by row_gate[r], stored at row c_rows[r]

struct Args {
  const void* A; int64_t lda; int64_t a_estride; const int32_t* a_gather;
  const void* B; int64_t ldb; int64_t b_estride; const int32_t* b_gather;   // b_gather: GROUP_K k rows of B
  int64_t gather_rows;          // rows of the tensor a_gather indexes (bounds of gathered loads)
  void* C; int64_t ldc; int64_t c_estride;
  const int32_t* c_rows;        // EPI_GATE_SCATTER: output row of each GEMM row
  void* C2; int64_t ldc2;
  float* C3; int64_t ldc3;
  const void* aux; int64_t ld_aux;
  const float* row_gate;
  const float* bias;
  const int32_t* offsets;       // [E+1] segment offsets (GROUP_M rows, GROUP_K reduction rows)
  const int32_t* tile_prefix;   // [E+1] prefix of per-expert m-tile counts (GROUP_M)
  const int32_t* tile_expert;   // [prefix[E]] expert of each m-tile (GROUP_M)
  const int4* chunks;           // GROUP_K: (expert, k_begin, k_end, partial slot or -1) per K chunk
  const int32_t* nchunks;       // GROUP_K: number of chunks (device)
  void* Cpart;                  // GROUP_K: partial outputs of chunks past an expert's first, stride c_estride
  // *_MX epilogues: MXFP8 codes [rows][q_ld] and stage-major scales [q_ld/64][q_srows][2] of the
  // quantised output, rows expert-padded (row r of expert e at r - offsets[e] + q_pad[e])
  uint8_t* q_codes; uint8_t* q_scales; int64_t q_ld; int64_t q_srows; const int32_t* q_pad;
  // EPI_DSWIGLU_MX: dH and gA also along the token axis (the weight gradients' K): codes
  // [2f][t_len] / [f][t_len] over expert-padded positions, scales [t_len/64][2f or f][2]
  uint8_t* t_codes; uint8_t* t_scales; uint8_t* t2_codes; uint8_t* t2_scales; int64_t t_len;
  int M, N, K, E, f;
  int tilesM, tilesN;
  int total_static;             // GROUP_K / GROUP_NONE: number of logical tiles
  int ksplit;                   // GROUP_NONE: number of K slices (1 = none)
  int64_t c_kstride;            // GROUP_NONE split-K: stride between partial outputs
};

MOE_DEV int swz(int row) { return (row ^ (row >> 3)) & 7; }
MOE_DEV int lds_off(int row, int byte) {  // byte offset inside a 128 B row
  return row * 128 + ((((byte >> 4) ^ swz(row)) << 4) | (byte & 15));
}

// ---------------------------------------------------------------- staging
// One operand tile: ROWS rows x 128 bytes of K.

template <typename T, int ROWS, int NT>
struct KcStage {  // K-contiguous source
  static constexpr int CHUNKS = ROWS * 8;
  static constexpr int PER = CHUNKS / NT;
  static constexpr int EPC = 16 / sizeof(T);
  static_assert(CHUNKS % NT == 0, "K-contiguous tile must split evenly");
  const T* rowp[PER];
  u32x4 v[PER];
  // rowfn(row) -> pointer to element (row, 0) of this tile's source row
  template <class RowFn>
  MOE_DEV void init(RowFn rowfn) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int c = threadIdx.x + i * NT;
      rowp[i] = rowfn(c >> 3) + (c & 7) * EPC;
    }
  }
  // k0: first K element of the stage; kvalid: valid K elements from k0 (per-chunk mask)
  MOE_DEV void load(int k0, int kvalid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int ch = (threadIdx.x + i * NT) & 7;
      if (ch * EPC < kvalid) v[i] = ldg16(rowp[i] + k0);
      else v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  MOE_DEV void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int c = threadIdx.x + i * NT;
      *reinterpret_cast<u32x4*>(lds + lds_off(c >> 3, (c & 7) << 4)) = v[i];
    }
  }
};

template <typename T, int ROWS, int NT>
struct MnStage {  // M/N-contiguous source: element (k, row) at base + k*ld + row
  static constexpr int V = 16 / sizeof(T);            // rows per 16 B vector
  static constexpr int BK = 128 / sizeof(T);
  static constexpr int EPT = ROWS * BK / NT;          // elements per thread
  static constexpr int R0 = EPT / V;                  // k values per thread
  static constexpr int R = R0 > 8 ? 8 : R0;           // k per unit
  static constexpr int UPT = R0 / R;                  // units per thread
  static_assert(EPT % V == 0 && R0 % R == 0 && R >= 2, "transposed tile must split evenly");
  static constexpr int RB = ROWS / V;                 // row blocks
  u32x4 v[UPT][R];
  // base points at (k0, row0); kvalid = valid k rows from k0; rvalid = valid rows
  MOE_DEV void load(const T* base, int64_t ld, int kvalid, int rvalid) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      int unit = threadIdx.x + u * NT;
      int rb = unit % RB, kb = unit / RB;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        int k = kb * R + r;
        int row = rb * V;
        if (k < kvalid && row < rvalid) v[u][r] = ldg16(base + (int64_t)k * ld + row);
        else v[u][r] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  MOE_DEV void store(char* lds) const {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      int unit = threadIdx.x + u * NT;
      int rb = unit % RB, kb = unit / RB;
      int kbyte = kb * R * (int)sizeof(T);
      if constexpr (sizeof(T) == 2) {
        // 8 rows x R k values of bf16: output row j collects element j of each k vector
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint32_t w[4];
#pragma unroll
          for (int p = 0; p < R / 2; ++p) {
            uint32_t a = v[u][2 * p][j >> 1], b = v[u][2 * p + 1][j >> 1];
            uint32_t lo = (j & 1) ? (a >> 16) : (a & 0xffffu);
            uint32_t hi = (j & 1) ? (b & 0xffff0000u) : (b << 16);
            w[p] = lo | hi;
          }
          char* dst = lds + lds_off(rb * 8 + j, kbyte);
          if constexpr (R == 8) *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
          else if constexpr (R == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
          else *reinterpret_cast<uint32_t*>(dst) = w[0];
        }
      } else {
        // 4 rows x R k values of fp32
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t w[8];
#pragma unroll
          for (int r = 0; r < R; ++r) w[r] = v[u][r][j];
          if constexpr (R >= 4) {
#pragma unroll
            for (int q = 0; q < R / 4; ++q)  // each 16 B chunk has its own swizzled slot
              *reinterpret_cast<u32x4*>(lds + lds_off(rb * 4 + j, kbyte + 16 * q)) =
                  u32x4{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
          } else {
            *reinterpret_cast<uint2*>(lds + lds_off(rb * 4 + j, kbyte)) = make_uint2(w[0], w[1]);
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------- MFMA step

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
  // one 16-byte fragment per lane = 8 k values -> one 32x32x16 MFMA
  static MOE_DEV void run(f32x16& acc, u32x4 a, u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  // one 16-byte fragment per lane = 4 k values -> four 32x32x2 MFMAs; lanes 0-31
  // and 32-63 hold different k, identically for A and B, so every product pairs up
  static MOE_DEV void run(f32x16& acc, u32x4 a, u32x4 b) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[j]), __uint_as_float(b[j]), acc, 0, 0, 0);
  }
};

// ---------------------------------------------------------------- 8-wide vectors

template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
  static MOE_DEV float rnd(float v) { return bf2f(f2bf(v)); }
  static MOE_DEV void load(const bf16_t* p, float* v) {
    u32x4 a = ldg16(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(a[q] << 16);
      v[2 * q + 1] = __uint_as_float(a[q] & 0xffff0000u);
    }
  }
  static MOE_DEV void store(bf16_t* p, const float* v) {
    u32x4 a;
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = pack_bf2(v[2 * q], v[2 * q + 1]);
    stg16(p, a);
  }
};
template <> struct Vec8<float> {
  static MOE_DEV float rnd(float v) { return v; }
  static MOE_DEV void load(const float* p, float* v) {
    u32x4 a = ldg16(p), b = ldg16(p + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = __uint_as_float(a[q]);
      v[4 + q] = __uint_as_float(b[q]);
    }
  }
  static MOE_DEV void store(float* p, const float* v) {
    stg16(p, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
    stg16(p + 4, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
  }
};

// ---------------------------------------------------------------- kernel

// Logical tile of this block, in XCD-aware order: hardware block b runs on XCD
// b % 8, so logical tile (b % 8) * per + b / 8 gives each XCD a contiguous run of
// logical tiles.  Returns false when the block has no tile.
struct TileCtx {
  int e, mt, nt, split;
  int row_begin, row_end;   // GROUP_M: rows of A / D of this tile's expert segment
  int k_begin, k_end;       // reduction range (segment rows for GROUP_K, a K slice for split-K)
  int m0, n0;
  int slot;                 // GROUP_K: partial-output slot of the chunk, -1 = the expert's own output
};

constexpr int kGroupM = 4;

// Number of logical tiles of the launch (GROUP_M: read from the plan on the device).
template <int GROUP>
MOE_DEV int total_tiles(const Args& args) {
  if constexpr (GROUP == GROUP_M) return args.tile_prefix[args.E] * args.tilesN;
  else if constexpr (GROUP == GROUP_K) return *args.nchunks * args.tilesM * args.tilesN;
  else return args.total_static;
}

// Tile coordinates of logical tile L (0 <= L < total_tiles).
template <int BM, int BN, int BK, int GROUP>
MOE_DEV void decode_at(const Args& args, int L, TileCtx& c) {
  int e = 0, mt = 0, nt = 0, split = 0, slot = -1;
  int row_begin = 0, row_end = 0;
  int k_begin = 0, k_end = args.K;
  if constexpr (GROUP == GROUP_M) {
    // expert e holds logical tiles [prefix[e]*tilesN, prefix[e+1]*tilesN), so
    // L / tilesN is one of its m-tile indices
    e = args.tile_expert[L / args.tilesN];
    int p0 = args.tile_prefix[e], cnt = args.tile_prefix[e + 1] - p0;
    int r = L - p0 * args.tilesN;
    // m-tiles of the expert in groups of kGroupM; inside a group the n-tile is
    // outer and the m-tile inner, so a window of consecutive tiles covers a few
    // m-tiles x several n-tiles and both operands are reused from L2
    const int g = r / (kGroupM * args.tilesN);
    const int gsize = min(kGroupM, cnt - g * kGroupM);
    const int within = r - g * kGroupM * args.tilesN;
    nt = within / gsize;
    mt = g * kGroupM + (within - nt * gsize);
    row_begin = args.offsets[e] + mt * BM;
    row_end = args.offsets[e + 1];
  } else if constexpr (GROUP == GROUP_K) {
    // logical tile L = chunk * tiles_per_chunk + r; a chunk is a piece of at most
    // a fixed number of one expert's rows, so tiles stay balanced however
    // unevenly the experts are loaded
    const int pe = args.tilesM * args.tilesN;
    const int q = L / pe;
    const int r = L - q * pe;
    const int4 ch = args.chunks[q];
    e = ch.x;
    k_begin = ch.y;
    k_end = ch.z;
    slot = ch.w;
    // n-tile fastest: consecutive tiles write one contiguous band of output rows
    mt = r / args.tilesN;
    nt = r - mt * args.tilesN;
  } else {
    int pe = args.tilesM * args.tilesN;
    split = L / pe;
    int r = L - split * pe;
    nt = r / args.tilesM;
    mt = r - nt * args.tilesM;
    int kc = (((args.K + args.ksplit - 1) / args.ksplit) + BK - 1) / BK * BK;
    k_begin = split * kc;
    k_end = min(args.K, k_begin + kc);
  }
  c.e = e; c.mt = mt; c.nt = nt; c.split = split;
  c.row_begin = row_begin; c.row_end = row_end;
  c.k_begin = k_begin; c.k_end = k_end;
  c.m0 = mt * BM; c.n0 = nt * BN;
  c.slot = slot;
}

// Output base of a GROUP_K tile: the expert's own slab, or a partial slot.
template <typename OT>
MOE_DEV OT* wgrad_out(const Args& args, const TileCtx& c) {
  return c.slot < 0 ? reinterpret_cast<OT*>(args.C) + (int64_t)c.e * args.c_estride
                    : reinterpret_cast<OT*>(args.Cpart) + (int64_t)c.slot * args.c_estride;
}

// GROUP_K tile of block index b: chunks go round robin over the XCDs (chunk q on
// XCD q % 8, block b on XCD b % 8), all tiles of a chunk on one XCD: its rows of
// both operands are read into one L2.  False past the last chunk (and for every
// later b of the same XCD).
// The chunk table is read with block-uniform addresses; a persistent kernel's
// stores keep the compiler from using scalar loads for it, so the values are
// moved to scalar registers explicitly (the buffer descriptors built from them
// must be uniform).
// Without a chunk table (args.chunks null) the launch is one reduction over K
// rows in args.ksplit chunks of equal length (a multiple of BK; the router
// weight gradient): chunk 0 writes C, chunk q > 0 partial slot q - 1.
template <int BM, int BN, int BK>
MOE_DEV bool decode_k_block(const Args& args, int b, TileCtx& c) {
  const int pe = args.tilesM * args.tilesN;
  const int t = b >> 3;
  const int q = (b & 7) + 8 * (t / pe);
  if (args.chunks == nullptr) {
    if (q >= args.ksplit) return false;
    const int kc = (((args.K + args.ksplit - 1) / args.ksplit) + BK - 1) / BK * BK;
    const int r = t % pe;
    c.e = 0; c.split = 0; c.slot = q - 1;
    c.k_begin = q * kc; c.k_end = min(args.K, c.k_begin + kc);
    c.row_begin = c.row_end = 0;
    c.mt = r / args.tilesN; c.nt = r - c.mt * args.tilesN;
    c.m0 = c.mt * BM; c.n0 = c.nt * BN;
    return true;
  }
  if (q >= __builtin_amdgcn_readfirstlane(*args.nchunks)) return false;
  decode_at<BM, BN, BK, GROUP_K>(args, q * pe + t % pe, c);
  c.e = __builtin_amdgcn_readfirstlane(c.e);
  c.k_begin = __builtin_amdgcn_readfirstlane(c.k_begin);
  c.k_end = __builtin_amdgcn_readfirstlane(c.k_end);
  c.slot = __builtin_amdgcn_readfirstlane(c.slot);
  return true;
}

template <int BM, int BN, int BK, int GROUP>
MOE_DEV bool decode_tile(const Args& args, TileCtx& c) {
  if constexpr (GROUP == GROUP_K) return decode_k_block<BM, BN, BK>(args, blockIdx.x, c);
  const int total = total_tiles<GROUP>(args);
  const int per = (total + 7) >> 3;
  const int b = blockIdx.x;
  if ((b >> 3) >= per) return false;
  const int L = (b & 7) * per + (b >> 3);
  if (L >= total) return false;
  decode_at<BM, BN, BK, GROUP>(args, L, c);
  return true;
}

// Epilogue shared by both main loops.  acc holds the wave's (BM/WM) x (BN/WN)
// tile as 32x32 MFMA sub-tiles; LDS (at least (BM/WM) * (BN+8) floats) must be
// free.  Ends with a barrier.
template <typename T, int BM, int BN, int WM, int WN, int GROUP, int EPI>
MOE_DEV void gemm_epilogue(const Args& args, const TileCtx& ctx, f32x16 (&acc)[BM / WM / 32][BN / WN / 32],
                           char* smem) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int e = ctx.e, nt = ctx.nt, split = ctx.split;
  const int row_begin = ctx.row_begin, row_end = ctx.row_end;
  const int m0 = ctx.m0, n0 = ctx.n0;
  (void)e; (void)split; (void)nt;
  // ---- epilogue.  The accumulators are staged through LDS one wave-row at a
  // time (sub-tile (i, j), register q holds row i*32 + 8*(q/4) + 4*(lane/32) + q%4,
  // column j*32 + lane%32 of the wave tile); then every thread works on 8
  // consecutive columns of one row, so global loads/stores are 16-byte vectors
  // and 32 consecutive lanes cover one 256-column row.
  constexpr int CS = BN + 8;          // staged row stride (floats)
  constexpr int CPR = BN / 8;         // 8-column chunks per row
  float* cs = reinterpret_cast<float*>(smem);
  for (int pass = 0; pass < WM; ++pass) {
    if (wm == pass) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q)
            cs[(i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)) * CS + wn * WTN + j * 32 + (lane & 31)] =
                acc[i][j][q];
    }
    __syncthreads();
    const int r0 = pass * WTM;
    if constexpr (EPI == EPI_SWIGLU) {
      // tile columns [0, BN/2) are gate columns g0.., [BN/2, BN) the matching up columns
      constexpr int HC = CPR / 2;
      T* H = reinterpret_cast<T*>(args.C);
      T* Aout = reinterpret_cast<T*>(args.C2);
      for (int u = threadIdx.x; u < WTM * HC; u += NT) {
        const int rr = u / HC, ch = u % HC;
        const int grow = row_begin + r0 + rr;
        if (grow >= row_end) continue;
        const float* src = cs + rr * CS + ch * 8;
        float hg[8], hu[8], a[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          hg[c] = Vec8<T>::rnd(src[c]);              // H as stored
          hu[c] = Vec8<T>::rnd(src[BN / 2 + c]);
          a[c] = hg[c] / (1.0f + expf(-hg[c])) * hu[c];
        }
        const int gcol = nt * (BN / 2) + ch * 8;
        T* hrow = H + (int64_t)grow * args.ldc;
        Vec8<T>::store(hrow + gcol, hg);
        Vec8<T>::store(hrow + args.f + gcol, hu);
        Vec8<T>::store(Aout + (int64_t)grow * args.ldc2 + gcol, a);
      }
    } else if constexpr (EPI == EPI_DSWIGLU) {
      // cs = dA' for columns n0.. of f.  aux = H [rows, 2f]; C = dH [rows, 2f];
      // C2 = gA [rows, f]; C3[nt * ldc3 + row] = this tile's part of dS = <dA', A>
      static_assert((WTM * CPR) % NT == 0 && CPR <= 64, "uniform trip count for the row reduction");
      const T* H = reinterpret_cast<const T*>(args.aux);
      T* dH = reinterpret_cast<T*>(args.C);
      T* gA = reinterpret_cast<T*>(args.C2);
      for (int u = threadIdx.x; u < WTM * CPR; u += NT) {
        const int rr = u / CPR, ch = u % CPR;
        const int grow = row_begin + r0 + rr;
        const int col = n0 + ch * 8;
        float part = 0.0f;
        if (grow < row_end && col < args.N) {
          const float* src = cs + rr * CS + ch * 8;
          const float g = args.row_gate[grow];
          const T* hrow = H + (int64_t)grow * args.ld_aux;
          float hg[8], hu[8], dhg[8], dhu[8], ga[8];
          Vec8<T>::load(hrow + col, hg);
          Vec8<T>::load(hrow + args.f + col, hu);
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float dap = src[c];
            const float sg = 1.0f / (1.0f + expf(-hg[c]));
            const float sl = hg[c] * sg;
            const float a = Vec8<T>::rnd(sl * hu[c]);      // A as stored in the forward
            part += dap * a;
            const float da = g * dap;
            dhg[c] = da * hu[c] * (sg * (1.0f + hg[c] * (1.0f - sg)));
            dhu[c] = da * sl;
            ga[c] = g * a;
          }
          T* drow = dH + (int64_t)grow * args.ldc;
          Vec8<T>::store(drow + col, dhg);
          Vec8<T>::store(drow + args.f + col, dhu);
          Vec8<T>::store(gA + (int64_t)grow * args.ldc2 + col, ga);
        }
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) part += __shfl_xor(part, o, 64);
        if (ch == 0 && grow < row_end) args.C3[(int64_t)nt * args.ldc3 + grow] = part;
      }
    } else {
      // EPI_ACT (act dtype), EPI_F32 (fp32, split-K partials / per-expert slabs), EPI_LOGITS (+ bias)
      using OT = typename std::conditional<EPI == EPI_ACT, T, float>::type;
      OT* C = reinterpret_cast<OT*>(args.C);
      if constexpr (GROUP == GROUP_K) C = wgrad_out<OT>(args, ctx);
      if constexpr (GROUP == GROUP_NONE) C += (int64_t)split * args.c_kstride;
      for (int u = threadIdx.x; u < WTM * CPR; u += NT) {
        const int rr = u / CPR, ch = u % CPR;
        int grow;
        bool ok;
        if constexpr (GROUP == GROUP_M) { grow = row_begin + r0 + rr; ok = grow < row_end; }
        else { grow = m0 + r0 + rr; ok = grow < args.M; }
        const int col = n0 + ch * 8;
        if (!ok || col >= args.N) continue;
        const float* src = cs + rr * CS + ch * 8;
        float v[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = src[c];
        OT* dst = C + (int64_t)grow * args.ldc + col;
        if constexpr (EPI == EPI_LOGITS) {   // + bias [N], + noise [M, N] (args.aux, routing noise)
          const float* nz = args.aux ? reinterpret_cast<const float*>(args.aux) + (int64_t)grow * args.ld_aux : nullptr;
#pragma unroll
          for (int c = 0; c < 8; ++c)
            if (col + c < args.N) dst[c] = (v[c] + (args.bias ? args.bias[col + c] : 0.0f)) + (nz ? nz[col + c] : 0.0f);
        } else {
          Vec8<OT>::store(dst, v);
        }
      }
    }
    __syncthreads();
  }
}

template <typename T, int BM, int BN, int WM, int WN, bool AKC, bool BKC, int GROUP, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm(Args args) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = 128 / sizeof(T);
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold a 32x32 MFMA tile");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // stage s: A tile at s*(BM+BN)*128, B tile right after it
  auto a_stage = [&](int st) -> char* { return smem + st * (BM + BN) * 128; };
  auto b_stage = [&](int st) -> char* { return smem + st * (BM + BN) * 128 + BM * 128; };

  TileCtx ctx;
  if (!decode_tile<BM, BN, BK, GROUP>(args, ctx)) return;
  const int e = ctx.e, nt = ctx.nt;
  const int row_begin = ctx.row_begin, row_end = ctx.row_end;
  const int k_begin = ctx.k_begin, k_end = ctx.k_end;
  const int m0 = ctx.m0, n0 = ctx.n0;
  const T* Ab = reinterpret_cast<const T*>(args.A) + (int64_t)e * args.a_estride;
  const T* Bb = reinterpret_cast<const T*>(args.B) + (int64_t)e * args.b_estride;

  // ---- operand row pointers (K-contiguous operands)
  auto a_row = [&](int row) -> const T* {
    if constexpr (GROUP == GROUP_M) {
      int g = row_begin + row;
      if (g >= row_end) g = row_end - 1;       // rows past the segment only feed unstored outputs
      int src = args.a_gather ? args.a_gather[g] : g;
      return Ab + (int64_t)src * args.lda;
    } else {
      int g = m0 + row;
      if (g >= args.M) g = args.M - 1;
      return Ab + (int64_t)g * args.lda;
    }
  };
  auto b_row = [&](int row) -> const T* {
    int j = n0 + row;
    if constexpr (EPI == EPI_SWIGLU) {
      // tile rows [0, BN/2): gate rows g0..; [BN/2, BN): the matching up rows
      const int g0 = nt * (BN / 2);
      j = (row < BN / 2) ? (g0 + row) : (args.f + g0 + row - BN / 2);
    }
    if (j >= args.N && EPI != EPI_SWIGLU) j = args.N - 1;
    return Bb + (int64_t)j * args.ldb;
  };

  using AStage = typename std::conditional<AKC, KcStage<T, BM, NT>, MnStage<T, BM, NT>>::type;
  using BStage = typename std::conditional<BKC, KcStage<T, BN, NT>, MnStage<T, BN, NT>>::type;
  AStage sa;
  BStage sb;
  if constexpr (AKC) sa.init(a_row);
  if constexpr (BKC) sb.init(b_row);

  auto load_tiles = [&](int k0) {
    int kvalid = k_end - k0;
    if constexpr (AKC) {
      sa.load(k0, kvalid);
    } else {
      // A stored [K, M]: rows of the tile are M positions
      sa.load(Ab + (int64_t)k0 * args.lda + m0, args.lda, kvalid, args.M - m0);
    }
    if constexpr (BKC) {
      sb.load(k0, kvalid);
    } else {
      sb.load(Bb + (int64_t)k0 * args.ldb + n0, args.ldb, kvalid, args.N - n0);
    }
  };

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  const int nk = (k_end > k_begin) ? (k_end - k_begin + BK - 1) / BK : 0;
  if (nk > 0) {
    load_tiles(k_begin);
    sa.store(a_stage(0));
    sb.store(b_stage(0));
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) load_tiles(k_begin + (kt + 1) * BK);
    const char* as = a_stage(cur);
    const char* bs = b_stage(cur);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kbyte = (ks * 2 + (lane >> 5)) << 4;
      u32x4 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(as + lds_off(wm * WTM + i * 32 + (lane & 31), kbyte));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const u32x4*>(bs + lds_off(wn * WTN + j * 32 + (lane & 31), kbyte));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) Mma<T>::run(acc[i][j], af[i], bfr[j]);
    }
    if (more) {
      sa.store(a_stage(cur ^ 1));
      sb.store(b_stage(cur ^ 1));
    }
    __syncthreads();
  }

  gemm_epilogue<T, BM, BN, WM, WN, GROUP, EPI>(args, ctx, acc, smem);
}

// Dynamic LDS of one block: two operand stages, or the staged accumulator rows
// of the epilogue, whichever is larger.
template <typename T, int BM, int BN, int WM, int WN>
constexpr size_t lds_bytes() {
  constexpr size_t main_loop = (size_t)2 * (BM + BN) * 128;
  constexpr size_t epi = (size_t)(BM / WM) * (BN + 8) * 4;
  return main_loop > epi ? main_loop : epi;
}

}  // namespace moe_gemm
