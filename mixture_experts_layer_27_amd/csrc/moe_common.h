// Shared device helpers for the gfx950 MoE kernels: bf16 conversions, vector
// types, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bfloat16 bit pattern

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define MOE_DEV __device__ __forceinline__

MOE_DEV float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// float -> bfloat16, round to nearest even; a NaN keeps its top payload bits and
// becomes quiet.  gfx950 converts in hardware (v_cvt_pk_bf16_f32), identical
// bit for bit to the integer rounding (u + 0x7fff + ((u >> 16) & 1)) >> 16 on
// every non-NaN input, which is what the conversion computes.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
MOE_DEV bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

MOE_DEV uint32_t pack_bf2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Element access for the two activation types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static MOE_DEV float load(const float* p) { return *p; }
  static MOE_DEV void store(float* p, float v) { *p = v; }
  static constexpr int bytes = 4;
};
template <> struct Elem<bf16_t> {
  static MOE_DEV float load(const bf16_t* p) { return bf2f(*p); }
  static MOE_DEV void store(bf16_t* p, float v) { *p = f2bf(v); }
  static constexpr int bytes = 2;
};

MOE_DEV float silu_f(float x) { return x / (1.0f + __expf(-x)); }
MOE_DEV float sigmoid_f(float x) { return 1.0f / (1.0f + __expf(-x)); }

// wave64 reductions
MOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
MOE_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

MOE_DEV int lane_id() { return threadIdx.x & 63; }

// 16-byte global/LDS copies
MOE_DEV u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// 16-byte load of data read once (a non-temporal hint: not kept in the caches).
// Streaming reads of HBM run at ~7.0 TB/s this way on MI355X against ~5.4 TB/s
// with ordinary loads.
MOE_DEV u32x4 ldg16_nt(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
MOE_DEV f32x4 ldf4_nt(const float* p) { return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)); }
MOE_DEV void stg16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
MOE_DEV void stg16_nt(void* p, u32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p)); }
