// Reference streaming kernels: the practical HBM rates of plain reads, writes
// and copies on this GPU, timed next to the layer's data-movement kernels
// (permute, combine, input-gradient gather) so their fractions of the ceiling
// are measured, not assumed.  Not part of the layer.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

// mode 0: read (non-temporal loads); 1: write; 2: copy, non-temporal loads and
// ordinary stores; 3: copy, non-temporal loads and stores.  Four 16-byte vectors
// per thread per pass, grid-stride over n vectors.
template <int MODE>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                     int64_t n) {
  constexpr int U = 4;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * 256 * U;
  for (int64_t i = (int64_t)blockIdx.x * 256 * U + threadIdx.x; i < n; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + (int64_t)u * 256;
      if constexpr (MODE == 1) v[u] = u32x4{(uint32_t)j, 0u, 0u, 0u};
      else v[u] = j < n ? ldg16_nt(src + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + (int64_t)u * 256;
      if constexpr (MODE == 0) acc ^= v[u];
      else if (j < n) {
        if constexpr (MODE == 3) stg16_nt(dst + j, v[u]);
        else stg16(dst + j, v[u]);
      }
    }
  }
  // mode 0: a store the loaded values decide, never taken for finite data patterns
  if (MODE == 0 && acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0xf39cc060u) dst[threadIdx.x & 0] = acc;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_ref_stream(const void* src, void* dst, int64_t bytes, int mode, void* stream) {
  if (bytes <= 0 || (bytes & 15) || mode < 0 || mode > 3) return MOE_EINVAL;
  if (!dst || (reinterpret_cast<uintptr_t>(dst) & 15)) return MOE_EINVAL;
  if (mode != 1 && (!src || (reinterpret_cast<uintptr_t>(src) & 15))) return MOE_EINVAL;
  const int64_t n = bytes / 16;
  int64_t g = (n + 1023) / 1024;
  if (g > 8192) g = 8192;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  switch (mode) {
    case 0: hipLaunchKernelGGL(stream_kernel<0>, dim3((int)g), dim3(256), 0, st, s, d, n); break;
    case 1: hipLaunchKernelGGL(stream_kernel<1>, dim3((int)g), dim3(256), 0, st, s, d, n); break;
    case 2: hipLaunchKernelGGL(stream_kernel<2>, dim3((int)g), dim3(256), 0, st, s, d, n); break;
    default: hipLaunchKernelGGL(stream_kernel<3>, dim3((int)g), dim3(256), 0, st, s, d, n); break;
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
