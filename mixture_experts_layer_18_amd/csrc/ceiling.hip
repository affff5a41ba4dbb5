// The matrix cores' sustained rate with no memory traffic: every wave runs
// rounds of eight independent MFMAs on register operands holding finite
// pseudo-random data (data that toggles draws the power a real product
// draws).  A measurement aid: the compute counterpart of a device-to-device
// copy as the practical HBM ceiling.
#include "kernels.h"

namespace moe {
namespace {

typedef float f32x4c_t __attribute__((ext_vector_type(4)));
typedef int v8ic_t __attribute__((ext_vector_type(8)));

MOE_DEV uint32_t lcg_next(uint32_t& s) {
  s = s * 1664525u + 1013904223u;
  return s;
}

// KIND: 0 bf16 32x32x16, 1 bf16 16x16x32, 2 e4m3 32x32x64, 3 e4m3 16x16x128
template <int KIND>
__global__ __launch_bounds__(512) void mfma_rate_kernel(int64_t iters, float* out) {
  uint32_t s = threadIdx.x * 7919u + blockIdx.x * 104729u + 1u;
  v8ic_t a[2], b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t r = lcg_next(s), q = lcg_next(s);
      if (KIND >= 2) {  // e4m3 bytes with exponent field <= 14: finite
        r &= 0x77777777u;
        q &= 0x77777777u;
      } else {          // bf16 pairs in [1, 2) with random sign and mantissa
        r = (r & 0x807f807fu) | 0x3f803f80u;
        q = (q & 0x807f807fu) | 0x3f803f80u;
      }
      a[i][j] = (int)r;
      b[i][j] = (int)q;
    }
  float total = 0.0f;
  if constexpr (KIND == 0 || KIND == 2) {
    f32x16_t acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[u][v] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if constexpr (KIND == 0) {
          const bf16x8_t aa = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a[u & 1], a[u & 1], 0, 1, 2, 3));
          const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(b[(u >> 1) & 1], b[(u >> 1) & 1], 0, 1, 2, 3));
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aa, bb, acc[u], 0, 0, 0);
        } else {
          acc[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[u & 1], b[(u >> 1) & 1], acc[u], 0, 0, 0, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) total += acc[u][v];
  } else {
    f32x4c_t acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if constexpr (KIND == 1) {
          const bf16x8_t aa = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a[u & 1], a[u & 1], 0, 1, 2, 3));
          const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(b[(u >> 1) & 1], b[(u >> 1) & 1], 0, 1, 2, 3));
          acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aa, bb, acc[u], 0, 0, 0);
        } else {
          acc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[u & 1], b[(u >> 1) & 1], acc[u], 0, 0, 0, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) total += acc[u][v];
  }
  // one write per launch keeps the products live
  if (blockIdx.x == 0 && threadIdx.x == 0) out[0] = total;
}

}  // namespace

int mfma_rate_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return 2 * cus;
}

hipError_t launch_mfma_rate(int kind, int64_t iters, float* out, hipStream_t st) {
  const dim3 grid((unsigned)mfma_rate_grid()), block(512);
  switch (kind) {
    case 0: mfma_rate_kernel<0><<<grid, block, 0, st>>>(iters, out); break;
    case 1: mfma_rate_kernel<1><<<grid, block, 0, st>>>(iters, out); break;
    case 2: mfma_rate_kernel<2><<<grid, block, 0, st>>>(iters, out); break;
    case 3: mfma_rate_kernel<3><<<grid, block, 0, st>>>(iters, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Streaming copy: one 16-byte vector per thread, nontemporal load and
// store, n vectors (the practical HBM ceiling the streaming kernels of the
// layer are rated against).
namespace {
typedef uint32_t cp_u4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_copy_kernel(const cp_u4* __restrict__ src, cp_u4* __restrict__ dst,
                                                          int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}
}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, int64_t n16, hipStream_t st) {
  if (n16 <= 0) return hipSuccess;
  stream_copy_kernel<<<dim3((unsigned)cdiv64(n16, 256)), dim3(256), 0, st>>>((const cp_u4*)src, (cp_u4*)dst, n16);
  return hipGetLastError();
}

}  // namespace moe
