// Row-wise fp8 (OCP e4m3) quantisation for the fp8 expert GEMMs (gfx950).
//
// Apex-3 code page ("What's inside": FP8 through torchao; "Run it yourself":
// --precision fp8_rowwise); KempnerForge README ("MoE roadmap": FP8 mixed
// precision).  Each row r of x is scaled by s_r = amax_r / 448 (fp32; 1 for
// an all-zero row) and every element becomes e4m3(x / s_r): the division in
// fp32, then round-to-nearest-even onto the e4m3 grid by v_cvt_pk_fp8_f32
// (which turns values beyond 464 into NaN, so the quotient is first clamped
// to +-448).  One wavefront per row; 16-byte loads, 8-byte stores.
#include "kernels.h"

namespace moe {

template <typename TX>
__global__ __launch_bounds__(256) void quantize_rowwise_kernel(const TX* __restrict__ x, int64_t R,
                                                               int C, uint8_t* __restrict__ q,
                                                               float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const TX* row = x + r * C;
  constexpr int V = 8;  // elements per 16-byte load (bf16) / two loads (fp32)
  float amax = 0.0f;
  for (int c = lane * V; c < C; c += 64 * V) {
    float f[V];
    if constexpr (sizeof(TX) == 2) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(row + c);
      f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
      f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    } else {
      const float4 a = reinterpret_cast<const float4*>(row + c)[0];
      const float4 b = reinterpret_cast<const float4*>(row + c)[1];
      f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
#pragma unroll
    for (int u = 0; u < V; ++u) amax = fmaxf(amax, fabsf(f[u]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (lane == 0) scale[r] = s;
  uint8_t* qrow = q + r * C;
  for (int c = lane * V; c < C; c += 64 * V) {
    float f[V];
    if constexpr (sizeof(TX) == 2) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(row + c);
      f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
      f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    } else {
      const float4 a = reinterpret_cast<const float4*>(row + c)[0];
      const float4 b = reinterpret_cast<const float4*>(row + c)[1];
      f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
#pragma unroll
    for (int u = 0; u < V; ++u) f[u] = fminf(fmaxf(f[u] / s, -448.0f), 448.0f);
    u32x2 o;
    o.x = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    o.x = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], o.x, true);
    o.y = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
    o.y = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], o.y, true);
    *reinterpret_cast<u32x2*>(qrow + c) = o;
  }
}

hipError_t launch_quantize_fp8(const void* x, int dtype, int64_t R, int C, uint8_t* q, float* scale,
                               hipStream_t st) {
  if (R == 0) return hipSuccess;
  const dim3 grid((unsigned)cdiv64(R, 4));
  if (dtype == MOE_BF16)
    quantize_rowwise_kernel<bf16_t><<<grid, 256, 0, st>>>((const bf16_t*)x, R, C, q, scale);
  else
    quantize_rowwise_kernel<float><<<grid, 256, 0, st>>>((const float*)x, R, C, q, scale);
  return hipGetLastError();
}

}  // namespace moe
