// Shared device helpers for the gfx950 MoE kernels (bf16 conversion, vector
// types, wave reductions).  Nothing here is specific to one kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

typedef uint16_t bf16_t;                                     // bf16 bit pattern
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));  // MFMA operand
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct alignas(16) u32x4 { uint32_t x, y, z, w; };
struct alignas(8) u32x2 { uint32_t x, y; };

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

MOE_DEV float bf16_to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even, one
// v_cvt_pk_bf16_f32 on gfx950.
MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> bf16, round to nearest even.
MOE_DEV bf16_t f32_to_bf16(float f) { return (bf16_t)(pack_bf16x2(f, 0.0f) & 0xffffu); }

MOE_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
MOE_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element access for the two storage types the library supports.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static MOE_DEV float load(const float* p, int64_t i) { return p[i]; }
  static MOE_DEV void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  static MOE_DEV float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static MOE_DEV void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// sigmoid and silu through the hardware exp and reciprocal (about 1 ulp each;
// every caller rounds the result to bf16 or accumulates it in fp32)
MOE_DEV float sigmoid_f(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
MOE_DEV float silu_f(float z) { return z * sigmoid_f(z); }

// Sum over the 64 lanes of a wavefront, identical result in every lane.
// The butterfly order is fixed, so the result is deterministic.
// fp8 formats of the quantised operands: OCP e4m3 (largest finite 448) and
// e5m2 (largest finite 57344)
enum { FP8_E4M3 = 0, FP8_E5M2 = 1 };
template <int FMT>
MOE_DEV constexpr float fp8_max() { return FMT == FP8_E5M2 ? 57344.0f : 448.0f; }

// Row-wise quantisation of 8 values with the row's scale s: each quotient
// f / s in IEEE fp32, clamped to the format's largest finite value (the
// conversions turn larger values into NaN or infinity), rounded to nearest
// even by v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32.
template <int FMT = FP8_E4M3>
MOE_DEV float fp8_row_scale(float amax) { return amax > 0.0f ? amax / fp8_max<FMT>() : 1.0f; }
template <int FMT = FP8_E4M3>
MOE_DEV u32x2 fp8_encode8(const float* f, float s) {
  constexpr float M = fp8_max<FMT>();
  float v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = fminf(fmaxf(f[u] / s, -M), M);
  u32x2 o;
  if constexpr (FMT == FP8_E5M2) {
    o.x = __builtin_amdgcn_cvt_pk_bf8_f32(v[0], v[1], 0, false);
    o.x = __builtin_amdgcn_cvt_pk_bf8_f32(v[2], v[3], o.x, true);
    o.y = __builtin_amdgcn_cvt_pk_bf8_f32(v[4], v[5], 0, false);
    o.y = __builtin_amdgcn_cvt_pk_bf8_f32(v[6], v[7], o.y, true);
  } else {
    o.x = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    o.x = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], o.x, true);
    o.y = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
    o.y = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], o.y, true);
  }
  return o;
}

MOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

MOE_DEV int ceil_div(int a, int b) { return (a + b - 1) / b; }

// First row of group g of a grouped product: offsets[g], or with no offset
// table (offsets == NULL, one group) 0 for g = 0 and M (all rows) for g = 1.
MOE_DEV int group_row(const int32_t* offsets, int g, int64_t M) {
  return offsets ? offsets[g] : (g == 0 ? 0 : (int)M);
}

// Number of blocks of `b` covering `a` (host and device).
__host__ __device__ inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Block-wide exclusive prefix sum over 256 threads (4 wavefronts).  Every
// thread must call it.  Returns the exclusive prefix of `v`; *total receives
// the sum of all 256 inputs.  `scratch` is 4 ints of LDS.
MOE_DEV int block_exclusive_scan256(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int s = scratch[w];
    if (w < wave) wbase += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}
