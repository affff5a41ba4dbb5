// fp8 (OCP e4m3) quantisation for the fp8 expert GEMMs (gfx950).
//
// Apex-3 code page ("What's inside": FP8 through torchao; "Run it yourself":
// --precision fp8_rowwise, --fp8-recipe tensorwise); KempnerForge README
// ("MoE roadmap": FP8 mixed precision).
//
// Row-wise: each row r of x is scaled by s_r = amax_r / 448 (fp32; 1 for an
// all-zero row).  Tensor-wise: one s = amax / 448 over the whole tensor (1 if
// it is all zero), written to every row's scale so that the same scaled GEMM
// consumes either.  Every element becomes e4m3(x / s): the division in fp32,
// then round-to-nearest-even onto the e4m3 grid by v_cvt_pk_fp8_f32 (which
// turns values beyond 464 into NaN, so the quotient is first clamped to
// +-448).  One wavefront per row; 16-byte loads, 8-byte stores.  Maxima are
// exact, so every result is deterministic.
#include "kernels.h"

namespace moe {
namespace q8 {

constexpr int V = 8;  // elements per 16-byte load (bf16) / two loads (fp32)

template <typename TX>
MOE_DEV void load8(const TX* row, int c, float* f) {
  if constexpr (sizeof(TX) == 2) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + c);
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  } else {
    const float4 a = reinterpret_cast<const float4*>(row + c)[0];
    const float4 b = reinterpret_cast<const float4*>(row + c)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

// max |x| over one row, the same value in every lane of the wave
template <typename TX>
MOE_DEV float row_amax(const TX* row, int C, int lane) {
  float amax = 0.0f;
  for (int c = lane * V; c < C; c += 64 * V) {
    float f[V];
    load8(row, c, f);
#pragma unroll
    for (int u = 0; u < V; ++u) amax = fmaxf(amax, fabsf(f[u]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  return amax;
}

MOE_DEV float scale_of(float amax) { return fp8_row_scale(amax); }

// q = fmt(clamp(x / s)) for one row; the codes are stored nontemporally (on
// the 7B-style layer's fp8 step the quantiser launches took 84 against 87 us)
template <typename TX, int FMT = FP8_E4M3>
MOE_DEV void encode_row(const TX* row, int C, float s, uint8_t* qrow, int lane) {
  typedef uint32_t nt_u2 __attribute__((ext_vector_type(2)));
  for (int c = lane * V; c < C; c += 64 * V) {
    float f[V];
    load8(row, c, f);
    const u32x2 q = fp8_encode8<FMT>(f, s);
    __builtin_nontemporal_store(nt_u2{q.x, q.y}, reinterpret_cast<nt_u2*>(qrow + c));
  }
}

template <typename TX, int FMT>
__global__ __launch_bounds__(256) void rowwise_kernel(const TX* __restrict__ x, int64_t R, int C,
                                                      uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const float s = fp8_row_scale<FMT>(row_amax(x + r * C, C, lane));
  if (lane == 0) scale[r] = s;
  encode_row<TX, FMT>(x + r * C, C, s, q + r * C, lane);
}

// tensor-wise, pass 1: the maximum of each row
template <typename TX>
__global__ __launch_bounds__(256) void row_amax_kernel(const TX* __restrict__ x, int64_t R, int C,
                                                       float* __restrict__ amax) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const float m = row_amax(x + r * C, C, lane);
  if (lane == 0) amax[r] = m;
}

// pass 2: one workgroup takes the maximum over the rows and writes the scale
// after them
__global__ __launch_bounds__(256) void tensor_scale_kernel(float* __restrict__ amax, int64_t R) {
  __shared__ float sh[4];
  float m = 0.0f;
  for (int64_t r = threadIdx.x; r < R; r += 256) m = fmaxf(m, amax[r]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) amax[R] = scale_of(fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3])));
}

// pass 3: every row with the tensor's scale
template <typename TX>
__global__ __launch_bounds__(256) void with_scale_kernel(const TX* __restrict__ x, int64_t R, int C,
                                                         const float* __restrict__ s_ptr,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const float s = *s_ptr;
  if (lane == 0) scale[r] = s;
  encode_row(x + r * C, C, s, q + r * C, lane);
}

// ---- along the first axis, stored transposed: x [G, R, C] -> q [G, C, R],
// scale [G, C] = amax_r |x[g, r, c]| / 448 (the weight of a data-gradient
// product quantised along its reduction dimension, laid out for the forward
// product).  R and C are multiples of 64.

template <typename TX>
MOE_DEV void load4(const TX* p, float* f) {
  if constexpr (sizeof(TX) == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  } else {
    const float4 v = *reinterpret_cast<const float4*>(p);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
}

// pass 1: one workgroup per (64 columns, matrix g): thread t takes columns
// 8 * (t % 8) .. +7 of every 32nd row from row t / 8; the 32 partial maxima of
// each column are combined through LDS
template <typename TX>
__global__ __launch_bounds__(256) void col_scale_kernel(const TX* __restrict__ x, int64_t R, int64_t C,
                                                        float* __restrict__ scale) {
  __shared__ float part[32][65];
  const int t = threadIdx.x, cq = (t & 7) * 8, rp = t >> 3;
  const int64_t g = blockIdx.y, c0 = (int64_t)blockIdx.x * 64;
  const TX* base = x + g * R * C + c0 + cq;
  float m[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) m[u] = 0.0f;
  for (int64_t r = rp; r < R; r += 32) {
    float f[8];
    load4(base + r * C, f);
    load4(base + r * C + 4, f + 4);
#pragma unroll
    for (int u = 0; u < 8; ++u) m[u] = fmaxf(m[u], fabsf(f[u]));
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) part[rp][cq + u] = m[u];
  __syncthreads();
  if (t < 64) {
    float a = 0.0f;
#pragma unroll 8
    for (int i = 0; i < 32; ++i) a = fmaxf(a, part[i][t]);
    scale[g * C + c0 + t] = scale_of(a);
  }
}

// pass 2: one workgroup per 64 x 64 tile (rows r0.., columns c0.. of matrix
// g): thread t encodes rows 4 (t / 16) .. +3 of columns 4 (t % 16) .. +3,
// packs each column's 4 codes into one word of an LDS tile [column][row],
// and the tile leaves as 64-byte runs of each output row q[g, c, r0..]
template <typename TX>
__global__ __launch_bounds__(256) void encode_transposed_kernel(const TX* __restrict__ x, int64_t R,
                                                                int64_t C, const float* __restrict__ scale,
                                                                uint8_t* __restrict__ q) {
  constexpr int PITCH = 80;  // bytes per LDS column (64 codes + 16), 16-byte aligned
  __shared__ __attribute__((aligned(16))) uint8_t tile[64 * PITCH];
  const int t = threadIdx.x, rr = (t >> 4) * 4, cc = (t & 15) * 4;
  const int64_t g = blockIdx.z, r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  float s[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) s[u] = scale[g * C + c0 + cc + u];
  float f[4][4];  // [row][column]
#pragma unroll
  for (int i = 0; i < 4; ++i) load4(x + (g * R + r0 + rr + i) * C + c0 + cc, f[i]);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = fminf(fmaxf(f[i][u] / s[u], -448.0f), 448.0f);
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
    *reinterpret_cast<uint32_t*>(tile + (cc + u) * PITCH + rr) = w;
  }
  __syncthreads();
  const int oc = t >> 2, orr = (t & 3) * 16;
  const u32x4 v = *reinterpret_cast<const u32x4*>(tile + oc * PITCH + orr);
  *reinterpret_cast<u32x4*>(q + (g * C + c0 + oc) * R + r0 + orr) = v;
}

// ---- along the rows of each group of a row-major matrix, stored transposed
// and padded: the operands of an fp8 weight gradient, whose reduction runs
// over the rows of one group (one expert's tokens).  Group g owns rows
// [offsets[g], offsets[g+1]) of x [M, C] (a row map, when given, names the
// source row of each); its codes form the block q[C * P_g ...] of C rows of
// P'_g = pad64(rows of g) bytes (row c holds column c of the group, zero past
// its last row), P_g = sum of the earlier groups' P'; scale[g, c] =
// max |x[., c]| over the group's rows / 448.

// the padded group offsets P_g (G + 1 entries): one workgroup
__global__ __launch_bounds__(256) void pad_offsets_kernel(const int32_t* __restrict__ offsets, int G, int64_t M,
                                                          int32_t* __restrict__ pad_off) {
  __shared__ int part[4];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int v = 0;
  if (t < G) {
    const int lo = offsets ? offsets[t] : 0, hi = offsets ? offsets[t + 1] : (int)M;
    v = (hi - lo + 63) / 64 * 64;
  }
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) part[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += part[i];
  if (t < G) pad_off[t] = base + incl - v;
  if (t == 0) pad_off[G] = part[0] + part[1] + part[2] + part[3];
}

// pass 1: one workgroup per (64 columns, group): thread t takes columns
// 8 (t % 8) .. +7 of every 32nd row of the group from row t / 8
template <typename TX>
__global__ __launch_bounds__(256) void seg_col_scale_kernel(const TX* __restrict__ x, const int32_t* __restrict__ rows,
                                                            const int32_t* __restrict__ offsets, int64_t M,
                                                            int64_t C, float* __restrict__ scale) {
  __shared__ float part[32][65];
  const int t = threadIdx.x, cq = (t & 7) * 8, rp = t >> 3;
  const int g = blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int64_t lo = offsets ? offsets[g] : 0, hi = offsets ? offsets[g + 1] : M;
  float m[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) m[u] = 0.0f;
  for (int64_t r = lo + rp; r < hi; r += 32) {
    const int64_t src = rows ? (int64_t)rows[r] : r;
    float f[8];
    load4(x + src * C + c0 + cq, f);
    load4(x + src * C + c0 + cq + 4, f + 4);
#pragma unroll
    for (int u = 0; u < 8; ++u) m[u] = fmaxf(m[u], fabsf(f[u]));
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) part[rp][cq + u] = m[u];
  __syncthreads();
  if (t < 64) {
    float a = 0.0f;
#pragma unroll 8
    for (int i = 0; i < 32; ++i) a = fmaxf(a, part[i][t]);
    scale[(int64_t)g * C + c0 + t] = scale_of(a);
  }
}

// pass 2: one workgroup per 64 x 64 tile of the padded groups (blockIdx.y:
// the 64-row tile counted over all groups' padded rows; beyond the last, none)
template <typename TX>
__global__ __launch_bounds__(256) void seg_encode_transposed_kernel(
    const TX* __restrict__ x, const int32_t* __restrict__ rows, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ pad_off, int G, int64_t M, int64_t C, const float* __restrict__ scale,
    uint8_t* __restrict__ q) {
  constexpr int PITCH = 80;
  __shared__ __attribute__((aligned(16))) uint8_t tile[64 * PITCH];
  const int tm = blockIdx.y;
  if ((int64_t)tm * 64 >= pad_off[G]) return;
  int lo_g = 0, hi_g = G;  // the group whose padded rows hold tile tm
  while (hi_g - lo_g > 1) {
    const int mid = (lo_g + hi_g) >> 1;
    if (pad_off[mid] <= tm * 64) lo_g = mid; else hi_g = mid;
  }
  const int g = lo_g;
  const int64_t pg = pad_off[g + 1] - pad_off[g], r0 = (int64_t)tm * 64 - pad_off[g];
  const int64_t lo = offsets ? offsets[g] : 0, hi = offsets ? offsets[g + 1] : M;
  const int t = threadIdx.x, rr = (t >> 4) * 4, cc = (t & 15) * 4;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  float s[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) s[u] = scale[(int64_t)g * C + c0 + cc + u];
  float f[4][4];  // [row][column]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = lo + r0 + rr + i;
    if (r < hi) {
      const int64_t src = rows ? (int64_t)rows[r] : r;
      load4(x + src * C + c0 + cc, f[i]);
    } else {
      f[i][0] = f[i][1] = f[i][2] = f[i][3] = 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = fminf(fmaxf(f[i][u] / s[u], -448.0f), 448.0f);
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
    *reinterpret_cast<uint32_t*>(tile + (cc + u) * PITCH + rr) = w;
  }
  __syncthreads();
  const int oc = t >> 2, orr = (t & 3) * 16;
  const u32x4 v = *reinterpret_cast<const u32x4*>(tile + oc * PITCH + orr);
  *reinterpret_cast<u32x4*>(q + C * (int64_t)pad_off[g] + (c0 + oc) * pg + r0 + orr) = v;
}

}  // namespace q8

hipError_t launch_quantize_fp8_colwise(const void* x, int dtype, const int32_t* rows, const int32_t* offsets,
                                       int G, int64_t M, int64_t C, int32_t* pad_off, uint8_t* q, float* scale,
                                       hipStream_t st) {
  if (G < 1 || G > 256) return hipErrorInvalidValue;
  q8::pad_offsets_kernel<<<1, 256, 0, st>>>(offsets, G, M, pad_off);
  const dim3 g1((unsigned)(C / 64), (unsigned)G), g2((unsigned)(C / 64), (unsigned)(cdiv64(M, 64) + G));
  if (dtype == MOE_BF16) {
    q8::seg_col_scale_kernel<bf16_t><<<g1, 256, 0, st>>>((const bf16_t*)x, rows, offsets, M, C, scale);
    q8::seg_encode_transposed_kernel<bf16_t><<<g2, 256, 0, st>>>((const bf16_t*)x, rows, offsets, pad_off, G, M,
                                                                 C, scale, q);
  } else {
    q8::seg_col_scale_kernel<float><<<g1, 256, 0, st>>>((const float*)x, rows, offsets, M, C, scale);
    q8::seg_encode_transposed_kernel<float><<<g2, 256, 0, st>>>((const float*)x, rows, offsets, pad_off, G, M,
                                                                C, scale, q);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_fp8_transposed(const void* x, int dtype, int64_t G, int64_t R, int64_t C,
                                          uint8_t* q, float* scale, hipStream_t st) {
  if (G == 0 || R == 0) return hipSuccess;
  const dim3 g1((unsigned)(C / 64), (unsigned)G), g2((unsigned)(C / 64), (unsigned)(R / 64), (unsigned)G);
  if (dtype == MOE_BF16) {
    q8::col_scale_kernel<bf16_t><<<g1, 256, 0, st>>>((const bf16_t*)x, R, C, scale);
    q8::encode_transposed_kernel<bf16_t><<<g2, 256, 0, st>>>((const bf16_t*)x, R, C, scale, q);
  } else {
    q8::col_scale_kernel<float><<<g1, 256, 0, st>>>((const float*)x, R, C, scale);
    q8::encode_transposed_kernel<float><<<g2, 256, 0, st>>>((const float*)x, R, C, scale, q);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const void* x, int dtype, int64_t R, int C, uint8_t* q, float* scale,
                               hipStream_t st, int fmt) {
  if (R == 0) return hipSuccess;
  const dim3 grid((unsigned)cdiv64(R, 4));
  if (fmt == FP8_E5M2) {
    if (dtype == MOE_BF16)
      q8::rowwise_kernel<bf16_t, FP8_E5M2><<<grid, 256, 0, st>>>((const bf16_t*)x, R, C, q, scale);
    else
      q8::rowwise_kernel<float, FP8_E5M2><<<grid, 256, 0, st>>>((const float*)x, R, C, q, scale);
  } else {
    if (dtype == MOE_BF16)
      q8::rowwise_kernel<bf16_t, FP8_E4M3><<<grid, 256, 0, st>>>((const bf16_t*)x, R, C, q, scale);
    else
      q8::rowwise_kernel<float, FP8_E4M3><<<grid, 256, 0, st>>>((const float*)x, R, C, q, scale);
  }
  return hipGetLastError();
}

size_t quantize_fp8_tensorwise_ws_bytes(int64_t R) { return (size_t)(R + 1) * sizeof(float); }

hipError_t launch_quantize_fp8_tensorwise(const void* x, int dtype, int64_t R, int C, uint8_t* q,
                                          float* scale, float* ws, hipStream_t st) {
  if (R == 0) return hipSuccess;
  const dim3 grid((unsigned)cdiv64(R, 4));
  if (dtype == MOE_BF16)
    q8::row_amax_kernel<bf16_t><<<grid, 256, 0, st>>>((const bf16_t*)x, R, C, ws);
  else
    q8::row_amax_kernel<float><<<grid, 256, 0, st>>>((const float*)x, R, C, ws);
  q8::tensor_scale_kernel<<<1, 256, 0, st>>>(ws, R);
  if (dtype == MOE_BF16)
    q8::with_scale_kernel<bf16_t><<<grid, 256, 0, st>>>((const bf16_t*)x, R, C, ws + R, q, scale);
  else
    q8::with_scale_kernel<float><<<grid, 256, 0, st>>>((const float*)x, R, C, ws + R, q, scale);
  return hipGetLastError();
}

}  // namespace moe
