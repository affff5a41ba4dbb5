// Grouped GEMM kernels for the expert FFNs (gfx950).
//
// The experts run as grouped GEMMs (Apex-3 code page, "What's inside", row
// "Fine-grained MoE"; Ultimate MoE Training Handbook, section 2.5, grouped
// GEMM over the local experts).  Each expert is a SwiGLU block without bias
// (Handbook 2.5, parameter accounting): the gate/up product is fused with the
// SwiGLU activation, and the data-gradient of the down product is fused with
// the SwiGLU derivative.
//
// The dispatcher below picks the kernel of each product:
//  * bf16 operands: the persistent 256 x 256 matrix-core kernel
//    (gemm_big.hip) where it takes the product, else the two-workgroup
//    matrix-core kernel (gemm_mfma.hip: the weight gradients with few output
//    tiles, as row slices);
//  * fp32 operands: 64x64x16 FMA tiles (here).
//
// Rows of a group form a ragged M dimension: M-tiles are enumerated group
// after group from the device-side offsets, so nothing is copied to the host
// and empty groups cost nothing (weight gradients of empty groups are zero).
#include "kernels.h"

namespace moe {

struct KArgs {
  int G;
  int nsplit;
  int64_t M_total, N, K;
  const int32_t* offsets;
  const void* A;
  const void* B;
  void* C;
  void* aux;
  float* part;  // split partial sums [nsplit][G][N][K] (TN only)
};

struct RowTile {
  int g, m_lo, m_hi;
  bool valid;
};

// Tile tm of the concatenation of every group's ceil(rows/BMt) row tiles.
// Block-wide (all 256 threads call it); G <= 256.
template <int BMt>
MOE_DEV RowTile find_row_tile(const int32_t* __restrict__ offsets, int G, int64_t M, int tm, int* s_pref,
                              int* scratch) {
  const int tid = threadIdx.x;
  int n = 0;
  if (tid < G) n = (group_row(offsets, tid + 1, M) - group_row(offsets, tid, M) + BMt - 1) / BMt;
  int tot;
  const int ex = block_exclusive_scan256(n, scratch, &tot);
  if (tid < G) s_pref[tid] = ex;
  __syncthreads();
  RowTile r;
  r.valid = tm < tot;
  r.g = 0;
  r.m_lo = r.m_hi = 0;
  if (!r.valid) return r;
  int lo = 0, hi = G;  // last g with s_pref[g] <= tm (never an empty group)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= tm)
      lo = mid;
    else
      hi = mid;
  }
  r.g = lo;
  r.m_lo = group_row(offsets, lo, M) + (tm - s_pref[lo]) * BMt;
  r.m_hi = min(r.m_lo + BMt, group_row(offsets, lo + 1, M));
  return r;
}

// Rows [lo, hi) of a group's reduction range assigned to split s of n.
MOE_DEV void split_range(int lo, int hi, int s, int n, int quantum, int* a, int* b) {
  const int len = hi - lo;
  int chunk = (len + n - 1) / n;
  chunk = (chunk + quantum - 1) / quantum * quantum;
  *a = min(hi, lo + s * chunk);
  *b = min(hi, *a + chunk);
}

// ============================================================================ fp32 / mixed FMA path
namespace simt {
constexpr int BM = 64, BN = 64, BR = 16;

template <int LAYOUT, int EPI, typename TA, typename TB, typename TC>
__global__ __launch_bounds__(256) void gemm_kernel(KArgs a) {
  __shared__ float sP[BR][BM + 4];
  __shared__ float sQ[BR][BN + 4];
  __shared__ float sQ2[EPI == MOE_EPI_SWIGLU ? BR : 1][BN + 4];
  __shared__ int s_pref[256];
  __shared__ int scratch[4];
  const int tid = threadIdx.x;
  const TA* A = (const TA*)a.A;
  const TB* B = (const TB*)a.B;
  const int64_t N = a.N, K = a.K;

  int g, split = 0;
  int64_t i_lo, i_hi, j0 = (int64_t)blockIdx.x * BN, r_lo, r_hi, ncols;
  if (LAYOUT == MOE_GEMM_TN) {
    g = blockIdx.z / a.nsplit;
    split = blockIdx.z % a.nsplit;
    int rl, rh;
    split_range(group_row(a.offsets, g, a.M_total), group_row(a.offsets, g + 1, a.M_total), split, a.nsplit, BR, &rl, &rh);
    r_lo = rl;
    r_hi = rh;
    i_lo = (int64_t)blockIdx.y * BM;
    i_hi = min(i_lo + BM, N);
    ncols = K;
  } else {
    const RowTile rt = find_row_tile<BM>(a.offsets, a.G, a.M_total, blockIdx.y, s_pref, scratch);
    if (!rt.valid) return;
    g = rt.g;
    i_lo = rt.m_lo;
    i_hi = rt.m_hi;
    r_lo = 0;
    r_hi = (LAYOUT == MOE_GEMM_NT) ? K : N;
    ncols = (LAYOUT == MOE_GEMM_NT) ? (EPI == MOE_EPI_SWIGLU ? N / 2 : N) : K;
  }
  if (j0 >= ncols) return;
  const int64_t F = N / 2;

  const int tx = tid % 16, ty = tid / 16;
  float acc[4][4] = {};
  float acc2[4][4] = {};

  for (int64_t r0 = r_lo; r0 < r_hi; r0 += BR) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + q * 256;
      int ii, rr;
      if (LAYOUT == MOE_GEMM_TN) {
        ii = e % BM;
        rr = e / BM;
      } else {
        ii = e / BR;
        rr = e % BR;
      }
      const int64_t i = i_lo + ii, r = r0 + rr;
      float v = 0.0f;
      if (i < i_hi && r < r_hi) {
        if (LAYOUT == MOE_GEMM_NT) v = Elem<TA>::load(A, i * K + r);
        else if (LAYOUT == MOE_GEMM_NN) v = Elem<TA>::load(A, i * N + r);
        else v = Elem<TA>::load(A, r * N + i);
      }
      sP[rr][ii] = v;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + q * 256;
      int jj, rr;
      if (LAYOUT == MOE_GEMM_NT) {
        jj = e / BR;
        rr = e % BR;
      } else {
        jj = e % BN;
        rr = e / BN;
      }
      const int64_t j = j0 + jj, r = r0 + rr;
      float v = 0.0f, v2 = 0.0f;
      if (j < ncols && r < r_hi) {
        if (LAYOUT == MOE_GEMM_NT) {
          const int64_t base = (int64_t)g * N * K;
          v = Elem<TB>::load(B, base + j * K + r);
          if (EPI == MOE_EPI_SWIGLU) v2 = Elem<TB>::load(B, base + (F + j) * K + r);
        } else if (LAYOUT == MOE_GEMM_NN) {
          v = Elem<TB>::load(B, (int64_t)g * N * K + r * K + j);
        } else {
          v = Elem<TB>::load(B, r * K + j);
        }
      }
      sQ[rr][jj] = v;
      if (EPI == MOE_EPI_SWIGLU) sQ2[rr][jj] = v2;
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < BR; ++rr) {
      float p[4], q[4], q2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        p[u] = sP[rr][ty * 4 + u];
        q[u] = sQ[rr][tx * 4 + u];
        if (EPI == MOE_EPI_SWIGLU) q2[u] = sQ2[rr][tx * 4 + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc[u][w] = fmaf(p[u], q[w], acc[u][w]);
          if (EPI == MOE_EPI_SWIGLU) acc2[u][w] = fmaf(p[u], q2[w], acc2[u][w]);
        }
    }
    __syncthreads();
  }

  TC* C = (TC*)a.C;
  TC* X = (TC*)a.aux;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = i_lo + ty * 4 + u;
    if (i >= i_hi) continue;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int64_t j = j0 + tx * 4 + w;
      if (j >= ncols) continue;
      const float v = acc[u][w];
      if (LAYOUT == MOE_GEMM_TN) {
        if (a.nsplit > 1)
          a.part[(((int64_t)split * a.G + g) * N + i) * K + j] = v;
        else
          Elem<TC>::store(C, ((int64_t)g * N + i) * K + j, v);
      } else if (EPI == MOE_EPI_SWIGLU) {
        const float u2 = acc2[u][w];
        Elem<TC>::store(C, i * F + j, silu_f(v) * u2);
        if (X) {
          Elem<TC>::store(X, i * N + j, v);
          Elem<TC>::store(X, i * N + F + j, u2);
        }
      } else if (EPI == MOE_EPI_DSWIGLU) {
        const float G = Elem<TC>::load(X, i * 2 * K + j);
        const float U = Elem<TC>::load(X, i * 2 * K + K + j);
        const float sg = sigmoid_f(G);
        Elem<TC>::store(C, i * 2 * K + j, v * U * sg * (1.0f + G * (1.0f - sg)));
        Elem<TC>::store(C, i * 2 * K + K + j, v * G * sg);
      } else {
        Elem<TC>::store(C, i * ncols + j, v);
      }
    }
  }
}
}  // namespace simt

// Sum of split partials in split order, rounded once to TC.
template <typename TC>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part,
                                                           int nsplit, int64_t n,
                                                           TC* __restrict__ C) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int p = 0; p < nsplit; ++p) s += part[(int64_t)p * n + i];
  Elem<TC>::store(C, i, s);
}

// ============================================================================ dispatch
static int simt_splits(const GemmProblem& p) {
  // fp32 weight gradients reduce over all rows of a group: split long
  // reductions so that enough workgroups run; partials are summed in a fixed
  // order afterwards.
  if (p.layout != MOE_GEMM_TN) return 1;
  const int64_t tiles = p.G * cdiv64(p.N, simt::BM) * cdiv64(p.K, simt::BN);
  const int64_t rows_per_group = cdiv64(p.M_total, p.G);
  int s = 1;
  while (tiles * s < 1024 && rows_per_group / (s * 2) >= 256 && s < 64) s *= 2;
  return s;
}

static bool use_mfma(const GemmProblem& p) {
  return p.ta == MOE_BF16 && p.tb == MOE_BF16 && p.tc == MOE_BF16;
}

size_t gemm_workspace_bytes(const GemmProblem& p) {
  if (use_mfma(p)) return gemm_big_supported(p) ? gemm_big_workspace_bytes(p) : gemm_mfma_workspace_bytes(p);
  const int s = simt_splits(p);
  if (s <= 1) return 0;
  return (size_t)s * p.G * p.N * p.K * sizeof(float);
}

// Same sum, four consecutive elements per thread (n a multiple of 4).
template <typename TC>
__global__ __launch_bounds__(256) void split_reduce4_kernel(const float4* __restrict__ part,
                                                            int nsplit, int64_t n4,
                                                            TC* __restrict__ C) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p = 0; p < nsplit; ++p) {
    const float4 v = part[(int64_t)p * n4 + i];
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  Elem<TC>::store(C, 4 * i, s.x);
  Elem<TC>::store(C, 4 * i + 1, s.y);
  Elem<TC>::store(C, 4 * i + 2, s.z);
  Elem<TC>::store(C, 4 * i + 3, s.w);
}

hipError_t launch_split_reduce(const float* part, int nsplit, int64_t n, void* out, int dtype,
                               hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (n % 4) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  const dim3 grid((unsigned)cdiv64(n4, 256));
  if (dtype == MOE_BF16)
    split_reduce4_kernel<bf16_t><<<grid, dim3(256), 0, st>>>((const float4*)part, nsplit, n4, (bf16_t*)out);
  else
    split_reduce4_kernel<float><<<grid, dim3(256), 0, st>>>((const float4*)part, nsplit, n4, (float*)out);
  return hipGetLastError();
}

hipError_t launch_split_reduce_f32(const float* part, int nsplit, int64_t n, float* out,
                                  hipStream_t st) {
  if (n == 0) return hipSuccess;
  split_reduce_kernel<float><<<dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, st>>>(part, nsplit, n, out);
  return hipGetLastError();
}

template <int LAYOUT, int EPI, typename TA, typename TB, typename TC>
static hipError_t run_simt(const KArgs& ka, const GemmProblem& p, hipStream_t st) {
  dim3 grid;
  if (LAYOUT == MOE_GEMM_TN) {
    grid = dim3((unsigned)cdiv64(p.K, simt::BN), (unsigned)cdiv64(p.N, simt::BM),
                (unsigned)(p.G * ka.nsplit));
  } else {
    const int64_t ncols = (LAYOUT == MOE_GEMM_NT) ? (EPI == MOE_EPI_SWIGLU ? p.N / 2 : p.N) : p.K;
    grid = dim3((unsigned)cdiv64(ncols, simt::BN),
                (unsigned)(cdiv64(p.M_total, simt::BM) + p.G), 1);
  }
  simt::gemm_kernel<LAYOUT, EPI, TA, TB, TC><<<grid, dim3(256), 0, st>>>(ka);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (LAYOUT == MOE_GEMM_TN && ka.nsplit > 1) {
    const int64_t n = p.G * p.N * p.K;
    split_reduce_kernel<TC><<<dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, st>>>(
        ka.part, ka.nsplit, n, (TC*)p.C);
    e = hipGetLastError();
  }
  return e;
}

template <typename TA, typename TB, typename TC>
static hipError_t dispatch_simt(const KArgs& ka, const GemmProblem& p, hipStream_t st) {
  if (p.layout == MOE_GEMM_NT && p.epilogue == MOE_EPI_NONE)
    return run_simt<MOE_GEMM_NT, MOE_EPI_NONE, TA, TB, TC>(ka, p, st);
  if (p.layout == MOE_GEMM_NT && p.epilogue == MOE_EPI_SWIGLU)
    return run_simt<MOE_GEMM_NT, MOE_EPI_SWIGLU, TA, TB, TC>(ka, p, st);
  if (p.layout == MOE_GEMM_NN && p.epilogue == MOE_EPI_NONE)
    return run_simt<MOE_GEMM_NN, MOE_EPI_NONE, TA, TB, TC>(ka, p, st);
  if (p.layout == MOE_GEMM_NN && p.epilogue == MOE_EPI_DSWIGLU)
    return run_simt<MOE_GEMM_NN, MOE_EPI_DSWIGLU, TA, TB, TC>(ka, p, st);
  if (p.layout == MOE_GEMM_TN && p.epilogue == MOE_EPI_NONE)
    return run_simt<MOE_GEMM_TN, MOE_EPI_NONE, TA, TB, TC>(ka, p, st);
  return hipErrorInvalidValue;
}

hipError_t launch_grouped_gemm(const GemmProblem& p, void* ws, size_t ws_bytes, hipStream_t st) {
  // gathered rows: the persistent kernel only
  if (p.rows && !gemm_big_supported(p)) return hipErrorInvalidValue;
  if (p.M_total == 0 && p.layout != MOE_GEMM_TN) return hipSuccess;
  KArgs ka;
  ka.G = (int)p.G;
  ka.M_total = p.M_total;
  ka.N = p.N;
  ka.K = p.K;
  ka.offsets = p.offsets;
  ka.A = p.A;
  ka.B = p.B;
  ka.C = p.C;
  ka.aux = p.aux;
  ka.part = (float*)ws;
  ka.nsplit = 1;
  if (use_mfma(p)) {
    if (gemm_big_supported(p)) return launch_gemm_big(p, ws, ws_bytes, st);
    return launch_gemm_mfma(p, ws, ws_bytes, st);
  }
  ka.nsplit = simt_splits(p);
  if (ka.nsplit > 1 && ws_bytes < gemm_workspace_bytes(p)) return hipErrorInvalidValue;
  // fp32 layers and the fp32 router products (A and/or B may be bf16 there)
  if (p.ta == MOE_F32 && p.tb == MOE_F32 && p.tc == MOE_F32) return dispatch_simt<float, float, float>(ka, p, st);
  if (p.ta == MOE_BF16 && p.tb == MOE_F32 && p.tc == MOE_F32) return dispatch_simt<bf16_t, float, float>(ka, p, st);
  if (p.ta == MOE_F32 && p.tb == MOE_BF16 && p.tc == MOE_F32) return dispatch_simt<float, bf16_t, float>(ka, p, st);
  return hipErrorInvalidValue;
}

}  // namespace moe
