// Combine (unpermute + gate-weighted sum), its backward with the router
// gradient, and the unpermute-sum of the input gradient (gfx950).
//
// The combine returns each expert's output to its token and weights it by the
// gate (Ultimate MoE Training Handbook, section 2.5: the experts' outputs must
// be returned to where they are needed); shared experts are added ungated
// (KempnerForge README, "Features / Architecture").  The router only receives
// gradient through the gate values, never through the selection, and the
// selection bias receives none (Apex-3 code page, "Fine-grained MoE"; the
// Handbook's single-expert check in 2.5, where the router gets zero gradient).
//
// All three kernels are HBM-bound row gathers: one wavefront per token, rows
// moved as 16-byte vectors, fp32 accumulation in a fixed order, one rounding.
// The rows each kernel streams once are read with nontemporal loads, and the
// layer's outputs y and dx written with nontemporal stores; the router weight
// rows, which every token re-reads, and dY~ (dy_perm), which the down data
// gradient reads next, move with ordinary ones.  Measured on the 7B-style
// layer: combine 117 -> 93 us, unpermute-sum 122 -> 113 us, combine backward
// 168 -> 155 us (178 us with nontemporal dY~ stores).
#include "kernels.h"

namespace moe {

typedef uint32_t nt_u4 __attribute__((ext_vector_type(4)));
MOE_DEV u32x4 nt_load16(const void* p) {
  return __builtin_bit_cast(u32x4, __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(p)));
}
MOE_DEV void nt_store16(void* p, const u32x4& v) {
  __builtin_nontemporal_store(__builtin_bit_cast(nt_u4, v), reinterpret_cast<nt_u4*>(p));
}

// 16-byte vector <-> floats for both storage types
template <typename T> struct Vec;
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  typedef u32x4 raw_t;
  static MOE_DEV raw_t load_raw(const bf16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
  static MOE_DEV raw_t load_nt(const bf16_t* p) { return nt_load16(p); }
  static MOE_DEV void unpack(const raw_t& v, float* f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
  static MOE_DEV void load(const bf16_t* p, float* f) { unpack(load_raw(p), f); }
  static MOE_DEV u32x4 pack(const float* f) {
    u32x4 v;
    v.x = pack_bf16x2(f[0], f[1]); v.y = pack_bf16x2(f[2], f[3]);
    v.z = pack_bf16x2(f[4], f[5]); v.w = pack_bf16x2(f[6], f[7]);
    return v;
  }
  static MOE_DEV void store(bf16_t* p, const float* f) { *reinterpret_cast<u32x4*>(p) = pack(f); }
  static MOE_DEV void store_nt(bf16_t* p, const float* f) { nt_store16(p, pack(f)); }
  static MOE_DEV void load_f_nt(const bf16_t* p, float* f) { unpack(load_nt(p), f); }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  typedef float4 raw_t;
  static MOE_DEV raw_t load_raw(const float* p) { return *reinterpret_cast<const float4*>(p); }
  static MOE_DEV raw_t load_nt(const float* p) { return __builtin_bit_cast(float4, nt_load16(p)); }
  static MOE_DEV void unpack(const raw_t& v, float* f) {
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
  static MOE_DEV void load(const float* p, float* f) { unpack(load_raw(p), f); }
  static MOE_DEV void store(float* p, const float* f) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
  static MOE_DEV void store_nt(float* p, const float* f) {
    nt_store16(p, __builtin_bit_cast(u32x4, make_float4(f[0], f[1], f[2], f[3])));
  }
  static MOE_DEV void load_f_nt(const float* p, float* f) { unpack(load_nt(p), f); }
};

// 16-byte chunks per lane whose loads the combine backward issues together
// (64 lanes x CG chunks of a row per group)
constexpr int CG = 4;

// y[t] = sum_j gate[t,j] * y_perm[pos[t*k+j]] (+ shared_y[t]), fp32, one rounding.
// One wavefront per token.  KK > 0 fixes the number of slots at compile time,
// so the KK row loads of a chunk (and of two chunks per step) are all in flight
// before any is consumed; KK == 0 is the generic runtime-k loop.
template <typename T, int KK>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y_perm,
                                                      const float* __restrict__ gate,
                                                      const int32_t* __restrict__ pos,
                                                      const T* shared_y, T* y, int Tn, int d,
                                                      int k) {
  constexpr int VN = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int nvec = d / VN;
  const int64_t tk = (int64_t)t * k;
  if constexpr (KK > 0) {
    int64_t row[KK];
    float g[KK];
#pragma unroll
    for (int j = 0; j < KK; ++j) {
      row[j] = (int64_t)pos[tk + j] * d;
      g[j] = gate[tk + j];
    }
#pragma unroll 2
    for (int c = lane; c < nvec; c += 64) {
      float v[KK][VN];
#pragma unroll
      for (int j = 0; j < KK; ++j) Vec<T>::load_f_nt(y_perm + row[j] + (int64_t)c * VN, v[j]);
      float sh[VN];
      if (shared_y) Vec<T>::load_f_nt(shared_y + (int64_t)t * d + (int64_t)c * VN, sh);
      float acc[VN];
#pragma unroll
      for (int u = 0; u < VN; ++u) acc[u] = 0.0f;
#pragma unroll
      for (int j = 0; j < KK; ++j)
#pragma unroll
        for (int u = 0; u < VN; ++u) acc[u] = fmaf(g[j], v[j][u], acc[u]);
      if (shared_y) {
#pragma unroll
        for (int u = 0; u < VN; ++u) acc[u] += sh[u];
      }
      Vec<T>::store_nt(y + (int64_t)t * d + (int64_t)c * VN, acc);
    }
  } else {
    for (int c = lane; c < nvec; c += 64) {
      float acc[VN];
#pragma unroll
      for (int u = 0; u < VN; ++u) acc[u] = 0.0f;
      for (int j = 0; j < k; ++j) {
        const float g = gate[tk + j];
        const int64_t p = pos[tk + j];
        float v[VN];
        Vec<T>::load_f_nt(y_perm + p * d + (int64_t)c * VN, v);
#pragma unroll
        for (int u = 0; u < VN; ++u) acc[u] = fmaf(g, v[u], acc[u]);
      }
      if (shared_y) {
        float v[VN];
        Vec<T>::load_f_nt(shared_y + (int64_t)t * d + (int64_t)c * VN, v);
#pragma unroll
        for (int u = 0; u < VN; ++u) acc[u] += v[u];
      }
      Vec<T>::store_nt(y + (int64_t)t * d + (int64_t)c * VN, acc);
    }
  }
}

MOE_DEV float sigmoid_rounded_f(float l) { return (float)(1.0 / (1.0 + exp(-(double)l))); }

// The e4m3 copies the fp8 backward quantises, written by the combine
// backward from the rows it forms: the row-wise codes and scales of the
// gate-weighted rows dy_perm (as rounded to bf16) and of dy itself.
struct Fp8Rows {
  uint8_t* q_perm;  // [A, d]
  float* s_perm;    // [A]
  uint8_t* q_dy;    // [T, d]
  float* s_dy;      // [T]
};

// max |x| over one bf16 row of d elements (exact), in every lane of the wave
MOE_DEV float bf16_row_amax(const bf16_t* row, int nvec, int lane) {
  float amax = 0.0f;
  for (int c = lane; c < nvec; c += 64) {
    float f[8];
    Vec<bf16_t>::load(row + (int64_t)c * 8, f);
#pragma unroll
    for (int u = 0; u < 8; ++u) amax = fmaxf(amax, fabsf(f[u]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  return amax;
}

// The bf16 value a stored fp32 result takes (round to nearest even)
MOE_DEV float bf16_round(float v) { return bf16_lo(pack_bf16x2(v, 0.0f)); }

// Combine backward and router backward for one token per wavefront:
//   dy_perm[pos[t,j]] = gate[t,j] * dy[t]
//   dgate[t,j]        = <dy[t], y_perm[pos[t,j]]>          (fp32)
//   dlogits[t,:]      from dgate through the gate function (selection fixed)
// The row data is streamed chunk by chunk; with KK > 0 the KK slot rows of a
// chunk are loaded together and the per-slot dot products kept in registers.
// Q8 (bf16, KK > 0): also the e4m3 copies of Fp8Rows.  A gate-weighted row's
// largest magnitude is bf16(gate * max|dy[t]|) exactly (rounding is monotone
// and symmetric), so a first pass over dy[t] gives every slot's scale before
// the rows are formed.
template <typename T, int KK, bool Q8 = false, int QF = FP8_E4M3>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const T* __restrict__ dy, const T* __restrict__ y_perm, const float* __restrict__ gate,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ idx,
    const float* __restrict__ logits, int score, int renorm, int Tn, int d, int E, int k,
    T* __restrict__ dy_perm, float* __restrict__ dlogits, Fp8Rows q8 = {}) {
  static_assert(!Q8 || (KK > 0 && sizeof(T) == 2), "fp8 copies: bf16 rows, compile-time slots");
  constexpr int VN = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int nvec = d / VN;
  const int64_t tk = (int64_t)t * k;
  float my_dg = 0.0f;  // lane j keeps dgate[t, j]
  if constexpr (KK > 0) {
    int64_t row[KK];
    float g[KK], dot[KK];
    float sq[KK > 0 ? KK : 1], s_dy = 1.0f;
#pragma unroll
    for (int j = 0; j < KK; ++j) {
      row[j] = (int64_t)pos[tk + j] * d;
      g[j] = gate[tk + j];
      dot[j] = 0.0f;
    }
    if constexpr (Q8) {
      const float amax = bf16_row_amax((const bf16_t*)dy + (int64_t)t * d, nvec, lane);
      s_dy = fp8_row_scale<QF>(amax);
#pragma unroll
      for (int j = 0; j < KK; ++j) sq[j] = fp8_row_scale<QF>(bf16_round(g[j] * amax));
      if (lane == 0) {
        q8.s_dy[t] = s_dy;
#pragma unroll
        for (int j = 0; j < KK; ++j) q8.s_perm[pos[tk + j]] = sq[j];
      }
    }
    // groups of CG chunks: every load of a group is issued before any of its
    // stores, so the loads are in flight together (a load issued after a
    // pending store is waited for together with that store)
    for (int c0 = lane; c0 < nvec; c0 += 64 * CG) {
      typename Vec<T>::raw_t dr[CG], vr[CG][KK];
#pragma unroll
      for (int i = 0; i < CG; ++i) {
        const int c = c0 + 64 * i;
        if (c < nvec) {
          dr[i] = Vec<T>::load_nt(dy + (int64_t)t * d + (int64_t)c * VN);
#pragma unroll
          for (int j = 0; j < KK; ++j) vr[i][j] = Vec<T>::load_nt(y_perm + row[j] + (int64_t)c * VN);
        }
      }
#pragma unroll
      for (int i = 0; i < CG; ++i) {
        const int c = c0 + 64 * i;
        if (c < nvec) {
          float dv[VN];
          Vec<T>::unpack(dr[i], dv);
          if constexpr (Q8)
            *reinterpret_cast<u32x2*>(q8.q_dy + (int64_t)t * d + (int64_t)c * VN) = fp8_encode8<QF>(dv, s_dy);
#pragma unroll
          for (int j = 0; j < KK; ++j) {
            float v[VN], o[VN];
            Vec<T>::unpack(vr[i][j], v);
#pragma unroll
            for (int u = 0; u < VN; ++u) {
              dot[j] = fmaf(dv[u], v[u], dot[j]);
              o[u] = g[j] * dv[u];
            }
            Vec<T>::store(dy_perm + row[j] + (int64_t)c * VN, o);
            if constexpr (Q8) {
              float b[VN];
#pragma unroll
              for (int u = 0; u < VN; ++u) b[u] = bf16_round(o[u]);
              *reinterpret_cast<u32x2*>(q8.q_perm + row[j] + (int64_t)c * VN) = fp8_encode8<QF>(b, sq[j]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KK; ++j) {
      const float s = wave_sum(dot[j]);
      if (lane == j) my_dg = s;
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const float g = gate[tk + j];
      const int64_t p = pos[tk + j];
      float dot = 0.0f;
      for (int c = lane; c < nvec; c += 64) {
        float dv[VN], v[VN], o[VN];
        Vec<T>::load_f_nt(dy + (int64_t)t * d + (int64_t)c * VN, dv);
        Vec<T>::load_f_nt(y_perm + p * d + (int64_t)c * VN, v);
#pragma unroll
        for (int u = 0; u < VN; ++u) {
          dot = fmaf(dv[u], v[u], dot);
          o[u] = g * dv[u];
        }
        Vec<T>::store_nt(dy_perm + p * d + (int64_t)c * VN, o);
      }
      dot = wave_sum(dot);
      if (lane == j) my_dg = dot;
    }
  }

  // ---- router backward
  const float* lrow = logits + (int64_t)t * E;
  float* drow = dlogits + (int64_t)t * E;
  const int my_e = (lane < k) ? idx[(int64_t)t * k + lane] : -1;
  if (score == MOE_SIGMOID || renorm) {
    // picked scores (sigmoid) or probabilities (softmax, renormalised)
    double sv = 0.0;
    if (score == MOE_SIGMOID) {
      if (lane < k) sv = (double)sigmoid_rounded_f(lrow[my_e]);
    } else {
      float m = -INFINITY;
      for (int e = lane; e < E; e += 64) m = fmaxf(m, lrow[e]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      double zs = 0.0;
      for (int e = lane; e < E; e += 64) zs += exp((double)lrow[e] - (double)m);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) zs += __shfl_xor(zs, o, 64);
      if (lane < k) sv = (double)(float)(exp((double)lrow[my_e] - (double)m) / zs);
    }
    double S = sv;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) S += __shfl_xor(S, o, 64);
    const double gj = (lane < k) ? sv / S : 0.0;
    double gdg = gj * (double)my_dg;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) gdg += __shfl_xor(gdg, o, 64);
    double dl = 0.0;
    if (lane < k) {
      if (score == MOE_SIGMOID) {
        const double ds = ((double)my_dg - gdg) / S;
        dl = ds * sv * (1.0 - sv);
      } else {
        dl = gj * ((double)my_dg - gdg);
      }
    }
    const float dlf = (float)dl;
    for (int e = lane; e < E; e += 64) {
      float v = 0.0f;
      for (int j = 0; j < k; ++j) {
        const int ej = __shfl(my_e, j, 64);
        const float dj = __shfl(dlf, j, 64);
        if (ej == e) v = dj;
      }
      drow[e] = v;
    }
  } else {
    // softmax without renormalisation: dl = p * (dp - <p, dp>), dp = dgate on picked
    float m = -INFINITY;
    for (int e = lane; e < E; e += 64) m = fmaxf(m, lrow[e]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    double zs = 0.0;
    for (int e = lane; e < E; e += 64) zs += exp((double)lrow[e] - (double)m);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) zs += __shfl_xor(zs, o, 64);
    double pdp = 0.0;
    if (lane < k) pdp = (double)(float)(exp((double)lrow[my_e] - (double)m) / zs) * (double)my_dg;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) pdp += __shfl_xor(pdp, o, 64);
    for (int e = lane; e < E; e += 64) {
      const double p = (double)(float)(exp((double)lrow[e] - (double)m) / zs);
      double dp = 0.0;
      for (int j = 0; j < k; ++j) {
        const int ej = __shfl(my_e, j, 64);
        const float dj = __shfl(my_dg, j, 64);
        if (ej == e) dp = (double)dj;
      }
      drow[e] = (float)(p * (dp - pdp));
    }
  }
}

// dx[t] = sum_j dx_perm[pos[t,j]] + dx_shared[t] + sum_e dlogits[t,e] W_r[e]
// (fp32, slot order, then shared, then router; one rounding).  For sigmoid
// and renormalised softmax routers dlogits is zero off the picked experts, so
// only those k rows of W_r are read.  KK > 0: compile-time slot count, all
// slot rows of a chunk in flight together.
template <typename T, int KK>
__global__ __launch_bounds__(256) void unpermute_sum_kernel(
    const T* __restrict__ dx_perm, const int32_t* __restrict__ pos, const T* dx_shared,
    const float* __restrict__ dlogits, const int32_t* __restrict__ idx,
    const float* __restrict__ w_router, int dense_router, int Tn, int d, int E, int k,
    T* __restrict__ dx) {
  constexpr int VN = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int nvec = d / VN;
  const int64_t tk = (int64_t)t * k;
  const int nr = dense_router ? E : k;
  if constexpr (KK > 0) {
    int64_t row[KK];
#pragma unroll
    for (int j = 0; j < KK; ++j) row[j] = (int64_t)pos[tk + j] * d;
    // sparse router term: the picked experts' dlogits and W_r rows are fixed
    // for the token, so their W_r chunks load together with the slot rows
    float dls[KK];
    const float* wrow[KK];
    if (!dense_router) {
#pragma unroll
      for (int j = 0; j < KK; ++j) {
        const int e = idx[tk + j];
        dls[j] = dlogits[(int64_t)t * E + e];
        wrow[j] = w_router + (int64_t)e * d;
      }
    }
#pragma unroll 2
    for (int c = lane; c < nvec; c += 64) {
      float v[KK][VN];
#pragma unroll
      for (int j = 0; j < KK; ++j) Vec<T>::load_f_nt(dx_perm + row[j] + (int64_t)c * VN, v[j]);
      float sh[VN];
      if (dx_shared) Vec<T>::load_f_nt(dx_shared + (int64_t)t * d + (int64_t)c * VN, sh);
      float wv[KK][VN];
      if (!dense_router) {
#pragma unroll
        for (int j = 0; j < KK; ++j)
#pragma unroll
          for (int u = 0; u < VN; u += 4) {
            const float4 q = *reinterpret_cast<const float4*>(wrow[j] + (int64_t)c * VN + u);
            wv[j][u] = q.x; wv[j][u + 1] = q.y; wv[j][u + 2] = q.z; wv[j][u + 3] = q.w;
          }
      }
      float acc[VN];
#pragma unroll
      for (int u = 0; u < VN; ++u) acc[u] = 0.0f;
#pragma unroll
      for (int j = 0; j < KK; ++j)
#pragma unroll
        for (int u = 0; u < VN; ++u) acc[u] += v[j][u];
      if (dx_shared) {
#pragma unroll
        for (int u = 0; u < VN; ++u) acc[u] += sh[u];
      }
      if (!dense_router) {
#pragma unroll
        for (int j = 0; j < KK; ++j)
#pragma unroll
          for (int u = 0; u < VN; ++u) acc[u] = fmaf(dls[j], wv[j][u], acc[u]);
      } else {
        for (int e = 0; e < E; ++e) {
          const float dl = dlogits[(int64_t)t * E + e];
          const float* wr = w_router + (int64_t)e * d + (int64_t)c * VN;
#pragma unroll
          for (int u = 0; u < VN; ++u) acc[u] = fmaf(dl, wr[u], acc[u]);
        }
      }
      Vec<T>::store_nt(dx + (int64_t)t * d + (int64_t)c * VN, acc);
    }
  } else {
    for (int c = lane; c < nvec; c += 64) {
      float acc[VN];
#pragma unroll
      for (int u = 0; u < VN; ++u) acc[u] = 0.0f;
      for (int j = 0; j < k; ++j) {
        const int64_t p = pos[tk + j];
        float v[VN];
        Vec<T>::load_f_nt(dx_perm + p * d + (int64_t)c * VN, v);
#pragma unroll
        for (int u = 0; u < VN; ++u) acc[u] += v[u];
      }
      if (dx_shared) {
        float v[VN];
        Vec<T>::load_f_nt(dx_shared + (int64_t)t * d + (int64_t)c * VN, v);
#pragma unroll
        for (int u = 0; u < VN; ++u) acc[u] += v[u];
      }
      for (int j = 0; j < nr; ++j) {
        const int e = dense_router ? j : idx[tk + j];
        const float dl = dlogits[(int64_t)t * E + e];
        const float* wr = w_router + (int64_t)e * d + (int64_t)c * VN;
#pragma unroll
        for (int u = 0; u < VN; ++u) acc[u] = fmaf(dl, wr[u], acc[u]);
      }
      Vec<T>::store_nt(dx + (int64_t)t * d + (int64_t)c * VN, acc);
    }
  }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// Dispatch a kernel template on the slot count: 1..8 at compile time, other
// counts through the generic loop (KK = 0).
#define MOE_K_DISPATCH(KERNEL, T, ...)                                      \
  switch (k) {                                                              \
    case 1: KERNEL<T, 1><<<grid, block, 0, st>>>(__VA_ARGS__); break;       \
    case 2: KERNEL<T, 2><<<grid, block, 0, st>>>(__VA_ARGS__); break;       \
    case 3: KERNEL<T, 3><<<grid, block, 0, st>>>(__VA_ARGS__); break;       \
    case 4: KERNEL<T, 4><<<grid, block, 0, st>>>(__VA_ARGS__); break;       \
    case 5: KERNEL<T, 5><<<grid, block, 0, st>>>(__VA_ARGS__); break;       \
    case 6: KERNEL<T, 6><<<grid, block, 0, st>>>(__VA_ARGS__); break;       \
    case 7: KERNEL<T, 7><<<grid, block, 0, st>>>(__VA_ARGS__); break;       \
    case 8: KERNEL<T, 8><<<grid, block, 0, st>>>(__VA_ARGS__); break;       \
    default: KERNEL<T, 0><<<grid, block, 0, st>>>(__VA_ARGS__); break;      \
  }

hipError_t launch_combine(int dtype, const void* y_perm, const float* gate, const int32_t* pos,
                          const void* shared_y, void* y, int T, int d, int k, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)cdiv64(T, 4)), block(256);
  if (dtype == MOE_BF16) {
    MOE_K_DISPATCH(combine_kernel, bf16_t, (const bf16_t*)y_perm, gate, pos, (const bf16_t*)shared_y,
                   (bf16_t*)y, T, d, k)
  } else {
    MOE_K_DISPATCH(combine_kernel, float, (const float*)y_perm, gate, pos, (const float*)shared_y,
                   (float*)y, T, d, k)
  }
  return hipGetLastError();
}

hipError_t launch_combine_bwd(int dtype, const void* dy, const void* y_perm, const float* gate,
                              const int32_t* pos, const int32_t* idx, const float* logits,
                              int score, int renorm, int T, int d, int E, int k, void* dy_perm,
                              float* dlogits, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)cdiv64(T, 4)), block(256);
  if (dtype == MOE_BF16) {
    MOE_K_DISPATCH(combine_bwd_kernel, bf16_t, (const bf16_t*)dy, (const bf16_t*)y_perm, gate, pos, idx,
                   logits, score, renorm, T, d, E, k, (bf16_t*)dy_perm, dlogits)
  } else {
    MOE_K_DISPATCH(combine_bwd_kernel, float, (const float*)dy, (const float*)y_perm, gate, pos, idx,
                   logits, score, renorm, T, d, E, k, (float*)dy_perm, dlogits)
  }
  return hipGetLastError();
}

hipError_t launch_combine_bwd_fp8(const void* dy, const void* y_perm, const float* gate, const int32_t* pos,
                                  const int32_t* idx, const float* logits, int score, int renorm, int T, int d,
                                  int E, int k, void* dy_perm, float* dlogits, uint8_t* q_perm, float* s_perm,
                                  uint8_t* q_dy, float* s_dy, hipStream_t st, int fmt) {
  if (T == 0) return hipSuccess;
  if (k < 1 || k > 8) return hipErrorInvalidValue;
  dim3 grid((unsigned)cdiv64(T, 4)), block(256);
  const Fp8Rows q{q_perm, s_perm, q_dy, s_dy};
#define MOE_Q8_CASE(K, F)                                                                                        \
  case K:                                                                                                        \
    combine_bwd_kernel<bf16_t, K, true, F><<<grid, block, 0, st>>>((const bf16_t*)dy, (const bf16_t*)y_perm, gate, \
                                                                   pos, idx, logits, score, renorm, T, d, E, k,    \
                                                                   (bf16_t*)dy_perm, dlogits, q);                 \
    break;
  if (fmt == FP8_E5M2) {
    switch (k) {
      MOE_Q8_CASE(1, FP8_E5M2) MOE_Q8_CASE(2, FP8_E5M2) MOE_Q8_CASE(3, FP8_E5M2) MOE_Q8_CASE(4, FP8_E5M2)
      MOE_Q8_CASE(5, FP8_E5M2) MOE_Q8_CASE(6, FP8_E5M2) MOE_Q8_CASE(7, FP8_E5M2) MOE_Q8_CASE(8, FP8_E5M2)
    }
  } else {
    switch (k) {
      MOE_Q8_CASE(1, FP8_E4M3) MOE_Q8_CASE(2, FP8_E4M3) MOE_Q8_CASE(3, FP8_E4M3) MOE_Q8_CASE(4, FP8_E4M3)
      MOE_Q8_CASE(5, FP8_E4M3) MOE_Q8_CASE(6, FP8_E4M3) MOE_Q8_CASE(7, FP8_E4M3) MOE_Q8_CASE(8, FP8_E4M3)
    }
  }
#undef MOE_Q8_CASE
  return hipGetLastError();
}

hipError_t launch_unpermute_sum(int dtype, const void* dx_perm, const int32_t* pos,
                                const void* dx_shared, const float* dlogits, const int32_t* idx,
                                const float* w_router, int dense_router, int T, int d, int E,
                                int k, void* dx, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)cdiv64(T, 4)), block(256);
  if (dtype == MOE_BF16) {
    MOE_K_DISPATCH(unpermute_sum_kernel, bf16_t, (const bf16_t*)dx_perm, pos, (const bf16_t*)dx_shared,
                   dlogits, idx, w_router, dense_router, T, d, E, k, (bf16_t*)dx)
  } else {
    MOE_K_DISPATCH(unpermute_sum_kernel, float, (const float*)dx_perm, pos, (const float*)dx_shared,
                   dlogits, idx, w_router, dense_router, T, d, E, k, (float*)dx)
  }
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  fill_i32_kernel<<<dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, st>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace moe
