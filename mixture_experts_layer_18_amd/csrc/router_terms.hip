// Router training terms (gfx950): the load-balancing losses, the router
// z-loss and the proportional bias update.
//
// Apex-3 code page ("What's inside", "Fine-grained MoE": a per-expert bias
// balances the load; "Run it yourself": router_bias_update=proportional,
// router_bias_rate, seq_aux_alpha); Ultimate MoE Training Handbook 2.5 (an
// auxiliary balance loss with coefficient 1e-3); KempnerForge README
// ("Features": router z-loss; "MoE roadmap": sequence aux loss, adaptive
// bias).
//
// With q[t, e] the router's distribution over the E experts (the softmax
// probabilities, or the sigmoid scores normalised to sum 1):
//   aux     = a_coef * E * sum_e f_e P_e,   f_e = counts_e / (T k),
//             P_e = mean_t q[t, e]
//   seq_aux = s_coef / n * sum_s sum_e f^s_e P^s_e over the n sequences of S
//             tokens, f^s_e = E / (k S) * #(tokens of s picking e),
//             P^s_e = mean over s of q[t, e]
//   z       = z_coef * mean_t lse_t^2,  lse_t = log sum_e exp l[t, e]
// The load shares f carry no gradient; the gradients reach the logits through
// q (and the softmax for z) and are added to dlogits.
//
// Everything is fp64 inside and deterministic: fixed-order block reductions,
// no atomics.  Four launches:
//   stats   one wavefront per token: lse_t and, for sigmoid, sum_e s[t, e]
//   colsum  one workgroup per (sequence, expert): sum over the sequence of
//           q[t, e] and the number of its tokens that picked e; the workgroup
//           of expert 0 also sums lse_t^2
//   grad    one wavefront per token: dlogits[t, :] += the three gradients
//   values  one workgroup: the three loss values
#include "kernels.h"

namespace moe {
namespace rterm {

// lanes per token cover the E experts in ceil(E / 64) passes
__global__ __launch_bounds__(256) void stats_kernel(const float* __restrict__ logits, int T, int E,
                                                    double* __restrict__ lse,
                                                    double* __restrict__ ssum) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + (int64_t)t * E;
  double m = -INFINITY;
  for (int e = lane; e < E; e += 64) m = fmax(m, (double)l[e]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
  double z = 0.0, s = 0.0;
  for (int e = lane; e < E; e += 64) {
    const double v = (double)l[e];
    z += exp(v - m);
    s += 1.0 / (1.0 + exp(-v));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    z += __shfl_xor(z, o, 64);
    s += __shfl_xor(s, o, 64);
  }
  if (lane == 0) {
    lse[t] = m + log(z);
    ssum[t] = s;
  }
}

MOE_DEV double q_of(double l, double lse_t, double ssum_t, int score) {
  return score == MOE_SOFTMAX ? exp(l - lse_t) : (1.0 / (1.0 + exp(-l))) / ssum_t;
}

// block-wide sum over 256 threads in a fixed order
MOE_DEV double block_sum(double v, double* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  return sh[0] + sh[1] + sh[2] + sh[3];
}

__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ logits,
                                                     const int32_t* __restrict__ idx,
                                                     const double* __restrict__ lse,
                                                     const double* __restrict__ ssum, int E, int k,
                                                     int S, int score, double* __restrict__ pseq,
                                                     int32_t* __restrict__ cseq,
                                                     double* __restrict__ zseq) {
  __shared__ double sh[4];
  const int e = blockIdx.x, sq = blockIdx.y;
  const int64_t t0 = (int64_t)sq * S;
  double p = 0.0, c = 0.0, z = 0.0;
  for (int i = threadIdx.x; i < S; i += 256) {
    const int64_t t = t0 + i;
    p += q_of((double)logits[t * E + e], lse[t], ssum[t], score);
    int hit = 0;
    for (int j = 0; j < k; ++j) hit |= (idx[t * k + j] == e);
    c += hit;
    if (e == 0) z += lse[t] * lse[t];
  }
  p = block_sum(p, sh);
  c = block_sum(c, sh);
  if (e == 0) z = block_sum(z, sh);
  if (threadIdx.x == 0) {
    pseq[(int64_t)sq * E + e] = p;
    cseq[(int64_t)sq * E + e] = (int32_t)c;
    if (e == 0) zseq[sq] = z;
  }
}

struct Coef {
  double a, s, z;  // aux, seq_aux and z coefficients
  int T, E, k, S, n, score;
};

// dL/dq[t, e] of the two balance losses
MOE_DEV double dq_balance(const Coef& c, const int32_t* counts, const int32_t* cseq, int sq, int e) {
  double g = 0.0;
  if (c.a != 0.0) g += c.a * c.E * ((double)counts[e] / ((double)c.T * c.k)) / c.T;
  if (c.s != 0.0)
    g += c.s / c.n * ((double)cseq[(int64_t)sq * c.E + e] * c.E / ((double)c.k * c.S)) / c.S;
  return g;
}

// one wavefront per token; lanes hold up to 4 experts each (E <= 256)
__global__ __launch_bounds__(256) void grad_kernel(const float* __restrict__ logits,
                                                   const double* __restrict__ lse,
                                                   const double* __restrict__ ssum,
                                                   const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ cseq, Coef c,
                                                   float* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= c.T) return;
  const int sq = t / c.S;
  const float* l = logits + (int64_t)t * c.E;
  const double L = lse[t], Ss = ssum[t];
  double q[4], g[4], sg[4];
  double qg = 0.0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = lane + 64 * u;
    q[u] = g[u] = sg[u] = 0.0;
    if (e < c.E) {
      const double v = (double)l[e];
      sg[u] = 1.0 / (1.0 + exp(-v));
      q[u] = c.score == MOE_SOFTMAX ? exp(v - L) : sg[u] / Ss;
      g[u] = dq_balance(c, counts, cseq, sq, e);
      qg += q[u] * g[u];
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) qg += __shfl_xor(qg, o, 64);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = lane + 64 * u;
    if (e >= c.E) continue;
    double dl;
    if (c.score == MOE_SOFTMAX) {
      dl = q[u] * (g[u] - qg);
    } else {
      const double ds = (g[u] - qg) / Ss;
      dl = ds * sg[u] * (1.0 - sg[u]);
    }
    if (c.z != 0.0) dl += c.z * 2.0 / c.T * L * exp((double)l[e] - L);
    float* p = dlogits + (int64_t)t * c.E + e;
    *p = (float)((double)*p + dl);
  }
}

__global__ __launch_bounds__(256) void values_kernel(const int32_t* __restrict__ counts,
                                                     const double* __restrict__ pseq,
                                                     const int32_t* __restrict__ cseq,
                                                     const double* __restrict__ zseq, Coef c,
                                                     float* __restrict__ out) {
  __shared__ double sh[4];
  double va = 0.0, vs = 0.0, vz = 0.0;
  for (int e = threadIdx.x; e < c.E; e += 256) {
    double P = 0.0;
    for (int sq = 0; sq < c.n; ++sq) {
      const double ps = pseq[(int64_t)sq * c.E + e];
      P += ps;
      vs += ((double)cseq[(int64_t)sq * c.E + e] * c.E / ((double)c.k * c.S)) * (ps / c.S);
    }
    va += ((double)counts[e] / ((double)c.T * c.k)) * (P / c.T);
  }
  for (int sq = threadIdx.x; sq < c.n; sq += 256) vz += zseq[sq];
  va = block_sum(va, sh);
  vs = block_sum(vs, sh);
  vz = block_sum(vz, sh);
  if (threadIdx.x == 0) {
    out[0] = (float)(c.a * c.E * va);
    out[1] = (float)(c.s / c.n * vs);
    out[2] = (float)(c.z * vz / c.T);
  }
}

__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts, int E,
                                                          double mean, float rate,
                                                          float* __restrict__ bias) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  bias[e] = (float)((double)bias[e] + (double)rate * (mean - (double)counts[e]) / mean);
}

}  // namespace rterm

size_t router_terms_ws_bytes(int64_t T, int64_t E) {
  // lse, ssum: T doubles each; per (sequence, expert) sums for up to T
  // sequences: T*E doubles and T*E int32; per-sequence z sums: T doubles
  return (size_t)T * (3 * sizeof(double)) + (size_t)T * E * (sizeof(double) + sizeof(int32_t));
}

hipError_t launch_router_terms(const float* logits, const int32_t* idx, const int32_t* counts,
                               int T, int E, int k, int score, float aux_coeff,
                               float seq_aux_coeff, float z_coeff, int seq_len, float* dlogits,
                               float* losses, void* ws, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int S = seq_len > 0 ? seq_len : T;
  const int n = T / S;
  char* w = (char*)ws;
  double* lse = (double*)w;
  double* ssum = lse + T;
  double* zseq = ssum + T;
  double* pseq = zseq + T;
  int32_t* cseq = (int32_t*)(pseq + (int64_t)T * E);
  rterm::Coef c{aux_coeff, seq_aux_coeff, z_coeff, T, E, k, S, n, score};
  const dim3 tok((unsigned)cdiv64(T, 4));
  rterm::stats_kernel<<<tok, 256, 0, st>>>(logits, T, E, lse, ssum);
  rterm::colsum_kernel<<<dim3((unsigned)E, (unsigned)n), 256, 0, st>>>(logits, idx, lse, ssum, E, k, S,
                                                                       score, pseq, cseq, zseq);
  rterm::grad_kernel<<<tok, 256, 0, st>>>(logits, lse, ssum, counts, cseq, c, dlogits);
  if (losses) rterm::values_kernel<<<1, 256, 0, st>>>(counts, pseq, cseq, zseq, c, losses);
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, int T, int E, int k, float rate, float* bias,
                              hipStream_t st) {
  if (T == 0 || E == 0) return hipSuccess;
  rterm::bias_update_kernel<<<(unsigned)cdiv64(E, 256), 256, 0, st>>>(counts, E, (double)T * k / E,
                                                                      rate, bias);
  return hipGetLastError();
}

}  // namespace moe
