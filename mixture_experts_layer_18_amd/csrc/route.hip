// Router top-k and token permutation kernels (gfx950).
//
// Routing follows the pages' description of the layer: a sigmoid router with a
// per-expert bias that only steers selection (Apex-3 code page, "What's
// inside", row "Fine-grained MoE"), or a softmax top-k router (KempnerForge
// README, "Features / Architecture"), on fp32 logits (Ultimate MoE Training
// Handbook, section 2.5, fp32 router dtype).  Permutation sends each token's
// row to its selected experts in expert-contiguous order (Handbook 2.5:
// tokens are sent to the selected experts).
#include "route_common.h"

namespace moe {

// One group of L lanes handles one token; lane i holds experts i, i+L, ...
// (V = ceil(E / L) values).  A workgroup of 256 threads handles one block of
// MOE_ROUTE_BLOCK tokens and writes that block's expert histogram.
template <int L, int V>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int k, int score, int renorm,
                                                    int32_t* __restrict__ idx,
                                                    float* __restrict__ gate,
                                                    int32_t* __restrict__ hist, int nblk) {
  __shared__ int s_hist[256];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) s_hist[e] = 0;
  __syncthreads();
  const int blk = blockIdx.x;
  const int li = tid % L;
  constexpr int GROUPS = 256 / L;
  for (int tl = tid / L; tl < MOE_ROUTE_BLOCK; tl += GROUPS) {
    const int t = blk * MOE_ROUTE_BLOCK + tl;
    if (t >= T) break;  // uniform within the group
    rte::route_token<L, V>(logits + (int64_t)t * E, bias, E, k, score, renorm, li, idx + (int64_t)t * k,
                           gate + (int64_t)t * k, s_hist);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) hist[(int64_t)e * nblk + blk] = s_hist[e];
}

// Per expert: exclusive prefix of its per-block counts (-> base) and total.
__global__ __launch_bounds__(256) void hist_scan_kernel(const int32_t* __restrict__ hist,
                                                        int nblk, int32_t* __restrict__ base,
                                                        int32_t* __restrict__ counts) {
  __shared__ int scratch[4];
  const int e = blockIdx.x;
  const int32_t* h = hist + (int64_t)e * nblk;
  int32_t* b = base + (int64_t)e * nblk;
  int carry = 0;
  for (int c0 = 0; c0 < nblk; c0 += 256) {
    const int i = c0 + threadIdx.x;
    const int v = (i < nblk) ? h[i] : 0;
    int tot;
    const int ex = block_exclusive_scan256(v, scratch, &tot);
    if (i < nblk) b[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// Stable scatter: within a block of MOE_ROUTE_BLOCK (= 32) tokens, the rank of
// assignment (t, j) among the block's assignments to the same expert is the
// number of earlier tokens of the block that picked that expert (each token
// picks an expert at most once), read off a 32-bit token mask per expert.
template <typename TX>
__global__ __launch_bounds__(256) void permute_kernel(
    const TX* __restrict__ x, const int32_t* __restrict__ idx, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ base, int T, int d, int E, int k, int nblk,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pos, int32_t* __restrict__ src,
    int32_t* __restrict__ tok, TX* __restrict__ x_perm) {
  static_assert(MOE_ROUTE_BLOCK == 32, "one mask word per expert");
  __shared__ int s_off[256];
  __shared__ uint32_t s_mask[256];
  __shared__ int s_pos[MOE_ROUTE_BLOCK * 16];
  __shared__ int scratch[4];
  const int tid = threadIdx.x;
  const int blk = blockIdx.x;
  const int t0 = blk * MOE_ROUTE_BLOCK;
  const int nt = min(MOE_ROUTE_BLOCK, T - t0);
  {
    const int c = (tid < E) ? counts[tid] : 0;
    int tot;
    const int ex = block_exclusive_scan256(c, scratch, &tot);
    s_off[tid] = ex;
    s_mask[tid] = 0u;
    if (blk == 0) {
      if (tid < E) offsets[tid] = ex;
      if (tid == 0) offsets[E] = tot;
    }
  }
  __syncthreads();
  const int na = nt * k;
  const int32_t* bidx = idx + (int64_t)t0 * k;
  // ids outside [0, E) (never written by moe_route) are skipped, not followed
  for (int i = tid; i < na; i += 256) {
    const int e = bidx[i];
    if ((unsigned)e < (unsigned)E) atomicOr(&s_mask[e], 1u << (i / k));
  }
  __syncthreads();
  for (int i = tid; i < na; i += 256) {
    const int tl = i / k;
    const int e = bidx[i];
    if ((unsigned)e >= (unsigned)E) {
      s_pos[i] = -1;
      continue;
    }
    const int rank = __popc(s_mask[e] & ((1u << tl) - 1u));
    const int p = s_off[e] + base[(int64_t)e * nblk + blk] + rank;
    const int a = t0 * k + i;
    pos[a] = p;
    src[p] = a;
    if (tok) tok[p] = t0 + tl;
    s_pos[i] = p;
  }
  // without x_perm the products read the token rows through tok
  if (!x_perm) return;
  __syncthreads();
  // row copies: the workgroup walks (token, 16-byte chunk) pairs with
  // consecutive threads on consecutive chunks, four pairs per thread in
  // flight; each loaded chunk is stored to the token's k permuted rows
  const int nvec = d * (int)sizeof(TX) / 16;
  const int total = nt * nvec;
  for (int i0 = tid; i0 < total; i0 += 4 * 256) {
    u32x4 v[4];
    int tl[4], c[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int i = i0 + u * 256;
      i = i < total ? i : total - 1;  // past the end: reload the last chunk, not stored
      tl[u] = i / nvec;
      c[u] = i - tl[u] * nvec;
      v[u] = reinterpret_cast<const u32x4*>(x + (int64_t)(t0 + tl[u]) * d)[c[u]];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (i0 + u * 256 >= total) continue;
      for (int j = 0; j < k; ++j) {
        const int p = s_pos[tl[u] * k + j];
        if (p < 0) continue;
        reinterpret_cast<u32x4*>(x_perm + (int64_t)p * d)[c[u]] = v[u];
      }
    }
  }
}

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int k, int score,
                        int renorm, int32_t* idx, float* gate, int32_t* hist, hipStream_t st) {
  const int nblk = (int)cdiv64(T, MOE_ROUTE_BLOCK);
  if (nblk == 0) return hipSuccess;
  dim3 grid(nblk), block(256);
  if (E <= 64)
    route_kernel<16, 4><<<grid, block, 0, st>>>(logits, bias, T, E, k, score, renorm, idx, gate,
                                                 hist, nblk);
  else if (E <= 128)
    route_kernel<32, 4><<<grid, block, 0, st>>>(logits, bias, T, E, k, score, renorm, idx, gate,
                                                 hist, nblk);
  else
    route_kernel<64, 4><<<grid, block, 0, st>>>(logits, bias, T, E, k, score, renorm, idx, gate,
                                                 hist, nblk);
  return hipGetLastError();
}

hipError_t launch_permute(const void* x, int dtype, const int32_t* idx, const int32_t* hist, int T,
                          int d, int E, int k, int32_t* base, int32_t* counts, int32_t* offsets,
                          int32_t* pos, int32_t* src, int32_t* tok, void* x_perm, hipStream_t st) {
  const int nblk = (int)cdiv64(T, MOE_ROUTE_BLOCK);
  hist_scan_kernel<<<dim3(E), dim3(256), 0, st>>>(hist, nblk, base, counts);
  if (nblk == 0) {
    // no tokens: offsets are all zero (a fill kernel, not a memset node)
    return launch_fill_i32(offsets, E + 1, 0, st);
  }
  if (dtype == MOE_BF16)
    permute_kernel<bf16_t><<<dim3(nblk), dim3(256), 0, st>>>(
        (const bf16_t*)x, idx, counts, base, T, d, E, k, nblk, offsets, pos, src, tok, (bf16_t*)x_perm);
  else
    permute_kernel<float><<<dim3(nblk), dim3(256), 0, st>>>(
        (const float*)x, idx, counts, base, T, d, E, k, nblk, offsets, pos, src, tok, (float*)x_perm);
  return hipGetLastError();
}

}  // namespace moe
