// Router products in fp32 on the gfx950 matrix cores.
//
// The router runs in fp32 (Ultimate MoE Training Handbook, section 2.5, the
// fp32 router dtype): the logits l = x W_r^T and the weight gradient
// dW_r = dl^T x are fp32 products with fp32 accumulation of a bf16 or fp32 x
// against the fp32 router weight.  E <= 256 experts makes these thin GEMMs:
//  * forward, fp32 x: a workgroup (4 waves) computes 64 tokens x 64 experts
//    on v_mfma_f32_32x32x2_f32; each wave one 32 x 32 tile, the reduction
//    over d staged through LDS in 32-deep steps, next step prefetched into
//    registers;
//  * forward, bf16 x: the same tiles on the bf16 matrix cores.  Each fp32
//    weight is split into three bf16 parts, w = hi + mid + lo exactly (each
//    part takes the next 8 significant bits of what the previous left, with
//    round-to-nearest), so x w = x hi + x mid + x lo where every product of
//    two bf16 values is exact in fp32, and the sum is accumulated in fp32:
//    the fp32 product up to the order of the fp32 additions, at the bf16
//    matrix-core rate (three 32x32x16 MFMAs per 16-deep step against eight
//    32x32x2 fp32 ones);
//  * weight gradient: a workgroup computes 64 experts x 64 columns of d over
//    a slice of the tokens; slices are summed afterwards in a fixed order, so
//    the result is deterministic.  For bf16 x on the bf16 matrix cores with
//    dlogits split the same way (below); for fp32 x on the fp32 ones.
#include "route_common.h"

namespace moe {
namespace rt {

constexpr int BK = 32;         // reduction step
constexpr int LP = BK + 1;     // LDS row pitch in floats (conflict-free column reads)

template <typename TX>
MOE_DEV void load8(const TX* p, float* f);
template <>
MOE_DEV void load8<bf16_t>(const bf16_t* p, float* f) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
template <>
MOE_DEV void load8<float>(const float* p, float* f) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// logits[T, E] = x[T, d] . W_r[E, d]^T
template <typename TX>
__global__ __launch_bounds__(256) void router_logits_kernel(const TX* __restrict__ x,
                                                            const float* __restrict__ w, int T,
                                                            int d, int E,
                                                            float* __restrict__ logits) {
  __shared__ float xs[64 * LP];
  __shared__ float ws[64 * LP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  // loader: thread -> row tid/4 (0..63), 8 consecutive k at (tid%4)*8
  const int lr = tid >> 2, lk = (tid & 3) * 8;
  const int tr = min(t0 + lr, T - 1), er = min(e0 + lr, E - 1);
  const TX* xp = x + (int64_t)tr * d + lk;
  const float* wp = w + (int64_t)er * d + lk;
  float xv[8], wv[8];
  load8<TX>(xp, xv);
  load8<float>(wp, wv);
  const int wt = wave >> 1, we = wave & 1;  // this wave's 32-token x 32-expert tile
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  for (int k0 = 0; k0 < d; k0 += BK) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      xs[lr * LP + lk + u] = xv[u];
      ws[lr * LP + lk + u] = wv[u];
    }
    __syncthreads();
    if (k0 + BK < d) {
      load8<TX>(xp + k0 + BK, xv);
      load8<float>(wp + k0 + BK, wv);
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += 2) {
      const float a = xs[(wt * 32 + (lane & 31)) * LP + kk + (lane >> 5)];
      const float b = ws[(we * 32 + (lane & 31)) * LP + kk + (lane >> 5)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // lane: expert (lane%32) of the wave tile, tokens (v/4)*8 + (lane/32)*4 + v%4
  const int e = e0 + we * 32 + (lane & 31);
  if (e >= E) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = t0 + wt * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
    if (t < T) logits[(int64_t)t * E + e] = acc[v];
  }
}

// logits[T, E] = x[T, d] . W_r[E, d]^T for bf16 x, 64-deep steps.  LDS holds
// per step x [64][64] and the three parts of W [3][64][64] as bf16 rows of
// 128 bytes whose 16-byte chunks are XOR-swizzled by row; two buffers, one
// barrier per step.
constexpr int SBK = 64;                         // reduction step (bf16 path)
constexpr int SROW = SBK * 2;                   // bytes per LDS row
constexpr int STILE = 64 * SROW;                // one 64-row tile (8 KB)

MOE_DEV int sw_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

// Routing of the kernel's own logits (ROUTE: E <= 64, so one workgroup holds
// every logit of its 64 tokens, two blocks of MOE_ROUTE_BLOCK): top-k, gates
// and the two blocks' expert histograms, as moe_route computes them.
struct RouteOut {
  const float* bias;
  int k, score, renorm, nblk;
  int32_t* idx;
  float* gate;
  int32_t* hist;
};

// KG groups of 4 waves split the reduction: group g takes the steps
// g, g + KG, g + 2 KG, ... with LDS buffers of its own, and the groups' sums
// are added in group order at the end (deterministic).  With KG = 2 two
// waves share each SIMD, so one wave's weight splitting, LDS traffic and
// barrier wait run under the other's MFMAs (one 4-wave workgroup per CU
// serialises them).
template <bool ROUTE, int KG>
__global__ __launch_bounds__(256 * KG) void router_logits_split_kernel(const bf16_t* __restrict__ x,
                                                                       const float* __restrict__ w, int T,
                                                                       int d, int E,
                                                                       float* __restrict__ logits,
                                                                       RouteOut ro) {
  __shared__ __attribute__((aligned(16))) char sm[2 * KG][4 * STILE];  // [group, buffer][x, hi, mid, lo]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave >> 2, ltid = tid & 255;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  // loader: thread -> row ltid/4, 16 consecutive k at (ltid%4)*16 (two 16-byte chunks)
  const int lr = ltid >> 2, lc = (ltid & 3) * 2;
  const int tr = min(t0 + lr, T - 1), er = min(e0 + lr, E - 1);
  const bf16_t* xp = x + (int64_t)tr * d + lc * 8;
  const float* wp = w + (int64_t)er * d + lc * 8;
  // two steps of operands in flight in registers (sets 0 and 1); plain
  // vector variables, no arrays, so that they stay in registers
  struct Ops {
    u32x4 x0, x1;
    float4 w0, w1, w2, w3;
  };
  Ops o0, o1;
  // past the end the last step is reloaded (not used): no branch in the loop
  auto gload = [&](int k0, Ops& o) __attribute__((always_inline)) {
    k0 = k0 < d ? k0 : d - SBK;
    const u32x4* xq = reinterpret_cast<const u32x4*>(xp + k0);
    const float4* wq = reinterpret_cast<const float4*>(wp + k0);
    o.x0 = xq[0];
    o.x1 = xq[1];
    o.w0 = wq[0];
    o.w1 = wq[1];
    o.w2 = wq[2];
    o.w3 = wq[3];
  };
  // three-way split of 4 weights into packed bf16 pairs: hi, mid, lo
  auto split4 = [](float4 v, u32x2& h, u32x2& m, u32x2& l) __attribute__((always_inline)) {
    h.x = pack_bf16x2(v.x, v.y);
    h.y = pack_bf16x2(v.z, v.w);
    const float r0 = v.x - bf16_lo(h.x), r1 = v.y - bf16_hi(h.x);
    const float r2 = v.z - bf16_lo(h.y), r3 = v.w - bf16_hi(h.y);
    m.x = pack_bf16x2(r0, r1);
    m.y = pack_bf16x2(r2, r3);
    l.x = pack_bf16x2(r0 - bf16_lo(m.x), r1 - bf16_hi(m.x));
    l.y = pack_bf16x2(r2 - bf16_lo(m.y), r3 - bf16_hi(m.y));
  };
  auto put = [&](char* buf, int chunk, u32x4 xv, float4 wa, float4 wb) __attribute__((always_inline)) {
    u32x2 ha, ma, la, hb, mb, lb;
    split4(wa, ha, ma, la);
    split4(wb, hb, mb, lb);
    const int off = lr * SROW + (sw_slot(lr, chunk) << 4);
    *reinterpret_cast<u32x4*>(buf + off) = xv;
    *reinterpret_cast<u32x4*>(buf + STILE + off) = u32x4{ha.x, ha.y, hb.x, hb.y};
    *reinterpret_cast<u32x4*>(buf + 2 * STILE + off) = u32x4{ma.x, ma.y, mb.x, mb.y};
    *reinterpret_cast<u32x4*>(buf + 3 * STILE + off) = u32x4{la.x, la.y, lb.x, lb.y};
  };
  auto lstore = [&](char* buf, const Ops& o) __attribute__((always_inline)) {
    put(buf, lc, o.x0, o.w0, o.w1);
    put(buf, lc + 1, o.x1, o.w2, o.w3);
  };
  const int wl = wave & 3;
  const int wt = wl >> 1, we = wl & 1;  // this wave's 32-token x 32-expert tile
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  const int xr = wt * 32 + (lane & 31), wr = we * 32 + (lane & 31);
  auto compute = [&](const char* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < SBK / 16; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(buf + xr * SROW + (sw_slot(xr, c) << 4));
#pragma unroll
      for (int part = 1; part <= 3; ++part) {
        const bf16x8_t bw =
            *reinterpret_cast<const bf16x8_t*>(buf + part * STILE + wr * SROW + (sw_slot(wr, c) << 4));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bw, acc, 0, 0, 0);
      }
    }
  };
  // step j of group g reads k0 = (j KG + g) SBK; register set j % 2, LDS
  // buffer j % 2 of the group; the loads of step j + 2 are in flight while
  // step j is computed.  One barrier per step separates its LDS stores from
  // its fragment reads; a buffer is rewritten two steps later, after the next
  // step's barrier, which every wave passes only once done reading it.
  // d is a multiple of 2 KG SBK (the launcher sends other widths elsewhere).
  char* b0 = sm[2 * grp];
  char* b1 = sm[2 * grp + 1];
  const int kstep = KG * SBK;
  gload(grp * SBK, o0);
  gload(grp * SBK + kstep, o1);
  for (int k0 = grp * SBK; k0 < d; k0 += 2 * kstep) {
    lstore(b0, o0);
    __syncthreads();
    gload(k0 + 2 * kstep, o0);
    compute(b0);
    lstore(b1, o1);
    __syncthreads();
    gload(k0 + 3 * kstep, o1);
    compute(b1);
  }
  if constexpr (KG == 2) {
    // group 1's sums join group 0's (fixed order), through LDS
    __syncthreads();  // every wave is done with the operand buffers
    float* red = reinterpret_cast<float*>(&sm[0][0]);
    if (grp == 1) {
#pragma unroll
      for (int v = 0; v < 16; ++v) red[(wl * 16 + v) * 64 + lane] = acc[v];
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] += red[(wl * 16 + v) * 64 + lane];
  }
  // group 0 writes the results; group 1 only takes part in the barriers below
  const bool out = grp == 0;
  // lane: expert (lane%32) of the wave tile, tokens (v/4)*8 + (lane/32)*4 + v%4
  const int e = e0 + we * 32 + (lane & 31);
  if constexpr (!ROUTE) {
    if (!out || e >= E) return;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int t = t0 + wt * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
      if (t < T) logits[(int64_t)t * E + e] = acc[v];
    }
  } else {
    // the 64 x E logits into LDS (rows padded to 65), then one group of 16
    // lanes per token routes from there
    constexpr int LPAD = 65;
    __syncthreads();  // every wave is done with the operand buffers (and the group sums)
    float* ls = reinterpret_cast<float*>(&sm[0][0]);
    int* s_hist = reinterpret_cast<int*>(ls + 64 * LPAD);  // [2 blocks][64 experts]
    if (out && e < E) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tl = wt * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        ls[tl * LPAD + (e - e0)] = acc[v];
        if (t0 + tl < T) logits[(int64_t)(t0 + tl) * E + e] = acc[v];
      }
    }
    if (tid < 128) s_hist[tid] = 0;
    __syncthreads();
    // every wave routes: 16 lanes per token, 16 KG tokens per pass
    {
      const int li = tid & 15;
      for (int tl = tid >> 4; tl < 64; tl += 16 * KG) {
        const int t = t0 + tl;
        if (t >= T) break;  // uniform within the 16-lane group
        rte::route_token<16, 4>(ls + tl * LPAD, ro.bias, E, ro.k, ro.score, ro.renorm, li,
                                ro.idx + (int64_t)t * ro.k, ro.gate + (int64_t)t * ro.k,
                                s_hist + (tl >> 5) * 64);
      }
    }
    __syncthreads();
    for (int i = tid; i < 2 * E; i += 256 * KG) {
      const int b = blockIdx.x * 2 + i / E, ee = i % E;
      if (b < ro.nblk) ro.hist[(int64_t)ee * ro.nblk + b] = s_hist[(i / E) * 64 + ee];
    }
  }
}

// part[s][E][d] = sum over tokens of slice s of dl[t, e] x[t, :]
template <typename TX>
__global__ __launch_bounds__(256) void router_wgrad_kernel(const float* __restrict__ dl,
                                                           const TX* __restrict__ x, int T,
                                                           int d, int E, int tok_per_split,
                                                           float* __restrict__ part) {
  __shared__ float ds[BK * 65];  // [token][expert]
  __shared__ float xs[BK * 65];  // [token][column]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = blockIdx.x * 64, e0 = blockIdx.y * 64, s = blockIdx.z;
  const int tlo = s * tok_per_split, thi = min(T, tlo + tok_per_split);
  // loader: thread -> token tid/8 (0..31), 8 consecutive columns at (tid%8)*8
  const int lt = tid >> 3, lc = (tid & 7) * 8;
  const int we = wave >> 1, wc = wave & 1;
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  for (int tb = tlo; tb < thi; tb += BK) {
    const int t = tb + lt;
    float dv[8], xv[8];
    if (t < thi) {
#pragma unroll
      for (int u = 0; u < 8; ++u) dv[u] = (e0 + lc + u < E) ? dl[(int64_t)t * E + e0 + lc + u] : 0.0f;
      load8<TX>(x + (int64_t)t * d + c0 + lc, xv);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) dv[u] = xv[u] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      ds[lt * 65 + lc + u] = dv[u];
      xs[lt * 65 + lc + u] = xv[u];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 2) {
      const float a = ds[(kk + (lane >> 5)) * 65 + we * 32 + (lane & 31)];
      const float b = xs[(kk + (lane >> 5)) * 65 + wc * 32 + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // lane: column (lane%32) of the wave tile, experts (v/4)*8 + (lane/32)*4 + v%4
  const int col = c0 + wc * 32 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int e = e0 + we * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
    if (e < E) part[((int64_t)s * E + e) * d + col] = acc[v];
  }
}

// part[s][E][d] for bf16 x on the bf16 matrix cores: dl (fp32) is split
// exactly into three bf16 parts as the weight is in the forward, so every
// partial product is exact and the sums accumulate in fp32.  Per 32-token
// step LDS holds the three parts of dl as [64 experts][32 tokens] and x as
// [64 columns][32 tokens] (bf16, 64-byte rows, 16-byte chunks XOR-swizzled
// by row): the token axis is the reduction, so both operands are stored
// transposed.  Loads run along experts (columns), 8 (4) bytes per lane.
constexpr int WBK = 32;                          // tokens per step
constexpr int WROW = WBK * 2;                    // bytes per LDS row
constexpr int WTILE = 64 * WROW;                 // one 64-row tile (4 KB)

MOE_DEV int wslot(int r, int c) { return c ^ ((r >> 2) & 3); }

__global__ __launch_bounds__(256) void router_wgrad_split_kernel(const float* __restrict__ dl,
                                                                 const bf16_t* __restrict__ x, int T,
                                                                 int d, int E, int tok_per_split,
                                                                 float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) char sm[4 * WTILE];  // dl hi, mid, lo; x
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = blockIdx.x * 64, e0 = blockIdx.y * 64, s = blockIdx.z;
  const int tlo = s * tok_per_split, thi = min(T, tlo + tok_per_split);
  // loader: thread -> a pair of experts (columns) p = tid % 32 and four
  // consecutive tokens q*4 .. q*4+3 with q = tid / 32
  const int p = tid & 31, q = tid >> 5;
  const int ep = min(e0 + 2 * p, E - 2);          // E is even (>= 2) on this path
  const int cp = c0 + 2 * p;
  const int we = wave >> 1, wc = wave & 1;        // this wave's 32-expert x 32-column tile
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  // experts beyond E (a partial expert block) contribute zero
  const bool e_ok0 = e0 + 2 * p < E, e_ok1 = e0 + 2 * p + 1 < E;
  // the operands of the step at token tb (zero past the slice end)
  auto gload = [&](int tb, float2* dv, uint32_t* xv) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = tb + q * 4 + u;
      if (t < thi) {
        dv[u] = *reinterpret_cast<const float2*>(dl + (int64_t)t * E + ep);
        xv[u] = *reinterpret_cast<const uint32_t*>(x + (int64_t)t * d + cp);
      } else {
        dv[u] = float2{0.0f, 0.0f};
        xv[u] = 0u;
      }
    }
  };
  // dl split exactly into three bf16 parts and x, transposed into LDS
  auto stage = [&](const float2* dv, const uint32_t* xv) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // the four tokens of expert (column) 2p + h, split and packed
      float f[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) f[u] = (h ? (e_ok1 ? dv[u].y : 0.0f) : (e_ok0 ? dv[u].x : 0.0f));
      const uint32_t h0 = pack_bf16x2(f[0], f[1]), h1 = pack_bf16x2(f[2], f[3]);
      const float r0 = f[0] - bf16_lo(h0), r1 = f[1] - bf16_hi(h0);
      const float r2 = f[2] - bf16_lo(h1), r3 = f[3] - bf16_hi(h1);
      const uint32_t m0 = pack_bf16x2(r0, r1), m1 = pack_bf16x2(r2, r3);
      const uint32_t l0 = pack_bf16x2(r0 - bf16_lo(m0), r1 - bf16_hi(m0));
      const uint32_t l1 = pack_bf16x2(r2 - bf16_lo(m1), r3 - bf16_hi(m1));
      const uint32_t xa = h ? (xv[0] >> 16) | (xv[1] & 0xffff0000u) : (xv[0] & 0xffffu) | (xv[1] << 16);
      const uint32_t xb = h ? (xv[2] >> 16) | (xv[3] & 0xffff0000u) : (xv[2] & 0xffffu) | (xv[3] << 16);
      const int r = 2 * p + h;
      const int off = r * WROW + (wslot(r, q >> 1) << 4) + (q & 1) * 8;
      *reinterpret_cast<u32x2*>(sm + off) = u32x2{h0, h1};
      *reinterpret_cast<u32x2*>(sm + WTILE + off) = u32x2{m0, m1};
      *reinterpret_cast<u32x2*>(sm + 2 * WTILE + off) = u32x2{l0, l1};
      *reinterpret_cast<u32x2*>(sm + 3 * WTILE + off) = u32x2{xa, xb};
    }
  };
  const int ar = we * 32 + (lane & 31), br = wc * 32 + (lane & 31);
  auto compute = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < WBK / 16; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(sm + 3 * WTILE + br * WROW + (wslot(br, c) << 4));
#pragma unroll
      for (int pt = 0; pt < 3; ++pt) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(sm + pt * WTILE + ar * WROW + (wslot(ar, c) << 4));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      }
    }
  };
  // steps in pairs, one register set per parity: the loads of step j + 2 are
  // in flight while step j is staged and computed
  float2 dA[4], dB[4];
  uint32_t xA[4], xB[4];
  gload(tlo, dA, xA);
  gload(tlo + WBK, dB, xB);
  for (int tb = tlo; tb < thi; tb += 2 * WBK) {
    __syncthreads();  // the previous step's fragments have been read
    stage(dA, xA);
    gload(tb + 2 * WBK, dA, xA);
    __syncthreads();
    compute();
    if (tb + WBK < thi) {  // uniform over the workgroup
      __syncthreads();
      stage(dB, xB);
      gload(tb + 3 * WBK, dB, xB);
      __syncthreads();
      compute();
    }
  }
  // lane: column (lane%32) of the wave tile, experts (v/4)*8 + (lane/32)*4 + v%4
  const int col = c0 + wc * 32 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int e = e0 + we * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
    if (e < E) part[((int64_t)s * E + e) * d + col] = acc[v];
  }
}

}  // namespace rt

int router_wgrad_splits(int T, int d, int E) {
  const int tiles = (int)(cdiv64(d, 64) * cdiv64(E, 64));
  int s = 1;
  while (tiles * s < 1024 && T / (s * 2) >= 256 && s < 64) s *= 2;
  return s;
}

hipError_t launch_router_logits(const void* x, int dtype, const float* w, int T, int d, int E,
                                float* logits, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)cdiv64(T, 64), (unsigned)cdiv64(E, 64)), block(256);
  if (dtype == MOE_BF16 && d % (4 * rt::SBK) == 0)
    rt::router_logits_split_kernel<false, 2><<<grid, dim3(512), 0, st>>>((const bf16_t*)x, w, T, d, E, logits,
                                                                        rt::RouteOut{});
  else if (dtype == MOE_BF16 && d % (2 * rt::SBK) == 0)
    rt::router_logits_split_kernel<false, 1><<<grid, block, 0, st>>>((const bf16_t*)x, w, T, d, E, logits,
                                                                      rt::RouteOut{});
  else if (dtype == MOE_BF16)
    rt::router_logits_kernel<bf16_t><<<grid, block, 0, st>>>((const bf16_t*)x, w, T, d, E, logits);
  else
    rt::router_logits_kernel<float><<<grid, block, 0, st>>>((const float*)x, w, T, d, E, logits);
  return hipGetLastError();
}

bool router_route_fused(int dtype, int d, int E) { return dtype == MOE_BF16 && d % (2 * rt::SBK) == 0 && E <= 64; }

hipError_t launch_router_route(const void* x, const float* w, int T, int d, int E, float* logits,
                               const float* bias, int k, int score, int renorm, int32_t* idx, float* gate,
                               int32_t* hist, hipStream_t st) {
  if (T == 0) return hipSuccess;
  rt::RouteOut ro;
  ro.bias = bias;
  ro.k = k;
  ro.score = score;
  ro.renorm = renorm;
  ro.nblk = (int)cdiv64(T, MOE_ROUTE_BLOCK);
  ro.idx = idx;
  ro.gate = gate;
  ro.hist = hist;
  static_assert(2 * MOE_ROUTE_BLOCK == 64, "two histogram blocks per workgroup");
  if (d % (4 * rt::SBK) == 0)
    rt::router_logits_split_kernel<true, 2><<<dim3((unsigned)cdiv64(T, 64)), dim3(512), 0, st>>>(
        (const bf16_t*)x, w, T, d, E, logits, ro);
  else
    rt::router_logits_split_kernel<true, 1><<<dim3((unsigned)cdiv64(T, 64)), dim3(256), 0, st>>>(
        (const bf16_t*)x, w, T, d, E, logits, ro);
  return hipGetLastError();
}

hipError_t launch_router_wgrad(const float* dl, const void* x, int dtype, int T, int d, int E,
                               float* part, float* dw, hipStream_t st) {
  const int S = router_wgrad_splits(T, d, E);
  const int per = (int)cdiv64(T > 0 ? T : 1, S);
  dim3 grid((unsigned)cdiv64(d, 64), (unsigned)cdiv64(E, 64), (unsigned)S), block(256);
  float* out = S > 1 ? part : dw;
  if (dtype == MOE_BF16 && E % 2 == 0)
    rt::router_wgrad_split_kernel<<<grid, block, 0, st>>>(dl, (const bf16_t*)x, T, d, E, per, out);
  else if (dtype == MOE_BF16)
    rt::router_wgrad_kernel<bf16_t><<<grid, block, 0, st>>>(dl, (const bf16_t*)x, T, d, E, per, out);
  else
    rt::router_wgrad_kernel<float><<<grid, block, 0, st>>>(dl, (const float*)x, T, d, E, per, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  return launch_split_reduce_f32(part, S, (int64_t)E * d, dw, st);
}

}  // namespace moe
