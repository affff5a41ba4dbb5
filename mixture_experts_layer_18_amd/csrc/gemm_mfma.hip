// bf16 grouped GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Experts run as grouped GEMMs (Apex-3 code page, "What's inside", row
// "Fine-grained MoE"; Ultimate MoE Training Handbook, section 2.5).  One
// kernel template covers the three products of a SwiGLU expert:
//   NT  C[m,n]   = sum_k A[m,k] B[g,n,k]        forward (+ SwiGLU epilogue)
//   NN  C[m,k]   = sum_n A[m,n] B[g,n,k]        data gradient (+ dSwiGLU)
//   TN  C[g,n,k] = sum_{m in g} A[m,n] B[m,k]   weight gradient
//
// Design (CDNA4-first):
//  * operands move HBM -> LDS with global_load_lds_dwordx4 (no staging
//    registers), STAGES k-steps of BK in flight, one barrier per k-step;
//  * two workgroups share a CU (72 KB of LDS and 256 registers per lane
//    each), so one workgroup's barriers, DMA issue and epilogue stores
//    overlap the other's matrix-core work;
//  * an operand whose reduction dimension is contiguous is stored as rows of
//    2*BK bytes whose 16-byte chunks are XOR-swizzled so that the 16 rows a
//    ds_read_b128 services together land in distinct banks (64 banks);
//  * an operand whose reduction dimension is strided (NN's B, both TN
//    operands) is stored in its natural [k][column] layout, chunks swizzled
//    by 4*(k % 4), and fed to the matrix cores through pairs of
//    ds_read_b64_tr_b16 transpose reads (each turns a 4 x 16 block held by
//    16 lanes into per-lane columns);
//  * each of the 4 wavefronts owns a (TM/2) x (TN/2) block of 32x32 MFMA
//    tiles with fp32 accumulators in AGPRs;
//  * ragged groups: row tiles are enumerated group after group from the
//    device-side offsets (no host copy); surplus workgroups of the
//    upper-bound grid exit at once;
//  * tile order is XCD-aware: the hardware deals workgroups to the 8 XCDs
//    round-robin, so linear tile ids are remapped to give every XCD a
//    contiguous range, keeping the tiles of one expert inside one L2.
#include "gemm_common.h"

namespace moe {
namespace mf {
using namespace gk;


struct Args {
  int G;
  int64_t M_total, N, K;
  const int32_t* offsets;
  const bf16_t* A;
  const bf16_t* B;
  bf16_t* C;
  bf16_t* aux;
  int splits;   // TN: row slices per group (> 1: fp32 partials in `part`)
  float* part;  // [splits][G][N][K]
};

// workgroups resident on one XCD at a time (32 CUs x 2)
constexpr int kResident = 64;

template <int LAYOUT, int EPI, int TM, int TN, int BK, int STAGES, int OCC>
__global__ __launch_bounds__(256, OCC) void gemm_kernel(Args a) {
  constexpr int WM = TM / 2, WN = TN / 2;  // wave tile
  constexpr int FI = WM / 32, FJ = WN / 32;
  constexpr bool P_KC = (LAYOUT != MOE_GEMM_TN);  // P reduction-contiguous
  constexpr bool Q_KC = (LAYOUT == MOE_GEMM_NT);
  constexpr int PB = TM * BK * 2, QB = TN * BK * 2, SB = PB + QB;
  constexpr int LP = PB / 4096, LQ = QB / 4096;  // DMA instructions per wave per k-step
  constexpr int LT = LP + LQ;
  constexpr int PRB = TM * 2, QRB = TN * 2;       // row bytes of strided layouts
  constexpr int KRB = BK * 2;                     // row bytes of contiguous layouts
  constexpr int KCPR = KRB / 16;                  // 16-byte chunks per contiguous row

  __shared__ __attribute__((aligned(1024))) char smem[STAGES * SB];
  __shared__ int s_pref[256];
  __shared__ int scratch[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t N = a.N, K = a.K;

  // ---------------------------------------------------------------- tile
  int g;
  int64_t i_lo, i_hi, j0, r_lo = 0, r_hi, ncols;
  int split = 0;
  if (LAYOUT == MOE_GEMM_TN) {
    const int ti_n = (int)cdiv64(N, TM), tj_n = (int)cdiv64(K, TN);
    const int per_g = ti_n * tj_n;
    int L = xcd_remap(blockIdx.x, a.G * per_g * a.splits);
    split = L / (a.G * per_g);
    L -= split * (a.G * per_g);
    g = L / per_g;
    const int rem = L - g * per_g;
    const int ti = rem / tj_n, tj = rem - ti * tj_n;
    r_lo = group_row(a.offsets, g, a.M_total);
    r_hi = group_row(a.offsets, g + 1, a.M_total);
    if (a.splits > 1) {
      // slice `split` of the group's rows, in whole k-steps
      const int64_t chunk = cdiv64(cdiv64(r_hi - r_lo, a.splits), BK) * BK;
      const int64_t lo = r_lo + split * chunk;
      r_lo = lo < r_hi ? lo : r_hi;
      r_hi = lo + chunk < r_hi ? lo + chunk : r_hi;
    }
    i_lo = (int64_t)ti * TM;
    i_hi = i_lo + TM < N ? i_lo + TM : N;
    j0 = (int64_t)tj * TN;
    ncols = K;
  } else {
    int n = 0;
    if (tid < a.G) n = (group_row(a.offsets, tid + 1, a.M_total) - group_row(a.offsets, tid, a.M_total) + TM - 1) / TM;
    int mt_total;
    const int ex = block_exclusive_scan256(n, scratch, &mt_total);
    if (tid < a.G) s_pref[tid] = ex;
    __syncthreads();
    ncols = (LAYOUT == MOE_GEMM_NT) ? (EPI == MOE_EPI_SWIGLU ? N / 2 : N) : K;
    const int colw = (EPI == MOE_EPI_SWIGLU) ? TN / 2 : TN;
    const int tn_n = (int)cdiv64(ncols, colw);
    const int total = mt_total * tn_n;
    if ((int)blockIdx.x >= total) return;
    const int L = xcd_remap(blockIdx.x, total);
    // group of tile L: its tiles are [s_pref[g]*tn_n, s_pref[g+1]*tn_n)
    const int tguess = L / tn_n;
    int lo = 0, hi = a.G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= tguess) lo = mid; else hi = mid;
    }
    g = lo;
    // Inside a group, tiles run in blocks of NB column tiles x all row tiles,
    // so the workgroups resident on one XCD at a time share both the group's
    // rows and its weight columns in L2.
    const int mt = (g + 1 < a.G ? s_pref[g + 1] : mt_total) - s_pref[g];
    const int l = L - s_pref[g] * tn_n;
    int NB = kResident / mt;
    NB = NB < 1 ? 1 : (NB > tn_n ? tn_n : NB);
    const int blk = l / (mt * NB);
    const int nbw = (tn_n - blk * NB) < NB ? (tn_n - blk * NB) : NB;
    const int rem = l - blk * mt * NB;
    const int tm_local = rem / nbw;
    const int tn = blk * NB + (rem - tm_local * nbw);
    i_lo = group_row(a.offsets, g, a.M_total) + (int64_t)tm_local * TM;
    const int64_t gend = group_row(a.offsets, g + 1, a.M_total);
    i_hi = i_lo + TM < gend ? i_lo + TM : gend;
    j0 = (int64_t)tn * colw;
    r_hi = (LAYOUT == MOE_GEMM_NT) ? K : N;
  }
  const int64_t F = N / 2;
  const int64_t nk = (r_hi - r_lo + BK - 1) / BK;

  // ---------------------------------------------------------------- DMA plan
  // Instruction i of wave w fills LDS bytes [(i*4+w)*1024, +1024) of a region.
  // Reduction-contiguous region: 1024/KRB rows of KRB bytes; lane l -> row
  // (i*4+w)*(1024/KRB) + l/KCPR, LDS slot l%KCPR <- chunk slot ^ kc_swz(row).
  // Strided region [64][R]: k-row (i*4+w)*(1024/RB) + l/(RB/16), slot l%(RB/16)
  // <- source chunk slot ^ 4*(k-row % 4).  Source addresses are recomputed at
  // every issue from a few per-lane values, which keeps the register budget
  // for the accumulators.
  const char* Ab = (const char*)a.A;
  const char* Bb = (const char*)a.B;
  const int kc_row = lane / KCPR;                    // row within a 1 KB block
  constexpr int P_CPR = PRB / 16, Q_CPR = QRB / 16;
  const int p_kr = lane / P_CPR;                     // strided: k-row within a block
  const int q_kr = lane / Q_CPR;
  const int64_t pld = (LAYOUT == MOE_GEMM_NT) ? K : N;
  const int64_t rows_left0 = r_hi - r_lo;  // strided operands: valid reduction rows
  const uint32_t smem_base = lds_addr(smem);

  // k-row (within the k-step) that instruction i of this lane fills, strided layouts
  auto p_krow = [&](int i) __attribute__((always_inline)) { return (i * 4 + wave) * (1024 / PRB) + p_kr; };
  auto q_krow = [&](int i) __attribute__((always_inline)) { return (i * 4 + wave) * (1024 / QRB) + q_kr; };

  auto issue = [&](int64_t kt) __attribute__((always_inline)) {
    const uint32_t st = smem_base + (uint32_t)(kt % STAGES) * SB;
    const int64_t r0 = kt * BK;
#pragma unroll
    for (int i = 0; i < LP; ++i) {
      const char* src;
      if (P_KC) {
        const int row = (i * 4 + wave) * (1024 / KRB) + kc_row;
        const int chunk = (lane % KCPR) ^ kc_swz<BK>(row);
        int64_t m = i_lo + row;
        m = m < i_hi ? m : i_hi - 1;
        src = Ab + (m * pld + r0 + chunk * 8) * 2;
      } else {
        const int kr = p_krow(i);
        const int chunk = (lane % P_CPR) ^ tr_swz(kr);
        int64_t col = i_lo + chunk * 8;
        col = col < N - 8 ? col : N - 8;
        int64_t row = r0 + kr;
        row = r_lo + (row < rows_left0 ? row : rows_left0 - 1);
        src = Ab + (row * N + col) * 2;
      }
      dma16(src, __builtin_amdgcn_readfirstlane(st + (i * 4 + wave) * 1024));
    }
#pragma unroll
    for (int i = 0; i < LQ; ++i) {
      const char* src;
      if (Q_KC) {
        const int qr = (i * 4 + wave) * (1024 / KRB) + kc_row;
        const int chunk = (lane % KCPR) ^ kc_swz<BK>(qr);
        int64_t row;
        if (EPI == MOE_EPI_SWIGLU) {
          const int wq_ = qr / WN, jt = (qr % WN) / 32, jj = qr % 32;
          const int up = jt >= FJ / 2 ? 1 : 0;
          row = up * F + j0 + wq_ * (WN / 2) + (jt % (FJ / 2)) * 32 + jj;
        } else {
          row = j0 + qr;
          row = row < N ? row : N - 1;
        }
        src = Bb + (((int64_t)g * N + row) * K + r0 + chunk * 8) * 2;
      } else {
        const int kr = q_krow(i);
        const int chunk = (lane % Q_CPR) ^ tr_swz(kr);
        int64_t col = j0 + chunk * 8;
        col = col < K - 8 ? col : K - 8;
        int64_t row;
        if (LAYOUT == MOE_GEMM_NN) {
          row = (int64_t)g * N + r0 + kr;
        } else {
          row = r0 + kr;
          row = r_lo + (row < rows_left0 ? row : rows_left0 - 1);
        }
        src = Bb + (row * K + col) * 2;
      }
      dma16(src, __builtin_amdgcn_readfirstlane(st + PB + (i * 4 + wave) * 1024));
    }
  };

  // ---------------------------------------------------------------- main loop
  f32x16_t acc[FI][FJ];
#pragma unroll
  for (int it = 0; it < FI; ++it)
#pragma unroll
    for (int jt = 0; jt < FJ; ++jt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[it][jt][v] = 0.0f;

  const int wp = wave >> 1, wq = wave & 1;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s);
  for (int64_t kt = 0; kt < nk; ++kt) {
    // the k-steps issued after this one may stay in flight
    const int64_t later = (nk - 1 - kt) < (STAGES - 2) ? (nk - 1 - kt) : (STAGES - 2);
    if (later >= 2) wait_vmcnt<2 * LT>();
    else if (later == 1) wait_vmcnt<LT>();
    else wait_vmcnt<0>();
    char* stage = smem + (kt % STAGES) * SB;
    if (LAYOUT == MOE_GEMM_TN && (kt + 1) * BK > rows_left0) {
      // zero the reduction rows past the group end that this lane loaded
      const uint4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < LP; ++i)
        if (kt * BK + p_krow(i) >= rows_left0)
          *reinterpret_cast<uint4*>(stage + (i * 4 + wave) * 1024 + lane * 16) = z;
#pragma unroll
      for (int i = 0; i < LQ; ++i)
        if (kt * BK + q_krow(i) >= rows_left0)
          *reinterpret_cast<uint4*>(stage + PB + (i * 4 + wave) * 1024 + lane * 16) = z;
    }
    __syncthreads();
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
    const char* sP = stage;
    const char* sQ = stage + PB;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t pa[FI], qb[FJ];
#pragma unroll
      for (int it = 0; it < FI; ++it)
        pa[it] = P_KC ? frag_kc<BK>(sP, wp * WM + it * 32, ks, lane)
                      : frag_tr<PRB>(sP, wp * WM + it * 32, ks, lane);
#pragma unroll
      for (int jt = 0; jt < FJ; ++jt)
        qb[jt] = Q_KC ? frag_kc<BK>(sQ, wq * WN + jt * 32, ks, lane)
                      : frag_tr<QRB>(sQ, wq * WN + jt * 32, ks, lane);
#pragma unroll
      for (int it = 0; it < FI; ++it)
#pragma unroll
        for (int jt = 0; jt < FJ; ++jt)
          acc[it][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qb[jt], pa[it], acc[it][jt], 0, 0, 0);
    }
  }

  // ---------------------------------------------------------------- epilogue
  // lane holds output row (.. + lane%32) and, per 32-wide tile, 4 groups of 4
  // consecutive columns: (v/4)*8 + (lane/32)*4 + v%4
  const int r32 = lane & 31, kh = lane >> 5;
  bf16_t* C = a.C;
  bf16_t* X = a.aux;

  if constexpr (EPI == MOE_EPI_DSWIGLU) {
    // The pre-activations G|U of the wave's rows are brought into LDS with
    // full-row DMA (one 1 KB instruction per 1024/RBW rows) in two phases,
    // instead of per-lane 8-byte loads, then read in the accumulator layout.
    constexpr int RBW = WN * 2;          // bytes of one wave-tile row of G (or U)
    constexpr int CPW = RBW / 16;        // 16-byte chunks per row
    constexpr int RPI = 1024 / RBW;      // rows per DMA instruction
    constexpr int NI = 32 / RPI;         // instructions per 32-row block of G (or U)
    constexpr int WBUF = 16384;          // LDS bytes per wave
    constexpr int IPP = WBUF / (64 * RBW);  // 32-row blocks per phase
    static_assert(IPP >= 1 && FI % IPP == 0 && 4 * WBUF <= STAGES * SB, "epilogue staging");
    // slot of chunk c in row r: c ^ swz(r) (16 consecutive rows read at one
    // chunk hit distinct 16-byte bank groups)
    auto swz = [](int r) __attribute__((always_inline)) { return RBW >= 256 ? (r & 15) : ((r >> 1) & 7); };
    __syncthreads();  // every wave has finished reading the last k-step
    const char* wbuf = smem + wave * WBUF;
    const uint32_t wbase = smem_base + wave * WBUF;
    const int lrow = lane / CPW, lchunk = lane % CPW;
#pragma unroll
    for (int ph = 0; ph < FI / IPP; ++ph) {
      if (ph > 0) __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): reads of the buffer done
#pragma unroll
      for (int u = 0; u < IPP; ++u)
#pragma unroll
        for (int gu = 0; gu < 2; ++gu)
#pragma unroll
          for (int q = 0; q < NI; ++q) {
            const int r = q * RPI + lrow;
            int64_t i = i_lo + wp * WM + (ph * IPP + u) * 32 + r;
            i = i < i_hi ? i : i_hi - 1;
            int64_t col = j0 + wq * WN + (int64_t)((lchunk ^ swz(r)) * 8);
            col = col < K - 8 ? col : K - 8;
            dma16(X + i * 2 * K + gu * K + col,
                  __builtin_amdgcn_readfirstlane(wbase + ((u * 2 + gu) * NI + q) * 1024));
          }
      wait_vmcnt<0>();
#pragma unroll
      for (int u = 0; u < IPP; ++u) {
        const int it = ph * IPP + u;
        const int64_t i = i_lo + wp * WM + it * 32 + r32;
        const char* Gb = wbuf + (u * 2) * NI * 1024;
        const char* Ub = Gb + NI * 1024;
#pragma unroll
        for (int jt = 0; jt < FJ; ++jt) {
          const int64_t c = j0 + wq * WN + jt * 32;
          float dG[16], dU[16];
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int off = r32 * RBW + (((jt * 4 + gq) ^ swz(r32)) << 4) + kh * 8;
            const u32x2 gw = *reinterpret_cast<const u32x2*>(Gb + off);
            const u32x2 uw = *reinterpret_cast<const u32x2*>(Ub + off);
            const float Gv[4] = {bf16_lo(gw.x), bf16_hi(gw.x), bf16_lo(gw.y), bf16_hi(gw.y)};
            const float Uv[4] = {bf16_lo(uw.x), bf16_hi(uw.x), bf16_lo(uw.y), bf16_hi(uw.y)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float sg = sigmoid_f(Gv[e]);
              const float dh = acc[it][jt][gq * 4 + e];
              dG[gq * 4 + e] = dh * Uv[e] * sg * (1.0f + Gv[e] * (1.0f - sg));
              dU[gq * 4 + e] = dh * Gv[e] * sg;
            }
          }
          if (i < i_hi) {
            store_tile_row(C + i * 2 * K + c, dG, kh, ncols - c);
            store_tile_row(C + i * 2 * K + K + c, dU, kh, ncols - c);
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int it = 0; it < FI; ++it) {
    const int64_t i = i_lo + wp * WM + it * 32 + r32;
    if (i >= i_hi) continue;
    if (EPI == MOE_EPI_SWIGLU) {
#pragma unroll
      for (int jt = 0; jt < FJ / 2; ++jt) {
        const int64_t c = j0 + wq * (WN / 2) + jt * 32;
        float Gv[16], Uv[16], H[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          Gv[u] = acc[it][jt][u];
          Uv[u] = acc[it][jt + FJ / 2][u];
          H[u] = silu_f(Gv[u]) * Uv[u];
        }
        store_tile_row(C + i * F + c, H, kh, 32);
        if (X) {
          store_tile_row(X + i * N + c, Gv, kh, 32);
          store_tile_row(X + i * N + F + c, Uv, kh, 32);
        }
      }
      continue;
    }
#pragma unroll
    for (int jt = 0; jt < FJ; ++jt) {
      const int64_t c = j0 + wq * WN + jt * 32;
      const int64_t lim = ncols - c;  // columns left in the output row
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = acc[it][jt][u];
      if (LAYOUT == MOE_GEMM_TN) {
        if (a.splits > 1) {
          // fp32 partial of this row slice: 4 groups of 4 consecutive columns
          if (lim > 0) {
            float* prow = a.part + (((int64_t)split * a.G + g) * N + i) * K + c;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
              *reinterpret_cast<float4*>(prow + gq * 8 + kh * 4) =
                  make_float4(v[gq * 4], v[gq * 4 + 1], v[gq * 4 + 2], v[gq * 4 + 3]);
          }
        } else {
          store_tile_row(C + ((int64_t)g * N + i) * K + c, v, kh, lim);
        }
      } else {
        store_tile_row(C + i * ncols + c, v, kh, lim);
      }
    }
  }
}

template <int LAYOUT, int EPI, int TM, int TN, int BK, int STAGES, int OCC>
static hipError_t run(const Args& a, hipStream_t st) {
  int64_t nb;
  if (LAYOUT == MOE_GEMM_TN) {
    nb = a.G * cdiv64(a.N, TM) * cdiv64(a.K, TN) * a.splits;
  } else {
    const int64_t ncols = (LAYOUT == MOE_GEMM_NT) ? (EPI == MOE_EPI_SWIGLU ? a.N / 2 : a.N) : a.K;
    const int64_t colw = (EPI == MOE_EPI_SWIGLU) ? TN / 2 : TN;
    nb = (cdiv64(a.M_total, TM) + a.G) * cdiv64(ncols, colw);
  }
  if (nb == 0) return hipSuccess;
  gemm_kernel<LAYOUT, EPI, TM, TN, BK, STAGES, OCC><<<dim3((unsigned)nb), dim3(256), 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || LAYOUT != MOE_GEMM_TN || a.splits <= 1) return e;
  return launch_split_reduce(a.part, a.splits, (int64_t)a.G * a.N * a.K, a.C, MOE_BF16, st);
}

// 32-deep k-steps, 3 in flight: 72 KB of LDS and at most 256 registers per
// lane (128 fp32 accumulators), so two workgroups run on each CU and hide
// each other's barriers, DMA issue and epilogues.  Row tiles of the ragged
// dimension are 128 high (half the padding of 256) when the output width is a
// multiple of 256 (SwiGLU: the hidden width a multiple of 128); otherwise, and
// for weight gradients, 256 x 128.
template <int LAYOUT, int EPI>
static hipError_t pick(const Args& a, hipStream_t st) {
  if constexpr (LAYOUT != MOE_GEMM_TN) {
    bool wide;
    if (EPI == MOE_EPI_SWIGLU) wide = (a.N / 2) % 128 == 0;
    else if (LAYOUT == MOE_GEMM_NT) wide = a.N % 256 == 0;
    else wide = a.K % 256 == 0;
    if (wide) return run<LAYOUT, EPI, 128, 256, 32, 3, 2>(a, st);
  }
  return run<LAYOUT, EPI, 256, 128, 32, 3, 2>(a, st);
}

}  // namespace mf

// Compute units of an MI355X.  The slice count below is a host-side
// function of the problem only (no device query), so the workspace queries
// stay pure host arithmetic and always agree with the launch.
constexpr int kMi355xCUs = 256;

// Weight gradients whose output tiles alone cannot fill the chip (the shared
// experts: one group) split each group's rows into slices written as fp32
// partials and summed afterwards in slice order.  The slice count minimises a
// cost model measured on MI355X: the 256 x 128 workgroups run in rounds of two
// per CU, one 32-row k-step of such a round takes about 1 us, and each slice
// adds its fp32 partials, written once and read once at about 4.5 TB/s.
// Slices keep at least 512 rows.
int gemm_mfma_tn_splits(const GemmProblem& p) {
  if (p.layout != MOE_GEMM_TN || p.G <= 0) return 1;
  const int64_t tiles = p.G * cdiv64(p.N, 256) * cdiv64(p.K, 128);
  const int64_t slots = 2 * (int64_t)kMi355xCUs;
  const int64_t rows = p.M_total / p.G;
  const double slice_us = (double)p.G * (double)p.N * (double)p.K * 8.0 / 4.5e6;
  int best = 1;
  double best_us = 0.0;
  for (int s = 1; s <= 16; ++s) {
    if (s > 1 && rows / s < 512) break;
    const double us = (double)cdiv64(tiles * s, slots) * (double)cdiv64(cdiv64(rows, s), 32) +
                      (s > 1 ? s * slice_us : 0.0);
    if (s == 1 || us < best_us) {
      best = s;
      best_us = us;
    }
  }
  return best;
}

size_t gemm_mfma_workspace_bytes(const GemmProblem& p) {
  const int s = gemm_mfma_tn_splits(p);
  return s > 1 ? (size_t)s * p.G * p.N * p.K * sizeof(float) : 0;
}

hipError_t launch_gemm_mfma(const GemmProblem& p, void* ws, size_t ws_bytes, hipStream_t st) {
  mf::Args a;
  a.splits = gemm_mfma_tn_splits(p);
  a.part = (float*)ws;
  if (a.splits > 1 && (!ws || ws_bytes < gemm_mfma_workspace_bytes(p))) return hipErrorInvalidValue;
  a.G = (int)p.G;
  a.M_total = p.M_total;
  a.N = p.N;
  a.K = p.K;
  a.offsets = p.offsets;
  a.A = (const bf16_t*)p.A;
  a.B = (const bf16_t*)p.B;
  a.C = (bf16_t*)p.C;
  a.aux = (bf16_t*)p.aux;
  if (p.layout == MOE_GEMM_NT && p.epilogue == MOE_EPI_NONE) return mf::pick<MOE_GEMM_NT, MOE_EPI_NONE>(a, st);
  if (p.layout == MOE_GEMM_NT && p.epilogue == MOE_EPI_SWIGLU) return mf::pick<MOE_GEMM_NT, MOE_EPI_SWIGLU>(a, st);
  if (p.layout == MOE_GEMM_NN && p.epilogue == MOE_EPI_NONE) return mf::pick<MOE_GEMM_NN, MOE_EPI_NONE>(a, st);
  if (p.layout == MOE_GEMM_NN && p.epilogue == MOE_EPI_DSWIGLU) return mf::pick<MOE_GEMM_NN, MOE_EPI_DSWIGLU>(a, st);
  if (p.layout == MOE_GEMM_TN && p.epilogue == MOE_EPI_NONE) return mf::pick<MOE_GEMM_TN, MOE_EPI_NONE>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace moe
