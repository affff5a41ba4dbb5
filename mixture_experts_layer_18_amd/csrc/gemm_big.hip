// Persistent bf16 grouped GEMM on gfx950 matrix cores with 256 x 256 tiles.
//
// Experts run as grouped GEMMs (Apex-3 code page, "What's inside", row
// "Fine-grained MoE"; Ultimate MoE Training Handbook, section 2.5).  This
// kernel covers the long products of the layer:
//   NT  C[m,n]   = sum_k A[m,k] B[g,n,k]        forward (+ SwiGLU epilogue)
//   NN  C[m,k]   = sum_n A[m,n] B[g,n,k]        data gradient
//   TN  C[g,n,k] = sum_{m in g} A[m,n] B[m,k]   weight gradient
//
// Why this shape (measured on MI355X):
//  * one workgroup per CU owning a 256 x 256 tile: the largest tile whose
//    fp32 accumulators fit the CU's registers, so the fewest operand bytes
//    per flop through the global->LDS DMA path and the LDS reads;
//  * 8 waves, two per SIMD, each owning 128 x 64 outputs (128 accumulators):
//    with one wave per SIMD (4 waves of 128 x 128) every DMA instruction
//    stalls that wave's MFMA issue for ~25 cycles (a probe: 32 MFMAs take
//    508 ns alone, 603 ns with 8 DMA instructions among them); with two
//    waves per SIMD one wave's DMA issue overlaps the other's MFMAs.  This
//    costs 1.5x the LDS fragment reads and measured 7-19 % faster per
//    product (TN most);
//  * four 32-deep LDS stages (128 KB), three in flight;
//  * one barrier per k-step, placed between its two 16-deep halves: before
//    it the wave runs the first half's MFMAs while the second half's
//    fragments arrive; after it, the next stage's first-half fragments are
//    requested and the second half's MFMAs run interleaved with the DMA
//    issue of the stage three steps ahead;
//  * every k-step issues the same number of vector-memory instructions
//    (past the end of the reduction, 4-byte pads into a scratch LDS area), so
//    every wait count is a constant and the loop body has one copy;
//  * persistent: workgroup w on XCD w%8 walks tiles L = n*W + (w%8)*(W/8) +
//    w/8, so the W/8 workgroups of one XCD work on neighbouring tiles (shared
//    A rows and B columns in that XCD's L2); the first stages of the next tile
//    are fetched before the current tile's epilogue or during it;
//  * results leave through LDS as whole 128-byte rows (staged in the last
//    stage slot, or, for dSwiGLU, over the G | U rows just read): stores of
//    32-byte pieces of 32 rows, the accumulator layout, stall the memory
//    pipeline far longer per kilobyte;
//  * DMA addresses are a wave-uniform tile base in SGPRs plus a 32-bit
//    per-lane offset recomputed at every issue (few live registers).
// Operands whose reduction dimension is contiguous (NT both, NN's A) sit in
// LDS as [256 rows][32] with 16-byte chunks XOR-swizzled by row; strided ones
// (NN's B, TN both) as [32][256] swizzled by k-row and are read with
// ds_read_b64_tr_b16 transposes.
//
// Gathered rows (GA): the operand indexed by the routed rows -- NT's A, TN's
// B -- is read through a row map from the un-permuted token matrix, so the
// permuted copy of the tokens is never written.  NT: each lane's four A rows
// are fixed for a tile; their byte offsets are loaded once per tile.  TN: the
// rows change every k-step; each wave DMAs the 32 map entries of stage s + 3
// into a small LDS ring together with stage s's operands, so the entries a
// DMA issue needs have landed (by the same wait) three steps before use.
#include "gemm_common.h"

namespace moe {
namespace pk {
using namespace gk;

constexpr int TM = 256, TN = 256, BK = 32, STAGES = 4;
constexpr int PB = TM * BK * 2, QB = TN * BK * 2, SB = PB + QB;
constexpr int KRB = BK * 2;                    // row bytes, reduction-contiguous layout
constexpr int SRB = TM * 2;                    // row bytes, reduction-strided layout
static_assert(TM == TN, "one strided row width");

// Wave layout of the 256 x 256 tile.  4 waves: 2 x 2 waves of 128 x 128
// (256 accumulators each, one wave per SIMD).  8 waves: 2 x 4 waves of
// 128 x 64 (128 accumulators, two waves per SIMD): a wave's DMA issue then
// overlaps the other wave's MFMAs, for 1.5x the LDS fragment reads; WIDE_:
// 4 x 2 waves of 64 x 128, the same accumulators and fragment reads.
template <int NW_, bool WIDE_ = false>
struct Waves {
  static constexpr int NW = NW_;
  static constexpr int WM = (NW_ == 8 && WIDE_) ? 64 : 128, WN = (NW_ == 4 || WIDE_) ? 128 : 64;
  static constexpr int WPR = TN / WN;          // waves along a tile row
  static constexpr int FI = WM / 32, FJ = WN / 32;
  static constexpr int LP = PB / (1024 * NW), LQ = QB / (1024 * NW), LT = LP + LQ;
  static constexpr int PAD_BYTES = LT * 256;   // scratch LDS for the 4-byte pads
  static_assert(NW_ == 4 || NW_ == 8, "4 or 8 waves");
  static_assert(WPR * (TM / WM) == NW, "waves cover the tile");
  static_assert((FI * FJ) % LT == 0, "MFMAs per DMA slot");
};

struct Args {
  int G;
  int64_t M_total, N, K;
  const int32_t* offsets;
  const bf16_t* A;
  const bf16_t* B;
  bf16_t* C;
  bf16_t* aux;
  const float* a_scale;  // fp8: per-row scales of A [M_total]
  const float* b_scale;  // fp8: per-row scales of B [G, N]
  const int32_t* rows;   // GA: source row of each routed row (NT: of A, TN: of B)
  int nslice;            // SL: row slices of the one group (C: fp32 partials [nslice, N, K])
};
constexpr int RING = 8;  // GA TN: map stages held per wave
template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// Exclusive prefix sum over the workgroup's threads (NW waves) of one value
// per thread; *total receives the sum.
template <int NW>
MOE_DEV int block_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int sv = scratch[w];
    if (w < wave) wbase += sv;
    tot += sv;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

struct Tile {
  int g;
  int64_t i_lo, i_hi;  // output rows (NT/NN: permuted rows of group g; TN: rows of C[g])
  int64_t j0;          // first output column
  int64_t r_lo, r_hi;  // reduction range (TN: the group's rows; else [0, K or N))
};

// F8: A and B hold OCP e4m3 codes (one byte each) with row scales; a k-step
// then covers 64 elements (still 64 bytes per LDS row) and one
// matrix-core product per 32x32 tile: the f8f6f4 builtin with zero scale
// operands, which the compiler emits as the unscaled
// v_mfma_f32_32x32x64_f8f6f4 (one instruction, no scale prefix).
// PF: the format of A's codes (P operand) in the fp8 products, FP8_E4M3 or
// FP8_E5M2 (the matrix cores take the operand formats as instruction fields);
// B's codes are e4m3.
// SL: a one-group weight gradient with too few output tiles to fill the chip
// runs as a.nslice equal row slices of the group (whole 32-row k-steps, the
// last slice ragged); slice s writes its fp32 sums to C[s] ([nslice, N, K]),
// which are added in slice order afterwards.
// MP: two weight gradients in one launch: b_in (one group over all tokens:
// the shared experts), whose few long tiles would leave CUs idle in a launch
// of their own, then a_in (the routed experts).  Every workgroup first walks
// b_in's tiles as in a launch of its own (lw, lw + W, ...); the workgroups
// without one in its last round then take R rounds of a_in's tiles, the
// tiles of largest groups, about one of b_in's tiles in k-steps; then every
// workgroup walks the rest of a_in's tiles.  With GA both gather their B rows
// (b_in's map may be the identity).
template <int LAYOUT, int EPI, bool F8, bool GA, int NWV, int PF = FP8_E4M3, bool SL = false, bool MP = false>
__global__ __launch_bounds__(64 * NWV, 1) void gemm_kernel(Args a_in, Args b_in) {
  // the forward gate/up product with gathered rows (bf16 and fp8): 64 x 128
  // wave tiles (64 hidden columns per wave, so that its SwiGLU results leave
  // as whole 128-byte rows; with the staged stores below, bf16 5 % faster
  // than 128 x 64)
  constexpr bool WIDE = (LAYOUT == MOE_GEMM_NT && EPI == MOE_EPI_SWIGLU && GA);
  using WV = Waves<NWV, WIDE>;
  constexpr int NW = WV::NW, WM = WV::WM, WN = WV::WN, WPR = WV::WPR, FI = WV::FI, FJ = WV::FJ;
  constexpr int LP = WV::LP, LQ = WV::LQ, LT = WV::LT, PAD_BYTES = WV::PAD_BYTES;
  // fp8 weight gradients (TN with F8) read both operands reduction-contiguous:
  // the padded, transposed group blocks of the column-wise quantiser
  constexpr bool W8 = F8 && LAYOUT == MOE_GEMM_TN;
  constexpr bool P_KC = (LAYOUT != MOE_GEMM_TN) || W8;
  constexpr bool Q_KC = (LAYOUT == MOE_GEMM_NT) || W8;
  static_assert(!F8 || LAYOUT != MOE_GEMM_NN, "fp8 operands: forward layout or weight gradient");
  static_assert(!W8 || (!GA && EPI == MOE_EPI_NONE), "fp8 weight gradient: plain");
  static_assert(!GA || LAYOUT != MOE_GEMM_NN, "gathered rows: NT or TN");
  static_assert(!GA || EPI != MOE_EPI_DSWIGLU, "gathered rows: no dSwiGLU epilogue");
  static_assert(!SL || (LAYOUT == MOE_GEMM_TN && !F8 && !GA), "row slices: bf16 weight gradient");
  static_assert(!MP || (LAYOUT == MOE_GEMM_TN && !F8 && !SL), "paired problems: bf16 weight gradients");
  constexpr bool GN = GA && LAYOUT == MOE_GEMM_NT;  // A rows gathered, fixed per tile
  constexpr bool GT = GA && LAYOUT == MOE_GEMM_TN;  // B k-rows gathered through the ring
  constexpr int LV = LT + (GT ? 1 : 0);             // vector-memory instructions per k-step
  constexpr int ES = F8 ? 1 : 2;         // bytes per operand element
  constexpr int BKE = BK * 2 / ES;       // elements per k-step (64 bytes per row)
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * SB + PAD_BYTES];
  __shared__ int s_pref[256];
  __shared__ int scratch_rows[LAYOUT == MOE_GEMM_TN ? 256 : 1];
  __shared__ int scratch[NW];
  __shared__ __attribute__((aligned(256))) int ring[GT ? NW * RING * 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: SGPR arithmetic
  const int nwg = gridDim.x, per = nwg >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int lw = xcd * per + slot;  // logical workgroup: XCD-contiguous

  // One walk over the tiles of problem a.  after_b (MP): a_in's walk, which
  // follows b_in's.
  auto walk = [&](const Args& a, const bool after_b) __attribute__((always_inline)) {
  const int64_t N = a.N, K = a.K;

  // ------------------------------------------------------------ tile table
  int total, tn_n, mt_total = 0;
  int64_t ncols;
  if (LAYOUT == MOE_GEMM_TN) {
    ncols = K;
    tn_n = (int)cdiv64(K, TN);
    total = (SL ? a.nslice : a.G) * (int)cdiv64(N, TM) * tn_n;
    if (!SL) {
      // Groups in order of decreasing row count (ties: lower index first), so
      // that the tiles of one round of the static walk reduce over similar
      // lengths: s_pref[rank] = group.  A weight-gradient tile costs its
      // group's rows, and experts' loads are ragged.
      if (tid < a.G) scratch_rows[tid] = group_row(a.offsets, tid + 1, a.M_total) - group_row(a.offsets, tid, a.M_total);
      __syncthreads();
      if (tid < a.G) {
        const int mine = scratch_rows[tid];
        int rank = 0;
        for (int h = 0; h < a.G; ++h) {
          const int o = scratch_rows[h];
          rank += (o > mine) || (o == mine && h < tid);
        }
        s_pref[rank] = tid;
      }
      __syncthreads();
    }
  } else {
    int n = 0;
    if (tid < a.G) n = (group_row(a.offsets, tid + 1, a.M_total) - group_row(a.offsets, tid, a.M_total) + TM - 1) / TM;
    const int ex = block_scan<NW>(n, scratch, &mt_total);
    if (tid < a.G) s_pref[tid] = ex;
    __syncthreads();
    ncols = (LAYOUT == MOE_GEMM_NT) ? (EPI == MOE_EPI_SWIGLU ? N / 2 : N) : K;
    const int colw = (EPI == MOE_EPI_SWIGLU) ? TN / 2 : TN;
    tn_n = (int)cdiv64(ncols, colw);
    total = mt_total * tn_n;
  }

  auto tile_of = [&](int L) __attribute__((always_inline)) {
    Tile t;
    if (LAYOUT == MOE_GEMM_TN) {
      const int per_g = (int)cdiv64(N, TM) * tn_n;
      const int gs = L / per_g, rem = L - gs * per_g;
      const int g = SL ? gs : s_pref[gs];
      const int ti = rem / tn_n, tj = rem - ti * tn_n;
      t.g = __builtin_amdgcn_readfirstlane(g);
      if constexpr (SL) {
        // slice g of the group's k-steps: kper whole steps each
        const int64_t r0 = group_row(a.offsets, 0, a.M_total), r1 = group_row(a.offsets, 1, a.M_total);
        const int64_t kper = cdiv64(cdiv64(r1 - r0, BK), a.nslice) * BK;
        const int64_t lo = r0 + t.g * kper, hi = lo + kper;
        t.r_lo = __builtin_amdgcn_readfirstlane((int)(lo < r1 ? lo : r1));
        t.r_hi = __builtin_amdgcn_readfirstlane((int)(hi < r1 ? hi : r1));
      } else {
        t.r_lo = __builtin_amdgcn_readfirstlane(group_row(a.offsets, t.g, a.M_total));
        t.r_hi = __builtin_amdgcn_readfirstlane(group_row(a.offsets, t.g + 1, a.M_total));
      }
      t.i_lo = (int64_t)__builtin_amdgcn_readfirstlane(ti) * TM;
      t.i_hi = t.i_lo + TM < N ? t.i_lo + TM : N;
      t.j0 = (int64_t)__builtin_amdgcn_readfirstlane(tj) * TN;
    } else {
      const int tguess = L / tn_n;
      int lo = 0, hi = a.G;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] <= tguess) lo = mid; else hi = mid;
      }
      const int g = lo;
      // inside a group: blocks of RB row tiles x NB column tiles (RB * NB
      // about `per`), so that the per workgroups of one XCD in one round
      // share RB row blocks of the group's rows and NB column blocks of its
      // weights.  A group of at most `per` row tiles is one row block (NB =
      // per / mt); a taller one (the shared experts: every token) takes
      // blocks of per / 4 row tiles x 4 column tiles.
      const int mt = (g + 1 < a.G ? s_pref[g + 1] : mt_total) - s_pref[g];
      const int l = L - s_pref[g] * tn_n;
      int RB = mt, NB = per / mt;
      if (mt > per) {
        NB = 4;
        RB = per / 4;
      }
      NB = NB < 1 ? 1 : (NB > tn_n ? tn_n : NB);
      RB = RB < 1 ? 1 : RB;
      const int rb = l / (RB * tn_n);
      const int rbh = (mt - rb * RB) < RB ? (mt - rb * RB) : RB;
      const int rem1 = l - rb * RB * tn_n;
      const int cb = rem1 / (rbh * NB);
      const int nbw = (tn_n - cb * NB) < NB ? (tn_n - cb * NB) : NB;
      const int rem2 = rem1 - cb * rbh * NB;
      const int tm_local = rb * RB + rem2 / nbw;
      const int tn = cb * NB + (rem2 - (rem2 / nbw) * nbw);
      t.g = __builtin_amdgcn_readfirstlane(g);
      const int glo = __builtin_amdgcn_readfirstlane(group_row(a.offsets, t.g, a.M_total));
      const int ghi = __builtin_amdgcn_readfirstlane(group_row(a.offsets, t.g + 1, a.M_total));
      t.i_lo = glo + (int64_t)__builtin_amdgcn_readfirstlane(tm_local) * TM;
      t.i_hi = t.i_lo + TM < ghi ? t.i_lo + TM : ghi;
      const int colw = (EPI == MOE_EPI_SWIGLU) ? TN / 2 : TN;
      t.j0 = (int64_t)__builtin_amdgcn_readfirstlane(tn) * colw;
      t.r_lo = 0;
      t.r_hi = (LAYOUT == MOE_GEMM_NT) ? K : N;
    }
    return t;
  };

  const char* Ab = (const char*)a.A;
  const char* Bb = (const char*)a.B;
  const uint32_t smem_base = lds_addr(smem);
  const uint32_t pad_lds = smem_base + STAGES * SB;
  const uint32_t ring_base = lds_addr(ring);
  const int64_t F = N / 2;

  // Instruction q (0..LT-1) of k-step kt of tile t: q < LP fills the P tile,
  // the rest the Q tile.  `ln` is the lane id (an opaque copy per call site).
  // gv: GN, the byte offsets of the lane's LP A rows; GT, the source rows of
  // the lane's LQ B k-rows of this k-step.
  auto issue = [&](const Tile& t, int64_t kt, int q, int ln, const uint32_t* gv) __attribute__((always_inline)) {
    const uint32_t st = smem_base + (uint32_t)(kt % STAGES) * SB;
    const bool isP = q < LP;
    const int i = isP ? q : q - LP;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(st + (isP ? 0 : PB) + (i * NW + wave) * 1024);
    if ((isP && P_KC) || (!isP && Q_KC)) {
      // [256 rows][32]: 16 rows of 64 bytes per instruction
      const int row = (i * NW + wave) * 16 + (ln >> 2);
      const int chunk = (ln & 3) ^ ((row >> 2) & 3);
      const uint32_t kb = (uint32_t)(kt * BK * 2) + chunk * 16;  // 64 bytes per row per k-step
      if (isP && GN) {
        dma16_off(Ab, gv[i] + kb, dst);
      } else if (isP && W8) {
        // group g's block of N rows of P'_g = r_hi - r_lo bytes at N * r_lo
        const int nrows = (int)(t.i_hi - t.i_lo);
        const int r = row < nrows ? row : nrows - 1;
        const int64_t pg = t.r_hi - t.r_lo;
        dma16_off(Ab + N * t.r_lo + t.i_lo * pg, (uint32_t)r * (uint32_t)pg + kb, dst);
      } else if (isP) {
        const int nrows = (int)(t.i_hi - t.i_lo);
        const int r = row < nrows ? row : nrows - 1;
        const int64_t ld = (LAYOUT == MOE_GEMM_NT) ? K : N;
        dma16_off(Ab + t.i_lo * ld * ES, (uint32_t)r * (uint32_t)(ld * ES) + kb, dst);
      } else if (W8) {  // the weight gradient's B' rows (K per group)
        const int nr = (int)(K - t.j0);
        const int r = row < nr ? row : nr - 1;
        const int64_t pg = t.r_hi - t.r_lo;
        dma16_off(Bb + K * t.r_lo + t.j0 * pg, (uint32_t)r * (uint32_t)pg + kb, dst);
      } else {  // NT's B rows
        uint32_t roff;
        if (EPI == MOE_EPI_SWIGLU) {
          // wave tile columns in 32-wide blocks: gate, up, gate, up
          const int wq_ = row / WN, jt = (row % WN) / 32, jj = row % 32;
          roff = (uint32_t)((jt & 1) * F) + wq_ * (WN / 2) + (jt >> 1) * 32 + jj;
        } else {
          const int nr = (int)(N - t.j0);
          roff = row < nr ? row : nr - 1;
        }
        dma16_off(Bb + ((int64_t)t.g * N + t.j0) * K * ES, roff * (uint32_t)(K * ES) + kb, dst);
      }
    } else {
      // [32][256]: 2 k-rows of 512 bytes per instruction
      const int kr = (i * NW + wave) * 2 + (ln >> 5);
      const int chunk = (ln & 31) ^ ((kr & 3) << 2);
      if (LAYOUT == MOE_GEMM_NN) {  // B[g, n, k]: k-row n, columns k
        int64_t col = t.j0 + chunk * 8;
        col = col < K - 8 ? col : K - 8;
        const uint32_t off = (uint32_t)((kt * BK + kr) * K + col) * 2;
        dma16_off(Bb + (int64_t)t.g * N * K * 2, off, dst);
      } else {  // TN: A[m, n] or B[m, k], rows of the group
        const int64_t ld = isP ? N : K;
        const int64_t c0 = isP ? t.i_lo : t.j0;
        int64_t col = c0 + chunk * 8;
        col = col < ld - 8 ? col : ld - 8;
        if (GT && !isP) {
          dma16_off(Bb, (gv[i] * (uint32_t)ld + (uint32_t)col) * 2u, dst);
        } else {
          const int64_t rows = t.r_hi - t.r_lo;
          int64_t r = kt * BK + kr;
          r = r < rows ? r : rows - 1;
          dma16_off((isP ? Ab : Bb) + t.r_lo * ld * 2, (uint32_t)(r * ld + col) * 2, dst);
        }
      }
    }
  };
  // TN: zero the rows of k-step kt past the group end that this lane loaded
  // (called after the lane's own DMA for kt completed, before the barrier)
  auto zero_tail = [&](const Tile& t, int64_t kt) __attribute__((always_inline)) {
    if (LAYOUT != MOE_GEMM_TN || W8) return;  // W8: the padding holds zero codes
    const int64_t rows = t.r_hi - t.r_lo;
    if ((kt + 1) * BK <= rows) return;
    char* st = smem + (kt % STAGES) * SB;
    const uint4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < LT; ++q) {
      const int i = q < LP ? q : q - LP;
      const int kr = (i * NW + wave) * 2 + (lane >> 5);
      if (kt * BK + kr >= rows)
        *reinterpret_cast<uint4*>(st + (q < LP ? 0 : PB) + (i * NW + wave) * 1024 + lane * 16) = z;
    }
  };
  // GT: the map entries of k-step s (32 rows, clamped to the group) into ring
  // slot s % RING of this wave; past the reduction a pad
  auto ring_dma = [&](const Tile& t, int64_t s, int64_t nk, int ln) __attribute__((always_inline)) {
    if (s < nk) {
      const int64_t rows = t.r_hi - t.r_lo;
      int64_t r = s * BK + (ln & 31);
      r = r < rows ? r : rows - 1;
      dma4_off(a.rows + t.r_lo, (uint32_t)r * 4u,
               __builtin_amdgcn_readfirstlane(ring_base + (wave * RING + (int)(s % RING)) * 256));
    } else {
      dma4_pad(Ab, pad_lds);
    }
  };
  // GN: byte offsets of the lane's A rows in tile t
  auto row_offsets = [&](const Tile& t, uint32_t* ao, int ln) __attribute__((always_inline)) {
    const int nrows = (int)(t.i_hi - t.i_lo);
#pragma unroll
    for (int i = 0; i < LP; ++i) {
      const int row = (i * NW + wave) * 16 + (ln >> 2);
      const int r = row < nrows ? row : nrows - 1;
      ao[i] = (uint32_t)a.rows[t.i_lo + r] * (uint32_t)(K * ES);
    }
  };
  // GT: source rows of the lane's B k-rows of k-step s, read directly
  auto direct_rows = [&](const Tile& t, int64_t s, uint32_t* gr, int ln) __attribute__((always_inline)) {
    const int64_t rows = t.r_hi - t.r_lo;
#pragma unroll
    for (int i = 0; i < LQ; ++i) {
      const int kr = (i * NW + wave) * 2 + (ln >> 5);
      int64_t r = s * BK + kr;
      r = r < rows ? r : rows - 1;
      gr[i] = rows > 0 ? (uint32_t)a.rows[t.r_lo + r] : 0u;
    }
  };
  // one k-step's operand DMA (GT: preceded by the map entries of k-step s+3)
  auto stage_dma = [&](const Tile& t, int64_t s, int64_t nk, int ln, const uint32_t* gv)
                       __attribute__((always_inline)) {
    if constexpr (GT) {
      ring_dma(t, s + 3, nk, ln);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < LT; ++q) {
      if (s < nk) issue(t, s, q, ln, gv);
      else dma4_pad(Ab, pad_lds + q * 256);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the first STAGES k-steps of tile t (GN: ao holds its row offsets; GT:
  // gr the source rows of its first STAGES k-steps)
  auto prologue = [&](const Tile& t, int64_t nk, int ln, const uint32_t* ao, const uint32_t (*gr)[LQ], int s0,
                      int s1) __attribute__((always_inline)) {
    if constexpr (GT) {
#pragma unroll
      for (int s = 0; s < STAGES; ++s)
        if (s >= s0 && s < s1) stage_dma(t, s, nk, ln, gr[s]);
    } else {
#pragma unroll
      for (int s = 0; s < STAGES; ++s)
        if (s >= s0 && s < s1) stage_dma(t, s, nk, ln, ao);
    }
  };

  auto frag_p = [&](const char* st, int it, int ks) __attribute__((always_inline)) {
    const int row = (wave / WPR) * WM + it * 32;
    return P_KC ? frag_kc<BK>(st, row, ks, lane) : frag_tr<SRB>(st, row, ks, lane);
  };
  auto frag_q = [&](const char* st, int jt, int ks) __attribute__((always_inline)) {
    const int row = (wave % WPR) * WN + jt * 32;
    return Q_KC ? frag_kc<BK>(st + PB, row, ks, lane) : frag_tr<SRB>(st + PB, row, ks, lane);
  };

  const int wp = wave / WPR, wq = wave % WPR;
  const int r32 = lane & 31, kh = lane >> 5;
  // dSwiGLU epilogue staging.  A wave's G (or U) rows of one 32-row block of
  // its outputs form a piece of E_NI 1 KB DMA instructions (E_RPI rows of
  // E_RBW bytes each, 16-byte chunks XOR-swizzled by row).  Piece j (0..3)
  // of a wave sits in LDS stage slot j at the wave's offset; the k-loop's
  // last four steps, which would issue pads, request pieces 0..3 (blocks 0
  // and 1, G then U), each into the slot its step frees (step kt frees slot
  // kt % 4).  Blocks 0 and 2 thus use slots 0 and 1, which the next tile's
  // first two stages take once block 2 is done.
  constexpr int E_RBW = WN * 2, E_CPW = E_RBW / 16, E_RPI = 1024 / E_RBW, E_NI = 32 / E_RPI;
  constexpr int E_WB = E_NI * 1024;  // bytes of one piece
  static_assert(EPI != MOE_EPI_DSWIGLU || (E_NI == LT && NW * E_WB == SB && FI == 4 && WN == 64), "epilogue pieces");
  auto e_swz = [](int r) __attribute__((always_inline)) { return E_RBW >= 256 ? (r & 15) : ((r >> 1) & 7); };
  auto e_piece = [&](int j) __attribute__((always_inline)) {
    return (uint32_t)j * SB + (uint32_t)(wave * E_WB);
  };
  // instruction q of piece j holding 32-row block blk of G (j even) or U
  auto epi_dma = [&](const Tile& t, int j, int blk, int q, int ln) __attribute__((always_inline)) {
    const int r = q * E_RPI + ln / E_CPW;
    const int rl = (int)(t.i_hi - t.i_lo) - 1;
    int ri = wp * WM + blk * 32 + r;
    ri = ri < rl ? ri : rl;
    int64_t col = t.j0 + wq * WN + (int64_t)(((ln % E_CPW) ^ e_swz(r)) * 8);
    col = col < ncols - 8 ? col : ncols - 8;
    const int64_t K2 = 2 * ncols;
    const uint32_t voff = (uint32_t)(((int64_t)ri * K2 + (j & 1) * ncols + col) * 2);
    dma16_off(a.aux + t.i_lo * K2, voff,
              __builtin_amdgcn_readfirstlane(smem_base + e_piece(j) + (uint32_t)(q * 1024)));
  };
  // this workgroup's k-th tile of the walk (false past its end)
  int r0 = 0, R = 0;
  if (MP && after_b) {
    // b_in's last round left workgroups r0.. without a tile: they first take
    // R rounds of this walk's tiles (largest groups first), the number whose
    // k-steps come closest to one of b_in's tiles (k-steps plus about 6 for
    // the epilogue)
    constexpr int EPI_K = 6;
    const int n0 = (int)(cdiv64(b_in.N, TM) * cdiv64(b_in.K, TN));
    r0 = n0 % nwg;
    if (r0 > 0) {
      const int64_t hc =
          cdiv64(group_row(b_in.offsets, 1, b_in.M_total) - group_row(b_in.offsets, 0, b_in.M_total), BK) + EPI_K;
      const int per_g = (int)cdiv64(N, TM) * tn_n;
      int64_t sum = 0;
      while (R < 256) {
        const int Lr = R * (nwg - r0);
        if (Lr >= total) break;
        const int64_t c = cdiv64(scratch_rows[s_pref[Lr / per_g]], BK) + EPI_K;
        if (sum + c / 2 > hc) break;
        sum += c;
        ++R;
      }
    }
  }
  // Weight gradients (tiles in order of decreasing cost): the XCDs take the
  // slices of a round in serpentine order (XCD x slice x in even rounds,
  // slice 7 - x in odd ones), so that no XCD always gets the dearest slice.
  auto lw_of = [&](int round) __attribute__((always_inline)) {
    if constexpr (LAYOUT == MOE_GEMM_TN && !SL) return ((round & 1) ? 7 - xcd : xcd) * per + slot;
    return lw;
  };
  auto item = [&](int k, int& L) __attribute__((always_inline)) -> bool {
    if (MP && after_b && r0 > 0) {
      const int p1 = lw >= r0 ? R : 0;
      if (k < p1) {
        L = (lw - r0) + k * (nwg - r0);
        return L < total;
      }
      L = R * (nwg - r0) + (k - p1) * nwg + lw_of(k - p1);
      return L < total;
    }
    L = lw_of(k) + k * nwg;
    return L < total;
  };
  int kk = 0, L = 0;
  if (!item(0, L)) return;
  Tile t = tile_of(L);
  int64_t nk = (t.r_hi - t.r_lo + BKE - 1) / BKE;
  uint32_t aoff[LP];
#pragma unroll
  for (int i = 0; i < LP; ++i) aoff[i] = 0u;
  {
    const int ln = opaque_i(lane);
    uint32_t gr[STAGES][LQ];
    if constexpr (GN) row_offsets(t, aoff, ln);
    if constexpr (GT)
#pragma unroll
      for (int s = 0; s < STAGES; ++s) direct_rows(t, s, gr[s], ln);
    prologue(t, nk, ln, aoff, gr, 0, STAGES);
  }

  // STG: the results leave through LDS as whole 128-byte rows, staged in
  // the last stage slot; the next tile's last stage is requested after this
  // tile's stores (the forward gate/up product with gathered rows and every
  // plain product but the one-group row slices and the fp8 weight
  // gradients; measured 1-11 % faster each)
  constexpr bool STG = WIDE || (!W8 && !SL && EPI == MOE_EPI_NONE);
  while (true) {
    // this tile's first stages are complete (STG: all but the last, which
    // was requested last: the vector-memory counter counts loads, LDS DMAs
    // and stores together, and they complete in issue order)
    // (dSwiGLU: all but the last two, requested after the previous tile's
    // last block)
    if constexpr (STG) wait_vmcnt<LV>();
    else if constexpr (EPI == MOE_EPI_DSWIGLU) wait_vmcnt<2 * LV>();
    else wait_vmcnt<0>();
    if (nk > 0) zero_tail(t, 0);
    lds_barrier();
    // GA: the next tile's row map is loaded now, so that it has arrived by
    // the time the next tile's first stages are issued
    int Ln = 0;
    const bool more = item(kk + 1, Ln);
    Tile tn = t;
    int64_t nk_n = 0;
    uint32_t aoff_n[LP];
#pragma unroll
    for (int i = 0; i < LP; ++i) aoff_n[i] = 0u;
    uint32_t gr_n[STAGES][LQ];
    if (GA && more) {
      tn = tile_of(Ln);
      nk_n = (tn.r_hi - tn.r_lo + BKE - 1) / BKE;
      const int lp = opaque_i(lane);
      if constexpr (GN) row_offsets(tn, aoff_n, lp);
      if constexpr (GT)
#pragma unroll
        for (int s = 0; s < STAGES; ++s) direct_rows(tn, s, gr_n[s], lp);
    }
    f32x16_t acc[FI][FJ];
#pragma unroll
    for (int it = 0; it < FI; ++it)
#pragma unroll
      for (int jt = 0; jt < FJ; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[it][jt][v] = 0.0f;
    // A wave whose outputs are all padding (the rows past a group's end in
    // its last row tile, the columns past the end in a last column tile)
    // runs the k-loop without fragment reads or MFMAs: the DMA issue and the
    // barriers only.  Its accumulators stay zero and are never stored, and
    // the other wave on its SIMD has the matrix core to itself.
    const int colw_w = (EPI == MOE_EPI_SWIGLU) ? WN / 2 : WN;
    const bool wact = __builtin_amdgcn_readfirstlane(
        (int)(wp * WM < t.i_hi - t.i_lo && (int64_t)wq * colw_w < ncols - t.j0));
    auto kloop = [&](auto act) __attribute__((always_inline)) {
    constexpr bool ACT = decltype(act)::value;
    if constexpr (F8) {
      // Both 32-byte halves of a lane's row fragment feed one MFMA, so a
      // k-step cannot be split in reduction halves as in the bf16 loop; it is
      // split in row blocks instead.  Entering step kt, Q (all column blocks)
      // and P[0..1] of stage kt are in registers.  The step reads P[2..3] of
      // stage kt while the MFMAs of row blocks 0..1 run, waits and passes
      // the barrier, requests Q and P[0..1] of stage kt+1, then runs the
      // MFMAs of row blocks 2..3 interleaved with the DMA issue.
      typedef int v4i_t __attribute__((ext_vector_type(4)));
      typedef int v8i_t __attribute__((ext_vector_type(8)));
      auto frag8 = [&](const char* st, int row) __attribute__((always_inline)) {
        const v4i_t lo = __builtin_bit_cast(v4i_t, frag_kc<BK>(st, row, 0, lane));
        const v4i_t hi = __builtin_bit_cast(v4i_t, frag_kc<BK>(st, row, 1, lane));
        return (v8i_t)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      constexpr int FH = FI / 2;
      v8i_t P[FH], Q[FJ];
      if constexpr (ACT) {
#pragma unroll
        for (int it = 0; it < FH; ++it) P[it] = frag8(smem, wp * WM + it * 32);
#pragma unroll
        for (int jt = 0; jt < FJ; ++jt) Q[jt] = frag8(smem + PB, wq * WN + jt * 32);
      }
      const int ln = opaque_i(lane);
      for (int64_t kt = 0; kt < nk; ++kt) {
        const char* sP = smem + (kt % STAGES) * SB;
        v8i_t P2[FH];
        if constexpr (ACT) {
#pragma unroll
          for (int it = 0; it < FH; ++it) P2[it] = frag8(sP, wp * WM + (FH + it) * 32);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ACT) {
#pragma unroll
          for (int it = 0; it < FH; ++it)
#pragma unroll
            for (int jt = 0; jt < FJ; ++jt)
              acc[it][jt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Q[jt], P[it], acc[it][jt], FP8_E4M3,
                                                                            PF, 0, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // k-step kt+1 landed for this wave; after the barrier every wave has
        // it and none reads stage kt from LDS any more
        wait_vmcnt<2 * LV>();
        lds_barrier();
        const char* nP = smem + ((kt + 1) % STAGES) * SB;
        v8i_t Pn[FH], Qn[FJ];
        if constexpr (ACT) {
#pragma unroll
          for (int jt = 0; jt < FJ; ++jt) Qn[jt] = frag8(nP + PB, wq * WN + jt * 32);
#pragma unroll
          for (int it = 0; it < FH; ++it) Pn[it] = frag8(nP, wp * WM + it * 32);
        }
        __builtin_amdgcn_sched_barrier(0);
        const bool real = kt + STAGES < nk;
        static_assert(FH * FJ == LT, "one MFMA per DMA slot");
#pragma unroll
        for (int q = 0; q < LT; ++q) {
          const int it = q / FJ, jt = q % FJ;
          if constexpr (ACT)
            acc[FH + it][jt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                Q[jt], P2[it], acc[FH + it][jt], FP8_E4M3, PF, 0, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          if (real) issue(t, kt + STAGES, q, ln, aoff);
          else if constexpr (EPI == MOE_EPI_DSWIGLU) epi_dma(t, (int)(kt % STAGES), (int)(kt % STAGES) >> 1, q, ln);
          else dma4_pad(Ab, pad_lds + q * 256);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (ACT) {
#pragma unroll
          for (int it = 0; it < FH; ++it) P[it] = Pn[it];
#pragma unroll
          for (int jt = 0; jt < FJ; ++jt) Q[jt] = Qn[jt];
        }
      }
    } else {
    bf16x8_t pa0[FI], qb0[FJ], pa1[FI], qb1[FJ];
      if constexpr (ACT) {
  #pragma unroll
        for (int it = 0; it < FI; ++it) pa0[it] = frag_p(smem, it, 0);
  #pragma unroll
        for (int jt = 0; jt < FJ; ++jt) qb0[jt] = frag_q(smem, jt, 0);
      }
      const int ln = opaque_i(lane);
      for (int64_t kt = 0; kt < nk; ++kt) {
        const char* sP = smem + (kt % STAGES) * SB;
        if constexpr (ACT) {
  #pragma unroll
          for (int it = 0; it < FI; ++it) pa1[it] = frag_p(sP, it, 1);
  #pragma unroll
          for (int jt = 0; jt < FJ; ++jt) qb1[jt] = frag_q(sP, jt, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ACT) {
  #pragma unroll
          for (int it = 0; it < FI; ++it)
  #pragma unroll
            for (int jt = 0; jt < FJ; ++jt)
              acc[it][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qb0[jt], pa0[it], acc[it][jt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // k-step kt+1 landed for this wave (kt+2, kt+3 may be in flight); after
        // the barrier every wave has it and is done reading k-step kt
        wait_vmcnt<2 * LV>();
        if (kt + 1 < nk) zero_tail(t, kt + 1);
        // GT: the map entries of k-step kt + STAGES landed with k-step kt + 1;
        // read before the barrier, whose LDS wait then covers them (after it
        // the 4-bit LDS counter could not single them out from the fragment
        // reads that follow)
        uint32_t gq[LQ];
        if constexpr (GT) {
          const int* rs = ring + (wave * RING + (int)((kt + STAGES) % RING)) * 64;
#pragma unroll
          for (int i = 0; i < LQ; ++i) gq[i] = (uint32_t)rs[(i * NW + wave) * 2 + (lane >> 5)];
        }
        lds_barrier();
        const char* nP = smem + ((kt + 1) % STAGES) * SB;
        if constexpr (ACT) {
  #pragma unroll
          for (int it = 0; it < FI; ++it) pa0[it] = frag_p(nP, it, 0);
  #pragma unroll
          for (int jt = 0; jt < FJ; ++jt) qb0[jt] = frag_q(nP, jt, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        const bool real = kt + STAGES < nk;
  #pragma unroll
        for (int q = 0; q < LT; ++q) {
  #pragma unroll
          for (int u = 0; u < (FI * FJ) / LT; ++u) {
            const int m = q * ((FI * FJ) / LT) + u, it = m / FJ, jt = m % FJ;
            if constexpr (ACT)
              acc[it][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qb1[jt], pa1[it], acc[it][jt], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (real) issue(t, kt + STAGES, q, ln, GT ? gq : aoff);
          else if constexpr (EPI == MOE_EPI_DSWIGLU) epi_dma(t, (int)(kt % STAGES), (int)(kt % STAGES) >> 1, q, ln);
          else dma4_pad(Ab, pad_lds + q * 256);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (GT) {
          ring_dma(t, kt + STAGES + 3, nk, ln);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    };
    if (wact) kloop(Flag<true>{});
    else kloop(Flag<false>{});
    // every wave is done with this tile's LDS stages: fetch the next tile's
    // first stages, then write this tile's results
    lds_barrier();
    // the next tile's stages s0 .. s1 - 1 (s0 = 0: its tile is found first)
    auto prefetch_next = [&](int s0, int s1) __attribute__((always_inline)) {
      if (more) {
        if constexpr (!GA) {
          if (s0 == 0) {
            tn = tile_of(Ln);
            nk_n = (tn.r_hi - tn.r_lo + BKE - 1) / BKE;
          }
        }
        const int lp = opaque_i(lane);
        prologue(tn, nk_n, lp, aoff_n, gr_n, s0, s1);
      }
    };

    // -------------------------------------------------------- epilogue
    bf16_t* C = a.C;
    bf16_t* X = a.aux;
    // fp8: the row scale of this lane's output row per row block, and the
    // column scales of the 16 columns a lane holds in a 32-wide block
    // (columns at or past N, never stored, read the last four scales: a
    // last column tile narrower than 256 stays inside b_scale)
    auto col_scales = [&](int64_t brow, float* sc) __attribute__((always_inline)) {
      // (W8: the output's columns are K per group)
      const int64_t NC = W8 ? K : N;
      const float* p = a.b_scale + (int64_t)t.g * NC;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        int64_t cidx = brow + kh * 4 + gq * 8;
        cidx = cidx < NC - 4 ? cidx : NC - 4;
        const float4 v = *reinterpret_cast<const float4*>(p + cidx);
        sc[gq * 4] = v.x; sc[gq * 4 + 1] = v.y; sc[gq * 4 + 2] = v.z; sc[gq * 4 + 3] = v.w;
      }
    };
    // fp8: the scale of output row i's source (GN: a token row, per token);
    // rows past the tile (never stored) read the last row's
    auto row_scale = [&](int64_t i) __attribute__((always_inline)) {
      i = i < t.i_hi ? i : t.i_hi - 1;
      return a.a_scale[GN ? (int64_t)a.rows[i] : i];
    };
    if constexpr (EPI == MOE_EPI_DSWIGLU) {
      // Data gradient through SwiGLU (NN bf16, or NT fp8 with the weight
      // stored transposed): the product is dH (fp8: times the row and column
      // scales); aux holds the forward pre-activations G | U ([M, 2W] for
      // output width W); C receives
      // dG = dH U silu'(G) | dU = dH silu(G).  Each wave brings the G and U
      // rows of its outputs into four 4 KB pieces of the LDS stages with
      // full-row DMA (two 32-row blocks at a time) and reads them in the
      // accumulator layout; the next tile's first stages are fetched after.
      // Pieces 0..3 (blocks 0 and 1) were requested by the k-loop's last
      // four steps; with fewer k-steps the missing ones are requested now.
      // Block b: each lane reads its G and U values, computes dG and dU and
      // writes them over the bytes it read; the wave then reads the block
      // back by whole rows and stores them as full 128-byte rows (the
      // accumulator layout would store 32-byte pieces of 32 rows, measured
      // 3-10 % slower); then (b < 2) block b + 2 is requested into the same
      // two pieces, its loads overlapping the stores of block b + 1; after
      // block 2 the next tile's first two stages are requested into its
      // slots, after block 3 the other two.
      const int ln = opaque_i(lane);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j >= nk)
#pragma unroll
          for (int q = 0; q < E_NI; ++q) epi_dma(t, j, j >> 1, q, ln);
      wait_vmcnt<0>();
#pragma unroll
      for (int it = 0; it < FI; ++it) {
        const int j0 = 2 * (it & 1);
        char* Gw = smem + e_piece(j0);
        char* Uw = smem + e_piece(j0 + 1);
        const int64_t i = t.i_lo + wp * WM + it * 32 + r32;
        // fp8: the row's scale (padding rows, never stored, read the last row's)
        const float sa = F8 ? a.a_scale[i < t.i_hi ? i : t.i_hi - 1] : 1.0f;
        const int64_t K2 = 2 * ncols;
#pragma unroll
        for (int jt = 0; jt < FJ; ++jt) {
          const int64_t c = t.j0 + wq * WN + jt * 32;
          float dG[16], dU[16], sc[16];
          if constexpr (F8) col_scales(c, sc);
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int off = r32 * E_RBW + (((jt * 4 + gq) ^ e_swz(r32)) << 4) + kh * 8;
            const u32x2 g2 = *reinterpret_cast<const u32x2*>(Gw + off);
            const u32x2 u2 = *reinterpret_cast<const u32x2*>(Uw + off);
            const float Gv[4] = {bf16_lo(g2.x), bf16_hi(g2.x), bf16_lo(g2.y), bf16_hi(g2.y)};
            const float Uv[4] = {bf16_lo(u2.x), bf16_hi(u2.x), bf16_lo(u2.y), bf16_hi(u2.y)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float sg = sigmoid_f(Gv[e]);
              const float dh = F8 ? agpr_read(acc[it][jt][gq * 4 + e]) * sa * sc[gq * 4 + e]
                                  : acc[it][jt][gq * 4 + e];
              dG[gq * 4 + e] = dh * Uv[e] * sg * (1.0f + Gv[e] * (1.0f - sg));
              dU[gq * 4 + e] = dh * Gv[e] * sg;
            }
          }
          // the lanes overwrite the G and U chunks they have just read (rows
          // 16..31 with their two 8-byte halves swapped)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int off = r32 * E_RBW + (((jt * 4 + gq) ^ e_swz(r32)) << 4) + ((kh ^ (r32 >> 4)) << 3);
            const u32x2 pg = {pack_bf16x2(dG[gq * 4], dG[gq * 4 + 1]), pack_bf16x2(dG[gq * 4 + 2], dG[gq * 4 + 3])};
            const u32x2 pu = {pack_bf16x2(dU[gq * 4], dU[gq * 4 + 1]), pack_bf16x2(dU[gq * 4 + 2], dU[gq * 4 + 3])};
            *reinterpret_cast<u32x2*>(Gw + off) = pg;
            *reinterpret_cast<u32x2*>(Uw + off) = pu;
          }
        }
        // the block's dG and dU rows leave as whole 128-byte rows: 8 lanes per row
        __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS writes are done
        {
          const int lr = lane >> 3, lc = lane & 7;
#pragma unroll
          for (int q = 0; q < 32 / 8; ++q) {
            const int r = q * 8 + lr;
            const int off = r * E_RBW + ((lc ^ e_swz(r)) << 4);
            u32x4 vg = *reinterpret_cast<const u32x4*>(Gw + off);
            u32x4 vu = *reinterpret_cast<const u32x4*>(Uw + off);
            if (q >= 2) {
              vg = u32x4{vg.z, vg.w, vg.x, vg.y};
              vu = u32x4{vu.z, vu.w, vu.x, vu.y};
            }
            const int64_t ir = t.i_lo + wp * WM + it * 32 + r;
            const int64_t cc = t.j0 + wq * WN + lc * 8;
            if (ir < t.i_hi && cc < ncols) {
              *reinterpret_cast<u32x4*>(C + ir * K2 + cc) = vg;
              *reinterpret_cast<u32x4*>(C + ir * K2 + ncols + cc) = vu;
            }
          }
        }
        if (it < 2) {
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the pieces are read back
#pragma unroll
          for (int gu = 0; gu < 2; ++gu)
#pragma unroll
            for (int q = 0; q < E_NI; ++q) epi_dma(t, j0 + gu, it + 2, q, ln);
        }
        // blocks 2 and 3 have landed (with the stores before them)
        if (it == 1) wait_vmcnt<0>();
        // every wave is done with slots 0 and 1 (block 2) or 2 and 3 (block
        // 3): the next tile's stages into them
        if (it >= 2) {
          lds_barrier();
          prefetch_next(it == 2 ? 0 : 2, it == 2 ? 2 : 4);
        }
      }
      if (!more) break;
      L = Ln;
      ++kk;
      t = tn;
      nk = nk_n;
#pragma unroll
      for (int i = 0; i < LP; ++i) aoff[i] = aoff_n[i];
      continue;
    }
    prefetch_next(0, STG ? STAGES - 1 : STAGES);
    if constexpr (STG) {
      // Each wave stages every 32-row block of its results in its own 4 KB
      // of the last stage slot (64 columns: the plain products' 64 x 2 blocks
      // of 32; SwiGLU with 64 x 128 wave tiles: the gate pre-activations, the
      // up ones, then h, 64 hidden columns each) and stores them as whole
      // 128-byte rows, 8 rows per instruction (the accumulator layout would
      // store 32-byte pieces of 32 rows); the next tile's last stage follows.
      static_assert(WN == (WIDE ? 128 : 64) && NW * 4096 <= SB, "result staging");
      char* wb = smem + (STAGES - 1) * SB + wave * 4096;
      // 16-byte chunk c of row r at slot c ^ sw(r); plain products: rows
      // 16..31 with the chunk's two 8-byte halves swapped, meant to spread
      // the 32 lanes of a half-wave over more banks (measured 6-9 % faster on
      // the data gradients, 4-7 % slower on the SwiGLU product)
      auto sw = [](int r) __attribute__((always_inline)) { return (r >> 1) & 7; };
      auto hs = [](int r) __attribute__((always_inline)) { return WIDE ? 0 : (r >> 4); };
      auto stage = [&](const float* v, int jb) __attribute__((always_inline)) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const u32x2 pk = {pack_bf16x2(v[gq * 4], v[gq * 4 + 1]), pack_bf16x2(v[gq * 4 + 2], v[gq * 4 + 3])};
          *reinterpret_cast<u32x2*>(wb + r32 * 128 + (((jb * 4 + gq) ^ sw(r32)) << 4) + ((kh ^ hs(r32)) << 3)) = pk;
        }
      };
      // rows i0 .. i0 + 31 of the block (those below t.i_hi), columns
      // base + 0 .. cw - 1 (cw a multiple of 8)
      auto flush = [&](bf16_t* base, int64_t ld, int64_t i0, int64_t cw) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS writes are done
        const int lr = lane >> 3, lc = lane & 7;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = q * 8 + lr;
          u32x4 val = *reinterpret_cast<const u32x4*>(wb + r * 128 + ((lc ^ sw(r)) << 4));
          if (!WIDE && q >= 2) val = u32x4{val.z, val.w, val.x, val.y};  // rows 16..31: halves swapped
          if (i0 + r < t.i_hi && lc * 8 < cw) *reinterpret_cast<u32x4*>(base + (i0 + r) * ld + lc * 8) = val;
        }
      };
      if constexpr (!WIDE) {
        // plain results (forward down, data and weight gradients): 64
        // columns per wave
        const int64_t c0 = t.j0 + wq * WN;
        bf16_t* base = (LAYOUT == MOE_GEMM_TN) ? C + (int64_t)t.g * N * K + c0 : C + c0;
        if (c0 < ncols) {
#pragma unroll
          for (int it = 0; it < FI; ++it) {
            const int64_t i0 = t.i_lo + wp * WM + it * 32;
            if (i0 >= t.i_hi) continue;
            const float sa = F8 ? row_scale(i0 + r32) : 1.0f;
#pragma unroll
            for (int jt = 0; jt < FJ; ++jt) {
              float v[16];
              if constexpr (F8) {
                float sc[16];
                col_scales(c0 + jt * 32, sc);
#pragma unroll
                for (int u = 0; u < 16; ++u) v[u] = agpr_read(acc[it][jt][u]) * sa * sc[u];
              } else {
#pragma unroll
                for (int u = 0; u < 16; ++u) v[u] = acc[it][jt][u];
              }
              stage(v, jt);
            }
            flush(base, ncols, i0, ncols - c0);
          }
        }
      }
      const int64_t cg = t.j0 + wq * (WN / 2);
#pragma unroll
      for (int it = 0; it < FI && WIDE; ++it) {
        const int64_t i0 = t.i_lo + wp * WM + it * 32;
        if (i0 >= t.i_hi) continue;
        const float sa = F8 ? row_scale(i0 + r32) : 1.0f;
        float v[16];
        if (X) {
#pragma unroll
          for (int gu = 0; gu < 2; ++gu) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
              for (int u = 0; u < 16; ++u) v[u] = opaque(acc[it][2 * jb + gu][u]);
              if constexpr (F8) {
                float sc[16];
                col_scales(gu * F + cg + jb * 32, sc);
#pragma unroll
                for (int u = 0; u < 16; ++u) v[u] = v[u] * sa * sc[u];
              }
              stage(v, jb);
            }
            flush(X + gu * F + cg, N, i0, 64);
          }
        }
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          if constexpr (F8) {
            float sg[16], su[16];
            col_scales(cg + jb * 32, sg);
            col_scales(F + cg + jb * 32, su);
#pragma unroll
            for (int u = 0; u < 16; ++u)
              v[u] = silu_f(opaque(acc[it][2 * jb][u]) * sa * sg[u]) * (opaque(acc[it][2 * jb + 1][u]) * sa * su[u]);
          } else {
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = silu_f(opaque(acc[it][2 * jb][u])) * opaque(acc[it][2 * jb + 1][u]);
          }
          stage(v, jb);
        }
        flush(C + cg, F, i0, 64);
      }
      lds_barrier();  // every wave is done with the last slot
      prefetch_next(STAGES - 1, STAGES);
      if (!more) break;
      L = Ln;
      ++kk;
      t = tn;
      nk = nk_n;
#pragma unroll
      for (int i = 0; i < LP; ++i) aoff[i] = aoff_n[i];
      continue;
    }
#pragma unroll
    for (int it = 0; it < FI; ++it) {
      __builtin_amdgcn_sched_barrier(0);
      const int64_t i = t.i_lo + wp * WM + it * 32 + r32;
      if (i >= t.i_hi) continue;
      // fp8: the scale of the row's source (GN: a token row, per token; W8:
      // per group and output row)
      const float sa = F8 ? a.a_scale[GN ? (int64_t)a.rows[i] : (W8 ? (int64_t)t.g * N + i : i)] : 1.0f;
      if (EPI == MOE_EPI_SWIGLU) {
        // block jt holds gate columns for even jt, up columns for odd jt
        if (X) {
#pragma unroll
          for (int jt = 0; jt < FJ; ++jt) {
            const int64_t c = (jt & 1) * F + t.j0 + wq * (WN / 2) + (jt >> 1) * 32;
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = opaque(acc[it][jt][u]);
            if constexpr (F8) {
              float sc[16];
              col_scales(c, sc);
#pragma unroll
              for (int u = 0; u < 16; ++u) v[u] = v[u] * sa * sc[u];
            }
            store_tile_row(X + i * N + c, v, kh, 32);
          }
        }
#pragma unroll
        for (int jt = 0; jt < FJ / 2; ++jt) {
          const int64_t c = t.j0 + wq * (WN / 2) + jt * 32;
          float h[16];
          if constexpr (F8) {
            float sg[16], su[16];
            col_scales(c, sg);
            col_scales(F + c, su);
#pragma unroll
            for (int u = 0; u < 16; ++u)
              h[u] = silu_f(opaque(acc[it][2 * jt][u]) * sa * sg[u]) * (opaque(acc[it][2 * jt + 1][u]) * sa * su[u]);
          } else {
#pragma unroll
            for (int u = 0; u < 16; ++u)
              h[u] = silu_f(opaque(acc[it][2 * jt][u])) * opaque(acc[it][2 * jt + 1][u]);
          }
          store_tile_row(C + i * F + c, h, kh, 32);
        }
      } else {
#pragma unroll
        for (int jt = 0; jt < FJ; ++jt) {
          const int64_t c = t.j0 + wq * WN + jt * 32;
          float v[16];
          if constexpr (F8) {
            float sc[16];
            col_scales(c, sc);
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = agpr_read(acc[it][jt][u]) * sa * sc[u];
          } else {
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = acc[it][jt][u];
          }
          if constexpr (SL) {
            // fp32 partial of slice t.g: lane kh holds columns gq*8 + kh*4 .. +3
            float* prow = reinterpret_cast<float*>(a.C) + ((int64_t)t.g * N + i) * K + c;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int cc = gq * 8 + kh * 4;
              if (c + cc < K)
                *reinterpret_cast<float4*>(prow + cc) =
                    make_float4(v[gq * 4], v[gq * 4 + 1], v[gq * 4 + 2], v[gq * 4 + 3]);
            }
            continue;
          }
          bf16_t* row = (LAYOUT == MOE_GEMM_TN) ? C + ((int64_t)t.g * N + i) * K : C + i * ncols;
          store_tile_row(row + c, v, kh, ncols - c);
        }
      }
    }
    if (!more) break;
    L = Ln;
    ++kk;
    t = tn;
    nk = nk_n;
#pragma unroll
    for (int i = 0; i < LP; ++i) aoff[i] = aoff_n[i];
  }
  };  // walk

  if constexpr (MP) {
    // b_in's walk, then a_in's, through one copy of the walk's code (two
    // inlined copies spilled more)
#pragma clang loop unroll(disable)
    for (int p = 0; p < 2; ++p) {
      if (p == 1) __syncthreads();  // the tile table is rebuilt for a_in
      walk(p == 0 ? b_in : a_in, p == 1);
    }
  } else {
    walk(a_in, false);
  }
}

// p[i] = i for i < n: the identity row map
__global__ __launch_bounds__(256) void iota_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = (int32_t)i;
}

// Workgroups of the persistent grid: one per CU.
static int grid_size() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    n = (cus + 7) / 8 * 8;
  }
  return n;
}

// waves per workgroup (Waves<4> is the one-wave-per-SIMD layout it replaced)
constexpr int kWaves = 8;
template <int LAYOUT, int EPI, bool F8 = false, bool GA = false, int NWV = kWaves, int PF = FP8_E4M3,
          bool SL = false>
static hipError_t run(const Args& a, hipStream_t st) {
  if (a.G == 0 || a.N == 0 || a.K == 0) return hipSuccess;
  gemm_kernel<LAYOUT, EPI, F8, GA, NWV, PF, SL><<<dim3((unsigned)grid_size()), dim3(64 * NWV), 0, st>>>(a, a);
  return hipGetLastError();
}
// two weight gradients in one launch (b: one group, walked first)
template <bool GA>
static hipError_t run_pair(const Args& a, const Args& b, hipStream_t st) {
  gemm_kernel<MOE_GEMM_TN, MOE_EPI_NONE, false, GA, kWaves, FP8_E4M3, false, true>
      <<<dim3((unsigned)grid_size()), dim3(64 * kWaves), 0, st>>>(a, b);
  return hipGetLastError();
}

}  // namespace pk

// A one-group weight gradient (shared experts) with fewer than 1024 output
// tiles: the number of equal row slices that gives at least 128 tiles (half
// the CUs) with every slice at least 32 k-steps long, 1 when the tiles alone
// reach 128; 0 when no such split exists (the two-workgroup kernel takes it).
// Measured on the 7B-style layer's shared experts: 176 tiles unsliced ran
// 18 % faster than the two-workgroup kernel's row slices, 88 tiles unsliced
// 50 % slower.
static int one_group_slices(const GemmProblem& p) {
  const int64_t tiles = cdiv64(p.N, 256) * cdiv64(p.K, 256);
  const int64_t ks = cdiv64(p.M_total, 32);
  int s = 1;
  while (tiles * s < 128 && s < 8 && ks >= 2 * s * 32) s *= 2;
  return tiles * s >= 128 ? s : 0;
}

// Which products this kernel takes (the rest go to the two-workgroup kernel):
// NT with either epilogue (SwiGLU: the hidden width a multiple of 128, so that
// a tile pairs 128 gate with 128 up columns), the plain data gradient, and the
// weight gradient when it has enough 256 x 256 tiles to fill the chip without
// row slices (gathered rows: any tile count), or is one group that row slices
// of its own bring to 128 tiles.
//
// Operand DMA offsets are 32-bit byte offsets from a per-tile base: NT's
// SwiGLU weight rows span one expert's whole [N, K] block (gate and up
// halves), NN's strided weight likewise, and TN's operands one group's rows.
// Products whose offsets could pass 2^32 bytes go to the two-workgroup kernel
// (64-bit addresses).
bool gemm_big_supported(const GemmProblem& p) {
  if (p.ta != MOE_BF16 || p.tb != MOE_BF16 || p.tc != MOE_BF16 || p.G > 256) return false;
  if (p.rows && p.layout == MOE_GEMM_NN) return false;
  const int64_t lim = int64_t(1) << 32;
  if (p.layout == MOE_GEMM_NT) {
    if (p.epilogue == MOE_EPI_SWIGLU) return (p.N / 2) % 128 == 0 && p.N * p.K * 2 <= lim;
    return p.epilogue == MOE_EPI_NONE;
  }
  if (p.layout == MOE_GEMM_TN) {
    // few tiles: row slices on the two-workgroup kernel fill the chip better,
    // but gathered rows are read by this kernel only.  A partial last column
    // tile (K not a multiple of 256) is clamped on load and masked on store.
    // Gathered rows: the row map's offsets are bounded by the caller's token
    // count (src_rows * K * 2 <= 2^32, checked where the map is accepted);
    // the group's own rows (A) by M_total * N * 2.
    if (p.M_total * p.N * 2 > lim) return false;
    if (p.rows) return p.K % 256 == 0;
    if (p.M_total * p.K * 2 > lim) return false;
    if (p.G * cdiv64(p.N, 256) * cdiv64(p.K, 256) >= 4 * 256) return true;
    return p.G == 1 && p.N % 8 == 0 && p.K % 8 == 0 && one_group_slices(p) > 0;
  }
  // (dSwiGLU: a tile's G | U rows are addressed with 32-bit offsets from
  // its first row, 256 rows of 2K values)
  if (p.layout == MOE_GEMM_NN)
    return (p.epilogue == MOE_EPI_NONE || (p.epilogue == MOE_EPI_DSWIGLU && p.K <= (int64_t(1) << 21))) &&
           p.N * p.K * 2 <= lim;
  return false;
}

size_t gemm_big_workspace_bytes(const GemmProblem& p) {
  if (p.layout != MOE_GEMM_TN || p.rows || p.G != 1 || p.G * cdiv64(p.N, 256) * cdiv64(p.K, 256) >= 4 * 256)
    return 0;
  const int s = one_group_slices(p);
  return s > 1 ? (size_t)s * p.N * p.K * sizeof(float) : 0;
}

// Two weight gradients in one launch: `routed` (many groups, on this kernel
// without row slices) and `one` (one group of bf16 rows whose operands have
// 32-bit offsets; with a row map exactly when `routed` has one).
bool gemm_big_pair_supported(const GemmProblem& routed, const GemmProblem& one) {
  if (routed.layout != MOE_GEMM_TN || one.layout != MOE_GEMM_TN) return false;
  if (routed.epilogue != MOE_EPI_NONE || one.epilogue != MOE_EPI_NONE) return false;
  if (!gemm_big_supported(routed) || gemm_big_workspace_bytes(routed) != 0) return false;
  if (one.G != 1 || (one.rows != nullptr) != (routed.rows != nullptr)) return false;
  if (one.ta != MOE_BF16 || one.tb != MOE_BF16 || one.tc != MOE_BF16) return false;
  const int64_t lim = int64_t(1) << 32;
  return one.M_total > 0 && one.N >= 8 && one.K >= 8 && one.N % 8 == 0 && one.K % 8 == 0 &&
         one.M_total * one.N * 2 <= lim && one.M_total * one.K * 2 <= lim;
}

static pk::Args big_args(const GemmProblem& p) {
  pk::Args a;
  a.G = (int)p.G;
  a.M_total = p.M_total;
  a.N = p.N;
  a.K = p.K;
  a.offsets = p.offsets;
  a.A = (const bf16_t*)p.A;
  a.B = (const bf16_t*)p.B;
  a.C = (bf16_t*)p.C;
  a.aux = (bf16_t*)p.aux;
  a.a_scale = a.b_scale = nullptr;
  a.rows = p.rows;
  a.nslice = 1;
  return a;
}

hipError_t launch_gemm_big_pair(const GemmProblem& routed, const GemmProblem& one, hipStream_t st) {
  if (!gemm_big_pair_supported(routed, one)) return hipErrorInvalidValue;
  const pk::Args a = big_args(routed), b = big_args(one);
  return routed.rows ? pk::run_pair<true>(a, b, st) : pk::run_pair<false>(a, b, st);
}

hipError_t launch_iota(int32_t* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  pk::iota_kernel<<<dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, st>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_gemm_big(const GemmProblem& p, void* ws, size_t ws_bytes, hipStream_t st) {
  pk::Args a;
  a.G = (int)p.G;
  a.M_total = p.M_total;
  a.N = p.N;
  a.K = p.K;
  a.offsets = p.offsets;
  a.A = (const bf16_t*)p.A;
  a.B = (const bf16_t*)p.B;
  a.C = (bf16_t*)p.C;
  a.aux = (bf16_t*)p.aux;
  a.a_scale = a.b_scale = nullptr;
  a.rows = p.rows;
  a.nslice = 1;
  if (const size_t wsb = gemm_big_workspace_bytes(p)) {
    // one group in row slices: fp32 partials in the workspace, summed in
    // slice order into C
    if (!ws || ws_bytes < wsb) return hipErrorInvalidValue;
    a.nslice = one_group_slices(p);
    a.C = (bf16_t*)ws;
    hipError_t e = pk::run<MOE_GEMM_TN, MOE_EPI_NONE, false, false, pk::kWaves, FP8_E4M3, true>(a, st);
    if (e != hipSuccess) return e;
    return launch_split_reduce((const float*)ws, a.nslice, p.N * p.K, p.C, MOE_BF16, st);
  }
  if (p.rows) {
    if (p.layout == MOE_GEMM_NT && p.epilogue == MOE_EPI_NONE)
      return pk::run<MOE_GEMM_NT, MOE_EPI_NONE, false, true>(a, st);
    if (p.layout == MOE_GEMM_NT && p.epilogue == MOE_EPI_SWIGLU)
      return pk::run<MOE_GEMM_NT, MOE_EPI_SWIGLU, false, true>(a, st);
    if (p.layout == MOE_GEMM_TN && p.epilogue == MOE_EPI_NONE)
      return pk::run<MOE_GEMM_TN, MOE_EPI_NONE, false, true>(a, st);
    return hipErrorInvalidValue;
  }
  if (p.layout == MOE_GEMM_NT && p.epilogue == MOE_EPI_NONE) return pk::run<MOE_GEMM_NT, MOE_EPI_NONE>(a, st);
  if (p.layout == MOE_GEMM_NT && p.epilogue == MOE_EPI_SWIGLU) return pk::run<MOE_GEMM_NT, MOE_EPI_SWIGLU>(a, st);
  if (p.layout == MOE_GEMM_NN && p.epilogue == MOE_EPI_NONE) return pk::run<MOE_GEMM_NN, MOE_EPI_NONE>(a, st);
  if (p.layout == MOE_GEMM_NN && p.epilogue == MOE_EPI_DSWIGLU)
    return pk::run<MOE_GEMM_NN, MOE_EPI_DSWIGLU>(a, st);
  if (p.layout == MOE_GEMM_TN && p.epilogue == MOE_EPI_NONE) return pk::run<MOE_GEMM_TN, MOE_EPI_NONE>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace moe

namespace moe {
// fp8 forward products: C (bf16) = a_scale[m] b_scale[g,n] sum_k A[m,k] B[g,n,k];
// with rows, A's row m and its scale are read at rows[m] (plain and SwiGLU
// epilogues)
hipError_t launch_gemm_fp8(int epilogue, int64_t G, int64_t M_total, int64_t N, int64_t K,
                           const int32_t* offsets, const uint8_t* A, const float* a_scale,
                           const uint8_t* B, const float* b_scale, void* C, void* aux,
                           const int32_t* rows, hipStream_t st, int a_fmt) {
  pk::Args a;
  a.G = (int)G;
  a.M_total = M_total;
  a.N = N;
  a.K = K;
  a.offsets = offsets;
  a.A = (const bf16_t*)A;
  a.B = (const bf16_t*)B;
  a.C = (bf16_t*)C;
  a.aux = (bf16_t*)aux;
  a.a_scale = a_scale;
  a.b_scale = b_scale;
  a.rows = rows;
  a.nslice = 1;
  if (a_fmt == FP8_E5M2) {
    // e5m2 A codes: the data gradients' gradient operands
    if (rows) return hipErrorInvalidValue;
    if (epilogue == MOE_EPI_NONE) return pk::run<MOE_GEMM_NT, MOE_EPI_NONE, true, false, pk::kWaves, FP8_E5M2>(a, st);
    if (epilogue == MOE_EPI_DSWIGLU)
      return pk::run<MOE_GEMM_NT, MOE_EPI_DSWIGLU, true, false, pk::kWaves, FP8_E5M2>(a, st);
    return hipErrorInvalidValue;
  }
  if (rows) {
    if (epilogue == MOE_EPI_NONE) return pk::run<MOE_GEMM_NT, MOE_EPI_NONE, true, true>(a, st);
    if (epilogue == MOE_EPI_SWIGLU) return pk::run<MOE_GEMM_NT, MOE_EPI_SWIGLU, true, true>(a, st);
    return hipErrorInvalidValue;
  }
  if (epilogue == MOE_EPI_NONE) return pk::run<MOE_GEMM_NT, MOE_EPI_NONE, true>(a, st);
  if (epilogue == MOE_EPI_SWIGLU) return pk::run<MOE_GEMM_NT, MOE_EPI_SWIGLU, true>(a, st);
  if (epilogue == MOE_EPI_DSWIGLU) return pk::run<MOE_GEMM_NT, MOE_EPI_DSWIGLU, true>(a, st);
  return hipErrorInvalidValue;
}

// fp8 weight gradient over the padded group blocks (pad_off: the padded group
// offsets, which set each group's reduction range and block base)
hipError_t launch_gemm_fp8_wgrad(int64_t G, int64_t N, int64_t K, const int32_t* pad_off, const uint8_t* A,
                                 const float* a_scale, const uint8_t* B, const float* b_scale, void* C,
                                 hipStream_t st) {
  pk::Args a;
  a.G = (int)G;
  a.M_total = 0;
  a.N = N;
  a.K = K;
  a.offsets = pad_off;
  a.A = (const bf16_t*)A;
  a.B = (const bf16_t*)B;
  a.C = (bf16_t*)C;
  a.aux = nullptr;
  a.a_scale = a_scale;
  a.b_scale = b_scale;
  a.rows = nullptr;
  a.nslice = 1;
  return pk::run<MOE_GEMM_TN, MOE_EPI_NONE, true>(a, st);
}
}  // namespace moe
