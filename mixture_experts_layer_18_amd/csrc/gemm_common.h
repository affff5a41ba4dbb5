// Device helpers shared by the bf16 matrix-core GEMM kernels (gfx950):
// direct global->LDS DMA, wait counters, the XCD-aware tile remap, 16-byte
// epilogue stores from the 32x32 MFMA accumulator layout, and the LDS
// fragment reads for reduction-contiguous and reduction-strided tiles.
#pragma once

#include "kernels.h"

namespace moe {
namespace gk {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// One 16-byte-per-lane DMA from global memory into LDS at m0 + 16*lane.
MOE_DEV void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_base)
               : "memory", "m0");
}

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt left unconstrained)
template <int n>
MOE_DEV void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

MOE_DEV uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_char*)p; }

// Consecutive workgroup ids go to XCD 0,1,..,7,0,..; return the logical tile
// so that XCD x owns a contiguous block of the nb tiles.
MOE_DEV int xcd_remap(int bid, int nb) {
  const int q = nb >> 3, r = nb & 7;
  const int x = bid & 7, local = bid >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
}

// Store one 32-column MFMA tile row from its fp32 accumulator layout as
// 16-byte chunks.  Lane l (kh = l/32) holds columns gq*8 + kh*4 + 0..3 of
// groups gq = 0..3 (v[gq*4..+3]); lanes l and l+32 share the row.  For each
// pair of groups (2p, 2p+1), v_permlane32_swap trades lanes 32..63 of the
// packed group-2p values with lanes 0..31 of the packed group-2p+1 values:
// lane kh then holds the 8 consecutive columns of group 2p+kh in the pair
// (first register: columns +0..3, second: +4..7), with no per-lane select.
// `row` points at the tile's column 0 in the output row; columns at or past
// `lim` (relative to that point) are not written.
MOE_DEV void store_tile_row(bf16_t* row, const float* v, int kh, int64_t lim) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float* lo = v + 8 * p;
    const float* hi = v + 8 * p + 4;
    const auto r0 = __builtin_amdgcn_permlane32_swap(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(hi[0], hi[1]), false,
                                                     false);
    const auto r1 = __builtin_amdgcn_permlane32_swap(pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[2], hi[3]), false,
                                                     false);
    u32x4 o;
    o.x = r0[0]; o.y = r1[0]; o.z = r0[1]; o.w = r1[1];
    const int c = (2 * p + kh) * 8;
    if (c < lim) *reinterpret_cast<u32x4*>(row + c) = o;
  }
}

// ---- fragment reads (lane l: tile row l%32, reduction values (l/32)*8 .. +7)
// Swizzle of a reduction-contiguous tile with rows of 2*BK bytes: the 16-byte
// chunk c of row r sits at slot c ^ kc_swz(r).  16 consecutive rows read at
// the same chunk then cover all 16 bank groups of 256 bytes.
template <int BK>
MOE_DEV int kc_swz(int r) {
  return BK == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
template <int BK>
MOE_DEV bf16x8_t frag_kc(const char* region, int row, int ks, int lane) {
  const int r = row + (lane & 31);
  const int c = ks * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8_t*>(region + r * (2 * BK) + ((c ^ kc_swz<BK>(r)) << 4));
}
// Reduction-strided tile [BK][R] (row bytes RB): chunk c of k-row k sits at
// slot c ^ 4*(k%4); two transpose reads give k = base+0..3 and base+4..7.
MOE_DEV int tr_swz(int k) { return (k & 3) << 2; }
template <int RB>
MOE_DEV bf16x8_t frag_tr(const char* region, int row, int ks, int lane) {
  const int L = lane & 15, grp = lane >> 4;
  const int n = row + (grp & 1) * 16 + (L & 3) * 4;
  const int k1 = ks * 16 + (grp >> 1) * 8 + (L >> 2);
  const int k2 = k1 + 4;
  const int o1 = k1 * RB + (((n >> 3) ^ tr_swz(k1)) << 4) + (n & 7) * 2;
  const int o2 = k2 * RB + (((n >> 3) ^ tr_swz(k2)) << 4) + (n & 7) * 2;
  const s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(region + o1));
  const s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(region + o2));
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  const s16x8_t v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// DMA with a wave-uniform 64-bit base (SGPRs) and a 32-bit per-lane byte
// offset: global_load_lds_dwordx4 in its saddr form.
MOE_DEV void dma16_off(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}

// 4 bytes per lane from sbase + voff into LDS at m0 + 4*lane.
MOE_DEV void dma4_off(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}

// A 4-byte-per-lane DMA into a scratch LDS area: one vector-memory
// instruction that moves almost nothing, used where a fixed instruction count
// per step keeps the wait counts compile-time constants.
MOE_DEV void dma4_pad(const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, %2" ::"v"(0u), "s"(lds_base), "s"(sbase)
               : "memory", "m0");
}

// s_waitcnt lgkmcnt(0), then s_barrier: every wave's LDS reads and writes
// issued so far have completed.
MOE_DEV void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
}

// A copy of v the compiler cannot see through.  Reading accumulators through
// it keeps the register allocator from moving every MFMA accumulator into
// VGPRs when an epilogue combines two of them.
MOE_DEV float opaque(float v) {
  asm volatile("" : "+v"(v));
  return v;
}
// An accumulator value read with an explicit v_accvgpr_read: the value must
// stay in an AGPR until here, which keeps the allocator from moving all the
// accumulators into VGPRs for an epilogue that scales them.
MOE_DEV float agpr_read(float v) {
  float o;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(o) : "a"(v));
  return o;
}
MOE_DEV int opaque_i(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

}  // namespace gk
}  // namespace moe
