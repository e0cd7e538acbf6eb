// tile_io.hpp — K/V tile staging for the prefill kernels: LDS tile geometry and the
// asynchronous global->LDS copy of one 64-key tile, shared by the dense and block-sparse
// forward kernels.
//
// LDS layout of one tile (keys 0..63 of the tile):
//  * K: MFMA-operand order. Slab (kb, s) (1 KiB) holds, for lane l, the 16 bytes of key row
//    32*kb + l%32 at head-dim chunk 2s + l/32, which is exactly the A operand of 32x32x16 k-step
//    s for key block kb. Every K-operand read is then a linear ds_read_b128, the LDS read
//    pattern that reaches full bandwidth.
//  * V: row-major, rows padded to 2D+64 bytes, which keeps the transposed V read (8 rows x 64
//    bytes per instruction) conflict-free. Padding slots receive a duplicate of the row's
//    first chunk and are never read.
// Every copy instruction moves 1 KiB (64 lanes x 16 bytes) and lands contiguously in LDS.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int BN = 64;                 // keys per tile

template <int N>
using ic = std::integral_constant<int, N>;

template <int D>
struct TileCfg {
  static constexpr int CPR = D / 8;                   // 16-byte chunks of data per row
  static constexpr int KSTEPS = D / 16;               // 32x32x16 MFMA steps over the head dim
  static constexpr int KSLABS = 2 * KSTEPS;           // K tile: 1 KiB operand slabs
  static constexpr int VROW = 2 * D + 64;             // padded V row (bytes)
  static constexpr int VSPR = VROW / 16;              // 16-byte slots per V row
  static constexpr int KT_BYTES = KSLABS * 1024;
  static constexpr int VT_BYTES = BN * VROW;
  static constexpr int STAGE_BYTES = KT_BYTES + VT_BYTES;
  static constexpr int KINSTR = KSLABS;               // 1 KiB copy instructions per K tile
  static constexpr int VINSTR = VT_BYTES / 1024;
  static constexpr int DVB = D / 32;                  // 32-wide output column blocks
  static_assert(VT_BYTES % 1024 == 0, "whole KiB tiles");
};

// K slab (kb, s) holds, for lane l, the 16 bytes of key row 32*kb + l%32 at head-dim chunk
// 2s + l/32: exactly the A operand of k-step s for key block kb, read linearly.
template <int D>
__device__ __forceinline__ void kslab_rc(int i, int l, uint32_t& r, uint32_t& c) {
  r = 32u * (uint32_t)(i / TileCfg<D>::KSTEPS) + (uint32_t)(l & 31);
  c = 2u * (uint32_t)(i % TileCfg<D>::KSTEPS) + (uint32_t)(l >> 5);
}

// Row r and chunk c that copy slot `slot` of a padded tile holds (padding slots duplicate
// chunk 0 of their row).
template <int SPR, int CPR>
__device__ __forceinline__ void slot_rc(uint32_t slot, uint32_t& r, uint32_t& c) {
  r = slot / SPR;
  const uint32_t cs = slot % SPR;
  c = cs < (uint32_t)CPR ? cs : 0u;
}

// vmcnt(0) in a form the compiler sees: afterwards it knows that every earlier load of the
// wave has completed and adds no waits of its own for those loads (it does not see the copies,
// so a wait it adds for an older register load would also drain the copies in flight).
__device__ __forceinline__ void wait_vmcnt_visible0() {
  // gfx9 encoding: vmcnt 0 (bits 3:0 and 15:14), expcnt and lgkmcnt at their maxima
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without a memory fence (the copies it orders are waited for explicitly).
__device__ __forceinline__ void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }

// Scalar-base tile copies. Wave w of NW issues the K copy instructions w, w+NW, ... and the V
// copy instructions w, w+NW, ... (KINSTR and VINSTR are multiples of NW), so which tensor an
// instruction reads is fixed at compile time. `ko` / `vo` hold the lane's byte offsets
// relative to the tile's first key row; maxrow < 63 describes a ragged last tile (rows past
// maxrow re-read row maxrow, so every copy stays inside the sequence). The K and V offsets are
// set separately because a K tile and a V tile of one LDS stage may belong to different keys.
template <int D, int NW>
struct TileByteOffsets {
  static constexpr int KI = (TileCfg<D>::KINSTR + NW - 1) / NW;
  static constexpr int VI = (TileCfg<D>::VINSTR + NW - 1) / NW;
  uint32_t ko[KI];
  uint32_t vo[VI];
  __device__ __forceinline__ void init_k(const FwdArgs& a, int w, int l, int maxrow = BN - 1) {
    using C = TileCfg<D>;
#pragma unroll
    for (int k = 0; k < KI; ++k) {
      uint32_t r, c;
      kslab_rc<D>(min(w + NW * k, C::KINSTR - 1), l, r, c);
      r = min(r, (uint32_t)maxrow);
      ko[k] = (r * (uint32_t)a.k_sl + c * 8u) * 2u;
    }
  }
  __device__ __forceinline__ void init_v(const FwdArgs& a, int w, int l, int maxrow = BN - 1) {
    using C = TileCfg<D>;
#pragma unroll
    for (int v = 0; v < VI; ++v) {
      uint32_t r, c;
      slot_rc<C::VSPR, C::CPR>((uint32_t)min(w + NW * v, C::VINSTR - 1) * 64u + (uint32_t)l, r, c);
      r = min(r, (uint32_t)maxrow);
      vo[v] = (r * (uint32_t)a.v_sl + c * 8u) * 2u;
    }
  }
};

// Copies one K tile (rows from ktile, wave-uniform) to LDS address `kdst` (wave-uniform) with
// the scalar-base copy instruction; wave wu issues the K instructions wu, wu+NW, ...
template <int D, int NW>
__device__ __forceinline__ void issue_k_sbase(uint32_t kdst, const uint16_t* ktile,
                                              const TileByteOffsets<D, NW>& o, int wu) {
  using C = TileCfg<D>;
#pragma unroll
  for (int k = 0; k < TileByteOffsets<D, NW>::KI; ++k) {
    const int i = wu + NW * k;
    if ((C::KINSTR % NW) == 0 || i < C::KINSTR) dma16_sbase(ktile, o.ko[k], kdst + (uint32_t)i * 1024u);
  }
}

// The same for one V tile (padded rows) at LDS address `vdst`.
template <int D, int NW>
__device__ __forceinline__ void issue_v_sbase(uint32_t vdst, const uint16_t* vtile,
                                              const TileByteOffsets<D, NW>& o, int wu) {
  using C = TileCfg<D>;
#pragma unroll
  for (int v = 0; v < TileByteOffsets<D, NW>::VI; ++v) {
    const int i = wu + NW * v;
    if ((C::VINSTR % NW) == 0 || i < C::VINSTR) dma16_sbase(vtile, o.vo[v], vdst + (uint32_t)i * 1024u);
  }
}

}  // namespace
}  // namespace attn
