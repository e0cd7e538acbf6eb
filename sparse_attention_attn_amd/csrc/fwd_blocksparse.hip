// fwd_blocksparse.hip — fused block-sparse attention forward (causal, GQA) on gfx950.
//
// What is computed: O = softmax(scale·Q·Kᵀ + mask)·V and LSE per query row ("Resumen Técnico:
// FlashMLA-ETAP", section "Mecanismo Central"), where a key is visible to a query only if its
// 64-key block is listed for the query's 64-row block or its column is listed for the query's
// head, and it is not in the query's causal future. The kernel visits only the listed key
// blocks, then the listed vertical key columns outside them (MInference article, paragraphs on
// the A-shape / vertical-slash / block-sparse patterns and the dynamically built sparse
// indices), with running softmax statistics kept on chip ("Activar Flash Attention con
// llama.cpp para optimizar la inferencia", section "¿Qué es Flash Attention y por qué es
// crucial para llama.cpp?").
//
// Work decomposition: one workgroup of 4 waves owns a pair of 64-row query blocks of one
// (batch, query head); each wave owns 32 rows. Keys stream through LDS in 64-key tiles (K tile
// + V tile), copied by gfx950's asynchronous global->LDS loads into a two-stage ring so the
// copy of tile t+1 overlaps the math on tile t; a tile is copied once for both query blocks.
//
// Per tile and wave, the product is formed transposed, Sᵀ = K·Qᵀ, with 32x32x16 bf16 MFMA:
// K (64 keys x D) is the A operand read from LDS, Qᵀ is the B operand held in registers for
// the whole loop. In the Sᵀ accumulator each lane holds 16 keys of ONE query, so the row max
// and row sum need only in-lane math plus one exchange between lanes l and l^32, and the
// same registers, rounded to bf16, are directly the B operand Pᵀ of Oᵀ += Vᵀ·Pᵀ. Vᵀ comes
// from the row-major V tile via the LDS transpose read. (The transposition here serves
// register layout; the M-padding reason the FlashMLA-ETAP page gives for its transposed flow
// does not arise with 32- or 16-row MFMA tiles.)
//
// LDS layout: the K tile is stored in MFMA-operand order (1 KiB slab per k-step and key block,
// lane l's 16 bytes at offset 16*l), so every K-operand read is a linear ds_read_b128, the
// pattern that reaches the full LDS read bandwidth (a row-major tile read by 32 rows per
// instruction reaches half of it). V rows are padded to 2D+64 bytes, which keeps the
// transposed V read (8 rows x 64 bytes per instruction) at full bandwidth. Every read address
// is a per-lane base plus a compile-time offset. The copy engine writes 1 KiB per instruction;
// V padding slots receive a duplicate chunk that is never read.
//
// Softmax: scores live in the exp2 domain (x = s·scale·log2 e). Each row keeps a reference m
// and its weights are exp2(x - m), computed with no maximum taken. After the weights of a
// 32-key unit, one compare per lane accepts the unit when the row already has a reference and
// the lane's running fp32 weight sum is at most 2^64 (so no weight or accumulator can come
// near overflow; inf and NaN fail too); otherwise the wave takes a slow path for that unit:
// the unit's row maxima move m, the accumulators and sums are rescaled and the unit's weights
// recomputed, before the unit's P·V. Weights may then exceed 1 (the reference can lag the true
// maximum), which fp32 and bf16 hold with the same relative precision; two sums are kept, the
// sum of the bf16-rounded weights, which normalises O (numerator and denominator use the same
// weights), and the fp32 sum, which gives the LSE.
//
// Schedule of one tile for one wave (keys in two 32-key units u0, u1): the MFMAs of Sᵀ(u0);
// those of Sᵀ(u1), each followed by a slice of u0's softmax on the VALU; those of P·V(u0),
// each followed by a slice of u1's softmax; those of P·V(u1). So a single wave keeps the
// matrix core and the VALU busy together in the middle half of the tile, and the second wave
// of the SIMD fills the rest. Operands are read from LDS two MFMA slots ahead of their use.

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "tile_io.hpp"

namespace attn {
namespace {

template <int D>
struct WaveState {
  bf16x8 qop[TileCfg<D>::KSTEPS];
  f32x16 acc[TileCfg<D>::DVB];
  float m;        // reference in the exp2 domain, -inf before any key (same in lanes l, l^32)
  float mu;       // m where finite, +inf otherwise (every weight is then 0)
  float lb;       // lane-partial sum of the bf16-rounded weights
  float lf;       // lane-partial sum of the fp32 weights
  uint32_t kofs;  // lane byte offset of its K-operand reads inside a tile
  uint32_t vofs;  // lane byte offset of its transposed V reads inside a tile
};

// Accepts a unit: the row has a reference and the lane's fp32 sum is at most 2^64 (bit
// compare: inf and NaN fail).
__device__ __forceinline__ bool unit_ok(float m, float sf) {
  return m != -INFINITY && __builtin_bit_cast(uint32_t, sf) <= kSumLimitBits;
}

// Slow path of a unit: moves the row's reference to the larger of m and the unit's row
// maximum, rescales the accumulators and the sums of the earlier units by exp2(m_old - m_new),
// and recomputes the unit's weights (Pᵀ operands p) and sums sb, sf.
template <int D>
__device__ __forceinline__ void slow_unit(WaveState<D>& ws, const f32x16& s, float sl2,
                                          bf16x8 (&p)[2], float& sb, float& sf) {
  float mx = max3f(s[0], s[1], s[2]);
#pragma unroll
  for (int j = 3; j + 1 < 16; j += 2) mx = max3f(mx, s[j], s[j + 1]);
  mx = fmaxf(mx, s[15]);
  const float mnew = fmaxf(ws.m, max_halves(mx) * sl2);
  const float munew = (mnew == -INFINITY) ? INFINITY : mnew;
  // m_old = -inf gives 0 (nothing accumulated yet); an unchanged finite m gives 1
  const float alpha = fast_exp2(ws.m - munew);
#pragma unroll
  for (int b = 0; b < TileCfg<D>::DVB; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) ws.acc[b][j] *= alpha;
  sb = ws.lb * alpha;
  sf = ws.lf * alpha;
  uint32_t pk[2][4];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e0 = fast_exp2(fmaf(s[8 * ks + 2 * i], sl2, -munew));
      const float e1 = fast_exp2(fmaf(s[8 * ks + 2 * i + 1], sl2, -munew));
      sf += e0;
      sf += e1;
      pk[ks][i] = pack_bf16x2(e0, e1);
      sb = add_bf16_pair(pk[ks][i], sb);
    }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    p[ks] = __builtin_bit_cast(bf16x8, make_uint4(pk[ks][0], pk[ks][1], pk[ks][2], pk[ks][3]));
  ws.m = mnew;
  ws.mu = munew;
}

// LDS tile of this kernel. K differs from the dense kernel's operand-order slabs: rows are
// stored row-major, each followed by one 16-byte pad slot (2D + 16 bytes per row). A copy
// instruction (64 lanes x 16 bytes, landing contiguously) then reads whole key rows, so its
// loads cover full cache lines; with the slab order each instruction touched 32 rows at 32
// bytes each, and the tiles here come from scattered blocks that are not in L2 (timing-only
// copies: 13.0 -> 10.9 ms of copy time at the 128K workload). The pad makes the row stride an
// odd number of 16-byte slots, so the MFMA operand read (16 consecutive rows of one chunk per
// quarter wave) hits distinct banks, and k-step s of a lane is its base address plus 32·s.
// V is the padded row-major tile shared with the dense kernel.
template <int D>
struct SpCfg {
  using T = TileCfg<D>;
  static constexpr int CPR = T::CPR;
  static constexpr int KSTEPS = T::KSTEPS;
  static constexpr int DVB = T::DVB;
  static constexpr int KSPR = CPR + 1;        // 16-byte slots per K row (one pad slot)
  static constexpr int KROW = 16 * KSPR;      // bytes per K row
  static constexpr int KT_BYTES = BN * KROW;  // = 1024 * KSPR
  static constexpr int KINSTR = KT_BYTES / 1024;
  static constexpr int VROW = T::VROW;
  static constexpr int VSPR = T::VSPR;
  static constexpr int VT_BYTES = T::VT_BYTES;
  static constexpr int VINSTR = T::VINSTR;
  static constexpr int STAGE_BYTES = KT_BYTES + VT_BYTES;
  static_assert(KT_BYTES % 1024 == 0, "whole KiB K tiles");
};

// Copy instruction i (K instructions first, then V) of one tile: copy slot q = 64·i' + l of
// the K (or V) part holds row q / SPR at chunk q % SPR (pad slots re-read chunk 0 of their
// row). key_of(r) returns the key of tile row r and must be a valid key, so every load is in
// bounds. `st` is the stage's LDS address; k_row_bytes / v_row_bytes are the byte strides
// between key rows.
template <int D, class KeyOf>
__device__ __forceinline__ void copy_instr_gather(uint32_t st, const uint16_t* kbase,
                                                  const uint16_t* vbase, uint32_t k_row_bytes,
                                                  uint32_t v_row_bytes, KeyOf key_of, int i, int l) {
  using C = SpCfg<D>;
  uint32_t r, c;
  if (i < C::KINSTR) {
    slot_rc<C::KSPR, C::CPR>((uint32_t)i * 64u + (uint32_t)l, r, c);
    dma16_vaddr((const char*)kbase + (int64_t)key_of((int)r) * k_row_bytes + c * 16u,
                st + (uint32_t)i * 1024u);
  } else {
    const int iv = i - C::KINSTR;
    slot_rc<C::VSPR, C::CPR>((uint32_t)iv * 64u + (uint32_t)l, r, c);
    dma16_vaddr((const char*)vbase + (int64_t)key_of((int)r) * v_row_bytes + c * 16u,
                st + C::KT_BYTES + (uint32_t)iv * 1024u);
  }
}

// Scalar-base copy of a tile of 64 consecutive key rows (the same slot maps, per-lane offsets
// from the tile's first row). Wave wu issues instructions wu, wu+NW, ... With LEAN, the lane id
// goes through an opaque copy, so the offsets are recomputed at every issue instead of being
// hoisted out of the caller's loop into registers held for the whole kernel (for kernels short
// of registers).
template <int D, int NW, bool LEAN>
__device__ __forceinline__ void issue_tile_sbase_lean(uint32_t stage, const uint16_t* ktile,
                                                      const uint16_t* vtile, uint32_t k_row_bytes,
                                                      uint32_t v_row_bytes, int wu, int l) {
  using C = SpCfg<D>;
  if constexpr (LEAN) asm volatile("" : "+v"(l));
#pragma unroll
  for (int k = 0; k < (C::KINSTR + NW - 1) / NW; ++k) {
    const int i = wu + NW * k;
    if ((C::KINSTR % NW) == 0 || i < C::KINSTR) {
      uint32_t r, c;
      slot_rc<C::KSPR, C::CPR>((uint32_t)i * 64u + (uint32_t)l, r, c);
      dma16_sbase(ktile, r * k_row_bytes + c * 16u, stage + (uint32_t)i * 1024u);
    }
  }
#pragma unroll
  for (int v = 0; v < (C::VINSTR + NW - 1) / NW; ++v) {
    const int i = wu + NW * v;
    if ((C::VINSTR % NW) == 0 || i < C::VINSTR) {
      uint32_t r, c;
      slot_rc<C::VSPR, C::CPR>((uint32_t)i * 64u + (uint32_t)l, r, c);
      dma16_sbase(vtile, r * v_row_bytes + c * 16u, stage + C::KT_BYTES + (uint32_t)i * 1024u);
    }
  }
}

// Gathered tile copy: wave w of NW issues copy instructions w, w+NW, ... (K first, then V)
// with per-lane source addresses. Like the scalar-base copy, it is invisible to the compiler:
// the caller orders later LDS reads with an explicit vmcnt wait and a workgroup barrier.
template <int D, int NW, class KeyOf>
__device__ __forceinline__ void issue_tile_gather(uint32_t st, const uint16_t* kbase,
                                                  const uint16_t* vbase, uint32_t k_row_bytes,
                                                  uint32_t v_row_bytes, KeyOf key_of, int w, int l) {
  using C = SpCfg<D>;
  constexpr int NI = (C::KINSTR + C::VINSTR + NW - 1) / NW;
  const int wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int i = wu + NW * ii;
    if (i < C::KINSTR + C::VINSTR)
      copy_instr_gather<D>(st, kbase, vbase, k_row_bytes, v_row_bytes, key_of, i, l);
  }
}

// Math of one tile for one wave. When `masked`, mask(U, s) sets the scores of invisible keys of
// unit U (0 or 1, a compile-time constant) to -inf; slot j of s holds local key
// 32*U + 8*(j/4) + 4*(l/32) + j%4. Otherwise every key is visible.
template <int D, class Mask>
__device__ __forceinline__ void tile_math_mask(const FwdArgs& a, WaveState<D>& ws, const char* st,
                                               bool masked, Mask mask, int l) {
  using C = SpCfg<D>;
  constexpr int NQ = C::KSTEPS;  // MFMAs of a unit's Sᵀ
  constexpr int NV = 2 * C::DVB;  // MFMAs of a unit's P·V
  static_assert(NQ == NV, "the two softmax phases have the same number of slots");
  constexpr int NITEMS = 9;       // softmax items of a unit: 8 weight groups + the last fold
  const uint32_t kt = lds_addr(st) + ws.kofs;
  const uint32_t vt = lds_addr(st) + C::KT_BYTES + ws.vofs;
  const float sl2 = a.sl2;

  // MFMA slot n of the tile: [0, NQ) Sᵀ(u0), [NQ, 2NQ) Sᵀ(u1), then P·V(u0), P·V(u1). P·V slot
  // v covers output block v % DVB and unit k-step v / DVB (keys 16·ks .. 16·ks+15 of the unit),
  // so consecutive MFMAs accumulate into different blocks.
  auto operand = [&](int n) -> bf16x8 {
    // K: row 32·u + l%32 of unit u = n / NQ, chunk 2·s + l/32 of k-step s = n % NQ
    if (n < 2 * NQ) return lds_read_b128_at(kt + (uint32_t)(32 * C::KROW * (n / NQ) + 32 * (n % NQ)));
    const int u = (n - 2 * NQ) / NV, v = (n - 2 * NQ) % NV;
    const uint32_t o = vt + (32u * u + 16u * (v / C::DVB)) * C::VROW + 64u * (v % C::DVB);
    return lds_read_tr_pair_at(o, o + 8u * C::VROW);
  };
  bf16x8 opr[2];
  opr[0] = operand(0);

  f32x16 s0, s1;
  bf16x8 p0[2], p1[2];
  float sb = ws.lb, sf = ws.lf;
  uint32_t pk[2][4];
  float ew[2][2];
  // Softmax item it of unit scores s: weights of group it (scores 2·it, 2·it+1) and the fold
  // of group it-1 into the sums and the packed operand (skewed, so no fold waits on the exp2
  // just issued).
  auto item = [&](auto IT, const f32x16& s) {
    constexpr int it = decltype(IT)::value;
    if constexpr (it < 8) {
      ew[it & 1][0] = fast_exp2(fmaf(s[2 * it], sl2, -ws.mu));
      ew[it & 1][1] = fast_exp2(fmaf(s[2 * it + 1], sl2, -ws.mu));
    }
    if constexpr (it >= 1) {
      constexpr int g = it - 1;
      sf += ew[g & 1][0];
      sf += ew[g & 1][1];
      pk[g >> 2][g & 3] = pack_bf16x2(ew[g & 1][0], ew[g & 1][1]);
      sb = add_bf16_pair(pk[g >> 2][g & 3], sb);
    }
  };
  auto packed = [&](bf16x8 (&p)[2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      p[ks] = __builtin_bit_cast(bf16x8, make_uint4(pk[ks][0], pk[ks][1], pk[ks][2], pk[ks][3]));
  };
  // One MFMA slot: the product, then the read two slots ahead.
  auto slot = [&](auto NI) {
    constexpr int n = decltype(NI)::value;
    const bf16x8 op = opr[n % 2];
    if constexpr (n < NQ) {
      s0 = mfma32(op, ws.qop[n], n == 0 ? f32x16{} : s0);
    } else if constexpr (n < 2 * NQ) {
      s1 = mfma32(op, ws.qop[n - NQ], n == NQ ? f32x16{} : s1);
    } else if constexpr (n < 2 * NQ + NV) {
      constexpr int v = n - 2 * NQ;
      ws.acc[v % C::DVB] = mfma32(op, p0[v / C::DVB], ws.acc[v % C::DVB]);
    } else {
      constexpr int v = n - 2 * NQ - NV;
      ws.acc[v % C::DVB] = mfma32(op, p1[v / C::DVB], ws.acc[v % C::DVB]);
    }
    if constexpr (n + 1 < 2 * NQ + 2 * NV) opr[(n + 1) % 2] = operand(n + 1);
  };

  // Sᵀ(u0)
  __builtin_amdgcn_s_setprio(1);
  static_for<0, NQ>([&](auto NI) { slot(NI); });
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  // Sᵀ(u1) with the softmax of u0
  if (masked) mask(icn<0>{}, s0);
  static_for<0, NQ>([&](auto I) {
    constexpr int i = decltype(I)::value;
    slot(icn<NQ + i>{});
    static_for<NITEMS * i / NQ, NITEMS * (i + 1) / NQ>([&](auto IT) { item(IT, s0); });
    __builtin_amdgcn_sched_barrier(0);
  });
  packed(p0);
  if (__builtin_expect(__any(!unit_ok(ws.m, sf)), 0)) slow_unit<D>(ws, s0, sl2, p0, sb, sf);
  ws.lb = sb;
  ws.lf = sf;
  // P·V(u0) with the softmax of u1
  if (masked) mask(icn<1>{}, s1);
  static_for<0, NV>([&](auto I) {
    constexpr int i = decltype(I)::value;
    slot(icn<2 * NQ + i>{});
    static_for<NITEMS * i / NV, NITEMS * (i + 1) / NV>([&](auto IT) { item(IT, s1); });
    __builtin_amdgcn_sched_barrier(0);
  });
  packed(p1);
  if (__builtin_expect(__any(!unit_ok(ws.m, sf)), 0)) slow_unit<D>(ws, s1, sl2, p1, sb, sf);
  ws.lb = sb;
  ws.lf = sf;
  // P·V(u1)
  __builtin_amdgcn_s_setprio(1);
  static_for<0, NV>([&](auto I) { slot(icn<2 * NQ + NV + decltype(I)::value>{}); });
  __builtin_amdgcn_s_setprio(0);
}

// LDS slot of one wave in the window phase: the 32 key rows a wave's 32 query rows meet on one
// slash line. K rows are stored unpadded with chunk c of row r at position c ^ swz(r), which
// keeps the MFMA operand read (16 consecutive rows of one chunk per quarter wave) on distinct
// banks; V rows use the padded row-major layout of the tiles. Two slots fit in a ring stage.
template <int D>
struct WinCfg {
  using T = TileCfg<D>;
  static constexpr int CPR = T::CPR;
  static constexpr int KROW = 2 * D;                   // bytes per K row
  static constexpr int KBYTES = 32 * KROW;
  static constexpr int KINSTR = KBYTES / 1024;
  static constexpr int VBYTES = 32 * T::VROW;
  static constexpr int VINSTR = VBYTES / 1024;
  static constexpr int BYTES = KBYTES + VBYTES;
  static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "whole copy instructions");
  static_assert(2 * BYTES + 512 <= SpCfg<D>::STAGE_BYTES,
                "two window slots and their column words per ring stage");
  static __device__ __forceinline__ uint32_t swz(uint32_t r) {
    return D == 128 ? (r & 15u) : ((r >> 1) & 7u);
  }
};

// One 32-key unit of the window phase, in two halves so that the copies of the next line's K
// and of this line's V can overlap them. window_scores: Sᵀ = K·Qᵀ over the wave's slot, every
// score but the kept one set to -inf (keep_slot: the accumulator slot j of this lane that
// holds a visible key, or -1), and the weights (Pᵀ operands p, running sums updated).
// window_pv: Oᵀ += Vᵀ·Pᵀ.
template <int D>
__device__ __forceinline__ void window_scores(const FwdArgs& a, WaveState<D>& ws, uint32_t slot,
                                              int keep_slot, int l, bf16x8 (&p)[2]) {
  using W = WinCfg<D>;
  using C = SpCfg<D>;
  const uint32_t i = (uint32_t)(l & 31), h = (uint32_t)(l >> 5);
  const uint32_t krow = slot + i * (uint32_t)W::KROW;
  f32x16 s = f32x16{};
#pragma unroll
  for (int st = 0; st < C::KSTEPS; ++st) {
    const uint32_t c = 2u * (uint32_t)st + h;
    s = mfma32(lds_read_b128_at(krow + ((c ^ W::swz(i)) << 4)), ws.qop[st], s);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j != keep_slot) s[j] = -INFINITY;
  const float sl2 = a.sl2;
  float sb = ws.lb, sf = ws.lf;
  uint32_t pk[2][4];
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const float e0 = fast_exp2(fmaf(s[2 * g], sl2, -ws.mu));
    const float e1 = fast_exp2(fmaf(s[2 * g + 1], sl2, -ws.mu));
    sf += e0;
    sf += e1;
    pk[g >> 2][g & 3] = pack_bf16x2(e0, e1);
    sb = add_bf16_pair(pk[g >> 2][g & 3], sb);
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    p[ks] = __builtin_bit_cast(bf16x8, make_uint4(pk[ks][0], pk[ks][1], pk[ks][2], pk[ks][3]));
  if (__builtin_expect(__any(!unit_ok(ws.m, sf)), 0)) slow_unit<D>(ws, s, sl2, p, sb, sf);
  ws.lb = sb;
  ws.lf = sf;
}

template <int D>
__device__ __forceinline__ void window_pv(WaveState<D>& ws, uint32_t slot, const bf16x8 (&p)[2]) {
  using W = WinCfg<D>;
  using C = SpCfg<D>;
  const uint32_t vt = slot + (uint32_t)W::KBYTES + ws.vofs;
#pragma unroll
  for (int v = 0; v < 2 * C::DVB; ++v) {
    const uint32_t o = vt + (16u * (uint32_t)(v / C::DVB)) * C::VROW + 64u * (uint32_t)(v % C::DVB);
    ws.acc[v % C::DVB] = mfma32(lds_read_tr_pair_at(o, o + 8u * C::VROW), p[v / C::DVB],
                                ws.acc[v % C::DVB]);
  }
}

// Copies into a wave's window slot the K rows (issue_window_k, with the two words of the
// column bitmap that cover those keys, to LDS address cw) or the V rows (issue_window_v) of keys
// k0 .. k0 + 31, clamped into [0, lkm1] so that every load is in bounds (the clamped rows are
// masked by the caller). Each first waits for the wave's earlier reads of the slot.
template <int D>
constexpr int kWinKCopies = WinCfg<D>::KINSTR + 1;  // copy instructions of issue_window_k
template <int D>
constexpr int kWinVCopies = WinCfg<D>::VINSTR;      // copy instructions of issue_window_v

template <int D>
__device__ __forceinline__ void issue_window_k(uint32_t slot, uint32_t cw, const uint16_t* kbase,
                                               uint32_t k_row_bytes, const uint32_t* cbits,
                                               int k0, int lkm1, int l) {
  using W = WinCfg<D>;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < W::KINSTR; ++i) {
    const uint32_t q = (uint32_t)i * 64u + (uint32_t)l;
    const uint32_t r = q / W::CPR, pos = q % W::CPR;
    const uint32_t c = pos ^ W::swz(r);
    const int key = min(max(k0 + (int)r, 0), lkm1);
    dma16_vaddr((const char*)kbase + (int64_t)key * k_row_bytes + c * 16u, slot + (uint32_t)i * 1024u);
  }
  // words max(k0, 0)/32 and the next one (lanes beyond 1 re-read them; the bitmap has two
  // spare words past the last key)
  dma4_vaddr(cbits + (max(k0, 0) >> 5) + (l & 1), cw);
}

template <int D>
__device__ __forceinline__ void issue_window_v(uint32_t slot, const uint16_t* vbase,
                                               uint32_t v_row_bytes, int k0, int lkm1, int l) {
  using W = WinCfg<D>;
  using C = SpCfg<D>;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < W::VINSTR; ++i) {
    uint32_t r, c;
    slot_rc<C::VSPR, C::CPR>((uint32_t)i * 64u + (uint32_t)l, r, c);
    const int key = min(max(k0 + (int)r, 0), lkm1);
    dma16_vaddr((const char*)vbase + (int64_t)key * v_row_bytes + c * 16u,
                slot + (uint32_t)W::KBYTES + (uint32_t)i * 1024u);
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Key-position form: kidx(local key) gives the key position, or -1 if the slot holds no key;
// keys beyond the causal limit of `row` are masked too.
template <int D, class KeyIdx>
__device__ __forceinline__ void tile_math(const FwdArgs& a, WaveState<D>& ws, const char* st,
                                          int row, bool masked, KeyIdx kidx, int l) {
  const int h = l >> 5;
  const int lim = a.causal ? row + a.off : 0x7fffffff;
  tile_math_mask<D>(a, ws, st, masked, [&](auto U, f32x16& s) {
    constexpr int u = decltype(U)::value;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int k = kidx(32 * u + 8 * (j >> 2) + 4 * h + (j & 3));
      if (k < 0 || k > lim) s[j] = -INFINITY;
    }
  }, l);
}

template <int D>
__device__ __forceinline__ void load_q(const FwdArgs& a, WaveState<D>& ws, int b, int hq, int row,
                                       int l) {
  using C = TileCfg<D>;
  const int h = l >> 5;
  if (row < a.Lq) {
    const uint16_t* qr = a.q + (int64_t)b * a.q_sb + (int64_t)row * a.q_sl + (int64_t)hq * a.q_sh;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) ws.qop[s] = load_q_bf16x8(qr + 16 * s + 8 * h, a.qsign);
  } else {
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) ws.qop[s] = zero_bf16x8();
  }
#pragma unroll
  for (int bb = 0; bb < C::DVB; ++bb) ws.acc[bb] = f32x16{};
  ws.m = -INFINITY;
  ws.mu = INFINITY;
  ws.lb = 0.f;
  ws.lf = 0.f;
  // K operand: row l%32 of the unit, chunk l/32 of the k-step
  ws.kofs = (uint32_t)(l & 31) * (uint32_t)SpCfg<D>::KROW + (uint32_t)(l >> 5) * 16u;
  // V operand: group G = l/16, row 4*(G/2) + (l%16)/4, column 16*(G%2) + 4*(l%4)
  const int G = l >> 4;
  ws.vofs = (uint32_t)(4 * (G >> 1) + ((l & 15) >> 2)) * C::VROW +
            (uint32_t)(16 * (G & 1) + 4 * (l & 3)) * 2u;
}

// Writes the wave's rows of O (obase: row 0 of this (b, head); o_sl: row stride) and, when
// lse_row is given (the LSE entries of this (b, head)), their LSE.
template <int D>
__device__ __forceinline__ void store_out(const WaveState<D>& ws, uint16_t* obase, int64_t o_sl,
                                          float* lse_row, int row, int Lq, int l) {
  using C = TileCfg<D>;
  const int h = l >> 5;
  const float tb = ws.lb + other_half(ws.lb);
  const float tf = ws.lf + other_half(ws.lf);
  if (row >= Lq) return;
  const float inv = tb > 0.f ? 1.0f / tb : 0.f;
  uint16_t* orow = obase + (int64_t)row * o_sl;
#pragma unroll
  for (int bb = 0; bb < C::DVB; ++bb) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int dv = 32 * bb + 8 * u + 4 * h;
      uint2 pk;
      pk.x = pack_bf16x2(ws.acc[bb][4 * u + 0] * inv, ws.acc[bb][4 * u + 1] * inv);
      pk.y = pack_bf16x2(ws.acc[bb][4 * u + 2] * inv, ws.acc[bb][4 * u + 3] * inv);
      *reinterpret_cast<uint2*>(orow + dv) = pk;
    }
  }
  if (lse_row != nullptr && h == 0) lse_row[row] = tf > 0.f ? ws.m * kLn2 + logf(tf) : -INFINITY;
}

// Maps blockIdx.x to a logical work id. The hardware deals workgroups round-robin over the 8
// XCDs (each with its own L2) in blockIdx order. Logical ids are cut into chunks of 16 (4
// groups of query blocks x 4 query heads of one KV head) and chunk c runs on XCD c % 8: the
// query blocks that share most of their local band of key blocks meet in one L2, while all
// XCDs work on neighbouring chunks, i.e. on the same KV head, whose K/V then fits the
// device-wide cache. (Measured at the 128K workloads: chunks of 16 beat 32 and 64 by 2-3%;
// 4 and 8 are within 1% of 16.)
__device__ __forceinline__ int logical_block(int xcd_remap) {
  const int bid = (int)blockIdx.x;
  if (!xcd_remap) return bid;
  const int x = bid & 7;
  const int j = bid >> 3;
  return 16 * x + 128 * (j >> 4) + (j & 15);
}

// ------------------------------------------------------------------------------------------
// Block-sparse forward: one workgroup of 2·QB waves per (b, query head, group of QB = 2
// consecutive 64-row query blocks QB·p .. QB·p+QB-1); waves 2q and 2q+1 own the rows of block
// QB·p+q, 32 rows each. Neighbouring blocks' lists share most of their key blocks (the local
// band moves by one block), so the workgroup streams each key tile once for the whole group,
// and a wave skips the tiles its own block does not list. With two such workgroups per CU
// every SIMD runs two waves, which hide each other's softmax and waits: while the waves of
// one workgroup skip a tile, the other workgroup's waves keep the matrix core busy. (Four
// blocks per workgroup, with eight waves, one workgroup per CU and a four-stage ring, shares
// more tiles but measured slower: the workgroup barrier of every tile then idles the six
// waves whose blocks do not list it.)
// Phase 1 walks the union of the group's listed-block sets in ascending order; phase 2
// gathers the head's vertical columns that are causally visible to the group and not inside
// a block every block of the group lists, 64 at a time, and each wave masks the columns
// inside its own listed blocks (so a key is never counted twice).
//
// With SLASH, phase 3 adds the head's slash lines (MInference article, paragraph on the
// vertical-slash pattern): the line at offset o >= 0 lets query row i see key i + off - o
// (off = Lk - Lq). Setup marks the 64-key blocks any line crosses inside the group's rows;
// phase 3 runs each marked block that the wave's own block does not list as a tile whose mask
// keeps a pair (row, key) only when row + off - key is a listed offset and key is not a listed
// column (those keys were counted in phase 2). The offsets and the columns of a head come as
// two bitmaps (vs_bits_kernel); the words of both that a tile's mask needs are copied into
// LDS together with the tile, and each lane reads the 96 + 64 bits its 32 scores need.
// ------------------------------------------------------------------------------------------
constexpr int kSeg = 256;              // ids examined per compaction pass
constexpr int kMaxBitmapWords = 512;   // listed-block bitmaps: up to 16384 key blocks (1M keys)
constexpr int kSlashBitmapWords = kVslashMaxLk / 64 / 32;  // crossed blocks (slash variant)
constexpr int kFlagShift = 24;         // phase-2 entry: column id below, block flags above
constexpr int kColMask = (1 << kFlagShift) - 1;
constexpr int kMaskOffWords = 48;      // offset-bitmap words copied per slash tile

template <int D, bool SLASH, int QB>
__global__ __launch_bounds__(2 * QB * 64, 2) void fwd_sparse_kernel(const FwdArgs a) {
  using C = SpCfg<D>;
  // listed-block bitmap words: the slash variant's shorter key limit frees LDS for its own
  // bitmap and mask words (two workgroups per CU need at most 80 KiB each)
  constexpr int BMW = SLASH ? kVslashMaxLk / 64 / 32 : kMaxBitmapWords;
  constexpr int NW = 2 * QB;
  constexpr int NT = NW * 64;
  constexpr int NS = 2;  // ring stages
  static_assert(QB == 2, "two query blocks per workgroup (two workgroups per CU)");
  static_assert(kFlagShift + QB <= 31, "phase-2 flags fit an int");
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE_BYTES];
  __shared__ uint32_t bm[QB][BMW];                             // listed blocks of the group
  __shared__ uint32_t tbits[SLASH ? kSlashBitmapWords : 1];  // blocks crossed by a slash line
  __shared__ int kept[kSeg];
  __shared__ int wave_cnt[NW];
  __shared__ uint32_t mwl[SLASH ? NS : 1][SLASH ? 64 : 1];  // per stage: a slash tile's mask words

  const int tid = (int)threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int nqb = a.n_qtiles;
  const int ngrp = (nqb + QB - 1) / QB;
  // the work ids are workgroup-uniform: pinned to scalar registers, so are the addresses
  // derived from them
  int lid = logical_block(a.xcd_remap);
  const int hg = __builtin_amdgcn_readfirstlane(lid % a.g);
  lid = __builtin_amdgcn_readfirstlane(lid / a.g);
  const int pr = __builtin_amdgcn_readfirstlane(ngrp - 1 - (lid % ngrp));
  lid = __builtin_amdgcn_readfirstlane(lid / ngrp);
  const int hkv = __builtin_amdgcn_readfirstlane(lid % a.Hkv);
  const int b = __builtin_amdgcn_readfirstlane(lid / a.Hkv);
  const int hq = hkv * a.g + hg;

  const int qbA = QB * pr;
  const int myq = w >> 1;  // this wave's block is qbA + myq
  const int q0 = qbA * 64;                       // first row of the workgroup
  const int qw0 = q0 + 64 * myq + 32 * (w & 1);  // first row of this wave
  const int row = qw0 + (l & 31);
  const bool active = qw0 < a.Lq;                // the wave has rows
  const int qlast = min(q0 + 64 * QB, a.Lq) - 1;  // last row of the workgroup
  const int qwlast = min(qw0 + 31, a.Lq - 1);
  const int klim = a.causal ? min(a.Lk - 1, qlast + a.off) : a.Lk - 1;  // last visible key
  const int lkm1 = a.Lk - 1;

  const int bh = b * a.Hq + hq;
  const int nwords = (a.nkb + 31) >> 5;
  // Uniform values the later phases and the epilogue need, derived here so that the kernel
  // arguments they come from die after setup instead of holding scalar registers throughout.
  uint16_t* const obase = a.o + (int64_t)b * a.o_sb + (int64_t)hq * a.o_sh;
  const int64_t o_sl = a.o_sl;
  float* const lse_row = a.lse != nullptr ? a.lse + (int64_t)bh * a.Lq : nullptr;
  const int Lq = a.Lq;
  const int cstart = a.col_ptr[bh];
  const int ncols = a.col_ptr[bh + 1] - cstart;
  const int* const cidx = a.col_idx + cstart;
  const uint32_t* const sbits = SLASH ? a.rl_bits + (int64_t)bh * a.bits_words : nullptr;
  const uint32_t* const cbits = SLASH ? a.cl_bits + (int64_t)bh * a.bits_words : nullptr;
  const int bits_last = a.bits_words - 1;
  const uint32_t k_row_bytes = (uint32_t)a.k_sl * 2u, v_row_bytes = (uint32_t)a.v_sl * 2u;
  auto listed = [&](int q, int kb) -> bool { return (bm[q][kb >> 5] >> (kb & 31)) & 1u; };
  // blocks listed by at least one / by every block of the group, word kb/32
  auto any_word = [&](int wd) -> uint32_t {
    uint32_t v = 0u;
#pragma unroll
    for (int q = 0; q < QB; ++q) v |= bm[q][wd];
    return v;
  };
  auto all_word = [&](int wd) -> uint32_t {
    uint32_t v = ~0u;
#pragma unroll
    for (int q = 0; q < QB; ++q) v &= bm[q][wd];
    return v;
  };

  for (int i = tid; i < nwords; i += NT) {
#pragma unroll
    for (int q = 0; q < QB; ++q) bm[q][i] = 0u;
  }
  if constexpr (SLASH)
    for (int i = tid; i < nwords; i += NT) tbits[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    if (qbA + q >= nqb) break;
    const int64_t lrow = (int64_t)bh * nqb + qbA + q;
    const int s1 = a.blk_ptr[lrow + 1];
    for (int i = a.blk_ptr[lrow] + tid; i < s1; i += NT) {
      const int kbk = a.blk_idx[i];
      if (kbk >= 0 && kbk < a.nkb) atomicOr(&bm[q][kbk >> 5], 1u << (kbk & 31));
    }
  }
  if constexpr (SLASH) {
    // the line at offset o meets rows q0..qlast at keys q0+off-o .. qlast+off-o (<= klim);
    // only lines inside a run of listed offsets go through the crossed tiles (isolated lines
    // take the window phase)
    // The list entries of a chunk of kSetupJ * NT are loaded first, then their run bits, so a
    // chunk costs two memory round trips rather than two per entry of each thread.
    constexpr int kSetupJ = 8;
    const int s0 = a.sl_ptr[bh], s1 = a.sl_ptr[bh + 1];
    const uint32_t* const rb = a.rl_bits + (int64_t)bh * a.bits_words;
    for (int c = s0; c < s1; c += kSetupJ * NT) {
      int o[kSetupJ];
      uint32_t rw[kSetupJ];
#pragma unroll
      for (int j = 0; j < kSetupJ; ++j) {
        const int i = c + j * NT + tid;
        o[j] = i < s1 ? a.sl_idx[i] : -1;
      }
#pragma unroll
      for (int j = 0; j < kSetupJ; ++j) {
        const bool in = o[j] >= 0 && o[j] <= qlast + a.off;
        rw[j] = in ? rb[(o[j] + 128) >> 5] : 0u;
      }
#pragma unroll
      for (int j = 0; j < kSetupJ; ++j) {
        if (((rw[j] >> ((o[j] + 128) & 31)) & 1u) == 0u) continue;  // not in reach or isolated
        const int hi = qlast + a.off - o[j];
        const int lo = max(0, q0 + a.off - o[j]);
        if (lo > lkm1) continue;
        for (int kb = lo >> 6; kb <= (min(hi, lkm1) >> 6); ++kb)
          atomicOr(&tbits[kb >> 5], 1u << (kb & 31));
      }
    }
  }
  __syncthreads();

  // Ordered compaction: for the items i < n whose keep(i) holds, value(i) goes to kept[] in
  // the order of i; returns their count (the same in every wave).
  // Passes over list entries hold one entry per thread (phases 2 and 3b read it once into a
  // register and pass it to compact, which then evaluates entry tid in thread tid).
  static_assert(kSeg == NT, "one list entry per thread in a pass");
  auto compact = [&](int n, auto keep_fn, auto value_fn) -> int {
    int cnt = 0;
    for (int rr = 0; rr < n; rr += NT) {
      const int i = rr + tid;
      const bool keep = i < n && keep_fn(i);
      const uint64_t mask = __ballot(keep);
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      if (l == 0) wave_cnt[w] = __popcll(mask);
      __syncthreads();
      int woff = 0, tot = 0;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const int cw = wave_cnt[ww];
        woff += (ww < w) ? cw : 0;
        tot += cw;
      }
      if (keep) kept[cnt + woff + below] = value_fn(i);
      cnt += tot;
      __syncthreads();
    }
    return cnt;
  };

  // Key blocks 0 .. nvis-1 can hold a key visible to a row of the group. A segment of block ids
  // whose candidate bits (word_fn of its words) are all clear is skipped without a compaction
  // pass; every thread reads the same LDS words, so the decision is uniform.
  const int nvis = (klim >> 6) + 1;
  auto seg_empty = [&](int c0, auto word_fn) -> bool {
    uint32_t v = 0u;
    const int w1 = min((c0 + kSeg) >> 5, nwords);
    for (int wd = c0 >> 5; wd < w1; ++wd) v |= word_fn(wd);
    return v == 0u;
  };

  WaveState<D> ws;
  load_q<D>(a, ws, b, hq, row, l);
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint16_t* kbp = a.k + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh;
  const uint16_t* vbp = a.v + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh;

  auto stage = [&](auto S) -> char* { return decltype(S)::value == 0 ? st0 : st1; };
  auto stage_addr = [&](auto S) -> uint32_t {
    return (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(stage(S)));
  };
  // copy of the 64-key block starting at key `base` (inside the sequence) into stage S
  auto issue_block = [&](auto S, int base) {
    if (base + BN <= a.Lk) {
      issue_tile_sbase_lean<D, NW, SLASH>(
          stage_addr(S), (const uint16_t*)((const char*)kbp + (int64_t)base * k_row_bytes),
          (const uint16_t*)((const char*)vbp + (int64_t)base * v_row_bytes), k_row_bytes,
          v_row_bytes, wu, l);
    } else {
      issue_tile_gather<D, NW>(stage_addr(S), kbp, vbp, k_row_bytes, v_row_bytes,
                               [&](int r) { return min(base + r, lkm1); }, w, l);
    }
  };
  // The two-stage ring over tiles 0..ntl-1 (tile t in stage t % 2). Step t waits for tile t
  // (this wave's copies, then the barrier for every wave's), starts the copy of tile t+1 into
  // the other stage, whose readers (the math of tile t-1) all passed the barrier, and runs the
  // math of tile t. The copies are invisible to the compiler, so it adds no waits of its own
  // before the LDS reads; the barrier carries no memory fence (nothing else needs ordering).
  // An empty pass returns at once: the compaction that produced it ended with a barrier, and it
  // issues no copies.
  auto run = [&](int ntl, auto issue_fn, auto math_fn) {
    if (ntl == 0) return;
    wait_vmcnt_visible0();  // the Q operands (and any earlier load) are in registers
    issue_fn(ic<0>{}, 0);
    auto step = [&](auto S, int t) {
      constexpr int s = decltype(S)::value;
      wait_dma_all();
      barrier_lds();
      if (t + 1 < ntl) issue_fn(ic<1 - s>{}, t + 1);
      math_fn(S, t);
    };
    for (int t = 0; t < ntl; t += NS) {
      step(ic<0>{}, t);
      if (t + 1 < ntl) step(ic<1>{}, t + 1);
    }
    __syncthreads();  // stages and kept[] free for the next pass
  };

  // ---- phase 1: the union of the group's listed key blocks, kSeg block ids per pass
  for (int c0 = 0; c0 < nvis; c0 += kSeg) {
    if (seg_empty(c0, any_word)) continue;
    const int cnt = compact(min(kSeg, nvis - c0),
                            [&](int i) {
                              const int kb = c0 + i;
                              return ((any_word(kb >> 5) >> (kb & 31)) & 1u) != 0u;
                            },
                            [&](int i) { return c0 + i; });
    run(cnt, [&](auto S, int t) { issue_block(S, kept[t] * BN); },
        [&](auto S, int t) {
          const int kb = kept[t];
          const int base = kb * BN;
          if (!active || !listed(myq, kb)) return;
          if (a.causal && base > qwlast + a.off) return;
          const bool masked = base + BN > a.Lk || (a.causal && base + BN - 1 > qw0 + a.off);
          // a key is visible up to min(causal limit of the row, Lk - 1); in local terms, slot
          // j of unit U holds key base + 4h + 32U + 8(j/4) + j%4
          const int hi = min(a.causal ? row + a.off : 0x7fffffff, a.Lk - 1) - base - 4 * (l >> 5);
          tile_math_mask<D>(a, ws, stage(S), masked, [&](auto U, f32x16& sc) {
            constexpr int u = decltype(U)::value;
#pragma unroll
            for (int j = 0; j < 16; ++j)
              if (32 * u + 8 * (j >> 2) + (j & 3) > hi) sc[j] = -INFINITY;
          }, l);
        });
  }

  // ---- phase 2: vertical columns. An entry is the column id with bit kFlagShift + q set
  // when the column lies inside a block that block q of the group lists.
  for (int seg = 0; seg < ncols; seg += kSeg) {
    if (cidx[seg] > klim) break;  // sorted: nothing further is visible
    const int n = min(kSeg, ncols - seg);
    // thread tid's column of the pass, read once (compact evaluates entry tid in thread tid)
    const int my_col = tid < n ? cidx[seg + tid] : -1;
    const int cnt = compact(n,
                            [&](int) {
                              const int col = my_col;
                              if (col < 0 || col > klim) return false;
                              return ((all_word(col >> 11) >> ((col >> 6) & 31)) & 1u) == 0u;
                            },
                            [&](int) {
                              const int col = my_col;
                              int e = col;
#pragma unroll
                              for (int q = 0; q < QB; ++q)
                                e |= (int)listed(q, col >> 6) << (kFlagShift + q);
                              return e;
                            });
    // cnt columns make ceil(cnt / 64) tiles; tile t gathers entries 64t .. 64t+63
    run((cnt + BN - 1) / BN,
        [&](auto S, int t) {
          const int cb = t * BN;
          issue_tile_gather<D, NW>(
              stage_addr(S), kbp, vbp, k_row_bytes, v_row_bytes,
              [&](int r) { return kept[cb + r < cnt ? cb + r : cb] & kColMask; }, w, l);
        },
        [&](auto S, int t) {
          const int cb = t * BN;
          if (!active) return;
          // columns are ascending: skip if even the first one is beyond this wave's horizon
          if (a.causal && (kept[cb] & kColMask) > qwlast + a.off) return;
          // no mask when every slot holds a column that every row of the wave sees and that
          // no block the wave's block lists contains (lane l checks entry cb + l)
          const int el = kept[min(cb + l, cnt - 1)];
          const bool hidden = cb + l >= cnt || ((el >> (kFlagShift + myq)) & 1) ||
                              (a.causal && (el & kColMask) > qw0 + a.off);
          tile_math<D>(a, ws, stage(S), row, __any(hidden),
                       [&](int kl) {
                         if (cb + kl >= cnt) return -1;
                         const int e = kept[cb + kl];
                         return ((e >> (kFlagShift + myq)) & 1) ? -1 : (e & kColMask);
                       }, l);
        });
  }

  // ---- phase 3: slash lines, over the crossed blocks the wave's own block does not list
  if constexpr (SLASH) {
    const int h = l >> 5;
    // Lane's window: bitmap bit (o + 128) of its local key c's offset is at rw - base + 59 - c.
    const int rw = row + a.off + 69 - 4 * h;
    const int rw0 = q0 + a.off + 65;  // smallest rw of the group (row q0, h = 1)
    // first offset word of the group's window for the tile at `base`
    auto win0 = [&](int base) { return max(rw0 - base, 0) >> 5; };
    for (int c0 = 0; c0 < nvis; c0 += kSeg) {
      if (seg_empty(c0, [&](int wd) { return tbits[wd] & ~all_word(wd); })) continue;
      const int cnt = compact(min(kSeg, nvis - c0),
                              [&](int i) {
                                const int kb = c0 + i;
                                const uint32_t all = all_word(kb >> 5);
                                return (((tbits[kb >> 5] & ~all) >> (kb & 31)) & 1u) != 0u;
                              },
                              [&](int i) { return c0 + i; });
      run(cnt,
          [&](auto S, int t) {
            constexpr int s = decltype(S)::value;
            const int base = kept[t] * BN;
            // Wave 0 copies the tile's mask words next to it: offset words win0 .. win0+47
            // (the pair's rows need at most 8 of them) and the two column words of the tile;
            // the ring's wait covers this copy with the tile's.
            if (wu == 0) {
              int lo = l;
              asm volatile("" : "+v"(lo));  // keep the addresses below from being hoisted
              const int j0 = win0(base);
              const uint32_t* src = lo < kMaskOffWords
                                        ? sbits + min(j0 + lo, bits_last)
                                        : cbits + (base >> 5) + (lo == kMaskOffWords + 1);
              dma4_vaddr(src, lds_addr(&mwl[s][0]));
            }
            issue_block(S, base);
          },
          [&](auto S, int t) {
            constexpr int s = decltype(S)::value;
            const int kb = kept[t];
            const int base = kb * BN;
            if (!active || listed(myq, kb)) return;
            if (base > qwlast + a.off) return;  // past every row of this wave on every line
            const int sh = max(rw - base, 0) & 31;
            const int j = (max(rw - base, 0) >> 5) - win0(base);
            const uint32_t m0 = mwl[s][j], m1 = mwl[s][j + 1], m2 = mwl[s][j + 2];
            const uint32_t m3 = mwl[s][kMaskOffWords], m4 = mwl[s][kMaskOffWords + 1];
            // offsets: bit x of (d1:d0) is local key c = 59 - x; reversed and shifted, bit c
            const uint32_t d0 = __builtin_amdgcn_alignbit(m1, m0, sh);
            const uint32_t d1 = __builtin_amdgcn_alignbit(m2, m1, sh);
            const uint32_t r0 = __builtin_bitreverse32(d1), r1 = __builtin_bitreverse32(d0);
            // listed columns: bit c is key base + 4h + c
            const uint32_t c0w = __builtin_amdgcn_alignbit(m4, m3, 4 * h);
            const uint32_t c1w = m4 >> (4 * h);
            // visible keys of unit u: bit 8*(j/4) + j%4 of vis[u] for slot j
            const uint32_t vis0 = ((r0 >> 4) | (r1 << 28)) & ~c0w;
            const uint32_t vis1 = (r1 >> 4) & ~c1w;
            // a line crossing the tile within the pair's rows may miss this wave's rows
            if (!__any((vis0 | vis1) != 0u)) return;
            // no mask when every slot of both units is visible in every lane
            constexpr uint32_t kSlots = 0x0F0F0F0Fu;
            const bool full = __all((vis0 & vis1 & kSlots) == kSlots);
            tile_math_mask<D>(a, ws, stage(S), !full, [&](auto U, f32x16& sc) {
              const uint32_t vis = decltype(U)::value == 0 ? vis0 : vis1;
#pragma unroll
              for (int jj = 0; jj < 16; ++jj)
                if (!((vis >> (8 * (jj >> 2) + (jj & 3))) & 1u)) sc[jj] = -INFINITY;
            }, l);
          });
    }

    // ---- phase 3b: isolated slash lines (no neighbour offset listed). On the line at offset
    // o the wave's rows qw0 .. qw0+31 meet the 32 consecutive keys qw0+off-o .. +31, one key
    // per row (the diagonal of that key range). Each wave copies those keys into its own LDS
    // slot (two slots per ring stage, free after phase 3a's last barrier), waits for its own
    // copies only, and runs them as one unit whose mask keeps the diagonal: no workgroup
    // barrier, and one unit of math per line instead of the two masked 64-key tiles the line
    // crosses. A key already counted (a listed column, or inside a block the wave's query
    // block lists) is masked.
    // The isolated offsets that reach the group's rows are first compacted into kept[] (256
    // list entries per pass), so each line costs one LDS read before its copy.
    {
      using W = WinCfg<D>;
      const uint32_t slot = (uint32_t)__builtin_amdgcn_readfirstlane(
          lds_addr(wu < 2 ? st0 : st1) + (uint32_t)(wu & 1) * (uint32_t)W::BYTES);
      // the wave's two column-bitmap words, past both slots of its stage
      const uint32_t cw = (uint32_t)__builtin_amdgcn_readfirstlane(
          lds_addr(wu < 2 ? st0 : st1) + 2u * (uint32_t)W::BYTES + 256u * (uint32_t)(wu & 1));
      const uint32_t* const rbits = a.rl_bits + (int64_t)bh * a.bits_words;
      const int* const sidx = a.sl_idx;
      const int i = l & 31, h = l >> 5;
      // the accumulator slot that holds local key i (this lane's row) in this lane, or -1
      const int jdiag = (((i >> 2) & 1) == h) ? 4 * (i >> 3) + (i & 3) : -1;
      const int s0 = a.sl_ptr[bh], s1 = a.sl_ptr[bh + 1];
      const int omax = qlast + a.off;  // larger offsets meet no row of the group
      for (int seg = s0; seg < s1; seg += kSeg) {
        if (sidx[seg] > omax) break;  // ascending
        // Thread tid holds entry seg + tid of the pass: its offset, read once, and whether it is
        // an isolated line in reach. A pass without one is skipped after one barrier.
        int my_o = -1;
        bool my_iso = false;
        if (seg + tid < s1) {
          my_o = sidx[seg + tid];
          my_iso = my_o >= 0 && my_o <= omax && my_o < a.Lk &&
                   ((rbits[(my_o + 128) >> 5] >> ((my_o + 128) & 31)) & 1u) == 0u;
        }
        if (!__syncthreads_or(my_iso)) continue;
        // with kSeg == NT, compact evaluates entry e = tid in thread tid
        const int cnt = compact(min(kSeg, s1 - seg), [&](int) { return my_iso; },
                                [&](int) { return my_o; });
        if (active) {
          // lines 0 .. n-1 of this pass reach the wave's rows: kept[] ascends, so they are the
          // entries at or below the wave's last row's offset limit, counted by ballots
          int n = 0;
          for (int i0 = 0; i0 < cnt; i0 += 64) {
            const int i = i0 + l;
            n += __popcll(__ballot(i < cnt && kept[i] <= qwlast + a.off));
          }
          n = __builtin_amdgcn_readfirstlane(n);  // wave-uniform: scalar loop control
          // Software pipeline over the wave's lines: K (with its column words) of line t+1 is
          // copied during the softmax and P·V of line t, V of line t+1 during the scores of
          // line t+1; the counted waits leave the other half's copies in flight.
          auto k0_of = [&](int t) { return qw0 + a.off - kept[t]; };
          if (n > 0) {
            issue_window_k<D>(slot, cw, kbp, k_row_bytes, cbits, k0_of(0), lkm1, l);
            issue_window_v<D>(slot, vbp, v_row_bytes, k0_of(0), lkm1, l);
          }
          for (int t = 0; t < n; ++t) {
            const int k0 = k0_of(t);
            wait_vmcnt_le<kWinVCopies<D>>();  // K and column words of line t landed
            const int key = k0 + i;
            bool keep = jdiag >= 0 && key >= 0 && row < Lq;
            if (keep) {
              const uint32_t cwd = *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(
                  cw + 4u * (uint32_t)((key >> 5) - (max(k0, 0) >> 5)));
              keep = ((cwd >> (key & 31)) & 1u) == 0u && !listed(myq, key >> 6);
            }
            bf16x8 p[2];
            window_scores<D>(a, ws, slot, keep ? jdiag : -1, l, p);
            const bool more = t + 1 < n;
            if (more) issue_window_k<D>(slot, cw, kbp, k_row_bytes, cbits, k0_of(t + 1), lkm1, l);
            if (more) wait_vmcnt_le<kWinKCopies<D>>();  // V of line t landed
            else wait_dma_all();
            window_pv<D>(ws, slot, p);
            if (more) issue_window_v<D>(slot, vbp, v_row_bytes, k0_of(t + 1), lkm1, l);
          }
        }
        __syncthreads();  // kept[] free for the next pass
      }
    }
  }
  store_out<D>(ws, obase, o_sl, lse_row, row, Lq, l);
}

// Per (b, h): bitmap of the listed slash offsets (bit o + 128, so a lane's window never starts
// below bit 0), of the listed columns (bit j), and of the listed offsets that have a listed
// neighbour offset (o - 1 or o + 1: the line lies inside a run of lines), nbw words each;
// out-of-range entries are ignored. The offsets are first collected in LDS, so the
// neighbour test reads a complete bitmap.
constexpr int kVsBitsMaxWords = vs_bits_words(kVslashMaxLk);

__global__ __launch_bounds__(256) void vs_bits_kernel(const FwdArgs a) {
  __shared__ uint32_t lb[kVsBitsMaxWords];
  const int bh = (int)blockIdx.x;
  const int nw = a.bits_words;
  uint32_t* sb = const_cast<uint32_t*>(a.sl_bits) + (int64_t)bh * nw;
  uint32_t* cb = const_cast<uint32_t*>(a.cl_bits) + (int64_t)bh * nw;
  uint32_t* rb = const_cast<uint32_t*>(a.rl_bits) + (int64_t)bh * nw;
  for (int i = (int)threadIdx.x; i < nw; i += 256) {
    lb[i] = 0u;
    cb[i] = 0u;
    rb[i] = 0u;
  }
  __threadfence();
  __syncthreads();
  const int s0 = a.sl_ptr[bh], s1 = a.sl_ptr[bh + 1];
  for (int i = s0 + (int)threadIdx.x; i < s1; i += 256) {
    const int o = a.sl_idx[i];
    if (o >= 0 && o < a.Lk) atomicOr(&lb[(o + 128) >> 5], 1u << ((o + 128) & 31));
  }
  for (int i = a.col_ptr[bh] + (int)threadIdx.x; i < a.col_ptr[bh + 1]; i += 256) {
    const int j = a.col_idx[i];
    if (j >= 0 && j < a.Lk) atomicOr(&cb[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  auto bit = [&](int x) { return (lb[x >> 5] >> (x & 31)) & 1u; };
  for (int i = (int)threadIdx.x; i < nw; i += 256) sb[i] = lb[i];
  for (int i = s0 + (int)threadIdx.x; i < s1; i += 256) {
    const int o = a.sl_idx[i];
    if (o < 0 || o >= a.Lk) continue;
    const int x = o + 128;
    if (bit(x - 1) | bit(x + 1)) atomicOr(&rb[x >> 5], 1u << (x & 31));
  }
}

// Query blocks per workgroup.
constexpr int kSparseQB = 2;

template <int D, bool SLASH>
hipError_t launch_sparse_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int QB = kSparseQB;
  const int64_t nwg = (int64_t)a.B * a.Hq * ((a.n_qtiles + QB - 1) / QB);
  FwdArgs aa = a;
  aa.xcd_remap = (nwg % 128 == 0) ? 1 : 0;
  if constexpr (SLASH)
    hipLaunchKernelGGL(vs_bits_kernel, dim3((unsigned)(a.B * a.Hq)), dim3(256), 0, stream, aa);
  hipLaunchKernelGGL((fwd_sparse_kernel<D, SLASH, QB>), dim3((unsigned)nwg), dim3(2 * QB * 64),
                     0, stream, aa);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_blocksparse(const FwdArgs& a, int d, hipStream_t stream) {
  if (d == 128) return launch_sparse_t<128, false>(a, stream);
  return launch_sparse_t<64, false>(a, stream);
}

hipError_t launch_fwd_vslash(const FwdArgs& a, int d, hipStream_t stream) {
  if (d == 128) return launch_sparse_t<128, true>(a, stream);
  return launch_sparse_t<64, true>(a, stream);
}

}  // namespace attn
