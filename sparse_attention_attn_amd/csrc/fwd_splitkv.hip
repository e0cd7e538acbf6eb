// fwd_splitkv.hip — split-KV decode partials and their log-sum-exp combine, on gfx950.
//
// Decode has very few query rows (Lq = 1..2) against a long KV cache ("Resumen Técnico:
// FlashMLA-ETAP", section "Planteamiento del Problema": 1–2 query tokens, KV up to 64K, and
// memory-bandwidth pressure from the long context). The kernel is therefore built so that the
// HBM read of the KV cache is the bound:
//
//  * Work decomposition: one 4-wave workgroup per (batch, KV head, 16-column query block,
//    split). The query columns are all (query head of the GQA group, query position) pairs
//    that share the KV head, so the cache is read once per KV head, not once per query head.
//    For the MLA shape (16 heads over one latent KV head, "Detalles de Implementación" and
//    "Limitaciones Notadas por los Autores") the 16 heads fill one 16-column MFMA block.
//  * Keys stream through an NST-stage LDS ring filled by asynchronous global->LDS copies
//    (non-temporal: the cache is read once); each tile is waited for with a counted vmcnt so
//    NST-1 tiles stay in flight.
//  * Each wave forms the whole score tile Sᵀ = K·Qᵀ (16x16x32 bf16 MFMA, keys as rows, query
//    columns as N) and its softmax statistics, then accumulates its own quarter of the output
//    columns, Oᵀ += Vᵀ·Pᵀ. For MLA, V is the first 512 columns of the same LDS tile that fed
//    K, so the latent cache is read from HBM once.
//  * Every split writes its normalised partial O_s (fp32) and LSE_s; attn_combine_lse merges
//    them with weights exp(LSE_s - max LSE).

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "validate.hpp"

namespace attn {
namespace {

__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  if constexpr (N == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    // gfx9 encoding: vmcnt[3:0] at bits 3:0, vmcnt[5:4] at bits 15:14, expcnt 6:4 and
    // lgkmcnt 11:8 left at their maxima (no wait on them).
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  }
}

template <int DQK, int DV, int BNK, int NST>
struct SplitCfg {
  static constexpr bool MLA = (DQK != DV);          // V is the first DV columns of the K tile
  static constexpr int KT_BYTES = BNK * DQK * 2;
  static constexpr int VT_BYTES = MLA ? 0 : BNK * DV * 2;
  static constexpr int STAGE = KT_BYTES + VT_BYTES;
  static constexpr int KINSTR = KT_BYTES / 1024;
  static constexpr int NINSTR = (KT_BYTES + VT_BYTES) / 1024;
  static constexpr int IPW = NINSTR / 4;            // DMA instructions per wave per tile
  static constexpr int QSTEPS = DQK / 32;
  static constexpr int KBLK = BNK / 16;
  static constexpr int DVW = DV / 4;                // output columns per wave
  static constexpr int DVB = DVW / 16;
  static constexpr int PVSTEPS = BNK / 32;
  static constexpr int VW = MLA ? DQK : DV;         // row width of the tile V is read from
  static_assert(NINSTR % 4 == 0, "tile must split evenly over 4 waves");
  static_assert(KT_BYTES % 1024 == 0, "K tile must be whole KiB");
};

template <int N>
using ic = std::integral_constant<int, N>;

// dma16_sbase with the non-temporal cache policy: every K/V byte of a decode step is read
// exactly once, so the copies stream past the caches instead of allocating lines that no
// later read hits. Measured per step against the default policy (paired runs on one box):
// GQA 4K decode 50.8-51.1 -> 48.2-48.5 us, MLA 64K decode 111.3-111.5 -> 101.7-102.0 us.
// (The device-scope policy, sc1, measured the same as the default.) The prefill and sparse
// kernels keep the default policy: their K/V tiles are re-read by other workgroups from L2.
__device__ __forceinline__ void dma16_sbase_stream(const void* sbase, uint32_t voff,
                                                   uint32_t lds) {
  const uint64_t p = (uint64_t)(uintptr_t)sbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint64_t ps = ((uint64_t)hi << 32) | (uint64_t)lo;
  // s_nop 4: the wait states dma16_sbase documents (VALU-written SGPR, SALU-written M0)
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(ps),
               "{m0}"((uint32_t)__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

template <int DQK, int DV, int BNK, int NST, int NCB>
__global__ __launch_bounds__(256) void splitkv_kernel(const SplitArgs a) {
  using C = SplitCfg<DQK, DV, BNK, NST>;
  static_assert(NCB == 1 || NCB == 2, "one or two 16-column blocks per workgroup");
  static_assert(NST >= 2 && NST <= 6, "2..6 stages");
  // One array per ring stage: with the stage fixed at compile time the compiler can tell the
  // stage being read from the stages still being filled, and does not wait for those copies.
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE];
  // stages beyond NST are 4-byte stubs, so that a 2-stage ring fits twice in one CU's LDS
  __shared__ __attribute__((aligned(NST > 2 ? 1024 : 4))) char st2[NST > 2 ? C::STAGE : 4];
  __shared__ __attribute__((aligned(NST > 3 ? 1024 : 4))) char st3[NST > 3 ? C::STAGE : 4];
  __shared__ __attribute__((aligned(NST > 4 ? 1024 : 4))) char st4[NST > 4 ? C::STAGE : 4];
  __shared__ __attribute__((aligned(NST > 5 ? 1024 : 4))) char st5[NST > 5 ? C::STAGE : 4];
  // MLA: the 4 waves split the Dqk reduction of Sᵀ and add their partial score tiles here.
  constexpr bool KSPLIT = C::MLA;
  constexpr int QW = KSPLIT ? (C::QSTEPS + 3) / 4 : C::QSTEPS;  // Qᵀ steps held per wave
  __shared__ f32x4 xbuf[KSPLIT ? 4 * NCB * C::KBLK * 64 : 1];
  auto stage = [&](auto S) -> char* {
    constexpr int s = decltype(S)::value;
    if constexpr (s == 0) return st0;
    else if constexpr (s == 1) return st1;
    else if constexpr (s == 2) return st2;
    else if constexpr (s == 3) return st3;
    else if constexpr (s == 4) return st4;
    else return st5;
  };

  const int tid = (int)threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l = tid & 63;
  // Block order: KV head fastest, so the workgroups running together read the same key rows
  // of a [B, L, H, D] cache for all heads (one contiguous stretch of memory per key range).
  int lid = (int)blockIdx.x;
  const int hkv = lid % a.Hkv;
  lid /= a.Hkv;
  const int sp = lid % a.num_splits;
  lid /= a.num_splits;
  const int cb = lid % a.ncolblk;
  const int b = lid / a.ncolblk;

  // The workgroup's query columns: NCB blocks of 16; lane l holds column l%16 of each block.
  const int ncols = a.g * a.Lq;
  bool col_ok[NCB];
  int pos[NCB], hq[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const int col = (cb * NCB + c) * 16 + (l & 15);
    col_ok[c] = col < ncols;
    pos[c] = col_ok[c] ? col / a.g : 0;
    hq[c] = hkv * a.g + (col_ok[c] ? col % a.g : 0);
  }

  // keys of this split, cut by the causal horizon of the workgroup's last column
  const int kstart = sp * a.chunk;
  int kend = min(a.Lk, kstart + a.chunk);
  const int last_col = min(ncols, (cb + 1) * NCB * 16) - 1;
  const int first_pos = (cb * NCB * 16) / a.g;
  const int last_pos = last_col / a.g;
  if (a.causal) kend = min(kend, last_pos + a.off + 1);
  // split bounds are uniform over the workgroup: keep them in scalar registers so the ring's
  // branches stay scalar
  kend = __builtin_amdgcn_readfirstlane(kend);
  const int ntiles = __builtin_amdgcn_readfirstlane(kend > kstart ? (kend - kstart + BNK - 1) / BNK : 0);
  // Tile order. Workgroup (b, split) starts its walk at tile rot = ntiles * r / (B * S) of its
  // split, r = b * S + split, and wraps around, so the workgroups running together read at
  // positions spread evenly over their key ranges instead of all at the same offset of
  // ranges that lie a fixed power-of-two apart. The result does not depend on the order (the
  // masks and the ragged tail follow each tile's key position; the softmax takes no running
  // maximum). Measured per call (rotating KV copies): 1 to 13% faster for D = 64 and for
  // D = 128 with 8 or more KV heads. It was 2 to 8% slower for D = 128 with 2 or 4 KV heads
  // and for the latent shape: those keep the plain order.
  const bool spread = !C::MLA && (DQK == 64 || a.Hkv >= 8);
  const int rot = __builtin_amdgcn_readfirstlane(
      spread && ntiles > 0
          ? (int)((((int64_t)b * a.num_splits + sp) * ntiles) / ((int64_t)a.B * a.num_splits))
          : 0);
  auto phys = [&](int t) {  // tile t of the walk -> tile index within the split
    const int p = t + rot;
    return p >= ntiles ? p - ntiles : p;
  };

  // Qᵀ operand: lane l holds column l%16, head-dim elements 32*s + 8*(l/16) .. +7
  // With KSPLIT, wave w holds the reduction steps [qs0, qs1) only (4 or 5 of 18 for MLA).
  const int qs0 = KSPLIT ? (C::QSTEPS * w) / 4 : 0;
  const int qs1 = KSPLIT ? (C::QSTEPS * (w + 1)) / 4 : C::QSTEPS;
  bf16x8 qop[NCB][QW];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const uint16_t* qr =
        a.q + (int64_t)b * a.q_sb + (int64_t)pos[c] * a.q_sl + (int64_t)hq[c] * a.q_sh;
#pragma unroll
    for (int i = 0; i < QW; ++i) {
      const int s = qs0 + i;
      qop[c][i] = (col_ok[c] && s < qs1) ? load_q_bf16x8(qr + 32 * s + 8 * (l >> 4), a.qsign) : zero_bf16x8();
    }
  }
  // Use the loaded operands here, before the copy ring starts: the compiler then waits for
  // these loads once, instead of at their first use inside the loop, where its wait would
  // also drain the tile copies in flight.
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int i = 0; i < QW; ++i) asm volatile("" ::"v"(qop[c][i]));

  const uint16_t* kb = a.k + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh;
  const uint16_t* vb = a.v + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh;
  const int kmax = kend - 1;

  // Per-lane source byte offsets (relative to the tile's first key row) of this wave's copy
  // instructions; instruction ii of wave w is tile copy w + 4*ii. `maxrow` < BNK-1 clamps the
  // rows of the last tile of a split to its last key (those rows are masked later).
  auto lane_offset = [&](int i, int maxrow) -> uint32_t {
    const bool is_k = C::MLA || i < C::KINSTR;
    const int li = is_k ? i : i - C::KINSTR;
    const uint32_t slot = (uint32_t)li * 64u + (uint32_t)l;
    const uint32_t cpr = is_k ? DQK / 8 : DV / 8;
    const uint32_t r = slot / cpr;
    const uint32_t c = (slot % cpr) ^ (is_k ? Swz<DQK>::f(r) : Swz<(C::MLA ? DQK : DV)>::f(r));
    const uint32_t rc = min(r, (uint32_t)maxrow);
    return (rc * (uint32_t)(is_k ? a.k_sl : a.v_sl) + c * 8u) * 2u;
  };
  uint32_t src_off[C::IPW];
#pragma unroll
  for (int ii = 0; ii < C::IPW; ++ii) src_off[ii] = lane_offset(w + 4 * ii, BNK - 1);

  // The copies are issued with the scalar-base instruction, which the compiler does not track:
  // it adds no waits of its own for them, and the ring below orders them with counted vmcnt
  // waits and barriers.
  auto issue = [&](auto S, int t) {
    const uint32_t st = lds_addr(stage(S));
    const int base = kstart + phys(t) * BNK;
    const bool tail = base + BNK - 1 > kmax;
    const uint16_t* kt = kb + (int64_t)base * a.k_sl;
    const uint16_t* vt = vb + (int64_t)base * a.v_sl;
#pragma unroll
    for (int ii = 0; ii < C::IPW; ++ii) {
      const int i = w + 4 * ii;
      const bool is_k = C::MLA || i < C::KINSTR;
      const int li = is_k ? i : i - C::KINSTR;
      const uint32_t dst = st + (is_k ? 0u : (uint32_t)C::KT_BYTES) + (uint32_t)li * 1024u;
      const uint32_t off = tail ? lane_offset(i, kmax - base) : src_off[ii];
      dma16_sbase_stream(is_k ? (const void*)kt : (const void*)vt, off, dst);
    }
  };

  // Per column block: Oᵀ accumulators; m: reference maximum (exp2 domain), -inf before any
  // visible key; mu: m where finite, +inf otherwise; sb / sf: lane-partial sums of the
  // bf16-rounded and of the fp32 weights.
  f32x4 acc[NCB][C::DVB];
  float m[NCB], mu[NCB], sb[NCB], sf[NCB];
  int lim[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
#pragma unroll
    for (int i = 0; i < C::DVB; ++i) acc[c][i] = f32x4{};
    m[c] = -INFINITY;
    mu[c] = INFINITY;
    sb[c] = 0.f;
    sf[c] = 0.f;
    lim[c] = a.causal ? pos[c] + a.off : 0x7fffffff;
  }

  const int G = l >> 4;
  const int jj = (l & 15) >> 2;
  const int cc = l & 3;
  const uint32_t krow = (uint32_t)(l & 15);

  auto compute = [&](auto S, int t) {
    const char* kt = stage(S);
    const char* vt = C::MLA ? kt : kt + C::KT_BYTES;
    const int base = kstart + phys(t) * BNK;

    // ---- Sᵀ: per column block, KBLK blocks of 16 keys x 16 columns
    f32x4 st[NCB][C::KBLK];
    auto kread = [&](int s, int k) {
      const uint32_t r = 16u * k + krow;
      const uint32_t c = (uint32_t)(4 * s + G);
      return lds_read_bf16x8(kt, (r * (DQK / 8) + (c ^ Swz<DQK>::f(r))) * 16u);
    };
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int k = 0; k < C::KBLK; ++k) st[c][k] = f32x4{};
    if constexpr (KSPLIT) {
      // this wave's share of the reduction, then the sum of the four partial tiles (added in
      // wave order, so every wave holds the same scores and the same softmax state)
#pragma unroll
      for (int i = 0; i < QW; ++i) {
        if (i + 1 < QW || qs0 + i < qs1) {
#pragma unroll
          for (int k = 0; k < C::KBLK; ++k) {
            const bf16x8 kk = kread(qs0 + i, k);
#pragma unroll
            for (int c = 0; c < NCB; ++c) st[c][k] = mfma16(kk, qop[c][i], st[c][k]);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int k = 0; k < C::KBLK; ++k) xbuf[((w * NCB + c) * C::KBLK + k) * 64 + l] = st[c][k];
      // LDS writes of all waves done; the copy ring's loads stay in flight
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int k = 0; k < C::KBLK; ++k) {
          f32x4 sum = xbuf[(c * C::KBLK + k) * 64 + l];
#pragma unroll
          for (int ww = 1; ww < 4; ++ww) sum += xbuf[((ww * NCB + c) * C::KBLK + k) * 64 + l];
          st[c][k] = sum;
        }
    } else {
      // K operands of step s read RA steps ahead (about 64 MFMA cycles of cover, more than
      // the LDS latency): with one wave per SIMD nothing else hides that latency.
      constexpr int RA = C::KBLK >= 4 ? 1 : 3;
      static_assert(C::QSTEPS > RA, "read-ahead deeper than the reduction");
      bf16x8 kr[RA + 1][C::KBLK];
#pragma unroll
      for (int s = 0; s < RA; ++s)
#pragma unroll
        for (int k = 0; k < C::KBLK; ++k) kr[s][k] = kread(s, k);
      static_for<0, C::QSTEPS>([&](auto SI) {
        constexpr int s = decltype(SI)::value;
#pragma unroll
        for (int k = 0; k < C::KBLK; ++k)
#pragma unroll
          for (int c = 0; c < NCB; ++c)
            st[c][k] = mfma16(kr[s % (RA + 1)][k], qop[c][s], st[c][k]);
        // refill the slot consumed one step earlier
        if constexpr (s + RA < C::QSTEPS) {
#pragma unroll
          for (int k = 0; k < C::KBLK; ++k) kr[(s + RA) % (RA + 1)][k] = kread(s + RA, k);
        }
      });
    }
    // ---- mask: slot (k, j) holds key base + 16*k + 4*(l/16) + j
    const bool need_mask = (base + BNK > kend) || (a.causal && base + BNK - 1 > first_pos + a.off);
    if (need_mask) {
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int k = 0; k < C::KBLK; ++k)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = base + 16 * k + 4 * G + j;
            if (key >= kend || key > lim[c]) st[c][k][j] = -INFINITY;
          }
    }
    // ---- weights against the column's reference mu, with no maximum taken; the running
    // fp32 sum then decides whether the tile was safe, else the slow path moves the reference
    f32x4 pw[NCB][C::KBLK];
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      float sfn = sf[c];
#pragma unroll
      for (int k = 0; k < C::KBLK; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pw[c][k][j] = fast_exp2(fmaf(st[c][k][j], a.sl2, -mu[c]));
          sfn += pw[c][k][j];
        }
      if (__builtin_expect(__any(!sum_ok(sfn)), 0)) {
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < C::KBLK; ++k)
#pragma unroll
          for (int j = 0; j < 4; ++j) mx = fmaxf(mx, st[c][k][j]);
        mx = fmaxf(mx, xor_shuffle(mx, 16));
        mx = fmaxf(mx, xor_shuffle(mx, 32));
        const float mnew = fmaxf(m[c], mx * a.sl2);
        const float munew = (mnew == -INFINITY) ? INFINITY : mnew;
        // 0 while nothing was accumulated, 1 if unmoved
        const float alpha = fast_exp2(m[c] - munew);
#pragma unroll
        for (int i = 0; i < C::DVB; ++i) acc[c][i] *= alpha;
        sb[c] *= alpha;
        sf[c] *= alpha;
        sfn = sf[c];
#pragma unroll
        for (int k = 0; k < C::KBLK; ++k)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pw[c][k][j] = fast_exp2(fmaf(st[c][k][j], a.sl2, -munew));
            sfn += pw[c][k][j];
          }
        m[c] = mnew;
        mu[c] = munew;
      }
      sf[c] = sfn;
    }

    // ---- Oᵀ += Vᵀ·Pᵀ over 32-key steps. Operand slot i of lane l covers key
    // 32*ps + 16*(i/4) + 4*(l/16) + i%4 (blocks 2ps and 2ps+1 of Sᵀ). Every V operand feeds
    // the MFMAs of all column blocks. The bf16 sum is taken over the packed weights the MFMAs
    // multiply.
#pragma unroll
    for (int ps = 0; ps < C::PVSTEPS; ++ps) {
      bf16x8 pop[NCB];
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const f32x4& x0 = pw[c][2 * ps];
        const f32x4& x1 = pw[c][2 * ps + 1];
        const uint4 pq = make_uint4(pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]),
                                    pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3]));
        sb[c] = add_bf16_pair(pq.x, sb[c]);
        sb[c] = add_bf16_pair(pq.y, sb[c]);
        sb[c] = add_bf16_pair(pq.z, sb[c]);
        sb[c] = add_bf16_pair(pq.w, sb[c]);
        pop[c] = __builtin_bit_cast(bf16x8, pq);
      }
      const uint32_t rlo = (uint32_t)(32 * ps + 4 * G + jj);
      bf16x8 vop[C::DVB];
#pragma unroll
      for (int i = 0; i < C::DVB; ++i) {
        const uint32_t dv = (uint32_t)(w * C::DVW + 16 * i + 4 * cc);
        vop[i] = lds_read_tr_pair(vt, elem_off<C::VW>(rlo, dv), elem_off<C::VW>(rlo + 16, dv));
      }
#pragma unroll
      for (int i = 0; i < C::DVB; ++i)
#pragma unroll
        for (int c = 0; c < NCB; ++c) acc[c][i] = mfma16(vop[i], pop[c], acc[c][i]);
    }
  };

  // One ring step: tile t sits in stage S; copies of the next NST-2 tiles may stay in flight.
  auto step = [&](auto S, int t) {
    constexpr int s = decltype(S)::value;
    if (t + NST - 2 < ntiles) wait_vmcnt<C::IPW * (NST - 2)>();
    else wait_vmcnt<0>();
    barrier_no_fence();
    if (t + NST - 1 < ntiles) issue(ic<(s + NST - 1) % NST>{}, t + NST - 1);
    compute(S, t);
  };

  if (0 < ntiles) issue(ic<0>{}, 0);
  if (NST > 2 && 1 < ntiles) issue(ic<1>{}, 1);
  if (NST > 3 && 2 < ntiles) issue(ic<2 % NST>{}, 2);
  if (NST > 4 && 3 < ntiles) issue(ic<3 % NST>{}, 3);
  if (NST > 5 && 4 < ntiles) issue(ic<4 % NST>{}, 4);
  for (int t = 0; t < ntiles; t += NST) {
    step(ic<0>{}, t);
    if (t + 1 < ntiles) step(ic<1>{}, t + 1);
    if constexpr (NST > 2) { if (t + 2 < ntiles) step(ic<2 % NST>{}, t + 2); }
    if constexpr (NST > 3) { if (t + 3 < ntiles) step(ic<3 % NST>{}, t + 3); }
    if constexpr (NST > 4) { if (t + 4 < ntiles) step(ic<4 % NST>{}, t + 4); }
    if constexpr (NST > 5) { if (t + 5 < ntiles) step(ic<5 % NST>{}, t + 5); }
  }

  // ---- partial outputs of this split
  // O_s is normalised by the sum of the bf16 weights the MFMAs multiplied (a column dominated
  // by one key returns its value exactly); LSE_s comes from the fp32 sum.
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    float tb = sb[c] + xor_shuffle(sb[c], 16);
    tb = tb + xor_shuffle(tb, 32);
    float tf = sf[c] + xor_shuffle(sf[c], 16);
    tf = tf + xor_shuffle(tf, 32);
    if (!col_ok[c]) continue;
    const float inv = tb > 0.f ? 1.0f / tb : 0.f;
    if (a.o != nullptr) {  // the only split: final O and LSE, no combine
      uint16_t* orow = a.o + (int64_t)b * a.o_sb + (int64_t)pos[c] * a.o_sl +
                       (int64_t)hq[c] * a.o_sh;
#pragma unroll
      for (int i = 0; i < C::DVB; ++i) {
        const int dv = w * C::DVW + 16 * i + 4 * G;
        uint2 pk;
        pk.x = pack_bf16x2(acc[c][i][0] * inv, acc[c][i][1] * inv);
        pk.y = pack_bf16x2(acc[c][i][2] * inv, acc[c][i][3] * inv);
        *reinterpret_cast<uint2*>(orow + dv) = pk;
      }
      if (a.lse != nullptr && w == 0 && G == 0)
        a.lse[((int64_t)b * a.Hq + hq[c]) * a.Lq + pos[c]] =
            tf > 0.f ? m[c] * kLn2 + logf(tf) : -INFINITY;
      continue;
    }
    const int64_t prow = (((int64_t)sp * a.B + b) * a.Hq + hq[c]) * a.Lq + pos[c];
    float* op = a.o_part + prow * DV;
    // Non-temporal stores: the partials are read once, by the combine launch, so they stream
    // out instead of sitting dirty in this XCD's L2 until the end-of-kernel write-back (MLA
    // 64K decode, 8 MB of partials: 112.6-113.0 -> 111.3-111.4 us per step; GQA unchanged).
#pragma unroll
    for (int i = 0; i < C::DVB; ++i) {
      const int dv = w * C::DVW + 16 * i + 4 * G;
      const f32x4 val = {acc[c][i][0] * inv, acc[c][i][1] * inv, acc[c][i][2] * inv,
                         acc[c][i][3] * inv};
      __builtin_nontemporal_store(val, reinterpret_cast<f32x4*>(op + dv));
    }
    if (w == 0 && G == 0) a.lse_part[prow] = tf > 0.f ? m[c] * kLn2 + logf(tf) : -INFINITY;
  }
}

// ------------------------------------------------------------------------------------------
// Combine: M = max_s LSE_s, w_s = exp(LSE_s - M), LSE = M + ln Σ w_s, O = Σ w_s O_s / Σ w_s.
// One workgroup per output row (b, query head, position). Its 256 threads are CPB float4
// columns x G split groups; group g takes splits g, g+G, ..., up to kCombineInFlight of them per
// pass with every load issued before any is used (one memory round trip for up to
// G * kCombineInFlight splits). A group keeps its own running maximum m_g; the groups meet in
// LDS, each scaled by exp(m_g - M). A split with no visible key (LSE_s = -inf) has weight 0.
// ------------------------------------------------------------------------------------------
constexpr int kCombineInFlight = 16;

template <int DV>
__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
  constexpr int CPB = DV / 4;       // float4 columns per row
  constexpr int G = 256 / CPB;      // split groups
  constexpr int U = kCombineInFlight;
  static_assert(CPB <= 256 && 256 % CPB == 0, "row must fit one workgroup");
  __shared__ float4 red[G][CPB];
  __shared__ float gmax[G];
  __shared__ float gden[G];
  const int64_t rows = (int64_t)a.B * a.Hq * a.Lq;
  const int64_t row = blockIdx.x;
  const int c4 = threadIdx.x % CPB;
  const int grp = threadIdx.x / CPB;

  float m = -INFINITY, den = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = grp; s0 < a.S; s0 += U * G) {
    float ls[U];
    float4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * G;
      if (s < a.S) {
        ls[u] = a.lse_part[(int64_t)s * rows + row];
        x[u] = *reinterpret_cast<const float4*>(a.o_part + ((int64_t)s * rows + row) * DV + 4 * c4);
      } else {
        ls[u] = -INFINITY;
        x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float cm = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) cm = fmaxf(cm, ls[u]);
    if (cm > m) {  // move this group's reference (exp(-inf) = 0 clears the first pass)
      const float r = expf(m - cm);
      den *= r;
      o.x *= r; o.y *= r; o.z *= r; o.w *= r;
      m = cm;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = (ls[u] == -INFINITY) ? 0.f : expf(ls[u] - m);
      den += w;
      o.x += w * x[u].x;
      o.y += w * x[u].y;
      o.z += w * x[u].z;
      o.w += w * x[u].w;
    }
  }
  red[grp][c4] = o;
  if (c4 == 0) { gmax[grp] = m; gden[grp] = den; }
  __syncthreads();
  if (grp != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int g = 0; g < G; ++g) M = fmaxf(M, gmax[g]);
  float dt = 0.f;
  float4 ot = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mg = gmax[g];
      const float r = (mg == -INFINITY) ? 0.f : expf(mg - M);
      const float4 v = red[g][c4];
      ot.x += r * v.x; ot.y += r * v.y; ot.z += r * v.z; ot.w += r * v.w;
      dt += r * gden[g];
    }
  }
  const float inv = dt > 0.f ? 1.0f / dt : 0.f;
  const int pos = (int)(row % a.Lq);
  const int hq = (int)((row / a.Lq) % a.Hq);
  const int b = (int)(row / ((int64_t)a.Lq * a.Hq));
  uint16_t* dst = a.o + (int64_t)b * a.o_sb + (int64_t)pos * a.o_sl + (int64_t)hq * a.o_sh + 4 * c4;
  uint2 pk;
  pk.x = pack_bf16x2(ot.x * inv, ot.y * inv);
  pk.y = pack_bf16x2(ot.z * inv, ot.w * inv);
  *reinterpret_cast<uint2*>(dst) = pk;
  if (a.lse != nullptr && c4 == 0) a.lse[row] = dt > 0.f ? M + logf(dt) : -INFINITY;
}

template <int DQK, int DV, int BNK, int NST, int NCB>
hipError_t launch_split_t(const SplitArgs& a, hipStream_t stream) {
  const int64_t nwg = (int64_t)a.B * a.Hkv * a.ncolblk * a.num_splits;
  if (nwg > 0x7fffffff) return hipErrorInvalidConfiguration;  // beyond one grid dimension
  hipLaunchKernelGGL((splitkv_kernel<DQK, DV, BNK, NST, NCB>), dim3((unsigned)nwg), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

// Few splits: one thread per (row, 4 columns), 256 / (DV/4) rows per workgroup, every split's
// partial loaded before any is used. Same formula and split order as combine_kernel's single
// group.
constexpr int kCombineRowsMaxS = 8;

template <int DV>
__global__ __launch_bounds__(256) void combine_rows_kernel(const CombineArgs a) {
  constexpr int CPB = DV / 4;
  constexpr int RPB = 256 / CPB;
  const int64_t rows = (int64_t)a.B * a.Hq * a.Lq;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / CPB;
  const int c4 = threadIdx.x % CPB;
  if (row >= rows) return;
  float ls[kCombineRowsMaxS];
  float4 x[kCombineRowsMaxS];
#pragma unroll
  for (int s = 0; s < kCombineRowsMaxS; ++s) {
    if (s < a.S) {
      ls[s] = a.lse_part[(int64_t)s * rows + row];
      x[s] = *reinterpret_cast<const float4*>(a.o_part + ((int64_t)s * rows + row) * DV + 4 * c4);
    } else {
      ls[s] = -INFINITY;
      x[s] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kCombineRowsMaxS; ++s) M = fmaxf(M, ls[s]);
  float den = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
#pragma unroll
    for (int s = 0; s < kCombineRowsMaxS; ++s) {
      const float w = (ls[s] == -INFINITY) ? 0.f : expf(ls[s] - M);
      den += w;
      o.x += w * x[s].x; o.y += w * x[s].y; o.z += w * x[s].z; o.w += w * x[s].w;
    }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  const int pos = (int)(row % a.Lq);
  const int hq = (int)((row / a.Lq) % a.Hq);
  const int b = (int)(row / ((int64_t)a.Lq * a.Hq));
  uint16_t* dst = a.o + (int64_t)b * a.o_sb + (int64_t)pos * a.o_sl + (int64_t)hq * a.o_sh + 4 * c4;
  uint2 pk;
  pk.x = pack_bf16x2(o.x * inv, o.y * inv);
  pk.y = pack_bf16x2(o.z * inv, o.w * inv);
  *reinterpret_cast<uint2*>(dst) = pk;
  if (a.lse != nullptr && c4 == 0) a.lse[row] = den > 0.f ? M + logf(den) : -INFINITY;
}

template <int DV>
hipError_t launch_combine_t(const CombineArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Hq * a.Lq;
  if (a.S <= kCombineRowsMaxS && DV <= 128) {
    constexpr int RPB = 256 / (DV / 4);
    hipLaunchKernelGGL((combine_rows_kernel<DV>), dim3((unsigned)((rows + RPB - 1) / RPB)),
                       dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((combine_kernel<DV>), dim3((unsigned)rows), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_splitkv(const SplitArgs& a, int dqk, int dv, hipStream_t stream) {
  if (dqk == 576) {
    if (split_cols(dqk, a.g * a.Lq) == 32) return launch_split_t<576, 512, 32, 4, 2>(a, stream);
    return launch_split_t<576, 512, 32, 4, 1>(a, stream);
  }
  // D = 128: grids of at most one workgroup per CU take a 4-stage ring of 32-key tiles (three
  // tiles in flight); larger grids a 2-stage ring of 64-key tiles (64 KiB of LDS) so that two
  // workgroups share a CU (split_ring32 states the rule and its measurements).
  const bool two = split_cols(dqk, a.g * a.Lq) == 32;
  if (dqk == 128) {
    const int64_t nwg = (int64_t)a.B * a.Hkv * a.ncolblk * a.num_splits;
    if (split_ring32(dqk, a.g * a.Lq, nwg)) return launch_split_t<128, 128, 32, 4, 1>(a, stream);
    return two ? launch_split_t<128, 128, 64, 2, 2>(a, stream)
               : launch_split_t<128, 128, 64, 2, 1>(a, stream);
  }
  return two ? launch_split_t<64, 64, 64, 4, 2>(a, stream)
             : launch_split_t<64, 64, 64, 4, 1>(a, stream);
}

hipError_t launch_combine(const CombineArgs& a, int dv, hipStream_t stream) {
  if (dv == 512) return launch_combine_t<512>(a, stream);
  if (dv == 128) return launch_combine_t<128>(a, stream);
  return launch_combine_t<64>(a, stream);
}

}  // namespace attn
