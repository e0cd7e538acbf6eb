// fwd_dense.hip — fused dense attention forward (prefill; causal or not, GQA) on gfx950.
//
// What is computed: O = softmax(scale·Q·Kᵀ + mask)·V and the LSE of every query row ("Resumen
// Técnico: FlashMLA-ETAP", section "Mecanismo Central"), tile by tile with running softmax
// statistics kept on chip ("Activar Flash Attention con llama.cpp para optimizar la
// inferencia", section "¿Qué es Flash Attention y por qué es crucial para llama.cpp?").
//
// Work decomposition. One workgroup of 8 waves owns 256 query rows of one (batch, query head);
// each wave owns one 32-row MFMA block, so every SIMD interleaves the instruction streams of two
// waves. (128-row workgroups of 4 waves, two per CU, measured 3% slower: each then streams its
// own copy of every K/V tile.)
//
// Per 64-key tile and wave, the products are formed transposed (the Sᵀ accumulator holds 16
// keys of ONE query per lane, so the same registers, rounded to bf16, are the B operand Pᵀ of
// Oᵀ += Vᵀ·Pᵀ):  Sᵀ = K·Qᵀ with 32x32x16 bf16 MFMA, K from LDS, Qᵀ in registers; Vᵀ from the
// row-major V tile through the LDS transpose read.
//
// Software pipeline. Iteration t of a wave issues the MFMAs of Sᵀ(t+1) and of Oᵀ += Vᵀ(t-1)·
// Pᵀ(t-1) and, independent of both, the softmax of tile t (max, exp2, bf16 packing, sums) on
// the vector ALU, so a single wave keeps the matrix core and the VALU busy at the same time.
// K/V tiles stream through a 2-stage LDS ring filled by asynchronous global->LDS copies. A stage
// holds K of tile t and V of tile t-1, the two operands that the same pipeline steps read, so
// two stages hide one tile of copy latency: iteration t copies the pair (K(t+2), V(t+1)) while
// the pair (K(t+1), V(t)) is in use. One workgroup barrier per iteration frees the stage of the
// pair (K(t), V(t-1)).
//
// Softmax. Scores live in the exp2 domain (x = s·scale·log2 e). Each row keeps a reference m,
// the largest score seen when it was last set, and weights are exp2(x - m). The reference is
// not moved by every larger score: the weights of a unit are computed against the current m
// with no maximum taken, and only afterwards one compare of the row's updated fp32 sum decides
// whether the unit was safe: the sum must be positive (the row has a reference) and at most
// kSumLimit (no weight can overflow the accumulators; inf and NaN fail too). If any row of the
// wave fails, the wave takes a slow path for that unit: it takes the unit's row maxima, moves
// m, rescales the accumulators and sums, and recomputes the unit's weights. The P·V of a unit
// runs one step after its weights, so the recomputed weights are the ones used. With a
// reference that can lag the true maximum the weights exceed 1, which fp32 and bf16 hold
// exactly as well in relative terms; two row sums are kept: the sum of the bf16-rounded
// weights, which normalises O (numerator and denominator then use the same weights, so a row
// dominated by one key returns that key's value exactly), and the fp32 sum of the unrounded
// weights, which gives the LSE.

#include "tile_io.hpp"

namespace attn {
namespace {

constexpr int kStages = 2;
// Waves per workgroup (each owns 32 query rows): 8 (256 rows, one workgroup per CU) or 4 (128
// rows, two per CU); launch_dense_t picks one per launch.
constexpr int wg_per_cu(int nw) { return nw == 4 ? 2 : 1; }
// MFMA slots between an operand's LDS read and its use.
#ifndef ATTN_DENSE_READ_AHEAD
#define ATTN_DENSE_READ_AHEAD 2
#endif
constexpr int kReadAhead = ATTN_DENSE_READ_AHEAD;
// Row blocks (32 query rows each) per wave of the dense kernel.
constexpr int kDenseNR = 1;

template <int D, int NR>
struct WaveRows {
  bf16x8 qop[NR][TileCfg<D>::KSTEPS];  // Qᵀ operands of the 32-row blocks
  f32x16 acc[NR][TileCfg<D>::DVB];     // Oᵀ accumulators
  float m[NR];                         // reference maxima (exp2 domain), -inf before any key
  float mu[NR];                        // m where finite, +inf otherwise (all weights then 0)
  float lb[NR];                        // lane-partial sums of the bf16-rounded weights
  float lf[NR];                        // lane-partial sums of the fp32 weights
};

// Sᵀ of one 32-key unit (key block kb of the tile whose K part starts at LDS address kt, plus
// this lane's 16-byte offset): s[r] = K(kb) · Qᵀ(r).
template <int D, int NR>
__device__ __forceinline__ void qk_unit(const WaveRows<D, NR>& ws, uint32_t kt, int kb,
                                        f32x16 (&s)[NR]) {
  using C = TileCfg<D>;
#pragma unroll
  for (int r = 0; r < NR; ++r) s[r] = f32x16{};
#pragma unroll
  for (int st = 0; st < C::KSTEPS; ++st) {
    const bf16x8 k = lds_read_b128_at(kt + 1024u * (kb * C::KSTEPS + st));
#pragma unroll
    for (int r = 0; r < NR; ++r) s[r] = mfma32(k, ws.qop[r][st], s[r]);
  }
}

// Masks unit u: slot (r, j) holds key 32*u + 8*(j/4) + 4*(l/32) + j%4 of query row
// qw0 + 32*r + l%32; keys past Lk or past the row's causal horizon get -inf.
template <int NR>
__device__ __forceinline__ void mask_unit(f32x16 (&s)[NR], int u, int qw0, int Lk, int causal,
                                          int off, int l) {
  const int kbase = 32 * u + 4 * (l >> 5);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int lim = causal ? min(Lk - 1, qw0 + 32 * r + (l & 31) + off) : Lk - 1;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = kbase + 8 * (j >> 2) + (j & 3);
      if (key > lim) s[r][j] = -INFINITY;
    }
  }
}

// One pipeline step of a wave, with an explicit issue schedule. It is written as NQ + NV MFMA
// slots (NR MFMAs each, one per row block): the NQ slots of Sᵀ(next) = K·Qᵀ, then the NV slots
// of Oᵀ += Vᵀ·Pᵀ(previous). Each slot is followed by a slice of the softmax of the current unit
// (row maxima, reference moves, then groups of two weights) and by the LDS reads that feed the
// MFMAs two slots later. Scheduling fences keep this order, so the VALU instructions issue
// while the matrix core is busy.
//
//   sc: Sᵀ of the current unit (consumed);   sn: Sᵀ of the next unit (produced)
//   pp: Pᵀ of the previous unit (consumed);  pc: Pᵀ of the current unit (produced)
//   kt/kb: K tile address (lane offset included) and key block of the next unit
//   vt/vkb: V tile address (lane offset included) and key block of the previous unit
//
// Operand slot i of lane l in P·V k-step ks covers unit key 16*ks + 8*(i/4) + 4*(l/32) + i%4,
// which is where the Sᵀ accumulator keeps that key (slot 8*ks + i); the two transposed V
// reads of an operand address rows 16*ks + 4*(l/32) + j and +8 (j = the lane's row inside its
// 16-lane group).
template <int D, int NR>
__device__ __forceinline__ void fused_step(WaveRows<D, NR>& ws, const f32x16 (&sc)[NR],
                                           f32x16 (&sn)[NR], const bf16x8 (&pp)[NR][2],
                                           bf16x8 (&pc)[NR][2], uint32_t kt, int kb, uint32_t vt,
                                           int vkb, float sl2, float (&sb)[NR], float (&sf)[NR],
                                           bool& ok) {
  using C = TileCfg<D>;
  constexpr int NQ = C::KSTEPS;
  constexpr int NV = 2 * C::DVB;
  constexpr int NP = NQ + NV;
  // Softmax items, skewed so that no instruction waits on an exp of its own slot: item k
  // computes the two weights of group k (fma, exp2) and folds in group k-1 (sums, bf16 pack);
  // the last item checks the sums.
  constexpr int NG = 8 * NR;
  constexpr int NITEMS = NG + 2;
  static_assert(NQ >= 2, "K read pipeline depth");

  uint32_t pk[NR][2][4];
  float ew[2][2];  // weights of the last two groups, by group parity
  constexpr int RA = kReadAhead;
  static_assert(NQ >= RA && NV >= RA, "read-ahead deeper than a phase");
  bf16x8 kop[RA], vop[RA + 1];

  auto kread = [&](int st) { return lds_read_b128_at(kt + 1024u * (kb * C::KSTEPS + st)); };
  // P·V slot v covers output column block b = v % DVB and k-step ks = v / DVB, so consecutive
  // slots accumulate into different blocks (no back-to-back dependent MFMAs).
  auto vread = [&](int v) {
    const uint32_t o = vt + (32u * vkb + 16u * (v / C::DVB)) * C::VROW + 64u * (v % C::DVB);
    return lds_read_tr_pair_at(o, o + 8u * C::VROW);
  };
  auto item = [&](auto IT) {
    constexpr int it = decltype(IT)::value;
    if constexpr (it < NG) {
      // group it: scores 8*ks + 2*i and +1 of row block r
      constexpr int r = it >> 3, ks = (it >> 2) & 1, i = it & 3;
      ew[it & 1][0] = fast_exp2(fmaf(sc[r][8 * ks + 2 * i], sl2, -ws.mu[r]));
      ew[it & 1][1] = fast_exp2(fmaf(sc[r][8 * ks + 2 * i + 1], sl2, -ws.mu[r]));
    }
    if constexpr (it >= 1 && it <= NG) {
      constexpr int g = it - 1;
      constexpr int r = g >> 3, ks = (g >> 2) & 1, i = g & 3;
      sf[r] += ew[g & 1][0];
      sf[r] += ew[g & 1][1];
      pk[r][ks][i] = pack_bf16x2(ew[g & 1][0], ew[g & 1][1]);
      sb[r] = add_bf16_pair(pk[r][ks][i], sb[r]);
    }
    if constexpr (it == NG + 1) {
      // 0 < sf <= 2^64 for every row of the lane (bit compare: 0, inf and NaN fail)
      ok = true;
#pragma unroll
      for (int r = 0; r < NR; ++r)
        ok = ok && sum_ok(sf[r]);
    }
  };

#pragma unroll
  for (int r = 0; r < NR; ++r) {
    sb[r] = ws.lb[r];
    sf[r] = ws.lf[r];
  }
#pragma unroll
  for (int i = 0; i < RA; ++i) kop[i] = kread(i);
  __builtin_amdgcn_sched_barrier(0);
  static_for<0, NP>([&](auto PI) {
    constexpr int i = decltype(PI)::value;
    if constexpr (i < NQ) {
      const bf16x8 k = kop[i % RA];
#pragma unroll
      for (int r = 0; r < NR; ++r) sn[r] = mfma32(k, ws.qop[r][i], i == 0 ? f32x16{} : sn[r]);
      if constexpr (i + RA < NQ) kop[i % RA] = kread(i + RA);
      if constexpr (i >= NQ - RA) vop[i - (NQ - RA)] = vread(i - (NQ - RA));
    } else {
      constexpr int v = i - NQ;
      const bf16x8 vv = vop[v % (RA + 1)];
#pragma unroll
      for (int r = 0; r < NR; ++r)
        ws.acc[r][v % C::DVB] = mfma32(vv, pp[r][v / C::DVB], ws.acc[r][v % C::DVB]);
      if constexpr (v + RA < NV) vop[(v + RA) % (RA + 1)] = vread(v + RA);
    }
    static_for<NITEMS * i / NP, NITEMS * (i + 1) / NP>(item);
    __builtin_amdgcn_sched_barrier(0);
  });
#pragma unroll
  for (int r = 0; r < NR; ++r) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      pc[r][ks] = __builtin_bit_cast(bf16x8, make_uint4(pk[r][ks][0], pk[r][ks][1], pk[r][ks][2],
                                                        pk[r][ks][3]));
  }
}

// Pins the weights and row sums of a unit to this point of the instruction stream: without it
// the compiler sinks their computation past the slow-path branch, away from the MFMAs it is
// meant to overlap with. Emits no instruction.
template <int NR>
__device__ __forceinline__ void anchor_weights(const bf16x8 (&p)[NR][2], const float (&sb)[NR],
                                               const float (&sf)[NR]) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) asm volatile("" ::"v"(p[r][ks]));
    asm volatile("" ::"v"(sb[r]), "v"(sf[r]));
  }
}

// Slow path of a unit (taken when some row's sum check failed): moves every row's reference to
// the larger of m and the unit's row maximum, rescales the accumulators and the sums of the
// earlier units by exp2(m_old - m_new), and recomputes the unit's weights, packed Pᵀ and sums.
template <int D, int NR>
__device__ __forceinline__ void slow_unit(WaveRows<D, NR>& ws, const f32x16 (&sc)[NR],
                                       bf16x8 (&pc)[NR][2], float sl2) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    float mx = max3f(sc[r][0], sc[r][1], sc[r][2]);
#pragma unroll
    for (int j = 3; j + 1 < 16; j += 2) mx = max3f(mx, sc[r][j], sc[r][j + 1]);
    mx = fmaxf(mx, sc[r][15]);
    const float mnew = fmaxf(ws.m[r], max_halves(mx) * sl2);
    const float munew = (mnew == -INFINITY) ? INFINITY : mnew;
    // m_old = -inf gives 0 (nothing accumulated yet); an unchanged finite m gives 1
    const float alpha = fast_exp2(ws.m[r] - munew);
#pragma unroll
    for (int b = 0; b < TileCfg<D>::DVB; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) ws.acc[r][b][j] *= alpha;
    float sb = ws.lb[r] * alpha, sf = ws.lf[r] * alpha;
    uint32_t pk[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e0 = fast_exp2(fmaf(sc[r][8 * ks + 2 * i], sl2, -munew));
        const float e1 = fast_exp2(fmaf(sc[r][8 * ks + 2 * i + 1], sl2, -munew));
        sf += e0;
        sf += e1;
        pk[ks][i] = pack_bf16x2(e0, e1);
        sb = add_bf16_pair(pk[ks][i], sb);
      }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      pc[r][ks] = __builtin_bit_cast(bf16x8, make_uint4(pk[ks][0], pk[ks][1], pk[ks][2], pk[ks][3]));
    ws.m[r] = mnew;
    ws.mu[r] = munew;
    ws.lb[r] = sb;
    ws.lf[r] = sf;
  }
}

template <int D, int NR>
__device__ __forceinline__ void load_q_rows(const FwdArgs& a, WaveRows<D, NR>& ws, int b, int hq,
                                            int qw0, int l) {
  using C = TileCfg<D>;
  const int h = l >> 5;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int row = qw0 + 32 * r + (l & 31);
    if (row < a.Lq) {
      const uint16_t* qr =
          a.q + (int64_t)b * a.q_sb + (int64_t)row * a.q_sl + (int64_t)hq * a.q_sh;
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) ws.qop[r][s] = load_q_bf16x8(qr + 16 * s + 8 * h, a.qsign);
    } else {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) ws.qop[r][s] = zero_bf16x8();
    }
#pragma unroll
    for (int bb = 0; bb < C::DVB; ++bb) ws.acc[r][bb] = f32x16{};
    ws.m[r] = -INFINITY;
    ws.mu[r] = INFINITY;
    ws.lb[r] = 0.f;
    ws.lf[r] = 0.f;
  }
}

template <int D, int NR>
__device__ __forceinline__ void store_rows(const FwdArgs& a, const WaveRows<D, NR>& ws, int b,
                                           int hq, int qw0, int l) {
  using C = TileCfg<D>;
  const int h = l >> 5;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float tb = ws.lb[r] + other_half(ws.lb[r]);
    const float tf = ws.lf[r] + other_half(ws.lf[r]);
    const int row = qw0 + 32 * r + (l & 31);
    if (row >= a.Lq) continue;
    const float inv = tb > 0.f ? 1.0f / tb : 0.f;
    uint16_t* orow = a.o + (int64_t)b * a.o_sb + (int64_t)row * a.o_sl + (int64_t)hq * a.o_sh;
#pragma unroll
    for (int bb = 0; bb < C::DVB; ++bb) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int dv = 32 * bb + 8 * u + 4 * h;
        uint2 pk;
        pk.x = pack_bf16x2(ws.acc[r][bb][4 * u + 0] * inv, ws.acc[r][bb][4 * u + 1] * inv);
        pk.y = pack_bf16x2(ws.acc[r][bb][4 * u + 2] * inv, ws.acc[r][bb][4 * u + 3] * inv);
        *reinterpret_cast<uint2*>(orow + dv) = pk;
      }
    }
    if (a.lse != nullptr && h == 0) {
      a.lse[((int64_t)b * a.Hq + hq) * a.Lq + row] =
          tf > 0.f ? ws.m[r] * kLn2 + logf(tf) : -INFINITY;
    }
  }
}

// Split form: the rows' normalised partial output O_s (fp32) and LSE_s over this workgroup's key
// range go to the split-KV partials, row (s, b, hq, row) of [S, B, Hq, Lq] (a row that sees no
// key of the range writes O_s = 0 and LSE_s = -inf).
template <int D, int NR>
__device__ __forceinline__ void store_part(const FwdArgs& a, const WaveRows<D, NR>& ws, int b,
                                           int hq, int qw0, int l, int sp) {
  using C = TileCfg<D>;
  const int h = l >> 5;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float tb = ws.lb[r] + other_half(ws.lb[r]);
    const float tf = ws.lf[r] + other_half(ws.lf[r]);
    const int row = qw0 + 32 * r + (l & 31);
    if (row >= a.Lq) continue;
    const float inv = tb > 0.f ? 1.0f / tb : 0.f;
    const int64_t prow = (((int64_t)sp * a.B + b) * a.Hq + hq) * a.Lq + row;
    float* orow = a.o_part + prow * D;
#pragma unroll
    for (int bb = 0; bb < C::DVB; ++bb) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int dv = 32 * bb + 8 * u + 4 * h;
        *reinterpret_cast<float4*>(orow + dv) =
            make_float4(ws.acc[r][bb][4 * u + 0] * inv, ws.acc[r][bb][4 * u + 1] * inv,
                        ws.acc[r][bb][4 * u + 2] * inv, ws.acc[r][bb][4 * u + 3] * inv);
      }
    }
    if (h == 0) a.lse_part[prow] = tf > 0.f ? ws.m[r] * kLn2 + logf(tf) : -INFINITY;
  }
}

// Maps blockIdx.x to a logical tile id. The hardware deals workgroups round-robin over the 8
// XCDs: workgroup bid runs on XCD bid % 8 as its (bid / 8)-th. The logical order is (b, KV head)
// groups, each a run of longest-first tiles. xcd_remap = c (set by the launcher for grids that
// are a multiple of 8; 0: no remap) splits the XCDs into clusters of c = 8 / gcd(groups, 8):
// cluster i takes the i-th (c / 8) of the logical order, i.e. whole groups, and deals it
// round-robin over its c XCDs. With 8, 16, ... groups every XCD holds whole groups (c = 1); with
// 1, 2 or 4 each group spreads over 8, 4 or 2 XCDs; with 12 two XCDs share three groups. Every
// XCD so gets the same mix of long and short tiles and as few KV heads as the counts allow.
// (Cutting a group's tiles into contiguous ranges gave one XCD only the longest tiles and
// another only the shortest: B 1, Hq 8, Hkv 2 at 32K tokens ran at 676 TFLOP/s.)
__device__ __forceinline__ int logical_block_xcd(int xcd_remap) {
  const int bid = (int)blockIdx.x;
  const int n = (int)gridDim.x;
  if (xcd_remap == 0) return bid;
  const int x = bid & 7, k = bid >> 3;
  const int c = xcd_remap;
  return (x / c) * ((n >> 3) * c) + k * c + (x % c);
}

template <int D, int NR, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64, wg_per_cu(NW)) void fwd_dense_kernel(const FwdArgs a) {
  using C = TileCfg<D>;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves per workgroup");
  constexpr int BM = 32 * NR * NW;
  __shared__ __attribute__((aligned(1024))) char smem[kStages * C::STAGE_BYTES];
  const uint32_t lds0 = lds_addr(smem);

  const int tid = (int)threadIdx.x;
  // wave index and everything derived from it are wave-uniform: keep them in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wu = w;
  const int l = tid & 63;
  int lid = logical_block_xcd(a.xcd_remap);
  const int hg = lid % a.g;
  lid /= a.g;
  int sp = 0;  // split form: the key range [sp * chunk, (sp + 1) * chunk) of this workgroup
  if constexpr (SPLIT) {
    sp = lid % a.num_splits;
    lid /= a.num_splits;
  }
  const int qt = a.n_qtiles - 1 - (lid % a.n_qtiles);
  lid /= a.n_qtiles;
  const int hkv = lid % a.Hkv;
  const int b = lid / a.Hkv;
  const int hq = hkv * a.g + hg;

  const int q0 = qt * BM;
  // Row block of this wave. Waves w and w + NW/2 share a SIMD; they take row blocks w and
  // NW-1-w, so near the causal diagonal (where a wave skips the units past its last row) every
  // SIMD skips the same number of units.
  const int rblk = w < NW / 2 ? w : (3 * NW / 2 - 1) - w;
  const int qw0 = q0 + 32 * NR * rblk;        // first row of this wave
  const int qlast = min(q0 + BM, a.Lq) - 1;   // last row of the workgroup
  // Key positions below are relative to the workgroup's range [kbeg, kbeg + rlk): all keys in
  // one launch, one split's keys in the split form; roff is the causal offset relative to it.
  const int kbeg = SPLIT ? sp * a.chunk : 0;
  const int rlk = SPLIT ? min(a.Lk, kbeg + a.chunk) - kbeg : a.Lk;
  const int roff = a.off - kbeg;
  int klimit = rlk;                           // keys [0, klimit) of the range can be visible
  if (a.causal) klimit = max(0, min(rlk, qlast + roff + 1));
  const int ntiles = __builtin_amdgcn_readfirstlane((klimit + BN - 1) / BN);

  WaveRows<D, NR> ws;
  load_q_rows<D, NR>(a, ws, b, hq, qw0, l);

  if (ntiles == 0) {  // no row of the workgroup sees any key (causal with Lq > Lk, or a split
                      // past the rows' horizon)
    if constexpr (SPLIT) store_part<D, NR>(a, ws, b, hq, qw0, l, sp);
    else store_rows<D, NR>(a, ws, b, hq, qw0, l);
    return;
  }

  TileByteOffsets<D, NW> off;
  off.init_k(a, w, l);
  off.init_v(a, w, l);
  const uint16_t* kb = a.k + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh + (int64_t)kbeg * a.k_sl;
  const uint16_t* vb = a.v + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh + (int64_t)kbeg * a.v_sl;

  // Units [0, nfull) are complete and visible to every row of this wave; later units are
  // masked (the causal diagonal, the ragged end, and the units past this wave's horizon that
  // the workgroup still streams for its other waves).
  int nfull = rlk / 32;
  if (a.causal) nfull = min(nfull, max(0, qw0 + roff + 1) / 32);
  nfull = __builtin_amdgcn_readfirstlane(nfull);
  // Last step with work for this wave: the P·V of the last unit holding a key visible to one of
  // its rows (with causal masking the workgroup streams later units for its other waves only).
  int jlast = 2 * ntiles;
  if (a.causal) {
    const int lastkey = min(rlk - 1, min(qw0 + 32 * NR - 1, a.Lq - 1) + roff);
    jlast = min(jlast, (lastkey + 32) / 32);  // last unit + 1 (0 when no key is visible)
  }
  jlast = __builtin_amdgcn_readfirstlane(jlast);

  auto stage_addr = [&](int t) -> uint32_t { return lds0 + (uint32_t)(t & 1) * C::STAGE_BYTES; };
  // Copies pair t (issued in increasing order of t <= ntiles) into its stage: K of tile t when
  // t < ntiles and V of tile t-1 when t >= 1. A ragged last tile re-reads its last key row in
  // the missing rows, so every copy stays inside the sequence; as it is the last K (V) tile
  // copied, its clamped offsets replace the full-tile ones in place.
  auto issue = [&](int t) {
    const uint32_t st = __builtin_amdgcn_readfirstlane(stage_addr(t));
    if (t < ntiles) {
      const int base = t * BN;
      if (base + BN > rlk) off.init_k(a, w, l, rlk - 1 - base);
      issue_k_sbase<D, NW>(st, kb + (int64_t)base * a.k_sl, off, wu);
    }
    if (t >= 1) {
      const int base = (t - 1) * BN;
      if (base + BN > rlk) off.init_v(a, w, l, rlk - 1 - base);
      issue_v_sbase<D, NW>(st + C::KT_BYTES, vb + (int64_t)base * a.v_sl, off, wu);
    }
  };

  f32x16 sc[2][NR];     // Sᵀ register sets (unit parity, row block)
  bf16x8 pw[2][NR][2];  // Pᵀ operand sets (unit parity, row block, k-step)
  const uint32_t kofs = (uint32_t)l * 16u;
  // V operand: group G = l/16, row 4*(G/2) + (l%16)/4, column 16*(G%2) + 4*(l%4)
  const int G = l >> 4;
  const uint32_t vofs = C::KT_BYTES + (uint32_t)(4 * (G >> 1) + ((l & 15) >> 2)) * C::VROW +
                        (uint32_t)(16 * (G & 1) + 4 * (l & 3)) * 2u;

  // Prologue: pair 0 (K of tile 0) copied and waited for, pair 1 in flight. The V part of
  // stage 0 (read by the P·V of "unit -1", whose weights are zero) is cleared so that it holds
  // finite values.
  issue(0);
  {
    char* v0 = smem + C::KT_BYTES;
    for (int i = tid; i < C::VT_BYTES / 16; i += NW * 64)
      *reinterpret_cast<uint4*>(v0 + 16 * i) = make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) pw[1][r][ks] = zero_bf16x8();
  wait_dma_all();
  __syncthreads();
  issue(1);
  qk_unit<D, NR>(ws, stage_addr(0) + kofs, 0, sc[0]);

  // Step j = 2t + H reads pair t + H.
  auto step = [&](auto HI, int t) {
    constexpr int H = decltype(HI)::value;
    const int j = 2 * t + H;
    if constexpr (H == 1) {
      wait_dma_all();  // pair t+1 landed (this wave's copies) ...
      barrier_lds();   // ... for every wave, and every wave is done with step 2t
      if (t + 2 <= ntiles) issue(t + 2);
    }
    if (j > jlast) return;  // every later unit is masked for all rows of this wave
    float sb[NR], sf[NR];
    bool ok;
    if (j >= nfull) mask_unit<NR>(sc[H], j, qw0, rlk, a.causal, roff, l);
    // Sᵀ(j+1): H = 0 -> second half of tile t; H = 1 -> first half of tile t+1.
    // P·V of unit j-1: H = 0 -> second half of tile t-1; H = 1 -> first half of tile t.
    const uint32_t st = stage_addr(t + H);
    fused_step<D, NR>(ws, sc[H], sc[1 - H], pw[1 - H], pw[H], st + kofs, 1 - H, st + vofs, 1 - H,
                      a.sl2, sb, sf, ok);
    anchor_weights<NR>(pw[H], sb, sf);
    if (__builtin_expect(__any(!ok), 0)) {
      slow_unit<D, NR>(ws, sc[H], pw[H], a.sl2);
    } else {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        ws.lb[r] = sb[r];
        ws.lf[r] = sf[r];
      }
    }
  };

  // 2*ntiles + 1 steps; the last one only finishes the P·V of the last unit (its Sᵀ reads a
  // K part that holds no tile and is never used). The loop body is a whole tile with a single
  // exit, so the accumulators keep their registers across it.
  for (int t = 0; t < ntiles; ++t) {
    step(icn<0>{}, t);
    step(icn<1>{}, t);
  }
  step(icn<0>{}, ntiles);
  wait_dma_all();
  if constexpr (SPLIT) store_part<D, NR>(a, ws, b, hq, qw0, l, sp);
  else store_rows<D, NR>(a, ws, b, hq, qw0, l);
}

template <int D, int NW, bool SPLIT = false>
hipError_t launch_dense_nw(const FwdArgs& a, hipStream_t stream) {
  constexpr int BM = 32 * kDenseNR * NW;
  FwdArgs aa = a;
  aa.n_qtiles = (a.Lq + BM - 1) / BM;
  const int64_t nwg = (int64_t)a.B * a.Hq * aa.n_qtiles * (SPLIT ? a.num_splits : 1);
  if (nwg > 0x7fffffff) return hipErrorInvalidConfiguration;  // beyond one grid dimension
  const int64_t groups = (int64_t)a.B * a.Hkv;
  int gcd8 = 8;
  while (groups % gcd8 != 0) gcd8 >>= 1;  // gcd(groups, 8)
  aa.xcd_remap = (nwg % 8 != 0) ? 0 : 8 / gcd8;
  hipLaunchKernelGGL((fwd_dense_kernel<D, kDenseNR, NW, SPLIT>), dim3((unsigned)nwg),
                     dim3(NW * 64), 0, stream, aa);
  return hipGetLastError();
}

// 256-row workgroups (8 waves, one per CU) unless that grid is a single round or less, or the
// keys are few: then 128-row workgroups (4 waves, two per CU). Measured per call: B 1, Hq 8,
// Hkv 2 at 2K / 4K / 8K tokens 60.4 / 113.6 / 222.4 -> 43.4 / 81.3 / 213.1 us, Hq 32 at 2K
// 60.1 -> 52.3 us; with at most 1024 keys a workgroup's start and drain weigh more than its
// tiles, and two per CU hide each other's (B 8, Hq 32 at 1K tokens 112.0 -> 104.2 us; B 16 at
// 512 78.9 -> 70.3 us; D = 64, B 4 at 1K 41.7 -> 37.3 us). Otherwise the 256-row form is
// ahead, each K/V tile feeding twice the rows (Hq 32 at 4K: 141.4 against 152.9 us; B 2 at
// 2K 82.2 against 86.5 us; at 8K 515.0 against 532.3 us).
template <int D>
hipError_t launch_dense_t(const FwdArgs& a, hipStream_t stream) {
  const int64_t nwg256 = (int64_t)a.B * a.Hq * ((a.Lq + 255) / 256);
  if (nwg256 <= kCUs || a.Lk <= 1024) return launch_dense_nw<D, 4>(a, stream);
  return launch_dense_nw<D, 8>(a, stream);
}

}  // namespace

hipError_t launch_fwd_dense(const FwdArgs& a, int d, hipStream_t stream) {
  if (d == 128) return launch_dense_t<128>(a, stream);
  return launch_dense_t<64>(a, stream);
}

// Split form (split-KV partials of a prefill-shaped query block): 128-row workgroups, one per
// (b, query head, row tile, split); the split count sets the grid.
hipError_t launch_fwd_dense_split(const FwdArgs& a, int d, hipStream_t stream) {
  if (d == 128) return launch_dense_nw<128, 4, true>(a, stream);
  return launch_dense_nw<64, 4, true>(a, stream);
}

}  // namespace attn
