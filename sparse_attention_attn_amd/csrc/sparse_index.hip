// sparse_index.hip — dynamic sparse-index builder on gfx950: per query head, the key-block list
// of every 64-row query block and the list of vertical key columns, built from Q and K, in the
// CSR format the block-sparse forward consumes.
//
// The pages fix that the indices are built on the fly, per head, by a fast approximation
// (MInference article, paragraphs on the three patterns and on dynamic sparse indices;
// "SparseAccelerate: Acelerando Modelos de Lenguaje", section "Patrones de Atención Dispersa
// Dinámicos"), and that a few top columns carry most of the attention mass (same article). They
// name no estimator; this one is the plainest reading (sizes square and causal, L = Lq = Lk):
//
//  * blocks: mean-pool each 64-row block of Q and of K; a causal key block kb <= qb scores
//    scale * <mean q_qb, mean k_kb>; query block qb lists its diagonal block and the top
//    (topk - 1) other causal blocks, ties to the lower block id (min(topk, qb + 1) blocks);
//  * columns: the last 64 query rows probe every key; a key's importance is the sum over those
//    rows of its causal softmax probability; the top n_cols keys are listed, ties to the lower
//    index.
//
// Kernels, in launch order: pool (Q, then K) -> block_topk -> probe_stats -> probe_combine ->
// probe_importance -> col_topk. Every reduction runs in a fixed order, so the lists are run-to-run identical.

#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __builtin_bit_cast(float, (uint32_t)u << 16);
}

// ---- mean of each 64-row block of one head, fp32: out[(b, h, blk), D], or with `transposed`
// out[(b, h), D, blk] (the block-list kernel then reads consecutive blocks of one dimension).
// One workgroup per (b, h, blk): thread (g, c) adds rows g, g + G, ... of the 8-dimension
// column chunk c with 16-byte loads; the G row-group partial sums are then added in order.
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* x, int64_t sb, int64_t sl,
                                                   int64_t sh, int H, int L, float* out,
                                                   int transposed) {
  constexpr int C = D / 8;    // 16-byte chunks per row
  constexpr int G = 256 / C;  // row groups
  __shared__ float part[G][D];
  const int nb = (L + kIndexBlock - 1) / kIndexBlock;
  int id = (int)blockIdx.x;
  const int blk = id % nb;
  id /= nb;
  const int h = id % H;
  const int b = id / H;
  const int tid = (int)threadIdx.x;
  const int c = tid % C, g = tid / C;
  const int r0 = blk * kIndexBlock;
  const int n = min(kIndexBlock, L - r0);
  const uint16_t* p = x + (int64_t)b * sb + (int64_t)r0 * sl + (int64_t)h * sh + 8 * c;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kIndexBlock / G; ++k) {
    const int r = g + k * G;
    if (r < n) {
      const uint4 u = *reinterpret_cast<const uint4*>(p + (int64_t)r * sl);
      const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_to_f32((uint16_t)(wv[e] & 0xffffu));
        acc[2 * e + 1] += bf16_to_f32((uint16_t)(wv[e] >> 16));
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[g][8 * c + e] = acc[e];
  __syncthreads();
  for (int d = tid; d < D; d += 256) {
    float t = 0.f;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) t += part[gg][d];
    const float mean = t / (float)n;
    if (transposed)
      out[((int64_t)(b * H + h) * D + d) * nb + blk] = mean;
    else
      out[((int64_t)(b * H + h) * nb + blk) * D + d] = mean;
  }
}

// Offset of query block qb's list inside its head's block list: sum over q < qb of
// min(topk, q + 1).
__device__ __forceinline__ int64_t blk_list_offset(int qb, int topk) {
  if (qb <= topk) return (int64_t)qb * (qb + 1) / 2;
  return (int64_t)topk * (topk + 1) / 2 + (int64_t)(qb - topk) * topk;
}

// fp32 -> uint32 whose unsigned order is the float order (-0 taken as +0, so the two compare
// equal as floats do).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i to XCD i % 8), each XCD
// with its own L2. This renumbering gives each XCD a contiguous range of logical ids.
__device__ __forceinline__ int xcd_major(int bid, int nwg) {
  if (nwg % 8) return bid;
  return (bid % 8) * (nwg / 8) + bid / 8;
}

__device__ __forceinline__ int wave_count(bool p) { return __popcll(__ballot(p)); }
__device__ __forceinline__ int lane_rank(uint64_t m) {  // set bits of m below this lane
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ---- block lists: one workgroup (4 waves) per (b, h, group of kTopkQ query blocks) ------------
// Block id i = 256 s + 64 w + lane sits in slot s of lane `lane` of wave w, for up to 8 slots.
// Each pooled-K value read serves the kTopkQ query blocks of the group. A query block's keys
// are the order keys of its causal block scores, the diagonal raised to the maximum key so that
// it is always listed. The need-th largest key T (need = min(topk, qb + 1)) is found bit by bit,
// from the top bit down, by counting keys >= candidate with wave ballots (one barrier per bit);
// every key above T is listed, and of the keys equal to T the lowest block ids, in ascending
// block order. Logical ids run head-major and are spread XCD-major, so one XCD takes a run of
// consecutive heads (one KV head's group at the full-size shapes) and its pooled K stays in
// that XCD's L2.
constexpr int kTopkQ = 8;
constexpr int kTopkSlots = kIndexMaxBlocks / 256;

template <int D>
__global__ __launch_bounds__(256) void block_topk_kernel(const float* qbar, const float* kbar,
                                                         int Hq, int Hkv, int nqb, float scale,
                                                         int topk, int32_t* blk_ptr,
                                                         int32_t* blk_idx, int64_t head_len,
                                                         int64_t total, int nbh) {
  __shared__ f32x4 qs[D][kTopkQ / 4];              // pooled q of the group's query blocks
  __shared__ int cnt[2][4][kTopkQ];                // per-bit counts, double-buffered
  __shared__ int gtc[kTopkQ][kTopkSlots][4];       // keys > T per (slot, wave)
  __shared__ int eqc[kTopkQ][kTopkSlots][4];       // keys == T per (slot, wave)
  const int tid = (int)threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ngrp = (nqb + kTopkQ - 1) / kTopkQ;
  const int id = xcd_major((int)blockIdx.x, (int)gridDim.x);
  const int qg = id % ngrp;
  const int bh = id / ngrp;
  const int h = bh % Hq;
  const int b = bh / Hq;
  const int hk = h / (Hq / Hkv);
  const int qb0 = qg * kTopkQ;
  const int nmax = min(nqb, qb0 + kTopkQ);  // key blocks any query block of the group can see
  const int nslots = (nmax + 255) / 256;

  for (int d = tid; d < D; d += 256) {
#pragma unroll
    for (int t4 = 0; t4 < kTopkQ / 4; ++t4) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 4 * t4 + e;
        v[e] = (qb0 + t < nqb) ? qbar[((int64_t)bh * nqb + qb0 + t) * D + d] : 0.f;
      }
      qs[d][t4] = v;
    }
  }
  __syncthreads();

  // scores -> order keys
  const float* kb0 = kbar + (int64_t)(b * Hkv + hk) * D * nqb;  // [D][nqb]
  uint32_t key[kTopkQ][kTopkSlots];
  static_for<0, kTopkSlots>([&](auto S) {
    constexpr int s = decltype(S)::value;
    if (s < nslots) {
      const int i = s * 256 + tid;
      const float* kp = kb0 + min(i, nmax - 1);
      float acc[kTopkQ] = {};
#pragma unroll 8
      for (int d = 0; d < D; ++d) {
        const float kv = kp[(int64_t)d * nqb];
#pragma unroll
        for (int t4 = 0; t4 < kTopkQ / 4; ++t4) {
          const f32x4 qv = qs[d][t4];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * t4 + e] = fmaf(qv[e], kv, acc[4 * t4 + e]);
        }
      }
#pragma unroll
      for (int t = 0; t < kTopkQ; ++t)
        key[t][s] = (i == qb0 + t) ? 0xffffffffu : order_key(scale * acc[t]);
    } else {
#pragma unroll
      for (int t = 0; t < kTopkQ; ++t) key[t][s] = 0u;
    }
  });

  int n[kTopkQ], need[kTopkQ];
#pragma unroll
  for (int t = 0; t < kTopkQ; ++t) {
    n[t] = (qb0 + t < nqb) ? qb0 + t + 1 : 0;
    need[t] = min(topk, n[t]);
  }
  // Blocks a query block does not see get key 0. Every candidate of the bit search is >= 1, so
  // the counts below need no bounds test; the listing keeps one (a NaN score can map to 0).
  static_for<0, kTopkSlots>([&](auto S) {
    constexpr int s = decltype(S)::value;
    const int i = s * 256 + tid;
#pragma unroll
    for (int t = 0; t < kTopkQ; ++t)
      if (i >= n[t]) key[t][s] = 0u;
  });

  // T_t: the largest value with at least need_t keys >= it
  uint32_t pre[kTopkQ] = {};
  for (int bit = 31; bit >= 0; --bit) {
    int c[kTopkQ] = {};
    static_for<0, kTopkSlots>([&](auto S) {
      constexpr int s = decltype(S)::value;
      if (s < nslots) {
#pragma unroll
        for (int t = 0; t < kTopkQ; ++t)
          c[t] += wave_count(key[t][s] >= (pre[t] | (1u << bit)));
      }
    });
    if ((tid & 63) == 0) {
#pragma unroll
      for (int t = 0; t < kTopkQ; ++t) cnt[bit & 1][w][t] = c[t];
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kTopkQ; ++t) {
      const int tot = cnt[bit & 1][0][t] + cnt[bit & 1][1][t] + cnt[bit & 1][2][t] +
                      cnt[bit & 1][3][t];
      if (tot >= need[t]) pre[t] |= 1u << bit;
    }
  }

  // ordered output: counts of keys above and equal to T per (slot, wave)
  static_for<0, kTopkSlots>([&](auto S) {
    constexpr int s = decltype(S)::value;
    const int i = s * 256 + tid;
#pragma unroll
    for (int t = 0; t < kTopkQ; ++t) {
      const bool v = s < nslots && i < n[t];
      const int g = wave_count(v && key[t][s] > pre[t]);
      const int e = wave_count(v && key[t][s] == pre[t]);
      if ((tid & 63) == 0) { gtc[t][s][w] = g; eqc[t][s][w] = e; }
    }
  });
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kTopkQ; ++t) {
    const int qb = qb0 + t;
    if (qb >= nqb) break;
    int gt_all = 0;
    for (int u = 0; u < nslots * 4; ++u) gt_all += gtc[t][u >> 2][u & 3];
    const int take_eq = need[t] - gt_all;  // keys equal to T to list, lowest ids first
    const int64_t base = (int64_t)bh * head_len + blk_list_offset(qb, topk);
    int gt_before = 0, eq_before = 0;
    static_for<0, kTopkSlots>([&](auto S) {
      constexpr int s = decltype(S)::value;
      if (s < nslots) {
        int gb = gt_before, eb = eq_before;
        for (int u = 0; u < w; ++u) { gb += gtc[t][s][u]; eb += eqc[t][s][u]; }
        const int i = s * 256 + tid;
        const bool v = i < n[t];
        const bool gt = v && key[t][s] > pre[t];
        const bool eq = v && key[t][s] == pre[t];
        const int eq_rank = eb + lane_rank(__ballot(eq));
        const bool sel = gt || (eq && eq_rank < take_eq);
        const int pos = gb + min(eb, take_eq) + lane_rank(__ballot(sel));
        if (sel) blk_idx[base + pos] = i;
        for (int u = 0; u < 4; ++u) { gt_before += gtc[t][s][u]; eq_before += eqc[t][s][u]; }
      }
    });
    if (tid == 0) {
      blk_ptr[(int64_t)bh * nqb + qb] = (int32_t)base;
      if (bh == nbh - 1 && qb == nqb - 1) blk_ptr[(int64_t)nbh * nqb] = (int32_t)total;
    }
  }
}

// ---- probe: scores of the last P = min(64, L) query rows against every key, on MFMA --------
// Both operands are rows with d contiguous; lane l feeds the d range
// [(D/2)(l/32) + 8 s, +8) at k-step s, the same permutation of d for both operands, so each
// lane reads one contiguous half row. Workgroups are dispatched round-robin over the 8 XCDs;
// the renumbering gives each XCD a contiguous range of logical ids, in which the query heads of
// one KV head, taking the same key chunk, are neighbours and share its K rows in one L2.

template <int D>
__device__ __forceinline__ void load_half_row(const uint16_t* row, bf16x8 (&op)[D / 16]) {
  const uint16_t* p = row + (D / 2) * ((threadIdx.x & 63) >> 5);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) op[s] = load_bf16x8(p + 8 * s);
}

template <int D>
__device__ __forceinline__ void load_probe_q(const IndexArgs& a, int b, int h, int pr,
                                             bf16x8 (&op)[D / 16]) {
  const int P = min(kProbeRows, a.L);
  if (pr < P) {
    load_half_row<D>(a.q + (int64_t)b * a.q_sb + (int64_t)(a.L - P + pr) * a.q_sl +
                         (int64_t)h * a.q_sh, op);
  } else {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) op[s] = zero_bf16x8();
  }
}

struct ProbeIds {
  int b, h, hk, ch;
};
__device__ __forceinline__ ProbeIds probe_ids(const IndexArgs& a) {
  int id = xcd_major((int)blockIdx.x, (int)gridDim.x);
  ProbeIds r;
  r.h = id % a.Hq;
  id /= a.Hq;
  r.b = id % a.B;
  r.ch = id / a.B;
  r.hk = r.h / (a.Hq / a.Hkv);
  return r;
}

// Pass 1, per (b, h, chunk of kProbeChunk keys; wave w takes a quarter): each probe row's
// running maximum and weight sum over the chunk (exp2 domain). Tile product
// C[key][row] = K_tile . Q_probe^T: lane l holds probe row 32 nt + l%32 and keys
// 8(j/4) + 4(l/32) + j%4 of the 32-key tile, so a row's tile maximum is taken in-lane.
template <int D>
__global__ __launch_bounds__(256) void probe_stats_kernel(const IndexArgs a, float* stats) {
  constexpr int KS = D / 16;
  __shared__ float sm[4][64], ss[4][64];
  const ProbeIds id = probe_ids(a);
  const int nch = (a.L + kProbeChunk - 1) / kProbeChunk;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int l = (int)threadIdx.x & 63;
  const int P = min(kProbeRows, a.L);
  const int r0 = a.L - P;
  bf16x8 qop[2][KS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) load_probe_q<D>(a, id.b, id.h, nt * 32 + (l & 31), qop[nt]);
  const uint16_t* kbase = a.k + (int64_t)id.b * a.k_sb + (int64_t)id.hk * a.k_sh;
  constexpr int kPerWave = kProbeChunk / 4;
  const int kbeg = id.ch * kProbeChunk + w * kPerWave;
  const int kend = min(a.L, kbeg + kPerWave);
  float m[2] = {-INFINITY, -INFINITY}, sum[2] = {0.f, 0.f};
  for (int j0 = kbeg; j0 < kend; j0 += 32) {
    bf16x8 kop[KS];
    load_half_row<D>(kbase + (int64_t)min(j0 + (l & 31), a.L - 1) * a.k_sl, kop);
    f32x16 acc[2] = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      acc[0] = mfma32(kop[s], qop[0][s], acc[0]);
      acc[1] = mfma32(kop[s], qop[1][s], acc[1]);
    }
    const bool edge = j0 + 31 >= r0;  // a key of the tile lies above some probe row or past L
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int row = r0 + nt * 32 + (l & 31);
      float x[16];
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = j0 + 8 * (j >> 2) + 4 * (l >> 5) + (j & 3);
        x[j] = (edge && key > row) ? -INFINITY : acc[nt][j] * a.sl2;
        tmax = fmaxf(tmax, x[j]);
      }
      if (tmax != -INFINITY) {
        const float mn = fmaxf(m[nt], tmax);
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) t += fast_exp2(x[j] - mn);
        sum[nt] = sum[nt] * fast_exp2(m[nt] - mn) + t;
        m[nt] = mn;
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float mo = other_half(m[nt]), so = other_half(sum[nt]);
    const float M = fmaxf(m[nt], mo);
    float S = 0.f;
    if (m[nt] != -INFINITY) S += sum[nt] * fast_exp2(m[nt] - M);
    if (mo != -INFINITY) S += so * fast_exp2(mo - M);
    if (l < 32) { sm[w][nt * 32 + l] = M; ss[w][nt * 32 + l] = S; }
  }
  __syncthreads();
  if (w == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm[ww][l]);
    float S = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww)
      if (sm[ww][l] != -INFINITY) S += ss[ww][l] * fast_exp2(sm[ww][l] - M);
    float* o = stats + (((int64_t)(id.b * a.Hq + id.h) * nch + id.ch) * 64 + l) * 2;
    o[0] = M;
    o[1] = S;
  }
}

// Per (b, h): each probe row's statistics over all chunks, folded into the one offset
// c = M + log2(S) with p(row, key) = exp2(x - c); +inf for rows without keys (so p = 0).
__global__ __launch_bounds__(64) void probe_combine_kernel(const float* stats, int L, int nch,
                                                          float* fin) {
  const int bh = (int)blockIdx.x;
  const int l = (int)threadIdx.x;
  const float* st = stats + (int64_t)bh * nch * 128 + l * 2;
  float M = -INFINITY;
#pragma unroll 16
  for (int c = 0; c < nch; ++c) M = fmaxf(M, st[c * 128]);
  float S = 0.f;
#pragma unroll 16
  for (int c = 0; c < nch; ++c) {
    const float mc = st[c * 128];
    if (mc != -INFINITY) S += st[c * 128 + 1] * fast_exp2(mc - M);
  }
  fin[bh * 64 + l] = (l < min(kProbeRows, L) && S > 0.f) ? M + log2f(S) : INFINITY;
}

// Pass 2: importance[key] = sum over probe rows of p(row, key). Tile product
// C[row][key] = Q_probe . K_tile^T: lane l holds key l%32 and probe rows
// 32 mt + 8(j/4) + 4(l/32) + j%4, so the sum over rows is in-lane plus one half swap.
template <int D>
__global__ __launch_bounds__(256) void probe_importance_kernel(const IndexArgs a,
                                                               const float* fin, float* imp) {
  constexpr int KS = D / 16;
  const ProbeIds id = probe_ids(a);
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int l = (int)threadIdx.x & 63;
  const int P = min(kProbeRows, a.L);
  const int r0 = a.L - P;
  const int bh = id.b * a.Hq + id.h;
  bf16x8 qop[2][KS];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) load_probe_q<D>(a, id.b, id.h, mt * 32 + (l & 31), qop[mt]);
  float c[2][16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      c[mt][j] = fin[bh * 64 + mt * 32 + 8 * (j >> 2) + 4 * (l >> 5) + (j & 3)];
  const uint16_t* kbase = a.k + (int64_t)id.b * a.k_sb + (int64_t)id.hk * a.k_sh;
  float* out = imp + (int64_t)bh * a.L;
  constexpr int kPerWave = kProbeChunk / 4;
  const int kbeg = id.ch * kProbeChunk + w * kPerWave;
  const int kend = min(a.L, kbeg + kPerWave);
  for (int j0 = kbeg; j0 < kend; j0 += 32) {
    const int key = j0 + (l & 31);
    bf16x8 kop[KS];
    load_half_row<D>(kbase + (int64_t)min(key, a.L - 1) * a.k_sl, kop);
    f32x16 acc[2] = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      acc[0] = mfma32(qop[0][s], kop[s], acc[0]);
      acc[1] = mfma32(qop[1][s], kop[s], acc[1]);
    }
    const bool edge = j0 + 31 >= r0;
    float t = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = r0 + mt * 32 + 8 * (j >> 2) + 4 * (l >> 5) + (j & 3);
        const float p = fast_exp2(fmaf(acc[mt][j], a.sl2, -c[mt][j]));
        t += (edge && key > row) ? 0.f : p;
      }
    t += other_half(t);
    if (l < 32 && key < a.L) out[key] = t;
  }
}

// Slash lines, per (b, h, 64 offsets o0 .. o0+63), one wave: probe row r = r0 + pr meets line
// o at key r - o, so the chunk needs keys r0 - o0 - 63 .. r0 - o0 + 63, a 128-key window. For
// each 32-key tile of the window the wave forms C[row][key] = Q_probe . K^T (the importance
// pass's layout, probe Q loaded once for the four tiles), turns it into probabilities and
// stores them in LDS as pl[pr][window key]; then lane t sums line o0 + t,
// pl[pr][pr - t + 63] over pr in order (rows >= P hold zeros).
template <int D>
__global__ __launch_bounds__(64) void probe_slash_kernel(const IndexArgs a, const float* fin,
                                                         float* simp) {
  constexpr int KS = D / 16;
  __shared__ float pl[kProbeRows][128 + 1];
  const int nsc = (a.L + 63) / 64;
  int id = (int)blockIdx.x;
  const int sc = id % nsc;
  id /= nsc;
  const int h = id % a.Hq;
  const int b = id / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int bh = b * a.Hq + h;
  const int l = (int)threadIdx.x;
  const int P = min(kProbeRows, a.L);
  const int r0 = a.L - P;
  const int o0 = sc * 64;
  const int kw0 = r0 - o0 - 63;  // window key 0
  bf16x8 qop[2][KS];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) load_probe_q<D>(a, b, h, mt * 32 + (l & 31), qop[mt]);
  float c[2][16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      c[mt][j] = fin[bh * 64 + mt * 32 + 8 * (j >> 2) + 4 * (l >> 5) + (j & 3)];
  const uint16_t* kbase = a.k + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int kk = 32 * kt + (l & 31);  // this lane's window key
    const int key = kw0 + kk;
    bf16x8 kop[KS];
    load_half_row<D>(kbase + (int64_t)min(max(key, 0), a.L - 1) * a.k_sl, kop);
    f32x16 acc[2] = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      acc[0] = mfma32(qop[0][s], kop[s], acc[0]);
      acc[1] = mfma32(qop[1][s], kop[s], acc[1]);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int pr = mt * 32 + 8 * (j >> 2) + 4 * (l >> 5) + (j & 3);
        const float p = fast_exp2(fmaf(acc[mt][j], a.sl2, -c[mt][j]));
        pl[pr][kk] = (key < 0 || key > r0 + pr) ? 0.f : p;
      }
  }
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int pr = 0; pr < kProbeRows; ++pr) t += pl[pr][pr - l + 63];
  if (o0 + l < a.L) simp[(int64_t)bh * a.L + o0 + l] = t;
}

// ---- column lists: one workgroup (1024 threads) per (b, h) -----------------------------------
// Radix select (four 8-bit digits of the non-negative fp32 bit patterns) finds the n-th largest
// importance T and how many of the keys equal to T to take. Then each wave takes a contiguous
// range of keys: it counts the keys above and equal to T in its range, the counts are exchanged
// once, and each wave lists its selected keys in ascending order (wave ballots give the ranks),
// the keys equal to T lowest index first.
__global__ __launch_bounds__(1024) void col_topk_kernel(const float* imp, int L, int ncols,
                                                        int32_t* col_ptr, int32_t* col_idx,
                                                        int nheads) {
  constexpr int kUnroll = 8;
  __shared__ int hist[256];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_remaining;
  __shared__ int wgt[16], weq[16];
  const int tid = (int)threadIdx.x;
  const int bh = (int)blockIdx.x;
  const uint32_t* v = reinterpret_cast<const uint32_t*>(imp + (int64_t)bh * L);
  const int n = min(ncols, L);
  const int64_t base = (int64_t)bh * n;
  if (tid == 0) {
    col_ptr[bh] = (int32_t)base;
    if (bh == nheads - 1) col_ptr[nheads] = (int32_t)(base + n);
  }
  if (n == 0) return;

  uint32_t prefix = 0, pmask = 0;
  int remaining = n;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += 1024) hist[i] = 0;
    __syncthreads();
    for (int j0 = 0; j0 < L; j0 += 1024 * kUnroll) {
      uint32_t xs[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int j = j0 + u * 1024 + tid;
        xs[u] = j < L ? v[j] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int j = j0 + u * 1024 + tid;
        if (j < L && (xs[u] & pmask) == prefix) atomicAdd(&hist[(xs[u] >> shift) & 255u], 1);
      }
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0, dsel = 0;
      for (int d = 255; d >= 0; --d) {
        if (acc + hist[d] >= remaining) { dsel = d; break; }
        acc += hist[d];
      }
      sh_prefix = prefix | ((uint32_t)dsel << shift);
      sh_remaining = remaining - acc;
    }
    __syncthreads();
    prefix = sh_prefix;
    remaining = sh_remaining;
    pmask |= 255u << shift;
    __syncthreads();
  }
  // prefix = bits of T; remaining = keys equal to T to take (lowest indices first)
  const int wv = tid >> 6, ln = tid & 63;
  const int R = ((L + 15) / 16 + 63) / 64 * 64;  // keys per wave, a multiple of 64
  const int lo = min(L, wv * R), hi = min(L, lo + R);
  int g = 0, e = 0;
  for (int j0 = lo; j0 < hi; j0 += 64 * kUnroll) {
    uint32_t xs[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = j0 + 64 * u + ln;
      xs[u] = j < hi ? v[j] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = j0 + 64 * u + ln;
      g += wave_count(j < hi && xs[u] > prefix);
      e += wave_count(j < hi && xs[u] == prefix);
    }
  }
  if (ln == 0) { wgt[wv] = g; weq[wv] = e; }
  __syncthreads();
  int run_gt = 0, run_eq = 0;
  for (int u = 0; u < wv; ++u) { run_gt += wgt[u]; run_eq += weq[u]; }
  for (int j0 = lo; j0 < hi; j0 += 64 * kUnroll) {
    uint32_t xs[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = j0 + 64 * u + ln;
      xs[u] = j < hi ? v[j] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = j0 + 64 * u + ln;
      const bool gt = j < hi && xs[u] > prefix;
      const bool eq = j < hi && xs[u] == prefix;
      const uint64_t beq = __ballot(eq);
      const bool sel = gt || (eq && run_eq + lane_rank(beq) < remaining);
      const int pos = run_gt + min(run_eq, remaining) + lane_rank(__ballot(sel));
      if (sel) col_idx[base + pos] = j;
      run_gt += wave_count(gt);
      run_eq += __popcll(beq);
    }
  }
}

template <int D>
hipError_t launch_index_t(const IndexArgs& a, hipStream_t stream) {
  const int nqb = (a.L + kIndexBlock - 1) / kIndexBlock;
  const int nch = (a.L + kProbeChunk - 1) / kProbeChunk;
  const int nbh = a.B * a.Hq;
  hipLaunchKernelGGL((pool_kernel<D>), dim3((unsigned)(nbh * nqb)), dim3(256), 0, stream, a.q,
                     a.q_sb, a.q_sl, a.q_sh, a.Hq, a.L, a.qbar, 0);
  hipLaunchKernelGGL((pool_kernel<D>), dim3((unsigned)(a.B * a.Hkv * nqb)), dim3(256), 0, stream,
                     a.k, a.k_sb, a.k_sl, a.k_sh, a.Hkv, a.L, a.kbar, 1);
  const int ngrp = (nqb + kTopkQ - 1) / kTopkQ;
  hipLaunchKernelGGL((block_topk_kernel<D>), dim3((unsigned)(nbh * ngrp)), dim3(256), 0, stream,
                     a.qbar, a.kbar, a.Hq, a.Hkv, nqb, a.scale, a.topk, a.blk_ptr, a.blk_idx,
                     a.blk_head_len, a.blk_total, nbh);
  hipLaunchKernelGGL((probe_stats_kernel<D>), dim3((unsigned)(nbh * nch)), dim3(256), 0, stream,
                     a, a.stats);
  hipLaunchKernelGGL(probe_combine_kernel, dim3((unsigned)nbh), dim3(64), 0, stream, a.stats,
                     a.L, nch, a.fin);
  hipLaunchKernelGGL((probe_importance_kernel<D>), dim3((unsigned)(nbh * nch)), dim3(256), 0,
                     stream, a, a.fin, a.imp);
  hipLaunchKernelGGL(col_topk_kernel, dim3((unsigned)nbh), dim3(1024), 0, stream, a.imp, a.L,
                     a.ncols, a.col_ptr, a.col_idx, nbh);
  return hipGetLastError();
}

template <int D>
hipError_t launch_vslash_index_t(const IndexArgs& a, hipStream_t stream) {
  const int nch = (a.L + kProbeChunk - 1) / kProbeChunk;
  const int nsc = (a.L + 63) / 64;
  const int nbh = a.B * a.Hq;
  hipLaunchKernelGGL((probe_stats_kernel<D>), dim3((unsigned)(nbh * nch)), dim3(256), 0, stream,
                     a, a.stats);
  hipLaunchKernelGGL(probe_combine_kernel, dim3((unsigned)nbh), dim3(64), 0, stream, a.stats,
                     a.L, nch, a.fin);
  hipLaunchKernelGGL((probe_importance_kernel<D>), dim3((unsigned)(nbh * nch)), dim3(256), 0,
                     stream, a, a.fin, a.imp);
  hipLaunchKernelGGL((probe_slash_kernel<D>), dim3((unsigned)(nbh * nsc)), dim3(64), 0, stream,
                     a, a.fin, a.simp);
  hipLaunchKernelGGL(col_topk_kernel, dim3((unsigned)nbh), dim3(1024), 0, stream, a.imp, a.L,
                     a.ncols, a.col_ptr, a.col_idx, nbh);
  hipLaunchKernelGGL(col_topk_kernel, dim3((unsigned)nbh), dim3(1024), 0, stream, a.simp, a.L,
                     a.nslash, a.sl_ptr, a.sl_idx, nbh);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_vslash_index(const IndexArgs& a, int d, hipStream_t stream) {
  if (d == 128) return launch_vslash_index_t<128>(a, stream);
  return launch_vslash_index_t<64>(a, stream);
}

hipError_t launch_build_index(const IndexArgs& a, int d, hipStream_t stream) {
  if (d == 128) return launch_index_t<128>(a, stream);
  return launch_index_t<64>(a, stream);
}

}  // namespace attn
