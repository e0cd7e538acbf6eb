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
// Kernels, in launch order: pool (Q, then K) -> block_topk -> probe_stats -> probe_importance
// -> col_topk. Every reduction runs in a fixed order, so the lists are run-to-run identical.

#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __builtin_bit_cast(float, (uint32_t)u << 16);
}

// ---- mean of each 64-row block of one head: out[(b, h, blk), D] fp32 -----------------------
template <int D>
__global__ __launch_bounds__(D) void pool_kernel(const uint16_t* x, int64_t sb, int64_t sl,
                                                 int64_t sh, int H, int L, float* out) {
  const int nb = (L + kIndexBlock - 1) / kIndexBlock;
  int id = (int)blockIdx.x;
  const int blk = id % nb;
  id /= nb;
  const int h = id % H;
  const int b = id / H;
  const int d = (int)threadIdx.x;
  const int r0 = blk * kIndexBlock;
  const int n = min(kIndexBlock, L - r0);
  const uint16_t* p = x + (int64_t)b * sb + (int64_t)r0 * sl + (int64_t)h * sh + d;
  float acc = 0.f;
  for (int r = 0; r < n; ++r) acc += bf16_to_f32(p[(int64_t)r * sl]);
  out[((int64_t)(b * H + h) * nb + blk) * D + d] = acc / (float)n;
}

// Offset of query block qb's list inside its head's block list: sum over q < qb of
// min(topk, q + 1).
__device__ __forceinline__ int64_t blk_list_offset(int qb, int topk) {
  if (qb <= topk) return (int64_t)qb * (qb + 1) / 2;
  return (int64_t)topk * (topk + 1) / 2 + (int64_t)(qb - topk) * topk;
}

// ---- block lists: one workgroup per (b, h, qb) ----------------------------------------------
// Scores of the qb + 1 causal blocks go to LDS (the diagonal as +inf, padding as -inf), a
// bitonic sort ranks them by (score descending, block id ascending), the first min(topk, qb+1)
// are flagged, and a scan over the flags writes them in ascending block order.
template <int D>
__global__ __launch_bounds__(256) void block_topk_kernel(const float* qbar, const float* kbar,
                                                         int Hq, int Hkv, int nqb, float scale,
                                                         int topk, int32_t* blk_ptr,
                                                         int32_t* blk_idx, int64_t head_len,
                                                         int64_t total) {
  __shared__ float qs[D];
  __shared__ float key[kIndexMaxBlocks];
  __shared__ int idx[kIndexMaxBlocks];
  __shared__ int flag[kIndexMaxBlocks];
  __shared__ int part[256];
  const int tid = (int)threadIdx.x;
  int id = (int)blockIdx.x;
  const int qb = id % nqb;
  id /= nqb;
  const int h = id % Hq;
  const int b = id / Hq;
  const int hk = h / (Hq / Hkv);

  for (int d = tid; d < D; d += 256) qs[d] = qbar[((int64_t)(b * Hq + h) * nqb + qb) * D + d];
  __syncthreads();

  const int n = qb + 1;
  int N = 1;
  while (N < n) N <<= 1;
  const float* kb0 = kbar + (int64_t)(b * Hkv + hk) * nqb * D;
  for (int i = tid; i < N; i += 256) {
    float s = -INFINITY;
    int ix = INT_MAX - N + i;  // padding sorts last (unique ids keep the order strict)
    if (i < n) {
      ix = i;
      if (i == qb) {
        s = INFINITY;
      } else {
        const float* kr = kb0 + (int64_t)i * D;
        float acc = 0.f;
#pragma unroll 8
        for (int d = 0; d < D; ++d) acc = fmaf(qs[d], kr[d], acc);
        s = scale * acc;
      }
    }
    key[i] = s;
    idx[i] = ix;
    flag[i] = 0;
  }
  __syncthreads();

  for (int kk = 2; kk <= N; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < N; i += 256) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const float a = key[i], c = key[ixj];
          const int ia = idx[i], ic = idx[ixj];
          const bool i_first = a > c || (a == c && ia < ic);   // i ranks before ixj
          const bool want_first = (i & kk) == 0;
          if (i_first != want_first) {
            key[i] = c; key[ixj] = a;
            idx[i] = ic; idx[ixj] = ia;
          }
        }
      }
      __syncthreads();
    }
  }

  const int cnt = min(topk, n);
  for (int i = tid; i < cnt; i += 256) flag[idx[i]] = 1;
  __syncthreads();

  // ordered compaction: thread t owns ids [t*per, (t+1)*per)
  const int per = (n + 255) / 256;
  const int lo = tid * per, hi = min(n, lo + per);
  int c = 0;
  for (int i = lo; i < hi; ++i) c += flag[i];
  part[tid] = c;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < 256; ++t) { const int v = part[t]; part[t] = run; run += v; }
  }
  __syncthreads();
  const int64_t base = (int64_t)(b * Hq + h) * head_len + blk_list_offset(qb, topk);
  int pos = part[tid];
  for (int i = lo; i < hi; ++i)
    if (flag[i]) blk_idx[base + pos++] = i;
  if (tid == 0) {
    blk_ptr[(int64_t)(b * Hq + h) * nqb + qb] = (int32_t)base;
    if (b * Hq + h == (int)(gridDim.x / nqb) - 1 && qb == nqb - 1) blk_ptr[(int64_t)gridDim.x] = (int32_t)total;
  }
}

// ---- probe pass 1: per (b, h, 1024-key chunk), each probe row's softmax statistics ------------
// Lane l of every wave is probe row L - P + l (P = min(64, L)); wave w takes keys c0 + w,
// c0 + w + 4, ...; the key row is wave-uniform. Scores are in the exp2 domain.
template <int D>
__device__ __forceinline__ float probe_dot(const float (&qv)[D], const uint16_t* kr) {
  const uint4* k4 = reinterpret_cast<const uint4*>(kr);  // rows are 16-byte aligned
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    const uint4 u = k4[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(qv[8 * i + 2 * e], __builtin_bit_cast(float, w[e] << 16), acc);
      acc = fmaf(qv[8 * i + 2 * e + 1], __builtin_bit_cast(float, w[e] & 0xffff0000u), acc);
    }
  }
  return acc;
}

template <int D>
__device__ __forceinline__ void probe_load_q(const uint16_t* q, int64_t sb, int64_t sl,
                                             int64_t sh, int b, int h, int row, bool act,
                                             float (&qv)[D]) {
  const uint16_t* p = q + (int64_t)b * sb + (int64_t)row * sl + (int64_t)h * sh;
#pragma unroll
  for (int d = 0; d < D; ++d) qv[d] = act ? bf16_to_f32(p[d]) : 0.f;
}

template <int D>
__global__ __launch_bounds__(256) void probe_stats_kernel(const IndexArgs a, float* stats) {
  __shared__ float sm[4][64], sl_[4][64];
  const int nch = (a.L + kProbeChunk - 1) / kProbeChunk;
  int id = (int)blockIdx.x;
  const int ch = id % nch;
  id /= nch;
  const int h = id % a.Hq;
  const int b = id / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int l = (int)threadIdx.x & 63;
  const int P = min(kProbeRows, a.L);
  const bool act = l < P;
  const int row = a.L - P + (act ? l : 0);
  float qv[D];
  probe_load_q<D>(a.q, a.q_sb, a.q_sl, a.q_sh, b, h, row, act, qv);
  const uint16_t* kbase = a.k + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh;
  const int c0 = ch * kProbeChunk, c1 = min(a.L, c0 + kProbeChunk);
  float m = -INFINITY, s = 0.f;
  for (int j = c0 + w; j < c1; j += 4) {
    const float x = probe_dot<D>(qv, kbase + (int64_t)j * a.k_sl) * a.sl2;
    if (act && j <= row) {
      const float mn = fmaxf(m, x);
      s = s * fast_exp2(m - mn) + fast_exp2(x - mn);
      m = mn;
    }
  }
  sm[w][l] = m;
  sl_[w][l] = s;
  __syncthreads();
  if (w == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm[ww][l]);
    float S = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww)
      if (sm[ww][l] != -INFINITY) S += sl_[ww][l] * fast_exp2(sm[ww][l] - M);
    float* o = stats + (((int64_t)(b * a.Hq + h) * nch + ch) * 64 + l) * 2;
    o[0] = M;
    o[1] = S;
  }
}

// ---- probe pass 2: importance[j] = sum over probe rows of p(row, j) --------------------------
template <int D>
__global__ __launch_bounds__(256) void probe_importance_kernel(const IndexArgs a,
                                                               const float* stats, float* imp) {
  const int nch = (a.L + kProbeChunk - 1) / kProbeChunk;
  int id = (int)blockIdx.x;
  const int ch = id % nch;
  id /= nch;
  const int h = id % a.Hq;
  const int b = id / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int l = (int)threadIdx.x & 63;
  const int P = min(kProbeRows, a.L);
  const bool act = l < P;
  const int row = a.L - P + (act ? l : 0);
  // the row's statistics over all chunks
  float M = -INFINITY, S = 0.f;
  const float* st = stats + ((int64_t)(b * a.Hq + h) * nch) * 128 + l * 2;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, st[c * 128]);
  for (int c = 0; c < nch; ++c) {
    const float mc = st[c * 128];
    if (mc != -INFINITY) S += st[c * 128 + 1] * fast_exp2(mc - M);
  }
  const float inv = (act && S > 0.f) ? 1.0f / S : 0.f;
  float qv[D];
  probe_load_q<D>(a.q, a.q_sb, a.q_sl, a.q_sh, b, h, row, act, qv);
  const uint16_t* kbase = a.k + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh;
  float* out = imp + (int64_t)(b * a.Hq + h) * a.L;
  const int c0 = ch * kProbeChunk, c1 = min(a.L, c0 + kProbeChunk);
  for (int j = c0 + w; j < c1; j += 4) {
    const float x = probe_dot<D>(qv, kbase + (int64_t)j * a.k_sl) * a.sl2;
    float p = (act && j <= row) ? fast_exp2(x - M) * inv : 0.f;
    // sum over the 64 probe rows (lanes), in a fixed tree order
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) p += __shfl_xor(p, o, 64);
    if (l == 0) out[j] = p;
  }
}

// ---- column lists: one workgroup (1024 threads) per (b, h) -----------------------------------
// Radix select (four 8-bit digits of the non-negative fp32 bit patterns) finds the n-th largest
// importance T and how many of the keys equal to T to take; an ordered pass then lists every
// key above T and the lowest-index keys equal to T, in ascending key order.
__global__ __launch_bounds__(1024) void col_topk_kernel(const float* imp, int L, int ncols,
                                                        int32_t* col_ptr, int32_t* col_idx,
                                                        int nheads) {
  __shared__ int hist[256];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_remaining;
  __shared__ int wcnt[2][16];
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
    for (int j = tid; j < L; j += 1024) {
      const uint32_t x = v[j];
      if ((x & pmask) == prefix) atomicAdd(&hist[(x >> shift) & 255u], 1);
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
  int ties_before = 0, sel_before = 0;
  for (int c0 = 0; c0 < L; c0 += 1024) {
    const int j = c0 + tid;
    const uint32_t x = j < L ? v[j] : 0u;
    const bool gt = j < L && x > prefix;
    const bool eq = j < L && x == prefix;
    const uint64_t beq = __ballot(eq);
    const int eq_rank_w = __builtin_amdgcn_mbcnt_hi((uint32_t)(beq >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)beq, 0u));
    if (ln == 0) wcnt[0][wv] = __popcll(beq);
    __syncthreads();
    int eq_off = 0, eq_tot = 0;
    for (int u = 0; u < 16; ++u) { eq_off += u < wv ? wcnt[0][u] : 0; eq_tot += wcnt[0][u]; }
    const bool sel = gt || (eq && ties_before + eq_off + eq_rank_w < remaining);
    const uint64_t bsel = __ballot(sel);
    const int sel_rank_w = __builtin_amdgcn_mbcnt_hi((uint32_t)(bsel >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bsel, 0u));
    if (ln == 0) wcnt[1][wv] = __popcll(bsel);
    __syncthreads();
    int sel_off = 0, sel_tot = 0;
    for (int u = 0; u < 16; ++u) { sel_off += u < wv ? wcnt[1][u] : 0; sel_tot += wcnt[1][u]; }
    if (sel) col_idx[base + sel_before + sel_off + sel_rank_w] = j;
    ties_before += eq_tot;
    sel_before += sel_tot;
    __syncthreads();
  }
}

template <int D>
hipError_t launch_index_t(const IndexArgs& a, hipStream_t stream) {
  const int nqb = (a.L + kIndexBlock - 1) / kIndexBlock;
  const int nch = (a.L + kProbeChunk - 1) / kProbeChunk;
  hipLaunchKernelGGL((pool_kernel<D>), dim3((unsigned)(a.B * a.Hq * nqb)), dim3(D), 0, stream,
                     a.q, a.q_sb, a.q_sl, a.q_sh, a.Hq, a.L, a.qbar);
  hipLaunchKernelGGL((pool_kernel<D>), dim3((unsigned)(a.B * a.Hkv * nqb)), dim3(D), 0, stream,
                     a.k, a.k_sb, a.k_sl, a.k_sh, a.Hkv, a.L, a.kbar);
  hipLaunchKernelGGL((block_topk_kernel<D>), dim3((unsigned)(a.B * a.Hq * nqb)), dim3(256), 0,
                     stream, a.qbar, a.kbar, a.Hq, a.Hkv, nqb, a.scale, a.topk, a.blk_ptr,
                     a.blk_idx, a.blk_head_len, a.blk_total);
  hipLaunchKernelGGL((probe_stats_kernel<D>), dim3((unsigned)(a.B * a.Hq * nch)), dim3(256), 0,
                     stream, a, a.stats);
  hipLaunchKernelGGL((probe_importance_kernel<D>), dim3((unsigned)(a.B * a.Hq * nch)), dim3(256),
                     0, stream, a, a.stats, a.imp);
  hipLaunchKernelGGL(col_topk_kernel, dim3((unsigned)(a.B * a.Hq)), dim3(1024), 0, stream,
                     a.imp, a.L, a.ncols, a.col_ptr, a.col_idx, a.B * a.Hq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_index(const IndexArgs& a, int d, hipStream_t stream) {
  if (d == 128) return launch_index_t<128>(a, stream);
  return launch_index_t<64>(a, stream);
}

}  // namespace attn
