// kernels.hpp — argument blocks and launchers shared by the host API and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Dense and block-sparse forward (one launch writes O and LSE).
struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;  // [B, Hq, Lq] or nullptr
  int64_t q_sb, q_sl, q_sh;
  int64_t k_sb, k_sl, k_sh;
  int64_t v_sb, v_sl, v_sh;
  int64_t o_sb, o_sl, o_sh;
  int B, Hq, Hkv, Lq, Lk, g;
  int causal;
  int off;        // Lk - Lq (bottom-right causal alignment)
  float sl2;      // |scale| * log2(e), > 0 (see exp2_scale)
  uint32_t qsign; // 0x80008000 when scale < 0: the kernels negate Q as they load it
  int n_qtiles;   // query tiles per (b, hq)
  int xcd_remap;  // how logical tiles map to XCDs (0: none; see the kernels' launchers)
  // split form of the dense kernel (launch_fwd_dense_split): split s covers keys
  // [s * chunk, min((s + 1) * chunk, Lk)) and writes its normalised partials here
  float* o_part;    // [S, B, Hq, Lq, Dv]
  float* lse_part;  // [S, B, Hq, Lq]
  int num_splits;
  int chunk;        // keys per split (multiple of 64)
  // block-sparse lists (device pointers), unused by the dense kernel
  const int32_t* blk_ptr;
  const int32_t* blk_idx;
  const int32_t* col_ptr;
  const int32_t* col_idx;
  int nkb;        // ceil(Lk / 64)
  // slash lines (vertical-slash pattern): per-head offsets and the two per-head bitmaps
  const int32_t* sl_ptr;
  const int32_t* sl_idx;
  const uint32_t* sl_bits;  // [B*Hq][bits_words]: bit o + 128 set for a listed offset o
  const uint32_t* cl_bits;  // [B*Hq][bits_words]: bit j set for a listed column j
  const uint32_t* rl_bits;  // [B*Hq][bits_words]: bit o + 128 set for a listed offset o whose
                            // neighbour o - 1 or o + 1 is listed too (a line inside a run)
  int bits_words;
};

// Longest key sequence of the vertical-slash forward (its kernel keeps three block bitmaps in
// LDS beside two 36 KiB stages, two workgroups per CU).
constexpr int kVslashMaxLk = 1 << 19;

// Words per head of each vertical-slash bitmap.
constexpr int vs_bits_words(int Lk) { return (Lk + 255) / 32 + 2; }
// Bitmaps per head in the vertical-slash workspace (offsets, columns, offsets inside runs).
constexpr int kVslashBitmaps = 3;

// Split-KV partials.
struct SplitArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* o_part;    // [S, B, Hq, Lq, Dv]
  float* lse_part;  // [S, B, Hq, Lq]
  int64_t q_sb, q_sl, q_sh;
  int64_t k_sb, k_sl, k_sh;
  int64_t v_sb, v_sl, v_sh;
  int B, Hq, Hkv, Lq, Lk, g;
  int causal;
  int off;
  float sl2;        // |scale| * log2(e), > 0 (see exp2_scale)
  uint32_t qsign;   // 0x80008000 when scale < 0: Q is negated as it is loaded
  int num_splits;
  int chunk;        // keys per split (multiple of 64)
  int ncolblk;      // ceil(g * Lq / split_cols(Dqk, g * Lq))
  // One split only: when o is set, the kernel writes the final O (bf16, strided like attn_fwd's
  // O) and LSE (fp32 [B, Hq, Lq] or nullptr) instead of the partials, and no combine follows.
  uint16_t* o;
  int64_t o_sb, o_sl, o_sh;
  float* lse;
};

struct CombineArgs {
  const float* o_part;
  const float* lse_part;
  uint16_t* o;
  float* lse;
  int64_t o_sb, o_sl, o_sh;
  int B, Hq, Lq, S;
};

// Dynamic sparse-index builder (square causal sizes, L = Lq = Lk).
struct IndexArgs {
  const uint16_t* q;
  const uint16_t* k;
  int64_t q_sb, q_sl, q_sh;
  int64_t k_sb, k_sl, k_sh;
  int B, Hq, Hkv, L;
  float scale;         // score scale of the pooled block scores
  float sl2;           // scale * log2(e): probe scores in the exp2 domain
  int topk;            // blocks listed per query block (at most; the diagonal included)
  int ncols;           // vertical columns listed per head (at most L)
  int32_t* blk_ptr;    // [B*Hq*nqb + 1]
  int32_t* blk_idx;    // [blk_total]
  int32_t* col_ptr;    // [B*Hq + 1]
  int32_t* col_idx;    // [B*Hq*min(ncols, L)]
  int64_t blk_head_len;  // block-list entries per head
  int64_t blk_total;     // B*Hq*blk_head_len
  float* qbar;         // workspace: pooled Q [B, Hq, nqb, D]
  float* kbar;         // workspace: pooled K, transposed [B, Hkv, D, nqb]
  float* stats;        // workspace: probe softmax statistics [B, Hq, nchunks, 64, 2]
  float* fin;          // workspace: per probe row, max + log2(sum) over all keys [B, Hq, 64]
  float* imp;          // workspace: column importance [B, Hq, L]
  float* simp;         // workspace: slash-line importance [B, Hq, L] (vertical-slash builder)
  int nslash;          // slash lines listed per head (vertical-slash builder)
  int32_t* sl_ptr;     // [B*Hq + 1] (vertical-slash builder)
  int32_t* sl_idx;     // [B*Hq*min(nslash, L)] (vertical-slash builder)
};

// Rows per pooled block, the largest block count one list builder workgroup sorts, probe rows,
// keys per probe workgroup.
constexpr int kIndexBlock = 64;
constexpr int kIndexMaxBlocks = 2048;
constexpr int kProbeRows = 64;
constexpr int kProbeChunk = 1024;

hipError_t launch_fwd_dense(const FwdArgs& a, int d, hipStream_t stream);
hipError_t launch_fwd_dense_split(const FwdArgs& a, int d, hipStream_t stream);
hipError_t launch_build_index(const IndexArgs& a, int d, hipStream_t stream);
hipError_t launch_fwd_vslash(const FwdArgs& a, int d, hipStream_t stream);
hipError_t launch_build_vslash_index(const IndexArgs& a, int d, hipStream_t stream);
hipError_t launch_fwd_blocksparse(const FwdArgs& a, int d, hipStream_t stream);
hipError_t launch_splitkv(const SplitArgs& a, int dqk, int dv, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, int dv, hipStream_t stream);

// Compute units of an MI355X (the launchers size their grids against it).
constexpr int kCUs = 256;
// Query rows per workgroup of the block-sparse kernel (one 64-row query block).
constexpr int kSparseBlockM = 64;
// Query columns per 16-column block of a split-KV workgroup (see split_cols in validate.hpp).
constexpr int kSplitCols = 16;

}  // namespace attn
