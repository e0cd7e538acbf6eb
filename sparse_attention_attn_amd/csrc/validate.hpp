// validate.hpp — host-side argument checks of the C ABI. Pure C++: no HIP dependency, so the
// same code is unit-tested on a machine without a GPU (and under host sanitizers).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/attn.h"

namespace attn {

// Thread-local message of the last failed call.
void set_last_error(const std::string& msg);
void clear_last_error();
const char* last_error_cstr();

// Records `msg` (prefixed with the entry point name) and returns `status`.
int fail(int status, const char* fn, const std::string& msg);

enum class Op { kDense, kSplit, kSparse };

// Common checks of sizes, head dims, scale, pointers, alignment and strides.
int check_attention_args(const char* fn, Op op, const attn_tensor_t& q, const attn_tensor_t& k,
                         const attn_tensor_t& v, const attn_tensor_t* o, const float* lse, int B,
                         int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv, float scale);

int check_num_splits(const char* fn, int num_splits, int Lk);

// Split count heuristic for a 256-CU MI355X (pure function).
// Query columns ((head, position) pairs of one KV head) per split-KV workgroup: 32 when there
// are more than 16 (two 16-column blocks then share every read of the cache: GQA groups of 32
// heads, 8 heads with 4 query tokens, the latent shape with 2 tokens), 16 otherwise.
inline int split_cols(int dqk, int ncols) { (void)dqk; return ncols > 16 ? 32 : 16; }

// D = 128 split-KV grids of one 16-column block per workgroup and at most one workgroup per CU
// (256) run the decode kernel with a 4-stage ring of 32-key tiles (64 KiB of LDS); larger grids
// run it with a 2-stage ring of 64-key tiles, two workgroups per CU. Measured per call over
// D = 128 decode shapes (B 1..64, 512..131072 keys): the 32-key ring at one round of one
// workgroup per CU against the 64-key ring at its best grid, 2-15% faster (B 16, 4K keys: 48.1
// -> 45.3 us at 2 splits instead of 4); at two workgroups per CU it is the slower one (B 64,
// one split: 24.3 -> 26.2 us at 512 keys), and so it is with two column blocks per workgroup.
inline bool split_ring32(int dqk, int ncols, int64_t nwg) {
  return dqk == 128 && split_cols(dqk, ncols) == 16 && nwg <= 256;
}

// Split-KV of a prefill-shaped query block (D = 64 or 128; at least 128 query rows, or 64 over
// at least 8192 keys): the dense kernel's split form computes the partials (128-row workgroups
// per key range) instead of the decode kernel, whose workgroups take at most 32 query columns of
// a KV head. Measured per call at B 1, Hq 32, Hkv 8: 64 rows over 32K keys 129.6 -> 93.7 us,
// 96 rows 202.0 -> 97.4 us; 64 rows over 4K keys 28.8 against 30.0 us, 32 rows over 32K 76.7
// against 83.7 us (the decode kernel ahead).
inline bool dense_split_shape(int dqk, int dv, int lq, int lk) {
  return dqk == dv && (dqk == 64 || dqk == 128) && (lq >= 128 || (lq >= 64 && lk >= 8192));
}

int pick_num_splits(int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv);

// Keys per split: 64 * ceil(ceil(Lk / S) / 64).
int split_chunk(int Lk, int num_splits);
// One-call decode workspace: the split partials O_part and LSE_part; byte offsets, 256-byte
// aligned.
struct DecodeWorkspace {
  int num_splits;
  size_t o_part, lse_part, total;
};
DecodeWorkspace decode_workspace(int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv);

size_t workspace_bytes(int B, int Hq, int Lq, int Dv, int num_splits);

int check_combine_args(const char* fn, const float* o_part, const float* lse_part, int num_splits,
                       const attn_tensor_t& o, const float* lse, int B, int Hq, int Lq, int Dv);

// CSR index-list structure check on HOST arrays.
int check_blocksparse_lists(const char* fn, const int32_t* blk_ptr, const int32_t* blk_idx,
                            const int32_t* col_ptr, const int32_t* col_idx, int B, int Hq, int Lq,
                            int Lk, int block_m, int block_n);

// Largest sequence stride (elements) of Q/K/V: in-tile offsets are 32-bit.
constexpr int64_t kMaxStrideL = int64_t(1) << 24;

// Largest key length the block-sparse kernel's listed-block bitmap covers.
constexpr int kSparseMaxLk = 1 << 20;

// Dynamic sparse-index builder (square causal sizes L = Lq = Lk).
constexpr int kIndexMaxL = 131072;  // 2048 key blocks: one builder workgroup sorts them in LDS
// Block-list entries per head: sum over query blocks qb of min(topk, qb + 1).
int check_slash_lists(const char* fn, const int32_t* slash_ptr, const int32_t* slash_idx, int B,
                      int Hq, int Lk);
int64_t index_blk_head_len(int L, int topk);
// Workspace layout (byte offsets, 256-byte aligned) and total size.
struct IndexWorkspace {
  size_t qbar, kbar, stats, fin, imp, simp, total;
};
IndexWorkspace index_workspace(int B, int Hq, int Hkv, int L, int D);
int check_index_args(const char* fn, const attn_tensor_t& q, const attn_tensor_t& k, int B, int Hq,
                     int Hkv, int L, int D, float scale, int topk, int ncols,
                     const int32_t* blk_ptr, const int32_t* blk_idx, const int32_t* col_ptr,
                     const int32_t* col_idx, const void* workspace, size_t workspace_bytes);

int check_vslash_index_args(const char* fn, const attn_tensor_t& q, const attn_tensor_t& k, int B,
                            int Hq, int Hkv, int L, int D, float scale, int ncols, int nslash,
                            const int32_t* col_ptr, const int32_t* col_idx,
                            const int32_t* slash_ptr, const int32_t* slash_idx,
                            const void* workspace, size_t workspace_bytes);

const char* status_string(int status);

}  // namespace attn
