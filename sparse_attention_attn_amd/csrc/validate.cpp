// validate.cpp — host-side argument checks of the C ABI (pure C++, no HIP).
#include "validate.hpp"

#include <algorithm>
#include <cmath>
#include <limits>
#include <sstream>

namespace attn {

namespace {
thread_local std::string g_last_error;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int check_tensor(const char* fn, const char* name, const attn_tensor_t& t) {
  if (t.data == nullptr) return fail(ATTN_ERR_INVALID_ARG, fn, std::string(name) + " is NULL");
  if (!aligned16(t.data))
    return fail(ATTN_ERR_INVALID_ARG, fn, std::string(name) + " data is not 16-byte aligned");
  if (t.stride_b < 0 || t.stride_l < 0 || t.stride_h < 0)
    return fail(ATTN_ERR_INVALID_ARG, fn, std::string(name) + " has a negative stride");
  if ((t.stride_b % 8) != 0 || (t.stride_l % 8) != 0 || (t.stride_h % 8) != 0)
    return fail(ATTN_ERR_INVALID_ARG, fn,
                std::string(name) + " strides must be multiples of 8 elements (16 bytes)");
  // In-tile offsets (row * stride_l + column, up to 64 rows) are kept in 32-bit registers.
  if (t.stride_l > kMaxStrideL)
    return fail(ATTN_ERR_UNSUPPORTED, fn,
                std::string(name) + " sequence stride exceeds 2^24 elements");
  return ATTN_OK;
}

bool dims_ok(Op op, int Dqk, int Dv) {
  if ((Dqk == 64 && Dv == 64) || (Dqk == 128 && Dv == 128)) return true;
  return op == Op::kSplit && Dqk == 576 && Dv == 512;
}
}  // namespace

void set_last_error(const std::string& msg) { g_last_error = msg; }
void clear_last_error() { g_last_error.clear(); }
const char* last_error_cstr() { return g_last_error.c_str(); }

int fail(int status, const char* fn, const std::string& msg) {
  g_last_error = std::string(fn) + ": " + msg;
  return status;
}

int check_attention_args(const char* fn, Op op, const attn_tensor_t& q, const attn_tensor_t& k,
                         const attn_tensor_t& v, const attn_tensor_t* o, const float* lse, int B,
                         int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv, float scale) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 1 || Lk < 1) {
    std::ostringstream s;
    s << "sizes must be >= 1 (B=" << B << " Hq=" << Hq << " Hkv=" << Hkv << " Lq=" << Lq
      << " Lk=" << Lk << ")";
    return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
  }
  if (Hq % Hkv != 0) {
    std::ostringstream s;
    s << "Hq (" << Hq << ") must be a multiple of Hkv (" << Hkv << ")";
    return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
  }
  if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, fn, "scale is not finite");
  if (!dims_ok(op, Dqk, Dv)) {
    std::ostringstream s;
    s << "head dims (Dqk=" << Dqk << ", Dv=" << Dv << ") not supported; supported: (64,64), (128,128)"
      << (op == Op::kSplit ? ", (576,512)" : "");
    return fail(ATTN_ERR_UNSUPPORTED, fn, s.str());
  }
  int st;
  if ((st = check_tensor(fn, "q", q)) != ATTN_OK) return st;
  if ((st = check_tensor(fn, "k", k)) != ATTN_OK) return st;
  if ((st = check_tensor(fn, "v", v)) != ATTN_OK) return st;
  if (o != nullptr && (st = check_tensor(fn, "o", *o)) != ATTN_OK) return st;
  if (lse != nullptr && !aligned4(lse))
    return fail(ATTN_ERR_INVALID_ARG, fn, "lse is not 4-byte aligned");
  if (Dqk != Dv && (v.data != k.data || v.stride_b != k.stride_b || v.stride_l != k.stride_l ||
                    v.stride_h != k.stride_h)) {
    return fail(ATTN_ERR_UNSUPPORTED, fn,
                "the (576, 512) latent shape requires v to alias k (same pointer and strides)");
  }
  // grid sizes and index arithmetic stay within 31 bits for the launch dimensions
  const int64_t rows = (int64_t)B * Hq * Lq;
  if (rows > (int64_t)std::numeric_limits<int>::max() / 4)
    return fail(ATTN_ERR_UNSUPPORTED, fn, "B*Hq*Lq too large");
  if (op == Op::kSparse && Lk > kSparseMaxLk) {
    std::ostringstream s;
    s << "Lk=" << Lk << " exceeds the block-sparse limit of " << kSparseMaxLk;
    return fail(ATTN_ERR_UNSUPPORTED, fn, s.str());
  }
  return ATTN_OK;
}

int check_num_splits(const char* fn, int num_splits, int Lk) {
  const int maxs = (Lk + 63) / 64;
  if (num_splits < 1 || num_splits > maxs) {
    std::ostringstream s;
    s << "num_splits=" << num_splits << " outside [1, ceil(Lk/64)=" << maxs << "]";
    return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
  }
  return ATTN_OK;
}

namespace {

// Split count for `units` split-KV work units aiming at `grid` workgroups (see pick_num_splits).
int splits_for_grid(int64_t units, int64_t grid, int Lk, int min_keys) {
  int64_t s = (grid + units - 1) / units;
  // A grid just past a whole number of rounds leaves a short last round (B 24 at D = 128:
  // 3 splits, 576 workgroups, 36.1 / 97.5 / 353.2 us at 1K / 4K / 16K keys). Take instead the
  // smallest split count that fills whole rounds with splits of at least 512 keys (8 splits:
  // 29.9 / 84.3 / 283.3 us), else the largest that stays within one round (2 splits: 26.9 /
  // 86.8 / 306.5 us); at B 48, 4 splits (147.8 / 549.5 us at 4K / 16K) or 1 (42.7 us at 1K)
  // against 2 (165.2 / 585.7 / 48.3 us).
  if ((units * s) % grid != 0) {
    int64_t fill = 0;
    for (int64_t t = s; t <= 8 * s && t <= 256; ++t)
      if ((units * t) % grid == 0 && Lk / t >= 512) {
        fill = t;
        break;
      }
    s = fill ? fill : std::max<int64_t>(1, grid / units);
  }
  const int64_t max_by_len = std::max<int64_t>(1, Lk / min_keys);
  const int64_t max_s = (Lk + 63) / 64;
  s = std::min(s, max_by_len);
  s = std::min(s, max_s);
  s = std::min<int64_t>(s, 256);
  s = std::max<int64_t>(s, 1);
  // splits are whole 64-key tiles: drop those the rounding of the split length leaves empty
  const int chunk = split_chunk(Lk, (int)s);
  return (int)((Lk + chunk - 1) / chunk);
}

}  // namespace

int pick_num_splits(int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv) {
  (void)Dv;
  if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 1 || Lk < 1 || Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (dense_split_shape(Dqk, Dv, Lq, Lk)) {
    // the dense kernel's split form: one round of two 128-row workgroups per CU, splits of at
    // least 1024 keys, none empty
    const int64_t units = (int64_t)B * Hq * ((Lq + 127) / 128);
    int64_t s = std::max<int64_t>(1, 512 / units);
    s = std::min<int64_t>(s, std::max<int64_t>(1, Lk / 1024));
    s = std::min<int64_t>(s, 256);
    const int chunk = split_chunk(Lk, (int)s);
    return (int)((Lk + chunk - 1) / chunk);
  }
  const int g = Hq / Hkv;
  const int cols = split_cols(Dqk, g * Lq);
  const int64_t colblk = ((int64_t)g * Lq + cols - 1) / cols;
  const int64_t units = (int64_t)B * Hkv * colblk;
  // Grid size and keys per split, measured over B 1..64, 512..131072 keys and the three head
  // shapes (GPU time per call, splits forced from 1 to 512): the best grids hold one round of
  // one D = 64 or latent workgroup per CU (256); a split keeps at least one 64-key tile (two for
  // the latent, whose 1152-byte rows make short splits pay for their partials), and more than
  // 256 splits only adds combine work (B 1, one KV head, 131072 keys: 24.4 us at 256 splits,
  // 26.1 at 512). D = 128 with one 16-column block per workgroup: one round of one workgroup
  // per CU (the 4-stage ring of 32-key tiles, split_ring32) when the units fit it, else one
  // round of two per CU (512, the 2-stage ring of 64-key tiles).
  const int min_keys = (Dqk == 576) ? 128 : 64;
  if (Dqk == 128 && cols == 16) {
    const int s = splits_for_grid(units, 256, Lk, min_keys);
    if (split_ring32(Dqk, g * Lq, units * s)) return s;
  }
  return splits_for_grid(units, Dqk == 128 ? 512 : 256, Lk, min_keys);
}

int split_chunk(int Lk, int num_splits) {
  const int per = (Lk + num_splits - 1) / num_splits;
  return 64 * ((per + 63) / 64);
}

size_t workspace_bytes(int B, int Hq, int Lq, int Dv, int num_splits) {
  if (B < 1 || Hq < 1 || Lq < 1 || Dv < 1 || num_splits < 1) return 0;
  const size_t rows = (size_t)num_splits * B * Hq * Lq;
  return rows * (size_t)Dv * sizeof(float) + rows * sizeof(float);
}

DecodeWorkspace decode_workspace(int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv) {
  DecodeWorkspace w{0, 0, 0, 0};
  const int s = pick_num_splits(B, Hq, Hkv, Lq, Lk, Dqk, Dv);
  if (s < 1) return w;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t rows = (size_t)s * B * Hq * Lq;
  w.num_splits = s;
  w.o_part = 0;
  w.lse_part = up(rows * (size_t)Dv * sizeof(float));
  w.total = up(w.lse_part + rows * sizeof(float));
  return w;
}

int check_combine_args(const char* fn, const float* o_part, const float* lse_part, int num_splits,
                       const attn_tensor_t& o, const float* lse, int B, int Hq, int Lq, int Dv) {
  if (B < 1 || Hq < 1 || Lq < 1 || num_splits < 1)
    return fail(ATTN_ERR_INVALID_ARG, fn, "sizes and num_splits must be >= 1");
  if (Dv != 64 && Dv != 128 && Dv != 512) {
    std::ostringstream s;
    s << "Dv=" << Dv << " not supported (64, 128, 512)";
    return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
  }
  if (o_part == nullptr || lse_part == nullptr)
    return fail(ATTN_ERR_WORKSPACE, fn, "o_part / lse_part is NULL");
  if (!aligned16(o_part) || !aligned4(lse_part))
    return fail(ATTN_ERR_INVALID_ARG, fn, "o_part must be 16-byte and lse_part 4-byte aligned");
  if (o.data == nullptr) return fail(ATTN_ERR_INVALID_ARG, fn, "o is NULL");
  if (!aligned16(o.data) || (o.stride_b % 8) || (o.stride_l % 8) || (o.stride_h % 8) ||
      o.stride_b < 0 || o.stride_l < 0 || o.stride_h < 0)
    return fail(ATTN_ERR_INVALID_ARG, fn, "o must be 16-byte aligned with strides multiple of 8");
  if (lse != nullptr && !aligned4(lse))
    return fail(ATTN_ERR_INVALID_ARG, fn, "lse is not 4-byte aligned");
  return ATTN_OK;
}

int check_blocksparse_lists(const char* fn, const int32_t* blk_ptr, const int32_t* blk_idx,
                            const int32_t* col_ptr, const int32_t* col_idx, int B, int Hq, int Lq,
                            int Lk, int block_m, int block_n) {
  if (B < 1 || Hq < 1 || Lq < 1 || Lk < 1)
    return fail(ATTN_ERR_INVALID_ARG, fn, "sizes must be >= 1");
  if (block_m != 64 || block_n != 64)
    return fail(ATTN_ERR_UNSUPPORTED, fn, "block_m and block_n must be 64");
  if (blk_ptr == nullptr || col_ptr == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, fn, "blk_ptr / col_ptr is NULL");
  const int64_t nqb = (Lq + 63) / 64;
  const int64_t nkb = (Lk + 63) / 64;
  const int64_t nrows = (int64_t)B * Hq * nqb;
  if (blk_ptr[0] != 0) return fail(ATTN_ERR_INVALID_ARG, fn, "blk_ptr[0] must be 0");
  for (int64_t r = 0; r < nrows; ++r) {
    const int32_t lo = blk_ptr[r], hi = blk_ptr[r + 1];
    if (hi < lo) {
      std::ostringstream s;
      s << "blk_ptr decreases at row " << r;
      return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
    }
    if (hi > lo && blk_idx == nullptr) return fail(ATTN_ERR_INVALID_ARG, fn, "blk_idx is NULL");
    for (int32_t i = lo; i < hi; ++i) {
      const int32_t x = blk_idx[i];
      if (x < 0 || x >= nkb) {
        std::ostringstream s;
        s << "blk_idx[" << i << "]=" << x << " outside [0, " << nkb << ")";
        return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
      }
      if (i > lo && blk_idx[i - 1] >= x) {
        std::ostringstream s;
        s << "blk_idx not strictly increasing at " << i;
        return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
      }
    }
  }
  if (col_ptr[0] != 0) return fail(ATTN_ERR_INVALID_ARG, fn, "col_ptr[0] must be 0");
  for (int64_t r = 0; r < (int64_t)B * Hq; ++r) {
    const int32_t lo = col_ptr[r], hi = col_ptr[r + 1];
    if (hi < lo) {
      std::ostringstream s;
      s << "col_ptr decreases at head row " << r;
      return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
    }
    if (hi > lo && col_idx == nullptr) return fail(ATTN_ERR_INVALID_ARG, fn, "col_idx is NULL");
    for (int32_t i = lo; i < hi; ++i) {
      const int32_t x = col_idx[i];
      if (x < 0 || x >= Lk) {
        std::ostringstream s;
        s << "col_idx[" << i << "]=" << x << " outside [0, " << Lk << ")";
        return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
      }
      if (i > lo && col_idx[i - 1] >= x) {
        std::ostringstream s;
        s << "col_idx not strictly increasing at " << i;
        return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
      }
    }
  }
  return ATTN_OK;
}

int check_slash_lists(const char* fn, const int32_t* slash_ptr, const int32_t* slash_idx, int B,
                      int Hq, int Lk) {
  if (B < 1 || Hq < 1 || Lk < 1) return fail(ATTN_ERR_INVALID_ARG, fn, "sizes must be >= 1");
  if (slash_ptr == nullptr) return fail(ATTN_ERR_INVALID_ARG, fn, "slash_ptr is NULL");
  if (slash_ptr[0] != 0) return fail(ATTN_ERR_INVALID_ARG, fn, "slash_ptr[0] must be 0");
  for (int64_t r = 0; r < (int64_t)B * Hq; ++r) {
    const int32_t lo = slash_ptr[r], hi = slash_ptr[r + 1];
    if (hi < lo) {
      std::ostringstream s;
      s << "slash_ptr decreases at head row " << r;
      return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
    }
    if (hi > lo && slash_idx == nullptr) return fail(ATTN_ERR_INVALID_ARG, fn, "slash_idx is NULL");
    for (int32_t i = lo; i < hi; ++i) {
      const int32_t x = slash_idx[i];
      if (x < 0 || x >= Lk) {
        std::ostringstream s;
        s << "slash_idx[" << i << "]=" << x << " outside [0, " << Lk << ")";
        return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
      }
      if (i > lo && slash_idx[i - 1] >= x) {
        std::ostringstream s;
        s << "slash_idx not strictly increasing at " << i;
        return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
      }
    }
  }
  return ATTN_OK;
}

int64_t index_blk_head_len(int L, int topk) {
  if (L < 1 || topk < 1) return 0;
  const int64_t nqb = (L + 63) / 64;
  if (nqb <= topk) return nqb * (nqb + 1) / 2;
  return (int64_t)topk * (topk + 1) / 2 + (nqb - topk) * (int64_t)topk;
}

IndexWorkspace index_workspace(int B, int Hq, int Hkv, int L, int D) {
  IndexWorkspace w{0, 0, 0, 0, 0, 0, 0};
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || D < 1) return w;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t nqb = (size_t)(L + 63) / 64;
  const size_t nch = (size_t)(L + 1023) / 1024;
  size_t off = 0;
  w.qbar = off; off = up(off + (size_t)B * Hq * nqb * D * 4);
  w.kbar = off; off = up(off + (size_t)B * Hkv * nqb * D * 4);
  w.stats = off; off = up(off + (size_t)B * Hq * nch * 64 * 2 * 4);
  w.fin = off; off = up(off + (size_t)B * Hq * 64 * 4);
  w.imp = off; off = up(off + (size_t)B * Hq * L * 4);
  w.simp = off; off = up(off + (size_t)B * Hq * L * 4);
  w.total = off;
  return w;
}

int check_index_args(const char* fn, const attn_tensor_t& q, const attn_tensor_t& k, int B, int Hq,
                     int Hkv, int L, int D, float scale, int topk, int ncols,
                     const int32_t* blk_ptr, const int32_t* blk_idx, const int32_t* col_ptr,
                     const int32_t* col_idx, const void* workspace, size_t workspace_bytes) {
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1) {
    std::ostringstream s;
    s << "sizes must be >= 1 (B=" << B << " Hq=" << Hq << " Hkv=" << Hkv << " L=" << L << ")";
    return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
  }
  if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, fn, "Hq must be a multiple of Hkv");
  if (topk < 1) return fail(ATTN_ERR_INVALID_ARG, fn, "topk_blocks must be >= 1");
  if (ncols < 0) return fail(ATTN_ERR_INVALID_ARG, fn, "n_cols must be >= 0");
  if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, fn, "scale is not finite");
  if (D != 64 && D != 128) {
    std::ostringstream s;
    s << "D=" << D << " not supported (64, 128)";
    return fail(ATTN_ERR_UNSUPPORTED, fn, s.str());
  }
  if (L > kIndexMaxL) {
    std::ostringstream s;
    s << "L=" << L << " exceeds the index builder's limit of " << kIndexMaxL;
    return fail(ATTN_ERR_UNSUPPORTED, fn, s.str());
  }
  int st;
  if ((st = check_tensor(fn, "q", q)) != ATTN_OK) return st;
  if ((st = check_tensor(fn, "k", k)) != ATTN_OK) return st;
  const int64_t nblk = (int64_t)B * Hq * index_blk_head_len(L, topk);
  const int64_t ncol = (int64_t)B * Hq * std::min(ncols, L);
  const int64_t nptr = (int64_t)B * Hq * ((L + 63) / 64) + 1;
  const int64_t imax = std::numeric_limits<int32_t>::max();
  if (nblk > imax || ncol > imax || nptr > imax)
    return fail(ATTN_ERR_UNSUPPORTED, fn, "an index list would exceed 2^31 entries");
  if (blk_ptr == nullptr || blk_idx == nullptr || col_ptr == nullptr ||
      (ncol > 0 && col_idx == nullptr))
    return fail(ATTN_ERR_INVALID_ARG, fn, "an output list pointer is NULL");
  if (!aligned4(blk_ptr) || !aligned4(blk_idx) || !aligned4(col_ptr) ||
      (col_idx != nullptr && !aligned4(col_idx)))
    return fail(ATTN_ERR_INVALID_ARG, fn, "output lists must be 4-byte aligned");
  const size_t need = index_workspace(B, Hq, Hkv, L, D).total;
  if (workspace == nullptr || workspace_bytes < need ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) {
    std::ostringstream s;
    s << "workspace must be non-NULL, 256-byte aligned and at least " << need << " bytes";
    return fail(ATTN_ERR_WORKSPACE, fn, s.str());
  }
  return ATTN_OK;
}

int check_vslash_index_args(const char* fn, const attn_tensor_t& q, const attn_tensor_t& k, int B,
                            int Hq, int Hkv, int L, int D, float scale, int ncols, int nslash,
                            const int32_t* col_ptr, const int32_t* col_idx,
                            const int32_t* slash_ptr, const int32_t* slash_idx,
                            const void* workspace, size_t workspace_bytes) {
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1) {
    std::ostringstream s;
    s << "sizes must be >= 1 (B=" << B << " Hq=" << Hq << " Hkv=" << Hkv << " L=" << L << ")";
    return fail(ATTN_ERR_INVALID_ARG, fn, s.str());
  }
  if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, fn, "Hq must be a multiple of Hkv");
  if (ncols < 0) return fail(ATTN_ERR_INVALID_ARG, fn, "n_cols must be >= 0");
  if (nslash < 0) return fail(ATTN_ERR_INVALID_ARG, fn, "n_slash must be >= 0");
  if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, fn, "scale is not finite");
  if (D != 64 && D != 128) {
    std::ostringstream s;
    s << "D=" << D << " not supported (64, 128)";
    return fail(ATTN_ERR_UNSUPPORTED, fn, s.str());
  }
  if (L > kIndexMaxL) {
    std::ostringstream s;
    s << "L=" << L << " exceeds the index builder's limit of " << kIndexMaxL;
    return fail(ATTN_ERR_UNSUPPORTED, fn, s.str());
  }
  int st;
  if ((st = check_tensor(fn, "q", q)) != ATTN_OK) return st;
  if ((st = check_tensor(fn, "k", k)) != ATTN_OK) return st;
  const int64_t ncol = (int64_t)B * Hq * std::min(ncols, L);
  const int64_t nsl = (int64_t)B * Hq * std::min(nslash, L);
  const int64_t imax = std::numeric_limits<int32_t>::max();
  if (ncol > imax || nsl > imax)
    return fail(ATTN_ERR_UNSUPPORTED, fn, "an index list would exceed 2^31 entries");
  if (col_ptr == nullptr || slash_ptr == nullptr || (ncol > 0 && col_idx == nullptr) ||
      (nsl > 0 && slash_idx == nullptr))
    return fail(ATTN_ERR_INVALID_ARG, fn, "an output list pointer is NULL");
  if (!aligned4(col_ptr) || !aligned4(slash_ptr) || (col_idx != nullptr && !aligned4(col_idx)) ||
      (slash_idx != nullptr && !aligned4(slash_idx)))
    return fail(ATTN_ERR_INVALID_ARG, fn, "output lists must be 4-byte aligned");
  const size_t need = index_workspace(B, Hq, Hkv, L, D).total;
  if (workspace == nullptr || workspace_bytes < need ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) {
    std::ostringstream s;
    s << "workspace must be non-NULL, 256-byte aligned and at least " << need << " bytes";
    return fail(ATTN_ERR_WORKSPACE, fn, s.str());
  }
  return ATTN_OK;
}

const char* status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH";
    default: return "ATTN_ERR_UNKNOWN";
  }
}

}  // namespace attn
