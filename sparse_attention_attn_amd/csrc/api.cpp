// api.cpp — the extern "C" entry points of libattn.so: validate on the host, then launch.
// Nothing here allocates device memory or synchronises; see include/attn.h for the contract.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <exception>
#include <mutex>
#include <sstream>
#include <string>

#include "../../include/attn.h"
#include "kernels.hpp"
#include "validate.hpp"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// The attention kernels work with a positive exp2-domain scale. A negative scale is folded
// into the sign of Q (the kernels negate Q as they load it), so masked scores stay -inf and
// row maxima stay maxima. A zero scale (or one whose |scale|·log2 e is not a normal float)
// becomes the smallest normal float: every visible key then gets weight exp2(~0) = 1 exactly,
// as with scale 0, and masking still works (-inf times a positive number).
void exp2_scale(float scale, float& sl2, uint32_t& qsign) {
  qsign = scale < 0.f ? 0x80008000u : 0u;
  const float s = std::fabs(scale) * kLog2e;
  sl2 = std::isnormal(s) ? s : FLT_MIN;
}

int launch_status(const char* fn, hipError_t e) {
  if (e == hipSuccess) return ATTN_OK;
  return attn::fail(ATTN_ERR_LAUNCH, fn, hipGetErrorString(e));
}

void fill_fwd(attn::FwdArgs& a, const attn_tensor_t& q, const attn_tensor_t& k,
              const attn_tensor_t& v, const attn_tensor_t& o, float* lse, int B, int Hq, int Hkv,
              int Lq, int Lk, int causal, float scale) {
  a.q = static_cast<const uint16_t*>(q.data);
  a.k = static_cast<const uint16_t*>(k.data);
  a.v = static_cast<const uint16_t*>(v.data);
  a.o = static_cast<uint16_t*>(o.data);
  a.lse = lse;
  a.q_sb = q.stride_b; a.q_sl = q.stride_l; a.q_sh = q.stride_h;
  a.k_sb = k.stride_b; a.k_sl = k.stride_l; a.k_sh = k.stride_h;
  a.v_sb = v.stride_b; a.v_sl = v.stride_l; a.v_sh = v.stride_h;
  a.o_sb = o.stride_b; a.o_sl = o.stride_l; a.o_sh = o.stride_h;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk; a.g = Hq / Hkv;
  a.causal = causal ? 1 : 0;
  a.off = Lk - Lq;
  exp2_scale(scale, a.sl2, a.qsign);
  a.xcd_remap = 0;
  a.blk_ptr = a.blk_idx = a.col_ptr = a.col_idx = nullptr;
  a.nkb = (Lk + 63) / 64;
  a.sl_ptr = a.sl_idx = nullptr;
  a.sl_bits = a.cl_bits = a.rl_bits = nullptr;
  a.bits_words = 0;
  a.o_part = a.lse_part = nullptr;
  a.num_splits = 1;
  a.chunk = 0;
}

// Split-KV partials of a prefill-shaped query block (attn::dense_split_shape) by the dense
// kernel's split form: same partial layout and split bounds as the decode kernel's.
int dense_split_launch(const char* fn, const attn_tensor_t& q, const attn_tensor_t& k,
                       const attn_tensor_t& v, float* o_part, float* lse_part, int num_splits,
                       int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int causal, float scale,
                       hipStream_t sm) {
  attn_tensor_t none{};
  attn::FwdArgs a;
  fill_fwd(a, q, k, v, none, nullptr, B, Hq, Hkv, Lq, Lk, causal, scale);
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.num_splits = num_splits;
  a.chunk = attn::split_chunk(Lk, num_splits);
  return launch_status(fn, attn::launch_fwd_dense_split(a, Dqk, sm));
}

// Split-KV decode into a checked workspace `wb` laid out by `ws`: the split kernel, then the
// combine (or the split kernel alone writing O and LSE when there is one split).
int decode_launch(const char* fn, const attn_tensor_t& q, const attn_tensor_t& k,
                  const attn_tensor_t& v, const attn_tensor_t& o, float* lse, int B, int Hq,
                  int Hkv, int Lq, int Lk, int Dqk, int Dv, int causal, float scale, char* wb,
                  const attn::DecodeWorkspace& ws, hipStream_t sm) {
  if (attn::dense_split_shape(Dqk, Dv, Lq, Lk)) {
    // a prefill-shaped query block: the dense kernel, whole (one split) or in splits + combine
    if (ws.num_splits == 1) {
      attn::FwdArgs f;
      fill_fwd(f, q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, causal, scale);
      return launch_status(fn, attn::launch_fwd_dense(f, Dqk, sm));
    }
    float* op = reinterpret_cast<float*>(wb + ws.o_part);
    float* lp = reinterpret_cast<float*>(wb + ws.lse_part);
    int st = dense_split_launch(fn, q, k, v, op, lp, ws.num_splits, B, Hq, Hkv, Lq, Lk, Dqk,
                                causal, scale, sm);
    if (st != ATTN_OK) return st;
    attn::CombineArgs c;
    c.o_part = op;
    c.lse_part = lp;
    c.o = static_cast<uint16_t*>(o.data);
    c.lse = lse;
    c.o_sb = o.stride_b; c.o_sl = o.stride_l; c.o_sh = o.stride_h;
    c.B = B; c.Hq = Hq; c.Lq = Lq; c.S = ws.num_splits;
    return launch_status(fn, attn::launch_combine(c, Dv, sm));
  }
  attn::SplitArgs a;
  a.q = static_cast<const uint16_t*>(q.data);
  a.k = static_cast<const uint16_t*>(k.data);
  a.v = static_cast<const uint16_t*>(v.data);
  a.o_part = reinterpret_cast<float*>(wb + ws.o_part);
  a.lse_part = reinterpret_cast<float*>(wb + ws.lse_part);
  a.q_sb = q.stride_b; a.q_sl = q.stride_l; a.q_sh = q.stride_h;
  a.k_sb = k.stride_b; a.k_sl = k.stride_l; a.k_sh = k.stride_h;
  a.v_sb = v.stride_b; a.v_sl = v.stride_l; a.v_sh = v.stride_h;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk; a.g = Hq / Hkv;
  a.causal = causal ? 1 : 0;
  a.off = Lk - Lq;
  exp2_scale(scale, a.sl2, a.qsign);
  a.num_splits = ws.num_splits;
  a.chunk = attn::split_chunk(Lk, ws.num_splits);
  const int cols = attn::split_cols(Dqk, a.g * Lq);
  a.ncolblk = (a.g * Lq + cols - 1) / cols;
  // One split: the split kernel writes O and LSE itself (the combine would only copy them).
  const bool direct = ws.num_splits == 1;
  a.o = direct ? static_cast<uint16_t*>(o.data) : nullptr;
  a.o_sb = o.stride_b; a.o_sl = o.stride_l; a.o_sh = o.stride_h;
  a.lse = direct ? lse : nullptr;
  int st = launch_status(fn, attn::launch_splitkv(a, Dqk, Dv, sm));
  if (st != ATTN_OK || direct) return st;
  attn::CombineArgs c;
  c.o_part = a.o_part;
  c.lse_part = a.lse_part;
  c.o = static_cast<uint16_t*>(o.data);
  c.lse = lse;
  c.o_sb = o.stride_b; c.o_sl = o.stride_l; c.o_sh = o.stride_h;
  c.B = B; c.Hq = Hq; c.Lq = Lq; c.S = ws.num_splits;
  return launch_status(fn, attn::launch_combine(c, Dv, sm));
}

}  // namespace

// Scratch of attn_fwd_decode_noalloc: the split-KV partials of callers that cannot allocate.
// In host code this name only stands in for the array; each device holds its own copy at its
// own address, which scratch_for_stream looks up once per device (hipGetSymbolAddress).
static __device__ __align__(256) char scratch[ATTN_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, set once

// Device address of `scratch` on the device that runs `stream` (the current device for the
// null stream). The first call on a device looks it up with that device current.
int scratch_for_stream(const char* fn, hipStream_t stream, char** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return attn::fail(ATTN_ERR_LAUNCH, fn, hipGetErrorString(e));
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return attn::fail(ATTN_ERR_LAUNCH, fn, hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) {
    std::ostringstream m;
    m << "device " << dev << " is beyond the " << kMaxDevices << " devices the scratch table holds";
    return attn::fail(ATTN_ERR_UNSUPPORTED, fn, m.str());
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return attn::fail(ATTN_ERR_LAUNCH, fn, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = dev != cur ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || p == nullptr) {
      std::ostringstream m;
      m << "hipGetSymbolAddress of the scratch array failed on device " << dev << ": "
        << (e != hipSuccess ? hipGetErrorString(e) : "null address");
      return attn::fail(ATTN_ERR_LAUNCH, fn, m.str());
    }
    if (e2 != hipSuccess) return attn::fail(ATTN_ERR_LAUNCH, fn, hipGetErrorString(e2));
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(attn_tensor_t q, attn_tensor_t k, attn_tensor_t v, attn_tensor_t o, float* lse,
             int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv, int causal, float scale,
             void* stream) {
  static const char* fn = "attn_fwd";
  try {
    attn::clear_last_error();
    int st = attn::check_attention_args(fn, attn::Op::kDense, q, k, v, &o, lse, B, Hq, Hkv, Lq,
                                        Lk, Dqk, Dv, scale);
    if (st != ATTN_OK) return st;
    attn::FwdArgs a;
    fill_fwd(a, q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, causal, scale);
    return launch_status(fn, attn::launch_fwd_dense(a, Dqk, static_cast<hipStream_t>(stream)));
  } catch (const std::exception& e) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, e.what());
  } catch (...) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, "unknown exception");
  }
}

int attn_splitkv_num_splits(int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv) {
  return attn::pick_num_splits(B, Hq, Hkv, Lq, Lk, Dqk, Dv);
}

size_t attn_splitkv_workspace_bytes(int B, int Hq, int Lq, int Dv, int num_splits) {
  return attn::workspace_bytes(B, Hq, Lq, Dv, num_splits);
}

int attn_fwd_splitkv(attn_tensor_t q, attn_tensor_t k, attn_tensor_t v, float* o_part,
                     float* lse_part, int num_splits, int B, int Hq, int Hkv, int Lq, int Lk,
                     int Dqk, int Dv, int causal, float scale, void* stream) {
  static const char* fn = "attn_fwd_splitkv";
  try {
    attn::clear_last_error();
    int st = attn::check_attention_args(fn, attn::Op::kSplit, q, k, v, nullptr, nullptr, B, Hq,
                                        Hkv, Lq, Lk, Dqk, Dv, scale);
    if (st != ATTN_OK) return st;
    if ((st = attn::check_num_splits(fn, num_splits, Lk)) != ATTN_OK) return st;
    if (o_part == nullptr || lse_part == nullptr)
      return attn::fail(ATTN_ERR_WORKSPACE, fn, "o_part / lse_part is NULL");
    if ((reinterpret_cast<uintptr_t>(o_part) & 15u) || (reinterpret_cast<uintptr_t>(lse_part) & 3u))
      return attn::fail(ATTN_ERR_WORKSPACE, fn, "o_part must be 16-byte and lse_part 4-byte aligned");
    if (attn::dense_split_shape(Dqk, Dv, Lq, Lk))
      return dense_split_launch(fn, q, k, v, o_part, lse_part, num_splits, B, Hq, Hkv, Lq, Lk,
                                Dqk, causal, scale, static_cast<hipStream_t>(stream));
    attn::SplitArgs a;
    a.q = static_cast<const uint16_t*>(q.data);
    a.k = static_cast<const uint16_t*>(k.data);
    a.v = static_cast<const uint16_t*>(v.data);
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.q_sb = q.stride_b; a.q_sl = q.stride_l; a.q_sh = q.stride_h;
    a.k_sb = k.stride_b; a.k_sl = k.stride_l; a.k_sh = k.stride_h;
    a.v_sb = v.stride_b; a.v_sl = v.stride_l; a.v_sh = v.stride_h;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk; a.g = Hq / Hkv;
    a.causal = causal ? 1 : 0;
    a.off = Lk - Lq;
    exp2_scale(scale, a.sl2, a.qsign);
    a.o = nullptr;  // the partials are this entry point's output, even for one split
    a.o_sb = a.o_sl = a.o_sh = 0;
    a.lse = nullptr;
    a.num_splits = num_splits;
    a.chunk = attn::split_chunk(Lk, num_splits);
    const int cols = attn::split_cols(Dqk, a.g * Lq);
    a.ncolblk = (a.g * Lq + cols - 1) / cols;
    return launch_status(fn, attn::launch_splitkv(a, Dqk, Dv, static_cast<hipStream_t>(stream)));
  } catch (const std::exception& e) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, e.what());
  } catch (...) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, "unknown exception");
  }
}

int attn_fwd_decode(attn_tensor_t q, attn_tensor_t k, attn_tensor_t v, attn_tensor_t o, float* lse,
                    int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv, int causal,
                    float scale, void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "attn_fwd_decode";
  try {
    attn::clear_last_error();
    int st = attn::check_attention_args(fn, attn::Op::kSplit, q, k, v, &o, lse, B, Hq, Hkv, Lq,
                                        Lk, Dqk, Dv, scale);
    if (st != ATTN_OK) return st;
    const attn::DecodeWorkspace ws = attn::decode_workspace(B, Hq, Hkv, Lq, Lk, Dqk, Dv);
    if (workspace == nullptr || workspace_bytes < ws.total ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) {
      std::ostringstream m;
      m << "workspace must be non-NULL, 256-byte aligned and at least " << ws.total << " bytes";
      return attn::fail(ATTN_ERR_WORKSPACE, fn, m.str());
    }
    return decode_launch(fn, q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, Dqk, Dv, causal, scale,
                         static_cast<char*>(workspace), ws, static_cast<hipStream_t>(stream));
  } catch (const std::exception& e) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, e.what());
  } catch (...) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, "unknown exception");
  }
}

int attn_fwd_decode_noalloc(attn_tensor_t q, attn_tensor_t k, attn_tensor_t v, attn_tensor_t o,
                            float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv,
                            int causal, float scale, void* stream) {
  static const char* fn = "attn_fwd_decode_noalloc";
  try {
    attn::clear_last_error();
    int st = attn::check_attention_args(fn, attn::Op::kSplit, q, k, v, &o, lse, B, Hq, Hkv, Lq,
                                        Lk, Dqk, Dv, scale);
    if (st != ATTN_OK) return st;
    const attn::DecodeWorkspace ws = attn::decode_workspace(B, Hq, Hkv, Lq, Lk, Dqk, Dv);
    // With one split the split kernel writes O and LSE directly and no partials exist.
    if (ws.num_splits > 1 && ws.total > (size_t)ATTN_DECODE_SCRATCH_BYTES) {
      std::ostringstream m;
      m << "these sizes need " << ws.total << " bytes of split-KV partials, more than the "
        << ATTN_DECODE_SCRATCH_BYTES << "-byte scratch array; call attn_fwd_decode with a "
        << "workspace instead";
      return attn::fail(ATTN_ERR_WORKSPACE, fn, m.str());
    }
    hipStream_t sm = static_cast<hipStream_t>(stream);
    char* wb = nullptr;
    if ((st = scratch_for_stream(fn, sm, &wb)) != ATTN_OK) return st;
    return decode_launch(fn, q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, Dqk, Dv, causal, scale, wb, ws,
                         sm);
  } catch (const std::exception& e) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, e.what());
  } catch (...) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, "unknown exception");
  }
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv) {
  return attn::decode_workspace(B, Hq, Hkv, Lq, Lk, Dqk, Dv).total;
}

int attn_combine_lse(const float* o_part, const float* lse_part, int num_splits, attn_tensor_t o,
                     float* lse, int B, int Hq, int Lq, int Dv, void* stream) {
  static const char* fn = "attn_combine_lse";
  try {
    attn::clear_last_error();
    int st = attn::check_combine_args(fn, o_part, lse_part, num_splits, o, lse, B, Hq, Lq, Dv);
    if (st != ATTN_OK) return st;
    attn::CombineArgs a;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.o = static_cast<uint16_t*>(o.data);
    a.lse = lse;
    a.o_sb = o.stride_b; a.o_sl = o.stride_l; a.o_sh = o.stride_h;
    a.B = B; a.Hq = Hq; a.Lq = Lq; a.S = num_splits;
    return launch_status(fn, attn::launch_combine(a, Dv, static_cast<hipStream_t>(stream)));
  } catch (const std::exception& e) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, e.what());
  } catch (...) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, "unknown exception");
  }
}

int attn_fwd_blocksparse(attn_tensor_t q, attn_tensor_t k, attn_tensor_t v, attn_tensor_t o,
                         float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv,
                         int causal, float scale, int block_m, int block_n,
                         const int32_t* blk_ptr, const int32_t* blk_idx, const int32_t* col_ptr,
                         const int32_t* col_idx, void* stream) {
  static const char* fn = "attn_fwd_blocksparse";
  try {
    attn::clear_last_error();
    int st = attn::check_attention_args(fn, attn::Op::kSparse, q, k, v, &o, lse, B, Hq, Hkv, Lq,
                                        Lk, Dqk, Dv, scale);
    if (st != ATTN_OK) return st;
    if (block_m != 64 || block_n != 64)
      return attn::fail(ATTN_ERR_UNSUPPORTED, fn, "block_m and block_n must be 64");
    // blk_idx / col_idx may be NULL when every list is empty: the kernel then never reads them.
    if (blk_ptr == nullptr || col_ptr == nullptr)
      return attn::fail(ATTN_ERR_INVALID_ARG, fn, "blk_ptr / col_ptr is NULL");
    attn::FwdArgs a;
    fill_fwd(a, q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, causal, scale);
    a.n_qtiles = (Lq + attn::kSparseBlockM - 1) / attn::kSparseBlockM;
    a.blk_ptr = blk_ptr;
    a.blk_idx = blk_idx;
    a.col_ptr = col_ptr;
    a.col_idx = col_idx;
    return launch_status(fn, attn::launch_fwd_blocksparse(a, Dqk, static_cast<hipStream_t>(stream)));
  } catch (const std::exception& e) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, e.what());
  } catch (...) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, "unknown exception");
  }
}

int attn_fwd_vertical_slash(attn_tensor_t q, attn_tensor_t k, attn_tensor_t v, attn_tensor_t o,
                            float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int Dqk, int Dv,
                            int causal, float scale, const int32_t* blk_ptr,
                            const int32_t* blk_idx, const int32_t* col_ptr,
                            const int32_t* col_idx, const int32_t* slash_ptr,
                            const int32_t* slash_idx, void* workspace, size_t workspace_bytes,
                            void* stream) {
  static const char* fn = "attn_fwd_vertical_slash";
  try {
    attn::clear_last_error();
    int st = attn::check_attention_args(fn, attn::Op::kSparse, q, k, v, &o, lse, B, Hq, Hkv, Lq,
                                        Lk, Dqk, Dv, scale);
    if (st != ATTN_OK) return st;
    if (blk_ptr == nullptr || col_ptr == nullptr || slash_ptr == nullptr)
      return attn::fail(ATTN_ERR_INVALID_ARG, fn, "blk_ptr / col_ptr / slash_ptr is NULL");
    if (Lk > attn::kVslashMaxLk) {
      std::ostringstream m;
      m << "Lk=" << Lk << " exceeds the vertical-slash limit of " << attn::kVslashMaxLk;
      return attn::fail(ATTN_ERR_UNSUPPORTED, fn, m.str());
    }
    const size_t need = attn_vertical_slash_workspace_bytes(B, Hq, Lk);
    if (workspace == nullptr || workspace_bytes < need ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) {
      std::ostringstream m;
      m << "workspace must be non-NULL, 256-byte aligned and at least " << need << " bytes";
      return attn::fail(ATTN_ERR_WORKSPACE, fn, m.str());
    }
    attn::FwdArgs a;
    fill_fwd(a, q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, causal, scale);
    a.n_qtiles = (Lq + attn::kSparseBlockM - 1) / attn::kSparseBlockM;
    a.blk_ptr = blk_ptr;
    a.blk_idx = blk_idx;
    a.col_ptr = col_ptr;
    a.col_idx = col_idx;
    a.sl_ptr = slash_ptr;
    a.sl_idx = slash_idx;
    a.bits_words = attn::vs_bits_words(Lk);
    uint32_t* bits = static_cast<uint32_t*>(workspace);
    a.sl_bits = bits;
    a.cl_bits = bits + (size_t)B * Hq * a.bits_words;
    a.rl_bits = bits + 2 * (size_t)B * Hq * a.bits_words;
    return launch_status(fn, attn::launch_fwd_vslash(a, Dqk, static_cast<hipStream_t>(stream)));
  } catch (const std::exception& e) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, e.what());
  } catch (...) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, "unknown exception");
  }
}

size_t attn_vertical_slash_workspace_bytes(int B, int Hq, int Lk) {
  if (B < 1 || Hq < 1 || Lk < 1) return 0;
  return attn::kVslashBitmaps * (size_t)B * Hq * attn::vs_bits_words(Lk) * sizeof(uint32_t);
}

int attn_vertical_slash_check(const int32_t* slash_ptr, const int32_t* slash_idx, int B, int Hq,
                              int Lk) {
  attn::clear_last_error();
  return attn::check_slash_lists("attn_vertical_slash_check", slash_ptr, slash_idx, B, Hq, Lk);
}

int attn_blocksparse_check(const int32_t* blk_ptr, const int32_t* blk_idx, const int32_t* col_ptr,
                           const int32_t* col_idx, int B, int Hq, int Lq, int Lk, int block_m,
                           int block_n) {
  attn::clear_last_error();
  return attn::check_blocksparse_lists("attn_blocksparse_check", blk_ptr, blk_idx, col_ptr,
                                       col_idx, B, Hq, Lq, Lk, block_m, block_n);
}

int attn_build_sparse_index(attn_tensor_t q, attn_tensor_t k, int B, int Hq, int Hkv, int L, int D,
                            float scale, int topk_blocks, int n_cols, int32_t* blk_ptr,
                            int32_t* blk_idx, int32_t* col_ptr, int32_t* col_idx, void* workspace,
                            size_t workspace_bytes, void* stream) {
  static const char* fn = "attn_build_sparse_index";
  try {
    attn::clear_last_error();
    int st = attn::check_index_args(fn, q, k, B, Hq, Hkv, L, D, scale, topk_blocks, n_cols,
                                    blk_ptr, blk_idx, col_ptr, col_idx, workspace,
                                    workspace_bytes);
    if (st != ATTN_OK) return st;
    const attn::IndexWorkspace ws = attn::index_workspace(B, Hq, Hkv, L, D);
    char* wb = static_cast<char*>(workspace);
    attn::IndexArgs a{};
    a.q = static_cast<const uint16_t*>(q.data);
    a.k = static_cast<const uint16_t*>(k.data);
    a.q_sb = q.stride_b; a.q_sl = q.stride_l; a.q_sh = q.stride_h;
    a.k_sb = k.stride_b; a.k_sl = k.stride_l; a.k_sh = k.stride_h;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.L = L;
    a.scale = scale;
    a.sl2 = scale * kLog2e;
    a.topk = topk_blocks;
    a.ncols = n_cols;
    a.blk_ptr = blk_ptr; a.blk_idx = blk_idx; a.col_ptr = col_ptr; a.col_idx = col_idx;
    a.blk_head_len = attn::index_blk_head_len(L, topk_blocks);
    a.blk_total = (int64_t)B * Hq * a.blk_head_len;
    a.qbar = reinterpret_cast<float*>(wb + ws.qbar);
    a.kbar = reinterpret_cast<float*>(wb + ws.kbar);
    a.stats = reinterpret_cast<float*>(wb + ws.stats);
    a.fin = reinterpret_cast<float*>(wb + ws.fin);
    a.imp = reinterpret_cast<float*>(wb + ws.imp);
    a.simp = reinterpret_cast<float*>(wb + ws.simp);
    return launch_status(fn, attn::launch_build_index(a, D, static_cast<hipStream_t>(stream)));
  } catch (const std::exception& e) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, e.what());
  } catch (...) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, "unknown exception");
  }
}

int attn_build_vslash_index(attn_tensor_t q, attn_tensor_t k, int B, int Hq, int Hkv, int L, int D,
                            float scale, int n_cols, int n_slash, int32_t* col_ptr,
                            int32_t* col_idx, int32_t* slash_ptr, int32_t* slash_idx,
                            void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "attn_build_vslash_index";
  try {
    attn::clear_last_error();
    int st = attn::check_vslash_index_args(fn, q, k, B, Hq, Hkv, L, D, scale, n_cols, n_slash,
                                           col_ptr, col_idx, slash_ptr, slash_idx, workspace,
                                           workspace_bytes);
    if (st != ATTN_OK) return st;
    const attn::IndexWorkspace ws = attn::index_workspace(B, Hq, Hkv, L, D);
    char* wb = static_cast<char*>(workspace);
    attn::IndexArgs a{};
    a.q = static_cast<const uint16_t*>(q.data);
    a.k = static_cast<const uint16_t*>(k.data);
    a.q_sb = q.stride_b; a.q_sl = q.stride_l; a.q_sh = q.stride_h;
    a.k_sb = k.stride_b; a.k_sl = k.stride_l; a.k_sh = k.stride_h;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.L = L;
    a.scale = scale;
    a.sl2 = scale * kLog2e;
    a.ncols = n_cols;
    a.nslash = n_slash;
    a.col_ptr = col_ptr; a.col_idx = col_idx;
    a.sl_ptr = slash_ptr; a.sl_idx = slash_idx;
    a.stats = reinterpret_cast<float*>(wb + ws.stats);
    a.fin = reinterpret_cast<float*>(wb + ws.fin);
    a.imp = reinterpret_cast<float*>(wb + ws.imp);
    a.simp = reinterpret_cast<float*>(wb + ws.simp);
    return launch_status(fn, attn::launch_build_vslash_index(a, D,
                                                             static_cast<hipStream_t>(stream)));
  } catch (const std::exception& e) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, e.what());
  } catch (...) {
    return attn::fail(ATTN_ERR_LAUNCH, fn, "unknown exception");
  }
}

int attn_sparse_index_sizes(int B, int Hq, int L, int topk_blocks, int n_cols, int64_t* n_blk_idx,
                            int64_t* n_col_idx) {
  attn::clear_last_error();
  if (B < 1 || Hq < 1 || L < 1 || topk_blocks < 1 || n_cols < 0)
    return attn::fail(ATTN_ERR_INVALID_ARG, "attn_sparse_index_sizes", "invalid sizes");
  if (n_blk_idx != nullptr) *n_blk_idx = (int64_t)B * Hq * attn::index_blk_head_len(L, topk_blocks);
  if (n_col_idx != nullptr) *n_col_idx = (int64_t)B * Hq * (n_cols < L ? n_cols : L);
  return ATTN_OK;
}

size_t attn_sparse_index_workspace_bytes(int B, int Hq, int Hkv, int L, int D) {
  return attn::index_workspace(B, Hq, Hkv, L, D).total;
}

const char* attn_status_string(int status) { return attn::status_string(status); }

const char* attn_last_error(void) { return attn::last_error_cstr(); }

}  // extern "C"
