// Read-rate probe: the ceilings that the copy phases of the attention kernels are compared
// with. They are measuring tools, built into their own library (libattn_probes.so) and used by
// the benchmark only; no attention entry point calls them.
//
// probe_read_tiles: every workgroup reads whole tiles (a contiguous run of bytes, e.g. the
// 32 KiB of one 64-key K/V tile pair) at caller-given tile indices, one tile after another, each
// lane with eight 16-byte loads in flight. With the indices in order this streams a buffer;
// with random indices it is the pattern of the listed far blocks of the block-sparse kernel.
// Over a region much larger than every cache the rate is HBM's; over a region larger than the
// eight L2s together (8 x 4 MiB) but well inside the 256 MiB Infinity Cache, launches after the
// first measure the Infinity Cache.
//
// probe_read_rows: every workgroup reads strided rows of one or two buffers, as one split-KV
// workgroup reads its keys' K and V rows; the decode kernels' step time is compared with it.
// The _nt entry points make the same reads with the non-temporal cache policy.
//
// probe_mfma_stream: back-to-back bf16 MFMAs on random operands, the rate the matrix cores
// sustain at the power limit (the prefill kernels' compute ceiling in practice).
//
// Each lane folds what it reads into one word and writes it only if it equals a value no input
// produces in practice, so the loads cannot be dropped and the probe writes (almost) nothing.

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr uint32_t kNever = 0x9e3779b9u;


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // a register-operand type for asm
__device__ inline uint32_t fold(u32x4 v) { return v.x ^ (v.y * 3u) ^ (v.z * 5u) ^ (v.w * 7u); }

// A 16-byte load with the default cache policy, or (NT) the non-temporal one, which the
// decode kernel's copies use.
template <bool NT>
__device__ inline u32x4 load16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Tiles of tile16 16-byte chunks; workgroup g reads tiles ids[g * per_wg + t], t < per_wg.
template <bool NT>
__global__ __launch_bounds__(kThreads) void read_tiles_kernel(const u32x4* __restrict__ buf,
                                                              const int32_t* __restrict__ ids,
                                                              int per_wg, int tile16,
                                                              uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int32_t* my = ids + (size_t)blockIdx.x * per_wg;
  for (int t = 0; t < per_wg; ++t) {
    const u32x4* tile = buf + (size_t)my[t] * tile16;
    int j = threadIdx.x;
    for (; j + (kUnroll - 1) * kThreads < tile16; j += kUnroll * kThreads) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = load16<NT>(tile + j + u * kThreads);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc += fold(v[u]);
    }
    for (; j < tile16; j += kThreads) acc += fold(load16<NT>(tile + j));
  }
  if (acc == kNever) sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// Rows of row16 16-byte chunks at a byte stride: workgroup g reads rows [0, nrows) from byte
// base[g] of `a`, and of `b` unless it is null, 64 rows at a time (the tile's chunks of `a`, then
// those of `b`). The chunks are numbered in that order and dealt out over the lanes, kRowsUnroll
// loads in flight per lane (a split-KV workgroup keeps up to four 36 KiB tiles in flight, so
// eight per lane, 32 KiB per workgroup, would understate what one workgroup per CU can read).
// The index is clamped rather than the load made conditional, so the loads stay independent.
constexpr int kRowsUnroll = 32;

template <bool NT>
__global__ __launch_bounds__(kThreads) void read_rows_kernel(const char* __restrict__ a,
                                                             const char* __restrict__ b,
                                                             const int64_t* __restrict__ base,
                                                             int nrows, int row16, int64_t stride,
                                                             uint32_t* __restrict__ sink) {
  const int64_t b0 = base[blockIdx.x];
  const int per_t = 64 * row16;                 // chunks of one buffer in a 64-row tile
  const int per_tile = b ? 2 * per_t : per_t;
  const int n = (nrows / 64) * per_tile;
  uint32_t acc = 0;
  for (int j0 = 0; j0 < n; j0 += kRowsUnroll * kThreads) {
    u32x4 v[kRowsUnroll];
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u) {
      const int j = min(j0 + u * kThreads + (int)threadIdx.x, n - 1);
      const int t = j / per_tile;
      const int rem = j - t * per_tile;
      const bool second = rem >= per_t;
      const int jj = second ? rem - per_t : rem;
      const int r = jj / row16, c = jj - r * row16;
      const char* src = second ? b : a;
      v[u] = load16<NT>(reinterpret_cast<const u32x4*>(src + b0 + (int64_t)(t * 64 + r) * stride +
                                                       (int64_t)c * 16));
    }
    // Every load of the batch is issued before the first fold waits for one: the empty asm
    // statements take the loaded registers as operands after a scheduling barrier, so the folds
    // (which the compiler would otherwise interleave with the loads) cannot move above them.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kRowsUnroll; u += 4)
      asm volatile("" : "+v"(v[u]), "+v"(v[u + 1]), "+v"(v[u + 2]), "+v"(v[u + 3]));
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u) acc += fold(v[u]);
  }
  if (acc == kNever) sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// MFMA stream: every wave runs `iters` rounds of 32x32x16 bf16 MFMAs, eight operand pairs
// (loaded once from `in`) against four independent accumulator chains, so nothing but the
// matrix core bounds the issue rate. The operands are the caller's random bits: on this part
// the MFMA rate follows the clock, and the clock follows the power the operand data draws
// (zero operands run faster than any real input).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kMfmaThreads = 512;
constexpr int kMfmaPairs = 8;
constexpr int kMfmaChains = 4;

__global__ __launch_bounds__(kMfmaThreads) void mfma_stream_kernel(const u32x4* __restrict__ in,
                                                                   int iters,
                                                                   uint32_t* __restrict__ sink) {
  const int l = threadIdx.x & 63;
  bf16x8_t a[kMfmaPairs], b[kMfmaPairs];
#pragma unroll
  for (int j = 0; j < kMfmaPairs; ++j) {
    a[j] = __builtin_bit_cast(bf16x8_t, in[(2 * j) * 64 + l]);
    b[j] = __builtin_bit_cast(bf16x8_t, in[(2 * j + 1) * 64 + l]);
  }
  f32x16_t acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x16_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaPairs; ++j)
#pragma unroll
      for (int c = 0; c < kMfmaChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc[c], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) r += acc[c][l & 15];
  if (__builtin_bit_cast(uint32_t, r) == kNever)
    sink[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = kNever;
}

}  // namespace

extern "C" {

// Reads grid * per_wg tiles of `tile_bytes` bytes (a multiple of 16) from `buf`: workgroup g
// reads the tiles whose indices are ids[g * per_wg .. (g + 1) * per_wg), each index naming the
// tile that starts at byte index * tile_bytes. The caller keeps every tile inside the buffer.
// `sink` is device memory of grid * 256 words that the kernel may write. Returns a hipError_t
// value (0 on success).
int probe_read_tiles(const void* buf, const int32_t* ids, int per_wg, int grid, int tile_bytes,
                     uint32_t* sink, void* stream) {
  if (!buf || !ids || !sink || grid <= 0 || per_wg <= 0 || tile_bytes <= 0 || tile_bytes % 16)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_tiles_kernel<false>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)buf, ids, per_wg, tile_bytes / 16, sink);
  return (int)hipGetLastError();
}

// probe_read_tiles with non-temporal loads.
int probe_read_tiles_nt(const void* buf, const int32_t* ids, int per_wg, int grid, int tile_bytes,
                        uint32_t* sink, void* stream) {
  if (!buf || !ids || !sink || grid <= 0 || per_wg <= 0 || tile_bytes <= 0 || tile_bytes % 16)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_tiles_kernel<true>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)buf, ids, per_wg, tile_bytes / 16, sink);
  return (int)hipGetLastError();
}

// Reads, in each of `grid` workgroups g, the rows r < nrows (a multiple of 64) of `row_bytes`
// bytes (a multiple of 16) that start at byte base[g] + r * stride of `a`, and of `b` at the same
// offsets unless `b` is null: the access pattern of one split-KV workgroup over a [B, L, H, D]
// cache. `base` is
// device memory of `grid` byte offsets; the caller keeps every row inside both buffers. `sink`
// is device memory of grid * 256 words that the kernel may write. Returns a hipError_t value
// (0 on success).
int probe_read_rows(const void* a, const void* b, const int64_t* base, int grid, int nrows,
                    int row_bytes, int64_t stride, uint32_t* sink, void* stream) {
  if (!a || !base || !sink || grid <= 0 || nrows <= 0 || nrows % 64 || row_bytes <= 0 ||
      row_bytes % 16 || stride < row_bytes)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_rows_kernel<false>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const char*)a, (const char*)b, base, nrows, row_bytes / 16, stride, sink);
  return (int)hipGetLastError();
}

// probe_read_rows with non-temporal loads (the cache policy of the decode kernel's copies).
int probe_read_rows_nt(const void* a, const void* b, const int64_t* base, int grid, int nrows,
                       int row_bytes, int64_t stride, uint32_t* sink, void* stream) {
  if (!a || !base || !sink || grid <= 0 || nrows <= 0 || nrows % 64 || row_bytes <= 0 ||
      row_bytes % 16 || stride < row_bytes)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_rows_kernel<true>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const char*)a, (const char*)b, base, nrows, row_bytes / 16, stride, sink);
  return (int)hipGetLastError();
}

// Runs `grid` workgroups of 512 lanes (8 waves), each wave doing iters * 32 MFMAs of
// 32x32x16 bf16 (32768 flops each) on operands read from `in`: device memory of 16 * 64
// 16-byte words (random bf16 bits). `sink` is device memory of grid * 512 words that the kernel
// may write. Flops per launch: grid * 8 * iters * 32 * 32768. Returns a hipError_t value.
int probe_mfma_stream(const void* in, int grid, int iters, uint32_t* sink, void* stream) {
  if (!in || !sink || grid <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_stream_kernel, dim3(grid), dim3(kMfmaThreads), 0, (hipStream_t)stream,
                     (const u32x4*)in, iters, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
