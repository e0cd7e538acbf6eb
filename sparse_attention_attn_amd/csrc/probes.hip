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
// Each lane folds what it reads into one word and writes it only if it equals a value no input
// produces in practice, so the loads cannot be dropped and the probe writes (almost) nothing.

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr uint32_t kNever = 0x9e3779b9u;

__device__ inline uint32_t fold(uint4 v) { return v.x ^ (v.y * 3u) ^ (v.z * 5u) ^ (v.w * 7u); }

// Tiles of tile16 16-byte chunks; workgroup g reads tiles ids[g * per_wg + t], t < per_wg.
__global__ __launch_bounds__(kThreads) void read_tiles_kernel(const uint4* __restrict__ buf,
                                                              const int32_t* __restrict__ ids,
                                                              int per_wg, int tile16,
                                                              uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int32_t* my = ids + (size_t)blockIdx.x * per_wg;
  for (int t = 0; t < per_wg; ++t) {
    const uint4* tile = buf + (size_t)my[t] * tile16;
    int j = threadIdx.x;
    for (; j + (kUnroll - 1) * kThreads < tile16; j += kUnroll * kThreads) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = tile[j + u * kThreads];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc += fold(v[u]);
    }
    for (; j < tile16; j += kThreads) acc += fold(tile[j]);
  }
  if (acc == kNever) sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
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
  hipLaunchKernelGGL(read_tiles_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint4*)buf, ids, per_wg, tile_bytes / 16, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
