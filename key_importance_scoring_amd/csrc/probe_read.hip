// Streaming-read probe: the HBM read rate that a persistent grid reaches when it
// streams contiguous tiles, the access shape of the score kernel (workgroups of 256
// threads, a static tile schedule, 16-byte loads with eight in flight per thread).
// It is a measuring instrument, not part of the pruning pass: the pass's kernels are
// rated against its rate as well as against the published HBM peak.
//
// Built into its own library (libtria_probe.so) with the same flags as libtria.so.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kInFlight = 8;          // 16-byte loads issued before any is used
constexpr uint32_t kNever = 0x9E3779B9u;

// Workgroup w reads tiles w, w + grid, ... of tile_vec 16-byte vectors each (the last
// tile may be short).  The XOR of everything a thread read is stored only if it
// equals kNever: the loads stay live, and the run writes nothing in practice.
__global__ __launch_bounds__(kThreads) void k_read_probe(const u32x4* __restrict__ src, int64_t n_vec,
                                                         int64_t tile_vec, uint32_t* __restrict__ sink) {
  const int64_t n_tiles = (n_vec + tile_vec - 1) / tile_vec;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
    const int64_t end = t * tile_vec + tile_vec < n_vec ? t * tile_vec + tile_vec : n_vec;
    int64_t i = t * tile_vec + threadIdx.x;
    for (; i + (kInFlight - 1) * kThreads < end; i += kInFlight * kThreads) {
      u32x4 v[kInFlight];
#pragma unroll
      for (int k = 0; k < kInFlight; ++k) v[k] = src[i + k * kThreads];
#pragma unroll
      for (int k = 0; k < kInFlight; ++k) acc ^= v[k];
    }
    for (; i < end; i += kThreads) acc ^= src[i];
  }
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == kNever) sink[blockIdx.x] = x;
}

}  // namespace

// Reads `bytes` bytes at `src` (device memory, 16-byte aligned, bytes a multiple of
// 16) once with `grid` workgroups, in tiles of `tile_bytes` (a multiple of 16).
// `sink` is device memory of at least `grid` 32-bit words that the kernel may write.
// Launch only; asynchronous on `stream`.  Returns 0, -1 for invalid arguments, or
// the hipError_t of the launch.
extern "C" int tria_probe_read(const void* src, int64_t bytes, int64_t tile_bytes, int grid, uint32_t* sink,
                               void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 || tile_bytes <= 0 || tile_bytes % 16 || grid <= 0 ||
      reinterpret_cast<uintptr_t>(src) % 16)
    return -1;
  hipLaunchKernelGGL(k_read_probe, dim3((unsigned)grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, tile_bytes / 16, sink);
  return (int)hipGetLastError();
}
