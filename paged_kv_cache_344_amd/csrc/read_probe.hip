// read_probe.hip - gfx950 kernel behind pa_read_probe: the HBM read rate that a kernel
// doing nothing but read reaches, as a reference for the attention kernels' own rates.
//
// A paged pool is read in tiles: at head size 128 and 2-byte elements one block of 16
// tokens of one KV head is 4 KiB of K and 4 KiB of V, each contiguous, at a position
// the block table gives ([RK] "什么是 LLM 中的分页注意力(Paged Attention)?它是如何工作的?",
// section 分页注意力是如何工作的).
// The probe reads 4 KiB tiles the same way: 256 threads a workgroup, one 16-byte
// non-temporal load each per tile (the cache policy the decode kernel uses on pools
// whose blocks no table shares), eight tiles in flight per workgroup, eight workgroups
// per compute unit.  Tiles come in order (a stream) or from an index list (a shuffled
// pool).  Every loaded word is folded (XOR) into one word per wave and stored, so no
// load can be dropped.
#include "read_probe.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_probe_kernel(const char* __restrict__ src,
                                                         int64_t tiles_in_src,
                                                         const int32_t* __restrict__ tiles,
                                                         int64_t n, uint32_t* __restrict__ sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t step = (int64_t)gridDim.x * kProbeTilesInFlight;
  for (int64_t i0 = (int64_t)blockIdx.x * kProbeTilesInFlight; i0 < n; i0 += step) {
    // this step's tile ids first (one round trip for all of them), then the loads
    int64_t tid8[kProbeTilesInFlight];
    if (i0 + kProbeTilesInFlight <= n && tiles) {  // a full step: unguarded, back to back
#pragma unroll
      for (int u = 0; u < kProbeTilesInFlight; ++u) tid8[u] = tiles[i0 + u];
    } else {
#pragma unroll
      for (int u = 0; u < kProbeTilesInFlight; ++u) {
        const int64_t i = i0 + u;
        tid8[u] = i < n ? (tiles ? (int64_t)tiles[i] : i) : -1;
      }
    }
    u32x4 v[kProbeTilesInFlight];
#pragma unroll
    for (int u = 0; u < kProbeTilesInFlight; ++u) {
      const int64_t t = tid8[u];
      // an index outside the buffer is skipped, never read
      v[u] = (t >= 0 && t < tiles_in_src)
                 ? __builtin_nontemporal_load(
                       reinterpret_cast<const u32x4*>(src + t * kProbeTile) + threadIdx.x)
                 : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kProbeTilesInFlight; ++u) acc ^= v[u];
  }
  uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) r ^= __shfl_xor(r, o);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * kProbeWaves + (threadIdx.x >> 6)] = r;
}

}  // namespace

hipError_t launch_read_probe(const char* src, int64_t tiles_in_src, const int32_t* tiles,
                             int64_t n_tiles, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink || tiles_in_src < 0 || n_tiles < 0) return hipErrorInvalidValue;
  if (n_tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)kProbeGrid), block(64 * kProbeWaves);
  hipLaunchKernelGGL(read_probe_kernel, grid, block, 0, stream, src, tiles_in_src, tiles, n_tiles,
                     sink);
  return hipGetLastError();
}

}  // namespace pa
