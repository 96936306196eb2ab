// cache_write.hip - gfx950 kernel behind pa_cache_write.
//
// Page cited: [RK] "什么是 LLM 中的分页注意力(Paged Attention)?它是如何工作的?"
// news.rkmt.cn, section 分页注意力是如何工作的: each new token's key and value go
// into the next free slot of the sequence's current block.  The slot id
// (phys * bs + offset) is chosen by the caller; this kernel only moves bytes.
//
// One wave per (token, KV head).  The key row is D contiguous elements in the
// cache, copied with 16-byte stores; the value is scattered down one column of the
// dimension-major value tile (stride bs).  A pure bit copy for every dtype, so
// only the element size matters.
#include "kernels.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define AS4 __attribute__((address_space(4)))

template <typename E>
__global__ __launch_bounds__(64) void cache_write_kernel(CacheWriteParams P) {
  const int64_t item = blockIdx.x;  // token * Hkv + head
  const int Hkv = P.num_kv_heads, D = P.head_dim, BS = P.block_size;
  const int64_t i = item / Hkv;
  const int g = (int)(item - i * Hkv);
  const int64_t slot = ((const int64_t AS4*)P.slot_mapping)[i];
  if (slot < 0 || slot >= P.num_slots) return;  // skipped token (or out of the pool)
  const int64_t b = slot / BS;
  const int o = (int)(slot - b * BS);
  const int lane = threadIdx.x;

  const E* ksrc = (const E*)P.k + item * D;
  const E* vsrc = (const E*)P.v + item * D;
  E* kdst = (E*)P.k_cache + ((b * Hkv + g) * BS + o) * (int64_t)D;
  E* vdst = (E*)P.v_cache + ((b * Hkv + g) * (int64_t)D) * BS + o;

  const int nvec = D * (int)sizeof(E) / 16;
  for (int v = lane; v < nvec; v += 64)
    reinterpret_cast<u32x4*>(kdst)[v] = reinterpret_cast<const u32x4*>(ksrc)[v];
  for (int d = lane; d < D; d += 64) vdst[(int64_t)d * BS] = vsrc[d];
}

}  // namespace

hipError_t launch_cache_write(int elem_bytes, const CacheWriteParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.num_tokens * p.num_kv_heads));
  CacheWriteParams arg = p;
  void* args[] = {&arg};
  if (elem_bytes == 2)
    return hipLaunchKernel((const void*)cache_write_kernel<uint16_t>, grid, dim3(64), args, 0,
                           stream);
  if (elem_bytes == 4)
    return hipLaunchKernel((const void*)cache_write_kernel<uint32_t>, grid, dim3(64), args, 0,
                           stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
