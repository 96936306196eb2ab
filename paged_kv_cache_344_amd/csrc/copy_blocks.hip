// copy_blocks.hip - gfx950 kernel behind pa_copy_blocks.
//
// Pages cited: [CY] "深入解析 PagedAttention：vLLM 显存优化的核心魔法" cygnushan.xyz,
// section 多序列共享 (copy-on-write of shared blocks); [ASP] "PagedAttention"
// awesome-system-papers, section 实现要点.
//
// A block of one cache is Hkv * bs * D contiguous elements ([N][Hkv][bs][D] and
// [N][Hkv][D][bs] both keep a block contiguous), so a block copy is a plain copy of
// block_bytes bytes.  One 256-thread workgroup moves 4 KiB (16 bytes a thread) of
// one block of one cache; grid = (4 KiB pieces of a block, 2 caches, pairs).
#include "kernels.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kPiece = 4096;

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksParams P) {
  const int pair = blockIdx.z;
  const int64_t src = P.pairs[2 * pair], dst = P.pairs[2 * pair + 1];
  char* base = blockIdx.y == 0 ? P.k_cache : P.v_cache;
  const int64_t off = (int64_t)blockIdx.x * kPiece + threadIdx.x * 16;
  if (off >= P.block_bytes) return;  // the last piece of a block may be partial
  const u32x4 v = *reinterpret_cast<const u32x4*>(base + src * P.block_bytes + off);
  *reinterpret_cast<u32x4*>(base + dst * P.block_bytes + off) = v;
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t stream) {
  if (p.n <= 0 || p.n > kCopyBatch || p.block_bytes <= 0 || p.block_bytes % 16)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((p.block_bytes + kPiece - 1) / kPiece), 2, (unsigned)p.n);
  CopyBlocksParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel((const void*)copy_blocks_kernel, grid, dim3(256), args, 0, stream);
}

}  // namespace pa
