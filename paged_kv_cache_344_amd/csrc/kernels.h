// kernels.h - what the C-ABI layer needs from the gfx950 kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Everything a decode launch needs; passed by value as the kernel argument.
struct DecodeParams {
  const void* q;                // [S][Hq][D]
  const void* k_cache;          // [N][Hkv][bs][D]
  const void* v_cache;          // [N][Hkv][D][bs]
  const int32_t* block_tables;  // [S][max_blocks]
  const int32_t* seq_lens;      // [S]
  void* out;                    // [S][Hq][D]
  float* ws_o;                  // [S][Hq][pmax][D]  unnormalised partition outputs
  float* ws_ml;                 // [S][Hq][pmax][2]  (running max in log2 units, sum)
  int64_t num_blocks;           // N
  int32_t num_seqs;             // S
  int32_t num_q_heads;          // Hq
  int32_t num_kv_heads;         // Hkv
  int32_t group;                // Hq / Hkv
  int32_t head_tiles;           // ceil(group / 16)
  int32_t max_blocks;           // row stride of block_tables
  int32_t max_tokens;           // max_blocks * bs
  int32_t part_tokens;          // tokens per partition, a multiple of 32
  int32_t pmax;                 // ceil(max_tokens / part_tokens)
  float scale_log2;             // scale * log2(e): logits are kept in base-2 units
};

struct CacheWriteParams {
  const void* k;                // [T][Hkv][D]
  const void* v;                // [T][Hkv][D]
  const int64_t* slot_mapping;  // [T]
  void* k_cache;                // [N][Hkv][bs][D]
  void* v_cache;                // [N][Hkv][D][bs]
  int64_t num_slots;            // N * bs
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
};

// dtype codes follow pa_dtype: 0 f32, 1 f16, 2 bf16.
// Each returns hipErrorInvalidValue for a (dtype, head_dim, block_size) that has
// no compiled instance; the caller checks support first.
hipError_t launch_decode_partitions(int dtype, int head_dim, int block_size,
                                    const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_merge(int dtype, int head_dim, const DecodeParams& p,
                               hipStream_t stream);
hipError_t launch_cache_write(int elem_bytes, const CacheWriteParams& p, hipStream_t stream);

constexpr int kMaxPartitions = 8192;  // merge kernel keeps one weight per partition in LDS
constexpr int kWavesPerGroup = 4;     // waves sharing one (sequence, KV head, partition)

}  // namespace pa
