// kernels.h - what the C-ABI layer needs from the gfx950 kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWavesPerGroup = 4;   // waves sharing one work item
constexpr int kScanMax = 1024;      // sequences one decode launch plans for (host slices above)
constexpr int kMergeFan = 16;       // partials combined per merge node
constexpr int kMaxPartitions = 8192;
constexpr int kSizeClasses = 17;    // classes the last partitions are ordered by
constexpr float kPartShare = 1.0f;  // default partition: this fraction of a workgroup's share
constexpr float kTailShare = 0.75f;  // ... when at that length no sequence would be split
constexpr size_t kStaticScratchBytes = size_t(64) << 20;  // pa_decode_noalloc's device scratch
constexpr int kPartSlot = 16;       // int32 slot of the decode workspace header (byte 64) that
                                    // records the partition length the last launch used

// Everything a decode launch needs; passed by value as the kernel argument.  The
// launch covers num_seqs sequences starting at the pointers given (the host slices
// larger batches); counters and partial buffers are indexed by the slice's own
// sequence numbers.
struct DecodeParams {
  const void* q;                // [S][Hq][D]
  const void* k_cache;          // [N][Hkv][bs][D]
  const void* v_cache;          // [N][Hkv][D][bs]
  const int32_t* block_tables;  // [S][max_blocks]
  const int32_t* seq_lens;      // [S]
  void* out;                    // [S][Hq][D]
  float* part_o;                // [S][pmax][Hq][D]   per-partition unnormalised outputs
  float* part_ml;               // [S][pmax][Hq][2]   (running max in log2 units, sum)
  float* node_o;                // [S][nodes][Hq][D]  merged groups of kMergeFan partitions
  float* node_ml;               // [S][nodes][Hq][2]
  int32_t* queue;               // [2]: next work item, finished workgroups (0 between calls);
                                // [kPartSlot]: the partition length the launch used
  int32_t* node_count;          // [S][Hkv*tiles][nodes]: partitions finished per group
  int32_t* root_count;          // [S][Hkv*tiles]: groups finished per sequence and head tile
  int64_t num_blocks;           // N
  int32_t num_seqs;             // S of this launch (<= kScanMax)
  int32_t num_q_heads;          // Hq
  int32_t num_kv_heads;         // Hkv
  int32_t group;                // Hq / Hkv
  int32_t head_tiles;           // ceil(group / 16)
  int32_t max_blocks;           // row stride of block_tables
  int32_t max_tokens;           // max_blocks * bs
  int32_t part_tokens;          // tokens per partition, a multiple of 32
  int32_t auto_part;            // 1: default size; the kernel may lengthen part_tokens
  int32_t stream_kv;            // 1: no table shares a block: K/V loads are non-temporal
  int32_t pmax;                 // ceil(max_tokens / part_tokens)
  int32_t nodes;                // ceil(pmax / kMergeFan)
  float scale_log2;             // scale * log2(e): logits are kept in base-2 units
  // fused cache write (pa_cache_write_decode), else slot_mapping is null
  const void* k_new;            // [S][Hkv][D]: sequence s's new token, at position seq_lens[s]-1
  const void* v_new;            // [S][Hkv][D]
  const int64_t* slot_mapping;  // [S]: the new tokens' slots (< 0 or >= num_slots: none)
  int64_t num_slots;            // N * bs
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

// A pa_multi_token launch: rows are (new token, query head) pairs of one KV head.
struct MultiTokenParams {
  const void* q;                // [T][Hq][D]
  const void* k_cache;          // [N][Hkv][bs][D]
  const void* v_cache;          // [N][Hkv][D][bs]
  const int32_t* block_tables;  // [S][max_blocks]
  const int32_t* seq_lens;      // [S]: cached tokens, the new ones included
  const int32_t* query_start;   // [S+1]: sequence s's new tokens are q rows qs[s] .. qs[s+1]-1
  void* out;                    // [T][Hq][D]
  int64_t num_blocks;           // N
  int32_t num_seqs;             // S
  int32_t num_tokens;           // T
  int32_t num_q_heads;          // Hq
  int32_t num_kv_heads;         // Hkv
  int32_t group;                // Hq / Hkv
  int32_t max_blocks;           // row stride of block_tables
  int32_t max_tokens;           // max_blocks * bs
  int32_t row_tiles;            // workgroup row tiles per (sequence, KV head)
  int32_t parts;                // context partitions per (sequence, KV head); 1: no split
  int32_t part_tokens;          // tokens per partition, a multiple of 32
  int32_t part_rows;            // rows stored per (row tile, partition): min(128, rows)
  float* part_o;                // [S][Hkv][row_tiles][parts][part_rows][D] unnormalised outputs
  float* part_ml;               // [S][Hkv][row_tiles][parts][part_rows][2] (max in log2 units, sum)
  float scale_log2;             // scale * log2(e)
};

constexpr int kCopyBatch = 128;  // block copies per launch (their ids travel as arguments)

struct CopyBlocksParams {
  char* k_cache;
  char* v_cache;
  int64_t block_bytes;  // Hkv * bs * D * element size: one physical block of one cache
  int32_t n;            // pairs in this launch
  int32_t pairs[2 * kCopyBatch];  // (src, dst) block ids
};

// dtype codes follow pa_dtype: 0 f32, 1 f16, 2 bf16.
// Each returns hipErrorInvalidValue for a (dtype, head_dim, block_size) that has
// no compiled instance; the caller checks support first.
hipError_t launch_decode(int dtype, int head_dim, int block_size, const DecodeParams& p,
                         int grid, hipStream_t stream);
// Workgroups of the decode kernel that fit on one compute unit at once.
hipError_t decode_blocks_per_cu(int dtype, int head_dim, int block_size, int* blocks);
hipError_t launch_cache_write(int elem_bytes, const CacheWriteParams& p, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t stream);
// (new token, query head) rows one multi-token workgroup covers
int multi_token_rows_per_group();
hipError_t launch_multi_token(int dtype, int head_dim, int block_size, MultiTokenParams p,
                              hipStream_t stream);
// The log-sum-exp combination of a split launch's partitions into out.
hipError_t launch_multi_token_merge(int dtype, int head_dim, const MultiTokenParams& p,
                                    hipStream_t stream);

// pa_decode_noalloc: the device address of this device's static scratch array
// (kStaticScratchBytes, 256-byte aligned), looked up once per device.
hipError_t static_scratch(void** ptr);
// Zero bytes (a multiple of 16) at p, 16-byte aligned, on stream.
hipError_t launch_clear(void* p, size_t bytes, hipStream_t stream);

}  // namespace pa
