// pa_api.cpp - the C ABI of libpa.so: argument checks, launch planning, dispatch.
//
// Every host-side argument is checked before the first HIP call, so a bad call
// returns a status without touching the GPU (and can be tested on a machine with
// none).  The library owns no device memory: the split-K workspace is the
// caller's, sized by pa_decode_workspace_bytes.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>
#include <string>

#include "kernels.h"
#include "pa.h"

namespace {

thread_local std::string g_error;

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  try {
    g_error = buf;
  } catch (...) {
  }
  return st;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool block_size_built(int bs) { return bs == 4 || bs == 8 || bs == 16 || bs == 32; }
bool dtype_valid(int dt) { return dt == PA_F32 || dt == PA_F16 || dt == PA_BF16; }

constexpr int kDefaultPartition = 512;
constexpr size_t kAlign = 256;
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
  int32_t part_tokens;
  int32_t pmax;
  int32_t head_tiles;
  int32_t max_tokens;
  size_t ws_o_bytes;  // 0 when no split is possible
  size_t ws_bytes;
};

pa_status plan_decode(const pa_decode_ext* ext, int32_t bs, int32_t hkv, Plan* pl) {
  if (!ext) return fail(PA_ERR_INVALID_ARG, "ext is NULL");
  const int32_t S = ext->num_seqs, Hq = ext->num_q_heads, D = ext->head_dim;
  const int32_t MB = ext->max_blocks_per_seq;
  if (S < 0 || S > 65535) return fail(PA_ERR_INVALID_ARG, "num_seqs %d outside [0, 65535]", S);
  if (Hq <= 0) return fail(PA_ERR_INVALID_ARG, "num_q_heads %d <= 0", Hq);
  if (hkv <= 0) return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d <= 0", hkv);
  if (Hq % hkv) return fail(PA_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", Hq, hkv);
  if (D <= 0) return fail(PA_ERR_INVALID_ARG, "head_dim %d <= 0", D);
  if (D != 64 && D != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %d (built: 64, 128)", D);
  if (bs <= 0) return fail(PA_ERR_INVALID_ARG, "block_size %d <= 0", bs);
  if (!block_size_built(bs)) return fail(PA_ERR_UNSUPPORTED, "block_size %d (built: 4, 8, 16, 32)", bs);
  if (MB <= 0) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d <= 0", MB);
  if (ext->num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks %lld <= 0", (long long)ext->num_blocks);
  if (!dtype_valid(ext->dtype)) return fail(PA_ERR_INVALID_ARG, "dtype %d", ext->dtype);
  const int64_t max_tokens = (int64_t)MB * bs;
  if (max_tokens > (int64_t(1) << 30)) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq * block_size too large");
  int64_t part;
  if (ext->partition_size == 0) {
    part = kDefaultPartition;
  } else if (ext->partition_size < 0) {
    part = (max_tokens + 31) / 32 * 32;  // one partition holds a whole sequence
  } else {
    part = ext->partition_size;
    if (part % 32) return fail(PA_ERR_INVALID_ARG, "partition_size %lld is not a multiple of 32", (long long)part);
  }
  const int64_t pmax = (max_tokens + part - 1) / part;
  if (pmax > pa::kMaxPartitions)
    return fail(PA_ERR_UNSUPPORTED, "%lld partitions per sequence (at most %d): raise partition_size",
                (long long)pmax, pa::kMaxPartitions);
  const int32_t G = Hq / hkv;
  const int32_t tiles = (G + 15) / 16;
  if ((int64_t)hkv * tiles > 65535) return fail(PA_ERR_UNSUPPORTED, "too many KV heads for one launch");
  pl->part_tokens = (int32_t)part;
  pl->pmax = (int32_t)pmax;
  pl->head_tiles = tiles;
  pl->max_tokens = (int32_t)max_tokens;
  if (pmax > 1) {
    const size_t rows = (size_t)S * Hq * (size_t)pmax;
    pl->ws_o_bytes = round_up(rows * D * sizeof(float), kAlign);
    pl->ws_bytes = pl->ws_o_bytes + round_up(rows * 2 * sizeof(float), kAlign);
  } else {
    pl->ws_o_bytes = pl->ws_bytes = 0;
  }
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_workspace_bytes(const pa_decode_ext* ext, int32_t block_size,
                                    int32_t num_kv_heads, size_t* bytes) {
  g_error.clear();
  if (!bytes) return fail(PA_ERR_INVALID_ARG, "bytes is NULL");
  Plan pl;
  const pa_status st = plan_decode(ext, block_size, num_kv_heads, &pl);
  if (st != PA_OK) return st;
  *bytes = pl.ws_bytes;
  return PA_OK;
}

pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, int32_t block_size,
                    int32_t num_kv_heads, float scale, void* out, const pa_decode_ext* ext) {
  g_error.clear();
  Plan pl;
  pa_status st = plan_decode(ext, block_size, num_kv_heads, &pl);
  if (st != PA_OK) return st;
  if (ext->num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out)
    return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return fail(PA_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(seq_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "block_tables and seq_lens must be 4-byte aligned");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  if (pl.ws_bytes) {
    if (!ext->workspace || ext->workspace_bytes < pl.ws_bytes)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", pl.ws_bytes,
                  ext->workspace ? ext->workspace_bytes : (size_t)0);
    if (!aligned(ext->workspace, 16)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }

  pa::DecodeParams p;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.out = out;
  p.ws_o = pl.ws_bytes ? static_cast<float*>(ext->workspace) : nullptr;
  p.ws_ml = pl.ws_bytes ? reinterpret_cast<float*>(static_cast<char*>(ext->workspace) + pl.ws_o_bytes)
                        : nullptr;
  p.num_blocks = ext->num_blocks;
  p.num_seqs = ext->num_seqs;
  p.num_q_heads = ext->num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = ext->num_q_heads / num_kv_heads;
  p.head_tiles = pl.head_tiles;
  p.max_blocks = ext->max_blocks_per_seq;
  p.max_tokens = pl.max_tokens;
  p.part_tokens = pl.part_tokens;
  p.pmax = pl.pmax;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);  // log2(e)

  hipStream_t stream = static_cast<hipStream_t>(ext->stream);
  hipError_t e = pa::launch_decode_partitions(ext->dtype, ext->head_dim, block_size, p, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  if (pl.pmax > 1) {
    e = pa::launch_decode_merge(ext->dtype, ext->head_dim, p, stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "merge launch: %s", hipGetErrorString(e));
  }
  return PA_OK;
}

pa_status pa_cache_write(const void* k, const void* v, const int64_t* slot_mapping,
                         void* k_cache, void* v_cache, const pa_cache_write_ext* ext) {
  g_error.clear();
  if (!ext) return fail(PA_ERR_INVALID_ARG, "ext is NULL");
  const int32_t T = ext->num_tokens, Hkv = ext->num_kv_heads, D = ext->head_dim;
  const int32_t bs = ext->block_size;
  if (T < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens %d < 0", T);
  if (Hkv <= 0) return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d <= 0", Hkv);
  if (D <= 0 || D % 8) return fail(PA_ERR_INVALID_ARG, "head_dim %d is not a positive multiple of 8", D);
  if (bs <= 0) return fail(PA_ERR_INVALID_ARG, "block_size %d <= 0", bs);
  if (!block_size_built(bs)) return fail(PA_ERR_UNSUPPORTED, "block_size %d (built: 4, 8, 16, 32)", bs);
  if (ext->num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks %lld <= 0", (long long)ext->num_blocks);
  if (!dtype_valid(ext->dtype)) return fail(PA_ERR_INVALID_ARG, "dtype %d", ext->dtype);
  if ((int64_t)T * Hkv > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "num_tokens * num_kv_heads too large");
  if (ext->num_blocks > (INT64_MAX / bs)) return fail(PA_ERR_INVALID_ARG, "num_blocks too large");
  if (T == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(PA_ERR_INVALID_ARG, "k, v, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(slot_mapping, 8)) return fail(PA_ERR_INVALID_ARG, "slot_mapping must be 8-byte aligned");

  pa::CacheWriteParams p;
  p.k = k;
  p.v = v;
  p.slot_mapping = slot_mapping;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.num_slots = ext->num_blocks * bs;
  p.num_tokens = T;
  p.num_kv_heads = Hkv;
  p.head_dim = D;
  p.block_size = bs;
  const int elem = ext->dtype == PA_F32 ? 4 : 2;
  const hipError_t e = pa::launch_cache_write(elem, p, static_cast<hipStream_t>(ext->stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "cache write launch: %s", hipGetErrorString(e));
  return PA_OK;
}

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* pa_last_error(void) { return g_error.c_str(); }

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

}  // extern "C"
