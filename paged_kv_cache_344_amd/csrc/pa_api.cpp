// pa_api.cpp - the C ABI of libpa.so: argument checks, launch planning, dispatch.
//
// Every host-side argument is checked before the first HIP call, so a bad call
// returns a status without touching the GPU (and can be tested on a machine with
// none).  The library owns no device memory: the decode workspace (work queue,
// merge counters, split-K partials) and the multi-token one (context-split partials)
// are the caller's, sized by pa_decode_workspace_bytes and
// pa_multi_token_workspace_bytes.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <string>
#include <vector>

#include "kernels.h"
#include "pa.h"
#include "pa_probe.h"
#include "read_probe.h"

static_assert(PA_READ_PROBE_TILE == pa::kProbeTile &&
                  PA_READ_PROBE_SINK_BYTES == (size_t)pa::kProbeGrid * pa::kProbeWaves * 4,
              "pa_probe.h and the read probe disagree on its tile or sink size");
static_assert(PA_NOALLOC_SCRATCH_BYTES == pa::kStaticScratchBytes,
              "pa.h and the library disagree on the no-allocation scratch size");

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

// Where everything lives inside a decode workspace (byte offsets).
struct Plan {
  int32_t part_tokens;
  int32_t pmax;        // partitions a sequence can have
  int32_t nodes;       // groups of kMergeFan partitions
  int32_t head_tiles;
  int32_t max_tokens;
  int32_t slice;       // sequences per launch
  size_t off_node_count, off_root_count, off_part_o, off_part_ml, off_node_o, off_node_ml;
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
  const int64_t ht2 = (int64_t)hkv * tiles;
  if (ht2 > 65535) return fail(PA_ERR_UNSUPPORTED, "too many KV heads for one launch");
  const int64_t nodes = (pmax + pa::kMergeFan - 1) / pa::kMergeFan;
  // work items of one launch, (full + last partitions) x head tiles, stay below 2^31
  const int64_t slice = std::min<int64_t>(pa::kScanMax, (INT32_MAX - (1 << 20)) / (pmax * ht2));
  pl->part_tokens = (int32_t)part;
  pl->pmax = (int32_t)pmax;
  pl->nodes = (int32_t)nodes;
  pl->head_tiles = tiles;
  pl->max_tokens = (int32_t)max_tokens;
  pl->slice = (int32_t)slice;
  // [queue: 2 ints][node counts][root counts][partition partials][group partials];
  // partials are [sequence][partition or group][query head][D] (and [..][2] for max, sum)
  size_t off = kAlign;
  pl->off_node_count = off;
  off = round_up(off + (size_t)S * ht2 * nodes * sizeof(int32_t), kAlign);
  pl->off_root_count = off;
  off = round_up(off + (size_t)S * ht2 * sizeof(int32_t), kAlign);
  const size_t rows = (size_t)S * Hq;
  pl->off_part_o = off;
  if (pmax > 1) off = round_up(off + rows * pmax * D * sizeof(float), kAlign);
  pl->off_part_ml = off;
  if (pmax > 1) off = round_up(off + rows * pmax * 2 * sizeof(float), kAlign);
  pl->off_node_o = off;
  if (nodes > 1) off = round_up(off + rows * nodes * D * sizeof(float), kAlign);
  pl->off_node_ml = off;
  if (nodes > 1) off = round_up(off + rows * nodes * 2 * sizeof(float), kAlign);
  pl->ws_bytes = off;
  return PA_OK;
}

// Workgroups of the persistent decode launch: as many as are resident at once.
// Cached per (device, kernel instance) after the first query.
std::atomic<int> g_grid_cache[16][3][2][4];

pa_status decode_grid(int dtype, int D, int bs, int* grid) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  const int bi = bs == 4 ? 0 : bs == 8 ? 1 : bs == 16 ? 2 : 3;
  std::atomic<int>* slot = (dev >= 0 && dev < 16) ? &g_grid_cache[dev][dtype][D == 128][bi] : nullptr;
  if (slot) {
    const int cached = slot->load(std::memory_order_relaxed);
    if (cached > 0) {
      *grid = cached;
      return PA_OK;
    }
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
  e = pa::decode_blocks_per_cu(dtype, D, bs, &per_cu);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
  *grid = std::max(1, cus) * std::max(1, per_cu);
  if (slot) slot->store(*grid, std::memory_order_relaxed);
  return PA_OK;
}


// Shapes of a pa_multi_token call, checked, and its context split.
struct MtPlan {
  bool empty = false;       // nothing to compute
  int32_t max_tokens = 0;   // L_max: max_seq_len if given, else max_blocks_per_seq * bs
  int32_t tiles = 0;        // 128-row tiles per (sequence, KV head)
  int32_t parts = 1;        // context partitions (1: no split)
  int32_t part_tokens = 0;  // positions per partition
  int32_t part_rows = 0;    // rows stored per (tile, partition)
  int64_t partial_rows = 0; // rows of partials in the workspace
  size_t ws_bytes = 0;
};

pa_status plan_multi_token(const pa_multi_token_ext* ext, int32_t bs, int32_t hkv, MtPlan* pl) {
  if (!ext) return fail(PA_ERR_INVALID_ARG, "ext is NULL");
  const int32_t S = ext->num_seqs, T = ext->num_tokens, Hq = ext->num_q_heads, D = ext->head_dim;
  const int32_t MB = ext->max_blocks_per_seq;
  if (S < 0 || S > 65535) return fail(PA_ERR_INVALID_ARG, "num_seqs %d outside [0, 65535]", S);
  if (T < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens %d < 0", T);
  if (ext->max_query_len < 0) return fail(PA_ERR_INVALID_ARG, "max_query_len %d < 0", ext->max_query_len);
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
  if (ext->max_seq_len < 0) return fail(PA_ERR_INVALID_ARG, "max_seq_len %d < 0", ext->max_seq_len);
  if ((int64_t)MB * bs > (int64_t(1) << 30)) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq * block_size too large");
  // L_max: the caller's bound on every length when given (the split is sized for it and
  // a longer sequence gets NaN rows), else what the table can hold
  const int64_t max_tokens = ext->max_seq_len > 0 ? std::min<int64_t>(ext->max_seq_len, (int64_t)MB * bs)
                                                  : (int64_t)MB * bs;
  const int32_t psz = ext->partition_size;
  if (psz > 0 && psz % 32) return fail(PA_ERR_INVALID_ARG, "partition_size %d is not a multiple of 32", psz);
  pl->max_tokens = (int32_t)max_tokens;
  if (S == 0 || T == 0 || ext->max_query_len == 0) {
    pl->empty = true;
    return PA_OK;
  }
  const int32_t G = Hq / hkv;
  const int64_t R = pa::multi_token_rows_per_group();
  const int64_t rows = (int64_t)std::min(ext->max_query_len, T) * G;
  const int64_t tiles = (rows + R - 1) / R;
  if ((int64_t)T * G > (int64_t)INT32_MAX - 1024 || (int64_t)T * Hq * D > ((int64_t)1 << 40))
    return fail(PA_ERR_UNSUPPORTED, "num_tokens %d too large for one launch", T);
  const int64_t triples = (int64_t)S * hkv * tiles;
  const int64_t part_rows = std::min(R, rows);
  int64_t part_tokens = 0;
  if (psz > 0) {
    part_tokens = psz;
  } else if (psz == 0) {
    // about 768 workgroups (one and a half rounds of the two per CU that fit on a
    // 256-CU device: fewer, longer partitions write and merge fewer partials, and
    // measured on draft verification 704-832 workgroups beat both 576 and 1024-2048),
    // partitions long enough that their partials ((D + 2) * 4 bytes per row) stay small
    // next to the K/V they replace (2 * D * 2 bytes per position): at least 16
    // positions per stored row
    const int64_t min_part = std::max<int64_t>(256, (16 * part_rows + 31) / 32 * 32);
    const int64_t want = (768 + triples - 1) / triples;
    const int64_t fit = max_tokens / min_part;
    const int64_t parts = std::min(want, fit);
    if (triples < 512 && parts >= 2) part_tokens = ((max_tokens + parts - 1) / parts + 31) / 32 * 32;
  }
  int64_t parts = part_tokens > 0 ? (max_tokens + part_tokens - 1) / part_tokens : 1;
  if (parts <= 1) {
    parts = 1;
    part_tokens = 0;
  }
  const int64_t wgs = (((int64_t)S * hkv + 7) / 8 * 8) * tiles * parts;  // groups dealt to 8 XCDs
  if (wgs > (int64_t)INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "%lld workgroups in one launch", (long long)wgs);
  pl->tiles = (int32_t)tiles;
  pl->parts = (int32_t)parts;
  pl->part_tokens = (int32_t)part_tokens;
  pl->part_rows = (int32_t)part_rows;
  if (parts > 1) {
    pl->partial_rows = triples * parts * part_rows;
    pl->ws_bytes = (size_t)pl->partial_rows * (size_t)(D + 2) * sizeof(float);
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

}  // extern "C"

namespace {

// Checks of a decode call's tensor arguments (the workspace is checked by the callers).
pa_status check_decode_args(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens, float scale,
                            const void* out) {
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out)
    return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return fail(PA_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(seq_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "block_tables and seq_lens must be 4-byte aligned");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  return PA_OK;
}

// The decode launches of a checked call, with ws (of at least pl.ws_bytes bytes) as the
// workspace.
// Fused cache write of pa_cache_write_decode: one new token per sequence (row s of
// k and v), to slot slot_mapping[s].
struct NewTokens {
  const void* k = nullptr;
  const void* v = nullptr;
  const int64_t* slot_mapping = nullptr;
};

pa_status decode_launches(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens, int32_t block_size,
                          int32_t num_kv_heads, float scale, void* out, const pa_decode_ext* ext,
                          const Plan& pl, char* ws, const NewTokens& nt = NewTokens()) {
  int grid = 0;
  pa_status st = decode_grid(ext->dtype, ext->head_dim, block_size, &grid);
  if (st != PA_OK) return st;

  const int32_t S = ext->num_seqs, Hq = ext->num_q_heads, D = ext->head_dim;
  const int64_t ht2 = (int64_t)num_kv_heads * pl.head_tiles;
  pa::DecodeParams p;
  p.num_blocks = ext->num_blocks;
  p.num_q_heads = Hq;
  p.num_kv_heads = num_kv_heads;
  p.group = Hq / num_kv_heads;
  p.head_tiles = pl.head_tiles;
  p.max_blocks = ext->max_blocks_per_seq;
  p.max_tokens = pl.max_tokens;
  p.part_tokens = pl.part_tokens;
  p.auto_part = ext->partition_size == 0 ? 1 : 0;
  p.pmax = pl.pmax;
  p.nodes = pl.nodes;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);  // log2(e)
  p.queue = reinterpret_cast<int32_t*>(ws);
  p.num_slots = ext->num_blocks * block_size;

  const size_t esz = ext->dtype == PA_F32 ? 4 : 2;
  hipStream_t stream = static_cast<hipStream_t>(ext->stream);
  // one launch per slice of at most pl.slice sequences, in order on the stream
  for (int32_t s0 = 0; s0 < S; s0 += pl.slice) {
    const int32_t n = std::min(pl.slice, S - s0);
    const size_t rows0 = (size_t)s0 * Hq;
    p.q = static_cast<const char*>(q) + rows0 * D * esz;
    p.out = static_cast<char*>(out) + rows0 * D * esz;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables + (size_t)s0 * ext->max_blocks_per_seq;
    p.seq_lens = seq_lens + s0;
    p.num_seqs = n;
    const size_t new_rows = (size_t)s0 * num_kv_heads * D * esz;
    p.k_new = nt.slot_mapping ? static_cast<const char*>(nt.k) + new_rows : nullptr;
    p.v_new = nt.slot_mapping ? static_cast<const char*>(nt.v) + new_rows : nullptr;
    p.slot_mapping = nt.slot_mapping ? nt.slot_mapping + s0 : nullptr;
    p.node_count = reinterpret_cast<int32_t*>(ws + pl.off_node_count) + (size_t)s0 * ht2 * pl.nodes;
    p.root_count = reinterpret_cast<int32_t*>(ws + pl.off_root_count) + (size_t)s0 * ht2;
    p.part_o = reinterpret_cast<float*>(ws + pl.off_part_o) + rows0 * pl.pmax * D;
    p.part_ml = reinterpret_cast<float*>(ws + pl.off_part_ml) + rows0 * pl.pmax * 2;
    p.node_o = reinterpret_cast<float*>(ws + pl.off_node_o) + rows0 * pl.nodes * D;
    p.node_ml = reinterpret_cast<float*>(ws + pl.off_node_ml) + rows0 * pl.nodes * 2;
    // no more workgroups than there can be items
    const int64_t most = (int64_t)n * pl.pmax * ht2;
    const int g = (int)std::min<int64_t>(grid, most);
    // Non-temporal K/V loads when no table shares a block and the launch can fill the
    // device; a launch of fewer items than resident workgroups (e.g. no split) streams
    // each sequence through one workgroup, which the default policy serves better.
    p.stream_kv = !ext->shared_blocks && most >= grid ? 1 : 0;
    const hipError_t e = pa::launch_decode(ext->dtype, D, block_size, p, g, stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  }
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, int32_t block_size,
                    int32_t num_kv_heads, float scale, void* out, const pa_decode_ext* ext) {
  g_error.clear();
  Plan pl;
  pa_status st = plan_decode(ext, block_size, num_kv_heads, &pl);
  if (st != PA_OK) return st;
  if (ext->num_seqs == 0) return PA_OK;
  st = check_decode_args(q, k_cache, v_cache, block_tables, seq_lens, scale, out);
  if (st != PA_OK) return st;
  if (!ext->workspace || ext->workspace_bytes < pl.ws_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", pl.ws_bytes,
                ext->workspace ? ext->workspace_bytes : (size_t)0);
  if (!aligned(ext->workspace, 16)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return decode_launches(q, k_cache, v_cache, block_tables, seq_lens, block_size, num_kv_heads,
                         scale, out, ext, pl, static_cast<char*>(ext->workspace));
}

pa_status pa_cache_write_decode(const void* k, const void* v, const int64_t* slot_mapping,
                                const void* q, void* k_cache, void* v_cache,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                int32_t block_size, int32_t num_kv_heads, float scale, void* out,
                                const pa_decode_ext* ext) {
  g_error.clear();
  Plan pl;
  pa_status st = plan_decode(ext, block_size, num_kv_heads, &pl);
  if (st != PA_OK) return st;
  if (ext->num_seqs == 0) return PA_OK;
  st = check_decode_args(q, k_cache, v_cache, block_tables, seq_lens, scale, out);
  if (st != PA_OK) return st;
  if (!k || !v || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "k, v or slot_mapping is NULL");
  if (!aligned(k, 16) || !aligned(v, 16)) return fail(PA_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  if (!aligned(slot_mapping, 8)) return fail(PA_ERR_INVALID_ARG, "slot_mapping must be 8-byte aligned");
  if (ext->num_blocks > INT64_MAX / block_size) return fail(PA_ERR_INVALID_ARG, "num_blocks too large");
  if (!ext->workspace || ext->workspace_bytes < pl.ws_bytes)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", pl.ws_bytes,
                ext->workspace ? ext->workspace_bytes : (size_t)0);
  if (!aligned(ext->workspace, 16)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  NewTokens nt;
  nt.k = k;
  nt.v = v;
  nt.slot_mapping = slot_mapping;
  return decode_launches(q, k_cache, v_cache, block_tables, seq_lens, block_size, num_kv_heads,
                         scale, out, ext, pl, static_cast<char*>(ext->workspace), nt);
}

pa_status pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            int32_t block_size, int32_t num_kv_heads, float scale, void* out,
                            const pa_decode_ext* ext) {
  g_error.clear();
  Plan pl;
  pa_status st = plan_decode(ext, block_size, num_kv_heads, &pl);
  if (st != PA_OK) return st;
  if (ext->num_seqs == 0) return PA_OK;
  st = check_decode_args(q, k_cache, v_cache, block_tables, seq_lens, scale, out);
  if (st != PA_OK) return st;
  if (pl.ws_bytes > pa::kStaticScratchBytes)
    return fail(PA_ERR_WORKSPACE, "this call needs %zu bytes of scratch; the static scratch holds %zu "
                "(use pa_decode with a workspace)", pl.ws_bytes, pa::kStaticScratchBytes);
  void* ws = nullptr;
  hipError_t e = pa::static_scratch(&ws);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "static scratch address: %s", hipGetErrorString(e));
  // the array keeps the previous call's contents: its queue and merge counters start at zero
  e = pa::launch_clear(ws, pl.off_part_o, static_cast<hipStream_t>(ext->stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "scratch clear launch: %s", hipGetErrorString(e));
  return decode_launches(q, k_cache, v_cache, block_tables, seq_lens, block_size, num_kv_heads,
                         scale, out, ext, pl, static_cast<char*>(ws));
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

pa_status pa_multi_token_workspace_bytes(const pa_multi_token_ext* ext, int32_t block_size,
                                         int32_t num_kv_heads, size_t* bytes) {
  g_error.clear();
  if (!bytes) return fail(PA_ERR_INVALID_ARG, "bytes is NULL");
  MtPlan pl;
  const pa_status st = plan_multi_token(ext, block_size, num_kv_heads, &pl);
  if (st != PA_OK) return st;
  *bytes = pl.ws_bytes;
  return PA_OK;
}

pa_status pa_multi_token(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* query_start, int32_t block_size, int32_t num_kv_heads,
                         float scale, void* out, const pa_multi_token_ext* ext) {
  g_error.clear();
  MtPlan pl;
  const pa_status st = plan_multi_token(ext, block_size, num_kv_heads, &pl);
  if (st != PA_OK) return st;
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  if (pl.empty) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start || !out)
    return fail(PA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return fail(PA_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(query_start, 4))
    return fail(PA_ERR_INVALID_ARG, "block_tables, seq_lens and query_start must be 4-byte aligned");
  if (pl.parts > 1) {
    if (!ext->workspace || ext->workspace_bytes < pl.ws_bytes)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", pl.ws_bytes,
                  ext->workspace ? ext->workspace_bytes : (size_t)0);
    if (!aligned(ext->workspace, 16)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  const int32_t hkv = num_kv_heads;
  pa::MultiTokenParams p;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.query_start = query_start;
  p.out = out;
  p.num_blocks = ext->num_blocks;
  p.num_seqs = ext->num_seqs;
  p.num_tokens = ext->num_tokens;
  p.num_q_heads = ext->num_q_heads;
  p.num_kv_heads = hkv;
  p.group = ext->num_q_heads / hkv;
  p.max_blocks = ext->max_blocks_per_seq;
  p.max_tokens = pl.max_tokens;
  p.row_tiles = pl.tiles;
  p.parts = pl.parts;
  p.part_tokens = pl.part_tokens;
  p.part_rows = pl.part_rows;
  p.part_o = nullptr;
  p.part_ml = nullptr;
  if (pl.parts > 1) {
    p.part_o = static_cast<float*>(ext->workspace);
    p.part_ml = p.part_o + pl.partial_rows * ext->head_dim;
  }
  p.scale_log2 = (float)((double)scale * 1.4426950408889634074);  // log2(e)
  hipStream_t stream = static_cast<hipStream_t>(ext->stream);
  hipError_t e = pa::launch_multi_token(ext->dtype, ext->head_dim, block_size, p, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "multi-token launch: %s", hipGetErrorString(e));
  if (pl.parts > 1) {
    e = pa::launch_multi_token_merge(ext->dtype, ext->head_dim, p, stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "multi-token merge launch: %s", hipGetErrorString(e));
  }
  return PA_OK;
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                         int32_t n, const pa_copy_blocks_ext* ext) {
  g_error.clear();
  if (!ext) return fail(PA_ERR_INVALID_ARG, "ext is NULL");
  const int32_t Hkv = ext->num_kv_heads, D = ext->head_dim, bs = ext->block_size;
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "n %d < 0", n);
  if (Hkv <= 0) return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d <= 0", Hkv);
  if (D <= 0 || D % 8) return fail(PA_ERR_INVALID_ARG, "head_dim %d is not a positive multiple of 8", D);
  if (bs <= 0) return fail(PA_ERR_INVALID_ARG, "block_size %d <= 0", bs);
  if (!block_size_built(bs)) return fail(PA_ERR_UNSUPPORTED, "block_size %d (built: 4, 8, 16, 32)", bs);
  if (ext->num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks %lld <= 0", (long long)ext->num_blocks);
  if (!dtype_valid(ext->dtype)) return fail(PA_ERR_INVALID_ARG, "dtype %d", ext->dtype);
  if (n == 0) return PA_OK;
  if (!k_cache || !v_cache || !src || !dst) return fail(PA_ERR_INVALID_ARG, "a pointer is NULL");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(PA_ERR_INVALID_ARG, "k_cache and v_cache must be 16-byte aligned");
  // ids in the pool, no self-copy, destinations distinct and never a source (a copy
  // must not read a block another copy of the same call writes)
  std::vector<int32_t> ds(dst, dst + n), ss(src, src + n);
  for (int32_t i = 0; i < n; ++i) {
    if (src[i] < 0 || src[i] >= ext->num_blocks || dst[i] < 0 || dst[i] >= ext->num_blocks)
      return fail(PA_ERR_INVALID_ARG, "pair %d (%d -> %d) outside the pool", i, src[i], dst[i]);
    if (src[i] == dst[i]) return fail(PA_ERR_INVALID_ARG, "pair %d copies block %d onto itself", i, src[i]);
  }
  std::sort(ds.begin(), ds.end());
  std::sort(ss.begin(), ss.end());
  for (int32_t i = 1; i < n; ++i)
    if (ds[(size_t)i] == ds[(size_t)i - 1]) return fail(PA_ERR_INVALID_ARG, "block %d is a destination twice", ds[(size_t)i]);
  for (size_t i = 0, j = 0; i < ds.size() && j < ss.size();) {
    if (ds[i] == ss[j]) return fail(PA_ERR_INVALID_ARG, "block %d is both a source and a destination", ds[i]);
    if (ds[i] < ss[j]) ++i;
    else ++j;
  }
  pa::CopyBlocksParams p;
  p.k_cache = static_cast<char*>(k_cache);
  p.v_cache = static_cast<char*>(v_cache);
  p.block_bytes = (int64_t)Hkv * bs * D * (ext->dtype == PA_F32 ? 4 : 2);
  hipStream_t stream = static_cast<hipStream_t>(ext->stream);
  for (int32_t i0 = 0; i0 < n; i0 += pa::kCopyBatch) {
    p.n = std::min(pa::kCopyBatch, n - i0);
    for (int32_t i = 0; i < p.n; ++i) {
      p.pairs[2 * i] = src[i0 + i];
      p.pairs[2 * i + 1] = dst[i0 + i];
    }
    const hipError_t e = pa::launch_copy_blocks(p, stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "copy launch: %s", hipGetErrorString(e));
  }
  return PA_OK;
}

pa_status pa_read_probe(const void* src, size_t src_bytes, const int32_t* tiles,
                        int64_t n_tiles, void* sink, size_t sink_bytes, void* stream) {
  g_error.clear();
  if (n_tiles < 0) return fail(PA_ERR_INVALID_ARG, "n_tiles %lld < 0", (long long)n_tiles);
  if (src_bytes % PA_READ_PROBE_TILE)
    return fail(PA_ERR_INVALID_ARG, "src_bytes %zu is not a multiple of %d", src_bytes, PA_READ_PROBE_TILE);
  const int64_t in_src = (int64_t)(src_bytes / PA_READ_PROBE_TILE);
  if (!tiles && n_tiles > in_src)
    return fail(PA_ERR_INVALID_ARG, "n_tiles %lld > %lld tiles in src", (long long)n_tiles, (long long)in_src);
  if (sink_bytes < PA_READ_PROBE_SINK_BYTES)
    return fail(PA_ERR_INVALID_ARG, "sink_bytes %zu < %zu", sink_bytes, (size_t)PA_READ_PROBE_SINK_BYTES);
  if (n_tiles == 0) return PA_OK;
  if (!src || !sink) return fail(PA_ERR_INVALID_ARG, "src or sink is NULL");
  if (!aligned(src, 16) || !aligned(sink, 4) || (tiles && !aligned(tiles, 4)))
    return fail(PA_ERR_INVALID_ARG, "src must be 16-byte aligned, sink and tiles 4-byte aligned");
  const hipError_t e = pa::launch_read_probe(static_cast<const char*>(src), in_src, tiles, n_tiles,
                                             static_cast<uint32_t*>(sink),
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "read probe launch: %s", hipGetErrorString(e));
  return PA_OK;
}

__attribute__((visibility("hidden"))) void pa_set_last_error_internal(const char* text) {
  try {
    g_error = text ? text : "";
  } catch (...) {
  }
}

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_CAPACITY: return "no free block, or a block table would overflow";
  }
  return "unknown status";
}

const char* pa_last_error(void) { return g_error.c_str(); }

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

}  // extern "C"
