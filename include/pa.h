/*
 * pa.h - paged decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpa.so.  Two operations make up the hot path of PagedAttention:
 *
 *   pa_cache_write  stores each new token's key and value in the cache slot its
 *                   slot id names.
 *   pa_decode       single-query attention for every sequence of a batch, reading
 *                   each sequence's keys and values through its block table.
 *
 * Pages cited (title, site):
 *   [AB]  "什么是分页注意力（PagedAttention）？"                     aiboss88.com wiki
 *   [CY]  "深入解析 PagedAttention：vLLM 显存优化的核心魔法"            cygnushan.xyz blog
 *   [ASP] "PagedAttention"                                          awesome-system-papers
 *   [RK]  "什么是 LLM 中的分页注意力(Paged Attention)?它是如何工作的?"  news.rkmt.cn
 *
 * ---- Storage (the pages fix no layout; this is the library's definition) ----
 * The KV cache is a pool of N fixed-size physical blocks of block_size (bs) token
 * slots each, for every KV head ([AB] 工作机制: the cache is cut into equal blocks
 * that may sit anywhere; [ASP] 核心思想: e.g. 16 tokens a block).  Two device
 * arrays, row-major, element type = the batch dtype:
 *
 *   k_cache [N][Hkv][bs][D]   one (block, KV head) tile holds bs key rows of D
 *   v_cache [N][Hkv][D][bs]   one (block, KV head) tile holds D value columns
 *
 * so every (block, KV head) tile of either array is bs*D contiguous elements:
 * inside a block, access stays contiguous ([ASP] 核心思想, the kernel rewrite).
 * The value tile is stored dimension-major so the attention kernel's weighted
 * sum over tokens reads whole 16-byte rows.
 *
 * Token t (0-based) of sequence s lives in physical block block_tables[s][t / bs]
 * at in-block offset t % bs ([RK] 块表: logical blocks numbered 0, 1, 2 map to
 * scattered physical blocks).  A slot id is phys * bs + offset.
 *
 * ---- Conventions -----------------------------------------------------------
 * - Every pointer argument that names tensor data is a DEVICE pointer owned by
 *   the caller; the library never allocates, frees or keeps memory, and keeps no
 *   pointer after a call returns.  Tensor pointers must be 16-byte aligned.
 * - Calls are asynchronous on the HIP stream given in the ext struct (NULL = the
 *   null stream).  No call synchronises the host.
 * - Every host-side argument is checked before anything is sent to the GPU; a
 *   bad argument returns an error status and launches nothing.  pa_last_error()
 *   then returns a readable reason.  No C++ exception crosses the ABI.
 * - Supported: dtype f32, f16, bf16; head_dim 64 or 128; block_size 4, 8, 16 or
 *   32; num_q_heads a multiple of num_kv_heads.  Anything else is
 *   PA_ERR_UNSUPPORTED or PA_ERR_INVALID_ARG.
 * - Calls are reentrant and thread-safe: no global mutable state beyond the
 *   thread-local error text and a per-device cache of the decode launch size.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* a null pointer, a bad size, a misaligned pointer       */
  PA_ERR_UNSUPPORTED = 2, /* valid but not built: dtype / head_dim / block_size ... */
  PA_ERR_WORKSPACE = 3,   /* a workspace missing or smaller than required            */
  PA_ERR_HIP = 4,         /* the HIP runtime refused a launch; see pa_last_error()   */
  PA_ERR_CAPACITY = 5     /* block manager: no free block, or a table would overflow */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

/* Shapes and options of a pa_decode call that its positional arguments leave out. */
typedef struct pa_decode_ext {
  int32_t num_seqs;           /* S >= 0 (0: nothing to do) and <= 65535               */
  int32_t num_q_heads;        /* Hq > 0, a multiple of num_kv_heads                    */
  int32_t head_dim;           /* D: 64 or 128                                          */
  int32_t max_blocks_per_seq; /* row stride of block_tables, >= 1                      */
  int64_t num_blocks;         /* N, physical blocks in the pool, >= 1                  */
  int32_t partition_size;     /* tokens per split-K partition: 0 = default (chosen on  */
                              /* the device from the lengths: one workgroup's even   */
                              /* share of the work, rounded up to a multiple of 256,  */
                              /* or 3/4 of it when no sequence would be split but the */
                              /* (sequence, head) units outnumber the workgroups; at  */
                              /* least 512), < 0 = never split, > 0 = that many (a    */
                              /* multiple of 32)                                      */
  int32_t dtype;              /* pa_dtype of q, k_cache, v_cache and out               */
  void* workspace;            /* device scratch: queue, counters, split-K partials;    */
                              /* caller-owned, zero-filled before first use            */
  size_t workspace_bytes;     /* its size; see pa_decode_workspace_bytes               */
  void* stream;               /* hipStream_t                                           */
  int32_t shared_blocks;      /* nonzero: block tables may share physical blocks       */
                              /* (common prefixes, parallel sampling, beam search):  */
                              /* K/V loads keep the default cache policy so a shared */
                              /* block read by one sequence stays cached for the     */
                              /* others; 0: every K/V byte is read once per call and */
                              /* is loaded non-temporally (when the launch can fill  */
                              /* the device).  Results are the same either way.      */
} pa_decode_ext;

/*
 * pa_decode - single-query decode attention over the paged cache.
 *
 * For every sequence s and query head h (KV head g = h / (Hq / Hkv), consecutive
 * grouping):
 *     z_t = scale * <q[s][h], K_s[t]>,     t = 0 .. seq_lens[s] - 1
 *     out[s][h] = sum_t exp(z_t - max z) V_s[t] / sum_t exp(z_t - max z)
 * where K_s[t], V_s[t] are token t's key and value for KV head g, found through
 * the block table.  Paging changes where K and V live, not this formula ([AB]
 * 边界与常见误解, first point); the kernel takes the block table and gathers K and
 * V block by block ([ASP] 实现要点, the custom kernel that accepts a block table).
 * seq_lens[s] counts every token attended, including one just stored with
 * pa_cache_write.  seq_lens[s] == 0 gives out[s] = 0.
 *
 *   q             [S][Hq][D]                 dtype
 *   k_cache       [N][Hkv][bs][D]            dtype
 *   v_cache       [N][Hkv][D][bs]            dtype
 *   block_tables  [S][max_blocks_per_seq]    int32; only the first
 *                 ceil(seq_lens[s] / bs) entries of row s are read (the rest may
 *                 hold anything, e.g. -1 as in [CY] 核心思想 / Block Table)
 *   seq_lens      [S]                        int32, device memory
 *   block_size    bs; num_kv_heads Hkv; scale: the logit scale (e.g. 1/sqrt(D))
 *   out           [S][Hq][D]                 dtype; written, rounded to nearest even
 *
 * Arithmetic: fp32 accumulation everywhere.  For f16 / bf16 the softmax weights
 * enter the weighted sum (a matrix-core product) as a hi + lo pair of the input
 * dtype, about 16 significant bits; the only rounding left is the output's.
 * Long sequences are split into partitions of partition_size tokens; each
 * partition keeps (running max, running sum, unnormalised output) in the
 * workspace, and the partitions are combined with log-sum-exp weights along a
 * fixed tree (groups of 16 partitions, then the groups) inside the same launch,
 * so results are deterministic and do not depend on physical placement or on
 * timing.
 *
 * Device-side contract (cannot be checked on the host without a sync): table
 * entries in the used range lie in [0, N) and 0 <= seq_lens[s] <=
 * max_blocks_per_seq * bs.  A violation never faults: an out-of-range table
 * entry or length makes every output row of that sequence NaN.
 *
 * Workspace (ext->workspace, ext->workspace_bytes): device memory owned by the
 * caller, of at least pa_decode_workspace_bytes bytes, needed by every call.  It
 * holds the work queue and merge counters of the launch and, when a sequence can
 * span several partitions, the per-partition partial results.  It must be
 * zero-filled before its first use.  Every call that returns PA_OK and runs to
 * completion returns its counters (the leading part of the workspace, up to the
 * partial results) to zero; the partial results are scratch that needs no
 * clearing.  So one workspace serves any number of calls of one shape (num_seqs,
 * num_q_heads, head_dim, max_blocks_per_seq, partition_size, block_size,
 * num_kv_heads).  Where the counters end depends on the shape, so a call of another
 * shape may leave partial results where this shape keeps counters: zero-fill the
 * workspace again before using it for a different shape (or keep one workspace per
 * shape).  Calls that share a workspace must be ordered on one stream: calls that
 * overlap on the same workspace race.  Bytes 64..67 of the workspace (an int32) are not
 * a counter: after a call they hold the partition length, in tokens, that it used (the
 * default one chosen on the device, or partition_size; with more than 1024 sequences,
 * that of the last launch of 1024).
 *
 * Execution: one persistent launch per 1024 sequences (about as many workgroups
 * as are resident on the device at once), each planning from seq_lens which
 * partitions hold tokens and taking work items from a queue in the workspace.
 * K/V loads are non-temporal unless ext->shared_blocks is set or the launch has
 * fewer possible items than resident workgroups; results are the same either way.
 */
pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, int32_t block_size,
                    int32_t num_kv_heads, float scale, void* out, const pa_decode_ext* ext);

/*
 * pa_cache_write_decode - one decode step in one launch: pa_cache_write of each
 * sequence's new token, then pa_decode, with the same results, bit for bit, as those two
 * calls in that order on one stream ([RK] 分页注意力是如何工作的: each step stores the new
 * token in the next slot of its sequence's last block and attends over all tokens so
 * far).
 *
 *   k, v          [S][Hkv][D]   dtype, device: row s is sequence s's new token
 *   slot_mapping  [S]           int64, device: its slot (< 0: sequence s has none)
 *   q ... out, ext              as for pa_decode (the same workspace rules)
 *
 * Contract, beyond the two calls': slot_mapping[s], when >= 0, is the slot of position
 * seq_lens[s] - 1 of sequence s (the slot the decode then reads the new token from), and
 * no block table reads a slot that another sequence's token is written to (a block
 * several tables share is copied first, [CY] 多序列共享).  Inside the launch the stores of
 * the new tokens and the reads of the cache are not ordered; the decode takes sequence
 * s's last key and value from k and v instead of the cache when slot_mapping[s] is that
 * position's slot (checked per sequence on the device).  If slot_mapping[s] names another
 * slot, the token is still stored there and the decode reads position seq_lens[s] - 1
 * from the cache as it stands; a slot both written and read in one call gives an
 * undefined value.  Errors: those of pa_decode, and PA_ERR_INVALID_ARG for NULL or
 * misaligned k, v (16 bytes) or slot_mapping (8 bytes).
 */
pa_status pa_cache_write_decode(const void* k, const void* v, const int64_t* slot_mapping,
                                const void* q, void* k_cache, void* v_cache,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                int32_t block_size, int32_t num_kv_heads, float scale, void* out,
                                const pa_decode_ext* ext);

/*
 * pa_decode_noalloc - pa_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops and harnesses that forbid allocation).
 *
 * Same arguments, results and errors as pa_decode, except that ext->workspace and
 * ext->workspace_bytes are ignored: the call uses a scratch array that the library
 * holds in device memory, PA_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU it runs on,
 * from that GPU's first such call until the process ends.  The call allocates nothing
 * (no hipMalloc, no allocating library routine); it clears the scratch's counters with a
 * small kernel on ext->stream, then launches the decode kernel there.  A call whose
 * shapes need more scratch than that (see pa_decode_workspace_bytes) returns
 * PA_ERR_WORKSPACE and launches nothing.  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (on different streams, or from several host
 * threads without ordering) race and give wrong results; calls ordered on one stream
 * are safe.  The partition length a call used is not reported.
 */
pa_status pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            int32_t block_size, int32_t num_kv_heads, float scale, void* out,
                            const pa_decode_ext* ext);

#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * pa_decode_workspace_bytes - bytes of workspace a pa_decode call with these
 * shapes needs (always > 0: a few hundred bytes of counters when no sequence can
 * span two partitions, plus S * Hq * pmax * (D + 2) * 4 bytes of partials when
 * one can, pmax = ceil(max_blocks_per_seq * bs / partition size), and a further
 * S * Hq * ceil(pmax / 16) * (D + 2) * 4 when pmax > 16).  Only the shape fields of
 * ext are read.  Returns PA_OK and sets *bytes, or an error status for the same
 * argument errors pa_decode would report.
 */
pa_status pa_decode_workspace_bytes(const pa_decode_ext* ext, int32_t block_size,
                                    int32_t num_kv_heads, size_t* bytes);

/* Shapes of a pa_cache_write call. */
typedef struct pa_cache_write_ext {
  int32_t num_tokens;   /* T >= 0 (0: nothing to do)                 */
  int32_t num_kv_heads; /* Hkv > 0                                   */
  int32_t head_dim;     /* D > 0, a multiple of 8                    */
  int32_t block_size;   /* bs: 4, 8, 16 or 32                        */
  int64_t num_blocks;   /* N >= 1                                    */
  int32_t dtype;        /* pa_dtype of k, v and the cache            */
  void* stream;         /* hipStream_t                               */
} pa_cache_write_ext;

/*
 * pa_cache_write - store each new token's key and value in its slot.
 *
 * For every token i with slot = slot_mapping[i] >= 0 and every KV head g:
 *     k_cache[slot / bs][g][slot % bs][:] = k[i][g][:]
 *     v_cache[slot / bs][g][:][slot % bs] = v[i][g][:]
 * A token fills the next free slot of its sequence's last block, and a new block
 * is taken only when that one is full ([RK] 分页注意力是如何工作的; [ASP] 核心思想, a
 * new block every bs tokens); choosing the slot is the caller's block manager's
 * job.  A bit copy: the written bytes equal the input bytes.  One launch writes
 * K and V for all tokens.
 *
 *   k, v          [T][Hkv][D]   dtype, device
 *   slot_mapping  [T]           int64, device; < 0 means "skip this token"
 *   k_cache, v_cache            as in pa_decode, updated in place
 *
 * Device-side contract: slots are unique.  Slots >= N * bs are skipped, never
 * written.  Do not write into a block that several tables share (such a write
 * needs copy-on-write first, [CY] 多序列共享; [ASP] 实现要点).
 */
pa_status pa_cache_write(const void* k, const void* v, const int64_t* slot_mapping,
                         void* k_cache, void* v_cache, const pa_cache_write_ext* ext);

/* Shapes and options of a pa_multi_token call. */
typedef struct pa_multi_token_ext {
  int32_t num_seqs;           /* S >= 0 (0: nothing to do) and <= 65535               */
  int32_t num_tokens;         /* T = query_start[S] >= 0: rows of q and out            */
  int32_t max_query_len;      /* >= every n_s: sizes the launch (0: nothing to do)     */
  int32_t num_q_heads;        /* Hq > 0, a multiple of num_kv_heads                    */
  int32_t head_dim;           /* D: 64 or 128                                          */
  int32_t max_blocks_per_seq; /* row stride of block_tables, >= 1                      */
  int64_t num_blocks;         /* N, physical blocks in the pool, >= 1                  */
  int32_t partition_size;     /* context split: 0 = automatic, < 0 = never split,      */
                              /* > 0 = that many tokens per partition (multiple of 32) */
  int32_t dtype;              /* pa_dtype of q, k_cache, v_cache and out               */
  void* workspace;            /* device scratch for split partials, caller-owned;      */
                              /* unused (may be NULL) when the call does not split     */
  size_t workspace_bytes;     /* its size; see pa_multi_token_workspace_bytes          */
  void* stream;               /* hipStream_t                                           */
  int32_t max_seq_len;        /* 0, or a bound L_max >= every seq_lens[s], at most     */
                              /* max_blocks_per_seq * bs: the context split and its    */
                              /* workspace are sized from it instead of the table's    */
                              /* capacity (a serving step knows its longest sequence)  */
} pa_multi_token_ext;

/*
 * pa_multi_token - attention for several new tokens per sequence over the paged cache:
 * a prompt chunk of a sequence that joins the batch, or draft tokens to verify
 * ([ASP] 实现要点, continuous batching; 已知局限, speculative decoding).
 *
 * Sequence s has seq_lens[s] = L_s tokens in the cache, the last n_s of them new
 * (their K/V already stored, e.g. by pa_cache_write).  Its new tokens' queries are
 * rows query_start[s] .. query_start[s+1]-1 of q, n_s = query_start[s+1] -
 * query_start[s].  New token j (0-based) sits at position L_s - n_s + j and attends
 * to positions 0 .. L_s - n_s + j of the sequence: itself and everything before it,
 * nothing after (the decoder attention of the scaled dot-product definition the cache
 * serves, [ASP] 引用本概念的论文).  Per query head h (KV head h / (Hq / Hkv)):
 *   out[row][h] = softmax_t(scale * <q[row][h], K_t>) . V, t over those positions.
 * With every n_s = 1 this is pa_decode.
 *
 *   q, out        device, [T][Hq][D], dtype ext->dtype, 16-byte aligned
 *   k_cache       device, [N][Hkv][bs][D];  v_cache  device, [N][Hkv][D][bs]
 *   block_tables  device int32 [S][max_blocks_per_seq] (entries past a sequence's
 *                 last block are never read)
 *   seq_lens      device int32 [S]
 *   query_start   device int32 [S+1], query_start[0] = 0, non-decreasing,
 *                 query_start[S] = T
 *   block_size    4, 8, 16 or 32;  scale  finite
 *
 * Device-side contract (not checked on the host, which never reads device memory):
 * n_s <= max_query_len and n_s <= L_s <= L_max, table entries in use lie in [0, N),
 * where L_max = max_seq_len when it is set, else max_blocks_per_seq * bs.  A sequence
 * whose query_start entries do not fit in [0, T] is skipped; one with n_s > L_s or
 * L_s > L_max, or a bad table entry, gets NaN rows; rows past max_query_len are not
 * written.
 *
 * Context split.  With few (sequence, KV head, 128-row tile) triples, e.g. a few draft
 * tokens per sequence over long contexts, one workgroup per triple leaves most of the
 * device idle.  The call then cuts every sequence's positions into partitions of
 * part_tokens positions, computes each partition's rows (running maximum, running
 * sum, unnormalised output) into the workspace and combines them with log-sum-exp
 * weights in partition order in a second launch: deterministic, and equal to the
 * unsplit result up to fp32 rounding.  partition_size > 0 fixes part_tokens; 0 picks
 * it from the shapes alone (rows per tile, L_max, the number of triples): a split only
 * when there are fewer than 512 triples and partitions of at least max(256, 16 * rows
 * per tile) tokens, and then about 768 workgroups.  Partitions past a sequence's
 * length do no work, so the choice fits sequences near L_max: callers whose sequences
 * are much shorter than the table's capacity set max_seq_len (or partition_size).
 *
 * Workspace (ext->workspace, ext->workspace_bytes): device memory owned by the
 * caller, of at least pa_multi_token_workspace_bytes bytes when the call splits (0
 * otherwise: workspace may then be NULL).  Scratch only: no zero-fill is needed, and
 * calls of any shapes may share it as long as they are ordered on one stream (calls
 * that overlap on one workspace race).
 *
 * Asynchronous on ext->stream: one launch, or two when the call splits.  Errors:
 * PA_ERR_INVALID_ARG for NULL or misaligned pointers, bad shapes or dtype, a
 * non-finite scale, a partition_size that is not a multiple of 32; PA_ERR_WORKSPACE
 * for a split call whose workspace is missing or too small; PA_ERR_UNSUPPORTED for a
 * head_dim or block_size not built or a launch too large; PA_ERR_HIP if a launch
 * fails.
 */
pa_status pa_multi_token(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* query_start, int32_t block_size, int32_t num_kv_heads,
                         float scale, void* out, const pa_multi_token_ext* ext);

/*
 * pa_multi_token_workspace_bytes - bytes of workspace a pa_multi_token call with these
 * shapes needs: 0 when it does not split, else S * Hkv * tiles * parts * rows * (D + 2)
 * * 4, tiles = ceil(max_query_len * G / 128), rows = min(128, max_query_len * G),
 * parts = ceil(L_max / part_tokens).  Only the shape fields of ext
 * are read.  Returns PA_OK and sets *bytes, or the error status pa_multi_token would
 * report for the same shapes.
 */
pa_status pa_multi_token_workspace_bytes(const pa_multi_token_ext* ext, int32_t block_size,
                                         int32_t num_kv_heads, size_t* bytes);

/* Shapes of a pa_copy_blocks call. */
typedef struct pa_copy_blocks_ext {
  int32_t num_kv_heads; /* Hkv > 0                                   */
  int32_t head_dim;     /* D > 0, a multiple of 8                    */
  int32_t block_size;   /* bs: 4, 8, 16 or 32                        */
  int64_t num_blocks;   /* N >= 1                                    */
  int32_t dtype;        /* pa_dtype of the caches                    */
  void* stream;         /* hipStream_t                               */
} pa_copy_blocks_ext;

/*
 * pa_copy_blocks - copy whole physical blocks of both caches (copy-on-write).
 *
 * For every i < n, block dst[i] of k_cache and of v_cache becomes a bit copy of
 * block src[i]: every KV head and every slot.  A sequence about to write into a
 * block that other sequences share gets a private copy first ([CY] 多序列共享;
 * [ASP] 实现要点); pa_bm_append (pa_block_manager.h) names the copies to make.
 *
 *   k_cache, v_cache   device, layouts as in pa_decode
 *   src, dst           HOST int32 arrays [n], each entry in [0, N); src[i] != dst[i];
 *                      destinations distinct and none of them a source
 *
 * The index arrays are read during the call (copied into the launch arguments,
 * 128 pairs a launch), so the caller may reuse them as soon as it returns, and the
 * call needs no device memory of its own.  Asynchronous on ext->stream.
 *
 * Errors: PA_ERR_INVALID_ARG for a NULL ext or pointer (when n > 0), caches not
 * 16-byte aligned, bad shapes or dtype, an id outside [0, N), src[i] == dst[i], a
 * repeated destination or a destination that is also a source -- all found before
 * anything is launched; PA_ERR_UNSUPPORTED for a block size not built; PA_ERR_HIP
 * if a launch fails (launches before it may have run).  n == 0 does nothing.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                         int32_t n, const pa_copy_blocks_ext* ext);

/* Static text for a status code. */
const char* pa_status_string(pa_status status);

/* Reason for the last non-PA_OK status returned on the calling thread ("" if none).
 * The pointer stays valid until the next library call on this thread. */
const char* pa_last_error(void);

/* ABI version of this header: bumped on any incompatible change. */
int32_t pa_abi_version(void);

#define PA_ABI_VERSION 4  /* 2: pa_decode_ext.shared_blocks; 3: pa_cache_write_decode;
                              4: pa_multi_token_ext.max_seq_len */

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
