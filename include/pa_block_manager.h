/*
 * pa_block_manager.h - host-side KV block manager for libpa.so (C ABI).
 *
 * The bookkeeping in front of the decode hot path: it decides which physical
 * block every token of every sequence lives in, and produces exactly the inputs
 * pa_cache_write and pa_decode take (slot ids, block tables, lengths) plus the
 * block copies a copy-on-write needs (pa_copy_blocks in pa.h).
 *
 * Pages cited (title, site):
 *   [AB]  "什么是分页注意力（PagedAttention）？"                     aiboss88.com wiki
 *   [CY]  "深入解析 PagedAttention：vLLM 显存优化的核心魔法"            cygnushan.xyz blog
 *   [ASP] "PagedAttention"                                          awesome-system-papers
 *   [RK]  "什么是 LLM 中的分页注意力(Paged Attention)?它是如何工作的?"  news.rkmt.cn
 *
 * What it does:
 *   - The pool has num_blocks physical blocks of block_size token slots; any free
 *     block can serve any sequence ([ASP] 核心思想: no external fragmentation).
 *     Free blocks are handed out in first-in first-out order; the initial order
 *     can be given (default 0, 1, 2, ...), and freed blocks go to the back.
 *   - Each sequence has a block table: logical block j -> physical block ([RK] 块表).
 *     A token is appended into the next free slot of the sequence's last block;
 *     a new block is taken only when the last one is full (or the sequence has
 *     none) ([RK] 分页注意力是如何工作的; [AB] 工作机制).
 *   - Blocks carry reference counts.  Forking a sequence (parallel sampling, beam
 *     search) gives the child the parent's table and adds one reference to every
 *     block; freeing a sequence drops one reference from each of its blocks, and a
 *     block whose count reaches zero returns to the free list ([CY] 多序列共享;
 *     [ASP] 实现要点).
 *   - Copy-on-write: appending to a sequence whose last block is shared and only
 *     partly filled would write into a block other sequences read, so the manager
 *     first takes a fresh block, records a (source, destination) copy for the
 *     caller to perform before the cache write, moves the sequence to the copy and
 *     drops its reference on the original ([CY] 多序列共享; [ASP] 实现要点).
 *
 * Conventions: host memory only, no GPU calls; every pointer is caller-owned and
 * not kept.  A manager is not thread-safe: calls on one manager must not overlap.
 * Errors return a pa_status (see pa.h) with the reason in pa_last_error(); a call
 * that fails changes nothing.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* num_blocks >= 1, block_size >= 1, max_blocks_per_seq >= 1 (the row length of the
 * block tables it exports).  free_order: NULL for 0 .. num_blocks-1, or a
 * permutation of 0 .. num_blocks-1 giving the order blocks are first handed out. */
pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                       const int32_t* free_order, pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* A new, empty sequence; its id is >= 0 and never reused. */
pa_status pa_bm_add_sequence(pa_block_manager* bm, int32_t* seq_out);

/* A new sequence sharing all of parent's tokens and blocks. */
pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child_out);

/* Drop a sequence; blocks no other sequence references become free. */
pa_status pa_bm_free_sequence(pa_block_manager* bm, int32_t seq);

/*
 * Append one token to each of seqs[0 .. n-1] (distinct sequences), in order.
 *   slot_mapping[i]  slot id (phys * block_size + offset) of seqs[i]'s new token
 *   copy_src/dst     copy-on-write block copies, *n_copies of them (at most n);
 *                    perform them (pa_copy_blocks) before writing the new tokens.
 * Fails with PA_ERR_CAPACITY (nothing changed) if the free list runs out or a
 * table would exceed max_blocks_per_seq.
 */
pa_status pa_bm_append(pa_block_manager* bm, const int32_t* seqs, int32_t n,
                       int64_t* slot_mapping, int32_t* copy_src, int32_t* copy_dst,
                       int32_t* n_copies);

/* Tokens in a sequence (its seq_lens entry). */
pa_status pa_bm_length(const pa_block_manager* bm, int32_t seq, int32_t* len);

/* Block tables and lengths of seqs[0 .. n-1], rows of max_blocks_per_seq entries
 * padded with -1 ([CY] 核心思想, the tables' unused entries). */
pa_status pa_bm_export(const pa_block_manager* bm, const int32_t* seqs, int32_t n,
                       int32_t* block_tables, int32_t* seq_lens);

/* Free blocks, and the reference count of one block. */
int64_t pa_bm_free_blocks(const pa_block_manager* bm);
pa_status pa_bm_ref_count(const pa_block_manager* bm, int32_t block, int32_t* count);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
