/*
 * pkv_block_manager.h - host-side block manager of libpkv, and the GPU block copy used
 * for copy-on-write.
 *
 * Sources (cited by page title and section):
 *   * "LLM 推理优化全景实战" (chenxutan.com) §2.2-§2.3: the KV cache is a shared pool of
 *     fixed-size physical blocks; each request owns a table from logical to physical
 *     blocks; blocks are allocated on demand while a request grows (write_kv allocates
 *     while the table is too short) and allocation fails when no block is free.
 *   * "09-inference-optimization" (LLM-Code-Hot-100), section PagedAttention: a free list
 *     of pages, a per-sequence page table, and freeing all of a sequence's pages when it
 *     ends.
 *   * "LLM推理与服务：面试问题与推荐回答" Q2 and Q15: physical blocks are shared between
 *     sequences (parallel sampling, beam search, common prefixes) until they diverge,
 *     with copy-on-write. The pages give no mechanism; here each block carries a
 *     reference count, and a write into a block whose count exceeds one first moves the
 *     writer to a fresh copy.
 *   * "推理机制动态图解（进阶）" demo 7: preemption by recompute frees a victim's blocks
 *     and later rebuilds its cache from scratch.
 *
 * Conventions:
 *   * A manager is an opaque host object. It is not thread-safe: one thread at a time.
 *   * Blocks never handed out are given in `free_order` (ascending when NULL); a freed
 *     block (reference count reaching zero) joins the back of the free list, after every
 *     never-used block (first in, first out).
 *   * Functions return PKV_OK (0) or a negative status (pkv.h codes plus those below); a
 *     failing call changes nothing (pkv_bm_append_slots: nothing beyond the items it
 *     reports as done).
 *   * Sequence ids are any int64 values chosen by the caller.
 */
#ifndef PKV_BLOCK_MANAGER_H
#define PKV_BLOCK_MANAGER_H

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

enum pkv_bm_status {
  PKV_ERR_OUT_OF_BLOCKS = -13,   /* not enough free blocks for the request */
  PKV_ERR_NO_SEQUENCE = -14,     /* unknown sequence id */
  PKV_ERR_SEQUENCE_EXISTS = -15, /* sequence id already in use */
  PKV_ERR_BAD_BLOCK = -16        /* block id outside [0, num_blocks) */
};

typedef struct pkv_block_manager pkv_block_manager;

/* A manager of num_blocks blocks of block_size tokens. free_order: NULL or a host array
 * holding a permutation of 0..num_blocks-1. Returns NULL on invalid arguments. */
pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size,
                                 const int32_t* free_order);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Register an empty sequence. */
int32_t pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id);

/* New sequence `child` sharing every block of `parent` (each block's count + 1). */
int32_t pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);

/* Drop a sequence; blocks whose count reaches zero return to the free list. */
int32_t pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id);

/* Make the table hold tokens 0..n_tokens-1, allocating blocks as needed (no copy). */
int32_t pkv_bm_grow(pkv_block_manager* bm, int64_t seq_id, int32_t n_tokens);

/* Reserve the slot of token `token_index`: grow the table to cover it, then, if its
 * block is shared, move this sequence to a fresh block (copy-on-write). Outputs the
 * physical block and the slot (token_index % block_size); *copy_src / *copy_dst receive
 * the block pair whose data the caller must copy (pkv_copy_blocks) before writing, or -1
 * when no copy is needed. Any output pointer may be NULL. */
int32_t pkv_bm_append_slot(pkv_block_manager* bm, int64_t seq_id, int32_t token_index,
                           int32_t* phys_block, int32_t* slot, int32_t* copy_src,
                           int32_t* copy_dst);

/* Batched pkv_bm_append_slot for one decode step: item i reserves token token_index[i]
 * of sequence seq_ids[i], in order. Outputs per item: phys_block[i], slot[i] and
 * copy_pairs[2i], copy_pairs[2i+1] (-1, -1 when no copy is needed); any output array may
 * be NULL. *n_done receives the number of items applied: all n on success; on a failure
 * at item i the items before i stay applied and the status of item i is returned. */
int32_t pkv_bm_append_slots(pkv_block_manager* bm, const int64_t* seq_ids,
                            const int32_t* token_index, int32_t n, int32_t* phys_block,
                            int32_t* slot, int32_t* copy_pairs, int32_t* n_done);

/* Free blocks left; reference count of one block (0 if free); table length of a
 * sequence. Negative status on error. */
int32_t pkv_bm_num_free(const pkv_block_manager* bm);
int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block);
int32_t pkv_bm_num_blocks_of(const pkv_block_manager* bm, int64_t seq_id);

/* Host table rows: out[i][0..max_blocks) = table of seq_ids[i], padded with -1.
 * PKV_ERR_SHAPE if a table is longer than max_blocks. */
int32_t pkv_bm_tables(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                      int32_t max_blocks, int32_t* out);

/* Host: group the sequences of a batch by the leading blocks their tables share, for
 * pkv_paged_decode_attention_shared_prefix. Source: "LLM推理与服务：面试问题与推荐回答"
 * Q2/Q3 (sequences with a common prefix hold the same physical blocks). tables: HOST int32
 * [num_seqs][max_blocks]; context_lens: HOST int32 [num_seqs]. Sequences whose first table
 * entry is the same block form a candidate set (in order of first appearance); a set of at
 * least min_members (>= 2) sequences becomes a group whose shared block count is the
 * longest run of leading entries equal in every member's table, cut so that each member
 * keeps its last token outside it; a set sharing no whole block forms no group.
 * Outputs: seq_group[num_seqs] (group id or -1), group_blocks[0 .. *n_groups) (caller
 * provides num_seqs entries), *n_groups, *max_group_size, *max_shared_blocks. */
int32_t pkv_find_shared_prefixes(const int32_t* tables, int32_t num_seqs, int32_t max_blocks,
                                 const int32_t* context_lens, int32_t block_size,
                                 int32_t min_members, int32_t* seq_group, int32_t* group_blocks,
                                 int32_t* n_groups, int32_t* max_group_size,
                                 int32_t* max_shared_blocks);

/* GPU: copy whole blocks in both pools, pool[dst] = pool[src] for every pair.
 * pairs: DEVICE int32 [n_pairs][2] (src, dst); pools as in pkv.h. Destinations must be
 * distinct and no destination may be a source of another pair. Pairs with an id outside
 * [0, num_blocks) are skipped. Source: the copy-on-write step named in
 * "LLM推理与服务：面试问题与推荐回答" Q2. */
int32_t pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int32_t n_pairs,
                        int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                        int32_t d_head, int32_t dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCK_MANAGER_H */
