/*
 * pkv.h - C ABI of libpkv: single-token decode attention over a paged KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (sources cited by page title and section):
 *
 *   * "LLM 推理优化全景实战" (chenxutan.com) §2.3: K and V live in two pools shaped
 *     [num_blocks, block_size, n_kv_heads, d_head]; each sequence owns a table that maps
 *     its logical block i to a physical block; token t sits in logical block
 *     t / block_size at slot t % block_size.
 *   * same page §2.4: decode attention for one query token gathers the sequence's
 *     blocks through its table, scores every cached token with q . k * scale, takes a
 *     softmax over the tokens and returns the probability-weighted sum of the V rows.
 *   * "09-inference-optimization" (LLM-Code-Hot-100), section "KV Cache": the new
 *     token's K/V enters the cache before attention is computed, the scale is
 *     1/sqrt(d_head), and a cache holds 2 * layers * batch * seq * kv_heads * d_head *
 *     dtype_bytes bytes.
 *   * "LLM推理与服务：面试问题与推荐回答" Q7 and "推理机制动态图解（进阶）" demo 1:
 *     grouped-query attention; query head h reads KV head h / (n_heads / n_kv_heads).
 *   * "推理机制动态图解（进阶）" demo 5: the softmax is taken online (running maximum,
 *     running sum, rescale on a new maximum, divide at the end); "Scaling Book 第 11 章"
 *     §11.8 (FlashDecoding): one long sequence is split over many compute units.
 *
 * Conventions shared by every entry point:
 *
 *   * Every pointer argument is DEVICE memory owned by the caller, except where stated.
 *     The library allocates nothing, frees nothing, keeps no state between calls and
 *     never synchronises: each call checks its arguments on the host, enqueues its
 *     kernels on `stream` and returns.
 *   * dtype is one of PKV_F32, PKV_F16, PKV_BF16; K, V, q, k_new, v_new and out share it.
 *     Arithmetic is fp32 (fp32 products and accumulation), with one exception: where
 *     the weighted sum of V runs on the matrix cores for 16 query columns at once
 *     (multi-query attention, the shared-prefix tasks and quantized caches, 16-bit
 *     dtypes), the softmax weights (and, for quantized caches, the dequantized V) are
 *     rounded to the dtype first, and the running sum uses the same rounded weights.
 *     Outputs are rounded to the dtype with round-to-nearest-even.
 *   * Supported shapes: block_size == 16, d_head in {64, 128}, 1 <= n_kv_heads <= 256,
 *     n_heads / n_kv_heads in {1, 2, 4, 8}. All device pointers must be 16-byte aligned.
 *   * Return value: PKV_OK (0) or a negative PKV_ERR_* code. Errors are found on the
 *     host before anything is enqueued (except PKV_ERR_LAUNCH). Device-side values
 *     (tables, lengths, positions) are not read by the host; a kernel that meets an
 *     out-of-range value never reads or writes out of bounds: kv_append skips that
 *     sequence, gather_kv skips that block, and paged_decode_attention writes NaN to
 *     every output of that sequence's affected heads.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pkv_dtype { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 };

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,        /* a required pointer is NULL */
  PKV_ERR_SHAPE = -2,       /* a size is non-positive or sizes disagree */
  PKV_ERR_DTYPE = -3,       /* dtype is not PKV_F32 / PKV_F16 / PKV_BF16 */
  PKV_ERR_HEAD_DIM = -4,    /* d_head is not 64 or 128 */
  PKV_ERR_BLOCK_SIZE = -5,  /* block_size is not 16 */
  PKV_ERR_GROUP = -6,       /* n_heads is not n_kv_heads * {1, 2, 4, 8} */
  PKV_ERR_CONTEXT = -7,     /* max_context_len < 1 or > max_blocks_per_seq * block_size */
  PKV_ERR_PARTITION = -8,   /* partition_tokens is negative or not a multiple of block_size */
  PKV_ERR_WORKSPACE = -9,   /* workspace is NULL or smaller than pkv_decode_workspace_bytes */
  PKV_ERR_LAUNCH = -10,     /* the HIP runtime rejected a kernel launch */
  PKV_ERR_ALIGN = -11,      /* a device pointer is not 16-byte aligned */
  PKV_ERR_ALIAS = -12,      /* out overlaps q, k_pool or v_pool */
  PKV_ERR_QUERIES = -17,    /* q_len < 1 or q_len * (n_heads / n_kv_heads) > 16 */
  PKV_ERR_SCRATCH = -18     /* the sizes need more than the static scratch's 32 MiB */
};

/*
 * pkv_kv_append - write each sequence's new token into its slot of the pools.
 *
 * Source: chenxutan §2.3 (write_kv: logical block t / block_size, offset
 * t % block_size, store K and V there); "09-inference-optimization" KV Cache (the write
 * precedes attention).
 *
 *   k_pool, v_pool  [num_blocks, block_size, n_kv_heads, d_head], dtype; written in place.
 *   k_new, v_new    [num_seqs, n_kv_heads, d_head], dtype; read only.
 *   block_tables    [num_seqs, max_blocks_per_seq] int32, row-major; entry i of row b is
 *                   the physical block holding sequence b's tokens 16*i .. 16*i+15.
 *   positions       [num_seqs] int32; positions[b] is the token index of the new token,
 *                   i.e. sequence b's context length before this step.
 *
 * The write is a byte copy (bit-exact). The table entry for the new token's block must
 * already be allocated by the caller; a sequence whose position or table entry is out of
 * range is skipped. Sequences must not share the slot they write (a shared block is
 * copied by the caller's block manager before the write). Enqueue this before
 * pkv_paged_decode_attention on the same stream so the new token is attended to.
 */
int32_t pkv_kv_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                      const int32_t* block_tables, const int32_t* positions,
                      int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                      int32_t block_size, int32_t n_kv_heads, int32_t d_head, int32_t dtype,
                      hipStream_t stream);

/*
 * pkv_kv_append_tokens - pkv_kv_append for n_tokens (1..16) consecutive new tokens per
 * sequence: token i of sequence b (k_new/v_new [num_seqs, n_tokens, n_kv_heads, d_head])
 * goes to position positions[b] + i. The blocks of every written position must be in the
 * table already. Same copy rule and error behaviour as pkv_kv_append.
 */
int32_t pkv_kv_append_tokens(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                             const int32_t* block_tables, const int32_t* positions,
                             int32_t num_seqs, int32_t n_tokens, int32_t max_blocks_per_seq,
                             int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                             int32_t d_head, int32_t dtype, hipStream_t stream);

/*
 * pkv_paged_decode_attention - one query token per sequence attends to its paged
 * context.
 *
 * Source: chenxutan §2.4 (gather through the page table, softmax(q K^T * scale) V);
 * "推理机制动态图解（进阶）" demo 5 (online softmax with deferred division);
 * "Scaling Book 第 11 章" §11.8 (split one sequence's KV across compute units).
 *
 *   out             [num_seqs, n_heads, d_head], dtype; written. Must not overlap q or
 *                   the pools.
 *   q               [num_seqs, n_heads, d_head], dtype.
 *   k_pool, v_pool  [num_blocks, block_size, n_kv_heads, d_head], dtype.
 *   block_tables    [num_seqs, max_blocks_per_seq] int32, row-major.
 *   context_lens    [num_seqs] int32; context_lens[b] = N_b, the number of tokens sequence
 *                   b attends to, INCLUDING the token just appended (1 <= N_b <=
 *                   max_context_len). A sequence with N_b outside that range, or whose
 *                   table holds an entry outside [0, num_blocks) among its first
 *                   ceil(N_b / 16) entries, gets NaN outputs.
 *   max_context_len host-side upper bound of context_lens; sizes the launch grid.
 *   scale           score multiplier, normally 1/sqrt(d_head).
 *   partition_tokens 0 (default): balanced split. The list of (KV-head group, sequence,
 *                   16-token block) units is cut into equal contiguous shares, one per
 *                   resident workgroup of the GPU, so every compute unit streams the same
 *                   number of KV bytes whatever the mix of context lengths; a sequence cut
 *                   between workgroups is finished by a merge kernel. Used when
 *                   max_context_len > 512 and num_seqs <= 4096; otherwise 0 selects fixed
 *                   512-token partitions (a single kernel when max_context_len <= 512).
 *                   > 0: fixed partitions of that many tokens (a multiple of 16); a sequence
 *                   longer than one partition is processed by several workgroups whose
 *                   partial results the merge kernel combines.
 *   workspace       device scratch of at least pkv_decode_workspace_bytes(...) bytes
 *                   (may be NULL when that size is 0); its contents on entry do not
 *                   matter and on return are unspecified.
 *
 * Query head h uses KV head h / (n_heads / n_kv_heads). Results do not depend on the
 * physical placement of blocks (bitwise), and are deterministic (no atomics).
 */
int32_t pkv_paged_decode_attention(void* out, const void* q, const void* k_pool,
                                   const void* v_pool, const int32_t* block_tables,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t max_blocks_per_seq, int32_t num_blocks,
                                   int32_t max_context_len, int32_t block_size,
                                   int32_t n_heads, int32_t n_kv_heads, int32_t d_head,
                                   float scale, int32_t partition_tokens, int32_t dtype,
                                   void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * pkv_paged_decode_step - pkv_kv_append followed by pkv_paged_decode_attention, in one
 * launch. Source: the new token's K/V enter the cache before attention
 * ("09-inference-optimization", KV Cache; "LLM 推理优化全景实战" §2.3 write_kv).
 * The appended token of sequence b is token context_lens[b] - 1 (positions are implied);
 * k_new, v_new [num_seqs, n_kv_heads, d_head] in dtype. The wave that attends over the
 * block holding that token takes the token's K/V straight from k_new / v_new and writes
 * them into the pool slot, so the pools afterwards equal those of the two separate calls
 * and `out` equals their result (same arithmetic). Sequences whose length is invalid get
 * NaN outputs and no append; a table entry outside the pool skips the write (NaN output).
 * k_pool, v_pool are written; the other arguments are those of pkv_paged_decode_attention
 * (workspace size from pkv_decode_workspace_bytes).
 */
int32_t pkv_paged_decode_step(void* out, const void* q, void* k_pool, void* v_pool,
                              const void* k_new, const void* v_new, const int32_t* block_tables,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_blocks_per_seq, int32_t num_blocks,
                              int32_t max_context_len, int32_t block_size, int32_t n_heads,
                              int32_t n_kv_heads, int32_t d_head, float scale,
                              int32_t partition_tokens, int32_t dtype, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_paged_decode_step_noalloc - pkv_paged_decode_step without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Its partial-result records live in a static
 * device array of the library (32 MiB, one copy per device, held from the first call on a
 * device until the process ends); the call itself allocates nothing.
 *
 * Arguments, outputs and errors as pkv_paged_decode_step, plus PKV_ERR_SCRATCH when the
 * sizes need more workspace than 32 MiB (pkv_decode_workspace_bytes(num_seqs, n_heads,
 * n_kv_heads, d_head, max_context_len, partition_tokens) > 32 MiB; for example 128
 * sequences of 32 / 8 heads, d_head 128, need 19 MB), found on the host before anything is
 * enqueued. The scratch needs no clearing: every record is written before it is read
 * within a call, and its contents between calls do not matter. All calls on one device
 * share its scratch, so calls that overlap in time on one device (different streams, or
 * host threads without ordering) race and give wrong results; serialise them (one stream).
 */
int32_t pkv_paged_decode_step_noalloc(void* out, const void* q, void* k_pool, void* v_pool,
                                      const void* k_new, const void* v_new,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t max_blocks_per_seq,
                                      int32_t num_blocks, int32_t max_context_len,
                                      int32_t block_size, int32_t n_heads, int32_t n_kv_heads,
                                      int32_t d_head, float scale, int32_t partition_tokens,
                                      int32_t dtype, hipStream_t stream);

/*
 * pkv_decode_workspace_bytes - scratch bytes pkv_paged_decode_attention needs for these
 * sizes (host only, no device call). 0 when no partial results are needed (fixed
 * partitions with every sequence in one partition). Returns 0 for invalid sizes as well;
 * pkv_paged_decode_attention then reports the invalid argument.
 *
 * Contents: fp32 partial-result records (running maximum, running sum, unnormalised
 * output of d_head values) and, in the balanced split, num_seqs + 1 int32 block prefix
 * sums. Fixed partitions hold num_seqs * n_heads * ceil(max_context_len /
 * partition_tokens) records; the balanced split at most (1024 + ceil(n_kv_heads / NW) *
 * num_seqs) * NW * (n_heads / n_kv_heads) records, NW = 8 if n_kv_heads is a multiple of
 * 8, else 4.
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t n_heads, int32_t n_kv_heads,
                                  int32_t d_head, int32_t max_context_len,
                                  int32_t partition_tokens);

/*
 * pkv_decode_split_workgroups - the grid of the balanced split on the current device: the
 * number of workgroups the decode kernel selected by these arguments launches, i.e. the
 * device's compute units times that kernel's own resident workgroups per compute unit
 * (kernels differ in registers and LDS, hence in occupancy), capped at 1024. The figure is
 * queried from the runtime once per kernel and device, then reused. fused_append != 0
 * selects the kernels of pkv_paged_decode_step / pkv_paged_multi_query_step; kv_format 0
 * the dtype pools, PKV_KV_INT8 / PKV_KV_FP8 (q_len 1, no fused append, dtype 16-bit) the
 * quantized kernels. The shared-prefix decode's split pass uses the kernel of q_len 1,
 * kv_format 0, no fused append. Host call (device attributes only, nothing is launched).
 * Returns the workgroup count (> 0) or a negative status: PKV_ERR_DTYPE, PKV_ERR_HEAD_DIM,
 * PKV_ERR_SHAPE, PKV_ERR_GROUP, PKV_ERR_QUERIES; PKV_ERR_LAUNCH if the runtime query fails.
 */
int32_t pkv_decode_split_workgroups(int32_t n_heads, int32_t n_kv_heads, int32_t d_head,
                                    int32_t q_len, int32_t dtype, int32_t kv_format,
                                    int32_t fused_append);

/*
 * pkv_paged_multi_query_attention - q_len new query tokens per sequence attend to the
 * paged context under a causal mask (speculative verification of q_len drafted tokens,
 * or a short chunk of new tokens).
 *
 * Source: "09-inference-optimization" KV Cache (with seq_len > 1 new tokens, key k is
 * hidden from new query i when k > K - seq_len + i, K counting all cached tokens);
 * "LLM推理与服务：面试问题与推荐回答" Q9 and "Scaling Book 第 11 章" §11.7 (the target model
 * checks all drafted tokens in one pass).
 *
 *   out, q          [num_seqs, q_len, n_heads, d_head], dtype.
 *   context_lens    N_b, INCLUDING the q_len new tokens (append them first, e.g. with
 *                   pkv_kv_append_tokens); new query i sees tokens 0 .. N_b - q_len + i.
 *                   q_len <= N_b <= max_context_len, else NaN outputs for that sequence.
 *   q_len           1 .. 16 / (n_heads / n_kv_heads).
 * Everything else as pkv_paged_decode_attention (q_len = 1 gives exactly its result);
 * workspace size from pkv_multi_query_workspace_bytes.
 */
int32_t pkv_paged_multi_query_attention(void* out, const void* q, const void* k_pool,
                                        const void* v_pool, const int32_t* block_tables,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t q_len, int32_t max_blocks_per_seq,
                                        int32_t num_blocks, int32_t max_context_len,
                                        int32_t block_size, int32_t n_heads, int32_t n_kv_heads,
                                        int32_t d_head, float scale, int32_t partition_tokens,
                                        int32_t dtype, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* Scratch bytes of pkv_paged_multi_query_attention (host only); the records of
 * pkv_decode_workspace_bytes times q_len. 0 for invalid sizes. */
size_t pkv_multi_query_workspace_bytes(int32_t num_seqs, int32_t q_len, int32_t n_heads,
                                       int32_t n_kv_heads, int32_t d_head,
                                       int32_t max_context_len, int32_t partition_tokens);

/*
 * pkv_paged_multi_query_step - pkv_kv_append_tokens followed by
 * pkv_paged_multi_query_attention, in one launch. Source: the q_len new tokens' K/V enter
 * the cache before they are attended to ("09-inference-optimization", KV Cache, with
 * seq_len > 1 new tokens; "LLM推理与服务：面试问题与推荐回答" Q9 speculative verification).
 * The appended tokens of sequence b are tokens context_lens[b] - q_len .. context_lens[b] - 1
 * (positions are implied); k_new, v_new [num_seqs, q_len, n_kv_heads, d_head] in dtype, row
 * i being token context_lens[b] - q_len + i. The waves that attend over the blocks holding
 * those tokens take their K/V straight from k_new / v_new and write them into the pool
 * slots, so the pools afterwards equal those of the two separate calls and `out` equals
 * their result (same arithmetic); q_len = 1 is pkv_paged_decode_step. Sequences whose
 * length is invalid get NaN outputs and no append; a table entry outside the pool skips the
 * writes into that block (NaN output). k_pool, v_pool are written; the other arguments are
 * those of pkv_paged_multi_query_attention (workspace size from
 * pkv_multi_query_workspace_bytes).
 */
int32_t pkv_paged_multi_query_step(void* out, const void* q, void* k_pool, void* v_pool,
                                   const void* k_new, const void* v_new,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   int32_t num_seqs, int32_t q_len, int32_t max_blocks_per_seq,
                                   int32_t num_blocks, int32_t max_context_len,
                                   int32_t block_size, int32_t n_heads, int32_t n_kv_heads,
                                   int32_t d_head, float scale, int32_t partition_tokens,
                                   int32_t dtype, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * pkv_paged_decode_attention_shared_prefix - pkv_paged_decode_attention for a batch in
 * which groups of sequences share the first blocks of their tables (a common prompt,
 * parallel sampling, beam search), reading every shared block once per group.
 *
 * Source: "LLM推理与服务：面试问题与推荐回答" Q2 and Q3 (sequences share physical blocks of a
 * common prefix, stored once); "Scaling Book 第 11 章" §11.3-§11.4 (prefix caching).
 * The attention computed is exactly that of pkv_paged_decode_attention; the grouping only
 * changes how the shared blocks are read. One kernel streams everything: its first
 * workgroups each take one prefix task (a 512-token partition of a group's shared blocks,
 * read once and scored against the queries of all members, up to 64 (member, head)
 * columns per KV head) and fewer of the sequences' own blocks, which the balanced split
 * hands to every workgroup; a merge kernel then combines the two kinds of records.
 *
 *   seq_group        [num_seqs] int32 device: group of each sequence in [0, n_groups), or
 *                    -1 for none.
 *   group_blocks     [n_groups] int32 device: number of leading table entries every member
 *                    of the group shares (whole blocks; 0 = nothing shared). The shared
 *                    blocks are read through the table of the group's first member (lowest
 *                    sequence index). NaN outputs mark broken promises: a member whose
 *                    table differs from the first member's inside the shared run, or whose
 *                    context ends inside it (the new token is never in a shared block);
 *                    every member of a group that shares blocks and has more than
 *                    max_group_size members, or more than max_shared_blocks (or
 *                    max_blocks_per_seq) shared blocks.
 *   max_group_size   host bound on members per group (sizes the prefix tasks).
 *   max_shared_blocks host bound on group_blocks (sizes the prefix records).
 * Other arguments as pkv_paged_decode_attention (balanced split, num_seqs <= 4096);
 * workspace size from pkv_shared_prefix_workspace_bytes.
 */
int32_t pkv_paged_decode_attention_shared_prefix(
    void* out, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_group,
    const int32_t* group_blocks, int32_t n_groups, int32_t max_group_size,
    int32_t max_shared_blocks, int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
    int32_t max_context_len, int32_t block_size, int32_t n_heads, int32_t n_kv_heads,
    int32_t d_head, float scale, int32_t dtype, void* workspace, size_t workspace_bytes,
    hipStream_t stream);

/* Scratch bytes of pkv_paged_decode_attention_shared_prefix (host only); 0 for invalid
 * sizes. */
size_t pkv_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t n_heads, int32_t n_kv_heads,
                                         int32_t d_head, int32_t max_shared_blocks);

/*
 * Quantized KV cache (8-bit codes). Source: "LLM 推理优化全景实战" §4.1, the affine
 * quantizer Q(x) = round(x / s) + z with dequantization x^ = s * (Q - z); "Scaling Book
 * 第 11 章" names FP8 and INT8 as the 8-bit choices.
 *
 *   kv_format PKV_KV_INT8: unsigned codes 0..255; per (token, KV head) the row's range is
 *       widened to include zero, lo = min(min x, 0), hi = max(max x, 0);
 *       s = (hi - lo) / 255 (1 when zero), z = clamp(round(-lo / s), 0, 255),
 *       Q = clamp(round(x / s) + z, 0, 255).
 *   kv_format PKV_KV_FP8: OCP E4M3 codes (bias 7, 3 mantissa bits, largest 448, no
 *       infinities); s = max|x| / 448 (1 when zero), z = 0, Q = E4M3(x / s) rounded to
 *       nearest even and saturated at +-448.
 *   Every quantizer step is binary32 and round() is round-half-to-even, so the codes and
 *   (s, z) are determined bit for bit by the input row.
 *   Code pools:  [num_blocks, block_size, n_kv_heads, d_head] uint8 (the layout of the
 *                dtype pools with 1-byte elements).
 *   Scale pools: [num_blocks, n_kv_heads, block_size, 2] float (s, z) per token slot.
 */
enum pkv_kv_format {
  PKV_KV_INT8 = 1,
  PKV_KV_FP8 = 2
};

/*
 * pkv_kv_append_quantized - quantize each sequence's new K and V (one token at
 * positions[b], as pkv_kv_append) into its slot of the code pools and its (s, z) into the
 * scale pools. k_new, v_new [num_seqs, n_kv_heads, d_head] in dtype (f32, f16 or bf16).
 * Sequences with an out-of-range position or table entry are skipped.
 */
int32_t pkv_kv_append_quantized(void* k_codes, void* v_codes, float* k_scales, float* v_scales,
                                const void* k_new, const void* v_new,
                                const int32_t* block_tables, const int32_t* positions,
                                int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                                int32_t block_size, int32_t n_kv_heads, int32_t d_head,
                                int32_t dtype, int32_t kv_format, hipStream_t stream);

/*
 * pkv_paged_decode_attention_quantized - pkv_paged_decode_attention over a quantized cache:
 * the attention of the dequantized K and V, x^ = s * (Q - z). q and out in dtype
 * (PKV_F16 or PKV_BF16). The scores contract q with the raw codes on the matrix cores and
 * apply s and z once per token, s (q.Q - z sum q), which equals q.x^ up to fp32 rounding;
 * the weighted sum of V uses the dequantized values rounded to dtype (see the precision
 * note at the top). Workspace size: pkv_decode_workspace_bytes (same arguments).
 */
int32_t pkv_paged_decode_attention_quantized(
    void* out, const void* q, const void* k_codes, const void* v_codes, const float* k_scales,
    const float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
    int32_t block_size, int32_t n_heads, int32_t n_kv_heads, int32_t d_head, float scale,
    int32_t partition_tokens, int32_t dtype, int32_t kv_format, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * pkv_stream_read - measurement utility: read `bytes` (a multiple of 16) of the device
 * buffer `buf` once with 16-byte non-temporal loads, the plain streaming read whose rate
 * is the achievable HBM ceiling for the decode kernels. Each of the workgroups * 256
 * threads writes the XOR of the 32-bit words it read to sink[thread] (device, at least
 * workgroups * 256 words; PKV_ERR_WORKSPACE otherwise). workgroups = 0 picks 8 per
 * compute unit. Nothing else is written.
 */
int32_t pkv_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                        int32_t workgroups, hipStream_t stream);

/*
 * pkv_kv_bytes_per_token - bytes one token occupies in the KV cache of a whole model:
 * 2 * n_layers * n_kv_heads * d_head * dtype_bytes (host only).
 *
 * Source: "09-inference-optimization" KV Cache (the size formula at batch = seq = 1);
 * "LLM推理与服务：面试问题与推荐回答" Q1 (about 0.5 MB for 32 layers x 32 heads x 128, fp16).
 * Returns -1 if an argument is negative.
 */
int64_t pkv_kv_bytes_per_token(int32_t n_layers, int32_t n_kv_heads, int32_t d_head,
                               int32_t dtype_bytes);

/*
 * pkv_gather_kv - copy each sequence's cached tokens into contiguous arrays (test and
 * inspection use; not on the decode path).
 *
 * Source: chenxutan §2.3 read_kv (the same slot rule as the append) and
 * "09-inference-optimization" PagedAttention get_kv (only used slots).
 *
 *   k_out, v_out    [num_seqs, max_context_len, n_kv_heads, d_head], dtype; row t of
 *                   sequence b is written for t < min(context_lens[b], max_context_len);
 *                   the rest is left untouched.
 * Other arguments as for pkv_paged_decode_attention. Blocks whose table entry is out of
 * range are skipped. Bit-exact copy.
 */
int32_t pkv_gather_kv(void* k_out, void* v_out, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* context_lens,
                      int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                      int32_t max_context_len, int32_t block_size, int32_t n_kv_heads,
                      int32_t d_head, int32_t dtype, hipStream_t stream);

/* pkv_status_str - static, NUL-terminated description of a status code (host only). */
const char* pkv_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
