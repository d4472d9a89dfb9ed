// C ABI of libpkv: host-side argument checks, workspace sizing and kernel dispatch (host
// C++; the kernels are behind the launchers of pkv_internal.h). The operations and their
// sources are documented in include/pkv.h and include/pkv_block_manager.h.

#include "../../include/pkv.h"
#include "../../include/pkv_block_manager.h"

#include <algorithm>
#include <cmath>

#include "pkv_internal.h"
#include "pkv_scratch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16:
    case PKV_BF16: return 2;
    default: return 0;
  }
}

bool valid_group(int32_t n_heads, int32_t n_kv_heads) {
  if (n_kv_heads <= 0 || n_heads <= 0 || n_heads % n_kv_heads) return false;
  const int32_t g = n_heads / n_kv_heads;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// How a decode call splits its work, and the workspace that needs.
struct Plan {
  bool split;            // balanced split over the GPU
  int32_t partition;     // fixed mode: tokens per partition
  int64_t parts;         // fixed mode: partitions of the longest sequence
  size_t records;        // partial-result records the workspace must hold
  size_t prefix_ints;    // split mode: block prefix sums
  size_t shared_records; // shared-prefix task records
  int32_t prefix_parts;  // shared-prefix task partitions
  size_t flag_ints;      // shared-prefix member flags
  size_t bytes;          // total workspace bytes
};

Plan make_plan(int32_t num_seqs, int32_t q_len, int32_t n_heads, int32_t n_kv_heads,
               int32_t d_head, int32_t max_context_len, int32_t partition_tokens,
               int32_t max_shared_blocks = -1) {
  Plan p{};
  if (max_shared_blocks >= 0) {          // shared-prefix decode: always the balanced split
    const int64_t nw = pkv::max_waves_per_workgroup(n_kv_heads);
    const int64_t hg = (n_kv_heads + nw - 1) / nw;
    const int64_t g = n_heads / n_kv_heads;
    p.split = true;
    p.records = (size_t)((pkv::kSplitMaxWorkgroups + hg * num_seqs) * nw * g);
    p.prefix_ints = (size_t)num_seqs + 1;
    p.prefix_parts = (int32_t)std::max<int64_t>(
        1, ((int64_t)max_shared_blocks * pkv::kBlockTokens + pkv::kPrefixPartition - 1) /
               pkv::kPrefixPartition);
    p.shared_records = (size_t)num_seqs * n_heads * p.prefix_parts;
    p.flag_ints = (size_t)num_seqs * p.prefix_parts;
    p.bytes = align256(p.prefix_ints * sizeof(int32_t)) + 2 * align256(p.records * sizeof(float)) +
              align256(p.records * d_head * sizeof(float)) +
              2 * align256(p.shared_records * sizeof(float)) +
              align256(p.shared_records * d_head * sizeof(float)) +
              align256(p.flag_ints * sizeof(int32_t));
    return p;
  }
  // 0 selects the balanced split, except when every sequence fits one 512-token partition
  // (one kernel, no merge) or there are more sequences than the split mode holds.
  p.split = partition_tokens == 0 && num_seqs <= pkv::kSplitMaxSeqs &&
            max_context_len > pkv::kFallbackPartition;
  if (p.split) {
    const int64_t nw = pkv::max_waves_per_workgroup(n_kv_heads);
    const int64_t hg = (n_kv_heads + nw - 1) / nw;
    const int64_t g = n_heads / n_kv_heads;
    p.records = (size_t)((pkv::kSplitMaxWorkgroups + hg * num_seqs) * nw * g * q_len);
    p.prefix_ints = (size_t)num_seqs + 1;
  } else {
    p.partition = partition_tokens == 0 ? pkv::kFallbackPartition : partition_tokens;
    p.parts = ((int64_t)max_context_len + p.partition - 1) / p.partition;
    p.records = p.parts > 1 ? (size_t)num_seqs * q_len * n_heads * (size_t)p.parts : 0;
  }
  if (p.records > 0)
    p.bytes = align256(p.prefix_ints * sizeof(int32_t)) + 2 * align256(p.records * sizeof(float)) +
              align256(p.records * d_head * sizeof(float));
  return p;
}

// Byte ranges [a, a + na) and [b, b + nb) overlap.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Checks shared by decode and gather.
int32_t check_pool_args(int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                        int32_t max_context_len, int32_t block_size, int32_t n_kv_heads,
                        int32_t d_head, int32_t dtype) {
  if (elem_bytes(dtype) == 0) return PKV_ERR_DTYPE;
  if (block_size != pkv::kBlockTokens) return PKV_ERR_BLOCK_SIZE;
  if (d_head != 64 && d_head != 128) return PKV_ERR_HEAD_DIM;
  if (num_seqs <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || n_kv_heads <= 0 ||
      n_kv_heads > pkv::kMaxKvHeads)
    return PKV_ERR_SHAPE;
  if (num_seqs > 65535) return PKV_ERR_SHAPE;   // grid z / y limit
  if (max_context_len < 1 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return PKV_ERR_CONTEXT;
  return PKV_OK;
}

bool valid_q_len(int32_t q_len, int32_t n_heads, int32_t n_kv_heads) {
  return q_len >= 1 && n_kv_heads > 0 && q_len * (n_heads / n_kv_heads) <= 16;
}

// Shared by the single- and multi-query entry points.
// kv_format 0: K/V pools in dtype; PKV_KV_INT8 / PKV_KV_FP8: 8-bit code pools with the
// (s, z) pools k_scales / v_scales (q and out in dtype, which must be 16-bit).
int32_t decode_impl(void* out, const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                    int32_t q_len, int32_t max_blocks_per_seq, int32_t num_blocks,
                    int32_t max_context_len, int32_t block_size, int32_t n_heads,
                    int32_t n_kv_heads, int32_t d_head, float scale, int32_t partition_tokens,
                    int32_t dtype, void* workspace, size_t workspace_bytes, hipStream_t stream,
                    int32_t kv_format = 0, const float* k_scales = nullptr,
                    const float* v_scales = nullptr, const void* k_new = nullptr,
                    const void* v_new = nullptr, bool fused_append = false,
                    bool static_scratch = false) {
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PKV_ERR_NULL;
  if (fused_append && (!k_new || !v_new)) return PKV_ERR_NULL;
  if (kv_format != 0 && (!k_scales || !v_scales)) return PKV_ERR_NULL;
  int32_t st = check_pool_args(num_seqs, max_blocks_per_seq, num_blocks, max_context_len,
                               block_size, n_kv_heads, d_head, dtype);
  if (st != PKV_OK) return st;
  if (kv_format != 0 && ((kv_format != PKV_KV_INT8 && kv_format != PKV_KV_FP8) ||
                         dtype == PKV_F32 || q_len != 1))
    return PKV_ERR_DTYPE;
  if (kv_format != 0 && (!aligned16(k_scales) || !aligned16(v_scales))) return PKV_ERR_ALIGN;
  if (!valid_group(n_heads, n_kv_heads)) return PKV_ERR_GROUP;
  if (!valid_q_len(q_len, n_heads, n_kv_heads)) return PKV_ERR_QUERIES;
  if (max_context_len < q_len) return PKV_ERR_CONTEXT;
  if (!std::isfinite(scale)) return PKV_ERR_SHAPE;
  if (partition_tokens < 0 || partition_tokens % pkv::kBlockTokens) return PKV_ERR_PARTITION;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return PKV_ERR_ALIGN;
  if (fused_append && (!aligned16(k_new) || !aligned16(v_new))) return PKV_ERR_ALIGN;
  const size_t eb = (size_t)elem_bytes(dtype);
  const size_t out_bytes = (size_t)num_seqs * q_len * n_heads * d_head * eb;
  const size_t pool_bytes =
      (size_t)num_blocks * pkv::kBlockTokens * n_kv_heads * d_head * (kv_format ? 1 : eb);
  const size_t scale_bytes = (size_t)num_blocks * pkv::kBlockTokens * n_kv_heads * 2 * sizeof(float);
  if (overlaps(out, out_bytes, q, out_bytes) || overlaps(out, out_bytes, k_pool, pool_bytes) ||
      overlaps(out, out_bytes, v_pool, pool_bytes))
    return PKV_ERR_ALIAS;
  if (kv_format != 0 && (overlaps(out, out_bytes, k_scales, scale_bytes) ||
                         overlaps(out, out_bytes, v_scales, scale_bytes)))
    return PKV_ERR_ALIAS;
  if (fused_append) {
    const size_t new_bytes = (size_t)num_seqs * q_len * n_kv_heads * d_head * eb;
    if (overlaps(out, out_bytes, k_new, new_bytes) || overlaps(out, out_bytes, v_new, new_bytes) ||
        overlaps(k_new, new_bytes, k_pool, pool_bytes) || overlaps(k_new, new_bytes, v_pool, pool_bytes) ||
        overlaps(v_new, new_bytes, k_pool, pool_bytes) || overlaps(v_new, new_bytes, v_pool, pool_bytes) ||
        overlaps(k_pool, pool_bytes, v_pool, pool_bytes))
      return PKV_ERR_ALIAS;
  }

  const Plan plan = make_plan(num_seqs, q_len, n_heads, n_kv_heads, d_head, max_context_len,
                              partition_tokens);
  if (!plan.split && plan.parts > 65535) return PKV_ERR_PARTITION;   // grid y limit
  if (static_scratch && plan.bytes > 0) {     // the library's static scratch, every check done
    if (plan.bytes > pkv::kScratchBytes) return PKV_ERR_SCRATCH;
    workspace = pkv::scratch_region();
    workspace_bytes = pkv::kScratchBytes;
    if (!workspace) return PKV_ERR_LAUNCH;
  }
  if (plan.bytes > 0 && (!workspace || workspace_bytes < plan.bytes || !aligned16(workspace)))
    return PKV_ERR_WORKSPACE;

  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = static_cast<const char*>(k_pool);
  a.v_pool = static_cast<const char*>(v_pool);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.n_heads = n_heads;
  a.n_kv_heads = n_kv_heads;
  a.q_len = q_len;
  a.split = plan.split ? 1 : 0;
  a.partition_tokens = plan.partition;
  a.max_partitions = (int32_t)plan.parts;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);   // log2(e)
  if (plan.bytes > 0) {
    char* ws = static_cast<char*>(workspace);
    const size_t pre = align256(plan.prefix_ints * sizeof(int32_t));
    const size_t vec = align256(plan.records * sizeof(float));
    a.ws_prefix = plan.prefix_ints ? reinterpret_cast<int32_t*>(ws) : nullptr;
    a.ws_m = reinterpret_cast<float*>(ws + pre);
    a.ws_l = reinterpret_cast<float*>(ws + pre + vec);
    a.ws_o = reinterpret_cast<float*>(ws + pre + 2 * vec);
  }
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.k_new = fused_append ? static_cast<const char*>(k_new) : nullptr;
  a.v_new = fused_append ? static_cast<const char*>(v_new) : nullptr;
  const hipError_t e =
      kv_format ? pkv::launch_decode_quantized(a, dtype, kv_format, d_head, n_heads / n_kv_heads,
                                               stream)
                : pkv::launch_decode(a, dtype, d_head, n_heads / n_kv_heads, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}


}  // namespace

extern "C" {

const char* pkv_status_str(int32_t status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "a size is non-positive or sizes disagree";
    case PKV_ERR_DTYPE: return "unsupported dtype (expected PKV_F32, PKV_F16 or PKV_BF16)";
    case PKV_ERR_HEAD_DIM: return "unsupported d_head (expected 64 or 128)";
    case PKV_ERR_BLOCK_SIZE: return "unsupported block_size (expected 16)";
    case PKV_ERR_GROUP: return "n_heads must be n_kv_heads times 1, 2, 4 or 8";
    case PKV_ERR_CONTEXT: return "max_context_len must be in [1, max_blocks_per_seq * block_size]";
    case PKV_ERR_PARTITION: return "partition_tokens must be 0 or a positive multiple of block_size";
    case PKV_ERR_WORKSPACE: return "workspace missing or smaller than pkv_decode_workspace_bytes";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_ALIGN: return "device pointers must be 16-byte aligned";
    case PKV_ERR_ALIAS: return "out overlaps an input";
    case PKV_ERR_OUT_OF_BLOCKS: return "not enough free blocks in the pool";
    case PKV_ERR_NO_SEQUENCE: return "unknown sequence id";
    case PKV_ERR_SEQUENCE_EXISTS: return "sequence id already in use";
    case PKV_ERR_BAD_BLOCK: return "block id outside the pool";
    case PKV_ERR_QUERIES: return "q_len must be >= 1 with q_len * (n_heads / n_kv_heads) <= 16";
    case PKV_ERR_SCRATCH: return "the sizes need more workspace than the library's 32 MiB static scratch";
    default: return "unknown status";
  }
}

int64_t pkv_kv_bytes_per_token(int32_t n_layers, int32_t n_kv_heads, int32_t d_head,
                               int32_t dtype_bytes) {
  if (n_layers < 0 || n_kv_heads < 0 || d_head < 0 || dtype_bytes < 0) return -1;
  return (int64_t)2 * n_layers * n_kv_heads * d_head * dtype_bytes;
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t n_heads, int32_t n_kv_heads,
                                  int32_t d_head, int32_t max_context_len,
                                  int32_t partition_tokens) {
  if (num_seqs <= 0 || n_heads <= 0 || d_head <= 0 || max_context_len <= 0 ||
      !valid_group(n_heads, n_kv_heads) || partition_tokens < 0 ||
      partition_tokens % pkv::kBlockTokens)
    return 0;
  return make_plan(num_seqs, 1, n_heads, n_kv_heads, d_head, max_context_len, partition_tokens).bytes;
}

int32_t pkv_kv_append_tokens(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                             const int32_t* block_tables, const int32_t* positions,
                             int32_t num_seqs, int32_t n_tokens, int32_t max_blocks_per_seq,
                             int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                             int32_t d_head, int32_t dtype, hipStream_t stream) {
  if (!k_pool || !v_pool || !k_new || !v_new || !block_tables || !positions) return PKV_ERR_NULL;
  if (elem_bytes(dtype) == 0) return PKV_ERR_DTYPE;
  if (block_size != pkv::kBlockTokens) return PKV_ERR_BLOCK_SIZE;
  if (d_head != 64 && d_head != 128) return PKV_ERR_HEAD_DIM;
  if (num_seqs <= 0 || num_seqs > 65535 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
      n_kv_heads <= 0 || n_kv_heads > pkv::kMaxKvHeads || n_tokens < 1 || n_tokens > 16)
    return PKV_ERR_SHAPE;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new))
    return PKV_ERR_ALIGN;
  pkv::AppendArgs a;
  a.k_pool = static_cast<char*>(k_pool);
  a.v_pool = static_cast<char*>(v_pool);
  a.k_new = static_cast<const char*>(k_new);
  a.v_new = static_cast<const char*>(v_new);
  a.block_tables = block_tables;
  a.positions = positions;
  a.num_seqs = num_seqs;
  a.n_tokens = n_tokens;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.row_bytes = n_kv_heads * d_head * elem_bytes(dtype);
  return pkv::launch_append(a, stream) == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int32_t pkv_kv_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                      const int32_t* block_tables, const int32_t* positions,
                      int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                      int32_t block_size, int32_t n_kv_heads, int32_t d_head, int32_t dtype,
                      hipStream_t stream) {
  return pkv_kv_append_tokens(k_pool, v_pool, k_new, v_new, block_tables, positions, num_seqs, 1,
                              max_blocks_per_seq, num_blocks, block_size, n_kv_heads, d_head,
                              dtype, stream);
}

int32_t pkv_kv_append_quantized(void* k_codes, void* v_codes, float* k_scales, float* v_scales,
                                const void* k_new, const void* v_new,
                                const int32_t* block_tables, const int32_t* positions,
                                int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                                int32_t block_size, int32_t n_kv_heads, int32_t d_head,
                                int32_t dtype, int32_t kv_format, hipStream_t stream) {
  if (!k_codes || !v_codes || !k_scales || !v_scales || !k_new || !v_new || !block_tables ||
      !positions)
    return PKV_ERR_NULL;
  if (elem_bytes(dtype) == 0 || (kv_format != PKV_KV_INT8 && kv_format != PKV_KV_FP8))
    return PKV_ERR_DTYPE;
  if (block_size != pkv::kBlockTokens) return PKV_ERR_BLOCK_SIZE;
  if (d_head != 64 && d_head != 128) return PKV_ERR_HEAD_DIM;
  if (num_seqs <= 0 || num_seqs > 65535 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
      n_kv_heads <= 0 || n_kv_heads > pkv::kMaxKvHeads)
    return PKV_ERR_SHAPE;
  if (!aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_scales) ||
      !aligned16(v_scales) || !aligned16(k_new) || !aligned16(v_new))
    return PKV_ERR_ALIGN;
  pkv::QuantAppendArgs a;
  a.k_codes = static_cast<char*>(k_codes);
  a.v_codes = static_cast<char*>(v_codes);
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.k_new = static_cast<const char*>(k_new);
  a.v_new = static_cast<const char*>(v_new);
  a.block_tables = block_tables;
  a.positions = positions;
  a.num_seqs = num_seqs;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.n_kv_heads = n_kv_heads;
  a.d_head = d_head;
  a.dtype = dtype;
  a.kv_format = kv_format;
  return pkv::launch_append_quantized(a, stream) == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int32_t pkv_paged_decode_step(void* out, const void* q, void* k_pool, void* v_pool,
                              const void* k_new, const void* v_new, const int32_t* block_tables,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_blocks_per_seq, int32_t num_blocks,
                              int32_t max_context_len, int32_t block_size, int32_t n_heads,
                              int32_t n_kv_heads, int32_t d_head, float scale,
                              int32_t partition_tokens, int32_t dtype, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, 1,
                     max_blocks_per_seq, num_blocks, max_context_len, block_size, n_heads,
                     n_kv_heads, d_head, scale, partition_tokens, dtype, workspace,
                     workspace_bytes, stream, 0, nullptr, nullptr, k_new, v_new, true);
}

int32_t pkv_paged_decode_step_noalloc(void* out, const void* q, void* k_pool, void* v_pool,
                                      const void* k_new, const void* v_new,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t max_blocks_per_seq,
                                      int32_t num_blocks, int32_t max_context_len,
                                      int32_t block_size, int32_t n_heads, int32_t n_kv_heads,
                                      int32_t d_head, float scale, int32_t partition_tokens,
                                      int32_t dtype, hipStream_t stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, 1,
                     max_blocks_per_seq, num_blocks, max_context_len, block_size, n_heads,
                     n_kv_heads, d_head, scale, partition_tokens, dtype, nullptr, 0, stream, 0,
                     nullptr, nullptr, k_new, v_new, true, /*static_scratch=*/true);
}

int32_t pkv_paged_decode_attention_quantized(
    void* out, const void* q, const void* k_codes, const void* v_codes, const float* k_scales,
    const float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
    int32_t block_size, int32_t n_heads, int32_t n_kv_heads, int32_t d_head, float scale,
    int32_t partition_tokens, int32_t dtype, int32_t kv_format, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  if (kv_format != PKV_KV_INT8 && kv_format != PKV_KV_FP8) return PKV_ERR_DTYPE;
  return decode_impl(out, q, k_codes, v_codes, block_tables, context_lens, num_seqs, 1,
                     max_blocks_per_seq, num_blocks, max_context_len, block_size, n_heads,
                     n_kv_heads, d_head, scale, partition_tokens, dtype, workspace,
                     workspace_bytes, stream, kv_format, k_scales, v_scales);
}

int32_t pkv_gather_kv(void* k_out, void* v_out, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* context_lens,
                      int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                      int32_t max_context_len, int32_t block_size, int32_t n_kv_heads,
                      int32_t d_head, int32_t dtype, hipStream_t stream) {
  if (!k_out || !v_out || !k_pool || !v_pool || !block_tables || !context_lens)
    return PKV_ERR_NULL;
  const int32_t st = check_pool_args(num_seqs, max_blocks_per_seq, num_blocks, max_context_len,
                                     block_size, n_kv_heads, d_head, dtype);
  if (st != PKV_OK) return st;
  if (!aligned16(k_out) || !aligned16(v_out) || !aligned16(k_pool) || !aligned16(v_pool))
    return PKV_ERR_ALIGN;
  pkv::GatherArgs a;
  a.k_out = static_cast<char*>(k_out);
  a.v_out = static_cast<char*>(v_out);
  a.k_pool = static_cast<const char*>(k_pool);
  a.v_pool = static_cast<const char*>(v_pool);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.row_bytes = n_kv_heads * d_head * elem_bytes(dtype);
  return pkv::launch_gather(a, stream) == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int32_t pkv_paged_decode_attention(void* out, const void* q, const void* k_pool,
                                   const void* v_pool, const int32_t* block_tables,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t max_blocks_per_seq, int32_t num_blocks,
                                   int32_t max_context_len, int32_t block_size,
                                   int32_t n_heads, int32_t n_kv_heads, int32_t d_head,
                                   float scale, int32_t partition_tokens, int32_t dtype,
                                   void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, 1,
                     max_blocks_per_seq, num_blocks, max_context_len, block_size, n_heads,
                     n_kv_heads, d_head, scale, partition_tokens, dtype, workspace,
                     workspace_bytes, stream);
}

int32_t pkv_decode_split_workgroups(int32_t n_heads, int32_t n_kv_heads, int32_t d_head,
                                    int32_t q_len, int32_t dtype, int32_t kv_format,
                                    int32_t fused_append) {
  if (elem_bytes(dtype) == 0) return PKV_ERR_DTYPE;
  if (d_head != 64 && d_head != 128) return PKV_ERR_HEAD_DIM;
  if (n_kv_heads <= 0 || n_kv_heads > pkv::kMaxKvHeads) return PKV_ERR_SHAPE;
  if (!valid_group(n_heads, n_kv_heads)) return PKV_ERR_GROUP;
  if (!valid_q_len(q_len, n_heads, n_kv_heads)) return PKV_ERR_QUERIES;
  if (kv_format != 0 && ((kv_format != PKV_KV_INT8 && kv_format != PKV_KV_FP8) ||
                         dtype == PKV_F32 || q_len != 1 || fused_append))
    return PKV_ERR_DTYPE;
  int32_t grid = 0;
  pkv::DecodeArgs a{};
  a.n_heads = n_heads;
  a.n_kv_heads = n_kv_heads;
  a.q_len = q_len;
  a.split = 1;
  a.grid_out = &grid;
  static const char kNonNull = 0;               // selects the fused-append kernels
  a.k_new = fused_append ? &kNonNull : nullptr;
  a.v_new = a.k_new;
  const hipError_t e =
      kv_format ? pkv::launch_decode_quantized(a, dtype, kv_format, d_head, n_heads / n_kv_heads,
                                               nullptr)
                : pkv::launch_decode(a, dtype, d_head, n_heads / n_kv_heads, nullptr);
  return e == hipSuccess && grid > 0 ? grid : PKV_ERR_LAUNCH;
}

size_t pkv_multi_query_workspace_bytes(int32_t num_seqs, int32_t q_len, int32_t n_heads,
                                       int32_t n_kv_heads, int32_t d_head,
                                       int32_t max_context_len, int32_t partition_tokens) {
  if (num_seqs <= 0 || n_heads <= 0 || d_head <= 0 || max_context_len <= 0 ||
      !valid_group(n_heads, n_kv_heads) || !valid_q_len(q_len, n_heads, n_kv_heads) ||
      partition_tokens < 0 || partition_tokens % pkv::kBlockTokens)
    return 0;
  return make_plan(num_seqs, q_len, n_heads, n_kv_heads, d_head, max_context_len,
                   partition_tokens).bytes;
}

int32_t pkv_paged_multi_query_attention(void* out, const void* q, const void* k_pool,
                                        const void* v_pool, const int32_t* block_tables,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t q_len, int32_t max_blocks_per_seq,
                                        int32_t num_blocks, int32_t max_context_len,
                                        int32_t block_size, int32_t n_heads, int32_t n_kv_heads,
                                        int32_t d_head, float scale, int32_t partition_tokens,
                                        int32_t dtype, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, q_len,
                     max_blocks_per_seq, num_blocks, max_context_len, block_size, n_heads,
                     n_kv_heads, d_head, scale, partition_tokens, dtype, workspace,
                     workspace_bytes, stream);
}

int32_t pkv_paged_multi_query_step(void* out, const void* q, void* k_pool, void* v_pool,
                                   const void* k_new, const void* v_new,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   int32_t num_seqs, int32_t q_len, int32_t max_blocks_per_seq,
                                   int32_t num_blocks, int32_t max_context_len,
                                   int32_t block_size, int32_t n_heads, int32_t n_kv_heads,
                                   int32_t d_head, float scale, int32_t partition_tokens,
                                   int32_t dtype, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, q_len,
                     max_blocks_per_seq, num_blocks, max_context_len, block_size, n_heads,
                     n_kv_heads, d_head, scale, partition_tokens, dtype, workspace,
                     workspace_bytes, stream, 0, nullptr, nullptr, k_new, v_new, true);
}

size_t pkv_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t n_heads, int32_t n_kv_heads,
                                         int32_t d_head, int32_t max_shared_blocks) {
  if (num_seqs <= 0 || num_seqs > pkv::kSplitMaxSeqs || n_heads <= 0 || d_head <= 0 ||
      !valid_group(n_heads, n_kv_heads) || max_shared_blocks < 0)
    return 0;
  return make_plan(num_seqs, 1, n_heads, n_kv_heads, d_head, 1, 0, max_shared_blocks).bytes;
}

int32_t pkv_paged_decode_attention_shared_prefix(
    void* out, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_group,
    const int32_t* group_blocks, int32_t n_groups, int32_t max_group_size,
    int32_t max_shared_blocks, int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
    int32_t max_context_len, int32_t block_size, int32_t n_heads, int32_t n_kv_heads,
    int32_t d_head, float scale, int32_t dtype, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !seq_group ||
      !group_blocks)
    return PKV_ERR_NULL;
  int32_t st = check_pool_args(num_seqs, max_blocks_per_seq, num_blocks, max_context_len,
                               block_size, n_kv_heads, d_head, dtype);
  if (st != PKV_OK) return st;
  if (!valid_group(n_heads, n_kv_heads)) return PKV_ERR_GROUP;
  if (!std::isfinite(scale)) return PKV_ERR_SHAPE;
  if (num_seqs > pkv::kSplitMaxSeqs || n_groups < 1 || n_groups > 65535 || max_group_size < 1 ||
      max_group_size > num_seqs || max_shared_blocks < 0 || max_shared_blocks > max_blocks_per_seq)
    return PKV_ERR_SHAPE;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return PKV_ERR_ALIGN;
  const size_t eb = (size_t)elem_bytes(dtype);
  const size_t out_bytes = (size_t)num_seqs * n_heads * d_head * eb;
  const size_t pool_bytes = (size_t)num_blocks * pkv::kBlockTokens * n_kv_heads * d_head * eb;
  if (overlaps(out, out_bytes, q, out_bytes) || overlaps(out, out_bytes, k_pool, pool_bytes) ||
      overlaps(out, out_bytes, v_pool, pool_bytes))
    return PKV_ERR_ALIAS;
  const Plan plan = make_plan(num_seqs, 1, n_heads, n_kv_heads, d_head, max_context_len, 0,
                              max_shared_blocks);
  if (!workspace || workspace_bytes < plan.bytes || !aligned16(workspace)) return PKV_ERR_WORKSPACE;
  const int32_t g = n_heads / n_kv_heads;
  // column sets of 16 (member, head) pairs, taken wph at a time by the waves of a KV head
  const int wph = pkv::prefix_waves_per_head(max_group_size, g);
  const int64_t sets = (((int64_t)max_group_size * g + 15) / 16 + wph - 1) / wph;
  // prefix tasks: at most (partitions x KV heads x column quads x groups)
  if ((int64_t)plan.prefix_parts * n_kv_heads * sets * n_groups > (int64_t(1) << 24))
    return PKV_ERR_SHAPE;

  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = static_cast<const char*>(k_pool);
  a.v_pool = static_cast<const char*>(v_pool);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.n_heads = n_heads;
  a.n_kv_heads = n_kv_heads;
  a.q_len = 1;
  a.split = 1;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);   // log2(e)
  a.seq_group = seq_group;
  a.group_blocks = group_blocks;
  a.n_groups = n_groups;
  a.prefix_parts = plan.prefix_parts;
  a.prefix_sets = (int32_t)sets;
  a.prefix_wph = wph;
  a.max_group_size = max_group_size;
  a.max_shared_blocks = max_shared_blocks;
  char* ws = static_cast<char*>(workspace);
  size_t off = 0;
  auto take = [&](size_t bytes) { char* p = ws + off; off += align256(bytes); return p; };
  a.ws_prefix = reinterpret_cast<int32_t*>(take(plan.prefix_ints * sizeof(int32_t)));
  a.ws_m = reinterpret_cast<float*>(take(plan.records * sizeof(float)));
  a.ws_l = reinterpret_cast<float*>(take(plan.records * sizeof(float)));
  a.ws_o = reinterpret_cast<float*>(take(plan.records * d_head * sizeof(float)));
  a.ws_pm = reinterpret_cast<float*>(take(plan.shared_records * sizeof(float)));
  a.ws_pl = reinterpret_cast<float*>(take(plan.shared_records * sizeof(float)));
  a.ws_po = reinterpret_cast<float*>(take(plan.shared_records * d_head * sizeof(float)));
  a.ws_flags = reinterpret_cast<int32_t*>(take(plan.flag_ints * sizeof(int32_t)));
  const hipError_t e = pkv::launch_shared_prefix(a, dtype, d_head, g, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int32_t pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int32_t n_pairs,
                        int32_t num_blocks, int32_t block_size, int32_t n_kv_heads,
                        int32_t d_head, int32_t dtype, hipStream_t stream) {
  if (!k_pool || !v_pool || (n_pairs > 0 && !pairs)) return PKV_ERR_NULL;
  const int32_t eb = elem_bytes(dtype);
  if (eb == 0) return PKV_ERR_DTYPE;
  if (block_size != pkv::kBlockTokens) return PKV_ERR_BLOCK_SIZE;
  if (d_head != 64 && d_head != 128) return PKV_ERR_HEAD_DIM;
  if (n_pairs < 0 || n_pairs > 65535 || num_blocks <= 0 || n_kv_heads <= 0 ||
      n_kv_heads > pkv::kMaxKvHeads)
    return PKV_ERR_SHAPE;
  if (!aligned16(k_pool) || !aligned16(v_pool)) return PKV_ERR_ALIGN;
  if (n_pairs == 0) return PKV_OK;
  const int64_t block_bytes = (int64_t)block_size * n_kv_heads * d_head * eb;
  const hipError_t e = pkv::launch_copy_blocks(static_cast<char*>(k_pool),
                                               static_cast<char*>(v_pool), pairs, n_pairs,
                                               num_blocks, block_bytes, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // extern "C"
