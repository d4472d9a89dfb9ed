// Internal launch interface between the C ABI (pkv_capi.cpp, host C++) and the kernels
// (*.hip). Host-only declarations: the C ABI and the block manager include it from plain
// C++ translation units.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlockTokens = 16;   // tokens per KV block (the only supported block size)
constexpr int kMaxKvHeads = 256;   // keeps byte offsets inside a block within 32 bits
constexpr int kFallbackPartition = 512;   // fixed partition size when the split mode cannot run
constexpr int kSplitMaxSeqs = 4096;       // split mode keeps the per-sequence prefix in LDS
constexpr int kSplitMaxWorkgroups = 1024; // upper bound of the split-mode grid
constexpr int kSplitMinBlocks = 8;        // fewest blocks a split-mode workgroup is given
constexpr int kMergeRowsWave = 1024;      // from this many output rows on, a wave per row
constexpr int kPrefixPartition = 512;     // tokens per prefix-task partition
constexpr int kPrefixWaves = 4;           // most prefix-task waves per KV head, 16 columns each

// Waves per KV head of a prefix task: enough 16-column sets for the largest group's
// (member, head) columns, rounded up to a power of two, at most kPrefixWaves.
inline int prefix_waves_per_head(long long max_group_size, int group) {
  const long long sets = (max_group_size * group + 15) / 16;
  return sets >= 3 ? kPrefixWaves : (sets == 2 ? 2 : 1);
}

// Quantized KV formats (values of the C ABI's kv_format) and the decode kernels' modes.
constexpr int kKvInt8 = 1;
constexpr int kKvFp8 = 2;
constexpr int kModeSingle = 0;      // one query per sequence, P.V on the vector ALU
constexpr int kModeMulti = 1;       // q_len queries per sequence, P.V on the matrix cores
constexpr int kModeQuantInt8 = 2;   // one query, INT8 codes + (s, z) per token and KV head
constexpr int kModeQuantFp8 = 3;    // one query, E4M3 codes + (s, 0) per token and KV head
constexpr int kModeSingleAppend = 4; // kModeSingle that also appends the new token (k_new)
constexpr int kModeMultiAppend = 5;  // kModeMulti that also appends the q_len new tokens
constexpr int kModeSinglePrefix = 6; // kModeSingle whose first workgroups also run the
                                     // shared-prefix tasks

// Waves per decode workgroup (one KV head each) used with this many KV heads. The
// launcher may use fewer (4) for kernels that do not fit 256 registers per lane; this is
// the upper bound the workspace is sized for.
inline int max_waves_per_workgroup(int n_kv_heads) { return n_kv_heads % 8 == 0 ? 8 : 4; }

struct AppendArgs {
  char* k_pool;
  char* v_pool;
  const char* k_new;
  const char* v_new;
  const int32_t* block_tables;
  const int32_t* positions;          // first new token of each sequence
  int32_t num_seqs, n_tokens, max_blocks_per_seq, num_blocks;
  int32_t row_bytes;                 // n_kv_heads * d_head * element bytes
};

struct GatherArgs {
  char* k_out;
  char* v_out;
  const char* k_pool;
  const char* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs, max_blocks_per_seq, num_blocks, max_context_len;
  int32_t row_bytes;
};

struct DecodeArgs {
  void* out;
  const void* q;
  const char* k_pool;
  const char* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  // Partial-result records (m, l, O[d_head]), fp32. Fixed mode: record
  // (b * n_heads + h) * max_partitions + p. Split mode: see decode_split_kernel.
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int32_t* ws_prefix;                // split mode: [num_seqs + 1] block prefix sums
  int32_t num_seqs, max_blocks_per_seq, num_blocks, max_context_len;
  int32_t n_heads, n_kv_heads;
  int32_t q_len;                     // new tokens (queries) per sequence, 1..16/group
  int32_t split;                     // 1: balanced split over the GPU; 0: fixed partitions
  int32_t partition_tokens, max_partitions;   // fixed mode
  int32_t split_workgroups;          // split mode: grid size W (set by the launcher)
  // Shared prefixes (optional, split mode, q_len 1): seq_group[b] is the group of
  // sequence b (-1: none); the members of group g share their first group_blocks[g]
  // table entries. The prefix tasks read those blocks once per group and leave records
  // ws_p* at (b * n_heads + h) * prefix_parts + p; the private units cover the rest.
  const int32_t* seq_group;
  const int32_t* group_blocks;
  int32_t n_groups, prefix_parts, prefix_sets;
  int32_t max_group_size, max_shared_blocks;  // host bounds the prefix tasks were sized for
  // Split mode with shared prefixes: workgroups 0 .. prefix_tasks - 1 each run one prefix
  // task first and are given prefix_cost fewer private blocks (set by the launcher).
  int32_t prefix_tasks, prefix_cost;
  int32_t prefix_wph;                // waves per KV head in a prefix task (1, 2 or 4)
  float* ws_pm;
  float* ws_pl;
  float* ws_po;
  int32_t* ws_flags;                 // [num_seqs * prefix_parts] nonzero: member b's table
                                     // disagrees with the group's in partition p, or the
                                     // group has more than max_group_size members
  float scale_log2;                  // scale * log2(e): scores are kept in base 2
  // Quantized caches: k_pool / v_pool hold 8-bit codes and these the (s, z) pairs,
  // [num_blocks][n_kv_heads][16][2] fp32.
  const float* k_scales;
  const float* v_scales;
  // Fused append (single query, dtype pools): the new token's K / V rows,
  // [num_seqs][n_kv_heads][d_head]; the token is context_lens[b] - 1. nullptr: no append.
  const char* k_new;
  const char* v_new;
  // Grid query (host side only): when set, the split-mode launcher stores the grid it would
  // use here and launches nothing.
  int32_t* grid_out;
};

// Quantizing append: one token per sequence, K and V rows of every KV head quantized to
// 8-bit codes with one (s, z) pair each.
struct QuantAppendArgs {
  char* k_codes;
  char* v_codes;
  float* k_scales;                   // [num_blocks][n_kv_heads][16][2]
  float* v_scales;
  const char* k_new;                 // [num_seqs][n_kv_heads][d_head] in dtype
  const char* v_new;
  const int32_t* block_tables;
  const int32_t* positions;
  int32_t num_seqs, max_blocks_per_seq, num_blocks, n_kv_heads, d_head;
  int32_t dtype;                     // of k_new / v_new: 0 f32, 1 f16, 2 bf16
  int32_t kv_format;                 // kKvInt8 or kKvFp8
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_append_quantized(const QuantAppendArgs& a, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);
// pool[dst] = pool[src] in both pools for each (src, dst) pair; block_bytes per block.
hipError_t launch_copy_blocks(char* k_pool, char* v_pool, const int32_t* pairs, int32_t n_pairs,
                              int32_t num_blocks, int64_t block_bytes, hipStream_t stream);
// dtype: 0 f32, 1 f16, 2 bf16; d_head 64/128; group 1/2/4/8 (validated by the caller).
hipError_t launch_decode(const DecodeArgs& a, int dtype, int d_head, int group,
                         hipStream_t stream);
// Decode over 8-bit codes (dtype 1 or 2 for q / out).
hipError_t launch_decode_quantized(const DecodeArgs& a, int dtype, int kv_format, int d_head,
                                   int group, hipStream_t stream);
// Shared-prefix decode (split mode, q_len 1): split kernel with the prefix tasks, merge.
hipError_t launch_shared_prefix(const DecodeArgs& a, int dtype, int d_head, int group,
                                hipStream_t stream);

// The decode kernels of one dtype DT. pkv_decode.hip is compiled once per dtype
// (-DPKV_DECODE_DTYPE=DT) and defines these three for its DT; launch_decode,
// launch_decode_quantized and launch_shared_prefix (pkv_dispatch.cpp) pick the dtype.
template <int DT>
hipError_t launch_decode_dtype(const DecodeArgs& a, int d_head, int group, hipStream_t stream);
template <int DT>
hipError_t launch_decode_quantized_dtype(const DecodeArgs& a, int kv_format, int d_head,
                                         int group, hipStream_t stream);
template <int DT>
hipError_t launch_shared_prefix_dtype(const DecodeArgs& a, int d_head, int group,
                                      hipStream_t stream);

}  // namespace pkv
