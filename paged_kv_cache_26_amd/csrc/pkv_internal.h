// Internal launch interface between the C ABI (pkv_capi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlockTokens = 16;   // tokens per KV block (the only supported block size)
constexpr int kDecodeWaves = 4;    // waves per decode workgroup
constexpr int kDefaultPartition = 512;

struct AppendArgs {
  char* k_pool;
  char* v_pool;
  const char* k_new;
  const char* v_new;
  const int32_t* block_tables;
  const int32_t* positions;
  int32_t num_seqs, max_blocks_per_seq, num_blocks;
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
  float* ws_m;                       // [num_seqs, n_heads, max_partitions]
  float* ws_l;
  float* ws_o;                       // [num_seqs, n_heads, max_partitions, d_head]
  int32_t num_seqs, max_blocks_per_seq, num_blocks, max_context_len;
  int32_t n_heads, n_kv_heads;
  int32_t partition_tokens, max_partitions;
  float scale_log2;                  // scale * log2(e): scores are kept in base 2
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);
// dtype: 0 f32, 1 f16, 2 bf16; d_head 64/128; group 1/2/4/8 (validated by the caller).
hipError_t launch_decode(const DecodeArgs& a, int dtype, int d_head, int group,
                         hipStream_t stream);

}  // namespace pkv
