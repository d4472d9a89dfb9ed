// KV append (scatter of the new token into its slot) and the test-only gather.
//
// Slot rule, chenxutan §2.3 (write_kv / read_kv): token t of a sequence lives in the
// physical block table[t / 16] at slot t % 16. One token's K (or V) for all KV heads is
// one contiguous row of n_kv_heads * d_head elements in the [num_blocks, 16, n_kv_heads,
// d_head] pool, so both kernels move whole rows with 16-byte vector accesses.

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// grid (num_seqs, 2 * n_tokens): y = 2i writes K, y = 2i + 1 writes V of new token i,
// which goes to position positions[b] + i. One thread per 16-byte chunk.
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const int i = blockIdx.y >> 1, which = blockIdx.y & 1;
  const int t = a.positions[b] + i;
  const int logical = t >> 4;
  if (t < 0 || logical >= a.max_blocks_per_seq) return;
  const int phys = a.block_tables[(size_t)b * a.max_blocks_per_seq + logical];
  if ((unsigned)phys >= (unsigned)a.num_blocks) return;
  const size_t slot_row = (size_t)phys * kBlockTokens + (t & 15);
  char* dst = (which == 0 ? a.k_pool : a.v_pool) + slot_row * a.row_bytes;
  const char* src = (which == 0 ? a.k_new : a.v_new) + ((size_t)b * a.n_tokens + i) * a.row_bytes;
  const int chunks = a.row_bytes >> 4;
  for (int k = threadIdx.x; k < chunks; k += blockDim.x)
    reinterpret_cast<u32x4*>(dst)[k] = reinterpret_cast<const u32x4*>(src)[k];
}

// grid (blocks of max_context_len, num_seqs): copies the used rows of one block.
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int blk = blockIdx.x;
  const int b = blockIdx.y;
  int n = a.context_lens[b];
  n = n < a.max_context_len ? n : a.max_context_len;
  const int t0 = blk * kBlockTokens;
  if (t0 >= n) return;
  const int phys = a.block_tables[(size_t)b * a.max_blocks_per_seq + blk];
  if ((unsigned)phys >= (unsigned)a.num_blocks) return;
  const int rows = (n - t0) < kBlockTokens ? (n - t0) : kBlockTokens;
  const int chunks = a.row_bytes >> 4;
  const size_t src_row = (size_t)phys * kBlockTokens;
  const size_t dst_row = (size_t)b * a.max_context_len + t0;
  for (int i = threadIdx.x; i < rows * chunks; i += blockDim.x) {
    const int r = i / chunks, c = i - r * chunks;
    const size_t so = (src_row + r) * a.row_bytes, dof = (dst_row + r) * a.row_bytes;
    reinterpret_cast<u32x4*>(a.k_out + dof)[c] = reinterpret_cast<const u32x4*>(a.k_pool + so)[c];
    reinterpret_cast<u32x4*>(a.v_out + dof)[c] = reinterpret_cast<const u32x4*>(a.v_pool + so)[c];
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const int chunks = a.row_bytes >> 4;
  const int threads = chunks < 256 ? ((chunks + 63) & ~63) : 256;
  hipLaunchKernelGGL(append_kernel, dim3(a.num_seqs, 2 * a.n_tokens), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
  const int nblk = (a.max_context_len + kBlockTokens - 1) / kBlockTokens;
  hipLaunchKernelGGL(gather_kernel, dim3(nblk, a.num_seqs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
