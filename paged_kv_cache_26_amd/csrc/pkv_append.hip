// KV append (scatter of the new token into its slot), its quantizing variant, the
// copy-on-write block copy, and the test-only gather.
//
// Slot rule, chenxutan §2.3 (write_kv / read_kv): token t of a sequence lives in the
// physical block table[t / 16] at slot t % 16. One token's K (or V) for all KV heads is
// one contiguous row of n_kv_heads * d_head elements in the [num_blocks, 16, n_kv_heads,
// d_head] pool, so both kernels move whole rows with 16-byte vector accesses.

#include <hip/hip_runtime.h>

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

// Nearest OCP E4M3 byte to y (ties to the even code), saturating at +-448: the binary32
// mantissa is rounded to 3 bits at bit 20 (round half to even) and the exponent rebiased
// from 127 to 7; below 2^-6 the code is the subnormal multiple round(|y| * 2^9).
__device__ __forceinline__ unsigned e4m3_encode(float y) {
  const unsigned bits = __float_as_uint(y);
  const float a = fabsf(y);
  unsigned code;
  if (!(a < 448.0f)) {
    code = 0x7E;
  } else if (a < 0.015625f) {
    code = (unsigned)rintf(a * 512.0f);        // exact scaling; 8 becomes the smallest normal
  } else {
    const unsigned m = __float_as_uint(a);
    code = ((m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  }
  return code | ((bits >> 24) & 0x80u);
}

// grid (n_pairs, 2): y selects the K or V pool; 16 bytes per thread per step. A pair with
// a block id outside the pool is skipped.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* k_pool, char* v_pool,
                                                          const int32_t* pairs, int32_t num_blocks,
                                                          int64_t block_bytes) {
  const int32_t src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) return;
  char* pool = blockIdx.y == 0 ? k_pool : v_pool;
  const u32x4* s = reinterpret_cast<const u32x4*>(pool + src * block_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(pool + dst * block_bytes);
  const int64_t n = block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) d[i] = s[i];
}

template <int DT>
__device__ __forceinline__ float load_elem(const char* base, size_t idx) {
  if constexpr (DT == 0) {
    return reinterpret_cast<const float*>(base)[idx];
  } else if constexpr (DT == 1) {
    return (float)reinterpret_cast<const _Float16*>(base)[idx];
  } else {
    return __uint_as_float((unsigned)reinterpret_cast<const uint16_t*>(base)[idx] << 16);
  }
}

// grid (num_seqs, 2): y = 0 quantizes K, y = 1 V. Wave w handles KV heads w, w + 4, ...;
// lane l holds elements EPL*l .. EPL*l + EPL - 1 of the row (EPL = d_head / 64). Every
// step is binary32 with the same operation order as the reference quantizer: the row's
// range [min(x, 0), max(x, 0)], s = (hi - lo) / 255, z = round(-lo / s),
// Q = clamp(round(x / s) + z, 0, 255) for INT8; s = max|x| / 448, Q = E4M3(x / s) for FP8.
template <int DT, int EPL, int FMT>
__global__ __launch_bounds__(256) void append_quant_kernel(QuantAppendArgs a) {
  const int b = blockIdx.x, which = blockIdx.y;
  const int t = a.positions[b];
  const int logical = t >> 4;
  if (t < 0 || logical >= a.max_blocks_per_seq) return;
  const int phys = a.block_tables[(size_t)b * a.max_blocks_per_seq + logical];
  if ((unsigned)phys >= (unsigned)a.num_blocks) return;
  const int off = t & 15;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int D = 64 * EPL;
  char* codes = which ? a.v_codes : a.k_codes;
  float* scales = which ? a.v_scales : a.k_scales;
  const char* src = which ? a.v_new : a.k_new;
  for (int j = wave; j < a.n_kv_heads; j += 4) {
    float x[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = load_elem<DT>(src, ((size_t)b * a.n_kv_heads + j) * D + EPL * lane + e);
    float sc, z = 0.f;
    unsigned q[EPL];
    if constexpr (FMT == kKvInt8) {
      float lo = x[0], hi = x[0];
#pragma unroll
      for (int e = 1; e < EPL; ++e) {
        lo = fminf(lo, x[e]);
        hi = fmaxf(hi, x[e]);
      }
#pragma unroll
      for (int sh = 32; sh > 0; sh >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, sh));
        hi = fmaxf(hi, __shfl_xor(hi, sh));
      }
      lo = fminf(lo, 0.f);
      hi = fmaxf(hi, 0.f);
      sc = (hi - lo) / 255.0f;
      if (sc == 0.f) sc = 1.0f;
      z = fminf(fmaxf(rintf(-lo / sc), 0.f), 255.f) + 0.0f;   // + 0: a zero point is +0, never -0
#pragma unroll
      for (int e = 0; e < EPL; ++e) q[e] = (unsigned)fminf(fmaxf(rintf(x[e] / sc) + z, 0.f), 255.f);
    } else {
      float amax = fabsf(x[0]);
#pragma unroll
      for (int e = 1; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
      for (int sh = 32; sh > 0; sh >>= 1) amax = fmaxf(amax, __shfl_xor(amax, sh));
      sc = amax / 448.0f;
      if (sc == 0.f) sc = 1.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) q[e] = e4m3_encode(x[e] / sc);
    }
    unsigned char* dst = reinterpret_cast<unsigned char*>(codes) +
                         (((size_t)phys * kBlockTokens + off) * a.n_kv_heads + j) * D + EPL * lane;
    if constexpr (EPL == 2) {
      *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(q[0] | (q[1] << 8));
    } else {
      dst[0] = (unsigned char)q[0];
    }
    if (lane == 0) {
      float* sz = scales + (((size_t)phys * a.n_kv_heads + j) * kBlockTokens + off) * 2;
      *reinterpret_cast<float2*>(sz) = make_float2(sc, z);
    }
  }
}

template <int DT, int EPL>
hipError_t launch_append_q(const QuantAppendArgs& a, hipStream_t stream) {
  if (a.kv_format == kKvInt8)
    hipLaunchKernelGGL((append_quant_kernel<DT, EPL, kKvInt8>), dim3(a.num_seqs, 2), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((append_quant_kernel<DT, EPL, kKvFp8>), dim3(a.num_seqs, 2), dim3(256), 0,
                       stream, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_append_q_dim(const QuantAppendArgs& a, hipStream_t stream) {
  return a.d_head == 128 ? launch_append_q<DT, 2>(a, stream) : launch_append_q<DT, 1>(a, stream);
}

}  // namespace

hipError_t launch_append_quantized(const QuantAppendArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case 0: return launch_append_q_dim<0>(a, stream);
    case 1: return launch_append_q_dim<1>(a, stream);
    case 2: return launch_append_q_dim<2>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const int chunks = a.row_bytes >> 4;
  const int threads = chunks < 256 ? ((chunks + 63) & ~63) : 256;
  hipLaunchKernelGGL(append_kernel, dim3(a.num_seqs, 2 * a.n_tokens), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(char* k_pool, char* v_pool, const int32_t* pairs, int32_t n_pairs,
                              int32_t num_blocks, int64_t block_bytes, hipStream_t stream) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n_pairs, 2), dim3(256), 0, stream, k_pool, v_pool,
                     pairs, num_blocks, block_bytes);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
  const int nblk = (a.max_context_len + kBlockTokens - 1) / kBlockTokens;
  hipLaunchKernelGGL(gather_kernel, dim3(nblk, a.num_seqs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
