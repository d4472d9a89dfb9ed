// Split-KV paged decode attention for gfx950 (CDNA4, wave64), and the partition merge.
//
// What is computed (chenxutan §2.4; "09-inference-optimization" KV Cache): for every
// sequence b and query head h, with KV head j = h / G,
//     out[b,h,:] = sum_t softmax_t(scale * q[b,h,:] . K[t,j,:]) * V[t,j,:]
// over the N_b cached tokens t, each found through the block table (chenxutan §2.3).
// The softmax is taken online ("推理机制动态图解（进阶）" demo 5): a running maximum m,
// a running sum l and an unnormalised output O, rescaled by 2^(m_old - m_new) when the
// maximum grows; O / l is formed once at the end. Scores are kept in base 2
// (scale * log2 e folded into one multiplier), which leaves the result unchanged.
//
// Work decomposition (FlashDecoding, "Scaling Book 第 11 章" §11.8): a sequence's tokens
// are cut into partitions of P tokens (a multiple of the 16-token block). One workgroup
// of 4 waves handles one (partition, KV head, sequence) and all G query heads of that KV
// head, so each K/V byte is read from HBM once per KV head. Waves take the partition's
// blocks round-robin; each keeps its own (m, l, O) and the four are merged through LDS.
// A sequence with one partition is finished in place; otherwise the workgroup writes its
// (m, l, O) to the workspace and merge_kernel combines the partitions by the same
// rescale rule.
//
// Per 16-token block, inside one wave (lane = 16 * r + c, r = 0..3, c = 0..15):
//   * QK^T on the matrix cores. The K tile is the MFMA A operand (row = token c of the
//     block), the G query vectors the B operand (column = head c, columns >= G are
//     zero). 16-bit types use v_mfma_f32_16x16x32_{bf16,f16}; fp32 uses
//     v_mfma_f32_16x16x4_f32. Lane (r, c) loads 16 bytes at byte 64*kk + 16*r of token
//     c's row, which is exactly its A-operand slice for step kk; the B operand uses the
//     same lane-to-k mapping, so the contraction is the plain dot product. The result
//     lands with token 4r + i, head c in accumulator i.
//   * softmax bookkeeping per head on that layout (two cross-row shuffles for the
//     block maximum; the running sum stays lane-partial until the end).
//   * P.V on the vector ALU in fp32: lane (r, c) loads d_head/16 consecutive elements
//     (chunk c) of token 4r + jj for jj = 0..3, and gets each head's probability for that
//     token from lane (r, h) with a DPP row broadcast.
// K and V of block i+1 are loaded while block i is computed (two register buffers).

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct ElemBytes { static constexpr int value = DT == 0 ? 4 : 2; };

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float as_f(unsigned u) { return __builtin_bit_cast(float, u); }

// Lane h of this lane's 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int H>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + H, 0xF, 0xF, false));
}

template <int N>
struct Int {
  static constexpr int value = N;
};
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(Int<N - 1>{});
  }
}

// Widen W packed 32-bit words of dtype DT into fp32.
template <int DT, int W>
__device__ __forceinline__ void widen(const unsigned (&w)[W], float* out) {
#pragma unroll
  for (int i = 0; i < W; ++i) {
    if constexpr (DT == 2) {
      out[2 * i] = as_f(w[i] << 16);
      out[2 * i + 1] = as_f(w[i] & 0xFFFF0000u);
    } else if constexpr (DT == 1) {
      const f16x2 h = __builtin_bit_cast(f16x2, w[i]);
      out[2 * i] = (float)h[0];
      out[2 * i + 1] = (float)h[1];
    } else {
      out[i] = as_f(w[i]);
    }
  }
}

template <int DT>
__device__ __forceinline__ void store_elem(void* base, size_t idx, float v) {
  if constexpr (DT == 0) {
    static_cast<float*>(base)[idx] = v;
  } else if constexpr (DT == 1) {
    static_cast<_Float16*>(base)[idx] = (_Float16)v;
  } else {
    static_cast<__bf16*>(base)[idx] = (__bf16)v;   // v_cvt_pk_bf16_f32: round to nearest even
  }
}

template <int DT, int D>
struct Geo {
  static constexpr int kE = ElemBytes<DT>::value;
  static constexpr int kRow = D * kE;          // bytes of one head's row
  static constexpr int kNK = kRow / 64;        // 16-byte K loads per lane per block
  static constexpr int kEPL = D / 16;          // V elements per lane per token
  static constexpr int kVW = kEPL * kE / 4;    // V 32-bit words per lane per token
};

// One block's K and V as held by one lane.
template <int DT, int D>
struct Tile {
  u32x4 k[Geo<DT, D>::kNK];
  unsigned v[4][Geo<DT, D>::kVW];
};

template <int DT, int D>
__device__ __forceinline__ void load_tile(Tile<DT, D>& t, const char* kblk, const char* vblk,
                                          size_t k_lane, size_t v_lane, size_t tok_stride) {
  using G_ = Geo<DT, D>;
  const char* kp = kblk + k_lane;
#pragma unroll
  for (int kk = 0; kk < G_::kNK; ++kk) t.k[kk] = *reinterpret_cast<const u32x4*>(kp + 64 * kk);
  const char* vp = vblk + v_lane;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const char* src = vp + jj * tok_stride;
    if constexpr (G_::kVW == 8) {
      const u32x4 a0 = reinterpret_cast<const u32x4*>(src)[0];
      const u32x4 a1 = reinterpret_cast<const u32x4*>(src)[1];
#pragma unroll
      for (int x = 0; x < 4; ++x) { t.v[jj][x] = a0[x]; t.v[jj][4 + x] = a1[x]; }
    } else if constexpr (G_::kVW == 4) {
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
      for (int x = 0; x < 4; ++x) t.v[jj][x] = a0[x];
    } else {
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 a0 = *reinterpret_cast<const u32x2*>(src);
      t.v[jj][0] = a0[0];
      t.v[jj][1] = a0[1];
    }
  }
}

template <int DT, int D, int G>
struct WaveState {
  float m = -INFINITY;                 // running max (base 2) of head c
  float l = 0.f;                       // lane-partial running sum of head c
  float o[G][Geo<DT, D>::kEPL] = {};   // lane-partial O[h][chunk c] for its row's tokens
};

template <int DT, int D, int G>
__device__ __forceinline__ void process_block(WaveState<DT, D, G>& st, const Tile<DT, D>& t,
                                              const u32x4 (&qf)[Geo<DT, D>::kNK], int tok0,
                                              int tok_end, float scale_log2) {
  using G_ = Geo<DT, D>;
  // S^T[token][head] for this block on the matrix cores.
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < G_::kNK; ++kk) {
    if constexpr (DT == 2) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[kk]),
                                                    __builtin_bit_cast(bf16x8, qf[kk]), acc, 0, 0, 0);
    } else if constexpr (DT == 1) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, t.k[kk]),
                                                   __builtin_bit_cast(f16x8, qf[kk]), acc, 0, 0, 0);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f(t.k[kk][s]), as_f(qf[kk][s]), acc, 0, 0, 0);
    }
  }
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = (tok0 + i < tok_end) ? acc[i] * scale_log2 : -INFINITY;

  float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  bm = fmaxf(bm, __shfl_xor(bm, 16));
  bm = fmaxf(bm, __shfl_xor(bm, 32));
  const float m_new = fmaxf(st.m, bm);       // finite: every block has a valid token
  const float alpha = exp2_fast(st.m - m_new);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = exp2_fast(s[i] - m_new);
  st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
  st.m = m_new;

  static_for<G>([&](auto hc) {
    constexpr int h = decltype(hc)::value;
    const float a = row_bcast<h>(alpha);
#pragma unroll
    for (int e = 0; e < G_::kEPL; ++e) st.o[h][e] *= a;
  });

#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    float v[G_::kEPL];
    widen<DT, G_::kVW>(t.v[jj], v);
    const bool valid = tok0 + jj < tok_end;
#pragma unroll
    for (int e = 0; e < G_::kEPL; ++e) v[e] = valid ? v[e] : 0.f;   // unused slots may hold NaN
    static_for<G>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const float ph = row_bcast<h>(p[jj]);
#pragma unroll
      for (int e = 0; e < G_::kEPL; ++e) st.o[h][e] = fmaf(ph, v[e], st.o[h][e]);
    });
  }
}

template <int DT, int D, int G>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  using G_ = Geo<DT, D>;
  constexpr int W = kDecodeWaves;
  const int p = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane >> 4, c = lane & 15;
  const int H = a.n_heads;

  __shared__ float sm_m[W][G], sm_l[W][G];
  __shared__ float sm_o[W][G][D];
  __shared__ int sm_bad[W];

  const int n_ctx = a.context_lens[b];
  if (n_ctx < 1 || n_ctx > a.max_context_len) {
    if (p == 0)
      for (int i = tid; i < G * D; i += 256)
        store_elem<DT>(a.out, ((size_t)b * H + j * G) * D + i, __builtin_nanf(""));
    return;
  }
  const int P = a.partition_tokens;
  const int n_part = (n_ctx + P - 1) / P;
  if (p >= n_part) return;
  const int tok_end = min(n_ctx, (p + 1) * P);
  const int blk_begin = (p * P) >> 4;
  const int blk_end = (tok_end + 15) >> 4;
  const int n_my = (blk_end - blk_begin - wave + W - 1) / W;   // this wave's blocks (may be 0)

  // Query fragments (MFMA B operand): head c of this KV group, zero for c >= G.
  u32x4 qf[G_::kNK];
  {
    const char* qrow = static_cast<const char*>(a.q) + ((size_t)b * H + j * G + (c < G ? c : 0)) * G_::kRow;
#pragma unroll
    for (int kk = 0; kk < G_::kNK; ++kk) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qf[kk] = c < G ? *reinterpret_cast<const u32x4*>(qrow + 64 * kk + 16 * r) : z;
    }
  }

  const size_t tok_stride = (size_t)a.n_kv_heads * G_::kRow;        // bytes between tokens
  const size_t blk_stride = tok_stride * kBlockTokens;
  const size_t head_off = (size_t)j * G_::kRow;
  const size_t k_lane = head_off + c * tok_stride + 16 * r;
  const size_t v_lane = head_off + (4 * r) * tok_stride + c * (G_::kEPL * G_::kE);
  const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks_per_seq;

  WaveState<DT, D, G> st;
  int bad = 0;
  int tbl = 0;   // lane i holds the table entry of this wave's block (chunk * 64 + i)
  auto load_table = [&](int first) {
    const int i = first + lane;
    tbl = i < n_my ? trow[blk_begin + wave + i * W] : 0;
  };
  auto fetch = [&](Tile<DT, D>& t, int i) {
    int pb = __builtin_amdgcn_readlane(tbl, i & 63);
    const bool ok = (unsigned)pb < (unsigned)a.num_blocks;
    bad |= !ok;
    pb = ok ? pb : 0;
    load_tile<DT, D>(t, a.k_pool + (size_t)pb * blk_stride, a.v_pool + (size_t)pb * blk_stride,
                     k_lane, v_lane, tok_stride);
  };
  auto tok0_of = [&](int i) { return (blk_begin + wave + i * W) * kBlockTokens + 4 * r; };

  if (n_my > 0) {
    Tile<DT, D> ta, tb;
    load_table(0);
    fetch(ta, 0);
    for (int i = 0; i < n_my; i += 2) {
      if (i + 1 < n_my) {
        if (((i + 1) & 63) == 0) load_table(i + 1);
        fetch(tb, i + 1);
      }
      process_block<DT, D, G>(st, ta, qf, tok0_of(i), tok_end, a.scale_log2);
      if (i + 1 >= n_my) break;
      if (i + 2 < n_my) {
        if (((i + 2) & 63) == 0) load_table(i + 2);
        fetch(ta, i + 2);
      }
      process_block<DT, D, G>(st, tb, qf, tok0_of(i + 1), tok_end, a.scale_log2);
    }
  }

  // Reduce the lane-partial l and O over the four rows, then merge the waves via LDS.
  st.l += __shfl_xor(st.l, 16);
  st.l += __shfl_xor(st.l, 32);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < G_::kEPL; ++e) {
      st.o[h][e] += __shfl_xor(st.o[h][e], 16);
      st.o[h][e] += __shfl_xor(st.o[h][e], 32);
    }
  if (r == 0) {
    if (c < G) {
      sm_m[wave][c] = st.m;
      sm_l[wave][c] = st.l;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < G_::kEPL; ++e) sm_o[wave][h][c * G_::kEPL + e] = st.o[h][e];
  }
  if (lane == 0) sm_bad[wave] = bad;
  __syncthreads();

  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) any_bad |= sm_bad[w];
  const float qnan = __builtin_nanf("");
  for (int i = tid; i < G * D; i += 256) {
    const int h = i / D, dd = i - h * D;
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, sm_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float f = exp2_fast(sm_m[w][h] - M);   // 0 for a wave that saw no block
      L = fmaf(sm_l[w][h], f, L);
      O = fmaf(sm_o[w][h][dd], f, O);
    }
    const size_t row = (size_t)b * H + j * G + h;
    if (n_part == 1) {
      store_elem<DT>(a.out, row * D + dd, any_bad ? qnan : O / L);
    } else {
      const size_t slot = row * a.max_partitions + p;
      a.ws_o[slot * D + dd] = any_bad ? qnan : O;
      if (dd == 0) {
        a.ws_m[slot] = any_bad ? qnan : M;
        a.ws_l[slot] = any_bad ? qnan : L;
      }
    }
  }
}

// One workgroup per (sequence, query head): combine that head's partitions.
template <int DT, int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
  constexpr int Q4 = D / 4;          // float4 chunks per output row
  constexpr int PR = 256 / Q4;       // partitions read side by side
  const int bh = blockIdx.x;
  const int b = bh / a.n_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_ctx = a.context_lens[b];
  if (n_ctx < 1 || n_ctx > a.max_context_len) return;     // decode wrote NaN
  const int n_part = (n_ctx + a.partition_tokens - 1) / a.partition_tokens;
  if (n_part <= 1) return;                               // decode wrote the output

  const float* m = a.ws_m + (size_t)bh * a.max_partitions;
  const float* l = a.ws_l + (size_t)bh * a.max_partitions;
  const float* o = a.ws_o + (size_t)bh * a.max_partitions * D;

  __shared__ float red[4];
  __shared__ f32x4 part[PR][Q4];

  float mx = -INFINITY;
  for (int i = tid; i < n_part; i += 256) mx = fmaxf(mx, m[i]);
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();

  float sum = 0.f;
  for (int i = tid; i < n_part; i += 256) sum = fmaf(l[i], exp2_fast(m[i] - M), sum);
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) sum += __shfl_xor(sum, s);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  const float L = (red[0] + red[1]) + (red[2] + red[3]);

  const int q = tid % Q4, pr = tid / Q4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int i = pr; i < n_part; i += PR) {
    const float f = exp2_fast(m[i] - M);
    acc += f * reinterpret_cast<const f32x4*>(o + (size_t)i * D)[q];
  }
  part[pr][q] = acc;
  __syncthreads();
  if (tid < Q4) {
    f32x4 t = part[0][tid];
#pragma unroll
    for (int k = 1; k < PR; ++k) t += part[k][tid];
    const float inv = 1.0f / L;
#pragma unroll
    for (int x = 0; x < 4; ++x) store_elem<DT>(a.out, (size_t)bh * D + 4 * tid + x, t[x] * inv);
  }
}

template <int DT, int D, int G>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.max_partitions, a.n_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_kernel<DT, D, G>), grid, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_partitions <= 1) return e;
  hipLaunchKernelGGL((merge_kernel<DT, D>), dim3(a.num_seqs * a.n_heads), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_group(const DecodeArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_typed<DT, D, 1>(a, stream);
    case 2: return launch_typed<DT, D, 2>(a, stream);
    case 4: return launch_typed<DT, D, 4>(a, stream);
    case 8: return launch_typed<DT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_dim(const DecodeArgs& a, int d_head, int group, hipStream_t stream) {
  if (d_head == 64) return launch_group<DT, 64>(a, group, stream);
  if (d_head == 128) return launch_group<DT, 128>(a, group, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int dtype, int d_head, int group, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_dim<0>(a, d_head, group, stream);
    case 1: return launch_dim<1>(a, d_head, group, stream);
    case 2: return launch_dim<2>(a, d_head, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
