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
// are cut into partitions of P tokens (a multiple of the 16-token block). One wave owns
// one (KV head, partition, sequence) and all G query heads of that KV head, so each K/V
// byte is read from HBM once. A workgroup holds NW waves = NW consecutive KV heads of the
// same partition: together they read whole token rows (all heads of a token are
// contiguous in the pool), which keeps each compute unit's request stream on neighbouring
// bytes. Waves never wait for each other. A sequence with one partition is finished in
// place; otherwise each wave writes its (m, l, O) to the workspace and merge_kernel
// combines the partitions by the same rescale rule.
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
// K and V are prefetched into registers one block ahead (stream_tiles_pipelined for the
// single-query kernels, stream_tiles for the multi-query and quantized ones). V rows are
// read with the non-temporal hint (each byte is used once); K keeps the default policy
// because two consecutive loads of a wave share each 128-byte line.

#include <hip/hip_runtime.h>

#include <atomic>

#include "pkv_internal.h"

#ifndef PKV_DECODE_DTYPE
#error "compile pkv_decode.hip once per dtype: -DPKV_DECODE_DTYPE=0 (f32), 1 (f16) or 2 (bf16)"
#endif

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));


template <int DT> struct ElemBytes { static constexpr int value = DT == 0 ? 4 : 2; };

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float as_f(unsigned u) { return __builtin_bit_cast(float, u); }

// Maximum over the four 16-lane rows of each column c (lanes c, c + 16, c + 32, c + 48),
// in every lane: the butterfly over lane bits 4 and 5 with gfx950's VALU row swaps
// (v_permlane16_swap / v_permlane32_swap), which need neither LDS nor a wait on it, where
// a lane shuffle is a ds_bpermute and an LDS round trip in each block's dependency chain.
// permlane16_swap(x, x) returns rows (0, 0, 2, 2) and (1, 1, 3, 3) of x;
// permlane32_swap(x, x) rows (0, 1, 0, 1) and (2, 3, 2, 3).
__device__ __forceinline__ float max_over_rows(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(as_f(s16[0]), as_f(s16[1]));
  const unsigned v = __builtin_bit_cast(unsigned, y);
  const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(as_f(s32[0]), as_f(s32[1]));
}

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
  // Blocks loaded ahead of the one being computed: two, unless one block already takes
  // 64 registers per lane (fp32 with d_head 128).
  static constexpr int kDepth = (4 * kNK + 4 * kVW) <= 32 ? 2 : 1;
};

// One block's K and V as held by one lane.
template <int DT, int D>
struct Tile {
  u32x4 k[Geo<DT, D>::kNK];
  unsigned v[4][Geo<DT, D>::kVW];
};

// kblk / vblk: the block's base in the K and V pools (the same for the whole wave, so it
// lives in scalar registers); k_lane / v_lane: this lane's byte offsets inside the block,
// which fit 32 bits (a block is at most 16 * 256 * 128 * 4 bytes), so each load is the
// scalar-base + 32-bit-offset form and needs no 64-bit address arithmetic per lane.
// V loads carry the non-temporal hint when each V byte is used once (NT_V); the shared-
// prefix tasks, whose four waves per KV head read the same blocks, keep them cacheable.
template <typename T, bool NT>
__device__ __forceinline__ T load_v(const char* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  else
    return *reinterpret_cast<const T*>(p);
}

template <int DT, int D, bool NT_V = true>
__device__ __forceinline__ void load_tile(Tile<DT, D>& t, const char* kblk, const char* vblk,
                                          uint32_t k_lane, uint32_t v_lane, uint32_t tok_stride) {
  using G_ = Geo<DT, D>;
#pragma unroll
  for (int kk = 0; kk < G_::kNK; ++kk)
    t.k[kk] = *reinterpret_cast<const u32x4*>(kblk + (k_lane + 64u * kk));
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const char* src = vblk + (v_lane + jj * tok_stride);
    if constexpr (G_::kVW == 8) {
      const u32x4 a0 = load_v<u32x4, NT_V>(src);
      const u32x4 a1 = load_v<u32x4, NT_V>(src + 16);
#pragma unroll
      for (int x = 0; x < 4; ++x) { t.v[jj][x] = a0[x]; t.v[jj][4 + x] = a1[x]; }
    } else if constexpr (G_::kVW == 4) {
      const u32x4 a0 = load_v<u32x4, NT_V>(src);
#pragma unroll
      for (int x = 0; x < 4; ++x) t.v[jj][x] = a0[x];
    } else {
      const u32x2 a0 = load_v<u32x2, NT_V>(src);
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

// One 16-token block starting at token blk_tok0; tokens >= tok_end are masked. PARTIAL:
// the block holds such tokens (only the last block of a sequence can); full blocks are
// compiled without the masking.
template <int DT, int D, int G, bool PARTIAL>
__device__ __forceinline__ void process_block(WaveState<DT, D, G>& st, const Tile<DT, D>& t,
                                              const u32x4 (&qf)[Geo<DT, D>::kNK], int blk_tok0,
                                              int tok_end, float scale_log2, int r) {
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
  constexpr bool partial = PARTIAL;
  const int tok0 = blk_tok0 + 4 * r;
  float s[4];
  if (partial) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = (tok0 + i < tok_end) ? acc[i] * scale_log2 : -INFINITY;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = acc[i] * scale_log2;
  }

  float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  bm = max_over_rows(bm);
  const float m_new = fmaxf(st.m, bm);       // finite: every block has a valid token
  const float alpha = exp2_fast(st.m - m_new);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = exp2_fast(s[i] - m_new);
  st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
  st.m = m_new;

  // once the maxima settle, alpha is exactly 1 in every column: skip the identity rescale
  if (__any(alpha != 1.0f)) {
    static_for<G>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const float a = row_bcast<h>(alpha);
#pragma unroll
      for (int e = 0; e < G_::kEPL; ++e) st.o[h][e] *= a;
    });
  }

#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    float v[G_::kEPL];
    widen<DT, G_::kVW>(t.v[jj], v);
    if (partial) {
      const bool valid = tok0 + jj < tok_end;
#pragma unroll
      for (int e = 0; e < G_::kEPL; ++e) v[e] = valid ? v[e] : 0.f;   // unused slots may hold NaN
    }
    static_for<G>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const float ph = row_bcast<h>(p[jj]);
#pragma unroll
      for (int e = 0; e < G_::kEPL; ++e) st.o[h][e] = fmaf(ph, v[e], st.o[h][e]);
    });
  }
}

// Store EPL consecutive outputs of one lane (16 or 8 bytes for 16-bit types).
template <int DT, int EPL>
__device__ __forceinline__ void store_row_chunk(void* base, size_t idx, const float* v) {
  if constexpr (DT == 0) {
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const f32x4 x = {v[e], v[e + 1], v[e + 2], v[e + 3]};
      *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx + e) = x;
    }
  } else {
    unsigned w[EPL / 2];
#pragma unroll
    for (int e = 0; e < EPL; e += 2) {
      if constexpr (DT == 1) {
        const f16x2 h = {(_Float16)v[e], (_Float16)v[e + 1]};
        w[e / 2] = __builtin_bit_cast(unsigned, h);
      } else {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 h = {(__bf16)v[e], (__bf16)v[e + 1]};
        w[e / 2] = __builtin_bit_cast(unsigned, h);
      }
    }
    if constexpr (EPL == 8) {
      const u32x4 x = {w[0], w[1], w[2], w[3]};
      *reinterpret_cast<u32x4*>(static_cast<char*>(base) + idx * 2) = x;
    } else {
      const u32x2 x = {w[0], w[1]};
      *reinterpret_cast<u32x2*>(static_cast<char*>(base) + idx * 2) = x;
    }
  }
}

// Stream blocks [blk_begin, blk_begin + n_my) of sequence b through one wave: table
// entries are preloaded 64 at a time into a VGPR, the tiles of the next kDepth blocks are in
// flight (`load(tile, physical_block)`) while `process(tile, first_token_of_block)` runs on
// the current one. bad is set if a table entry is outside the pool (that block's data is
// then not read).
template <typename TileT, int kDepth, typename L, typename F>
__device__ __forceinline__ void stream_tiles(const DecodeArgs& a, int b, int blk_begin, int n_my,
                                             int lane, int& bad, L&& load, F&& process) {
  const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks_per_seq + blk_begin;
  int tbl = 0;   // lane i holds the table entry of block (chunk * 64 + i) of the range
  auto load_table = [&](int first) {
    const int i = first + lane;
    tbl = i < n_my ? trow[i] : 0;
  };
  auto fetch = [&](TileT& t, int i) {
    int pb = __builtin_amdgcn_readlane(tbl, i & 63);
    const bool ok = (unsigned)pb < (unsigned)a.num_blocks;
    bad |= !ok;
    load(t, ok ? pb : 0);
  };

  constexpr int NB = kDepth + 1;
  TileT tt[NB];
  load_table(0);
#pragma unroll
  for (int d0 = 0; d0 < kDepth; ++d0)
    if (d0 < n_my) fetch(tt[d0], d0);
  for (int i0 = 0; i0 < n_my; i0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int i = i0 + u;
      if (i >= n_my) break;
      if (i + kDepth < n_my) {
        if (((i + kDepth) & 63) == 0) load_table(i + kDepth);
        fetch(tt[(u + kDepth) % NB], i + kDepth);
      }
      process(tt[u], (blk_begin + i) * kBlockTokens);
    }
  }
}

// The same stream with a branch-free steady-state loop: every iteration loads one table
// entry (for the block it fetches next time) and one tile, so the compiler's wait analysis
// sees the same sequence of loads on every path and waits for exactly the tile being
// processed. In stream_tiles the table refill every 64 blocks and the fetches skipped in the
// last iterations make it wait for every outstanding load before each fetch; there the
// wave keeps one block in flight, fetched a whole block ahead. With kDepth = 1 this loop
// keeps one block in flight too, but without the drains and with the last blocks in a
// loop of their own; the single-query kernels and the 8-bit kernels (one block ahead) and
// the shared-prefix tasks (kPrefixDepth ahead) run faster with it, the multi-query kernels
// do not and keep stream_tiles. `first_entry` is the table entry of block blk_begin, loaded
// by the caller (the split kernel loads each segment's while the previous one streams, so
// a segment's first tile is not waiting for a table load). `begin()` runs once, before the
// first tile's load is issued. With kEntryRing the table entries go through a ring of NB
// registers instead, each loaded a whole unroll group (NB iterations) before its fetch, so
// waiting for an entry never waits for the tiles issued after it either; the private
// segments of the shared-prefix launch stream two blocks ahead this way.
template <typename TileT, int kDepth, bool kEntryRing = false, typename L, typename F,
          typename S>
__device__ __forceinline__ void stream_tiles_pipelined(const DecodeArgs& a, int b, int blk_begin,
                                                       int n_my, int first_entry, int& bad,
                                                       L&& load, F&& process, S&& begin) {
  const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks_per_seq + blk_begin;
  auto entry = [&](int i) { return trow[min(i, n_my - 1)]; };   // same address in all lanes
  auto fetch = [&](TileT& t, int pb) {
    pb = __builtin_amdgcn_readfirstlane(pb);
    const bool ok = (unsigned)pb < (unsigned)a.num_blocks;
    bad |= !ok;
    load(t, ok ? pb : 0);
  };

  constexpr int NB = kDepth + 1;
  TileT tt[NB];
  if constexpr (kEntryRing) {
    // before iteration i, ent[i % NB] holds the entry of block i + kDepth (the block that
    // iteration fetches); block i's tile is tt[i % NB]
    int ent[NB];
    begin();
#pragma unroll
    for (int u = 0; u < NB; ++u) ent[u] = entry(kDepth + u);
#pragma unroll
    for (int d0 = 0; d0 < kDepth; ++d0) fetch(tt[d0], d0 == 0 ? first_entry : entry(d0));
    const int n_fetching = n_my - kDepth;
    int i0 = 0;
    for (; i0 + NB <= n_fetching; i0 += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int i = i0 + u;
        const int pb = ent[u];
        ent[u] = entry(i + kDepth + NB);
        fetch(tt[(u + kDepth) % NB], pb);
        process(tt[u], (blk_begin + i) * kBlockTokens);
      }
    }
    for (; i0 < n_my; i0 += NB) {            // at most NB + kDepth - 1 blocks, no refills
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int i = i0 + u;
        if (i >= n_my) break;
        if (i < n_fetching) fetch(tt[(u + kDepth) % NB], ent[u]);
        process(tt[u], (blk_begin + i) * kBlockTokens);
      }
    }
    return;
  }
  // Loads in the order of the loop body (entry of block d + 1, then tile d), so the loop is
  // entered with the same outstanding loads as it repeats with; a segment shorter than
  // kDepth blocks loads its last block again instead of skipping the load.
  int e_next = first_entry;                 // table entry of the next block to fetch
  begin();
#pragma unroll
  for (int d0 = 0; d0 < kDepth; ++d0) {
    const int pb = e_next;
    e_next = entry(d0 + 1);
    fetch(tt[d0], pb);
  }
  const int n_fetching = n_my - kDepth;     // iterations i < n_fetching fetch block i + kDepth
  int i0 = 0;
  for (; i0 + NB <= n_fetching; i0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int i = i0 + u;
      const int pb = e_next;
      e_next = entry(i + kDepth + 1);
      fetch(tt[(u + kDepth) % NB], pb);
      process(tt[u], (blk_begin + i) * kBlockTokens);
    }
  }
  for (; i0 < n_my; i0 += NB) {              // at most NB + kDepth - 1 blocks
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int i = i0 + u;
      if (i >= n_my) break;
      if (i < n_fetching) {
        const int pb = e_next;
        e_next = entry(i + kDepth + 1);
        fetch(tt[(u + kDepth) % NB], pb);
      }
      process(tt[u], (blk_begin + i) * kBlockTokens);
    }
  }
}

// stream_tiles over the K/V pools of KV head j in the storage dtype.
struct NoBegin {
  __device__ void operator()() const {}
};

template <int DT, int D, int kDepth = Geo<DT, D>::kDepth, bool NT_V = true,
          bool kPipelined = false, bool kEntryRing = false, typename F, typename S = NoBegin>
__device__ __forceinline__ void stream_blocks(const DecodeArgs& a, int b, int j, int blk_begin,
                                              int n_my, int first_entry, int lane, int& bad,
                                              F&& process, S&& begin = S{}) {
  using G_ = Geo<DT, D>;
  const int r = lane >> 4, c = lane & 15;
  const uint32_t tok_stride = (uint32_t)a.n_kv_heads * G_::kRow;    // bytes between tokens
  const size_t blk_stride = (size_t)tok_stride * kBlockTokens;
  const uint32_t head_off = (uint32_t)j * G_::kRow;
  const uint32_t k_lane = head_off + c * tok_stride + 16 * r;
  const uint32_t v_lane = head_off + (4 * r) * tok_stride + c * (G_::kEPL * G_::kE);
  auto load = [&](Tile<DT, D>& t, int pb) {
    load_tile<DT, D, NT_V>(t, a.k_pool + (size_t)pb * blk_stride,
                           a.v_pool + (size_t)pb * blk_stride, k_lane, v_lane, tok_stride);
  };
  if constexpr (kPipelined) {
    stream_tiles_pipelined<Tile<DT, D>, kDepth, kEntryRing>(a, b, blk_begin, n_my, first_entry,
                                                            bad, load, process, begin);
  } else {
    begin();
    stream_tiles<Tile<DT, D>, kDepth>(a, b, blk_begin, n_my, lane, bad, load, process);
  }
}

// Query fragments (MFMA B operand) for lane column c: 16-byte slices at 64*kk + 16*r of
// the query row `row` of the output layout, zero when the column is unused.
template <int DT, int D>
__device__ __forceinline__ void load_query(const DecodeArgs& a, bool used, size_t row, int r,
                                           u32x4 (&qf)[Geo<DT, D>::kNK]) {
  using G_ = Geo<DT, D>;
  const char* qrow = static_cast<const char*>(a.q) + (used ? row : 0) * G_::kRow;
#pragma unroll
  for (int kk = 0; kk < G_::kNK; ++kk) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    qf[kk] = used ? *reinterpret_cast<const u32x4*>(qrow + 64 * kk + 16 * r) : z;
  }
}

// One wave: blocks [blk_begin, blk_begin + n_my) of sequence b, KV head j, into st
// (lane-partial; finish_rows completes it). Tokens >= tok_end are masked.
// Fused append (kAppend): token t_new = N_b - 1 of sequence b is the one this launch
// appends; its K/V rows for KV head j are k_new / v_new[b][j]. The wave whose blocks
// include t_new's block loads the two rows into registers (one 16-byte piece per lane)
// before its stream and writes them to its LDS slot (1 KiB per wave) in the stream's begin
// hook, while the first table entry is in flight; the registers are dead before the block
// loop. When that block is processed its lanes take the token's slot from LDS instead of
// the pool's (new_into_tile), and after the stream the rows are stored into the slot
// (table[b][t_new / 16], t_new % 16) (new_into_pool). Exactly one wave per (b, j)
// processes that block and no other wave of the launch reads the slot, so the store needs
// no ordering within the launch; an out-of-range table entry skips it (the sequence's
// output is NaN anyway). (Direct-to-LDS loads, which the multi-query append uses, would
// make the compiler drain every outstanding load at each block of the pipelined stream:
// it treats each LDS access in the loop as possibly reading what they write.)
template <int DT, int D>
__device__ __forceinline__ u32x4 new_rows_load(const DecodeArgs& a, int b, int j, int lane) {
  constexpr int kL = Geo<DT, D>::kRow / 16;            // 16-byte pieces per row
  const size_t row = ((size_t)b * a.n_kv_heads + j) * Geo<DT, D>::kRow;
  u32x4 piece = {0u, 0u, 0u, 0u};
  if (lane < 2 * kL)                                    // lane l holds slot[l]
    piece = *reinterpret_cast<const u32x4*>((lane < kL ? a.k_new : a.v_new) + row +
                                            16 * (lane % kL));
  return piece;
}

template <int DT, int D>
__device__ __forceinline__ void new_into_tile(Tile<DT, D>& t, const u32x4* slot, int off,
                                              int lane) {
  using G_ = Geo<DT, D>;
  constexpr int kL = G_::kRow / 16;
  const int r = lane >> 4, c = lane & 15;
  const u32x4* sl = slot;         // written by this wave's begin hook
  if (c == off) {                 // K: this lane's pieces 4 kk + r of the K row
#pragma unroll
    for (int kk = 0; kk < G_::kNK; ++kk) t.k[kk] = sl[4 * kk + r];
  }
  // V: lanes of row r = off / 4 hold token off in t.v[off % 4]; chunk c of the V row
  const unsigned* vrow = reinterpret_cast<const unsigned*>(sl + kL) + c * G_::kVW;
  unsigned w[G_::kVW];
#pragma unroll
  for (int x = 0; x < G_::kVW; ++x) w[x] = vrow[x];
  const bool vrow_mine = r == (off >> 2);
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const bool take = vrow_mine && jj == (off & 3);
#pragma unroll
    for (int x = 0; x < G_::kVW; ++x) t.v[jj][x] = take ? w[x] : t.v[jj][x];
  }
}

template <int DT, int D>
__device__ __forceinline__ void new_into_pool(const DecodeArgs& a, const u32x4* slot, int b,
                                              int j, int t_new, int lane) {
  constexpr int kL = Geo<DT, D>::kRow / 16;
  const int pb = a.block_tables[(size_t)b * a.max_blocks_per_seq + (t_new >> 4)];
  if ((unsigned)pb >= (unsigned)a.num_blocks || lane >= 2 * kL) return;
  const size_t dst = (((size_t)pb * kBlockTokens + (t_new & (kBlockTokens - 1))) *
                      a.n_kv_heads + j) * Geo<DT, D>::kRow + 16 * (lane % kL);
  char* pool = const_cast<char*>(lane < kL ? a.k_pool : a.v_pool);
  *reinterpret_cast<u32x4*>(pool + dst) = slot[lane];
}

template <int DT, int D, int G, bool kAppend, bool kTwoAhead = false>
__device__ __forceinline__ void attend(WaveState<DT, D, G>& st, int& bad, const DecodeArgs& a,
                                       int b, int j, int blk_begin, int n_my, int tok_end,
                                       int n_ctx, int first_entry, int lane) {
  const int r = lane >> 4, c = lane & 15;
  u32x4 qf[Geo<DT, D>::kNK];
  load_query<DT, D>(a, c < G, (size_t)b * a.n_heads + (size_t)j * G + c, r, qf);
  const int t_new = n_ctx - 1;
  const int new_tok0 = t_new & ~(kBlockTokens - 1);
  const bool has_new = kAppend && (new_tok0 >> 4) >= blk_begin && (new_tok0 >> 4) < blk_begin + n_my;
  u32x4* slot = nullptr;
  u32x4 piece = {0u, 0u, 0u, 0u};
  if constexpr (kAppend) {
    __shared__ u32x4 sm_new[8][64];                     // one 1 KiB slot per wave
    slot = sm_new[threadIdx.x >> 6];
    if (has_new) piece = new_rows_load<DT, D>(a, b, j, lane);
  }
  // the pipelined stream one block ahead (two measured no faster); kTwoAhead: two blocks
  // ahead with the table entries in a ring (the shared-prefix launch's private segments,
  // which are short, so a wave starts many of them)
  stream_blocks<DT, D, kTwoAhead ? 2 : 1, true, true, kTwoAhead>(
      a, b, j, blk_begin, n_my, first_entry, lane, bad, [&](Tile<DT, D>& t, int tok0) {
    if constexpr (kAppend)
      if (tok0 == new_tok0) new_into_tile<DT, D>(t, slot, t_new & (kBlockTokens - 1), lane);
    // only the last block of a sequence can be partial (partitions are block aligned)
    if (tok0 + kBlockTokens > tok_end)
      process_block<DT, D, G, true>(st, t, qf, tok0, tok_end, a.scale_log2, r);
    else
      process_block<DT, D, G, false>(st, t, qf, tok0, tok_end, a.scale_log2, r);
  }, [&]() {
    if constexpr (kAppend)
      if (has_new) slot[lane] = piece;
  });
  if constexpr (kAppend)
    if (has_new) new_into_pool<DT, D>(a, slot, b, j, t_new, lane);
}

// ---------------------------------------------------------------------------------------
// Several new tokens per sequence (q_len = QL > 1): the 16 MFMA columns are the pairs
// (new query i, head h), column c = i * G + h, C = G * QL <= 16. Query i of sequence b sees
// tokens 0 .. N_b - QL + i (the causal mask of "09-inference-optimization", KV Cache). With
// every column in use, P.V also runs on the matrix cores: lane (r, c) holds
// V[tokens 4r..4r+3][d = EPL*c + e] — the A operand of instance e — and
// P[column c][tokens 4r..4r+3], its own softmax output — the B operand (fp32:
// v_mfma_f32_16x16x4_f32, one token per instance; 16-bit types: one 16x16x16 instance per
// e over the whole block). No broadcast is needed; the result lands as
// O[column c][d = EPL*(4r'+i) + e] in accumulator e, element i.
// ---------------------------------------------------------------------------------------

template <int DT, int D>
struct MqState {
  float m = -INFINITY;                          // running max (base 2) of column c
  float l = 0.f;                                // lane-partial running sum of column c
  f32x4 o[Geo<DT, D>::kEPL] = {};               // see above
};

// lim: this lane's column sees tokens < lim; lim_min: the smallest lim of the wave.
// PARTIAL: some column sees only part of the block (blk_tok0 + 16 > lim_min); blocks seen
// whole by every column are compiled without the masking.
template <int DT, int D, bool PARTIAL>
__device__ __forceinline__ void process_block_mq(MqState<DT, D>& st, const Tile<DT, D>& t,
                                                 const u32x4 (&qf)[Geo<DT, D>::kNK], int blk_tok0,
                                                 int tok_end, int lim, int lim_min,
                                                 float scale_log2, int r) {
  using G_ = Geo<DT, D>;
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
  constexpr bool partial = PARTIAL;
  const int tok0 = blk_tok0 + 4 * r;
  float s[4];
  if constexpr (partial) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = (tok0 + i < lim) ? acc[i] * scale_log2 : -INFINITY;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = acc[i] * scale_log2;
  }
  float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  bm = max_over_rows(bm);
  const float m_new = fmaxf(st.m, bm);
  // a column can see none of a block's tokens (its causal limit lies before the block)
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = exp2_fast(st.m - m_use);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = exp2_fast(s[i] - m_use);
  if (__any(alpha != 1.0f)) {                 // skip the identity rescale
#pragma unroll
    for (int e = 0; e < G_::kEPL; ++e) st.o[e] *= alpha;
  }
  const bool tail = partial && blk_tok0 + kBlockTokens > tok_end;   // lim_min <= tok_end
  if constexpr (DT == 0) {
    st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float v[G_::kEPL];
      widen<DT, G_::kVW>(t.v[jj], v);
      if (tail) {
        const bool valid = tok0 + jj < tok_end;
#pragma unroll
        for (int e = 0; e < G_::kEPL; ++e) v[e] = valid ? v[e] : 0.f;   // unused slots may hold NaN
      }
#pragma unroll
      for (int e = 0; e < G_::kEPL; ++e)
        st.o[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[e], p[jj], st.o[e], 0, 0, 0);
    }
  } else {
    // 16-bit storage: P is rounded to the storage type and multiplied into V with
    // v_mfma_f32_16x16x16_{bf16,f16}, whose K = 16 is the block's 16 tokens. Lane (r, c)
    // supplies A = V[tokens 4r..4r+3][d = EPL*c + e] and B = P[tokens 4r..4r+3][column c];
    // the running sum takes the rounded P, so O / l stays a convex combination of V rows.
    unsigned pw[2];
    if constexpr (DT == 2) {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 p01 = {(__bf16)p[0], (__bf16)p[1]}, p23 = {(__bf16)p[2], (__bf16)p[3]};
      pw[0] = __builtin_bit_cast(unsigned, p01);
      pw[1] = __builtin_bit_cast(unsigned, p23);
      st.l = st.l * alpha + ((as_f(pw[0] << 16) + as_f(pw[0] & 0xFFFF0000u)) +
                             (as_f(pw[1] << 16) + as_f(pw[1] & 0xFFFF0000u)));
    } else {
      const f16x2 p01 = {(_Float16)p[0], (_Float16)p[1]}, p23 = {(_Float16)p[2], (_Float16)p[3]};
      pw[0] = __builtin_bit_cast(unsigned, p01);
      pw[1] = __builtin_bit_cast(unsigned, p23);
      st.l = st.l * alpha + (((float)p01[0] + (float)p01[1]) + ((float)p23[0] + (float)p23[1]));
    }
    const u32x2 pb = {pw[0], pw[1]};
    unsigned w[4][G_::kVW];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const bool valid = !tail || tok0 + jj < tok_end;      // unused slots may hold NaN
#pragma unroll
      for (int x = 0; x < G_::kVW; ++x) w[jj][x] = valid ? t.v[jj][x] : 0u;
    }
#pragma unroll
    for (int e = 0; e < G_::kEPL; ++e) {
      // one byte permute per word: {tokens 4r+1, 4r} and {4r+3, 4r+2} of element e
      // (v_perm_b32 selects from {S0, S1}: bytes 0-3 are S1's, 4-7 S0's)
      const int x = e >> 1;
      const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
      u32x2 va;
      va[0] = __builtin_amdgcn_perm(w[1][x], w[0][x], sel);
      va[1] = __builtin_amdgcn_perm(w[3][x], w[2][x], sel);
      if constexpr (DT == 2) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        st.o[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            __builtin_bit_cast(bf16x4, va), __builtin_bit_cast(bf16x4, pb), st.o[e], 0, 0, 0);
      } else {
        typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
        st.o[e] = __builtin_amdgcn_mfma_f32_16x16x16f16(
            __builtin_bit_cast(f16x4, va), __builtin_bit_cast(f16x4, pb), st.o[e], 0, 0, 0);
      }
    }
  }
  st.m = m_new;
}

// Output row of column c of KV head j: [b][i][j*G + h] in the [B, q_len, H] row layout.
template <int G>
__device__ __forceinline__ size_t mq_row(const DecodeArgs& a, int b, int j, int c) {
  const int i = c / G, h = c - i * G;
  return ((size_t)b * a.q_len + i) * a.n_heads + (size_t)j * G + h;
}

// Fused append of q_len > 1 tokens (kAppend): tokens t0n = N_b - q_len .. N_b - 1 of
// sequence b are appended by this launch; row i of k_new / v_new[b][i][j] is token
// t0n + i's K / V for KV head j. As for one token (attend with kAppend), a wave whose
// blocks hold any of them copies all q_len rows into its LDS slot with direct-to-LDS loads
// before its first tile, takes the new tokens' slots of a tile from LDS, and after the
// stream stores the rows of the tokens in its own blocks into their pool slots. The (at
// most two) blocks holding new tokens may belong to different waves; each writes only its
// own blocks, which no other wave of the launch reads.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void global_void_t;

template <int DT, int D, int G>
struct NewRowsMq {
  static constexpr int kL = Geo<DT, D>::kRow / 16;      // 16-byte pieces per row
  static constexpr int kRowsMax = 16 / G;               // q_len <= 16 / G
  static constexpr int kVOff = kRowsMax * kL;           // V rows follow the K rows
  static constexpr int kPieces = 2 * kVOff;
};

template <int DT, int D, int G>
__device__ __forceinline__ void new_rows_to_lds_mq(const DecodeArgs& a, int b, int j, int lane,
                                                   u32x4* slot) {
  using N_ = NewRowsMq<DT, D, G>;
  const int n = a.q_len * N_::kL;                       // pieces of the K (or V) rows
  for (int x0 = 0; x0 < n; x0 += 64) {
    const int x = x0 + lane, i = x / N_::kL, pc = x - i * N_::kL;
    const size_t row = (((size_t)b * a.q_len + i) * a.n_kv_heads + j) * Geo<DT, D>::kRow;
    if (x < n) {
      __builtin_amdgcn_global_load_lds((global_void_t*)(a.k_new + row + 16 * pc),
                                       (lds_void_t*)(slot + x0), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((global_void_t*)(a.v_new + row + 16 * pc),
                                       (lds_void_t*)(slot + N_::kVOff + x0), 16, 0, 0);
    }
  }
}

template <int DT, int D, int G>
__device__ __forceinline__ void new_into_tile_mq(Tile<DT, D>& t, const u32x4* slot, int tok0,
                                                 int t0n, int q_len, int lane) {
  using G_ = Geo<DT, D>;
  using N_ = NewRowsMq<DT, D, G>;
  const int r = lane >> 4, c = lane & 15;
  int z;                                                // orders the LDS reads after the tile
  asm volatile("v_mov_b32 %0, 0" : "=v"(z) : "v"(t.k[0][0]));
  const u32x4* sl = slot + z;
  const int tk = tok0 + c - t0n;                        // new-token row of this lane's K
  if ((unsigned)tk < (unsigned)q_len) {
#pragma unroll
    for (int kk = 0; kk < G_::kNK; ++kk) t.k[kk] = sl[tk * N_::kL + 4 * kk + r];
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {                      // token 4r + jj, chunk c of its V row
    const int tv = tok0 + 4 * r + jj - t0n;
    const bool take = (unsigned)tv < (unsigned)q_len;
    const unsigned* vrow =
        reinterpret_cast<const unsigned*>(sl + N_::kVOff + (take ? tv : 0) * N_::kL) + c * G_::kVW;
#pragma unroll
    for (int x = 0; x < G_::kVW; ++x) {
      const unsigned w = vrow[x];
      t.v[jj][x] = take ? w : t.v[jj][x];
    }
  }
}

template <int DT, int D, int G>
__device__ __forceinline__ void new_into_pool_mq(const DecodeArgs& a, const u32x4* slot, int b,
                                                 int j, int t0n, int blk_begin, int n_my,
                                                 int lane) {
  using N_ = NewRowsMq<DT, D, G>;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // the direct-to-LDS loads are done
  const int n = a.q_len * N_::kL;
  for (int x = lane; x < n; x += 64) {
    const int i = x / N_::kL, pc = x - i * N_::kL;
    const int tok = t0n + i, blk = tok >> 4;
    if (blk < blk_begin || blk >= blk_begin + n_my) continue;   // another wave's block
    const int pb = a.block_tables[(size_t)b * a.max_blocks_per_seq + blk];
    if ((unsigned)pb >= (unsigned)a.num_blocks) continue;
    const size_t dst = (((size_t)pb * kBlockTokens + (tok & (kBlockTokens - 1))) * a.n_kv_heads +
                        j) * Geo<DT, D>::kRow + 16 * pc;
    *reinterpret_cast<u32x4*>(const_cast<char*>(a.k_pool) + dst) = slot[x];
    *reinterpret_cast<u32x4*>(const_cast<char*>(a.v_pool) + dst) = slot[N_::kVOff + x];
  }
}

template <int DT, int D, int G, bool kAppend>
__device__ __forceinline__ void attend_mq(MqState<DT, D>& st, int& bad, const DecodeArgs& a,
                                          int b, int j, int blk_begin, int n_my, int tok_end,
                                          int n_ctx, int lane) {
  const int C = G * a.q_len;
  const int r = lane >> 4, c = lane & 15;
  u32x4 qf[Geo<DT, D>::kNK];
  load_query<DT, D>(a, c < C, mq_row<G>(a, b, j, c < C ? c : 0), r, qf);
  const int first_visible_end = n_ctx - a.q_len + 1;     // limit of query 0
  const int lim = c < C ? min(tok_end, first_visible_end + c / G) : tok_end;
  const int lim_min = min(tok_end, first_visible_end);
  const int t0n = n_ctx - a.q_len;                      // first appended token (kAppend)
  const bool has_new = kAppend && (t0n >> 4) < blk_begin + n_my && ((n_ctx - 1) >> 4) >= blk_begin;
  u32x4* slot = nullptr;
  if constexpr (kAppend) {
    __shared__ u32x4 sm_new[8][NewRowsMq<DT, D, G>::kPieces];   // one slot per wave
    slot = sm_new[threadIdx.x >> 6];
    if (has_new) new_rows_to_lds_mq<DT, D, G>(a, b, j, lane, slot);
  }
  stream_blocks<DT, D>(a, b, j, blk_begin, n_my, 0, lane, bad, [&](Tile<DT, D>& t, int tok0) {
    if constexpr (kAppend)
      if (has_new && tok0 + kBlockTokens > t0n) new_into_tile_mq<DT, D, G>(t, slot, tok0, t0n, a.q_len, lane);
    if (tok0 + kBlockTokens > lim_min)
      process_block_mq<DT, D, true>(st, t, qf, tok0, tok_end, lim, lim_min, a.scale_log2, r);
    else
      process_block_mq<DT, D, false>(st, t, qf, tok0, tok_end, lim, lim_min, a.scale_log2, r);
  });
  if constexpr (kAppend)
    if (has_new) new_into_pool_mq<DT, D, G>(a, slot, b, j, t0n, blk_begin, n_my, lane);
}

template <int DT, int D, int G>
__device__ __forceinline__ void write_final_mq(const DecodeArgs& a, const MqState<DT, D>& st,
                                               int bad, int b, int j, int lane) {
  using G_ = Geo<DT, D>;
  const int r = lane >> 4, c = lane & 15;
  if (c >= G * a.q_len) return;
  const float inv = 1.0f / st.l;
  const float qnan = __builtin_nanf("");
  const size_t row = mq_row<G>(a, b, j, c);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[G_::kEPL];
#pragma unroll
    for (int e = 0; e < G_::kEPL; ++e) v[e] = bad ? qnan : st.o[e][i] * inv;
    store_row_chunk<DT, G_::kEPL>(a.out, row * D + G_::kEPL * (4 * r + i), v);
  }
}

// Record of column c at index rec(c).
template <int DT, int D, int G, typename R>
__device__ __forceinline__ void write_record_mq(const DecodeArgs& a, const MqState<DT, D>& st,
                                                int bad, int lane, R&& rec) {
  using G_ = Geo<DT, D>;
  const int r = lane >> 4, c = lane & 15;
  if (c >= G * a.q_len) return;
  const float qnan = __builtin_nanf("");
  const size_t idx = rec(c);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* dst = a.ws_o + idx * D + G_::kEPL * (4 * r + i);
#pragma unroll
    for (int e = 0; e < G_::kEPL; e += 4) {
      const f32x4 x = {bad ? qnan : st.o[e][i], bad ? qnan : st.o[e + 1][i],
                       bad ? qnan : st.o[e + 2][i], bad ? qnan : st.o[e + 3][i]};
      *reinterpret_cast<f32x4*>(dst + e) = x;
    }
  }
  if (r == 0) {
    a.ws_m[idx] = bad ? qnan : st.m;
    a.ws_l[idx] = bad ? qnan : st.l;
  }
}

// ---------------------------------------------------------------------------------------
// Quantized caches ("LLM 推理优化全景实战" §4.1 affine quantization; "Scaling Book 第 11 章"
// FP8 / INT8): K and V hold one 8-bit code per element and one (s, z) pair per token and
// KV head, x^ = s * (Q - z) (FP8: Q is the E4M3 value, z = 0). q and out stay 16-bit.
// Per block, lane (r, c) holds
//   * K codes of token c, elements (D/4) r .. (D/4) r + D/4 - 1. Each code converts
//     exactly to the 16-bit type, so the MFMA contracts q with the raw codes, the query
//     fragments using the same element mapping d = (D/4) r + 8 kk + i; the score of token
//     t is then s_t (q.Q_t - z_t sum(q)), the zero point entering once per token;
//   * V codes of tokens 4r .. 4r + 3, elements EPL c .. EPL c + EPL - 1, dequantized in
//     fp32 and rounded to the 16-bit type as the A operand of the P.V MFMA (the
//     multi-query layout with C = G columns);
//   * (s, z) of K and of V for tokens 4r .. 4r + 3.
// ---------------------------------------------------------------------------------------

template <int D>
struct QGeo {
  static constexpr int kNK = D / 64;           // 16-byte K code loads per lane per block
  static constexpr int kEPL = D / 16;          // V codes per lane per token
  static constexpr int kVW = kEPL / 4;         // V code words per lane per token
};

template <int D>
struct QTile {
  u32x4 k[QGeo<D>::kNK];
  unsigned v[4][QGeo<D>::kVW];
  // Lane (r, c) holds value c of row r's scales: c = 2i, 2i + 1 the K (s, z) of token
  // 4r + i, c = 8 + 2i, 9 + 2i its V (s, z). One register per lane instead of the 16 that
  // every lane of a row would hold as plain loads; the block processor takes each value
  // from its row with a DPP row broadcast.
  float sc;
};

// Two codes (bytes 2H, 2H + 1 of w) as fp32, exactly.
template <int FMT, int H>
__device__ __forceinline__ void codes_to_f32(unsigned w, float& x0, float& x1) {
  if constexpr (FMT == kKvInt8) {
    x0 = (float)((w >> (16 * H)) & 0xFFu);
    x1 = (float)((w >> (16 * H + 8)) & 0xFFu);
  } else {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, H != 0);   // OCP E4M3 on gfx950
    x0 = f[0];
    x1 = f[1];
  }
}

// Two fp32 values rounded (to nearest even) into one word of the 16-bit type DT.
// Two FP8 codes (bytes 2H, 2H + 1 of w) as a packed bf16 pair, low half first, with
// gfx950's v_cvt_scalef32_pk_bf16_fp8 at scale 1: every E4M3 value is exact in bf16, and
// the instruction decodes all 256 bytes bitwise as v_cvt_pk_f32_fp8 followed by rounding
// to bf16 (checked on the GPU), in one instruction instead of two.
template <int H>
__device__ __forceinline__ unsigned fp8_pair_bf16(unsigned w) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, H != 0));
}

template <int DT>
__device__ __forceinline__ unsigned pack16(float x0, float x1) {
  if constexpr (DT == 2) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 h = {(__bf16)x0, (__bf16)x1};
    return __builtin_bit_cast(unsigned, h);
  } else {
    const f16x2 h = {(_Float16)x0, (_Float16)x1};
    return __builtin_bit_cast(unsigned, h);
  }
}

// x rounded (to nearest even) to the 16-bit type DT, returned as fp32.
template <int DT>
__device__ __forceinline__ float round16(float x) {
  if constexpr (DT == 2)
    return (float)(__bf16)x;
  else
    return (float)(_Float16)x;
}

template <int DT>
__device__ __forceinline__ f32x4 mfma32(const u32x4& a, const u32x4& b, const f32x4& c) {
  if constexpr (DT == 2)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ f32x4 mfma16(const u32x2& a, const u32x2& b, const f32x4& c) {
  if constexpr (DT == 2) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                     __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
  } else {
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
}

// Query fragments for the code mapping d = (D/4) r + 8 kk + i, and sum(q) of column c.
template <int DT, int D>
__device__ __forceinline__ void load_query_q(const DecodeArgs& a, bool used, size_t row, int r,
                                             u32x4 (&qf)[D / 32], float& sumq) {
  const char* qrow = static_cast<const char*>(a.q) + (used ? row : 0) * (D * 2);
  float sum = 0.f;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    qf[kk] = used ? *reinterpret_cast<const u32x4*>(qrow + 2 * ((D / 4) * r + 8 * kk)) : z;
    unsigned w[4] = {qf[kk][0], qf[kk][1], qf[kk][2], qf[kk][3]};
    float x[8];
    widen<DT, 4>(w, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += x[i];
  }
  sum += __shfl_xor(sum, 16);
  sum += __shfl_xor(sum, 32);
  sumq = sum;
}

// Running state of a quantized-cache wave: the multi-query state plus, for INT8 codes
// with bf16 weights, the lane-partial zero-point term sum_t w_t z_t of column c.
template <int DT, int D>
struct QState : MqState<DT, D> {
  float corr = 0.f;
};

template <int DT, int D, int FMT>
__device__ __forceinline__ void process_block_q(QState<DT, D>& st, const QTile<D>& t,
                                                const u32x4 (&qf)[D / 32], float sumq,
                                                int blk_tok0, int tok_end, float scale_log2,
                                                int r) {
  constexpr int EPL = QGeo<D>::kEPL;
  constexpr int VW = QGeo<D>::kVW;
  // q . Q_t over the raw codes: kk-th group of 8 codes is bytes 8 kk .. 8 kk + 7 of this
  // lane's K chunk.
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const unsigned w0 = t.k[kk >> 1][(kk & 1) * 2], w1 = t.k[kk >> 1][(kk & 1) * 2 + 1];
    u32x4 a16;
    if constexpr (FMT == kKvFp8 && DT == 2) {
      a16 = u32x4{fp8_pair_bf16<0>(w0), fp8_pair_bf16<1>(w0), fp8_pair_bf16<0>(w1),
                  fp8_pair_bf16<1>(w1)};
    } else {
      float x[8];
      codes_to_f32<FMT, 0>(w0, x[0], x[1]);
      codes_to_f32<FMT, 1>(w0, x[2], x[3]);
      codes_to_f32<FMT, 0>(w1, x[4], x[5]);
      codes_to_f32<FMT, 1>(w1, x[6], x[7]);
      a16 = u32x4{pack16<DT>(x[0], x[1]), pack16<DT>(x[2], x[3]), pack16<DT>(x[4], x[5]),
                  pack16<DT>(x[6], x[7])};
    }
    acc = mfma32<DT>(a16, qf[kk], acc);
  }
  const float sk[4] = {row_bcast<0>(t.sc), row_bcast<2>(t.sc), row_bcast<4>(t.sc), row_bcast<6>(t.sc)};
  const float zk[4] = {row_bcast<1>(t.sc), row_bcast<3>(t.sc), row_bcast<5>(t.sc), row_bcast<7>(t.sc)};
  const bool tail = blk_tok0 + kBlockTokens > tok_end;
  const int tok0 = blk_tok0 + 4 * r;
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float dot = FMT == kKvInt8 ? fmaf(-zk[i], sumq, acc[i]) : acc[i];
    s[i] = dot * (sk[i] * scale_log2);
    if (tail) s[i] = tok0 + i < tok_end ? s[i] : -INFINITY;   // unused slots: NaN scales
  }
  float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  bm = max_over_rows(bm);
  const float m_new = fmaxf(st.m, bm);            // finite: every block has a valid token
  const float alpha = exp2_fast(st.m - m_new);
  st.m = m_new;
  if (__any(alpha != 1.0f)) {                     // skip the identity rescale
#pragma unroll
    for (int e = 0; e < EPL; ++e) st.o[e] *= alpha;
  }
  float sv[4] = {row_bcast<8>(t.sc), row_bcast<10>(t.sc), row_bcast<12>(t.sc), row_bcast<14>(t.sc)};
  float zv[4] = {row_bcast<9>(t.sc), row_bcast<11>(t.sc), row_bcast<13>(t.sc), row_bcast<15>(t.sc)};
  if (tail) {                                     // unused slots hold NaN scales
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = tok0 + i < tok_end ? sv[i] : 0.f;
      zv[i] = tok0 + i < tok_end ? zv[i] : 0.f;
    }
  }

  if constexpr (DT == 2) {
    // bf16: the V scale joins the weight, w_t = p_t s_t (bf16's exponent range holds any
    // product), the raw codes are the A operand (exact in bf16), and the zero point leaves
    // the sum as one term per token: O = sum_t w_t Q_t - sum_t w_t z_t.
    float p[4], w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2_fast(s[i] - m_new);
      w[i] = round16<DT>(p[i] * sv[i]);
    }
    st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    if constexpr (FMT == kKvInt8)
      st.corr = st.corr * alpha + ((w[0] * zv[0] + w[1] * zv[1]) + (w[2] * zv[2] + w[3] * zv[3]));
    const u32x2 wb = {pack16<DT>(w[0], w[1]), pack16<DT>(w[2], w[3])};   // exact
    unsigned vw[4][VW];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int x = 0; x < VW; ++x)            // codes of unused slots may decode to NaN
        vw[jj][x] = (!tail || tok0 + jj < tok_end) ? t.v[jj][x] : 0u;
    if constexpr (FMT == kKvFp8) {
      // byte e' of word x of tokens 2p and 2p + 1 side by side (one byte permute per two
      // elements), then each pair converted at once: va[p] for element 4x + e'
#pragma unroll
      for (int x = 0; x < VW; ++x) {
        unsigned lo[2], hi[2];
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          lo[pr] = __builtin_amdgcn_perm(vw[2 * pr + 1][x], vw[2 * pr][x], 0x05010400u);
          hi[pr] = __builtin_amdgcn_perm(vw[2 * pr + 1][x], vw[2 * pr][x], 0x07030602u);
        }
        const u32x2 v0 = {fp8_pair_bf16<0>(lo[0]), fp8_pair_bf16<0>(lo[1])};
        const u32x2 v1 = {fp8_pair_bf16<1>(lo[0]), fp8_pair_bf16<1>(lo[1])};
        const u32x2 v2 = {fp8_pair_bf16<0>(hi[0]), fp8_pair_bf16<0>(hi[1])};
        const u32x2 v3 = {fp8_pair_bf16<1>(hi[0]), fp8_pair_bf16<1>(hi[1])};
        st.o[4 * x] = mfma16<DT>(v0, wb, st.o[4 * x]);
        st.o[4 * x + 1] = mfma16<DT>(v1, wb, st.o[4 * x + 1]);
        st.o[4 * x + 2] = mfma16<DT>(v2, wb, st.o[4 * x + 2]);
        st.o[4 * x + 3] = mfma16<DT>(v3, wb, st.o[4 * x + 3]);
      }
    } else {
      float c[4][EPL];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int x = 0; x < VW; ++x) {
          codes_to_f32<FMT, 0>(vw[jj][x], c[jj][4 * x], c[jj][4 * x + 1]);
          codes_to_f32<FMT, 1>(vw[jj][x], c[jj][4 * x + 2], c[jj][4 * x + 3]);
        }
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const u32x2 va = {pack16<DT>(c[0][e], c[1][e]), pack16<DT>(c[2][e], c[3][e])};
        st.o[e] = mfma16<DT>(va, wb, st.o[e]);
      }
    }
  } else {
    // f16: the weights are rounded alone (an f16 product p s could fall below f16's range)
    // and the V rows are dequantized in fp32, then rounded to f16 as the A operand.
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = round16<DT>(exp2_fast(s[i] - m_new));
    const u32x2 pb = {pack16<DT>(pr[0], pr[1]), pack16<DT>(pr[2], pr[3])};   // exact
    st.l = st.l * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    float xv[4][EPL];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const bool valid = !tail || tok0 + jj < tok_end;
      const float bias = FMT == kKvInt8 ? -sv[jj] * zv[jj] : 0.f;
#pragma unroll
      for (int x = 0; x < VW; ++x) {
        float cc[4];
        codes_to_f32<FMT, 0>(t.v[jj][x], cc[0], cc[1]);
        codes_to_f32<FMT, 1>(t.v[jj][x], cc[2], cc[3]);
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[jj][4 * x + i] = valid ? fmaf(sv[jj], cc[i], bias) : 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const u32x2 va = {pack16<DT>(xv[0][e], xv[1][e]), pack16<DT>(xv[2][e], xv[3][e])};
      st.o[e] = mfma16<DT>(va, pb, st.o[e]);
    }
  }
}

template <int DT, int D, int G, int FMT>
__device__ __forceinline__ void attend_q(QState<DT, D>& st, int& bad, const DecodeArgs& a,
                                         int b, int j, int blk_begin, int n_my, int tok_end,
                                         int first_entry, int lane) {
  const int r = lane >> 4, c = lane & 15;
  u32x4 qf[D / 32];
  float sumq;
  load_query_q<DT, D>(a, c < G, (size_t)b * a.n_heads + (size_t)j * G + c, r, qf, sumq);
  const uint32_t tok_stride = (uint32_t)a.n_kv_heads * D;           // code bytes per token
  const size_t blk_stride = (size_t)tok_stride * kBlockTokens;
  const uint32_t head_off = (uint32_t)j * D;
  const uint32_t k_lane = head_off + c * tok_stride + (D / 4) * r;
  const uint32_t v_lane = head_off + (4 * r) * tok_stride + c * QGeo<D>::kEPL;
  const char* kc = static_cast<const char*>(a.k_pool);
  const char* vc = static_cast<const char*>(a.v_pool);
  // This lane's scale value (see QTile) in block pb: sc_base[pb * sc_blk].
  const float* sc_base =
      (c < 8 ? a.k_scales : a.v_scales) + (size_t)j * kBlockTokens * 2 + 8 * r + (c & 7);
  const size_t sc_blk = (size_t)a.n_kv_heads * kBlockTokens * 2;
  // The pipelined stream one block ahead: with the scales in one register per lane the
  // 8-bit kernels fit it; measured on the GQA shape against the former stream_tiles with 16
  // scale registers per tile, INT8 147.4 -> 142.0 us and FP8 145.2 -> 139.8 us, the outputs
  // bitwise unchanged (two and three blocks ahead: 143.2 / 140.6 and 144.2 / 141.5 us).
  stream_tiles_pipelined<QTile<D>, 1>(
      a, b, blk_begin, n_my, first_entry, bad,
      [&](QTile<D>& t, int pb) {
        const char* kb = kc + (size_t)pb * blk_stride;
        const char* vb = vc + (size_t)pb * blk_stride;
#pragma unroll
        for (int x = 0; x < QGeo<D>::kNK; ++x)
          t.k[x] = *reinterpret_cast<const u32x4*>(kb + (k_lane + 16u * x));
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const char* src = vb + (v_lane + jj * tok_stride);
          if constexpr (QGeo<D>::kVW == 2) {
            const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
            t.v[jj][0] = w[0];
            t.v[jj][1] = w[1];
          } else {
            t.v[jj][0] = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(src));
          }
        }
        t.sc = sc_base[(size_t)pb * sc_blk];
      },
      [&](const QTile<D>& t, int tok0) {
        process_block_q<DT, D, FMT>(st, t, qf, sumq, tok0, tok_end, a.scale_log2, r);
      },
      NoBegin{});
}

// Sum the lane-partial l and O over the four rows: afterwards every lane holds l of
// head c, and lane (r, c) holds O[h][chunk c] for every head h.
template <int DT, int D, int G>
__device__ __forceinline__ void finish_rows(WaveState<DT, D, G>& st) {
  st.l += __shfl_xor(st.l, 16);
  st.l += __shfl_xor(st.l, 32);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < Geo<DT, D>::kEPL; ++e) {
      st.o[h][e] += __shfl_xor(st.o[h][e], 16);
      st.o[h][e] += __shfl_xor(st.o[h][e], 32);
    }
}

// out[head_row0 + h] = O[h] / l[h] for the G heads of the wave.
template <int DT, int D, int G>
__device__ __forceinline__ void write_final(const DecodeArgs& a, const WaveState<DT, D, G>& st,
                                            int bad, size_t head_row0, int lane) {
  using G_ = Geo<DT, D>;
  const int r = lane >> 4, c = lane & 15;
  float inv[G];
  static_for<G>([&](auto hc) {
    constexpr int h = decltype(hc)::value;
    inv[h] = 1.0f / row_bcast<h>(st.l);
  });
  if (r != 0) return;
  const float qnan = __builtin_nanf("");
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float v[G_::kEPL];
#pragma unroll
    for (int e = 0; e < G_::kEPL; ++e) v[e] = bad ? qnan : st.o[h][e] * inv[h];
    store_row_chunk<DT, G_::kEPL>(a.out, (head_row0 + h) * D + c * G_::kEPL, v);
  }
}

// Partial record of head h at index rec(h).
template <int DT, int D, int G, typename R>
__device__ __forceinline__ void write_record(const DecodeArgs& a, const WaveState<DT, D, G>& st,
                                             int bad, int lane, R&& rec) {
  using G_ = Geo<DT, D>;
  const int r = lane >> 4, c = lane & 15;
  if (r != 0) return;
  const float qnan = __builtin_nanf("");
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float* dst = a.ws_o + rec(h) * D + c * G_::kEPL;
#pragma unroll
    for (int e = 0; e < G_::kEPL; e += 4) {
      const f32x4 x = {bad ? qnan : st.o[h][e], bad ? qnan : st.o[h][e + 1],
                       bad ? qnan : st.o[h][e + 2], bad ? qnan : st.o[h][e + 3]};
      *reinterpret_cast<f32x4*>(dst + e) = x;
    }
  }
  if (c < G) {
    const size_t idx = rec(c);
    a.ws_m[idx] = bad ? qnan : st.m;
    a.ws_l[idx] = bad ? qnan : st.l;
  }
}

template <int DT, int D>
__device__ __forceinline__ void write_nan_rows(const DecodeArgs& a, size_t row0, int rows,
                                               int tid, int nthreads) {
  for (int i = tid; i < rows * D; i += nthreads)
    store_elem<DT>(a.out, row0 * D + i, __builtin_nanf(""));
}

// A whole-sequence-or-segment of one wave: attend over blocks [blk_begin, +n_my) of
// sequence b for KV head j, then write the outputs (whole) or the records rec(column).
template <int DT, int D, int G, int MODE, typename R>
__device__ __forceinline__ void run_segment(const DecodeArgs& a, int b, int j, int blk_begin,
                                            int n_my, int tok_end, int n_ctx, bool whole,
                                            int first_entry, int lane, R&& rec) {
  int bad = 0;
  if constexpr (MODE == kModeQuantInt8 || MODE == kModeQuantFp8) {
    QState<DT, D> st;
    attend_q<DT, D, G, MODE == kModeQuantInt8 ? kKvInt8 : kKvFp8>(st, bad, a, b, j, blk_begin,
                                                                n_my, tok_end, first_entry, lane);
    st.l += __shfl_xor(st.l, 16);
    st.l += __shfl_xor(st.l, 32);
    if constexpr (MODE == kModeQuantInt8 && DT == 2) {     // O -= sum_t w_t z_t (column c)
      st.corr += __shfl_xor(st.corr, 16);
      st.corr += __shfl_xor(st.corr, 32);
#pragma unroll
      for (int e = 0; e < Geo<DT, D>::kEPL; ++e) st.o[e] -= st.corr;
    }
    if (whole)
      write_final_mq<DT, D, G>(a, st, bad, b, j, lane);
    else
      write_record_mq<DT, D, G>(a, st, bad, lane, rec);
  } else if constexpr (MODE == kModeSingle || MODE == kModeSingleAppend ||
                       MODE == kModeSinglePrefix) {
    WaveState<DT, D, G> st;
    attend<DT, D, G, MODE == kModeSingleAppend, MODE == kModeSinglePrefix>(
        st, bad, a, b, j, blk_begin, n_my, tok_end, n_ctx, first_entry, lane);
    finish_rows<DT, D, G>(st);
    if (whole)
      write_final<DT, D, G>(a, st, bad, (size_t)b * a.n_heads + (size_t)j * G, lane);
    else
      write_record<DT, D, G>(a, st, bad, lane, rec);
  } else {
    MqState<DT, D> st;
    attend_mq<DT, D, G, MODE == kModeMultiAppend>(st, bad, a, b, j, blk_begin, n_my, tok_end,
                                                n_ctx, lane);
    st.l += __shfl_xor(st.l, 16);
    st.l += __shfl_xor(st.l, 32);
    if (whole)
      write_final_mq<DT, D, G>(a, st, bad, b, j, lane);
    else
      write_record_mq<DT, D, G>(a, st, bad, lane, rec);
  }
}

__device__ __forceinline__ bool valid_len(const DecodeArgs& a, int n) {
  return n >= a.q_len && n <= a.max_context_len;
}

// Shared blocks skipped by the split pass for sequence b (0 without a group); -1 when the
// group id or its block count is out of range, or the shared blocks leave no private
// token (the new token never lives in a shared block).
__device__ __forceinline__ int shared_blocks_of(const DecodeArgs& a, int b, int n_ctx) {
  if (!a.seq_group) return 0;
  const int g = a.seq_group[b];
  if (g < 0) return 0;
  if (g >= a.n_groups) return -1;
  const int sb = a.group_blocks[g];
  return (sb < 0 || sb > a.max_blocks_per_seq || (long long)sb * kBlockTokens >= n_ctx) ? -1 : sb;
}

// Usable sequence for the split pass: its length is valid and its group (if any) is.
__device__ __forceinline__ bool usable(const DecodeArgs& a, int b, int n_ctx) {
  return valid_len(a, n_ctx) && shared_blocks_of(a, b, n_ctx) >= 0;
}

// Shares of the balanced split. Workgroup w < W takes the private units [begin(w),
// begin(w + 1)). Without prefix tasks begin(w) = floor(w T / W): equal shares. With them,
// workgroups w < Pw run one prefix task first and are given ceff fewer units:
// begin(w) = floor(w S / W) - ceff * min(w, Pw) with S = T + Pw * ceff, which still ends at
// begin(W) = T. ceff is capped so that every workgroup keeps at least one unit
// (floor(S / W) >= ceff + 1), hence the segments of one stream still come from consecutive
// workgroups. W is at most kSplitMaxWorkgroups (the records are sized for it) and gives
// each workgroup at least kSplitMinBlocks units.
struct SplitShares {
  long long T, W, Pw, ceff, S;
  __device__ long long begin(long long w) const { return w * S / W - ceff * min(w, Pw); }
  // the workgroup owning unit x < T: the largest w with begin(w) <= x
  __device__ long long owner(long long x) const {
    const long long w2 = ((x + ceff * Pw + 1) * W - 1) / S;   // among w >= Pw
    if (w2 >= Pw) return w2;
    return ((x + 1) * W - 1) / (S - ceff * W);                // begin(w) = floor(w (S - ceff W) / W)
  }
};

__device__ __forceinline__ SplitShares split_shares(const DecodeArgs& a, long long T, long long grid) {
  SplitShares x;
  x.T = T;
  x.W = min(min(grid, (long long)kSplitMaxWorkgroups), (T + kSplitMinBlocks - 1) / kSplitMinBlocks);
  x.Pw = min((long long)a.prefix_tasks, x.W);
  x.ceff = x.W > x.Pw ? max(0LL, min((long long)a.prefix_cost, (T - x.W) / (x.W - x.Pw))) : 0;
  x.S = T + x.Pw * x.ceff;
  return x;
}

// Prefix-task blocks in flight per wave on the register stream (fp32, or fewer than four
// waves per KV head): K and V of one block take 4 * kNK + 4 * kVW
// registers per lane; 64 registers go to prefetch (two blocks ahead for 16-bit d 128). On
// the pipelined stream two blocks ahead measured fastest for the shared-prefix workload
// (with the prefix work then in a kernel of its own): 84.4 us, against 85.4 / 85.6 /
// 86.7 us at 3 / 4 / 5 and 90.2 us at 8.
template <int DT, int D>
constexpr int kPrefixDepth =
    64 / (4 * Geo<DT, D>::kNK + 4 * Geo<DT, D>::kVW) > 1
        ? 64 / (4 * Geo<DT, D>::kNK + 4 * Geo<DT, D>::kVW) : 1;

// Blocks in flight per KV head in the staged prefix stream (four and six measured the same
// on the shared-prefix workload; four take fewer registers).
constexpr int kPrefixStage = 4;

// Whether a prefix task streams its blocks through prefix_stream_staged: four waves per KV
// head and a 16-bit dtype. The fp32 d 128 kernel already runs one wave per SIMD, and the
// staged stream made its shared-prefix attention slower (86.3 / 100.1 against 77.7 / 94.7
// us warm / cold on the 8 x 16-sequence batch, 16 / 4 heads); every 16-bit shape measured
// the same or faster.
inline __host__ __device__ bool prefix_staged(int dt, int wph) {
  return dt != 0 && wph == kPrefixWaves;
}

// s_barrier after this wave's LDS stores have completed, without the workgroup-scope
// fence of __syncthreads() (which also waits for every outstanding global load).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Staged stream of a prefix task with four waves per KV head: wave q of a head loads rows
// 4q .. 4q + 3 of K and V of each block (16-byte chunks) into a register ring kPrefixStage
// blocks deep, stores them into the head's LDS double buffer, and after one barrier per
// block every wave of the head reads the whole tile from LDS in load_tile's layout. So
// each block is loaded once per KV head instead of once per wave, and kPrefixStage blocks
// stay in flight per head for 8 registers per lane each (a whole tile in registers takes
// 32). K rows are stored with their 16-byte chunks permuted by the row index
// (chunk ^ row), so the K operand reads (one chunk of 16 rows per lane group) spread over
// the banks. Every wave of the workgroup runs the same number of iterations (the
// barrier); head_ok false: the wave's head does not exist (its loads read head 0 and
// nobody reads its buffer).
template <int DT, int D, int NW, typename F>
__device__ __forceinline__ void prefix_stream_staged(const DecodeArgs& a, int b, int j,
                                                     bool head_ok, int blk_begin, int n_my,
                                                     int lane, int& bad, F&& process) {
  using G_ = Geo<DT, D>;
  constexpr int kCpr = G_::kRow / 16;               // 16-byte chunks per token row
  constexpr int kWaveChunks = 4 * kCpr;             // four rows
  constexpr int kPer = (kWaveChunks + 63) / 64;     // chunks per lane and block
  constexpr int kSwz = kCpr < 16 ? kCpr - 1 : 15;
  constexpr int S = kPrefixStage;
  constexpr int NB = S;
  static_assert(kPrefixPartition / kBlockTokens <= 64, "one table entry per lane");
  __shared__ u32x4 ring[NW / 4][2][2][16 * kCpr];   // [head][buffer][K, V][chunk]
  const int wave = threadIdx.x >> 6, q = wave & 3, hs = wave >> 2;
  const int r = lane >> 4, c = lane & 15;
  const uint32_t tok_stride = (uint32_t)a.n_kv_heads * G_::kRow;
  const size_t blk_stride = (size_t)tok_stride * kBlockTokens;
  const uint32_t head_off = (uint32_t)(head_ok ? j : 0) * G_::kRow;
  // Every lane loads and stores unconditionally (branches around the loads would make
  // the compiler wait for all of them): with fewer chunks than lanes the upper lanes
  // repeat the lower ones' chunks, and a wave whose head does not exist reads head 0.
  uint32_t goff[kPer];
  int kdst[kPer], vdst[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int x = (lane + 64 * i) % kWaveChunks;
    const int row = 4 * q + x / kCpr, ch = x % kCpr;
    goff[i] = head_off + (uint32_t)row * tok_stride + 16u * ch;
    kdst[i] = row * kCpr + (ch ^ (row & kSwz));
    vdst[i] = row * kCpr + ch;
  }
  // the partition's table entries, lane i holding block i's (n_my <= 64), loaded before any
  // tile so that reading them never waits for tile loads
  const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks_per_seq + blk_begin;
  const int tbl = lane < n_my ? trow[lane] : 0;
  u32x4 rk[NB][kPer], rv[NB][kPer];
  auto fetch = [&](int s, int i) {
    const int pb = __builtin_amdgcn_readlane(tbl, i);
    const bool ok = (unsigned)pb < (unsigned)a.num_blocks;
    bad |= !ok;
    const char* kb = a.k_pool + (size_t)(ok ? pb : 0) * blk_stride;
    const char* vb = a.v_pool + (size_t)(ok ? pb : 0) * blk_stride;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      rk[s][i] = *reinterpret_cast<const u32x4*>(kb + goff[i]);
      rv[s][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + goff[i]));
    }
  };
  auto step = [&](int s, int i, bool refill) {
    const int buf = i & 1;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      ring[hs][buf][0][kdst[k]] = rk[s][k];
      ring[hs][buf][1][vdst[k]] = rv[s][k];
    }
    if (refill) fetch(s, i + S);
    lds_barrier();
    Tile<DT, D> t;
    const u32x4* kr = ring[hs][buf][0];
#pragma unroll
    for (int kk = 0; kk < G_::kNK; ++kk) t.k[kk] = kr[c * kCpr + ((4 * kk + r) ^ (c & kSwz))];
    const unsigned* vr = reinterpret_cast<const unsigned*>(ring[hs][buf][1]);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const unsigned* src = vr + (4 * r + jj) * (G_::kRow / 4) + c * G_::kVW;
      if constexpr (G_::kVW == 8) {
        const u32x4 a0 = reinterpret_cast<const u32x4*>(src)[0], a1 = reinterpret_cast<const u32x4*>(src)[1];
#pragma unroll
        for (int x = 0; x < 4; ++x) { t.v[jj][x] = a0[x]; t.v[jj][4 + x] = a1[x]; }
      } else if constexpr (G_::kVW == 4) {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
        for (int x = 0; x < 4; ++x) t.v[jj][x] = a0[x];
      } else {
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(src);
        t.v[jj][0] = a0[0];
        t.v[jj][1] = a0[1];
      }
    }
    process(t, (blk_begin + i) * kBlockTokens);
  };
  // a partition shorter than S blocks loads its last block again instead of skipping loads
#pragma unroll
  for (int d0 = 0; d0 < S; ++d0) fetch(d0, min(d0, n_my - 1));
  const int n_fetching = n_my - S;          // iterations i < n_fetching refill block i + S
  int i0 = 0;
  for (; i0 + NB <= n_fetching; i0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) step(u, i0 + u, true);
  }
  for (; i0 < n_my; i0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int i = i0 + u;
      if (i >= n_my) break;
      step(u, i, i < n_fetching);
    }
  }
}

// Shared-prefix task `task` of a split workgroup of NW waves: prefix partition p
// (kPrefixPartition tokens) of group g, KV heads jp * NW/wph .. and column-set group cs4,
// with wph = prefix_wph waves per KV head (enough 16-column sets for the largest group's
// columns, up to four). Wave v takes KV head j = jp * NW/wph + v / wph and the 16 columns
// k = (cs4 * wph + v % wph) * 16 + c (lane column c), column k being the pair (member
// m = k / G, head h = k % G), members being the sequences of group g in increasing order.
// Every wave reads its partition's K/V blocks through the first member's table and runs
// them against its query tile with the multi-query block processor (no causal limit: every shared token is visible to every member), then
// leaves one (m, l, O) record per (member, head) of its columns for partition p. The tasks
// of KV-head set 0 and column-set group 0 also compare every member's table with the first
// member's over their partition and leave one flag per (member, partition) for the merge.
// Tasks are numbered KV-head set fastest, then partition, column-set group and group, so
// the tasks reading one partition's token rows run side by side. Every thread of the
// workgroup calls it (it has barriers); no barrier follows its record stores. With four
// waves per KV head and a 16-bit dtype the blocks come through prefix_stream_staged (one
// load per head); otherwise each wave streams them itself (the register stream,
// kPrefixDepth ahead; the waves of a head read the same bytes, so HBM sees them once).
template <int DT, int D, int G, int NW>
__device__ __forceinline__ void prefix_task(const DecodeArgs& a, int task) {
  using G_ = Geo<DT, D>;
  constexpr int kThreads = 64 * NW;
  static_assert(NW % kPrefixWaves == 0, "whole KV heads per task");
  const int wph = a.prefix_wph;                 // 1, 2 or 4: divides NW
  const int heads_per_task = NW / wph;
  __shared__ int sm_members[kSplitMaxSeqs];
  __shared__ unsigned char sm_flag[kSplitMaxSeqs];
  __shared__ int sm_wsum[NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int B = a.num_seqs;
  const int HP = (a.n_kv_heads + heads_per_task - 1) / heads_per_task;
  int t = task;
  const int jp = t % HP;
  t /= HP;
  const int p = t % a.prefix_parts;
  t /= a.prefix_parts;
  const int cs4 = t % a.prefix_sets;
  const int g = t / a.prefix_sets;
  if (g >= a.n_groups) return;                             // uniform: before any barrier

  const int sb = a.group_blocks[g];
  if (sb <= 0 || sb > a.max_blocks_per_seq || sb > a.max_shared_blocks) return;
  constexpr int kPartBlocks = kPrefixPartition / kBlockTokens;
  const int blk_begin = p * kPartBlocks;
  const int blk_end = min(sb, blk_begin + kPartBlocks);
  if (blk_begin >= blk_end) return;

  // Members of g, in sequence order: per-thread counts over a contiguous chunk, an
  // exclusive scan (waves, then wave totals), scatter.
  const int chunk = (B + kThreads - 1) / kThreads;
  const int s0 = min(B, tid * chunk), s1 = min(B, s0 + chunk);
  int cnt = 0;
  for (int s = s0; s < s1; ++s) cnt += a.seq_group[s] == g;
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) sm_wsum[wave] = incl;
  __syncthreads();
  int pos = incl - cnt, M = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const int x = sm_wsum[v];
    pos += v < wave ? x : 0;
    M += x;
  }
  for (int s = s0; s < s1; ++s)
    if (a.seq_group[s] == g) sm_members[pos++] = s;
  __syncthreads();
  if (M == 0) return;                                      // uniform
  const int leader = sm_members[0];
  const int32_t* lead_row = a.block_tables + (size_t)leader * a.max_blocks_per_seq;
  const bool too_many = M > a.max_group_size;

  if (jp == 0 && cs4 == 0) {        // uniform over the workgroup
    // one (member, block) pair per thread and step, so the table reads go out together
    const int nblk = blk_end - blk_begin;
    for (int m = tid; m < M; m += kThreads) sm_flag[m] = too_many;
    __syncthreads();
#pragma unroll 4
    for (int x = tid; x < M * nblk; x += kThreads) {
      const int m = x / nblk, k = blk_begin + (x - m * nblk);
      if (a.block_tables[(size_t)sm_members[m] * a.max_blocks_per_seq + k] != lead_row[k])
        sm_flag[m] = 1;            // every writer stores the same value
    }
    __syncthreads();
    for (int m = tid; m < M; m += kThreads)
      a.ws_flags[(size_t)sm_members[m] * a.prefix_parts + p] = sm_flag[m];
  }
  const int j = jp * heads_per_task + wave / wph;
  const int k0 = (cs4 * wph + wave % wph) * 16;                     // first column of this wave
  const int tok_end = blk_end * kBlockTokens;
  const int k = k0 + c;
  const bool used = k < M * G;
  u32x4 qf[G_::kNK];
  MqState<DT, D> st;
  int bad = 0;
  auto proc = [&](const Tile<DT, D>& tl, int tok0) {
    if (tok0 + kBlockTokens > tok_end)
      process_block_mq<DT, D, true>(st, tl, qf, tok0, tok_end, tok_end, tok_end, a.scale_log2, r);
    else
      process_block_mq<DT, D, false>(st, tl, qf, tok0, tok_end, tok_end, tok_end, a.scale_log2, r);
  };
  if (prefix_staged(DT, wph)) {       // uniform: the staged stream, barriers per block
    if (too_many) return;
    const bool head_ok = j < a.n_kv_heads;
    const bool active = head_ok && k0 < M * G;   // waves without columns still load
    load_query<DT, D>(a, used && active,
                      used && active ? (size_t)sm_members[k / G] * a.n_heads + (size_t)j * G + k % G : 0,
                      r, qf);
    prefix_stream_staged<DT, D, NW>(a, leader, j, head_ok, blk_begin, blk_end - blk_begin, lane,
                                    bad, [&](const Tile<DT, D>& tl, int tok0) {
      if (active) proc(tl, tok0);
    });
    if (!active) return;                         // no barrier below
  } else {
    if (too_many || j >= a.n_kv_heads || k0 >= M * G) return;       // no barrier below
    load_query<DT, D>(a, used, used ? (size_t)sm_members[k / G] * a.n_heads + (size_t)j * G + k % G : 0,
                      r, qf);
    // The waves of a KV head read the same blocks, so each keeps more of them in flight
    // than a decode wave does.
    stream_blocks<DT, D, kPrefixDepth<DT, D>, false, true>(a, leader, j, blk_begin,
                                                           blk_end - blk_begin, lead_row[blk_begin],
                                                           lane, bad, proc);
  }
  st.l += __shfl_xor(st.l, 16);
  st.l += __shfl_xor(st.l, 32);
  if (!used) return;
  const float qnan = __builtin_nanf("");
  const int b = sm_members[k / G];
  const size_t idx = ((size_t)b * a.n_heads + (size_t)j * G + k % G) * a.prefix_parts + p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* dst = a.ws_po + idx * D + G_::kEPL * (4 * r + i);
#pragma unroll
    for (int e = 0; e < G_::kEPL; e += 4) {
      const f32x4 x = {bad ? qnan : st.o[e][i], bad ? qnan : st.o[e + 1][i],
                       bad ? qnan : st.o[e + 2][i], bad ? qnan : st.o[e + 3][i]};
      *reinterpret_cast<f32x4*>(dst + e) = x;
    }
  }
  if (r == 0) {
    a.ws_pm[idx] = bad ? qnan : st.m;
    a.ws_pl[idx] = bad ? qnan : st.l;
  }
}

// Fixed partitions: workgroup = NW waves = KV heads hg*NW .. hg*NW+NW-1 of one
// (partition, sequence); grid (head groups, partitions, sequences).
template <int DT, int D, int G, int NW, int MODE>
__global__ __launch_bounds__(64 * NW) void decode_fixed_kernel(DecodeArgs a) {
  const int hg = blockIdx.x, p = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = hg * NW + wave;                 // this wave's KV head
  if (j >= a.n_kv_heads) return;                // no barrier below: waves are independent
  const int C = G * a.q_len;                    // output rows of this wave

  const int n_ctx = a.context_lens[b];
  if (!valid_len(a, n_ctx)) {
    if (p == 0)
      for (int c = 0; c < C; ++c) write_nan_rows<DT, D>(a, mq_row<G>(a, b, j, c), 1, lane, 64);
    return;
  }
  const int P = a.partition_tokens;
  const int n_part = (n_ctx + P - 1) / P;
  if (p >= n_part) return;
  const int tok_end = min(n_ctx, (p + 1) * P);
  const int blk_begin = (p * P) >> 4;
  const int n_my = ((tok_end + 15) >> 4) - blk_begin;     // >= 1
  const int first_entry = a.block_tables[(size_t)b * a.max_blocks_per_seq + blk_begin];
  run_segment<DT, D, G, MODE>(a, b, j, blk_begin, n_my, tok_end, n_ctx, n_part == 1,
                            first_entry, lane,
                            [&](int c) { return mq_row<G>(a, b, j, c) * a.max_partitions + p; });
}

// Balanced split: the work is the list of units (head group hg, sequence b, block k) in
// that order, T units in all. Workgroup w of the W in the grid takes units
// [w*T/W, (w+1)*T/W) — every workgroup gets the same number of blocks to stream, whatever
// the mix of context lengths. The part of one sequence inside one workgroup is a
// segment; a segment holding a whole sequence is finished in place, any other one leaves
// a record for merge_kernel. Segments of stream s = hg * num_seqs + b are produced by
// consecutive workgroups in increasing order of w, so (w + s) names each segment
// uniquely: the record of its column c (of C = G * q_len) is ((w + s) * NW + wave) * C + c.
// kModeSinglePrefix (shared prefixes): the units are each sequence's blocks after its
// group's shared ones, and workgroups w < prefix_tasks first run prefix task w with a
// correspondingly smaller share (SplitShares), so the prefix tasks, which wait on their
// block chain more than on HBM, overlap the streaming of the other workgroups.
template <int DT, int D, int G, int NW, int MODE>
__global__ __launch_bounds__(64 * NW) void decode_split_kernel(DecodeArgs a) {
  constexpr int kThreads = 64 * NW;
  constexpr int kScanChunks = kSplitMaxSeqs / 64;
  static_assert(kScanChunks <= 64, "one lane per chunk of 64 sequences");
  __shared__ int sm_pref[kSplitMaxSeqs + 1];   // blocks of sequences before b
  __shared__ int sm_chunk[kScanChunks];         // blocks of each chunk of 64 sequences
  // The shared-prefix launch, whose short private parts make many segments, gets each
  // segment's first table entry loaded while the previous segment streams, and reads a
  // sequence's length from LDS: its tokens in its last block (1..16, stored minus one) and
  // its shared blocks (plus kGroupedBit if it belongs to a group); the block counts give the
  // rest. Measured on the 8 x 16-sequence shared-prefix batch (us warm / cold, same box):
  // bf16 32 / 8 heads d 128 69.5 / 85.2 -> 68.4 / 84.1, d 64 50.4 / 59.4 -> 48.4 / 55.7,
  // 64 / 8 heads 128.0 / 142.3 -> 125.2 / 140.2, fp32 78.1 / 94.0 -> 76.9 / 92.8. The other
  // kernels, with one or two long segments per workgroup, load the entry at the segment's
  // start: with the look-ahead the decode of the GQA batch measured 247.4 -> 248.2 us.
  constexpr bool kEntryAhead = MODE == kModeSinglePrefix;
  constexpr int kGroupedBit = 1 << 30;          // shared blocks are below 2^27
  __shared__ unsigned char sm_last[kEntryAhead ? kSplitMaxSeqs : 1];
  __shared__ int sm_skg[MODE == kModeSinglePrefix ? kSplitMaxSeqs : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.num_seqs;

  // Exclusive prefix sum of the block counts (sequences with an invalid length count 0).
  // Wave v scans chunks v, v + NW, ... of 64 sequences across its lanes; after one barrier
  // every wave scans the chunk totals and adds each chunk's offset: two barriers in all.
  const int n_chunks = (B + 63) / 64;
  auto inclusive_scan = [&](int x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    return x;
  };
  for (int c = wave; c < n_chunks; c += NW) {
    const int s = c * 64 + lane;
    int nb = 0;
    if (s < B) {
      const int n = a.context_lens[s];
      const int skip = shared_blocks_of(a, s, n);
      nb = valid_len(a, n) && skip >= 0 ? (n + kBlockTokens - 1) / kBlockTokens - skip : 0;
      if constexpr (kEntryAhead) sm_last[s] = nb > 0 ? (n - 1) & (kBlockTokens - 1) : 0;
      if constexpr (MODE == kModeSinglePrefix)
        sm_skg[s] = nb > 0 ? skip | (a.seq_group[s] >= 0 ? kGroupedBit : 0) : 0;
    }
    const int incl = inclusive_scan(nb);
    if (s < B) sm_pref[s] = incl - nb;
    if (lane == 63) sm_chunk[c] = incl;
  }
  __syncthreads();
  {
    const int tot = lane < n_chunks ? sm_chunk[lane] : 0;
    const int incl = inclusive_scan(tot);
    const int excl = incl - tot;                // blocks of the chunks before chunk `lane`
    for (int c = wave; c < n_chunks; c += NW) {
      const int off = __shfl(excl, c);
      const int s = c * 64 + lane;
      if (s < B) sm_pref[s] += off;
    }
    const int total = __shfl(incl, 63);
    if (tid == 0) sm_pref[B] = total;
  }
  __syncthreads();

  const int w = blockIdx.x;
  const int HG = (a.n_kv_heads + NW - 1) / NW;
  const int T1 = sm_pref[B];                    // blocks per head group
  const long long T = (long long)T1 * HG;
  const SplitShares sh = split_shares(a, T, gridDim.x);
  const long long W = sh.W;                     // workgroups with private units
  if (w == 0)
    for (int s = tid; s <= B; s += kThreads) a.ws_prefix[s] = sm_pref[s];
  const int rows_per_seq = a.q_len * a.n_heads;
  for (int s = w; s < B; s += gridDim.x)        // invalid lengths or groups: NaN outputs
    if (!usable(a, s, a.context_lens[s]))
      write_nan_rows<DT, D>(a, (size_t)s * rows_per_seq, rows_per_seq, tid, kThreads);
  if constexpr (MODE == kModeSinglePrefix) {
    if (w < a.prefix_tasks) prefix_task<DT, D, G, NW>(a, w);   // uniform over the workgroup
  }
  if (w >= W) return;
  const int C = G * a.q_len;
  const long long u1 = sh.begin(w + 1);
  long long u = sh.begin(w);
  // Unit x lies in stream (hg, b), at block blk0 of b's unshared blocks; the table entry of
  // a segment's first block is loaded while the previous segment streams.
  struct Where { int hg, b, blk0, skg; };
  auto locate = [&](long long x) {
    Where p;
    p.hg = (int)(x / T1);
    const int rem = (int)(x - (long long)p.hg * T1);
    int lo = 0, hi = B;                         // last b with sm_pref[b] <= rem
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sm_pref[mid] <= rem) lo = mid; else hi = mid;
    }
    p.b = __builtin_amdgcn_readfirstlane(lo);                      // uniform
    p.blk0 = __builtin_amdgcn_readfirstlane(rem - sm_pref[p.b]);
    p.skg = 0;
    if constexpr (MODE == kModeSinglePrefix) p.skg = __builtin_amdgcn_readfirstlane(sm_skg[p.b]);
    return p;
  };
  auto first_entry_of = [&](const Where& p) {
    return a.block_tables[(size_t)p.b * a.max_blocks_per_seq + (p.skg & (kGroupedBit - 1)) + p.blk0];
  };
  Where cur = locate(u);
  int e_cur = kEntryAhead && u < u1 ? first_entry_of(cur) : 0;
  while (u < u1) {
    if constexpr (!kEntryAhead) e_cur = first_entry_of(cur);    // unused by multi-query
    const int hg = cur.hg, b = cur.b, blk0 = cur.blk0;
    const int skip = cur.skg & (kGroupedBit - 1);     // b's shared blocks (0 ungrouped)
    const int nb = sm_pref[b + 1] - sm_pref[b];
    const int n_ctx = kEntryAhead ? (skip + nb - 1) * kBlockTokens + sm_last[b] + 1
                                  : a.context_lens[b];
    const long long seg_end = min(u1, (long long)hg * T1 + sm_pref[b + 1]);
    const int n_my = (int)(seg_end - u);
    Where nxt = cur;
    int e_nxt = 0;
    if (kEntryAhead && seg_end < u1) {
      nxt = locate(seg_end);
      e_nxt = first_entry_of(nxt);
    }
    const int j = hg * NW + wave;
    if (j < a.n_kv_heads) {
      const int tok_end = min(n_ctx, (skip + blk0 + n_my) * kBlockTokens);
      const size_t rec0 = ((size_t)(w + (long long)hg * B + b) * NW + wave) * C;
      // a sequence with a shared prefix always leaves a record: the merge adds the prefix
      run_segment<DT, D, G, MODE>(a, b, j, skip + blk0, n_my, tok_end, n_ctx,
                                skip == 0 && blk0 == 0 && n_my == nb && !(cur.skg & kGroupedBit),
                                e_cur, lane, [&](int c) { return rec0 + c; });
    }
    u = seg_end;
    cur = kEntryAhead || u >= u1 ? nxt : locate(u);
    e_cur = e_nxt;
  }
}

// One workgroup per output row (sequence b, new query i, head h): combine that row's
// records by the rescale rule. Fixed mode: the partitions. Split mode: the segments of its
// stream, then, for a grouped sequence, its shared-prefix records. The records form two
// arithmetic runs, (base, stride, n_rec) and (pbase, 1, n_pre), each read by its own loop.
template <int DT, int D, int NW>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
  constexpr int Q4 = D / 4;          // float4 chunks per output row
  constexpr int PR = 256 / Q4;       // records read side by side
  const int row = blockIdx.x;        // (b * q_len + i) * n_heads + h
  const int per_seq = a.q_len * a.n_heads;
  const int b = row / per_seq;
  const int i = (row - b * per_seq) / a.n_heads;
  const int h = row - b * per_seq - i * a.n_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_ctx = a.context_lens[b];
  if (!usable(a, b, n_ctx)) return;                      // decode wrote NaN

  size_t base, stride, pbase = 0;
  int n_rec, n_pre = 0;
  int nan_row = 0;
  if (a.split) {
    const int B = a.num_seqs;
    const int G = a.n_heads / a.n_kv_heads;
    const int C = G * a.q_len;
    const int j = h / G, hh = h - j * G;
    const int hg = j / NW, wv = j - hg * NW;
    const int HG = (a.n_kv_heads + NW - 1) / NW;
    const int T1 = a.ws_prefix[B];
    const long long T = (long long)T1 * HG;
    const SplitShares sh = split_shares(a, T, a.split_workgroups);
    const int nb = a.ws_prefix[b + 1] - a.ws_prefix[b];      // >= 1 for a usable sequence
    const long long U = (long long)hg * T1 + a.ws_prefix[b];
    const long long first = sh.owner(U);
    const long long last = sh.owner(U + nb - 1);
    const int grp = a.seq_group ? a.seq_group[b] : -1;
    if (first == last && grp < 0) return;                   // decode wrote the output
    n_rec = (int)(last - first + 1);
    base = ((size_t)(first + (long long)hg * B + b) * NW + wv) * C + (size_t)i * G + hh;
    stride = (size_t)NW * C;
    if (grp >= 0) {
      const int sb = a.group_blocks[grp];                   // <= max_blocks_per_seq here
      if (sb > a.max_shared_blocks) {
        nan_row = 1;
      } else {
        n_pre = (sb * kBlockTokens + kPrefixPartition - 1) / kPrefixPartition;
        pbase = ((size_t)b * a.n_heads + h) * a.prefix_parts;
        for (int p = tid; p < n_pre; p += 256) nan_row |= a.ws_flags[(size_t)b * a.prefix_parts + p];
      }
      // the group broke its promise (see prefix_task): NaN row
      if (__syncthreads_or(nan_row)) {
        for (int x = tid; x < D; x += 256) store_elem<DT>(a.out, (size_t)row * D + x, __builtin_nanf(""));
        return;
      }
    }
  } else {
    n_rec = (n_ctx + a.partition_tokens - 1) / a.partition_tokens;
    if (n_rec <= 1) return;                                 // decode wrote the output
    base = (size_t)row * a.max_partitions;
    stride = 1;
  }

  __shared__ float red[4];
  __shared__ f32x4 part[PR][Q4];

  float mx = -INFINITY;
  for (int k = tid; k < n_rec; k += 256) mx = fmaxf(mx, a.ws_m[base + k * stride]);
  for (int k = tid; k < n_pre; k += 256) mx = fmaxf(mx, a.ws_pm[pbase + k]);
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();

  float sum = 0.f;
  for (int k = tid; k < n_rec; k += 256) {
    const size_t r = base + k * stride;
    sum = fmaf(a.ws_l[r], exp2_fast(a.ws_m[r] - M), sum);
  }
  for (int k = tid; k < n_pre; k += 256)
    sum = fmaf(a.ws_pl[pbase + k], exp2_fast(a.ws_pm[pbase + k] - M), sum);
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) sum += __shfl_xor(sum, s);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  const float L = (red[0] + red[1]) + (red[2] + red[3]);

  const int q = tid % Q4, pr = tid / Q4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = pr; k < n_rec; k += PR) {
    const size_t r = base + k * stride;
    const float f = exp2_fast(a.ws_m[r] - M);
    acc += f * reinterpret_cast<const f32x4*>(a.ws_o + r * D)[q];
  }
  for (int k = pr; k < n_pre; k += PR) {
    const size_t r = pbase + k;
    const float f = exp2_fast(a.ws_pm[r] - M);
    acc += f * reinterpret_cast<const f32x4*>(a.ws_po + r * D)[q];
  }
  part[pr][q] = acc;
  __syncthreads();
  if (tid < Q4) {
    f32x4 t = part[0][tid];
#pragma unroll
    for (int k = 1; k < PR; ++k) t += part[k][tid];
    const float inv = 1.0f / L;
#pragma unroll
    for (int x = 0; x < 4; ++x) store_elem<DT>(a.out, (size_t)row * D + 4 * tid + x, t[x] * inv);
  }
}


// merge_kernel for many rows with few records each: one wave per output row, four rows
// per workgroup. The wave reads the row's records (lane: D / 64 consecutive elements of O)
// eight at a time in one round of loads and combines them by the rescale rule; no barrier,
// and a quarter of the workgroups. Used when the launch has at least kMergeRowsWave rows
// (a batch of many sequences, or q_len > 1, cuts each sequence into few segments); a few
// long sequences, each cut into many segments, keep merge_kernel's four waves per row.
template <int DT, int D, int NW>
__global__ __launch_bounds__(256) void merge_rows_kernel(DecodeArgs a) {
  constexpr int EL = D / 64;                   // output elements per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);   // (b * q_len + i) * n_heads + h
  const int per_seq = a.q_len * a.n_heads;
  if (row >= a.num_seqs * per_seq) return;     // no barrier in this kernel
  const int b = row / per_seq;
  const int i = (row - b * per_seq) / a.n_heads;
  const int h = row - b * per_seq - i * a.n_heads;
  const int n_ctx = a.context_lens[b];
  if (!usable(a, b, n_ctx)) return;            // decode wrote NaN

  size_t base, stride, pbase = 0;
  int n_rec, n_pre = 0, nan_row = 0;
  if (a.split) {
    const int B = a.num_seqs;
    const int G = a.n_heads / a.n_kv_heads;
    const int C = G * a.q_len;
    const int j = h / G, hh = h - j * G;
    const int hg = j / NW, wv = j - hg * NW;
    const int HG = (a.n_kv_heads + NW - 1) / NW;
    const int T1 = a.ws_prefix[B];
    const long long T = (long long)T1 * HG;
    const SplitShares sh = split_shares(a, T, a.split_workgroups);
    const int nb = a.ws_prefix[b + 1] - a.ws_prefix[b];      // >= 1 for a usable sequence
    const long long U = (long long)hg * T1 + a.ws_prefix[b];
    const long long first = sh.owner(U);
    const long long last = sh.owner(U + nb - 1);
    const int grp = a.seq_group ? a.seq_group[b] : -1;
    if (first == last && grp < 0) return;                   // decode wrote the output
    n_rec = (int)(last - first + 1);
    base = ((size_t)(first + (long long)hg * B + b) * NW + wv) * C + (size_t)i * G + hh;
    stride = (size_t)NW * C;
    if (grp >= 0) {
      const int sb = a.group_blocks[grp];                   // <= max_blocks_per_seq here
      if (sb > a.max_shared_blocks) {
        nan_row = 1;
      } else {
        n_pre = (sb * kBlockTokens + kPrefixPartition - 1) / kPrefixPartition;
        pbase = ((size_t)b * a.n_heads + h) * a.prefix_parts;
      }
    }
  } else {
    n_rec = (n_ctx + a.partition_tokens - 1) / a.partition_tokens;
    if (n_rec <= 1) return;                                 // decode wrote the output
    base = (size_t)row * a.max_partitions;
    stride = 1;
  }

  // Records k < n_rec are the segments' (base + k * stride), the next n_pre the prefix
  // partitions' (pbase + k - n_rec). They are read kChunk at a time with every load of a
  // chunk issued before any is used, the prefix flags of a grouped sequence in the first
  // round too; a later chunk rescales the sums so far by 2^(M_old - M_new). Up to kChunk
  // records this is exactly the two-pass sum (maximum first, then the weighted sums).
  constexpr int kChunk = 8;
  const int n_all = n_rec + n_pre;
  float M = -INFINITY, L = 0.f, acc[EL] = {};
  for (int k0 = 0; k0 < n_all; k0 += kChunk) {
    float m[kChunk], l[kChunk], o[kChunk][EL];
#pragma unroll
    for (int x = 0; x < kChunk; ++x) {
      const int k = k0 + x;
      m[x] = -INFINITY;
      l[x] = 0.f;
#pragma unroll
      for (int e = 0; e < EL; ++e) o[x][e] = 0.f;
      if (k < n_rec) {
        const size_t r = base + k * stride;
        m[x] = a.ws_m[r];
        l[x] = a.ws_l[r];
#pragma unroll
        for (int e = 0; e < EL; ++e) o[x][e] = a.ws_o[r * D + EL * lane + e];
      } else if (k < n_all) {
        const size_t r = pbase + (k - n_rec);
        m[x] = a.ws_pm[r];
        l[x] = a.ws_pl[r];
#pragma unroll
        for (int e = 0; e < EL; ++e) o[x][e] = a.ws_po[r * D + EL * lane + e];
      }
    }
    if (k0 == 0)
      for (int p = lane; p < n_pre; p += 64) nan_row |= a.ws_flags[(size_t)b * a.prefix_parts + p];
    if (__any(nan_row)) break;
    float mc = M;
#pragma unroll
    for (int x = 0; x < kChunk; ++x)
      if (k0 + x < n_all) mc = fmaxf(mc, m[x]);
    const float sc = exp2_fast(M - mc);     // first chunk: M = -inf, sc = 0, sums still 0
    L *= sc;
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[e] *= sc;
#pragma unroll
    for (int x = 0; x < kChunk; ++x) {
      if (k0 + x >= n_all) break;
      const float f = exp2_fast(m[x] - mc);
      L = fmaf(l[x], f, L);
#pragma unroll
      for (int e = 0; e < EL; ++e) acc[e] = fmaf(f, o[x][e], acc[e]);
    }
    M = mc;
  }
  // the group broke its promise (see prefix_task): NaN row
  if (__any(nan_row)) {
    for (int x = lane; x < D; x += 64) store_elem<DT>(a.out, (size_t)row * D + x, __builtin_nanf(""));
    return;
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int e = 0; e < EL; ++e) store_elem<DT>(a.out, (size_t)row * D + EL * lane + e, acc[e] * inv);
}


// Resident workgroups of kernel K on the current device: compute units times the
// kernel's own occupancy. K is a template argument, so every kernel instantiation keeps
// its own figures (instantiations differ in registers and LDS, hence in occupancy); they
// are queried once per device and kept per device. Concurrent first calls store the same
// value.
constexpr int kMaxDevices = 64;

template <auto K>
int resident_workgroups(int threads) {
  static std::atomic<int> cached[kMaxDevices];   // 0: not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const int slot = dev < kMaxDevices ? dev : kMaxDevices - 1;
  int n = dev < kMaxDevices ? cached[slot].load(std::memory_order_relaxed) : 0;
  if (n <= 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, K, threads, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 1;
    n = per_cu * cus;
    if (dev < kMaxDevices) cached[slot].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Private units a workgroup gives up for running one prefix task (units: one block of
// the workgroup's NW KV heads). A task runs kPrefixPartition tokens (32 blocks) through
// every wave, a chain of 32 multi-query blocks per wave. Measured on the shared-prefix
// workload (bf16, d 128, G 4, four waves per KV head; attention us warm / cold, same box).
// Register stream: eight-wave workgroups cost 0: 88.8 / 107.5, 12: 79.2 / 97.4,
// 18: 75.0 / 94.0, 24: 71.6 / 90.5, 32: 76.0 / 97.3; four-wave workgroups (units of four
// KV heads) 16-20: 71.0 / 89.8. Staged stream (prefix_stream_staged, same box: register
// stream at 24 72.2 / 91.1): eight-wave workgroups 12: 71.8 / 87.7, 16: 69.0 / 85.2,
// 20: 69.4 / 87.6, 24: 71.6 / 89.0; four-wave workgroups 16: 69.7 / 85.7, 24: 70.1 / 86.4,
// 32: 76.4 / 94.7. So a staged task takes about as long as 16 private units, a register-
// stream task about 24 (eight heads) or 18 (four).
inline int prefix_task_cost(int dt, int nw, int wph) {
  if (prefix_staged(dt, wph)) return kPrefixPartition / kBlockTokens / 2;
  return (kPrefixPartition / kBlockTokens) * (nw == 8 ? 12 : 9) / 16;
}

template <int DT, int D, int G, int NW, int MODE>
hipError_t launch_typed(DecodeArgs a, hipStream_t stream) {
  bool need_merge;
  if (a.split) {
    constexpr auto kernel = decode_split_kernel<DT, D, G, NW, MODE>;
    a.split_workgroups = min(kSplitMaxWorkgroups, resident_workgroups<kernel>(64 * NW));
    a.prefix_tasks = 0;
    a.prefix_cost = 0;
    if constexpr (MODE == kModeSinglePrefix) {
      // one task per (partition, KV heads of a workgroup, column quad, group); the first
      // prefix_tasks workgroups run them (the grid grows if there are more tasks than
      // resident workgroups)
      const int hpt = NW / a.prefix_wph;
      const long long heads = (a.n_kv_heads + hpt - 1) / hpt;
      const long long tasks = (long long)a.prefix_parts * heads * a.prefix_sets * a.n_groups;
      if (tasks > (1 << 24)) return hipErrorInvalidValue;
      a.prefix_tasks = (int)tasks;
      a.prefix_cost = prefix_task_cost(DT, NW, a.prefix_wph);
      a.split_workgroups = max(a.split_workgroups, a.prefix_tasks);
    }
    if (a.grid_out) {                             // grid query: report, launch nothing
      *a.grid_out = a.split_workgroups;
      return hipSuccess;
    }
    hipLaunchKernelGGL(kernel, dim3(a.split_workgroups), dim3(64 * NW), 0, stream, a);
    need_merge = true;
  } else if constexpr (MODE != kModeSinglePrefix) {
    const dim3 grid((a.n_kv_heads + NW - 1) / NW, a.max_partitions, a.num_seqs);
    hipLaunchKernelGGL((decode_fixed_kernel<DT, D, G, NW, MODE>), grid, dim3(64 * NW), 0, stream, a);
    need_merge = a.max_partitions > 1;
  } else {
    return hipErrorInvalidValue;                  // shared prefixes need the balanced split
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !need_merge) return e;
  const int rows = a.num_seqs * a.q_len * a.n_heads;
  if (rows >= kMergeRowsWave)
    hipLaunchKernelGGL((merge_rows_kernel<DT, D, NW>), dim3((rows + 3) / 4), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((merge_kernel<DT, D, NW>), dim3(rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int DT, int D, int G, int NW>
hipError_t launch_mq(const DecodeArgs& a, hipStream_t stream) {
  if (a.q_len == 1)
    return a.k_new ? launch_typed<DT, D, G, NW, kModeSingleAppend>(a, stream)
                   : launch_typed<DT, D, G, NW, kModeSingle>(a, stream);
  return a.k_new ? launch_typed<DT, D, G, NW, kModeMultiAppend>(a, stream)
                 : launch_typed<DT, D, G, NW, kModeMulti>(a, stream);
}

template <int DT, int D, int G>
hipError_t launch_waves(const DecodeArgs& a, hipStream_t stream) {
  // Eight KV heads per workgroup when they divide evenly and the kernel fits 256 registers
  // per lane (16-bit types, G <= 4); otherwise four (waves past the last head exit).
  if constexpr (DT != 0 && G <= 4) {
    if (max_waves_per_workgroup(a.n_kv_heads) == 8) return launch_mq<DT, D, G, 8>(a, stream);
  }
  return launch_mq<DT, D, G, 4>(a, stream);
}

template <int DT, int D>
hipError_t launch_group(const DecodeArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_waves<DT, D, 1>(a, stream);
    case 2: return launch_waves<DT, D, 2>(a, stream);
    case 4: return launch_waves<DT, D, 4>(a, stream);
    case 8: return launch_waves<DT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_dim(const DecodeArgs& a, int d_head, int group, hipStream_t stream) {
  if (d_head == 64) return launch_group<DT, 64>(a, group, stream);
  if (d_head == 128) return launch_group<DT, 128>(a, group, stream);
  return hipErrorInvalidValue;
}

template <int DT, int D, int G>
hipError_t launch_quant_group(const DecodeArgs& a, int fmt, hipStream_t stream) {
  // eight KV heads per workgroup when they divide evenly (every variant fits 256 registers)
  if (max_waves_per_workgroup(a.n_kv_heads) == 8) {
    if (fmt == kKvInt8) return launch_typed<DT, D, G, 8, kModeQuantInt8>(a, stream);
    return launch_typed<DT, D, G, 8, kModeQuantFp8>(a, stream);
  }
  if (fmt == kKvInt8) return launch_typed<DT, D, G, 4, kModeQuantInt8>(a, stream);
  return launch_typed<DT, D, G, 4, kModeQuantFp8>(a, stream);
}

template <int DT, int D>
hipError_t launch_quant_dim(const DecodeArgs& a, int fmt, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_quant_group<DT, D, 1>(a, fmt, stream);
    case 2: return launch_quant_group<DT, D, 2>(a, fmt, stream);
    case 4: return launch_quant_group<DT, D, 4>(a, fmt, stream);
    case 8: return launch_quant_group<DT, D, 8>(a, fmt, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_quant_dtype(const DecodeArgs& a, int fmt, int d_head, int group,
                              hipStream_t stream) {
  if (d_head == 64) return launch_quant_dim<DT, 64>(a, fmt, group, stream);
  if (d_head == 128) return launch_quant_dim<DT, 128>(a, fmt, group, stream);
  return hipErrorInvalidValue;
}

template <int DT, int D, int G>
hipError_t launch_prefix_typed(const DecodeArgs& a, hipStream_t stream) {
  // the workgroup shapes of launch_waves: the prefix tasks run inside the split kernel
  if constexpr (DT != 0 && G <= 4) {
    if (max_waves_per_workgroup(a.n_kv_heads) == 8)
      return launch_typed<DT, D, G, 8, kModeSinglePrefix>(a, stream);
  }
  return launch_typed<DT, D, G, 4, kModeSinglePrefix>(a, stream);
}

template <int DT, int D>
hipError_t launch_prefix_group(const DecodeArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_prefix_typed<DT, D, 1>(a, stream);
    case 2: return launch_prefix_typed<DT, D, 2>(a, stream);
    case 4: return launch_prefix_typed<DT, D, 4>(a, stream);
    case 8: return launch_prefix_typed<DT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_prefix_dim(const DecodeArgs& a, int d_head, int group, hipStream_t stream) {
  if (d_head == 64) return launch_prefix_group<DT, 64>(a, group, stream);
  if (d_head == 128) return launch_prefix_group<DT, 128>(a, group, stream);
  return hipErrorInvalidValue;
}

}  // namespace

// The launchers of this translation unit's dtype (pkv_dispatch.cpp selects among them).
template <>
hipError_t launch_decode_dtype<PKV_DECODE_DTYPE>(const DecodeArgs& a, int d_head, int group,
                                                 hipStream_t stream) {
  return launch_dim<PKV_DECODE_DTYPE>(a, d_head, group, stream);
}

template <>
hipError_t launch_shared_prefix_dtype<PKV_DECODE_DTYPE>(const DecodeArgs& a, int d_head,
                                                        int group, hipStream_t stream) {
  return launch_prefix_dim<PKV_DECODE_DTYPE>(a, d_head, group, stream);
}

template <>
hipError_t launch_decode_quantized_dtype<PKV_DECODE_DTYPE>(const DecodeArgs& a, int kv_format,
                                                           int d_head, int group,
                                                           hipStream_t stream) {
  if constexpr (PKV_DECODE_DTYPE == 0) {
    return hipErrorInvalidValue;               // q and out must be 16-bit over 8-bit codes
  } else {
    if (kv_format != kKvInt8 && kv_format != kKvFp8) return hipErrorInvalidValue;
    return launch_quant_dtype<PKV_DECODE_DTYPE>(a, kv_format, d_head, group, stream);
  }
}

}  // namespace pkv
