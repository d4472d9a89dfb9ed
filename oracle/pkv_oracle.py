"""Plain, slow, fp64 CPU oracle for single-token decode attention over a paged KV cache.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline leg of
the benchmark may import this module. The product path (the HIP library and its Python
binding) never imports it, and this module imports nothing from the product path.

Sources (the pages this follows, cited by page title and section):

* "LLM 推理优化全景实战" (chenxutan.com), §2.3 "PagedAttention 的实现细节": the block pool
  is shaped [num_blocks, block_size, num_heads, head_dim]; a request's page table maps
  logical block -> physical block; a token at index t lives in logical block
  t // block_size at offset t % block_size (write_kv / read_kv).
* same page, §2.4 "PagedAttention 的注意力计算": gather the request's blocks through the
  page table, score = q . k / sqrt(head_dim), softmax over tokens, output = weights . V.
* "09-inference-optimization" (LLM-Code-Hot-100), section "KV Cache": the new token's
  K/V is written into the cache *before* attention, the scale is 1/sqrt(head_dim), and
  the per-layer cache size is 2 * batch * kv_heads * seq * head_dim * dtype_bytes;
  section "PagedAttention": only the used slots of a page are part of the sequence
  (get_kv slices each page to its used slots).
* "LLM推理与服务：面试问题与推荐回答", Q7: grouped-query attention, G query heads share one
  KV head; "推理机制动态图解（进阶）" demo 1 assigns query heads 0-15 with KV heads 0-3,
  i.e. groups are contiguous: kv_head(h) = h // G.
* "推理机制动态图解（进阶）" demo 5 "FlashAttention：分块与在线 softmax": running max m,
  exponent sum l and unnormalised output O, rescaled by exp(m_old - m_new) whenever the
  max grows; the final O / l equals the standard softmax result.

What is computed here is the plain definition: gather every used slot through the table,
score in fp64, two-pass softmax (subtract the maximum, exponentiate, normalise) and the
fp64 weighted sum of V. The online / partitioned form in `online_softmax_attention`
follows demo 5's steps and is kept to pin the reading that partition results merge by
the same rescale rule; it is checked against the two-pass definition, not the other way
round.

Storage dtypes: "f32" (numpy float32), "f16" (numpy float16) and "bf16" (numpy uint16
holding the upper 16 bits of an IEEE binary32, since numpy has no bfloat16).

Every function here is pinned by a CPU test (closed forms, hand-worked values, a library
attention routine, invariants); none is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

STORAGE_DTYPES = ("f32", "f16", "bf16")
_NUMPY_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def storage_to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Decode stored elements to fp64 exactly.

    bf16 is the upper half of an IEEE binary32: shifting the 16 stored bits into the
    high half of a 32-bit word gives the binary32 value, which fp64 holds exactly.
    """
    if dtype == "bf16":
        if arr.dtype != np.uint16:
            raise TypeError("bf16 arrays are stored as uint16 bit patterns")
        with np.errstate(invalid="ignore"):     # signalling-NaN patterns stay NaN
            return (arr.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype not in ("f32", "f16"):
        raise ValueError(f"unknown storage dtype {dtype!r}")
    if arr.dtype != _NUMPY_STORAGE[dtype]:
        raise TypeError(f"{dtype} arrays must be {_NUMPY_STORAGE[dtype].__name__}")
    return arr.astype(np.float64)


# --------------------------------------------------------------------------------------
# KV-cache size ("09-inference-optimization", section "KV Cache": the size formula and
# analyze_kv_cache_memory; "LLM推理与服务：面试问题与推荐回答" Q1: ~0.5 MB per token).
# --------------------------------------------------------------------------------------

def kv_cache_bytes(n_layers: int, batch: int, seq_len: int, n_kv_heads: int,
                   d_head: int, dtype_bytes: int) -> int:
    """2 (K and V) x layers x batch x seq_len x kv_heads x head_dim x bytes per element."""
    return 2 * n_layers * batch * seq_len * n_kv_heads * d_head * dtype_bytes


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, d_head: int, dtype_bytes: int) -> int:
    """Bytes one token adds to the cache across all layers: the formula at batch = seq = 1."""
    return kv_cache_bytes(n_layers, 1, 1, n_kv_heads, d_head, dtype_bytes)


# --------------------------------------------------------------------------------------
# Append and read through the page table (chenxutan §2.3 write_kv / read_kv).
# --------------------------------------------------------------------------------------

def _slot(table_row: np.ndarray, token_idx: int, block_size: int) -> tuple[int, int]:
    logical_block = token_idx // block_size
    block_offset = token_idx % block_size
    return int(table_row[logical_block]), block_offset


def kv_append(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              block_tables: np.ndarray, positions: np.ndarray, block_size: int):
    """Return copies of the pools with each sequence's new token written at its position.

    k_pool, v_pool: [num_blocks, block_size, n_kv_heads, d_head] (stored dtype).
    k_new, v_new:   [B, n_kv_heads, d_head] (same stored dtype).
    positions[b]:   token index of the new token (the context length before the step).
    The write is a plain element copy, so the result is exact in the stored dtype.
    """
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for b in range(k_new.shape[0]):
        phys, off = _slot(block_tables[b], int(positions[b]), block_size)
        k_out[phys, off] = k_new[b]
        v_out[phys, off] = v_new[b]
    return k_out, v_out


def read_kv(pool: np.ndarray, table_row: np.ndarray, token_idx: int, block_size: int) -> np.ndarray:
    """One token's [n_kv_heads, d_head] slice, found through the page table."""
    phys, off = _slot(table_row, token_idx, block_size)
    return pool[phys, off]


def gather_kv(pool: np.ndarray, table_row: np.ndarray, n_tokens: int, block_size: int,
              kv_head: int | None = None) -> np.ndarray:
    """Tokens 0..n_tokens-1 of one sequence in logical order, stored dtype.

    Returns [n_tokens, n_kv_heads, d_head], or [n_tokens, d_head] for one kv_head. Only
    the used slots are read: slots at or past n_tokens are never touched. This is
    read_kv applied to every token index, written as one indexed read.
    """
    t = np.arange(n_tokens, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[t // block_size]
    off = t % block_size
    if kv_head is None:
        return pool[phys, off]
    return pool[phys, off, kv_head]


# --------------------------------------------------------------------------------------
# Decode attention, plain definition (chenxutan §2.4; "09-inference-optimization",
# AttentionWithKVCache with a single query token, where no causal mask applies).
# --------------------------------------------------------------------------------------

def softmax_two_pass(scores: np.ndarray) -> np.ndarray:
    """Numerically stable softmax over the last axis: exp(s - max) / sum(exp(s - max))."""
    m = np.max(scores, axis=-1, keepdims=True)
    e = np.exp(scores - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def paged_decode_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                           block_tables: np.ndarray, context_lens: np.ndarray,
                           block_size: int, scale: float, dtype: str,
                           pairs=None) -> np.ndarray:
    """fp64 attention output for one query token per sequence.

    q:            [B, n_heads, d_head] stored dtype.
    k_pool/v_pool:[num_blocks, block_size, n_kv_heads, d_head] stored dtype, *after* the
                  append (the new token is part of the context).
    block_tables: [B, max_blocks_per_seq] int.
    context_lens: [B] tokens attended, including the just-appended one (N_b >= 1).
    pairs:        optional iterable of (b, h) to compute; other outputs stay NaN.
    Returns [B, n_heads, d_head] fp64.
    """
    B, n_heads, d_head = q.shape
    n_kv_heads = k_pool.shape[2]
    if n_heads % n_kv_heads:
        raise ValueError("n_heads must be a multiple of n_kv_heads")
    group = n_heads // n_kv_heads
    out = np.full((B, n_heads, d_head), np.nan, dtype=np.float64)

    wanted = {}
    if pairs is None:
        for b in range(B):
            for h in range(n_heads):
                wanted.setdefault((b, h // group), []).append(h)
    else:
        for b, h in pairs:
            wanted.setdefault((int(b), int(h) // group), []).append(int(h))

    for (b, j) in sorted(wanted):
        n_tok = int(context_lens[b])
        if n_tok < 1:
            raise ValueError("every sequence attends to at least its new token")
        keys = storage_to_f64(gather_kv(k_pool, block_tables[b], n_tok, block_size, j), dtype)
        vals = storage_to_f64(gather_kv(v_pool, block_tables[b], n_tok, block_size, j), dtype)
        for h in sorted(set(wanted[(b, j)])):
            qh = storage_to_f64(q[b, h], dtype)
            scores = scale * (keys @ qh)            # [n_tok]
            weights = softmax_two_pass(scores)      # [n_tok]
            out[b, h] = weights @ vals              # [d_head]
    return out


# --------------------------------------------------------------------------------------
# Online softmax over tiles and the merge of partition results ("推理机制动态图解（进阶）"
# demo 5; the split of one sequence's KV over many workers is "Scaling Book 第 11 章"
# §11.8 FlashDecoding). Kept in fp64 to pin the reading that partitions merge by the
# rescale rule.
# --------------------------------------------------------------------------------------

def online_softmax_partial(q_vec: np.ndarray, keys: np.ndarray, vals: np.ndarray,
                           scale: float, tile_tokens: int):
    """Run demo 5's loop over consecutive tiles of keys/vals; return (m, l, O).

    Start with m = -inf, l = 0, O = 0. For each tile: S = scale * q . K_tile; the new
    maximum m_new = max(m, max S); the old l and O are multiplied by exp(m - m_new); the
    tile adds sum exp(S - m_new) to l and exp(S - m_new) . V_tile to O. The caller
    divides O by l (deferred normalisation).
    """
    m = -math.inf
    l = 0.0
    o = np.zeros(vals.shape[-1], dtype=np.float64)
    for start in range(0, keys.shape[0], tile_tokens):
        k_tile = keys[start:start + tile_tokens]
        v_tile = vals[start:start + tile_tokens]
        s = scale * (k_tile @ q_vec)
        m_new = max(m, float(np.max(s)))
        rescale = math.exp(m - m_new) if m != -math.inf else 0.0
        p = np.exp(s - m_new)
        l = l * rescale + float(np.sum(p))
        o = o * rescale + p @ v_tile
        m = m_new
    return m, l, o


def merge_partitions(ms, ls, os_):
    """Combine partition results (m_p, l_p, O_p) into the attention output.

    The same rescale rule as between tiles: m* = max m_p, each partition is weighted by
    exp(m_p - m*), and the merged O is divided by the merged l. Partitions with no tokens
    carry m = -inf, l = 0 and contribute nothing.
    """
    m_star = max(ms)
    weights = [math.exp(m - m_star) if m != -math.inf else 0.0 for m in ms]
    l_star = sum(w * l for w, l in zip(weights, ls))
    o_star = sum(w * o for w, o in zip(weights, os_))
    return o_star / l_star


def online_softmax_attention(q_vec: np.ndarray, keys: np.ndarray, vals: np.ndarray,
                             scale: float, tile_tokens: int = 16,
                             partition_tokens: int | None = None) -> np.ndarray:
    """fp64 output via tiles (and optional partitions merged by the rescale rule)."""
    if partition_tokens is None:
        m, l, o = online_softmax_partial(q_vec, keys, vals, scale, tile_tokens)
        return o / l
    parts = [online_softmax_partial(q_vec, keys[s:s + partition_tokens],
                                    vals[s:s + partition_tokens], scale, tile_tokens)
             for s in range(0, keys.shape[0], partition_tokens)]
    return merge_partitions([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])


# --------------------------------------------------------------------------------------
# Several new tokens per sequence ("09-inference-optimization", section KV Cache: with
# seq_len > 1 new tokens the scores get a causal mask — key k is hidden from new query i
# when k > K - seq_len + i, K counting every cached token; speculative verification checks
# k drafted tokens in one pass of the target model: "LLM推理与服务：面试问题与推荐回答" Q9,
# "Scaling Book 第 11 章" §11.7).
# --------------------------------------------------------------------------------------

def paged_multi_query_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                                block_tables: np.ndarray, context_lens: np.ndarray,
                                block_size: int, scale: float, dtype: str,
                                pairs=None) -> np.ndarray:
    """fp64 outputs for q_len new query tokens per sequence, causally masked.

    q:            [B, q_len, n_heads, d_head] stored dtype.
    context_lens: [B] cached tokens INCLUDING the q_len new ones (N_b >= q_len).
    New query i (0-based) of sequence b sees tokens 0 .. N_b - q_len + i.
    pairs:        optional iterable of (b, i, h) to compute; others stay NaN.
    Returns [B, q_len, n_heads, d_head] fp64.
    """
    B, q_len, n_heads, d_head = q.shape
    n_kv_heads = k_pool.shape[2]
    if n_heads % n_kv_heads:
        raise ValueError("n_heads must be a multiple of n_kv_heads")
    group = n_heads // n_kv_heads
    out = np.full((B, q_len, n_heads, d_head), np.nan, dtype=np.float64)
    wanted = {}
    if pairs is None:
        pairs = [(b, i, h) for b in range(B) for i in range(q_len) for h in range(n_heads)]
    for b, i, h in pairs:
        wanted.setdefault((int(b), int(h) // group), []).append((int(i), int(h)))
    for (b, j) in sorted(wanted):
        n_tok = int(context_lens[b])
        if n_tok < q_len:
            raise ValueError("every sequence holds at least its q_len new tokens")
        keys = storage_to_f64(gather_kv(k_pool, block_tables[b], n_tok, block_size, j), dtype)
        vals = storage_to_f64(gather_kv(v_pool, block_tables[b], n_tok, block_size, j), dtype)
        for i, h in sorted(set(wanted[(b, j)])):
            visible = n_tok - q_len + i + 1                  # causal limit of query i
            qh = storage_to_f64(q[b, i, h], dtype)
            scores = scale * (keys[:visible] @ qh)
            weights = softmax_two_pass(scores)
            out[b, i, h] = weights @ vals[:visible]
    return out


# --------------------------------------------------------------------------------------
# Quantized KV cache. "LLM 推理优化全景实战" §4.1 gives the affine quantizer
# Q(x) = round(x / s) + z and its inverse x^ = s * (Q(x) - z); "Scaling Book 第 11 章"
# names FP8 and INT8 as the 8-bit choices. Readings taken where the pages are silent:
# one (s, z) per token and KV head, computed when the token is appended; INT8 codes are
# unsigned bytes 0..255 whose range [min(x, 0), max(x, 0)] includes zero (so zero is exact);
# FP8 is the OCP E4M3 format (sign, 4 exponent bits with bias 7, 3 mantissa bits, no
# infinities, S.1111.111 is NaN, largest finite 448) with s = max|x| / 448 and z = 0.
# Every quantizer step runs in binary32, the precision the GPU kernel uses, so both sides
# reach the same integer codes; dequantization and attention are fp64.
# Code pools:  [num_blocks, block_size, n_kv_heads, d_head] uint8.
# Scale pools: [num_blocks, n_kv_heads, block_size, 2] float32 holding (s, z).
# --------------------------------------------------------------------------------------

KV_FORMATS = ("int8", "fp8")
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """fp64 value of each E4M3 byte, from the field definition."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


_E4M3_POS = e4m3_decode(np.arange(0x7F))          # codes 0..126: the finite non-negatives


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 byte to each binary32 value (ties to the even code), saturating at
    +-448. Found by search over the 127 finite magnitudes; the sign bit is copied."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    hi = np.clip(np.searchsorted(_E4M3_POS, a), 1, 126)   # first value >= a
    lo = hi - 1
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= E4M3_MAX, 126, pick)
    return (pick | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def quantize_row(x: np.ndarray, fmt: str):
    """One token's row of one KV head (any float array) -> (codes uint8, s, z), binary32 steps.

    int8: lo = min(min x, 0), hi = max(max x, 0), s = (hi - lo) / 255 (1 if zero),
          z = clamp(round(-lo / s), 0, 255) (stored as +0 when zero),
          Q = clamp(round(x / s) + z, 0, 255).
    fp8:  s = max|x| / 448 (1 if zero), z = 0, Q = E4M3(x / s).
    round is round-half-to-even.
    """
    x32 = np.asarray(x, dtype=np.float32)
    f255 = np.float32(255.0)
    if fmt == "int8":
        lo = np.minimum(np.min(x32), np.float32(0.0))
        hi = np.maximum(np.max(x32), np.float32(0.0))
        s = np.float32(np.float32(hi - lo) / f255)
        if s == 0:
            s = np.float32(1.0)
        # adding +0 turns a -0 (from -lo = -0.0) into +0: the stored z is never -0
        z = np.float32(np.clip(np.rint(np.float32(-lo) / s), np.float32(0.0), f255) + np.float32(0.0))
        q = np.clip(np.rint(x32 / s) + z, np.float32(0.0), f255)
        return q.astype(np.uint8), np.float32(s), np.float32(z)
    if fmt == "fp8":
        amax = np.max(np.abs(x32))
        s = np.float32(amax / np.float32(E4M3_MAX))
        if s == 0:
            s = np.float32(1.0)
        return e4m3_encode(x32 / s), np.float32(s), np.float32(0.0)
    raise ValueError(f"unknown KV format {fmt!r}")


def dequantize(codes: np.ndarray, s, z, fmt: str) -> np.ndarray:
    """x^ = s * (Q - z) in fp64 (for fp8, Q is the E4M3 value and z = 0). s and z broadcast
    over the last axis of codes."""
    s = np.asarray(s, dtype=np.float64)[..., None]
    z = np.asarray(z, dtype=np.float64)[..., None]
    if fmt == "int8":
        return s * (np.asarray(codes, dtype=np.float64) - z)
    if fmt == "fp8":
        return s * (e4m3_decode(codes) - z)
    raise ValueError(f"unknown KV format {fmt!r}")


def kv_append_quantized(k_codes: np.ndarray, v_codes: np.ndarray, k_scales: np.ndarray,
                        v_scales: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                        block_tables: np.ndarray, positions: np.ndarray, block_size: int,
                        fmt: str, dtype: str):
    """Copies of the code and scale pools with each sequence's new token quantized into
    its slot (chenxutan §2.3 slot rule; quantizer above). k_new, v_new: [B, n_kv_heads,
    d_head] in the stored dtype `dtype`."""
    kc, vc, ks, vs = k_codes.copy(), v_codes.copy(), k_scales.copy(), v_scales.copy()
    for b in range(k_new.shape[0]):
        phys, off = _slot(block_tables[b], int(positions[b]), block_size)
        for j in range(k_new.shape[1]):
            for codes, scales, new in ((kc, ks, k_new), (vc, vs, v_new)):
                row = storage_to_f64(new[b, j], dtype)          # exact in binary32
                q, s, z = quantize_row(row, fmt)
                codes[phys, off, j] = q
                scales[phys, j, off] = (s, z)
    return kc, vc, ks, vs


def gather_dequantized(codes: np.ndarray, scales: np.ndarray, table_row: np.ndarray,
                       n_tokens: int, block_size: int, kv_head: int, fmt: str) -> np.ndarray:
    """Tokens 0..n_tokens-1 of one sequence and KV head, dequantized: [n_tokens, d_head]."""
    t = np.arange(n_tokens, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[t // block_size]
    off = t % block_size
    sz = scales[phys, kv_head, off]                          # [n_tokens, 2]
    return dequantize(codes[phys, off, kv_head], sz[:, 0], sz[:, 1], fmt)


def paged_decode_attention_quantized(q: np.ndarray, k_codes: np.ndarray, v_codes: np.ndarray,
                                     k_scales: np.ndarray, v_scales: np.ndarray,
                                     block_tables: np.ndarray, context_lens: np.ndarray,
                                     block_size: int, scale: float, fmt: str, dtype: str,
                                     pairs=None) -> np.ndarray:
    """The decode attention definition (chenxutan §2.4) over dequantized K and V.

    q: [B, n_heads, d_head] in the stored dtype `dtype`; pools as above, after the append.
    Returns [B, n_heads, d_head] fp64 (NaN outside `pairs` when given)."""
    B, n_heads, d_head = q.shape
    n_kv_heads = k_codes.shape[2]
    group = n_heads // n_kv_heads
    out = np.full((B, n_heads, d_head), np.nan, dtype=np.float64)
    wanted = {}
    for b, h in (pairs if pairs is not None else
                 [(b, h) for b in range(B) for h in range(n_heads)]):
        wanted.setdefault((int(b), int(h) // group), []).append(int(h))
    for (b, j) in sorted(wanted):
        n_tok = int(context_lens[b])
        keys = gather_dequantized(k_codes, k_scales, block_tables[b], n_tok, block_size, j, fmt)
        vals = gather_dequantized(v_codes, v_scales, block_tables[b], n_tok, block_size, j, fmt)
        for h in sorted(set(wanted[(b, j)])):
            qh = storage_to_f64(q[b, h], dtype)
            weights = softmax_two_pass(scale * (keys @ qh))
            out[b, h] = weights @ vals
    return out
