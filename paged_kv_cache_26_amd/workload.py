"""Seeded synthetic workloads and the host-side block manager.

This module builds inputs only: block pools, per-sequence block tables, context lengths,
queries and the new tokens' K/V. It holds none of the attention arithmetic. Both the HIP
path (tests, benchmark) and the fp64 oracle (tests) consume what it returns.

Workload recipe (the same recipe is stated in the design notes):

* seed: ``numpy.random.default_rng(seed)``; the five named workloads use seed = id.
* draw order: context lengths -> physical-block permutation -> per-token K then V of each
  sequence in logical token order (shared prefixes first, one per group) -> q -> k_new ->
  v_new.
* values are drawn in fp32 and rounded to the stored dtype with round-to-nearest-even
  (fp16 via numpy, bf16 via torch's CPU conversion).
* every slot and block not holding a token is filled with NaN ("poison"), so a kernel
  that reads outside a sequence's used slots produces NaN.
* quantized-cache workloads (``kv_format`` "int8" / "fp8") draw each cached token's 8-bit
  codes uniformly (E4M3 NaN bytes excluded) and its per-KV-head (s, z) from the ranges
  below, in the same order (per sequence: K codes, K scales, V codes, V scales); unused
  slots hold code 0x7F and NaN scales. Quantizing the new token is the method's work and
  happens in the library (and in the oracle), not here.
* "context length" in a workload description is the length L_b *before* the decode step.
  The step appends one token at position L_b (q_len tokens at L_b .. L_b + q_len - 1 for
  multi-query steps), then attends over N_b = L_b + q_len tokens.

The block manager follows the paging scheme of "LLM 推理优化全景实战" §2.3 (a shared pool
of fixed-size blocks, a per-request table from logical to physical block, allocation on
demand, an error when the pool is empty) and "09-inference-optimization" (LLM-Code-Hot-100)
section PagedAttention (free list, free a whole sequence). Copy-on-write sharing is named
by "LLM推理与服务：面试问题与推荐回答" Q2 without a mechanism; here it is a per-block
reference count: a write into a block whose count exceeds one first copies the block into
a fresh one and repoints the writer's table entry.
"""

from __future__ import annotations

import collections
import dataclasses
import math

import numpy as np

BLOCK_SIZE = 16

_NAN_BITS = {"f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}
_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


class OutOfBlocksError(RuntimeError):
    """The pool has no free block left."""


def storage_dtype(dtype: str):
    return _STORAGE[dtype]


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the stored dtype (round to nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(x).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def poison_pool(shape, dtype: str) -> np.ndarray:
    """A pool filled with NaN in the stored dtype."""
    if dtype == "f32":
        return np.full(shape, np.nan, dtype=np.float32)
    if dtype == "f16":
        return np.full(shape, np.float16(np.nan), dtype=np.float16)
    return np.full(shape, _NAN_BITS["bf16"], dtype=np.uint16)


# --------------------------------------------------------------------------------------
# Host block manager
# --------------------------------------------------------------------------------------

class BlockManager:
    """Free list, per-sequence block tables and per-block reference counts.

    ``free_order`` fixes the order never-used blocks are handed out; a seeded permutation
    gives random physical placement. Freed blocks go to the back of the free list (first
    in, first out).
    """

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE, free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        if free_order is None:
            self._fresh = iter(range(self.num_blocks))
            self._n_fresh = self.num_blocks
        else:
            order = [int(x) for x in free_order]
            if sorted(order) != list(range(self.num_blocks)):
                raise ValueError("free_order must be a permutation of the pool")
            self._fresh = iter(order)
            self._n_fresh = len(order)
        self._returned: collections.deque[int] = collections.deque()
        self._ref: dict[int, int] = {}
        self.tables: dict[int, list[int]] = {}
        self.copies: list[tuple[int, int]] = []   # (src, dst) block copies made by copy-on-write
        self.n_allocations = 0

    # allocation ------------------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return self._n_fresh + len(self._returned)

    def refcount(self, blk: int) -> int:
        return self._ref.get(int(blk), 0)

    def refcount_array(self) -> np.ndarray:
        out = np.zeros(self.num_blocks, dtype=np.int32)
        for blk, n in self._ref.items():
            out[blk] = n
        return out

    def allocate(self) -> int:
        if self._n_fresh:
            blk = next(self._fresh)
            self._n_fresh -= 1
        elif self._returned:
            blk = self._returned.popleft()
        else:
            raise OutOfBlocksError("no free blocks in the pool")
        self._ref[blk] = 1
        self.n_allocations += 1
        return blk

    def add_sequence(self, seq_id: int) -> None:
        if seq_id in self.tables:
            raise KeyError(f"sequence {seq_id} exists")
        self.tables[seq_id] = []

    def blocks_for(self, n_tokens: int) -> int:
        return -(-int(n_tokens) // self.block_size)

    def grow(self, seq_id: int, n_tokens: int) -> None:
        """Make the table long enough to hold tokens 0..n_tokens-1."""
        table = self.tables[seq_id]
        while len(table) < self.blocks_for(n_tokens):
            table.append(self.allocate())

    # sharing ---------------------------------------------------------------------------
    def fork(self, parent: int, child: int) -> None:
        """The child shares every block of the parent (reference counts go up)."""
        self.add_sequence(child)
        for blk in self.tables[parent]:
            self._ref[blk] += 1
        self.tables[child] = list(self.tables[parent])

    def make_writable(self, seq_id: int, logical_block: int):
        """Copy-on-write: give the sequence a private copy of a shared block.

        Returns (src, dst) when a copy is needed (the caller moves the data), else None.
        """
        table = self.tables[seq_id]
        src = table[logical_block]
        if self._ref[src] <= 1:
            return None
        dst = self.allocate()
        self._release(src)
        table[logical_block] = dst
        self.copies.append((src, dst))
        return src, dst

    # release ---------------------------------------------------------------------------
    def _release(self, blk: int) -> None:
        self._ref[blk] -= 1
        if self._ref[blk] == 0:
            del self._ref[blk]
            self._returned.append(blk)

    def free_sequence(self, seq_id: int) -> None:
        for blk in self.tables.pop(seq_id):
            self._release(blk)

    def table_array(self, seq_ids, max_blocks: int | None = None) -> np.ndarray:
        """[len(seq_ids), max_blocks] int32, unused entries = -1."""
        rows = [self.tables[s] for s in seq_ids]
        width = max(len(r) for r in rows) if max_blocks is None else int(max_blocks)
        out = np.full((len(rows), width), -1, dtype=np.int32)
        for i, r in enumerate(rows):
            out[i, :len(r)] = r
        return out


# --------------------------------------------------------------------------------------
# Workload specifications
# --------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    dtype: str
    batch: int
    n_heads: int
    n_kv_heads: int
    d_head: int
    dist: str                          # "normal" | "half_normal" | "gqa"
    lengths: tuple | None = None       # fixed context lengths L_b (before the step)
    len_range: tuple | None = None     # L_b ~ U{lo..hi}
    pool_blocks: int | None = None     # fixed pool size; None = sized to fit exactly
    groups: int = 0                    # shared-prefix groups (0 = none)
    prefix_len: int = 0
    suffix_range: tuple | None = None  # per-sequence suffix ~ U{lo..hi}
    block_size: int = BLOCK_SIZE
    q_len: int = 1                     # new tokens (queries) per sequence this step
    kv_format: str | None = None       # None: K/V stored in `dtype`; "int8" / "fp8" codes

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads


SPECS = {
    # Tiny MHA step, fp32.
    1: Spec("tiny-mha-f32", "f32", 4, 4, 4, 64, "normal", lengths=(17, 33, 64, 100),
            pool_blocks=64),
    # LLaMA-2-7B-shaped layer, fp16, 32 q / 32 kv heads.
    2: Spec("llama2-7b-layer-f16", "f16", 32, 32, 32, 128, "half_normal",
            len_range=(512, 4096)),
    # GQA layer, bf16, 32 q / 8 kv heads.
    3: Spec("gqa-bf16", "bf16", 64, 32, 8, 128, "gqa", len_range=(4096, 8192)),
    # Long-context GQA, bf16.
    4: Spec("long-context-gqa-bf16", "bf16", 4, 32, 8, 128, "gqa",
            lengths=(32768, 65536, 98304, 131072)),
    # Shared-prefix continuous batch: 8 groups of 16 sequences, 2048-token prefix.
    5: Spec("shared-prefix-bf16", "bf16", 128, 32, 8, 128, "gqa", groups=8,
            prefix_len=2048, suffix_range=(64, 1024)),
}

# Reduced variants with the same structure, sized so the fp64 oracle finishes in seconds
# while still spanning several 16-token blocks, several partitions and a ragged tail.
SMALL_SPECS = {
    1: SPECS[1],
    2: Spec("llama2-7b-layer-f16-small", "f16", 5, 32, 32, 128, "half_normal",
            len_range=(40, 1300)),
    3: Spec("gqa-bf16-small", "bf16", 6, 32, 8, 128, "gqa", len_range=(300, 1500)),
    4: Spec("long-context-gqa-bf16-small", "bf16", 2, 32, 8, 128, "gqa",
            lengths=(2999, 5003)),
    # 200-token prefix ends inside block 12, so every child's first suffix token lands in
    # a shared, partially filled block and triggers a copy-on-write.
    5: Spec("shared-prefix-bf16-small", "bf16", 8, 32, 8, 128, "gqa", groups=2,
            prefix_len=200, suffix_range=(5, 60)),
}


# Quantized-cache workloads: the GQA layer shape with 8-bit K/V codes and per-(token,
# KV head) scales; q, the new tokens and the output stay bf16.
QUANT_SPECS = {
    "int8": Spec("gqa-int8kv", "bf16", 64, 32, 8, 128, "gqa", len_range=(4096, 8192),
                 kv_format="int8"),
    "fp8": Spec("gqa-fp8kv", "bf16", 64, 32, 8, 128, "gqa", len_range=(4096, 8192),
                kv_format="fp8"),
}
QUANT_SMALL_SPECS = {
    "int8": Spec("gqa-int8kv-small", "bf16", 6, 32, 8, 128, "gqa", len_range=(300, 1500),
                 kv_format="int8"),
    "fp8": Spec("gqa-fp8kv-small", "bf16", 6, 32, 8, 128, "gqa", len_range=(300, 1500),
                kv_format="fp8"),
}

# Scale draws of the quantized workloads: s = base / levels * U(0.5, 1.5), so the
# dequantized K spans about +-3 and V about +-1, like the GQA workload's N(0, 1) keys and
# U(-1, 1) values; int8 zero points z ~ U{112..144}, fp8 z = 0.
_QUANT_BASE = {"k": 6.0, "v": 2.0}
_QUANT_LEVELS = {"int8": 255.0, "fp8": 448.0}


def _draw_codes(rng, shape, fmt: str) -> np.ndarray:
    if fmt == "int8":
        return rng.integers(0, 256, size=shape, dtype=np.uint8)
    u = rng.integers(0, 254, size=shape, dtype=np.int64)    # every E4M3 byte but the NaNs
    return np.where(u < 0x7F, u, u + 1).astype(np.uint8)


def _draw_scales(rng, shape, fmt: str, role: str) -> np.ndarray:
    """[..., 2] float32 (s, z) for the given leading shape."""
    base = _QUANT_BASE[role] / _QUANT_LEVELS[fmt]
    if fmt == "fp8":
        base *= 0.5                       # E4M3 spans +-448 around zero: half the range
    sz = np.empty(shape + (2,), dtype=np.float32)
    sz[..., 0] = base * rng.uniform(0.5, 1.5, size=shape)
    sz[..., 1] = rng.integers(112, 145, size=shape) if fmt == "int8" else 0.0
    return sz


@dataclasses.dataclass
class Workload:
    spec: Spec
    seed: int
    k_pool: np.ndarray          # [num_blocks, block_size, n_kv_heads, d_head], before append
    v_pool: np.ndarray
    block_tables: np.ndarray    # [B, max_blocks_per_seq] int32, unused = -1
    positions: np.ndarray       # [B] int32, L_b (where the first new token goes)
    context_lens: np.ndarray    # [B] int32, N_b = L_b + q_len
    q: np.ndarray               # [B, n_heads, d_head] ([B, q_len, n_heads, d_head] if q_len > 1)
    k_new: np.ndarray           # [B, n_kv_heads, d_head] ([B, q_len, n_kv_heads, d_head] if q_len > 1)
    v_new: np.ndarray
    refcount: np.ndarray
    shared_tokens: int          # tokens counted more than once across sequences
    logical_k: list | None = None   # per sequence [L_b, n_kv_heads, d_head] (stored dtype)
    logical_v: list | None = None
    # quantized caches: k_pool / v_pool hold uint8 codes and these the (s, z) pairs,
    # [num_blocks, n_kv_heads, block_size, 2] float32
    k_scales: np.ndarray | None = None
    v_scales: np.ndarray | None = None

    # convenience -------------------------------------------------------------------------
    @property
    def dtype(self) -> str:
        return self.spec.dtype

    @property
    def batch(self) -> int:
        return self.spec.batch

    @property
    def num_blocks(self) -> int:
        return self.k_pool.shape[0]

    @property
    def max_blocks_per_seq(self) -> int:
        return self.block_tables.shape[1]

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.spec.d_head)

    def kv_bytes_per_token(self) -> int:
        """K+V bytes of one token over all KV heads (codes plus (s, z) when quantized)."""
        s = self.spec
        if s.kv_format:
            return 2 * s.n_kv_heads * (s.d_head + 8)
        return 2 * s.n_kv_heads * s.d_head * DTYPE_BYTES[s.dtype]

    def kv_bytes_logical(self) -> int:
        """K+V bytes a decode step reads: every attended token, once per KV head."""
        return int(self.context_lens.sum()) * self.kv_bytes_per_token()

    def kv_bytes_unique(self) -> int:
        """As above, with tokens shared between sequences counted once."""
        tok = int(self.context_lens.sum()) - self.shared_tokens
        return tok * self.kv_bytes_per_token()


def _draw(rng, shape, dist: str, role: str) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "half_normal":
        return np.float32(0.5) * rng.standard_normal(shape, dtype=np.float32)
    if dist == "gqa":
        if role == "v":
            return rng.random(shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
        return rng.standard_normal(shape, dtype=np.float32)
    raise ValueError(dist)


def _write_blocks(pool, phys_ids, data, block_size):
    """Store tokens [n, H_kv, d] into consecutive blocks phys_ids (last one may be partial)."""
    n = data.shape[0]
    nb = len(phys_ids)
    if n == 0:
        return
    padded = poison_pool((nb * block_size,) + data.shape[1:], _dtype_of(pool))
    padded[:n] = data
    pool[np.asarray(phys_ids, dtype=np.int64)] = padded.reshape((nb, block_size) + data.shape[1:])


def _dtype_of(pool) -> str:
    if pool.dtype == np.float32:
        return "f32"
    if pool.dtype == np.float16:
        return "f16"
    return "bf16"


def _allocate(mgr: BlockManager, spec: Spec, ctx_before, prefix_of):
    """Allocation sequence shared by the dry run and the real build.

    Groups first (one parent per group holding the prefix), then each sequence: fork from
    its group's parent (or start empty), copy-on-write the shared partial block it will
    write into, grow to hold its own tokens plus the new one.
    """
    B = spec.batch
    parents = {}
    if spec.groups:
        for g in range(spec.groups):
            pid = -(g + 1)
            mgr.add_sequence(pid)
            mgr.grow(pid, spec.prefix_len)
            parents[g] = pid
    for b in range(B):
        if spec.groups:
            mgr.fork(parents[prefix_of[b]], b)
            first_private = spec.prefix_len // spec.block_size
            if spec.prefix_len % spec.block_size and ctx_before[b] + spec.q_len > spec.prefix_len:
                mgr.make_writable(b, first_private)
        else:
            mgr.add_sequence(b)
        mgr.grow(b, ctx_before[b] + spec.q_len)
    if spec.groups:
        for g in range(spec.groups):
            mgr.free_sequence(parents[g])
    return parents


def make_workload(spec: Spec | int, seed: int | None = None, *, keep_logical: bool = False,
                  small: bool = False) -> Workload:
    """Build one seeded workload (pools before the append, tables after allocation)."""
    if isinstance(spec, int):
        seed = spec if seed is None else seed
        spec = (SMALL_SPECS if small else SPECS)[spec]
    if seed is None:
        raise ValueError("seed required for a custom spec")
    rng = np.random.default_rng(seed)
    B, Hkv, d, bs = spec.batch, spec.n_kv_heads, spec.d_head, spec.block_size

    # 1. context lengths (before the step)
    if spec.groups:
        suffix = rng.integers(spec.suffix_range[0], spec.suffix_range[1], size=B,
                              endpoint=True).astype(np.int64)
        ctx = [int(spec.prefix_len + s) for s in suffix]
        per_group = B // spec.groups
        prefix_of = [b // per_group for b in range(B)]
    elif spec.lengths is not None:
        ctx = [int(x) for x in spec.lengths]
        suffix = None
        prefix_of = [0] * B
    else:
        ctx = [int(x) for x in rng.integers(spec.len_range[0], spec.len_range[1], size=B,
                                            endpoint=True)]
        suffix = None
        prefix_of = [0] * B
    if len(ctx) != B:
        raise ValueError("lengths do not match batch")

    # 2. physical placement: a seeded permutation is the free-list order
    dry = BlockManager(2 ** 31 - 1, bs)
    _allocate(dry, spec, ctx, prefix_of)
    needed = dry.n_allocations
    num_blocks = spec.pool_blocks if spec.pool_blocks is not None else needed
    if num_blocks < needed:
        raise ValueError("pool too small for the workload")
    perm = rng.permutation(num_blocks)
    mgr = BlockManager(num_blocks, bs, free_order=perm)

    fmt = spec.kv_format
    if fmt is not None:
        if spec.groups or spec.q_len != 1:
            raise ValueError("quantized workloads are single-query without shared prefixes")
        # codes of unused slots: 0x7F (an E4M3 NaN); their scales: NaN
        k_pool = np.full((num_blocks, bs, Hkv, d), 0x7F, dtype=np.uint8)
        v_pool = np.full((num_blocks, bs, Hkv, d), 0x7F, dtype=np.uint8)
        k_scales = np.full((num_blocks, Hkv, bs, 2), np.nan, dtype=np.float32)
        v_scales = np.full((num_blocks, Hkv, bs, 2), np.nan, dtype=np.float32)
    else:
        k_pool = poison_pool((num_blocks, bs, Hkv, d), spec.dtype)
        v_pool = poison_pool((num_blocks, bs, Hkv, d), spec.dtype)
        k_scales = v_scales = None

    # allocation, replayed on the real manager; data written in draw order below
    _allocate(mgr, spec, ctx, prefix_of)
    tables = mgr.table_array(range(B))
    logical_k = [] if keep_logical else None
    logical_v = [] if keep_logical else None

    # 3. per-token K, V in logical order
    shared_tokens = 0
    if spec.groups:
        prefix_k, prefix_v = [], []
        for g in range(spec.groups):
            pk = to_storage(_draw(rng, (spec.prefix_len, Hkv, d), spec.dist, "k"), spec.dtype)
            pv = to_storage(_draw(rng, (spec.prefix_len, Hkv, d), spec.dist, "v"), spec.dtype)
            prefix_k.append(pk)
            prefix_v.append(pv)
        # the parents' blocks hold the prefix; children that did not copy still point there
        n_pref_blocks = -(-spec.prefix_len // bs)
        written = set()
        for b in range(B):
            g = prefix_of[b]
            ids = tuple(int(x) for x in tables[b, :n_pref_blocks])
            key = (g, ids)
            if key not in written:
                _write_blocks(k_pool, list(ids), prefix_k[g], bs)
                _write_blocks(v_pool, list(ids), prefix_v[g], bs)
                written.add(key)
        per_group = B // spec.groups
        shared_tokens = spec.groups * (per_group - 1) * spec.prefix_len
        for b in range(B):
            g = prefix_of[b]
            s_len = ctx[b] - spec.prefix_len
            sk = to_storage(_draw(rng, (s_len, Hkv, d), spec.dist, "k"), spec.dtype)
            sv = to_storage(_draw(rng, (s_len, Hkv, d), spec.dist, "v"), spec.dtype)
            full_k = np.concatenate([prefix_k[g], sk])
            full_v = np.concatenate([prefix_v[g], sv])
            first = spec.prefix_len // bs          # first block this sequence may write
            nb = -(-ctx[b] // bs)
            ids = [int(x) for x in tables[b, first:nb]]
            _write_blocks(k_pool, ids, full_k[first * bs:], bs)
            _write_blocks(v_pool, ids, full_v[first * bs:], bs)
            if keep_logical:
                logical_k.append(full_k)
                logical_v.append(full_v)
    elif fmt is not None:
        for b in range(B):
            nb = -(-ctx[b] // bs)
            ids = np.asarray(tables[b, :nb], dtype=np.int64)
            t = np.arange(ctx[b])
            for codes, scales, role in ((k_pool, k_scales, "k"), (v_pool, v_scales, "v")):
                c = _draw_codes(rng, (ctx[b], Hkv, d), fmt)
                sz = _draw_scales(rng, (ctx[b], Hkv), fmt, role)
                codes[ids[t // bs], t % bs] = c
                scales[ids[t // bs], :, t % bs] = sz
            if keep_logical:
                logical_k.append(None)
                logical_v.append(None)
    else:
        for b in range(B):
            kk = to_storage(_draw(rng, (ctx[b], Hkv, d), spec.dist, "k"), spec.dtype)
            vv = to_storage(_draw(rng, (ctx[b], Hkv, d), spec.dist, "v"), spec.dtype)
            nb = -(-ctx[b] // bs)
            ids = [int(x) for x in tables[b, :nb]]
            _write_blocks(k_pool, ids, kk, bs)
            _write_blocks(v_pool, ids, vv, bs)
            if keep_logical:
                logical_k.append(kk)
                logical_v.append(vv)

    # 4. query, 5. new token's K and V
    ql = spec.q_len
    lead = (B,) if ql == 1 else (B, ql)
    q = to_storage(_draw(rng, lead + (spec.n_heads, d), spec.dist, "q"), spec.dtype)
    k_new = to_storage(_draw(rng, lead + (Hkv, d), spec.dist, "k"), spec.dtype)
    v_new = to_storage(_draw(rng, lead + (Hkv, d), spec.dist, "v"), spec.dtype)

    positions = np.asarray(ctx, dtype=np.int32)
    return Workload(spec=spec, seed=seed, k_pool=k_pool, v_pool=v_pool, block_tables=tables,
                    positions=positions, context_lens=positions + ql, q=q, k_new=k_new,
                    v_new=v_new, refcount=mgr.refcount_array(), shared_tokens=shared_tokens,
                    logical_k=logical_k, logical_v=logical_v, k_scales=k_scales,
                    v_scales=v_scales)


def relabel_blocks(wl: Workload, seed: int) -> Workload:
    """Move every physical block to a new id given by a seeded permutation.

    The data moves with its block and the tables are rewritten, so each sequence sees the
    same tokens in the same logical order.
    """
    rng = np.random.default_rng(seed)
    perm = rng.permutation(wl.num_blocks)          # old id -> new id
    k_pool = np.empty_like(wl.k_pool)
    v_pool = np.empty_like(wl.v_pool)
    k_pool[perm] = wl.k_pool
    v_pool[perm] = wl.v_pool
    tables = wl.block_tables.copy()
    used = tables >= 0
    tables[used] = perm[tables[used]]
    refcount = np.empty_like(wl.refcount)
    refcount[perm] = wl.refcount
    scales = {}
    for name in ("k_scales", "v_scales"):
        src = getattr(wl, name)
        if src is not None:
            scales[name] = np.empty_like(src)
            scales[name][perm] = src
    return dataclasses.replace(wl, k_pool=k_pool, v_pool=v_pool, block_tables=tables,
                               refcount=refcount, **scales)


def to_torch(wl: Workload, device="cuda"):
    """The workload's arrays as torch tensors on ``device`` (bf16 reinterpreted from bits)."""
    import torch

    def conv(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(a).to(device)

    out = {
        "k_pool": conv(wl.k_pool), "v_pool": conv(wl.v_pool),
        "k_new": conv(wl.k_new), "v_new": conv(wl.v_new), "q": conv(wl.q),
        "block_tables": torch.from_numpy(wl.block_tables).to(device),
        "positions": torch.from_numpy(wl.positions).to(device),
        "context_lens": torch.from_numpy(wl.context_lens).to(device),
    }
    if wl.k_scales is not None:
        out["k_scales"] = torch.from_numpy(wl.k_scales).to(device)
        out["v_scales"] = torch.from_numpy(wl.v_scales).to(device)
    return out


def from_torch(t, dtype: str) -> np.ndarray:
    """A tensor back in the stored numpy representation (bf16 as uint16 bits)."""
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
