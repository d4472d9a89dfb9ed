"""Python handle for libpkv's native block manager (include/pkv_block_manager.h).

Argument marshalling only: allocation, sharing and copy-on-write run in the C++ manager.
"""

from __future__ import annotations

import ctypes

import numpy as np

from . import pkv


class OutOfBlocks(RuntimeError):
    """The pool has no free block left for the request."""


class NativeBlockManager:
    """Free list, per-sequence block tables and reference counts, kept in libpkv."""

    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        self._lib = pkv.load_library()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            ptr = order.ctypes.data_as(ctypes.c_void_p)
        else:
            ptr = None
        self._h = self._lib.pkv_bm_create(int(num_blocks), int(block_size), ptr)
        if not self._h:
            raise ValueError("invalid block manager arguments (free_order must be a permutation)")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if self._h:
            self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, status: int, where: str) -> int:
        if status == -13:
            raise OutOfBlocks(f"{where}: {pkv.pkv_status_str(status)}")
        if status < 0:
            raise pkv.PkvError(status, where)
        return status

    def add_sequence(self, seq_id: int) -> None:
        self._check(self._lib.pkv_bm_add_sequence(self._h, seq_id), "add_sequence")

    def fork(self, parent: int, child: int) -> None:
        self._check(self._lib.pkv_bm_fork(self._h, parent, child), "fork")

    def free_sequence(self, seq_id: int) -> None:
        self._check(self._lib.pkv_bm_free_sequence(self._h, seq_id), "free_sequence")

    def grow(self, seq_id: int, n_tokens: int) -> None:
        self._check(self._lib.pkv_bm_grow(self._h, seq_id, int(n_tokens)), "grow")

    def append_slot(self, seq_id: int, token_index: int):
        """(physical block, slot, copy pair or None) for writing token `token_index`."""
        out = (ctypes.c_int32 * 4)()
        self._check(self._lib.pkv_bm_append_slot(
            self._h, seq_id, int(token_index), ctypes.byref(out, 0), ctypes.byref(out, 4),
            ctypes.byref(out, 8), ctypes.byref(out, 12)), "append_slot")
        copy = None if out[2] < 0 else (int(out[2]), int(out[3]))
        return int(out[0]), int(out[1]), copy

    def append_slots(self, seq_ids, token_index):
        """Batched append_slot; returns (blocks, slots, copy_pairs [n, 2] with -1 = none).

        Raises on the first failing item; the items before it stay applied."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        toks = np.ascontiguousarray(token_index, dtype=np.int32)
        n = len(ids)
        blocks = np.empty(n, dtype=np.int32)
        slots = np.empty(n, dtype=np.int32)
        pairs = np.empty((n, 2), dtype=np.int32)
        done = ctypes.c_int32(0)
        vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
        st = self._lib.pkv_bm_append_slots(self._h, vp(ids), vp(toks), n, vp(blocks), vp(slots),
                                           vp(pairs), ctypes.byref(done))
        self._check(st, f"append_slots (item {done.value})")
        return blocks, slots, pairs

    @property
    def num_free(self) -> int:
        return self._check(self._lib.pkv_bm_num_free(self._h), "num_free")

    def refcount(self, block: int) -> int:
        return self._check(self._lib.pkv_bm_refcount(self._h, int(block)), "refcount")

    def num_blocks_of(self, seq_id: int) -> int:
        return self._check(self._lib.pkv_bm_num_blocks_of(self._h, seq_id), "num_blocks_of")

    def table_array(self, seq_ids, max_blocks: int | None = None) -> np.ndarray:
        ids = np.ascontiguousarray(list(seq_ids), dtype=np.int64)
        if max_blocks is None:
            max_blocks = max((self.num_blocks_of(int(s)) for s in ids), default=0)
        out = np.empty((len(ids), int(max_blocks)), dtype=np.int32)
        self._check(self._lib.pkv_bm_tables(self._h, ids.ctypes.data_as(ctypes.c_void_p),
                                            len(ids), int(max_blocks),
                                            out.ctypes.data_as(ctypes.c_void_p)), "tables")
        return out


class SharedPrefixes:
    """Groups of a batch for pkv_paged_decode_attention_shared_prefix."""

    def __init__(self, seq_group, group_blocks, max_group_size, max_shared_blocks):
        self.seq_group = seq_group            # [B] int32, group id or -1
        self.group_blocks = group_blocks      # [n_groups] int32, shared leading blocks
        self.max_group_size = max_group_size
        self.max_shared_blocks = max_shared_blocks

    @property
    def n_groups(self) -> int:
        return int(self.group_blocks.shape[0])


def find_shared_prefixes(tables, context_lens, block_size: int = 16,
                         min_members: int = 2) -> SharedPrefixes:
    """Group sequences by the leading physical blocks their tables share (native host code,
    pkv_find_shared_prefixes)."""
    lib = pkv.load_library()
    t = np.ascontiguousarray(tables, dtype=np.int32)
    n = np.ascontiguousarray(context_lens, dtype=np.int32)
    B = t.shape[0]
    if t.ndim != 2 or n.shape != (B,):
        raise ValueError("tables must be [B, max_blocks] and context_lens [B]")
    seq_group = np.empty(B, np.int32)
    group_blocks = np.empty(max(B, 1), np.int32)
    out = [ctypes.c_int32(0) for _ in range(3)]
    vp = ctypes.c_void_p
    st = lib.pkv_find_shared_prefixes(t.ctypes.data_as(vp), B, t.shape[1], n.ctypes.data_as(vp),
                                      int(block_size), int(min_members),
                                      seq_group.ctypes.data_as(vp), group_blocks.ctypes.data_as(vp),
                                      *[ctypes.byref(o) for o in out])
    if st != 0:
        raise pkv.PkvError(st, "pkv_find_shared_prefixes")
    ng, mg, ms = (o.value for o in out)
    return SharedPrefixes(seq_group, group_blocks[:ng].copy(), mg, ms)
