"""Python binding of libpkv's host-side prefix index (include/pkv_prefix.h).

Argument marshalling only: matching, allocation and eviction run in the C++
of libpkv.so. ``PrefixCache`` turns a request's token IDs into the block
table, prefix length and slot mapping that ``append`` and
``suffix_prefill_attn`` consume; ``RadixTree`` is the token-path matcher.
"""
from __future__ import annotations

import ctypes
from typing import List, Sequence, Tuple

import numpy as np

from . import PkvError, lib

__all__ = ["PrefixCache", "RadixTree", "NoBlocks", "NotFound"]

PKV_ERR_NO_BLOCKS = 8
PKV_ERR_NOT_FOUND = 9

_p64 = ctypes.POINTER(ctypes.c_int64)
_p32 = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p

_SIGS = {
    "pkv_pc_create": [ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(_vp)],
    "pkv_pc_admit": [_vp, _p32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64, _p32, ctypes.c_int64, _p64,
                     _p64, _p64],
    "pkv_pc_append": [_vp, ctypes.c_int64, ctypes.c_int32, _p64],
    "pkv_pc_commit": [_vp, ctypes.c_int64, _p64],
    "pkv_pc_release": [_vp, ctypes.c_int64],
    "pkv_pc_block_table": [_vp, ctypes.c_int64, _p32, ctypes.c_int64, _p64],
    "pkv_pc_stats": [_vp, _p64, _p64, _p64],
    "pkv_radix_create": [ctypes.c_int32, ctypes.POINTER(_vp)],
    "pkv_radix_match": [_vp, _p32, ctypes.c_int64, _p64, _p64],
    "pkv_radix_insert": [_vp, _p32, ctypes.c_int64, _p64, _p64],
    "pkv_radix_lock": [_vp, _p32, ctypes.c_int64],
    "pkv_radix_unlock": [_vp, _p32, ctypes.c_int64],
    "pkv_radix_evict": [_vp, ctypes.c_int64, _p64, ctypes.c_int64, _p64],
    "pkv_radix_total_tokens": [_vp, _p64],
}
for _name, _args in _SIGS.items():
    getattr(lib, _name).argtypes = _args
    getattr(lib, _name).restype = ctypes.c_int
lib.pkv_pc_destroy.argtypes = [_vp]
lib.pkv_pc_destroy.restype = None
lib.pkv_radix_destroy.argtypes = [_vp]
lib.pkv_radix_destroy.restype = None


class NoBlocks(PkvError):
    """The pool has too few free or evictable blocks."""


class NotFound(PkvError):
    """Unknown request id, prefix not stored, or unlock without lock."""


def _check(fn: str, rc: int) -> None:
    if rc == 0:
        return
    msg = lib.pkv_last_error().decode(errors="replace")
    cls = {PKV_ERR_NO_BLOCKS: NoBlocks, PKV_ERR_NOT_FOUND: NotFound}.get(rc, PkvError)
    raise cls(fn, rc, msg)


def _i32(tokens: Sequence[int]) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    if a.size and (a.min() < -(1 << 31) or a.max() >= (1 << 31)):
        raise ValueError("token IDs must fit in int32")
    return a.astype(np.int32)


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(ctypes.POINTER(t))


class PrefixCache:
    """Chain-hash prefix cache over a pool of ``num_blocks`` blocks of
    ``block_size`` tokens (page A §05; tenant salt §06)."""

    def __init__(self, num_blocks: int, block_size: int):
        h = _vp()
        _check("pkv_pc_create", lib.pkv_pc_create(num_blocks, block_size, ctypes.byref(h)))
        self._h = h
        self.block_size = block_size

    def __del__(self, _destroy=lib.pkv_pc_destroy):  # bound now: module globals may be gone at exit
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _destroy(h)
            self._h = None

    def admit(self, tokens: Sequence[int], salt: int = 0, extra: int = 0
              ) -> Tuple[int, List[int], int, List[int]]:
        """(request id, block table, prefix length, slots of tokens prefix..n-1)."""
        t = _i32(tokens)
        n = int(t.size)
        nblk = max(1, -(-n // self.block_size))
        table = np.zeros(nblk, dtype=np.int32)
        slots = np.zeros(max(n, 1), dtype=np.int64)
        prefix, rid = ctypes.c_int64(), ctypes.c_int64()
        _check("pkv_pc_admit", lib.pkv_pc_admit(self._h, _ptr(t, ctypes.c_int32), n, ctypes.c_uint64(salt),
                                                ctypes.c_uint64(extra), _ptr(table, ctypes.c_int32), nblk,
                                                _ptr(slots, ctypes.c_int64), ctypes.byref(prefix),
                                                ctypes.byref(rid)))
        p = prefix.value
        return rid.value, table.tolist(), p, slots[:n - p].tolist()

    def append(self, request_id: int, token: int) -> int:
        slot = ctypes.c_int64()
        _check("pkv_pc_append", lib.pkv_pc_append(self._h, request_id, int(token), ctypes.byref(slot)))
        return slot.value

    def commit(self, request_id: int) -> int:
        n = ctypes.c_int64()
        _check("pkv_pc_commit", lib.pkv_pc_commit(self._h, request_id, ctypes.byref(n)))
        return n.value

    def release(self, request_id: int) -> None:
        _check("pkv_pc_release", lib.pkv_pc_release(self._h, request_id))

    def block_table(self, request_id: int) -> List[int]:
        n = ctypes.c_int64()
        _check("pkv_pc_block_table", lib.pkv_pc_block_table(self._h, request_id, None, 0, ctypes.byref(n)))
        out = np.zeros(max(n.value, 1), dtype=np.int32)
        _check("pkv_pc_block_table", lib.pkv_pc_block_table(self._h, request_id, _ptr(out, ctypes.c_int32),
                                                            n.value, ctypes.byref(n)))
        return out[:n.value].tolist()

    def stats(self) -> Tuple[int, int, int]:
        """(free blocks, evictable cached blocks, cached blocks)."""
        f, e, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check("pkv_pc_stats", lib.pkv_pc_stats(self._h, ctypes.byref(f), ctypes.byref(e), ctypes.byref(c)))
        return f.value, e.value, c.value


class RadixTree:
    """Radix tree of token sequences with one int64 value per stored token,
    matched in whole pages of ``page`` tokens (page A §03-§04)."""

    def __init__(self, page: int = 1):
        h = _vp()
        _check("pkv_radix_create", lib.pkv_radix_create(page, ctypes.byref(h)))
        self._h = h
        self.page = page

    def __del__(self, _destroy=lib.pkv_radix_destroy):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _destroy(h)
            self._h = None

    def match_prefix(self, tokens: Sequence[int]) -> Tuple[int, List[int]]:
        t = _i32(tokens)
        vals = np.zeros(max(t.size, 1), dtype=np.int64)
        m = ctypes.c_int64()
        _check("pkv_radix_match", lib.pkv_radix_match(self._h, _ptr(t, ctypes.c_int32), t.size,
                                                      _ptr(vals, ctypes.c_int64), ctypes.byref(m)))
        return m.value, vals[:m.value].tolist()

    def insert(self, tokens: Sequence[int], values: Sequence[int]) -> int:
        t = _i32(tokens)
        v = np.ascontiguousarray(np.asarray(values, dtype=np.int64))
        if v.size < t.size - t.size % self.page:
            raise ValueError("one value per token")
        v = v if v.size else np.zeros(1, dtype=np.int64)
        e = ctypes.c_int64()
        _check("pkv_radix_insert", lib.pkv_radix_insert(self._h, _ptr(t, ctypes.c_int32), t.size,
                                                        _ptr(v, ctypes.c_int64), ctypes.byref(e)))
        return e.value

    def lock(self, tokens: Sequence[int], length: int) -> None:
        t = _i32(tokens)
        _check("pkv_radix_lock", lib.pkv_radix_lock(self._h, _ptr(t, ctypes.c_int32), length))

    def unlock(self, tokens: Sequence[int], length: int) -> None:
        t = _i32(tokens)
        _check("pkv_radix_unlock", lib.pkv_radix_unlock(self._h, _ptr(t, ctypes.c_int32), length))

    def total_tokens(self) -> int:
        n = ctypes.c_int64()
        _check("pkv_radix_total_tokens", lib.pkv_radix_total_tokens(self._h, ctypes.byref(n)))
        return n.value

    def evict(self, num_tokens: int) -> List[int]:
        cap = max(self.total_tokens(), 1)
        vals = np.zeros(cap, dtype=np.int64)
        n = ctypes.c_int64()
        _check("pkv_radix_evict", lib.pkv_radix_evict(self._h, num_tokens, _ptr(vals, ctypes.c_int64), cap,
                                                      ctypes.byref(n)))
        return vals[:n.value].tolist()
