"""Paged-KV attention with prefix reuse on MI355X: Python binding of libpkv.

Argument marshalling only: every computation runs in the HIP kernels of
``libpkv.so`` (built in-tree by ``prefix_reuse_amd.build``). PyTorch provides
device memory and the current stream. If the library is missing this module
raises at import; there is no fallback.

Physical cache layout (see include/pkv.h): ``k_cache[num_blocks, H_kv, B, d]``
and ``v_cache[num_blocks, H_kv, d, B]``; a token's slot is
``physical_block * B + offset``. ``k_logical``/``v_logical`` give views in the
order ``[num_blocks, B, H_kv, d]``.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path
from typing import Optional, Tuple

import torch

__all__ = [
    "LIB_PATH", "lib", "PkvError",
    "append", "decode_attn", "decode_attn_noalloc", "decode_step_attn", "suffix_prefill_attn",
    "suffix_prefill_attn_split", "suffix_prefill_workspace_bytes", "decode_workspace_bytes",
    "cascade_decode_attn", "cascade_workspace_bytes",
    "empty_caches", "caches_from_logical", "k_logical", "v_logical", "abi_version",
]

# PKV_LIBRARY selects another build of the same library (the CPU sanitizer
# build, libpkv_san.so); by default the in-tree libpkv.so is loaded
LIB_PATH = Path(os.environ.get("PKV_LIBRARY") or Path(__file__).resolve().parent / "libpkv.so")

_DT = {
    torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float8_e4m3fn: 3,
    torch.int32: 4, torch.int64: 5,
}


class PkvTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


class PkvError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not LIB_PATH.exists():
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m prefix_reuse_amd.build` "
            "(hipcc, gfx950). There is no CPU fallback.")
    L = ctypes.CDLL(str(LIB_PATH))
    P = ctypes.POINTER(PkvTensor)
    L.pkv_append.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
    L.pkv_append.restype = ctypes.c_int
    L.pkv_decode_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]
    L.pkv_decode_workspace_bytes.restype = ctypes.c_size_t
    L.pkv_decode_attn.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                  ctypes.c_void_p, ctypes.c_size_t, P, ctypes.c_void_p]
    L.pkv_decode_attn.restype = ctypes.c_int
    L.pkv_decode_attn_noalloc.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_float, P,
                                          ctypes.c_void_p]
    L.pkv_decode_attn_noalloc.restype = ctypes.c_int
    L.pkv_decode_step_attn.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_void_p, ctypes.c_size_t, P, ctypes.c_void_p]
    L.pkv_decode_step_attn.restype = ctypes.c_int
    L.pkv_suffix_prefill_attn.argtypes = [P, P, P, P, P, P, ctypes.c_float, ctypes.c_float,
                                          ctypes.c_float, P, ctypes.c_void_p]
    L.pkv_suffix_prefill_attn.restype = ctypes.c_int
    L.pkv_suffix_prefill_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]
    L.pkv_suffix_prefill_workspace_bytes.restype = ctypes.c_size_t
    L.pkv_suffix_prefill_attn_split.argtypes = [P, P, P, P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                                ctypes.c_void_p, ctypes.c_size_t, P, ctypes.c_void_p]
    L.pkv_suffix_prefill_attn_split.restype = ctypes.c_int
    L.pkv_cascade_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    L.pkv_cascade_workspace_bytes.restype = ctypes.c_size_t
    L.pkv_cascade_decode_attn.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                          ctypes.c_void_p, ctypes.c_size_t, P, ctypes.c_void_p]
    L.pkv_cascade_decode_attn.restype = ctypes.c_int
    L.pkv_last_error.argtypes = []
    L.pkv_last_error.restype = ctypes.c_char_p
    L.pkv_abi_version.argtypes = []
    L.pkv_abi_version.restype = ctypes.c_int
    return L


lib = _load()


def abi_version() -> int:
    return lib.pkv_abi_version()


def _desc(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() > 4:
        raise ValueError("at most 4 dims")
    d = PkvTensor()
    d.data = t.data_ptr() if t.numel() > 0 else 0
    d.dtype = _DT[t.dtype]
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ref(d):
    return ctypes.byref(d) if d is not None else None


def _stream(device: torch.device) -> int:
    if device.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    # the library launches on the current HIP device, so the tensors must be there
    current = torch.cuda.current_device()
    if device.index is not None and device.index != current:
        raise ValueError(f"tensors live on cuda:{device.index} but the current device is cuda:{current}; "
                         f"call under torch.cuda.device({device.index})")
    return torch.cuda.current_stream(device).cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise PkvError(fn, rc, lib.pkv_last_error().decode())


# ---------------------------------------------------------------------------
# cache allocation and layout views (plumbing)
# ---------------------------------------------------------------------------
def empty_caches(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                 dtype: torch.dtype, device="cuda") -> Tuple[torch.Tensor, torch.Tensor]:
    k = torch.empty(num_blocks, num_kv_heads, block_size, head_dim, dtype=dtype, device=device)
    v = torch.empty(num_blocks, num_kv_heads, head_dim, block_size, dtype=dtype, device=device)
    return k, v


def k_logical(k_cache: torch.Tensor) -> torch.Tensor:
    """View [num_blocks, B, H_kv, d] of a physical K cache."""
    return k_cache.permute(0, 2, 1, 3)


def v_logical(v_cache: torch.Tensor) -> torch.Tensor:
    """View [num_blocks, B, H_kv, d] of a physical V cache."""
    return v_cache.permute(0, 3, 1, 2)


def caches_from_logical(k_pool: torch.Tensor, v_pool: torch.Tensor, device="cuda"):
    """Physical caches holding the contents of logical [NB, B, H_kv, d] pools."""
    k = k_pool.permute(0, 2, 1, 3).contiguous().to(device)
    v = v_pool.permute(0, 2, 3, 1).contiguous().to(device)
    return k, v


# ---------------------------------------------------------------------------
# the three operations
# ---------------------------------------------------------------------------
def append(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
           v_cache: torch.Tensor, k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Write rows k[i], v[i] ([T, H_kv, d]) into slot slot_mapping[i] of the caches."""
    dk, dv, ds, dkc, dvc = map(_desc, (k, v, slot_mapping, k_cache, v_cache))
    rc = lib.pkv_append(_ref(dk), _ref(dv), _ref(ds), _ref(dkc), _ref(dvc), float(k_scale),
                        float(v_scale), _stream(k_cache.device))
    _check("pkv_append", rc)


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           max_blocks_per_seq: int, block_size: int) -> int:
    return int(lib.pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              max_blocks_per_seq, block_size))


def decode_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                out: Optional[torch.Tensor] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One paged decode step; returns ``out`` [num_seqs, H_q, d]."""
    if out is None:
        out = torch.empty_like(q)
    ws_ptr, ws_bytes = _decode_workspace(q, k_cache, block_tables, workspace)
    dq, dkc, dvc, dbt, dcl, do = map(_desc, (q, k_cache, v_cache, block_tables, context_lens, out))
    rc = lib.pkv_decode_attn(_ref(dq), _ref(dkc), _ref(dvc), _ref(dbt), _ref(dcl), float(scale),
                             float(k_scale), float(v_scale), ws_ptr, ws_bytes, _ref(do),
                             _stream(q.device))
    _check("pkv_decode_attn", rc)
    return out


def decode_attn_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                        out: Optional[torch.Tensor] = None, k_scale: float = 1.0,
                        v_scale: float = 1.0) -> torch.Tensor:
    """pkv_decode_attn without a workspace: the library's device-resident
    scratch holds the partial results (see include/pkv.h). Pass ``out`` to
    avoid the one allocation this wrapper would otherwise make."""
    if out is None:
        out = torch.empty_like(q)
    dq, dkc, dvc, dbt, dcl, do = map(_desc, (q, k_cache, v_cache, block_tables, context_lens, out))
    rc = lib.pkv_decode_attn_noalloc(_ref(dq), _ref(dkc), _ref(dvc), _ref(dbt), _ref(dcl), float(scale),
                                     float(k_scale), float(v_scale), _ref(do), _stream(q.device))
    _check("pkv_decode_attn_noalloc", rc)
    return out


def _decode_workspace(q, k_cache, block_tables, workspace):
    need = decode_workspace_bytes(q.shape[0], q.shape[1], k_cache.shape[1], q.shape[2],
                                  block_tables.shape[1], k_cache.shape[2])
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)  # no initial contents needed
    if not need:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def decode_step_attn(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                     v_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                     scale: float, out: Optional[torch.Tensor] = None, k_scale: float = 1.0,
                     v_scale: float = 1.0, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A decode step in one call: each sequence's newest K/V row (k_new[s],
    v_new[s]) goes to position context_lens[s] - 1 of the cache, and its query
    attends to all context_lens[s] tokens; returns ``out``."""
    if out is None:
        out = torch.empty_like(q)
    ws_ptr, ws_bytes = _decode_workspace(q, k_cache, block_tables, workspace)
    dq, dkn, dvn, dkc, dvc, dbt, dcl, do = map(_desc, (q, k_new, v_new, k_cache, v_cache, block_tables,
                                                        context_lens, out))
    rc = lib.pkv_decode_step_attn(_ref(dq), _ref(dkn), _ref(dvn), _ref(dkc), _ref(dvc), _ref(dbt), _ref(dcl),
                                  float(scale), float(k_scale), float(v_scale), ws_ptr, ws_bytes, _ref(do),
                                  _stream(q.device))
    _check("pkv_decode_step_attn", rc)
    return out


def suffix_prefill_attn(q_suffix: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        block_tables: torch.Tensor, prefix_lens: torch.Tensor,
                        suffix_lens: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                        k_scale: float = 1.0, v_scale: float = 1.0) -> torch.Tensor:
    """Attention of the packed suffix rows over their cached prefix + causal suffix."""
    if out is None:
        out = torch.empty_like(q_suffix)
    dq, dkc, dvc, dbt, dp, dsl, do = map(_desc, (q_suffix, k_cache, v_cache, block_tables,
                                                  prefix_lens, suffix_lens, out))
    rc = lib.pkv_suffix_prefill_attn(_ref(dq), _ref(dkc), _ref(dvc), _ref(dbt), _ref(dp), _ref(dsl),
                                     float(scale), float(k_scale), float(v_scale), _ref(do),
                                     _stream(q_suffix.device))
    _check("pkv_suffix_prefill_attn", rc)
    return out


def suffix_prefill_workspace_bytes(total_suffix_tokens: int, num_requests: int, num_q_heads: int,
                                   num_kv_heads: int, head_dim: int, max_blocks_per_seq: int,
                                   block_size: int) -> int:
    """Workspace bytes pkv_suffix_prefill_attn_split needs (0: the batch takes no split)."""
    return lib.pkv_suffix_prefill_workspace_bytes(total_suffix_tokens, num_requests, num_q_heads, num_kv_heads,
                                                  head_dim, max_blocks_per_seq, block_size)


def suffix_prefill_attn_split(q_suffix: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              block_tables: torch.Tensor, prefix_lens: torch.Tensor,
                              suffix_lens: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                              k_scale: float = 1.0, v_scale: float = 1.0,
                              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """suffix_prefill_attn with the keys of each row tile split over several
    work-groups when the batch has too few rows to fill the GPU."""
    if out is None:
        out = torch.empty_like(q_suffix)
    need = suffix_prefill_workspace_bytes(q_suffix.shape[0], prefix_lens.shape[0], q_suffix.shape[1],
                                          k_cache.shape[1], q_suffix.shape[2], block_tables.shape[1],
                                          k_cache.shape[2])
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q_suffix.device)  # no initial contents needed
    ws_ptr, ws_bytes = (workspace.data_ptr(), workspace.numel() * workspace.element_size()) if need else (None, 0)
    dq, dkc, dvc, dbt, dp, dsl, do = map(_desc, (q_suffix, k_cache, v_cache, block_tables,
                                                  prefix_lens, suffix_lens, out))
    rc = lib.pkv_suffix_prefill_attn_split(_ref(dq), _ref(dkc), _ref(dvc), _ref(dbt), _ref(dp), _ref(dsl),
                                           float(scale), float(k_scale), float(v_scale), ws_ptr, ws_bytes,
                                           _ref(do), _stream(q_suffix.device))
    _check("pkv_suffix_prefill_attn_split", rc)
    return out


def cascade_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int) -> int:
    return lib.pkv_cascade_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim)


def cascade_decode_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        block_tables: torch.Tensor, context_lens: torch.Tensor, group_starts: torch.Tensor,
                        shared_lens: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                        k_scale: float = 1.0, v_scale: float = 1.0,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode for groups of sequences sharing prefix blocks (the shared part is
    read once per group); same result as ``decode_attn``."""
    if out is None:
        out = torch.empty_like(q)
    need = cascade_workspace_bytes(q.shape[0], q.shape[1], k_cache.shape[1], q.shape[2])
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if (need and workspace is not None) else None
    ws_bytes = workspace.numel() * workspace.element_size() if (need and workspace is not None) else 0
    descs = list(map(_desc, (q, k_cache, v_cache, block_tables, context_lens, group_starts, shared_lens, out)))
    rc = lib.pkv_cascade_decode_attn(*[_ref(d) for d in descs[:7]], float(scale), float(k_scale), float(v_scale),
                                     ws_ptr, ws_bytes, _ref(descs[7]), _stream(q.device))
    _check("pkv_cascade_decode_attn", rc)
    return out
