"""Shared plumbing of the GPU tests: moving workload inputs to the device,
running the HIP path through the C ABI, running the oracle on the same inputs
and comparing. The oracle never sees a value the HIP path produced."""
from __future__ import annotations

import math
from dataclasses import dataclass

import os

import numpy as np
import torch

import _margins
import oracle
import prefix_reuse_amd as pkv
import workloads

TOL = {torch.float32: 2e-3, torch.float16: 2e-3, torch.bfloat16: 2e-3, "fp8": 2e-2}


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a tensor (for exact comparisons, NaN included)."""
    t = t.detach().cpu().contiguous()
    view = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()]
    return t.view(view).numpy()


_MANTISSA_BITS = {torch.float32: 23, torch.float16: 10, torch.bfloat16: 7}


def half_ulp(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Half a unit in the last place of ``dtype`` at magnitude |x| (normal range;
    the binade is taken one ulp up so a value rounding across a power of two
    is covered)."""
    m = _MANTISSA_BITS[dtype]
    a = np.maximum(np.abs(x) * (1 + 2.0 ** -m), 2.0 ** -14)
    return 0.5 * np.exp2(np.floor(np.log2(a)) - m)


def report(name: str, got: np.ndarray, ref: np.ndarray, out_dtype=None, tol=None, record: bool = True) -> float:
    """Print the worst error and return it as a multiple of the allowed error.

    Allowed error per element = tol + half an ulp of the output dtype at |ref|:
    the kernels accumulate in fp32 and round once when storing a 16-bit result,
    and that final rounding alone reaches half an ulp (3.9e-3 for bf16 values in
    [1, 2)). With ``out_dtype=None`` the bare ``tol`` is returned as is."""
    err = np.abs(got - ref)
    if err.size == 0:
        return 0.0
    i = np.unravel_index(np.nanargmax(err), err.shape)
    worst = float(np.nanmax(err))
    msg = f"[{name}] max|err|={worst:.3e} at {tuple(int(x) for x in i)} max|o|={float(np.nanmax(np.abs(ref))):.3e}"
    if out_dtype is None or tol is None:
        print(msg, flush=True)
        return worst
    allowed = tol + half_ulp(ref, out_dtype)
    ratio = float(np.nanmax(err / allowed))
    bad = int(np.sum(~(err <= allowed)))
    if bad:  # a NaN or inf where the oracle is finite counts as a violation, not as a skipped element
        ratio = max(ratio, float("inf") if np.any(~np.isfinite(err)) else ratio)
    print(msg + f" worst err/allowed={ratio:.3f} (tol {tol:g} + half-ulp of {out_dtype}), violations={bad}",
          flush=True)
    test = os.environ.get("PYTEST_CURRENT_TEST", "")
    family = test.split(" ")[0].split("[")[0].replace("tests/", "") or name
    if record:
        _margins.record(family, name, ratio, worst, float(np.nanmax(np.abs(ref))))
    return ratio


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
@dataclass
class DecodeRun:
    out: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor


def gpu_decode(case: workloads.DecodeCase, device="cuda", append_new=True) -> DecodeRun:
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, device)
    if append_new:
        pkv.append(case.k_new.to(device), case.v_new.to(device), case.slot_mapping.to(device), kc, vc)
    out = pkv.decode_attn(case.q.to(device), kc, vc, case.block_tables.to(device),
                          case.context_lens.to(device), case.scale)
    torch.cuda.synchronize()
    return DecodeRun(out, kc, vc)


def oracle_decode(case: workloads.DecodeCase, seqs=None) -> np.ndarray:
    kc, vc = oracle.append(np64(case.k_pool), np64(case.v_pool), np64(case.k_new), np64(case.v_new),
                           case.slot_mapping.numpy())
    return oracle.decode_attention(np64(case.q), kc, vc, case.block_tables.numpy(),
                                   case.context_lens.numpy(), case.scale, seqs=seqs)


# ---------------------------------------------------------------------------
# fp8 caches: every live token is appended (quantized) from its raw row
# ---------------------------------------------------------------------------
@dataclass
class Fp8Inputs:
    rows_k: torch.Tensor   # [T, Hkv, d] raw rows (row dtype)
    rows_v: torch.Tensor
    slots: torch.Tensor    # int64 [T]
    k_scale: float
    v_scale: float
    num_blocks: int


def fp8_inputs_from_pools(case, row_dtype=torch.float32) -> Fp8Inputs:
    """Turn a case with float pools into raw rows + the slots they occupy
    (including the rows a decode step appends), with scale = amax / 448."""
    b = case.block_size
    pools_k = case.k_pool.float()
    pools_v = case.v_pool.float()
    live = ~torch.isnan(pools_k[:, :, 0, 0])
    idx = live.nonzero()
    slots = idx[:, 0] * b + idx[:, 1]
    rk = pools_k[idx[:, 0], idx[:, 1]]
    rv = pools_v[idx[:, 0], idx[:, 1]]
    if getattr(case, "k_new", None) is not None:
        keep = case.slot_mapping >= 0
        slots = torch.cat([slots, case.slot_mapping[keep]])
        rk = torch.cat([rk, case.k_new.float()[keep]])
        rv = torch.cat([rv, case.v_new.float()[keep]])
    rk = rk.to(row_dtype)
    rv = rv.to(row_dtype)
    k_scale = float(np.float32(rk.float().abs().max().item()) / np.float32(448.0))
    v_scale = float(np.float32(rv.float().abs().max().item()) / np.float32(448.0))
    return Fp8Inputs(rk, rv, slots.to(torch.int64), k_scale, v_scale, case.k_pool.shape[0])


def nan_fp8_caches(case, device="cuda"):
    nb, b, h, d = case.k_pool.shape
    kc, vc = pkv.empty_caches(nb, b, h, d, torch.float8_e4m3fn, device)
    kc.view(torch.uint8).fill_(workloads.fp8_nan_code)
    vc.view(torch.uint8).fill_(workloads.fp8_nan_code)
    return kc, vc


def oracle_fp8_caches(case, inp: Fp8Inputs):
    nb, b, h, d = case.k_pool.shape
    kc = np.full((nb, b, h, d), workloads.fp8_nan_code, np.uint8)
    vc = np.full((nb, b, h, d), workloads.fp8_nan_code, np.uint8)
    return oracle.append(kc, vc, inp.rows_k.float().numpy(), inp.rows_v.float().numpy(),
                         inp.slots.numpy(), fp8=True, k_scale=inp.k_scale, v_scale=inp.v_scale)


def gpu_fp8_decode(case, inp: Fp8Inputs, q_dtype, device="cuda"):
    kc, vc = nan_fp8_caches(case, device)
    pkv.append(inp.rows_k.to(device), inp.rows_v.to(device), inp.slots.to(device), kc, vc,
               inp.k_scale, inp.v_scale)
    out = pkv.decode_attn(case.q.to(q_dtype).to(device), kc, vc, case.block_tables.to(device),
                          case.context_lens.to(device), case.scale, k_scale=inp.k_scale,
                          v_scale=inp.v_scale)
    torch.cuda.synchronize()
    return DecodeRun(out, kc, vc)


# ---------------------------------------------------------------------------
# suffix prefill
# ---------------------------------------------------------------------------
def gpu_prefill(case: workloads.PrefillCase, device="cuda"):
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, device)
    pkv.append(case.k_new.to(device), case.v_new.to(device), case.slot_mapping.to(device), kc, vc)
    out = pkv.suffix_prefill_attn(case.q_suffix.to(device), kc, vc, case.block_tables.to(device),
                                  case.prefix_lens.to(device), case.suffix_lens.to(device), case.scale)
    torch.cuda.synchronize()
    return DecodeRun(out, kc, vc)


def oracle_prefill(case: workloads.PrefillCase, rows=None) -> np.ndarray:
    kc, vc = oracle.append(np64(case.k_pool), np64(case.v_pool), np64(case.k_new), np64(case.v_new),
                           case.slot_mapping.numpy())
    return oracle.suffix_prefill_attention(np64(case.q_suffix), kc, vc, case.block_tables.numpy(),
                                           case.prefix_lens.numpy(), case.suffix_lens.numpy(),
                                           case.scale, rows=rows)
