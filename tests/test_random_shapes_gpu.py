"""Seeded random shapes through every attention entry point, against the
oracle: block size, head dim, GQA grouping (up to 32 query heads per KV head,
two head chunks), cache dtype (f16, bf16, fp8 with bf16/f16 q), ragged and
empty lengths, and for the prefill heavy-tailed key scales that move the
softmax maximum along the keys. Each seed draws one shape; a failure names
its seed and shape."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import prefix_reuse_amd as pkv
import workloads
from _helpers import (TOL, bits, fp8_inputs_from_pools, nan_fp8_caches, np64, oracle_decode, oracle_fp8_caches,
                      oracle_prefill, gpu_prefill, report)
from test_cascade_gpu import run_cascade

pytestmark = pytest.mark.gpu


def _shape(rng):
    b = int(rng.choice([16, 32]))
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8, 16, 32]))
    return b, d, hkv * g, hkv


def _cache_kind(rng):
    return ["f16", "bf16", "fp8"][int(rng.integers(3))]


def _same(a, b):
    """Bit-for-bit equality (the caches hold NaN in their unused slots)."""
    return np.array_equal(bits(a), bits(b))


def _heavy_tailed_keys(case, rng, dtype):
    """Scale every live cached key row (and every new one) by exp(N(0, 1.2))."""
    k = case.k_pool.float()
    live = ~torch.isnan(k[:, :, 0, 0])
    f = torch.from_numpy(np.exp(rng.normal(0.0, 1.2, size=tuple(live.shape)))).float()
    case.k_pool = torch.where(live[:, :, None, None], k * f[:, :, None, None], k).to(dtype)
    fn = torch.from_numpy(np.exp(rng.normal(0.0, 1.2, size=(case.k_new.shape[0],)))).float()
    case.k_new = (case.k_new.float() * fn[:, None, None]).to(dtype)


@pytest.mark.parametrize("seed", [*range(12), *range(100, 112)])
def test_random_decode_step_and_noalloc(seed):
    """pkv_decode_attn, pkv_decode_step_attn and pkv_decode_attn_noalloc on one
    random batch (up to 150 sequences of 0-800 tokens)."""
    rng = np.random.default_rng(7000 + seed)
    b, d, hq, hkv = _shape(rng)
    kind = _cache_kind(rng)
    lens = [int(x) for x in rng.integers(0, 801, int(rng.integers(1, 151)))]
    print(f"seed {seed}: decode {len(lens)} seqs, {kind} cache, d={d} B={b} {hq}/{hkv}", flush=True)
    dev = "cuda"
    if kind == "fp8":
        q_dtype = [torch.bfloat16, torch.float16][int(rng.integers(2))]
        case = workloads.make_decode_case(7000 + seed, lens, hq, hkv, d, b, torch.float32)
        inp = fp8_inputs_from_pools(case, q_dtype)
        ek, ev = oracle_fp8_caches(case, inp)
        ref = oracle.decode_attention(np64(case.q.to(q_dtype)), ek, ev, case.block_tables.numpy(),
                                      case.context_lens.numpy(), case.scale, fp8=True,
                                      k_scale=inp.k_scale, v_scale=inp.v_scale)
        kc, vc = nan_fp8_caches(case, dev)
        pkv.append(inp.rows_k.to(dev), inp.rows_v.to(dev), inp.slots.to(dev), kc, vc, inp.k_scale, inp.v_scale)
        q = case.q.to(q_dtype).to(dev)
        scales = dict(k_scale=inp.k_scale, v_scale=inp.v_scale)
        out_dtype, tol = q_dtype, TOL["fp8"]
    else:
        dtype = torch.float16 if kind == "f16" else torch.bfloat16
        case = workloads.make_decode_case(7000 + seed, lens, hq, hkv, d, b, dtype)
        ref = oracle_decode(case)
        kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, dev)
        pkv.append(case.k_new.to(dev), case.v_new.to(dev), case.slot_mapping.to(dev), kc, vc)
        q = case.q.to(dev)
        scales = {}
        out_dtype, tol = dtype, TOL[dtype]
    bt, cl = case.block_tables.to(dev), case.context_lens.to(dev)
    out = pkv.decode_attn(q, kc, vc, bt, cl, case.scale, **scales)
    torch.cuda.synchronize()
    assert report(f"random decode {seed}", np64(out), ref, out_dtype, tol) <= 1.0
    # the no-allocation entry point takes batches whose workspace fits its 32 MiB
    need = pkv.decode_workspace_bytes(len(lens), hq, hkv, d, case.block_tables.shape[1], b)
    if need <= 32 << 20:
        out_na = pkv.decode_attn_noalloc(q, kc, vc, bt, cl, case.scale, **scales)
        torch.cuda.synchronize()
        assert _same(out, out_na), "the no-allocation entry point differs from pkv_decode_attn"
    if kind != "fp8":
        # the step form from the cache before the newest tokens went in
        kc2, vc2 = pkv.caches_from_logical(case.k_pool, case.v_pool, dev)
        out_s = pkv.decode_step_attn(q, case.k_new.to(dev), case.v_new.to(dev), kc2, vc2, bt, cl, case.scale)
        torch.cuda.synchronize()
        assert _same(out, out_s), "the step form differs from append + decode"
        assert _same(kc, kc2) and _same(vc, vc2), "the step form left different caches"


@pytest.mark.parametrize("seed", [*range(12), *range(100, 112)])
def test_random_suffix_prefill(seed):
    """pkv_suffix_prefill_attn and pkv_suffix_prefill_attn_split on random
    requests (up to 6, prefixes 0-1,000, suffixes 0-200), half of them with
    heavy-tailed key scales."""
    rng = np.random.default_rng(7100 + seed)
    b, d, hq, hkv = _shape(rng)
    kind = _cache_kind(rng)
    r = int(rng.integers(1, 7))
    plen = [int(x) for x in rng.integers(0, 1001, r)]
    slen = [int(x) for x in rng.integers(0, 201, r)]
    heavy = bool(rng.random() < 0.5)
    print(f"seed {seed}: prefill P={plen} S={slen}, {kind} cache, d={d} B={b} {hq}/{hkv}, heavy keys {heavy}",
          flush=True)
    if kind == "fp8":
        q_dtype = [torch.bfloat16, torch.float16][int(rng.integers(2))]
        case = workloads.make_prefill_case(7100 + seed, plen, slen, hq, hkv, d, b, torch.float32)
        if heavy:
            _heavy_tailed_keys(case, rng, torch.float32)
        inp = fp8_inputs_from_pools(case, q_dtype)
        kc, vc = nan_fp8_caches(case)
        pkv.append(inp.rows_k.cuda(), inp.rows_v.cuda(), inp.slots.cuda(), kc, vc, inp.k_scale, inp.v_scale)
        q = case.q_suffix.to(q_dtype)
        args = (q.cuda(), kc, vc, case.block_tables.cuda(), case.prefix_lens.cuda(), case.suffix_lens.cuda(),
                case.scale)
        out = pkv.suffix_prefill_attn(*args, k_scale=inp.k_scale, v_scale=inp.v_scale)
        out_split = pkv.suffix_prefill_attn_split(*args, k_scale=inp.k_scale, v_scale=inp.v_scale)
        torch.cuda.synchronize()
        ek, ev = oracle_fp8_caches(case, inp)
        ref = oracle.suffix_prefill_attention(np64(q), ek, ev, case.block_tables.numpy(), case.prefix_lens.numpy(),
                                              case.suffix_lens.numpy(), case.scale, fp8=True,
                                              k_scale=inp.k_scale, v_scale=inp.v_scale)
        assert report(f"random prefill {seed}", np64(out), ref, q_dtype, TOL["fp8"]) <= 1.0
        assert report(f"random split prefill {seed}", np64(out_split), ref, q_dtype, TOL["fp8"]) <= 1.0
    else:
        dtype = torch.float16 if kind == "f16" else torch.bfloat16
        case = workloads.make_prefill_case(7100 + seed, plen, slen, hq, hkv, d, b, dtype)
        if heavy:
            _heavy_tailed_keys(case, rng, dtype)
        run = gpu_prefill(case)
        out = run.out
        out_split = pkv.suffix_prefill_attn_split(case.q_suffix.cuda(), run.k_cache, run.v_cache,
                                                  case.block_tables.cuda(), case.prefix_lens.cuda(),
                                                  case.suffix_lens.cuda(), case.scale)
        torch.cuda.synchronize()
        assert np.isfinite(np64(out)).all() and np.isfinite(np64(out_split)).all()
        ref = oracle_prefill(case)
        assert report(f"random prefill {seed}", np64(out), ref, dtype, TOL[dtype]) <= 1.0
        assert report(f"random split prefill {seed}", np64(out_split), ref, dtype, TOL[dtype]) <= 1.0


@pytest.mark.parametrize("seed", [*range(8), *range(100, 108)])
def test_random_cascade(seed):
    """pkv_cascade_decode_attn on random groupings (1-5 groups of 1-40
    sequences, shared prefixes 0-400 tokens, private parts 0-300)."""
    rng = np.random.default_rng(7200 + seed)
    b, d, hq, hkv = _shape(rng)
    dtype = [torch.float16, torch.bfloat16][int(rng.integers(2))]
    groups = []
    for _ in range(int(rng.integers(1, 6))):
        sh = int(rng.integers(0, 401))
        groups.append(([int(sh + x) for x in rng.integers(0, 301, int(rng.integers(1, 41)))], sh))
    print(f"seed {seed}: cascade {[(len(g), s) for g, s in groups]}, {dtype} d={d} B={b} {hq}/{hkv}", flush=True)
    case = workloads.make_grouped_decode_case(7200 + seed, groups, hq, hkv, d, b, dtype)
    out = run_cascade(case)
    assert report(f"random cascade {seed}", np64(out), oracle_decode(case), dtype, TOL[dtype]) <= 1.0
