"""Suffix-prefill parity: the HIP path against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import prefix_reuse_amd as pkv
import workloads
from _helpers import TOL, fp8_inputs_from_pools, gpu_prefill, nan_fp8_caches, np64, oracle_fp8_caches, oracle_prefill, report

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("block,dim", [(16, 128), (32, 128), (16, 64), (32, 64)])
def test_prefill_ragged(dtype, block, dim):
    print(f"prefill ragged dtype={dtype} B={block} d={dim}", flush=True)
    prefix = [0, 4, 31, 100, 257, 0, 45]
    suffix = [1, 1, 33, 70, 40, 130, 9]
    case = workloads.make_prefill_case(500 + block + dim, prefix, suffix, 8, 2, dim, block, dtype)
    run = gpu_prefill(case)
    assert report("prefill", np64(run.out), oracle_prefill(case), dtype, TOL[dtype]) <= 1.0


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 2), (12, 4), (32, 1)])
def test_prefill_group_sizes(hq, hkv):
    print(f"prefill group hq={hq} hkv={hkv}", flush=True)
    case = workloads.make_prefill_case(600 + hq + hkv, [10, 77], [50, 21], hq, hkv, 128, 16, torch.bfloat16)
    run = gpu_prefill(case)
    assert report("group", np64(run.out), oracle_prefill(case), torch.bfloat16, TOL[torch.bfloat16]) <= 1.0


def test_prefill_many_requests():
    """150 requests (some with empty suffixes, one with a suffix of 80 rows
    that spans two work-groups at G=4): each work-group finds its request
    among batches of 64, so the third batch is reached."""
    rng = np.random.default_rng(604)
    prefix = [int(x) for x in rng.integers(0, 120, 150)]
    suffix = [int(x) for x in rng.integers(0, 12, 150)]
    suffix[140] = 80
    case = workloads.make_prefill_case(604, prefix, suffix, 8, 2, 64, 16, torch.float16)
    print(f"prefill 150 requests, {sum(suffix)} rows", flush=True)
    run = gpu_prefill(case)
    assert report("150 requests", np64(run.out), oracle_prefill(case), torch.float16, TOL[torch.float16]) <= 1.0


def test_prefill_what_day_is_it_shape():
    # 4 cached tokens, 1 new token: the new row equals a decode of 5 tokens
    case = workloads.make_prefill_case(601, [4], [1], 32, 8, 128, 16, torch.bfloat16)
    run = gpu_prefill(case)
    assert report("P4S1", np64(run.out), oracle_prefill(case), torch.bfloat16, TOL[torch.bfloat16]) <= 1.0


def test_prefill_empty_suffix_requests_are_skipped():
    case = workloads.make_prefill_case(602, [30, 10, 0], [0, 25, 0], 8, 2, 128, 16, torch.float16)
    run = gpu_prefill(case)
    assert run.out.shape[0] == 25
    assert report("empty", np64(run.out), oracle_prefill(case), torch.float16, TOL[torch.float16]) <= 1.0


@pytest.mark.parametrize("q_dtype", [torch.bfloat16, torch.float16])
def test_prefill_fp8_cache(q_dtype):
    case = workloads.make_prefill_case(603, [64, 300, 0], [40, 17, 90], 8, 2, 128, 32, torch.float32)
    # the cached prefix and the new suffix rows are both quantized by append
    inp = fp8_inputs_from_pools(case, q_dtype)
    kc, vc = nan_fp8_caches(case)
    pkv.append(inp.rows_k.cuda(), inp.rows_v.cuda(), inp.slots.cuda(), kc, vc, inp.k_scale, inp.v_scale)
    q = case.q_suffix.to(q_dtype)
    out = pkv.suffix_prefill_attn(q.cuda(), kc, vc, case.block_tables.cuda(), case.prefix_lens.cuda(),
                                  case.suffix_lens.cuda(), case.scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
    torch.cuda.synchronize()
    ek, ev = oracle_fp8_caches(case, inp)
    ref = oracle.suffix_prefill_attention(np64(q), ek, ev, case.block_tables.numpy(), case.prefix_lens.numpy(),
                                          case.suffix_lens.numpy(), case.scale, fp8=True,
                                          k_scale=inp.k_scale, v_scale=inp.v_scale)
    assert report("prefill-fp8", np64(out), ref, q_dtype, TOL["fp8"]) <= 1.0


@pytest.mark.slow
def test_config4_suffix_prefill_sampled_rows():
    case = workloads.config4_suffix_prefill()
    run = gpu_prefill(case)
    out = np64(run.out)
    assert np.isfinite(out).all()
    # every request's first two and last two rows, plus a seeded sample
    rng = np.random.default_rng(4)
    rows = set()
    for r in range(16):
        rows |= {100 * r, 100 * r + 1, 100 * r + 98, 100 * r + 99}
    rows |= set(rng.choice(1600, 40, replace=False).tolist())
    rows = sorted(rows)
    ref = oracle_prefill(case, rows=rows)
    assert report("config4", out[rows], ref[rows], torch.bfloat16, TOL[torch.bfloat16]) <= 1.0


@pytest.mark.slow
@pytest.mark.parametrize("dtype,block", [(torch.bfloat16, 16), (torch.float16, 32)])
def test_prefill_long_prefix_sampled_rows(dtype, block):
    """Prefixes of 30,000 and 12,345 cached tokens (each work-group runs
    hundreds of stages through its LDS ring), checked on sampled rows. q is
    scaled by 4 and every V row carries a per-(KV head, dim) mean in
    [0.5, 2] with a random sign, so that |out| is of order 1 over these long
    contexts and an all-zero or garbage output fails the gate."""
    case = workloads.make_prefill_case(640 + block, [30000, 12345], [64, 37], 32, 8, 128, block, dtype)
    g = torch.Generator().manual_seed(641)
    mean = (torch.rand(8, 128, generator=g) * 1.5 + 0.5) * (torch.randint(0, 2, (8, 128), generator=g) * 2 - 1)
    case.v_pool = (case.v_pool.float() + mean).to(dtype)  # unused slots stay NaN
    case.v_new = (case.v_new.float() + mean).to(dtype)
    case.q_suffix = (case.q_suffix.float() * 4).to(dtype)
    print(f"{dtype} B={block}", flush=True)
    out = np64(gpu_prefill(case).out)
    assert np.isfinite(out).all()
    rows = sorted({0, 1, 62, 63, 64, 65, 99, 100} | set(np.random.default_rng(642).choice(101, 6, replace=False).tolist()))
    ref = oracle_prefill(case, rows=rows)
    assert np.abs(ref[rows]).max() > 0.5
    assert report(f"long prefix {dtype} B={block}", out[rows], ref[rows], dtype, TOL[dtype]) <= 1.0


@pytest.mark.slow
@pytest.mark.parametrize("q_dtype", [torch.bfloat16, torch.float16])
def test_prefill_fp8_long_prefix_sampled_rows(q_dtype):
    """The long-prefix case over an fp8 cache (prefix and suffix rows
    quantized by append, per-tensor scales): 24,000 and 9,000 cached tokens,
    q scaled by 4, V with a per-(KV head, dim) mean, sampled rows against
    the oracle over the same codes."""
    case = workloads.make_prefill_case(650, [24000, 9000], [48, 29], 32, 8, 128, 32, torch.float32)
    g = torch.Generator().manual_seed(651)
    mean = (torch.rand(8, 128, generator=g) * 1.5 + 0.5) * (torch.randint(0, 2, (8, 128), generator=g) * 2 - 1)
    case.v_pool = case.v_pool + mean  # unused slots stay NaN
    case.v_new = case.v_new + mean
    case.q_suffix = case.q_suffix * 4
    inp = fp8_inputs_from_pools(case, q_dtype)
    kc, vc = nan_fp8_caches(case)
    pkv.append(inp.rows_k.cuda(), inp.rows_v.cuda(), inp.slots.cuda(), kc, vc, inp.k_scale, inp.v_scale)
    q = case.q_suffix.to(q_dtype)
    print(f"fp8, q {q_dtype}", flush=True)
    out = np64(pkv.suffix_prefill_attn(q.cuda(), kc, vc, case.block_tables.cuda(), case.prefix_lens.cuda(),
                                       case.suffix_lens.cuda(), case.scale, k_scale=inp.k_scale,
                                       v_scale=inp.v_scale))
    torch.cuda.synchronize()
    assert np.isfinite(out).all()
    rows = sorted({0, 1, 46, 47, 48, 49, 75, 76} | set(np.random.default_rng(652).choice(77, 6, replace=False).tolist()))
    ek, ev = oracle_fp8_caches(case, inp)
    ref = oracle.suffix_prefill_attention(np64(q), ek, ev, case.block_tables.numpy(), case.prefix_lens.numpy(),
                                          case.suffix_lens.numpy(), case.scale, fp8=True, k_scale=inp.k_scale,
                                          v_scale=inp.v_scale, rows=rows)
    assert np.abs(ref[rows]).max() > 0.5
    assert report(f"fp8 long prefix q {q_dtype}", out[rows], ref[rows], q_dtype, TOL["fp8"]) <= 1.0


@pytest.mark.slow
def test_config4_reuse_equals_full_recompute_on_gpu():
    """The 2,000-token request with 1,900 cached gives the same 100 rows as
    prefilling all 2,000 (prefix reuse does not change the output)."""
    full = workloads.make_prefill_case(1004, [0], [2000], 32, 8, 128, 16, torch.bfloat16)
    run_full = gpu_prefill(full)
    kc, vc = run_full.k_cache, run_full.v_cache
    q_tail = full.q_suffix[1900:].cuda()
    out = pkv.suffix_prefill_attn(q_tail, kc, vc, full.block_tables.cuda(), torch.tensor([1900], dtype=torch.int32).cuda(),
                                  torch.tensor([100], dtype=torch.int32).cuda(), full.scale)
    torch.cuda.synchronize()
    # suffix-only rows against the full-prefill rows (two GPU results) ...
    assert report("reuse-vs-full", np64(out), np64(run_full.out[1900:]), torch.bfloat16, TOL[torch.bfloat16]) <= 1.0
    # ... and both against the oracle on a sample of rows
    rows = [0, 1, 50, 98, 99]
    ref = oracle_prefill(full, rows=[1900 + r for r in rows])
    assert report("reuse-oracle", np64(out)[rows], ref[[1900 + r for r in rows]], torch.bfloat16, TOL[torch.bfloat16]) <= 1.0


@pytest.mark.parametrize("big", [65280.0, 70000.0, -1.0e6])
def test_prefill_bf16_large_values(big):
    """bf16 values are converted to f16 for the value product when every live
    value fits (65280 is the largest bf16 value below f16's overflow
    threshold); a work-group that meets a larger one (70000, -1e6) redoes its
    rows without the conversion. Either way the result matches the oracle.

    Tolerance: an output is a convex combination of value rows and linear in
    V, so the 2e-3 gate (stated for values of order 1) is applied to the
    problem scaled by max|V|, i.e. 2e-3 * max|V| plus half an output ulp."""
    print(f"prefill bf16 planted V value {big}", flush=True)
    case = workloads.make_prefill_case(604, [40, 300, 7], [30, 60, 90], 8, 2, 128, 16, torch.bfloat16)
    b = case.block_size
    for r, t, h, d in ((0, 5, 0, 7), (1, 290, 1, 100)):  # live prefix tokens
        blk = int(case.block_tables[r, t // b])
        case.v_pool[blk, t % b, h, d] = big
    case.v_new[12, 1, 3] = big  # a suffix token of request 0
    run = gpu_prefill(case)
    ref = oracle_prefill(case)
    assert np.isfinite(np64(run.out)).all()
    scale = max(1.0, abs(big))
    assert report(f"big {big}", np64(run.out), ref, torch.bfloat16, TOL[torch.bfloat16] * scale) <= 1.0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("shape", ["gradual", "jump"])
def test_prefill_scores_that_grow_along_the_keys(dtype, shape):
    """Softmax maxima that keep moving while the stage loop runs. "gradual":
    every cached key row is scaled by 1 + 3t/P, so a row's largest score grows
    by ~10 (base 2) along the prefix and the running max has to move inside
    the loop's full steps. "jump": one late cached key of request 0 is 40 x the
    query of suffix row 0 (head 0), a score hundreds of units (base 2) above
    every earlier one, far past what a running max can absorb in fp32 without
    moving. Both against the oracle."""
    case = workloads.make_prefill_case(610, [1500, 700], [64, 40], 8, 2, 128, 16, dtype)
    b = case.block_size
    k = case.k_pool.float()
    if shape == "gradual":
        for r, plen in enumerate(case.prefix_lens.tolist()):
            for t in range(plen):
                blk = int(case.block_tables[r, t // b])
                k[blk, t % b] *= 1.0 + 3.0 * t / plen
    else:
        t = 1400
        blk = int(case.block_tables[0, t // b])
        k[blk, t % b, 0] = 40.0 * case.q_suffix[0, 0].float()
    case.k_pool = k.to(dtype)
    print(f"prefill {dtype} keys {shape}", flush=True)
    run = gpu_prefill(case)
    ref = oracle_prefill(case)
    assert np.isfinite(np64(run.out)).all()
    assert report(f"keys {shape} {dtype}", np64(run.out), ref, dtype, TOL[dtype]) <= 1.0


@pytest.mark.parametrize("seed", range(3))
def test_prefill_heavy_tailed_key_scales(seed):
    """Every cached and new key row scaled by exp(N(0, 1.5)): row maxima jump up
    and down along the keys, so the bf16 fast pass's full steps move the
    running max (and rescale P) many times. Against the oracle."""
    rng = np.random.default_rng(620 + seed)
    case = workloads.make_prefill_case(620 + seed, [900, 1300, 260], [70, 33, 128], 16, 4, 128, 16, torch.bfloat16)
    k = case.k_pool.float()
    live = ~torch.isnan(k[:, :, 0, 0])
    f = torch.from_numpy(np.exp(rng.normal(0.0, 1.5, size=tuple(live.shape)))).float()
    k = torch.where(live[:, :, None, None], k * f[:, :, None, None], k)
    case.k_pool = k.to(torch.bfloat16)
    fn = torch.from_numpy(np.exp(rng.normal(0.0, 1.5, size=(case.k_new.shape[0],)))).float()
    case.k_new = (case.k_new.float() * fn[:, None, None]).to(torch.bfloat16)
    print(f"prefill heavy-tailed key scales, seed {seed}", flush=True)
    run = gpu_prefill(case)
    ref = oracle_prefill(case)
    assert np.isfinite(np64(run.out)).all()
    assert report(f"heavy-tailed keys {seed}", np64(run.out), ref, torch.bfloat16, TOL[torch.bfloat16]) <= 1.0


@pytest.mark.parametrize("jump", [100.0, 118.0, 124.0, 126.0, 126.5, 127.0, 127.5, 128.0, 131.0])
def test_prefill_score_jump_near_float_range(jump):
    """One late cached key of request 0 set to a multiple of the query of suffix
    row 0 (head 0), so that its score (base 2, scale included) is `jump` units
    above zero: P computed against the running max is finite but up to 2^128,
    and moving the max must not lose it (a factor of 2^-jump computed as exp2
    flushes to 0 below 2^-126). Against the oracle, bf16 and f16."""
    for dtype in (torch.bfloat16, torch.float16):
        case = workloads.make_prefill_case(611, [1500, 300], [40, 20], 8, 2, 128, 16, dtype)
        b = case.block_size
        q0 = case.q_suffix[0, 0].float()
        c = case.scale * math.log2(math.e)
        alpha = jump / (float((q0 * q0).sum()) * c)
        k = case.k_pool.float()
        t = 1400
        blk = int(case.block_tables[0, t // b])
        k[blk, t % b, 0] = alpha * q0
        case.k_pool = k.to(dtype)
        print(f"prefill {dtype} score jump {jump}", flush=True)
        run = gpu_prefill(case)
        ref = oracle_prefill(case)
        assert np.isfinite(np64(run.out)).all()
        assert report(f"jump {jump} {dtype}", np64(run.out), ref, dtype, TOL[dtype]) <= 1.0
