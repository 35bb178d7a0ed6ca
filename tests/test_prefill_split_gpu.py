"""pkv_suffix_prefill_attn_split: the suffix prefill with each row tile's keys
split over several work-groups (chunks of the prefix, then the rest of the
keys causally) and the parts merged by log-sum-exp. Checked against the
oracle on every row, across cache dtypes, block sizes, head dims and
groupings, prefix lengths on and off the 64-key stage grid, empty suffixes,
forced part counts, any softmax scale, V values beyond f16 range (the bf16
cache's exact pass) and any workspace contents."""
import numpy as np
import pytest
import torch

import oracle
import prefix_reuse_amd as pkv
import workloads
from _helpers import (TOL, bits, fp8_inputs_from_pools, half_ulp, nan_fp8_caches, np64, oracle_fp8_caches,
                      oracle_prefill, report)

pytestmark = pytest.mark.gpu


def run_split(case, workspace=None):
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, "cuda")
    pkv.append(case.k_new.cuda(), case.v_new.cuda(), case.slot_mapping.cuda(), kc, vc)
    out = pkv.suffix_prefill_attn_split(case.q_suffix.cuda(), kc, vc, case.block_tables.cuda(),
                                        case.prefix_lens.cuda(), case.suffix_lens.cuda(), case.scale,
                                        workspace=workspace)
    torch.cuda.synchronize()
    return out


SHAPES = [
    # (prefix lens, suffix lens, H_q, H_kv, d, B, dtype)
    ([5000], [100], 32, 8, 128, 16, torch.bfloat16),       # one conversation's next turn
    ([4097], [37], 32, 8, 128, 32, torch.float16),         # prefix off the 64-key grid
    ([50], [20], 8, 2, 128, 16, torch.bfloat16),           # prefix shorter than one stage: only the last part
    ([0], [64], 8, 2, 64, 16, torch.float16),              # no prefix
    ([3000, 0, 1200], [9, 0, 1], 16, 4, 64, 32, torch.bfloat16),  # an empty suffix, a one-token suffix
    ([2500, 700], [40, 200], 32, 1, 128, 16, torch.float16),      # G = 32
]


@pytest.mark.parametrize("shape", range(len(SHAPES)))
def test_split_prefill_matches_oracle(shape):
    plen, slen, hq, hkv, d, b, dtype = SHAPES[shape]
    case = workloads.make_prefill_case(1200 + shape, plen, slen, hq, hkv, d, b, dtype)
    need = pkv.suffix_prefill_workspace_bytes(sum(slen), len(plen), hq, hkv, d, case.block_tables.shape[1], b)
    print(f"P={plen} S={slen} {hq}/{hkv} d={d} B={b} {dtype}: workspace {need} bytes", flush=True)
    out = np64(run_split(case))
    assert np.isfinite(out).all()
    assert report(f"split prefill {shape}", out, oracle_prefill(case), dtype, TOL[dtype]) <= 1.0


@pytest.mark.parametrize("parts", [2, 3, 5, 17])
def test_split_prefill_forced_part_counts(parts, monkeypatch):
    """Many requests (the merge finds each token's request among 70) and
    every part count, against the oracle and against the plain launch."""
    monkeypatch.setenv("PKV_PREFILL_SPLITS", str(parts))
    rng = np.random.default_rng(1300 + parts)
    plen = [int(x) for x in rng.integers(0, 1500, 70)]
    slen = [int(x) for x in rng.integers(0, 12, 70)]
    case = workloads.make_prefill_case(1300 + parts, plen, slen, 8, 2, 128, 16, torch.bfloat16)
    print(f"parts {parts}", flush=True)
    out = run_split(case)
    ref = oracle_prefill(case)
    assert report(f"split prefill, {parts} parts", np64(out), ref, torch.bfloat16, TOL[torch.bfloat16]) <= 1.0
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, "cuda")
    pkv.append(case.k_new.cuda(), case.v_new.cuda(), case.slot_mapping.cuda(), kc, vc)
    plain = pkv.suffix_prefill_attn(case.q_suffix.cuda(), kc, vc, case.block_tables.cuda(), case.prefix_lens.cuda(),
                                    case.suffix_lens.cuda(), case.scale)
    torch.cuda.synchronize()
    # two roundings to bf16 of results that differ only in summation order:
    # within 2e-3 plus one bf16 ulp of each other
    a, b = np64(out), np64(plain)
    assert (np.abs(a - b) <= 2e-3 + 2 * half_ulp(b, torch.bfloat16)).all()


@pytest.mark.parametrize("q_dtype", [torch.bfloat16, torch.float16])
def test_split_prefill_fp8_cache(q_dtype):
    case = workloads.make_prefill_case(1400, [6000, 900], [30, 7], 32, 8, 128, 32, torch.float32)
    inp = fp8_inputs_from_pools(case, q_dtype)
    kc, vc = nan_fp8_caches(case)
    pkv.append(inp.rows_k.cuda(), inp.rows_v.cuda(), inp.slots.cuda(), kc, vc, inp.k_scale, inp.v_scale)
    q = case.q_suffix.to(q_dtype)
    out = pkv.suffix_prefill_attn_split(q.cuda(), kc, vc, case.block_tables.cuda(), case.prefix_lens.cuda(),
                                        case.suffix_lens.cuda(), case.scale, k_scale=inp.k_scale,
                                        v_scale=inp.v_scale)
    torch.cuda.synchronize()
    ek, ev = oracle_fp8_caches(case, inp)
    ref = oracle.suffix_prefill_attention(np64(q), ek, ev, case.block_tables.numpy(), case.prefix_lens.numpy(),
                                          case.suffix_lens.numpy(), case.scale, fp8=True, k_scale=inp.k_scale,
                                          v_scale=inp.v_scale)
    assert report(f"split prefill fp8 q {q_dtype}", np64(out), ref, q_dtype, TOL["fp8"]) <= 1.0


@pytest.mark.parametrize("scale", [-0.3, 0.0])
def test_split_prefill_any_scale(scale):
    case = workloads.make_prefill_case(1500, [2000], [50], 8, 2, 128, 16, torch.float16)
    case.scale = scale
    out = np64(run_split(case))
    assert report(f"split prefill scale {scale}", out, oracle_prefill(case), torch.float16,
                  TOL[torch.float16]) <= 1.0


@pytest.mark.parametrize("big", [70000.0, -1.0e6])
def test_split_prefill_bf16_values_beyond_f16(big):
    """A V value beyond f16 range sends the parts that meet it to the bf16
    cache's exact pass; the merged rows stay exact."""
    case = workloads.make_prefill_case(1600, [3000], [40], 8, 2, 128, 16, torch.bfloat16)
    v = case.v_pool.float()
    blk = int(case.block_tables[0, 100])
    v[blk, 3, 1, 17] = big  # a prefix key in one chunk
    case.v_pool = v.to(torch.bfloat16)
    out = np64(run_split(case))
    ref = oracle_prefill(case)
    assert report(f"split prefill V {big}", out, ref, torch.bfloat16, TOL[torch.bfloat16]) <= 1.0


@pytest.mark.parametrize("fill", [0x00, 0xFF, 0x7F])
def test_split_prefill_any_workspace_contents(fill):
    case = workloads.make_prefill_case(1700, [4000, 100], [20, 60], 32, 8, 128, 16, torch.bfloat16)
    need = pkv.suffix_prefill_workspace_bytes(80, 2, 32, 8, 128, case.block_tables.shape[1], 16)
    assert need > 0
    ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
    ref = oracle_prefill(case)
    outs = [run_split(case, workspace=ws) for _ in range(2)]
    assert report(f"split prefill workspace 0x{fill:02x}", np64(outs[0]), ref, torch.bfloat16,
                  TOL[torch.bfloat16]) <= 1.0
    assert np.array_equal(bits(outs[0]), bits(outs[1]))


def test_split_prefill_next_turn_workload_every_row():
    """The timed next-turn workload (one request, 8,000 cached + 100 new
    tokens, 32/8 heads, d = 128, bf16, blocks of 16) in the launch
    configuration the benchmark times: the default part count and a
    workspace of the queried size, filled with NaN bytes first. Every row
    against the oracle, and the plain launch's outputs within one rounding."""
    case = workloads.next_turn_suffix_prefill()
    need = pkv.suffix_prefill_workspace_bytes(case.q_suffix.shape[0], 1, case.num_q_heads, case.num_kv_heads,
                                              case.head_dim, case.block_tables.shape[1], case.block_size)
    print(f"next turn: workspace {need} bytes", flush=True)
    assert need > 0  # the default takes a split here
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    out = np64(run_split(case, workspace=ws))
    assert np.isfinite(out).all()
    assert report("split prefill next turn", out, oracle_prefill(case), torch.bfloat16, TOL[torch.bfloat16]) <= 1.0
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, "cuda")
    pkv.append(case.k_new.cuda(), case.v_new.cuda(), case.slot_mapping.cuda(), kc, vc)
    plain = np64(pkv.suffix_prefill_attn(case.q_suffix.cuda(), kc, vc, case.block_tables.cuda(),
                                         case.prefix_lens.cuda(), case.suffix_lens.cuda(), case.scale))
    assert (np.abs(out - plain) <= 2e-3 + 2 * half_ulp(plain, torch.bfloat16)).all()
