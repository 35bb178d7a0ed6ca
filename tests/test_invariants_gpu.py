"""Invariants the pages fix, checked on the GPU results themselves: scattered
physical blocks are read as one logical sequence (outputs must not change by a
single bit when blocks move or are aliased), runs are deterministic, unused
slots never leak into outputs, and any split of the context gives the same
result up to float32 rounding."""
import os

import numpy as np
import pytest
import torch

import prefix_reuse_amd as pkv
import workloads
from _helpers import TOL, bits, gpu_decode, gpu_prefill, np64, oracle_decode, report

pytestmark = pytest.mark.gpu


def _permute_case(case, seed):
    nb = case.k_pool.shape[0]
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(nb))
    k2 = torch.empty_like(case.k_pool)
    v2 = torch.empty_like(case.v_pool)
    k2[perm] = case.k_pool
    v2[perm] = case.v_pool
    bt = perm[case.block_tables.long()].to(torch.int32)
    slots = torch.where(case.slot_mapping >= 0,
                        perm[case.slot_mapping // case.block_size] * case.block_size + case.slot_mapping % case.block_size,
                        case.slot_mapping)
    return k2, v2, bt, slots


@pytest.mark.parametrize("dtype,block", [(torch.float16, 16), (torch.bfloat16, 32), (torch.float32, 16)])
def test_decode_bitwise_invariant_under_block_permutation(dtype, block):
    case = workloads.make_decode_case(900, [700, 33, 1500, 64], 32, 8, 128, block, dtype)
    base = gpu_decode(case).out
    k2, v2, bt, slots = _permute_case(case, 1)
    case.k_pool, case.v_pool, case.block_tables, case.slot_mapping = k2, v2, bt, slots
    again = gpu_decode(case).out
    assert np.array_equal(bits(base), bits(again))


def test_prefill_bitwise_invariant_under_block_permutation():
    case = workloads.make_prefill_case(901, [300, 17], [60, 100], 32, 8, 128, 16, torch.bfloat16)
    base = gpu_prefill(case).out
    k2, v2, bt, slots = _permute_case(case, 2)
    case.k_pool, case.v_pool, case.block_tables, case.slot_mapping = k2, v2, bt, slots
    again = gpu_prefill(case).out
    assert np.array_equal(bits(base), bits(again))


def test_decode_shared_prefix_bitwise_equals_private_copies():
    case = workloads.make_decode_case(902, [1100, 1040, 1500], 32, 8, 128, 32, torch.bfloat16,
                                      shared_prefix_tokens=1000)
    shared = gpu_decode(case).out
    # private copies of the 31 shared blocks for sequences 1 and 2
    nb = case.k_pool.shape[0]
    extra = []
    bt = case.block_tables.clone()
    for s in (1, 2):
        for j in range(31):
            extra.append(int(bt[s, j]))
            bt[s, j] = nb + len(extra) - 1
    idx = torch.tensor(extra)
    case.k_pool = torch.cat([case.k_pool, case.k_pool[idx]])
    case.v_pool = torch.cat([case.v_pool, case.v_pool[idx]])
    case.block_tables = bt
    private = gpu_decode(case).out
    assert np.array_equal(bits(shared), bits(private))


def test_decode_run_to_run_bitwise_deterministic():
    case = workloads.make_decode_case(903, [4000, 100, 2500, 17], 32, 8, 128, 16, torch.float16)
    a = gpu_decode(case).out
    b = gpu_decode(case).out
    assert np.array_equal(bits(a), bits(b))


@pytest.mark.parametrize("waves", [1, 8, 24, 200, 5000])
def test_decode_partition_invariance(waves, monkeypatch):
    """Any number of waves per KV head (1: one wave walks every sequence; 5000:
    most chunks get a wave of their own) gives the oracle's result within
    rounding, and the default partition's result within a few fp32 ulps."""
    case = workloads.make_decode_case(904, [4000, 129, 2500, 1000, 3, 0, 33], 32, 8, 128, 16, torch.float16)
    case.slot_mapping[5] = -1
    base = np64(gpu_decode(case).out)
    monkeypatch.setenv("PKV_DECODE_WAVES", str(waves))
    forced = np64(gpu_decode(case).out)
    monkeypatch.delenv("PKV_DECODE_WAVES")
    assert report(f"waves{waves}", forced, base, torch.float16, 1e-3) <= 1.0
    assert report(f"waves{waves}-oracle", forced, oracle_decode(case), torch.float16, TOL[torch.float16]) <= 1.0


def test_poisoned_slots_never_reach_outputs():
    # every pool slot that holds no live token is NaN; the block-table padding
    # points at an all-NaN block: outputs must all be finite
    case = workloads.make_decode_case(905, [1, 2, 17, 31, 45], 32, 8, 128, 32, torch.bfloat16,
                                      extra_free_blocks=5)
    assert torch.isnan(case.k_pool.float()).any()
    out = gpu_decode(case).out
    assert torch.isfinite(out.float()).all()
    pcase = workloads.make_prefill_case(906, [3, 0, 40], [5, 9, 1], 32, 8, 128, 16, torch.bfloat16,
                                        extra_free_blocks=4)
    assert torch.isfinite(gpu_prefill(pcase).out.float()).all()


@pytest.mark.parametrize("nseq", [63, 64, 65, 130])
@pytest.mark.parametrize("waves", [0, 7, 150])
def test_decode_batches_around_one_wave_of_sequences(nseq, waves, monkeypatch):
    """The decode's waves find their sequences through per-lane copies of the
    first 64 sequences' lengths and through memory for the rest: batches of 63
    to 130 ragged sequences (empty ones included), under several wave counts
    (0: the default), against the oracle; and the default partition's result
    within a few fp32 ulps of the one-wave-per-head walk."""
    rng = np.random.default_rng(960 + nseq)
    lens = [int(x) for x in rng.integers(0, 300, nseq)]
    for s in rng.choice(nseq, 4, replace=False):
        lens[int(s)] = 0
    case = workloads.make_decode_case(960 + nseq, lens, 32, 8, 128, 16, torch.float16)
    if waves:
        monkeypatch.setenv("PKV_DECODE_WAVES", str(waves))
    got = np64(gpu_decode(case).out)
    monkeypatch.setenv("PKV_DECODE_WAVES", "8")
    walk = np64(gpu_decode(case).out)
    monkeypatch.delenv("PKV_DECODE_WAVES")
    assert report(f"{nseq} seqs, waves {waves or 'default'}", got, oracle_decode(case), torch.float16,
                  TOL[torch.float16]) <= 1.0
    assert report(f"{nseq} seqs, waves {waves or 'default'} vs one wave per head", got, walk, torch.float16,
                  1e-3) <= 1.0


@pytest.mark.slow
@pytest.mark.parametrize("dtype,b", [(torch.float16, 16), (torch.bfloat16, 32)])
def test_decode_four_thousand_short_sequences(dtype, b):
    """4,096 sequences of 0-64 tokens (one in eight empty): the partition's
    first pass runs 64 batches of sequences, most waves find their first
    sequence in memory rather than in the lanes, and the merge runs 16,384
    work-groups. Decode against the oracle on every sequence and head; the
    step form bit for bit against append + decode, caches included."""
    rng = np.random.default_rng(970 + b)
    lens = [int(x) for x in rng.integers(1, 65, 4096)]
    for s in rng.choice(4096, 512, replace=False):
        lens[int(s)] = 0
    case = workloads.make_decode_case(970 + b, lens, 32, 8, 128, b, dtype)
    print(f"{dtype} B={b}", flush=True)
    run = gpu_decode(case)
    out = np64(run.out)
    assert np.array_equal(out[np.array(lens) == 0], np.zeros_like(out[np.array(lens) == 0]))
    assert report(f"4096 seqs {dtype}", out, oracle_decode(case), dtype, TOL[dtype]) <= 1.0
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, "cuda")
    step = pkv.decode_step_attn(case.q.cuda(), case.k_new.cuda(), case.v_new.cuda(), kc, vc,
                                case.block_tables.cuda(), case.context_lens.cuda(), case.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits(step), bits(run.out))
    assert np.array_equal(bits(kc), bits(run.k_cache)) and np.array_equal(bits(vc), bits(run.v_cache))
