"""Cascade decode (pkv_cascade_decode_attn) against the oracle: grouped
shared-prefix batches across dtypes, block sizes and head dims, members
shorter than their group's prefix, empty sequences, groups without a shared
prefix, an fp8 cache, and the full 256-sequence shared-prompt workload."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import prefix_reuse_amd as pkv
import workloads
from _helpers import (TOL, fp8_inputs_from_pools, gpu_decode, nan_fp8_caches, np64, oracle_decode,
                      oracle_fp8_caches, report)

pytestmark = pytest.mark.gpu

GROUPS = [
    [([40, 70, 33, 200], 32)],
    [([40, 70, 33], 32), ([5], 0), ([100, 90, 300], 64), ([17], 16)],
    [([20, 50], 48), ([0, 17], 16), ([16, 33], 16), ([1], 0)],
    [([500, 700, 640, 900, 513], 496)],
]


def run_cascade(case, device="cuda", k_scale=1.0, v_scale=1.0, caches=None):
    if caches is None:
        kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, device)
        pkv.append(case.k_new.to(device), case.v_new.to(device), case.slot_mapping.to(device), kc, vc)
    else:
        kc, vc = caches
    out = pkv.cascade_decode_attn(case.q.to(device), kc, vc, case.block_tables.to(device),
                                  case.context_lens.to(device), case.meta["group_starts"].to(device),
                                  case.meta["shared_lens"].to(device), case.scale, k_scale=k_scale,
                                  v_scale=v_scale)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("gi", range(len(GROUPS)))
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("d,b,hq,hkv", [(128, 16, 32, 8), (128, 32, 8, 2), (64, 16, 6, 2), (64, 32, 16, 1)])
def test_cascade_matches_oracle(gi, dtype, d, b, hq, hkv):
    groups = [(lens, (shared // b) * b) for lens, shared in GROUPS[gi]]
    case = workloads.make_grouped_decode_case(500 + gi, groups, hq, hkv, d, b, dtype)
    print(f"groups {gi} {dtype} d={d} B={b} {hq}/{hkv}", flush=True)
    got = np64(run_cascade(case))
    ref = oracle_decode(case)
    assert report(f"cascade g{gi}", got, ref, dtype, TOL[dtype]) <= 1.0


@pytest.mark.parametrize("q_dtype", [torch.bfloat16, torch.float16])
def test_cascade_fp8_cache(q_dtype):
    case = workloads.make_grouped_decode_case(610, [([300, 130, 257], 128), ([64], 0), ([90, 45], 32)], 8, 2, 128,
                                              32, torch.float32)
    case.q = case.q.to(q_dtype)
    inp = fp8_inputs_from_pools(case)
    kc, vc = nan_fp8_caches(case)
    pkv.append(inp.rows_k.cuda(), inp.rows_v.cuda(), inp.slots.cuda(), kc, vc, inp.k_scale, inp.v_scale)
    got = np64(run_cascade(case, k_scale=inp.k_scale, v_scale=inp.v_scale, caches=(kc, vc)))
    ek, ev = oracle_fp8_caches(case, inp)
    ref = oracle.decode_attention(np64(case.q), ek, ev, case.block_tables.numpy(), case.context_lens.numpy(),
                                  case.scale, fp8=True, k_scale=inp.k_scale, v_scale=inp.v_scale)
    assert report("cascade fp8", got, ref, q_dtype, TOL["fp8"]) <= 1.0


def test_cascade_workload_shared_prompt_full():
    """256 sequences on one 1,000-token system prompt (31 shared 32-token
    blocks): every output against the oracle, and close to the plain decode."""
    case = workloads.config3_shared_prefix_decode()
    case.meta["group_starts"] = torch.tensor([0, case.num_seqs], dtype=torch.int32)
    case.meta["shared_lens"] = torch.full((case.num_seqs,), case.shared_blocks * case.block_size, dtype=torch.int32)
    got = run_cascade(case)
    ref = oracle_decode(case)
    assert report("cascade config3", np64(got), ref, torch.bfloat16, TOL[torch.bfloat16]) <= 1.0
    plain = gpu_decode(case).out
    assert report("cascade vs decode", np64(got), np64(plain)) <= 2 * TOL[torch.bfloat16] + 8e-3


def test_cascade_is_deterministic_and_ignores_physical_order():
    groups = [([300, 257, 140], 128), ([33], 0)]
    case = workloads.make_grouped_decode_case(620, groups, 16, 4, 128, 16, torch.bfloat16)
    a = run_cascade(case)
    b = run_cascade(case)
    assert torch.equal(a, b)


def test_cascade_many_groups():
    """60 groups of 1-4 sequences: more shared-part work-groups than half the
    CUs, so the decode waves get the smallest share of the device."""
    rng = np.random.default_rng(630)
    groups = []
    for _ in range(60):
        shared = int(rng.integers(0, 12)) * 16
        lens = [int(x) for x in rng.integers(1, 300, int(rng.integers(1, 5)))]
        groups.append((lens, shared))
    case = workloads.make_grouped_decode_case(630, groups, 32, 8, 128, 16, torch.float16)
    got = np64(run_cascade(case))
    ref = oracle_decode(case)
    assert report("cascade 60 groups", got, ref, torch.float16, TOL[torch.float16]) <= 1.0


def test_cascade_more_groups_than_a_wave():
    """70 groups: the shared part's work-groups find their group among
    batches of 64."""
    rng = np.random.default_rng(660)
    groups = []
    for _ in range(70):
        shared = int(rng.integers(0, 6)) * 16
        lens = [int(x) for x in rng.integers(1, 150, int(rng.integers(1, 4)))]
        groups.append((lens, shared))
    case = workloads.make_grouped_decode_case(660, groups, 8, 2, 128, 16, torch.bfloat16)
    got = np64(run_cascade(case))
    ref = oracle_decode(case)
    assert report("cascade 70 groups", got, ref, torch.bfloat16, TOL[torch.bfloat16]) <= 1.0


def test_cascade_long_shared_short_private():
    """One group of 300 sequences on a 2,000-token prefix with 1-40 tokens of
    their own: the shared part dominates the launch. Checked on every sequence
    for 4 of the 32 heads."""
    rng = np.random.default_rng(640)
    lens = [2000 + int(x) for x in rng.integers(1, 41, 300)]
    case = workloads.make_grouped_decode_case(640, [(lens, 2000)], 32, 8, 128, 32, torch.bfloat16)
    got = np64(run_cascade(case))
    heads = [0, 9, 18, 31]
    ek, ev = oracle.append(np64(case.k_pool), np64(case.v_pool), np64(case.k_new), np64(case.v_new),
                           case.slot_mapping.numpy())
    ref = oracle.decode_attention(np64(case.q), ek, ev, case.block_tables.numpy(), case.context_lens.numpy(),
                                  case.scale, heads=heads)
    assert report("cascade long shared", got[:, heads], ref[:, heads], torch.bfloat16, TOL[torch.bfloat16]) <= 1.0


@pytest.mark.slow
@pytest.mark.parametrize("dtype,b", [(torch.bfloat16, 32), (torch.float16, 16)])
def test_cascade_long_shared_prefix_order_one_outputs(dtype, b):
    """Two groups on shared prefixes of 20,000 and 6,000 tokens (the shared
    part runs hundreds of stages), 24 and 9 sequences with 1-300 tokens of
    their own. q is scaled by 4 and every V row carries a per-(KV head, dim)
    mean in [0.5, 2] with a random sign, so that |out| is of order 1 and an
    all-zero output fails; every sequence is checked on 4 of the 32 heads."""
    rng = np.random.default_rng(670)
    groups = [([20000 + int(x) for x in rng.integers(1, 301, 24)], 20000),
              ([6000 + int(x) for x in rng.integers(1, 301, 9)], 6000)]
    case = workloads.make_grouped_decode_case(670 + b, groups, 32, 8, 128, b, dtype)
    g = torch.Generator().manual_seed(671)
    mean = (torch.rand(8, 128, generator=g) * 1.5 + 0.5) * (torch.randint(0, 2, (8, 128), generator=g) * 2 - 1)
    case.v_pool = (case.v_pool.float() + mean).to(dtype)  # unused slots stay NaN
    case.v_new = (case.v_new.float() + mean).to(dtype)
    case.q = (case.q.float() * 4).to(dtype)
    print(f"{dtype} B={b}", flush=True)
    got = np64(run_cascade(case))
    assert np.isfinite(got).all()
    heads = [0, 13, 22, 31]
    ek, ev = oracle.append(np64(case.k_pool), np64(case.v_pool), np64(case.k_new), np64(case.v_new),
                           case.slot_mapping.numpy())
    ref = oracle.decode_attention(np64(case.q), ek, ev, case.block_tables.numpy(), case.context_lens.numpy(),
                                  case.scale, heads=heads)
    assert np.abs(ref[:, heads]).max() > 0.5
    assert report(f"cascade long shared {dtype}", got[:, heads], ref[:, heads], dtype, TOL[dtype]) <= 1.0


@pytest.mark.parametrize("fill", [0x00, 0xFF, 0x7F])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_cascade_any_workspace_contents(fill, dtype):
    """The workspace needs no initial contents: whatever bytes it holds
    (here all-0, all-1 bits and 0x7F in every byte), the result matches the
    oracle, on the first call and bit for bit on a second one that finds
    the first call's partials and partition info there."""
    groups = [(lens, (shared // 16) * 16) for lens, shared in GROUPS[0]]
    case = workloads.make_grouped_decode_case(500, groups, 32, 8, 128, 16, dtype)
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, "cuda")
    pkv.append(case.k_new.cuda(), case.v_new.cuda(), case.slot_mapping.cuda(), kc, vc)
    need = pkv.cascade_workspace_bytes(case.num_seqs, 32, 8, 128)
    ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
    ref = oracle_decode(case)
    print(f"workspace fill 0x{fill:02x} {dtype}", flush=True)
    outs = []
    for _ in range(2):
        out = pkv.cascade_decode_attn(case.q.cuda(), kc, vc, case.block_tables.cuda(), case.context_lens.cuda(),
                                      case.meta["group_starts"].cuda(), case.meta["shared_lens"].cuda(), case.scale,
                                      workspace=ws)
        torch.cuda.synchronize()
        outs.append(out.clone())
        assert report(f"cascade workspace 0x{fill:02x}", np64(out), ref, dtype, TOL[dtype]) <= 1.0
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("seed", range(8))
def test_cascade_random_groupings(seed):
    """Seeded random batches: 1-12 groups of 1-9 sequences, shared prefixes of
    0-20 blocks, own lengths 0-400, random dtype, head dim, block size and GQA
    grouping."""
    rng = np.random.default_rng(900 + seed)
    b = int(rng.choice([16, 32]))
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    dtype = [torch.float16, torch.bfloat16][int(rng.integers(2))]
    groups = []
    for _ in range(int(rng.integers(1, 13))):
        shared = int(rng.integers(0, 21)) * b
        lens = [shared + int(x) for x in rng.integers(-shared // 2 if shared else 0, 401, int(rng.integers(1, 10)))]
        groups.append(([max(x, 0) for x in lens], shared))
    case = workloads.make_grouped_decode_case(900 + seed, groups, hq, hkv, d, b, dtype)
    print(f"seed {seed}: {len(groups)} groups, {case.num_seqs} seqs, {dtype} d={d} B={b} {hq}/{hkv}", flush=True)
    got = np64(run_cascade(case))
    ref = oracle_decode(case)
    assert report(f"cascade random {seed}", got, ref, dtype, TOL[dtype]) <= 1.0


@pytest.mark.parametrize("splits", [2, 3, 9, 16])
def test_cascade_shared_keys_in_several_chunks(splits, monkeypatch):
    """The shared keys cut into 2-16 chunks, each a work-group of its own whose
    partial joins the merge: 9 and 16 chunks take the merge past its first
    batch of eight partials. Members shorter than the prefix see fewer chunks."""
    monkeypatch.setenv("PKV_CASCADE_SPLITS", str(splits))
    groups = [([1100, 1300, 1050, 1500, 700, 40], 1024), ([60, 90], 32), ([300], 0)]
    case = workloads.make_grouped_decode_case(650, groups, 16, 4, 128, 32, torch.bfloat16)
    print(f"cascade with {splits} shared key chunks", flush=True)
    got = np64(run_cascade(case))
    ref = oracle_decode(case)
    assert report(f"cascade {splits} chunks", got, ref, torch.bfloat16, TOL[torch.bfloat16]) <= 1.0
