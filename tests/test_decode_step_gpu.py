"""The one-call decode step (pkv_decode_step_attn) against pkv_append followed
by pkv_decode_attn: outputs and whole caches bit for bit, across cache dtypes
(fp8 included), block sizes, head dims, GQA groups (32: two head chunks),
lengths that end a chunk or a block exactly, length 1 and empty sequences, and
the full Llama-3-8B-shaped batch; one case also against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import prefix_reuse_amd as pkv
import workloads
from _helpers import TOL, bits, nan_fp8_caches, np64, oracle_decode, report

pytestmark = pytest.mark.gpu

LENS = [1, 31, 32, 33, 0, 64, 100, 257, 16, 17, 700]


def two_ways(case, kc0, vc0, q, k_new, v_new, k_scale=1.0, v_scale=1.0):
    """(out, k_cache, v_cache) of append + decode and of the one-call step."""
    dev = "cuda"
    bt, cl = case.block_tables.to(dev), case.context_lens.to(dev)
    ka, va = kc0.clone(), vc0.clone()
    pkv.append(k_new, v_new, case.slot_mapping.to(dev), ka, va, k_scale, v_scale)
    out_a = pkv.decode_attn(q, ka, va, bt, cl, case.scale, k_scale=k_scale, v_scale=v_scale)
    kb, vb = kc0.clone(), vc0.clone()
    out_b = pkv.decode_step_attn(q, k_new, v_new, kb, vb, bt, cl, case.scale, k_scale=k_scale, v_scale=v_scale)
    torch.cuda.synchronize()
    return (out_a, ka, va), (out_b, kb, vb)


def assert_same(a, b):
    for x, y, what in zip(a, b, ("out", "k_cache", "v_cache")):
        assert np.array_equal(bits(x), bits(y)), f"{what} differs"


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("d,b,hq,hkv", [(128, 16, 32, 8), (128, 32, 8, 2), (64, 16, 6, 2), (64, 32, 32, 1)])
def test_step_equals_append_then_decode(dtype, d, b, hq, hkv):
    case = workloads.make_decode_case(700 + d + b + hq, LENS, hq, hkv, d, b, dtype)
    print(f"{dtype} d={d} B={b} {hq}/{hkv}", flush=True)
    kc0, vc0 = pkv.caches_from_logical(case.k_pool, case.v_pool, "cuda")
    a, s = two_ways(case, kc0, vc0, case.q.cuda(), case.k_new.cuda(), case.v_new.cuda())
    assert_same(a, s)


@pytest.mark.parametrize("q_dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("b", [16, 32])
def test_step_fp8_cache(q_dtype, b):
    case = workloads.make_decode_case(760 + b, LENS, 16, 4, 128, b, torch.float32)
    pools = case.k_pool.float(), case.v_pool.float()
    live = ~torch.isnan(pools[0][:, :, 0, 0])
    idx = live.nonzero()
    slots = (idx[:, 0] * b + idx[:, 1]).cuda()
    rk = pools[0][idx[:, 0], idx[:, 1]].to(q_dtype)
    rv = pools[1][idx[:, 0], idx[:, 1]].to(q_dtype)
    k_new, v_new = case.k_new.to(q_dtype), case.v_new.to(q_dtype)
    ks = float(np.float32(max(rk.float().abs().max().item(), k_new.float().abs().max().item())) / np.float32(448))
    vs = float(np.float32(max(rv.float().abs().max().item(), v_new.float().abs().max().item())) / np.float32(448))
    kc0, vc0 = nan_fp8_caches(case)
    pkv.append(rk.cuda(), rv.cuda(), slots, kc0, vc0, ks, vs)
    a, s = two_ways(case, kc0, vc0, case.q.to(q_dtype).cuda(), k_new.cuda(), v_new.cuda(), ks, vs)
    assert_same(a, s)


def test_step_llama_batch_and_oracle():
    """The 64-sequence Llama-3-8B-shaped decode batch: bit for bit against
    append + decode, and every output against the oracle."""
    case = workloads.config2_llama_decode()
    kc0, vc0 = pkv.caches_from_logical(case.k_pool, case.v_pool, "cuda")
    a, s = two_ways(case, kc0, vc0, case.q.cuda(), case.k_new.cuda(), case.v_new.cuda())
    assert_same(a, s)
    ref = oracle_decode(case)
    assert report("step config2", np64(s[0]), ref, case.dtype, TOL[case.dtype]) <= 1.0


def test_step_rejects_bad_rows():
    case = workloads.make_decode_case(790, [5, 9], 8, 2, 64, 16, torch.float16)
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, "cuda")
    args = (case.q.cuda(), case.k_new.cuda(), case.v_new.cuda(), kc, vc, case.block_tables.cuda(),
            case.context_lens.cuda(), case.scale)
    with pytest.raises(pkv.PkvError):
        pkv.decode_step_attn(args[0], args[1].float(), *args[2:])  # dtype differs from the cache
    with pytest.raises(pkv.PkvError):
        pkv.decode_step_attn(args[0], args[1][:1], args[2][:1], *args[3:])  # one row for two sequences


@pytest.mark.parametrize("seed", range(6))
def test_step_random_batches(seed):
    """Seeded random batches (1-80 sequences of 0-3,000 tokens, random dtype,
    head dim, block size and GQA grouping up to 32): bit for bit against
    append + decode."""
    rng = np.random.default_rng(950 + seed)
    b = int(rng.choice([16, 32]))
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * int(rng.choice([1, 4, 8, 32]))
    dtype = [torch.float32, torch.float16, torch.bfloat16][int(rng.integers(3))]
    lens = [int(x) for x in rng.integers(0, 3001, int(rng.integers(1, 81)))]
    case = workloads.make_decode_case(950 + seed, lens, hq, hkv, d, b, dtype)
    print(f"seed {seed}: {len(lens)} seqs, {dtype} d={d} B={b} {hq}/{hkv}", flush=True)
    kc0, vc0 = pkv.caches_from_logical(case.k_pool, case.v_pool, "cuda")
    a, s = two_ways(case, kc0, vc0, case.q.cuda(), case.k_new.cuda(), case.v_new.cuda())
    assert_same(a, s)


@pytest.mark.parametrize("nseq", [64, 65, 130])
def test_step_batches_around_one_wave_of_sequences(nseq):
    """The step form over batches on both sides of 64 sequences (the first 64
    sequences' lengths are kept in lanes, the rest read from memory): bit for
    bit against append + decode, caches included."""
    rng = np.random.default_rng(970 + nseq)
    lens = [int(x) for x in rng.integers(0, 400, nseq)]
    lens[int(rng.integers(nseq))] = 0
    case = workloads.make_decode_case(970 + nseq, lens, 32, 8, 128, 16, torch.bfloat16)
    kc0, vc0 = pkv.caches_from_logical(case.k_pool, case.v_pool, "cuda")
    a, s = two_ways(case, kc0, vc0, case.q.cuda(), case.k_new.cuda(), case.v_new.cuda())
    assert_same(a, s)
