"""Decode parity: the HIP path against the oracle, element by element, on
seeded inputs (tolerance 2e-3 for f32/f16/bf16 caches, 2e-2 for fp8)."""
import math

import numpy as np
import pytest
import torch

import oracle
import prefix_reuse_amd as pkv
import workloads
from _helpers import (TOL, bits, fp8_inputs_from_pools, gpu_decode, gpu_fp8_decode, np64, oracle_decode,
                      oracle_fp8_caches, report)

pytestmark = pytest.mark.gpu

# lengths around block and chunk edges: 1, B-1, B, B+1, 31/32/33, a few chunks, a ragged tail
RAGGED = [1, 15, 16, 17, 31, 32, 33, 100, 257, 600, 1029]


def test_config1_tiny_decode_fp32():
    case = workloads.config1_tiny_decode()
    run = gpu_decode(case)
    ref = oracle_decode(case)
    err = report("config1", np64(run.out), ref)
    assert err <= TOL[torch.float32]
    print(f"  fp32 informational bound 1e-5: {'met' if err <= 1e-5 else 'not met'} ({err:.2e})")


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("block,dim", [(16, 64), (16, 128), (32, 64), (32, 128)])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (16, 1)])
def test_decode_ragged(dtype, block, dim, hq, hkv):
    print(f"decode ragged dtype={dtype} B={block} d={dim} hq={hq} hkv={hkv}", flush=True)
    case = workloads.make_decode_case(300 + dim + block + hq, RAGGED, hq, hkv, dim, block, dtype)
    run = gpu_decode(case)
    ref = oracle_decode(case)
    assert report("ragged", np64(run.out), ref, dtype, TOL[dtype]) <= 1.0


@pytest.mark.parametrize("q_dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("block,dim", [(16, 128), (32, 128), (32, 64)])
def test_decode_fp8_ragged(q_dtype, block, dim):
    print(f"decode fp8 q={q_dtype} B={block} d={dim}", flush=True)
    case = workloads.make_decode_case(400 + dim + block, RAGGED, 8, 2, dim, block, torch.float32)
    inp = fp8_inputs_from_pools(case, q_dtype)
    run = gpu_fp8_decode(case, inp, q_dtype)
    kc, vc = oracle_fp8_caches(case, inp)
    ref = oracle.decode_attention(np64(case.q.to(q_dtype)), kc, vc, case.block_tables.numpy(),
                                  case.context_lens.numpy(), case.scale, fp8=True,
                                  k_scale=inp.k_scale, v_scale=inp.v_scale)
    assert report("fp8", np64(run.out), ref, q_dtype, TOL["fp8"]) <= 1.0


def test_decode_large_group_needs_two_head_chunks():
    case = workloads.make_decode_case(77, [50, 300, 7], 40, 2, 64, 16, torch.float16)
    run = gpu_decode(case)
    assert report("G=20", np64(run.out), oracle_decode(case), torch.float16, TOL[torch.float16]) <= 1.0


def test_decode_zero_length_rows_are_zero():
    case = workloads.make_decode_case(78, [40, 1, 90], 8, 2, 128, 16, torch.bfloat16)
    case.context_lens[1] = 0
    case.slot_mapping[1] = -1
    run = gpu_decode(case)
    out = np64(run.out)
    assert np.array_equal(out[1], np.zeros_like(out[1]))
    ref = oracle_decode(case)
    assert report("zero-len", out, ref, torch.bfloat16, TOL[torch.bfloat16]) <= 1.0


@pytest.mark.parametrize("fill", [0x00, 0xFF, 0x7F, None])
def test_decode_any_workspace_contents(fill):
    """The workspace (partials of the sequences that several waves share, and
    the partition info the merge reads) needs no initial contents. Whatever
    bytes it holds (all-0, all-1 bits, 0x7F in every byte, seeded random
    bytes), three decode calls in a row, a smaller batch on the same
    workspace between the first two, and a decode step after them match the
    oracle, and the repeated calls agree bit for bit."""
    dtype = torch.float16
    lens = [3000, 1, 0, 2500, 700, 4100, 33]
    case = workloads.make_decode_case(79, lens, 32, 8, 128, 16, dtype)
    small = workloads.make_decode_case(80, [900, 0, 40], 32, 8, 128, 16, dtype)
    need = max(pkv.decode_workspace_bytes(c.num_seqs, 32, 8, 128, c.block_tables.shape[1], 16) for c in (case, small))
    if fill is None:
        ws = torch.from_numpy(np.random.default_rng(81).integers(0, 256, need, dtype=np.uint8)).cuda()
    else:
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
    print(f"workspace fill {fill}", flush=True)

    def on_gpu(c):
        kc, vc = pkv.caches_from_logical(c.k_pool, c.v_pool, "cuda")
        pkv.append(c.k_new.cuda(), c.v_new.cuda(), c.slot_mapping.cuda(), kc, vc)
        return c.q.cuda(), kc, vc, c.block_tables.cuda(), c.context_lens.cuda()

    q, kc, vc, bt, cl = on_gpu(case)
    sq, skc, svc, sbt, scl = on_gpu(small)
    ref, ref_small = oracle_decode(case), oracle_decode(small)
    outs = []
    for i in range(3):
        out = pkv.decode_attn(q, kc, vc, bt, cl, case.scale, workspace=ws)
        torch.cuda.synchronize()
        assert report(f"workspace {fill} call {i}", np64(out), ref, dtype, TOL[dtype]) <= 1.0
        outs.append(out.clone())
        if i == 0:
            out_small = pkv.decode_attn(sq, skc, svc, sbt, scl, small.scale, workspace=ws)
            torch.cuda.synchronize()
            assert report(f"workspace {fill} small batch", np64(out_small), ref_small, dtype, TOL[dtype]) <= 1.0
    for o in outs[1:]:
        assert np.array_equal(bits(o), bits(outs[0]))
    kc2, vc2 = pkv.caches_from_logical(case.k_pool, case.v_pool, "cuda")
    out_s = pkv.decode_step_attn(q, case.k_new.cuda(), case.v_new.cuda(), kc2, vc2, bt, cl, case.scale, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_s), bits(outs[0]))


def test_decode_strided_q_and_out():
    case = workloads.make_decode_case(79, [64, 200], 8, 2, 128, 32, torch.float16)
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool)
    pkv.append(case.k_new.cuda(), case.v_new.cuda(), case.slot_mapping.cuda(), kc, vc)
    big = torch.zeros(2, 8 * 3, 128, dtype=torch.float16, device="cuda")
    q = big[:, ::3]  # head stride 3 rows
    q.copy_(case.q.cuda())
    outbuf = torch.full((2, 16, 128), 7.0, dtype=torch.float16, device="cuda")
    out = outbuf[:, 8:]
    pkv.decode_attn(q, kc, vc, case.block_tables.cuda(), case.context_lens.cuda(), case.scale, out=out)
    torch.cuda.synchronize()
    assert torch.all(outbuf[:, :8] == 7.0)
    assert report("strided", np64(out), oracle_decode(case), torch.float16, TOL[torch.float16]) <= 1.0


@pytest.mark.slow
def test_config2_llama_decode_full():
    case = workloads.config2_llama_decode()
    run = gpu_decode(case)
    ref = oracle_decode(case)
    assert report("config2", np64(run.out), ref, torch.float16, TOL[torch.float16]) <= 1.0


@pytest.mark.slow
def test_config3_shared_prefix_decode_full():
    case = workloads.config3_shared_prefix_decode()
    run = gpu_decode(case)
    ref = oracle_decode(case)
    assert report("config3", np64(run.out), ref, torch.bfloat16, TOL[torch.bfloat16]) <= 1.0


def _fp8_decode_vs_oracle(case, q_dtype, name):
    inp = fp8_inputs_from_pools(case, q_dtype)
    run = gpu_fp8_decode(case, inp, q_dtype)
    kc, vc = oracle_fp8_caches(case, inp)
    ref = oracle.decode_attention(np64(case.q.to(q_dtype)), kc, vc, case.block_tables.numpy(),
                                  case.context_lens.numpy(), case.scale, fp8=True,
                                  k_scale=inp.k_scale, v_scale=inp.v_scale)
    return np64(run.out), ref


@pytest.mark.parametrize("waves", [2, 8, 24])
@pytest.mark.parametrize("q_dtype", [torch.bfloat16, torch.float16])
def test_decode_fp8_many_chunks_per_wave(waves, q_dtype, monkeypatch):
    """The long-context path over an fp8 cache: with PKV_DECODE_WAVES forcing
    few waves, every wave walks many 32-token chunks, crosses sequences and
    writes partials that the combine merges (2 KV heads: 1, 4 or 12 waves per
    head over ~430 chunks)."""
    print(f"fp8 decode, {waves} waves, q {q_dtype}", flush=True)
    case = workloads.make_decode_case(420, [6000, 129, 2500, 1000, 3, 0, 33, 4100], 8, 2, 128, 32, torch.float32)
    monkeypatch.setenv("PKV_DECODE_WAVES", str(waves))
    got, ref = _fp8_decode_vs_oracle(case, q_dtype, "fp8 waves")
    assert report(f"fp8 waves={waves}", got, ref, q_dtype, TOL["fp8"]) <= 1.0


def sharpen(case, q_mult=8.0, seed=0):
    """A long-context stress input whose outputs are of order 1: q scaled by
    q_mult (a sharp softmax over few keys) and V given a per-(KV head, dim)
    mean in [0.5, 2] with a random sign. With plain N(0,1) data an output over
    n keys has magnitude ~ 1/sqrt(n), so at long contexts an absolute gate
    could not tell a result from zeros."""
    g = torch.Generator().manual_seed(seed)
    h, d = case.num_kv_heads, case.head_dim
    mu = (0.5 + 1.5 * torch.rand(h, d, generator=g)) * torch.where(torch.rand(h, d, generator=g) < 0.5, -1.0, 1.0)
    case.q = (case.q.float() * q_mult).to(case.q.dtype)
    case.v_pool = (case.v_pool.float() + mu).to(case.v_pool.dtype)  # NaN poison stays NaN
    case.v_new = (case.v_new.float() + mu).to(case.v_new.dtype)
    return mu


@pytest.mark.parametrize("waves", [4, 0])
def test_decode_fp8_sharp_long_context(waves, monkeypatch):
    """fp8 cache, 20,000- and 9,000-token contexts with a sharpened q and V
    carrying a per-dimension mean, so that |out| = O(1) and the 2e-2 gate can
    fail; with 4 waves in all (2 per KV head) each wave walks ~450 chunks. An
    all-zero output must fail the same gate."""
    case = workloads.make_decode_case(421, [20000, 9000], 8, 2, 128, 32, torch.float32)
    sharpen(case, seed=421)
    if waves:
        monkeypatch.setenv("PKV_DECODE_WAVES", str(waves))
    got, ref = _fp8_decode_vs_oracle(case, torch.bfloat16, "fp8 sharp")
    assert np.abs(ref).max() >= 0.5
    assert report(f"fp8 sharp waves={waves}", got, ref, torch.bfloat16, TOL["fp8"]) <= 1.0
    assert report("zeros (must fail)", np.zeros_like(ref), ref, torch.bfloat16, TOL["fp8"], record=False) > 1.0
