"""Softmax scales of any sign, and device-side lengths and block ids that are
out of range.

Scale: softmax(scale * q K^T) V is defined for any finite scale (page "KV
Cache에 대해 알아보자 (Feat. Attention)" §1 writes it with 1/sqrt(d_k)). The
matrix-core kernels take the row maximum before scaling, so a negative scale
is applied by negating q and a zero one by zeroing q; decode, suffix prefill
and the cascade must all match the oracle, whose closed form for scale 0 is
the mean of the visible values.

Bounds: lengths and block ids live in device memory and are clamped, never
trusted. With prefix/suffix/context lengths at the int32 extremes and block
ids far outside the pool, every call must finish and leave every byte outside
its output untouched (guard regions around the outputs; caches compared bit
for bit where the call does not write them)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import prefix_reuse_amd as pkv
import workloads
from _helpers import TOL, bits, gpu_decode, gpu_prefill, np64, oracle_decode, oracle_prefill, report

pytestmark = pytest.mark.gpu

I32_MAX, I32_MIN = 2 ** 31 - 1, -2 ** 31


@pytest.mark.parametrize("scale", [-0.0883883, 0.0, -1.5])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_prefill_any_scale(scale, dtype):
    print(f"prefill scale {scale} {dtype}", flush=True)
    case = workloads.make_prefill_case(710, [0, 37, 300], [45, 1, 70], 8, 2, 128, 16, dtype, scale=scale)
    run = gpu_prefill(case)
    ref = oracle_prefill(case)
    assert report(f"prefill scale {scale}", np64(run.out), ref, dtype, TOL[dtype]) <= 1.0


@pytest.mark.parametrize("scale", [-0.0883883, 0.0])
def test_decode_any_scale(scale):
    case = workloads.make_decode_case(711, [1, 40, 700, 33], 8, 2, 128, 16, torch.float16, scale=scale)
    run = gpu_decode(case)
    assert report(f"decode scale {scale}", np64(run.out), oracle_decode(case), torch.float16, TOL[torch.float16]) <= 1.0


@pytest.mark.parametrize("scale", [-0.0883883, 0.0])
def test_cascade_any_scale(scale):
    case = workloads.make_grouped_decode_case(712, [([300, 130, 257], 128), ([64], 0)], 8, 2, 128, 32,
                                              torch.bfloat16)
    case.scale = scale
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool)
    pkv.append(case.k_new.cuda(), case.v_new.cuda(), case.slot_mapping.cuda(), kc, vc)
    out = pkv.cascade_decode_attn(case.q.cuda(), kc, vc, case.block_tables.cuda(), case.context_lens.cuda(),
                                  case.meta["group_starts"].cuda(), case.meta["shared_lens"].cuda(), scale)
    torch.cuda.synchronize()
    assert report(f"cascade scale {scale}", np64(out), oracle_decode(case), torch.bfloat16,
                  TOL[torch.bfloat16]) <= 1.0


def test_zero_scale_gives_the_mean_of_visible_values():
    """Closed form, checked on the GPU result itself: with scale 0 every
    visible key has the same weight, so suffix row i of a request is the mean
    of the values at positions 0 .. P + i."""
    case = workloads.make_prefill_case(713, [20, 0], [5, 3], 4, 2, 64, 16, torch.float16, scale=0.0)
    run = gpu_prefill(case)
    ek, ev = oracle.append(np64(case.k_pool), np64(case.v_pool), np64(case.k_new), np64(case.v_new),
                           case.slot_mapping.numpy())
    got = np64(run.out)
    row = 0
    for r, (p, s) in enumerate(zip(case.prefix_lens.tolist(), case.suffix_lens.tolist())):
        vals = oracle.gather(ev, case.block_tables[r].numpy(), p + s)  # [n, H_kv, d]
        for i in range(s):
            mean = vals[:p + i + 1].mean(axis=0)  # [H_kv, d]
            for h in range(case.num_q_heads):
                assert np.abs(got[row, h] - mean[h // 2]).max() <= 2e-3
            row += 1


def _guarded(shape, dtype, fill):
    """A tensor with 4 KiB of guard bytes before and after it."""
    n = int(np.prod(shape))
    el = torch.tensor([], dtype=dtype).element_size()
    pad = 4096 // el
    buf = torch.empty(n + 2 * pad, dtype=dtype, device="cuda")
    buf.view(torch.uint8).fill_(fill)
    return buf, buf[pad:pad + n].view(shape), pad


def _guards_intact(buf, pad, fill):
    raw = buf.view(torch.uint8).cpu().numpy()
    el = buf.element_size()
    return bool((raw[:pad * el] == fill).all() and (raw[-pad * el:] == fill).all())


def test_prefill_out_of_range_device_values_stay_in_bounds():
    case = workloads.make_prefill_case(714, [40, 10, 5], [20, 20, 10], 8, 2, 128, 16, torch.bfloat16)
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool)
    k0, v0 = bits(kc), bits(vc)
    bt = case.block_tables.clone()
    bt[0, 1] = 10 ** 9
    bt[1, 0] = -5
    bt[2, :] = I32_MAX
    cases = [
        ([I32_MAX, -5, 1000], [I32_MAX, 20, I32_MIN]),
        ([I32_MIN, I32_MAX, I32_MAX], [10, I32_MAX, I32_MAX]),
        ([0, 0, 0], [I32_MIN, I32_MIN, 50]),
    ]
    for plens, slens in cases:
        print(f"prefix_lens {plens} suffix_lens {slens}", flush=True)
        buf, out, pad = _guarded(tuple(case.q_suffix.shape), torch.bfloat16, 0x5A)
        pkv.suffix_prefill_attn(case.q_suffix.cuda(), kc, vc, bt.cuda(), torch.tensor(plens, dtype=torch.int32).cuda(),
                                torch.tensor(slens, dtype=torch.int32).cuda(), case.scale, out=out)
        torch.cuda.synchronize()
        assert _guards_intact(buf, pad, 0x5A)
    assert np.array_equal(k0, bits(kc)) and np.array_equal(v0, bits(vc))


def test_decode_and_cascade_out_of_range_device_values_stay_in_bounds():
    case = workloads.make_decode_case(715, [40, 70, 33, 200], 8, 2, 128, 16, torch.float16)
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool)
    k0, v0 = bits(kc), bits(vc)
    bt = case.block_tables.clone()
    bt[0, 0] = 10 ** 9
    bt[1, :] = -1
    bt[3, 2] = I32_MAX
    for lens in ([I32_MAX, -7, 50, I32_MIN], [I32_MAX] * 4, [I32_MIN] * 4):
        print(f"context_lens {lens}", flush=True)
        cl = torch.tensor(lens, dtype=torch.int32).cuda()
        buf, out, pad = _guarded(tuple(case.q.shape), torch.float16, 0xA5)
        pkv.decode_attn(case.q.cuda(), kc, vc, bt.cuda(), cl, case.scale, out=out)
        torch.cuda.synchronize()
        assert _guards_intact(buf, pad, 0xA5)
        for gs, sl in (([0, I32_MAX], [I32_MAX] * 4), ([0, 2, -3, 4], [64, -64, I32_MIN, 16]), ([0, 4], [48] * 4)):
            buf, out, pad = _guarded(tuple(case.q.shape), torch.float16, 0xA5)
            pkv.cascade_decode_attn(case.q.cuda(), kc, vc, bt.cuda(), cl, torch.tensor(gs, dtype=torch.int32).cuda(),
                                    torch.tensor(sl, dtype=torch.int32).cuda(), case.scale, out=out)
            torch.cuda.synchronize()
            assert _guards_intact(buf, pad, 0xA5)
    assert np.array_equal(k0, bits(kc)) and np.array_equal(v0, bits(vc))
