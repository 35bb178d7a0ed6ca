"""pkv_append on the GPU: the whole cache must come back bit for bit equal to
the oracle's expected cache (so a stray write anywhere shows), for copies and
for fp8 quantization."""
import numpy as np
import pytest
import torch

import oracle
import prefix_reuse_amd as pkv
import workloads
from _helpers import bits, fp8_inputs_from_pools, nan_fp8_caches, np64, oracle_fp8_caches

pytestmark = pytest.mark.gpu

SHAPES = [(16, 64), (16, 128), (32, 64), (32, 128)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("block,dim", SHAPES)
@pytest.mark.parametrize("slot_dtype", [torch.int64, torch.int32])
def test_append_copy_bitexact(dtype, block, dim, slot_dtype):
    print(f"append copy dtype={dtype} B={block} d={dim} slots={slot_dtype}", flush=True)
    case = workloads.make_decode_case(100 + block + dim, [1, 15, 16, 17, 40, 3], 8, 2, dim, block, dtype,
                                      extra_free_blocks=3)
    # one extra row with a negative slot: it must not land anywhere
    k_new = torch.cat([case.k_new, case.k_new[:1] * 7])
    v_new = torch.cat([case.v_new, case.v_new[:1] * 7])
    slots = torch.cat([case.slot_mapping, torch.tensor([-1])]).to(slot_dtype)
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool)
    pkv.append(k_new.cuda(), v_new.cuda(), slots.cuda(), kc, vc)
    torch.cuda.synchronize()
    ek, ev = oracle.append(bits(case.k_pool), bits(case.v_pool), bits(k_new), bits(v_new), slots.numpy())
    assert np.array_equal(bits(pkv.k_logical(kc)), ek)
    assert np.array_equal(bits(pkv.v_logical(vc)), ev)


@pytest.mark.parametrize("row_dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("block,dim", SHAPES)
def test_append_fp8_quantize_bitexact(row_dtype, block, dim):
    print(f"append fp8 rows={row_dtype} B={block} d={dim}", flush=True)
    case = workloads.make_decode_case(200 + block + dim, [5, 33, 64, 1], 8, 2, dim, block, torch.float32,
                                      extra_free_blocks=2)
    inp = fp8_inputs_from_pools(case, row_dtype)
    # plant edge values: grid midpoints (ties), saturation, subnormals, signed zero
    grid = oracle.e4m3fn_decode(np.arange(127))
    mids = (grid[:-1] + grid[1:]) / 2
    special = np.concatenate([mids, -mids[::7], [463.9, 464.0, 470.0, 1e6, -1e6, 0.0, -0.0, 2.0 ** -10]])
    flat = inp.rows_k.reshape(-1).clone()
    sp = torch.tensor(special, dtype=torch.float32).to(row_dtype)
    flat[: sp.numel()] = sp  # with k_scale 1 the planted ties stay exact ties
    inp.rows_k = flat.view_as(inp.rows_k)
    inp.k_scale = 1.0
    kc, vc = nan_fp8_caches(case)
    pkv.append(inp.rows_k.cuda(), inp.rows_v.cuda(), inp.slots.cuda(), kc, vc, inp.k_scale, inp.v_scale)
    torch.cuda.synchronize()
    ek, ev = oracle_fp8_caches(case, inp)
    gk, gv = bits(pkv.k_logical(kc)), bits(pkv.v_logical(vc))
    print(f"  mismatching K codes: {int((gk != ek).sum())}, V codes: {int((gv != ev).sum())}", flush=True)
    assert np.array_equal(gk, ek)
    assert np.array_equal(gv, ev)


def test_append_empty_and_all_negative_slots_write_nothing():
    case = workloads.make_decode_case(7, [20, 9], 4, 2, 64, 16, torch.float16)
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool)
    before_k, before_v = bits(kc), bits(vc)
    pkv.append(case.k_new.cuda()[:0], case.v_new.cuda()[:0], case.slot_mapping.cuda()[:0], kc, vc)
    pkv.append(case.k_new.cuda(), case.v_new.cuda(), torch.full_like(case.slot_mapping, -5).cuda(), kc, vc)
    big = torch.full_like(case.slot_mapping, kc.shape[0] * 16)  # one past the last slot: skipped
    pkv.append(case.k_new.cuda(), case.v_new.cuda(), big.cuda(), kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc), before_k) and np.array_equal(bits(vc), before_v)
