"""pkv_decode_attn_noalloc, the decode entry point that allocates nothing
(its partial results live in the library's device-resident scratch), against
pkv_decode_attn with a caller workspace: the same kernels run, so the outputs
must agree bit for bit, on two calls in a row (the second smaller, so that it
reuses the scratch the first one left behind), and both must match the
oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import prefix_reuse_amd as pkv
import workloads
from _helpers import TOL, bits, np64, oracle_decode, report

pytestmark = pytest.mark.gpu


def _run_both(case):
    dev = torch.device("cuda")
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, dev)
    pkv.append(case.k_new.to(dev), case.v_new.to(dev), case.slot_mapping.to(dev), kc, vc)
    q, bt, cl = case.q.to(dev), case.block_tables.to(dev), case.context_lens.to(dev)
    ref = pkv.decode_attn(q, kc, vc, bt, cl, case.scale)
    out = torch.full_like(q, float("nan"))
    pkv.decode_attn_noalloc(q, kc, vc, bt, cl, case.scale, out=out)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_decode_matches_workspace_decode_on_two_calls():
    big = workloads.make_decode_case(730, [4000, 17, 2500, 1, 900, 3333, 64, 0, 1200], 32, 8, 128, 16,
                                     torch.float16)
    small = workloads.make_decode_case(731, [33, 500, 7], 8, 2, 64, 32, torch.bfloat16)
    for name, case in (("first call (9 sequences)", big), ("second call (3 sequences)", small)):
        print(f"noalloc decode, {name}", flush=True)
        ref, out = _run_both(case)
        assert np.array_equal(bits(ref), bits(out)), name
        assert report(f"noalloc {name}", np64(out), oracle_decode(case), case.dtype, TOL[case.dtype]) <= 1.0


def test_noalloc_decode_rejects_a_batch_beyond_its_scratch():
    case = workloads.make_decode_case(732, [20, 30], 32, 8, 128, 16, torch.float16)
    dev = torch.device("cuda")
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, dev)
    s = 4000  # (waves + 4000) * 32 heads * 130 floats > 32 MiB
    q = torch.zeros(s, 32, 128, dtype=torch.float16, device=dev)
    bt = torch.zeros(s, 4, dtype=torch.int32, device=dev)
    cl = torch.ones(s, dtype=torch.int32, device=dev)
    with pytest.raises(pkv.PkvError) as e:
        pkv.decode_attn_noalloc(q, kc, vc, bt, cl, case.scale, out=torch.empty_like(q))
    assert e.value.code == 6 and "scratch" in str(e.value)
