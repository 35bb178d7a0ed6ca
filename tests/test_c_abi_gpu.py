"""pkv_append + pkv_decode_attn called from plain C (tests/c_abi_consumer.c,
run as a child process with its own HIP context) on a ragged f16 batch that
this test writes to files; the output is checked against the oracle."""
import subprocess

import numpy as np
import pytest
import torch

import prefix_reuse_amd as pkv
import workloads
from _helpers import TOL, oracle_decode, report
from test_c_abi_host import consumer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("block,dim,hq,hkv", [(16, 128, 32, 8), (32, 64, 8, 2)])
def test_decode_from_c(tmp_path, block, dim, hq, hkv):
    lens = [1, 15, 16, 17, 100, 1029, 0, 3000]
    case = workloads.make_decode_case(90 + block + dim, lens, hq, hkv, dim, block, torch.float16)
    case.slot_mapping[lens.index(0)] = -1  # an empty sequence appends nothing
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, "cpu")
    files = {"q.bin": case.q, "k_cache.bin": kc, "v_cache.bin": vc, "k_new.bin": case.k_new,
             "v_new.bin": case.v_new, "block_tables.bin": case.block_tables.to(torch.int32),
             "context_lens.bin": case.context_lens.to(torch.int32),
             "slot_mapping.bin": case.slot_mapping.to(torch.int64)}
    for name, t in files.items():
        t.contiguous().view(torch.uint8).numpy().tofile(tmp_path / name)
    nb = kc.shape[0]
    (tmp_path / "meta.txt").write_text(f"{len(lens)} {hq} {hkv} {dim} {block} {nb} {case.block_tables.shape[1]} "
                                       f"{case.scale!r}\n")
    print(f"B={block} d={dim} {hq}/{hkv}", flush=True)
    res = subprocess.run([str(consumer()), "decode", str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "decode ok"
    out = np.fromfile(tmp_path / "out.bin", dtype=np.float16).astype(np.float64).reshape(len(lens), hq, dim)
    assert np.array_equal(out[lens.index(0)], np.zeros((hq, dim)))
    assert report(f"decode from C B={block} d={dim}", out, oracle_decode(case), torch.float16,
                  TOL[torch.float16]) <= 1.0
