"""Device-side lengths past a block table's capacity are cut to that capacity,
and negative ones count as zero (the library's stated handling of lengths it
does not trust): a suffix row then sees every key of the table up to its own
position, and a decode row every key of the table.

Checked for the suffix prefill, plain and key-split, and for the decode,
against the oracle's decode over the cut key counts. Capacities of a whole
number of 64-key stages (8 blocks of 16) and not (9 blocks) are both covered.
The split's workspace starts filled with NaN bytes, so a partial that no
work-group wrote would show. That matters when a prefix fills a capacity of
whole stages: every key then lies in the prefix chunks and the last part has
none."""
import numpy as np
import pytest
import torch

import oracle
import prefix_reuse_amd as pkv
from _helpers import TOL, np64, report

pytestmark = pytest.mark.gpu

HQ, HKV, D, B = 8, 2, 128, 16
# (prefix length, suffix length): past the capacity, across it, inside it, negative
REQUESTS = [(10_000, 5), (None, 20), (40, 30), (-7, 4)]


def pools(seed, num_blocks, dtype):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(num_blocks, B, HKV, D, generator=g).to(dtype)
    v = torch.randn(num_blocks, B, HKV, D, generator=g).to(dtype)
    return k, v


def table_rows(seed, rows, max_blocks, num_blocks):
    rng = np.random.default_rng(seed)
    ids = rng.permutation(num_blocks)[: rows * max_blocks]
    return torch.tensor(ids.reshape(rows, max_blocks), dtype=torch.int32)


def oracle_rows(q, k_pool, v_pool, bt_rows, counts, scale):
    """The oracle's decode of each row over its own key count."""
    return oracle.decode_attention(np64(q), np64(k_pool), np64(v_pool), bt_rows.numpy(),
                                   np.asarray(counts, dtype=np.int64), scale)


@pytest.mark.parametrize("mode", ["plain", 2, 3, 5])
@pytest.mark.parametrize("max_blocks", [8, 9])
def test_prefill_lengths_past_capacity(max_blocks, mode, monkeypatch):
    cap = max_blocks * B
    plen = [cap - 3 if p is None else p for p, _ in REQUESTS]
    slen = [s for _, s in REQUESTS]
    num_blocks = 4 * max_blocks + 5
    k_pool, v_pool = pools(2100 + max_blocks, num_blocks, torch.bfloat16)
    bt = table_rows(2200 + max_blocks, len(REQUESTS), max_blocks, num_blocks)
    total = sum(slen)
    g = torch.Generator().manual_seed(2300 + max_blocks)
    q = torch.randn(total, HQ, D, generator=g).to(torch.bfloat16)
    scale = D ** -0.5
    kc, vc = pkv.caches_from_logical(k_pool, v_pool, "cuda")
    args = (q.cuda(), kc, vc, bt.cuda(), torch.tensor(plen, dtype=torch.int32).cuda(),
            torch.tensor(slen, dtype=torch.int32).cuda(), scale)
    print(f"capacity {cap}, mode {mode}", flush=True)
    if mode == "plain":
        out = pkv.suffix_prefill_attn(*args)
    else:
        monkeypatch.setenv("PKV_PREFILL_SPLITS", str(mode))
        need = pkv.suffix_prefill_workspace_bytes(total, len(REQUESTS), HQ, HKV, D, max_blocks, B)
        assert need > 0
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
        out = pkv.suffix_prefill_attn_split(*args, workspace=ws)
    torch.cuda.synchronize()
    # row i of request r sees keys 0 .. min(P_r, cap) + i, at most cap of them
    counts, rows_bt = [], []
    for r, (p, s) in enumerate(zip(plen, slen)):
        pc = min(max(p, 0), cap)
        for i in range(s):
            counts.append(min(pc + i + 1, cap))
            rows_bt.append(bt[r])
    ref = oracle_rows(q, k_pool, v_pool, torch.stack(rows_bt), counts, scale)
    got = np64(out)
    assert np.isfinite(got).all()
    assert report(f"prefill past capacity {cap} ({mode})", got, ref, torch.bfloat16, TOL[torch.bfloat16]) <= 1.0


@pytest.mark.parametrize("max_blocks", [8, 9])
def test_decode_lengths_past_capacity(max_blocks):
    cap = max_blocks * B
    ctx = [1_000_000, cap + 1, cap, cap - 1, 37, 0, -5]
    num_blocks = len(ctx) * max_blocks + 3
    k_pool, v_pool = pools(2400 + max_blocks, num_blocks, torch.float16)
    bt = table_rows(2500 + max_blocks, len(ctx), max_blocks, num_blocks)
    g = torch.Generator().manual_seed(2600 + max_blocks)
    q = torch.randn(len(ctx), HQ, D, generator=g).to(torch.float16)
    scale = D ** -0.5
    kc, vc = pkv.caches_from_logical(k_pool, v_pool, "cuda")
    out = pkv.decode_attn(q.cuda(), kc, vc, bt.cuda(), torch.tensor(ctx, dtype=torch.int32).cuda(), scale)
    torch.cuda.synchronize()
    ref = oracle_rows(q, k_pool, v_pool, bt, [min(max(c, 0), cap) for c in ctx], scale)
    got = np64(out)
    assert np.isfinite(got).all()
    assert report(f"decode past capacity {cap}", got, ref, torch.float16, TOL[torch.float16]) <= 1.0


@pytest.mark.parametrize("seed", range(12))
def test_split_prefill_random_lengths_around_capacity(seed, monkeypatch):
    """Random capacities (1-39 blocks of 16), 1-4 requests whose prefixes lie
    within 200 tokens of the capacity (some negative), 0-59 new tokens each,
    and a forced part count of 2-17: the key-split and plain prefill against
    the oracle's decode over the cut key counts."""
    rng = np.random.default_rng(9000 + seed)
    max_blocks = int(rng.integers(1, 40))
    cap = max_blocks * B
    r = int(rng.integers(1, 5))
    plen = [int(x) for x in rng.integers(max(cap - 200, -10), cap + 200, r)]
    slen = [int(x) for x in rng.integers(0, 60, r)]
    if sum(slen) == 0:
        slen[0] = 1
    parts = int(rng.integers(2, 18))
    print(f"seed {seed}: capacity {cap}, P={plen} S={slen}, {parts} parts", flush=True)
    monkeypatch.setenv("PKV_PREFILL_SPLITS", str(parts))
    num_blocks = r * max_blocks + 3
    k_pool, v_pool = pools(seed, num_blocks, torch.bfloat16)
    bt = table_rows(seed + 1, r, max_blocks, num_blocks)
    total = sum(slen)
    g = torch.Generator().manual_seed(seed + 2)
    q = torch.randn(total, HQ, D, generator=g).to(torch.bfloat16)
    scale = D ** -0.5
    kc, vc = pkv.caches_from_logical(k_pool, v_pool, "cuda")
    args = (q.cuda(), kc, vc, bt.cuda(), torch.tensor(plen, dtype=torch.int32).cuda(),
            torch.tensor(slen, dtype=torch.int32).cuda(), scale)
    need = pkv.suffix_prefill_workspace_bytes(total, r, HQ, HKV, D, max_blocks, B)
    ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    outs = {"split": pkv.suffix_prefill_attn_split(*args, workspace=ws), "plain": pkv.suffix_prefill_attn(*args)}
    torch.cuda.synchronize()
    counts, rows_bt = [], []
    for i_r, (p, s) in enumerate(zip(plen, slen)):
        pc = min(max(p, 0), cap)
        for i in range(s):
            counts.append(min(pc + i + 1, cap))
            rows_bt.append(bt[i_r])
    ref = oracle_rows(q, k_pool, v_pool, torch.stack(rows_bt), counts, scale)
    for name, o in outs.items():
        got = np64(o)
        assert np.isfinite(got).all(), name
        assert report(f"prefill around capacity {seed} ({name})", got, ref, torch.bfloat16,
                      TOL[torch.bfloat16]) <= 1.0
