"""Prefix reuse end to end: token IDs go through the C++ prefix cache
(include/pkv_prefix.h), which hands out block tables, prefix lengths and slot
mappings; the suffix K/V are appended and the suffix prefill (and a decode
step) run on the GPU through the C ABI. Every output is compared with the
oracle's full recompute over K/V computed directly from the tokens, so a
reused block that held the wrong tokens would show."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import prefix_reuse_amd as pkv
from _helpers import TOL, bits, report
from prefix_reuse_amd.prefix_index import PrefixCache

pytestmark = pytest.mark.gpu

H_Q, H_KV, D, B, NB = 8, 2, 128, 16, 512
VOCAB, MAX_POS = 500, 4096
DT = torch.bfloat16


def tables(seed):
    g = torch.Generator().manual_seed(seed)
    emb = {w: torch.randn(VOCAB, H_KV, D, generator=g) for w in "kv"}
    pos = {w: 0.5 * torch.randn(MAX_POS, H_KV, D, generator=g) for w in "kv"}
    return emb, pos


def kv_rows(emb, pos, tokens, start, end):
    """K and V of positions start..end-1: a function of the token and its
    position only, so equal prefixes have equal K/V (as in a model)."""
    t = torch.tensor(tokens[start:end], dtype=torch.long)
    p = torch.arange(start, end)
    return tuple((emb[w][t] + pos[w][p]).to(DT) for w in "kv")


def dense_logical(emb, pos, tokens):
    """Logical [nblk, B, H_kv, d] pools of every token computed directly, with
    the identity block table: the full-recompute input of the oracle."""
    n = len(tokens)
    nblk = -(-n // B)
    k, v = kv_rows(emb, pos, tokens, 0, n)
    out = []
    for x in (k, v):
        pool = torch.zeros(nblk * B, H_KV, D, dtype=DT)
        pool[:n] = x
        out.append(pool.view(nblk, B, H_KV, D).double().numpy())
    return out[0], out[1], np.arange(nblk)[None, :]


def test_prefix_cache_to_suffix_prefill_and_decode():
    dev = torch.device("cuda")
    emb, pos = tables(2024)
    rng = np.random.default_rng(7)
    prompt = rng.integers(0, VOCAB, 1000).tolist()  # one shared system prompt
    reqs = {
        "A": (prompt + rng.integers(0, VOCAB, 150).tolist(), 0),
        "B": (prompt + rng.integers(0, VOCAB, 90).tolist(), 0),
        "C": (None, 7),  # B's tokens under another tenant's salt
    }
    reqs["C"] = (reqs["B"][0], 7)
    kc, vc = pkv.empty_caches(NB, B, H_KV, D, DT, dev)
    kc.view(torch.int16).fill_(0x7FC0)  # NaN everywhere no token was written
    vc.view(torch.int16).fill_(0x7FC0)
    pc = PrefixCache(NB, B)
    scale = D ** -0.5
    max_blocks = 128
    rids, tabs, prefixes = {}, {}, {}
    snapshot = None
    for name in ("A", "B", "C"):
        tokens, salt = reqs[name]
        rid, table, p, slots = pc.admit(tokens, salt)
        n = len(tokens)
        print(f"request {name}: {n} tokens, prefix {p} reused, {n - p} computed, blocks {len(table)}", flush=True)
        k, v = kv_rows(emb, pos, tokens, p, n)
        if name == "B":
            snapshot = (bits(kc[tabs["A"][:62]]), bits(vc[tabs["A"][:62]]))
        pkv.append(k.to(dev), v.to(dev), torch.tensor(slots, dtype=torch.int64, device=dev), kc, vc)
        g = torch.Generator().manual_seed({"A": 1, "B": 2, "C": 3}[name])
        q = torch.randn(n - p, H_Q, D, generator=g).to(DT)
        bt = torch.zeros(1, max_blocks, dtype=torch.int32)
        bt[0, :len(table)] = torch.tensor(table, dtype=torch.int32)
        out = pkv.suffix_prefill_attn(q.to(dev), kc, vc, bt.to(dev), torch.tensor([p], dtype=torch.int32, device=dev),
                                      torch.tensor([n - p], dtype=torch.int32, device=dev), scale)
        torch.cuda.synchronize()
        lk, lv, ident = dense_logical(emb, pos, tokens)
        ref = oracle.suffix_prefill_attention(q.double().numpy(), lk, lv, ident, np.array([p]), np.array([n - p]),
                                              scale)
        assert report(f"e2e prefill {name}", out.double().cpu().numpy(), ref, DT, TOL[DT]) <= 1.0
        pc.commit(rid)
        rids[name], tabs[name], prefixes[name] = rid, table, p
    # reuse happened where the pages say it should, and only there
    assert prefixes["A"] == 0
    assert prefixes["B"] == (1000 // B) * B and tabs["B"][:62] == tabs["A"][:62]
    assert prefixes["C"] == 0 and not set(tabs["C"]) & set(tabs["A"])
    # B's append wrote none of the blocks it shares with A
    assert np.array_equal(snapshot[0], bits(kc[tabs["A"][:62]]))
    assert np.array_equal(snapshot[1], bits(vc[tabs["A"][:62]]))

    # a decode step of B: the cache hands out the new token's slot
    tokens_b = list(reqs["B"][0])
    new_tok = int(rng.integers(0, VOCAB))
    slot = pc.append(rids["B"], new_tok)
    tokens_b.append(new_tok)
    n = len(tokens_b)
    k, v = kv_rows(emb, pos, tokens_b, n - 1, n)
    pkv.append(k.to(dev), v.to(dev), torch.tensor([slot], dtype=torch.int64, device=dev), kc, vc)
    table = pc.block_table(rids["B"])
    bt = torch.zeros(1, max_blocks, dtype=torch.int32)
    bt[0, :len(table)] = torch.tensor(table, dtype=torch.int32)
    q = torch.randn(1, H_Q, D, generator=torch.Generator().manual_seed(99)).to(DT)
    out = pkv.decode_attn(q.to(dev), kc, vc, bt.to(dev), torch.tensor([n], dtype=torch.int32, device=dev), scale)
    torch.cuda.synchronize()
    lk, lv, ident = dense_logical(emb, pos, tokens_b)
    ref = oracle.decode_attention(q.double().numpy(), lk, lv, ident, np.array([n]), scale)
    assert report("e2e decode B", out.double().cpu().numpy(), ref, DT, TOL[DT]) <= 1.0

    # finished requests leave their published blocks matchable
    for name in ("A", "B", "C"):
        pc.release(rids[name])
    _, table_d, p_d, _ = pc.admit(prompt + [1, 2, 3])
    assert p_d == (1000 // B) * B and table_d[:62] == tabs["A"][:62]
