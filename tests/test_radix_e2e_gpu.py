"""The radix tree driving the hot path end to end (page "PagedAttention과
RadixAttention으로 LLM KV 캐시 최적화" §03-§04; page "KV Cache 완전 정리",
RadixAttention): token IDs are matched against a radix tree whose pages are
the cache's blocks and whose values are KV slots; the matched prefix is read
in place, only the suffix is computed (pkv_append, then
pkv_suffix_prefill_attn), a decode step follows, and the request's whole
blocks are inserted into the tree afterwards. When the pool runs out, unlocked
leaves are evicted least recently used first and their blocks are handed to
new requests. Every output is compared with the oracle's full recompute over
K/V computed directly from the tokens, so a block that was reused while
holding the wrong tokens would show."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import prefix_reuse_amd as pkv
from _helpers import TOL, report
from prefix_reuse_amd.prefix_index import RadixTree

pytestmark = pytest.mark.gpu

H_Q, H_KV, D, B, NB = 8, 2, 128, 16, 36
VOCAB, MAX_POS, MAX_BLOCKS = 300, 1024, 64
DT = torch.bfloat16


def kv_tables(seed):
    g = torch.Generator().manual_seed(seed)
    emb = {w: torch.randn(VOCAB, H_KV, D, generator=g) for w in "kv"}
    pos = {w: 0.5 * torch.randn(MAX_POS, H_KV, D, generator=g) for w in "kv"}
    return emb, pos


def kv_rows(emb, pos, tokens, start, end):
    """K, V of positions start..end-1: a function of token and position only."""
    t = torch.tensor(tokens[start:end], dtype=torch.long)
    p = torch.arange(start, end)
    return tuple((emb[w][t] + pos[w][p]).to(DT) for w in "kv")


def dense_logical(emb, pos, tokens):
    n = len(tokens)
    nblk = -(-n // B)
    out = []
    for x in kv_rows(emb, pos, tokens, 0, n):
        pool = torch.zeros(nblk * B, H_KV, D, dtype=DT)
        pool[:n] = x
        out.append(pool.view(nblk, B, H_KV, D).double().numpy())
    return out[0], out[1], np.arange(nblk)[None, :]


class Engine:
    """Test-side serving loop: the radix tree holds (token -> slot); the free
    list holds blocks no stored prefix or running request uses."""

    def __init__(self, dev):
        self.dev = dev
        self.tree = RadixTree(page=B)
        self.free = list(range(NB))
        self.kc, self.vc = pkv.empty_caches(NB, B, H_KV, D, DT, dev)
        self.kc.view(torch.int16).fill_(0x7FC0)  # NaN wherever no token was written
        self.vc.view(torch.int16).fill_(0x7FC0)
        self.emb, self.pos = kv_tables(77)
        self.evicted_blocks = []

    def alloc(self, n_blocks):
        if len(self.free) < n_blocks:
            vals = self.tree.evict((n_blocks - len(self.free)) * B)
            blocks = sorted({v // B for v in vals})
            assert len(vals) == len(blocks) * B  # whole pages go
            self.evicted_blocks += blocks
            self.free += blocks
        assert len(self.free) >= n_blocks, "pool exhausted"
        out, self.free = self.free[:n_blocks], self.free[n_blocks:]
        return out

    def run(self, tokens, seed, decode_token=None):
        """Admit, prefill the suffix, optionally one decode step, insert, release.
        Returns (matched prefix length, block table)."""
        n = len(tokens)
        m, vals = self.tree.match_prefix(tokens)
        if m == n:  # every token cached: recompute the last page (one token must go through the model)
            m -= B
            vals = vals[:m]
        if m:
            self.tree.lock(tokens, m)
        own = [vals[j * B] // B for j in range(m // B)]
        for j, blk in enumerate(own):  # the matched slots are whole, in-order blocks
            assert vals[j * B:(j + 1) * B] == list(range(blk * B, blk * B + B))
        total = n + (1 if decode_token is not None else 0)
        table = own + self.alloc(-(-total // B) - len(own))
        slots = [table[t // B] * B + t % B for t in range(m, n)]
        k, v = kv_rows(self.emb, self.pos, tokens, m, n)
        dev = self.dev
        pkv.append(k.to(dev), v.to(dev), torch.tensor(slots, dtype=torch.int64, device=dev), self.kc, self.vc)
        bt = torch.zeros(1, MAX_BLOCKS, dtype=torch.int32)
        bt[0, :len(table)] = torch.tensor(table, dtype=torch.int32)
        q = torch.randn(n - m, H_Q, D, generator=torch.Generator().manual_seed(seed)).to(DT)
        out = pkv.suffix_prefill_attn(q.to(dev), self.kc, self.vc, bt.to(dev),
                                      torch.tensor([m], dtype=torch.int32, device=dev),
                                      torch.tensor([n - m], dtype=torch.int32, device=dev), D ** -0.5)
        torch.cuda.synchronize()
        lk, lv, ident = dense_logical(self.emb, self.pos, tokens)
        ref = oracle.suffix_prefill_attention(q.double().numpy(), lk, lv, ident, np.array([m]), np.array([n - m]),
                                              D ** -0.5)
        assert report(f"radix prefill (n={n}, reused {m})", out.double().cpu().numpy(), ref, DT, TOL[DT]) <= 1.0
        if decode_token is not None:  # one decode step: the new token joins the request's last block
            tokens = list(tokens) + [decode_token]
            n += 1
            kn, vn = kv_rows(self.emb, self.pos, tokens, n - 1, n)
            qd = torch.randn(1, H_Q, D, generator=torch.Generator().manual_seed(seed + 1)).to(DT)
            out = pkv.decode_step_attn(qd.to(dev), kn.to(dev), vn.to(dev), self.kc, self.vc, bt.to(dev),
                                       torch.tensor([n], dtype=torch.int32, device=dev), D ** -0.5)
            torch.cuda.synchronize()
            lk, lv, ident = dense_logical(self.emb, self.pos, tokens)
            ref = oracle.decode_attention(qd.double().numpy(), lk, lv, ident, np.array([n]), D ** -0.5)
            assert report(f"radix decode (n={n})", out.double().cpu().numpy(), ref, DT, TOL[DT]) <= 1.0
        # the request's whole blocks join the tree; a page already stored keeps
        # its old slots, so the block computed again for it goes back to the pool
        full = n - n % B
        existing = self.tree.insert(tokens[:full], [table[t // B] * B + t % B for t in range(full)])
        assert existing >= min(m, full)
        dup = table[m // B:existing // B]
        tail = table[full // B:]
        self.free += dup + tail
        if m:
            self.tree.unlock(tokens, m)
        return m, table


def test_radix_tree_drives_prefill_decode_and_eviction():
    eng = Engine(torch.device("cuda"))
    rng = np.random.default_rng(3)
    prompt = rng.integers(0, VOCAB, 160).tolist()                 # 10 blocks, shared by A, B, C, E
    a_tok = prompt + rng.integers(0, VOCAB, 50).tolist()          # 210 tokens
    b_tok = prompt + rng.integers(0, VOCAB, 70).tolist()          # 230
    m, table_a = eng.run(a_tok, 1)
    assert m == 0
    m, table_b = eng.run(b_tok, 2)
    assert m == 160 and table_b[:10] == table_a[:10]              # the prompt is read in place
    # C continues A's conversation: A's 13 whole blocks are reused; a decode step follows
    c_tok = a_tok[:208] + rng.integers(0, VOCAB, 30).tolist()
    m, table_c = eng.run(c_tok, 3, decode_token=int(rng.integers(0, VOCAB)))
    assert m == 208 and table_c[:13] == table_a[:13]
    assert eng.tree.total_tokens() == 160 + 48 + 16 + 64          # prompt, A's tail, C's block, B's tail
    # D shares nothing and needs 25 blocks: leaves go, least recently used first,
    # and the prompt (still an interior node with a stored prefix) survives
    d_tok = rng.integers(0, VOCAB, 400).tolist()
    free_before = len(eng.free)
    m, table_d = eng.run(d_tok, 4)
    assert m == 0 and free_before < 25
    assert set(eng.evicted_blocks) & set(table_d)                 # evicted blocks were handed out again
    assert not set(eng.evicted_blocks) & set(table_a[:10])        # the shared prompt was not evicted
    assert eng.tree.match_prefix(prompt)[0] == 160
    # E repeats A after its tail was evicted: only the prompt is reused, the
    # rest is recomputed into reused blocks, with the prompt locked meanwhile
    m, table_e = eng.run(a_tok, 5)
    assert m == 160 and table_e[:10] == table_a[:10]
    assert set(table_e[10:]) & set(eng.evicted_blocks)
