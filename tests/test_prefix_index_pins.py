"""Pins of the prefix-index oracle (oracle/prefix_index.py) on what the pages
fix: their worked examples (tests/golden/prefix_examples.json), brute force on
small inputs, and invariants. CPU only."""
from __future__ import annotations

import json
import random
from pathlib import Path

import pytest

from oracle.prefix_index import ChainHashPrefixCache, OutOfBlocks, RadixTree

GOLDEN = json.loads((Path(__file__).parent / "golden" / "prefix_examples.json").read_text())


def chars(word):
    return [ord(c) for c in word]


# ---------------------------------------------------------------- radix tree
def test_firm_insertion():
    g = GOLDEN["firm_insert"]
    t = RadixTree(page=1)
    for w in g["stored"]:
        t.insert(chars(w), list(w))
    n, vals = t.match_prefix(chars(g["insert"]))
    assert n == g["shared_tokens"] and "".join(vals) == g["insert"][:n]
    before = t.total_tokens()
    assert t.insert(chars(g["insert"]), list(g["insert"])) == g["shared_tokens"]
    assert t.total_tokens() - before == g["new_tokens"]
    shape = {"".join(map(chr, k)) for k, _ in t.paths()}
    # 'fire' and 'firm' now hang off one shared 'fir' node, next to 'fat'
    assert {"f", "fat", "fir", "fire", "firm", "do", "dog", "dot", "pump"} == shape


def test_today_tomorrow():
    g = GOLDEN["today_tomorrow"]
    vocab = {w: i for i, w in enumerate(sorted(set(g["request_1"] + g["request_2"])))}
    r1 = [vocab[w] for w in g["request_1"]]
    r2 = [vocab[w] for w in g["request_2"]]
    t = RadixTree(page=1)
    n1, _ = t.match_prefix(r1)
    assert len(r1) - n1 == g["computed_1"]
    t.insert(r1, list(range(len(r1))))
    n2, vals = t.match_prefix(r2)
    assert len(r2) - n2 == g["computed_2"]
    assert vals == [0, 1, 2, 3]  # the KV of request I's first four tokens


def test_reuse_2000_1900_token_level_and_paged():
    g = GOLDEN["reuse_2000_1900"]
    rng = random.Random(5)
    prefix = [rng.randrange(32000) for _ in range(g["cached_tokens"])]
    req = prefix + [rng.randrange(32000) for _ in range(g["request_tokens"] - g["cached_tokens"])]
    t = RadixTree(page=1)
    t.insert(prefix, list(range(len(prefix))))
    n, _ = t.match_prefix(req)
    assert g["request_tokens"] - n == g["prefilled_tokens"]
    # with 16-token pages only whole cached pages match: 118 pages = 1,888 tokens
    tp = RadixTree(page=16)
    tp.insert(prefix, list(range(len(prefix))))
    assert tp.match_prefix(req)[0] == (g["cached_tokens"] // 16) * 16
    # the chain-hash cache matches the same whole blocks
    c = ChainHashPrefixCache(num_blocks=400, block_size=16)
    rid, _, p0, _ = c.admit(prefix)
    assert p0 == 0
    c.commit(rid)
    _, _, p1, slots = c.admit(req)
    assert p1 == (g["cached_tokens"] // 16) * 16 and len(slots) == g["request_tokens"] - p1


def test_chatbot_system_prompt_saving():
    g = GOLDEN["chatbot_system_prompt"]
    rng = random.Random(11)
    prompt = [rng.randrange(32000) for _ in range(g["prompt_tokens"])]
    t = RadixTree(page=1)
    prompt_computed = 0
    for _ in range(g["requests"]):
        q = prompt + [rng.randrange(32000) for _ in range(rng.randrange(5, 40))]
        n, _ = t.match_prefix(q)
        prompt_computed += max(0, g["prompt_tokens"] - n)
        t.insert(q, list(range(len(q))))
    assert prompt_computed == g["prompt_computations_with_reuse"] * g["prompt_tokens"]
    assert 1 - prompt_computed / g["prefill_without_reuse"] >= g["saving_at_least"]
    # block-granular reuse (B=16): the 62 full prompt blocks are shared; the
    # last 8 prompt tokens share a block with each question and are recomputed
    c = ChainHashPrefixCache(num_blocks=20000, block_size=16)
    prompt_computed = 0
    for _ in range(g["requests"]):
        q = prompt + [rng.randrange(32000) for _ in range(rng.randrange(5, 40))]
        rid, _, p, _ = c.admit(q)
        prompt_computed += max(0, g["prompt_tokens"] - p)
        c.commit(rid)
        c.release(rid)
    assert prompt_computed == g["prompt_tokens"] + (g["requests"] - 1) * (g["prompt_tokens"] % 16)
    assert 1 - prompt_computed / g["prefill_without_reuse"] >= g["saving_at_least"]


@pytest.mark.parametrize("page", [1, 2, 4])
def test_radix_match_is_brute_force_longest_prefix(page):
    rng = random.Random(100 + page)
    t = RadixTree(page=page)
    inserted = []
    for _ in range(60):
        base = rng.choice(inserted) if inserted and rng.random() < 0.7 else []
        cut = rng.randrange(len(base) + 1) if base else 0
        seq = list(base[:cut]) + [rng.randrange(4) for _ in range(rng.randrange(1, 12))]
        t.insert(seq, [("v", tuple(seq[:i + 1])) for i in range(len(seq))])
        inserted.append(seq)
    for _ in range(200):
        base = rng.choice(inserted)
        q = list(base[:rng.randrange(len(base) + 1)]) + [rng.randrange(4) for _ in range(rng.randrange(0, 6))]
        n, vals = t.match_prefix(q)
        brute = 0
        for s in inserted:
            m = 0
            while m + page <= min(len(s), len(q)) and s[m:m + page] == q[m:m + page]:
                m += page
            brute = max(brute, m)
        assert n == brute
        # every value is the one stored for exactly that prefix
        assert vals == [("v", tuple(q[:i + 1])) for i in range(n)]


def test_radix_eviction_is_leaf_first_lru_and_spares_locked_paths():
    t = RadixTree(page=1)
    shared = chars("sys:")
    a, b, c = shared + chars("alpha"), shared + chars("beta"), shared + chars("gamma")
    for s in (a, b, c):
        t.insert(s, s)
    t.match_prefix(a)          # a used most recently, then c is older than a
    t.match_prefix(c)
    t.lock(b, len(b))          # b is held by a running request
    freed = t.evict(5)
    # the least recently used unlocked leaf is 'alpha' (used before 'gamma')
    assert bytes(freed).decode() == "alpha"
    # the shared interior node is never removed while it has children
    freed = t.evict(100)
    assert bytes(freed).decode() == "gamma"
    assert {"".join(map(chr, k)) for k, _ in t.paths()} == {"sys:", "sys:beta"}
    t.unlock(b, len(b))
    assert bytes(t.evict(100)).decode() == "betasys:"  # now leaf 'beta', then 'sys:'
    assert t.total_tokens() == 0


def test_radix_lock_splits_and_counts():
    t = RadixTree(page=1)
    t.insert(chars("abcdef"), list("abcdef"))
    t.lock(chars("abcdef"), 3)
    assert [(("".join(map(chr, k))), l) for k, l in t.paths()] == [("abc", 1), ("abcdef", 0)]
    with pytest.raises(ValueError):
        t.unlock(chars("abcdef"), 6)


# ----------------------------------------------------------- chain-hash cache
class _Device:
    """What the pool's slots hold: the (salt, token, position) written there."""

    def __init__(self, num_blocks, B):
        self.slot = [None] * (num_blocks * B)

    def write(self, slots, salt, tokens, start):
        for i, s in enumerate(slots):
            self.slot[s] = (salt, tokens[start + i], start + i)


def test_chain_hash_reuse_reads_exactly_the_request_prefix():
    """Brute force on a random trace: every cached position a request reuses
    holds that request's own token (same tenant, same position), block
    counts are conserved and reference counts match the live requests."""
    rng = random.Random(7)
    B, NB = 4, 64
    c = ChainHashPrefixCache(NB, B)
    dev = _Device(NB, B)
    live = {}
    prompts = [[rng.randrange(6) for _ in range(rng.randrange(1, 20))] for _ in range(6)]
    for step in range(600):
        op = rng.random()
        if op < 0.45 or not live:
            base = rng.choice(prompts)
            toks = list(base[:rng.randrange(len(base) + 1)]) + [rng.randrange(6) for _ in range(rng.randrange(0, 9))]
            if not toks:
                toks = [1]
            salt = rng.choice([0, 0, 0, 7])
            try:
                rid, table, p, slots = c.admit(toks, salt)
            except OutOfBlocks:
                continue
            assert p % B == 0 and p < len(toks)
            assert len(table) == -(-len(toks) // B) and len(set(table)) == len(table)
            for t in range(p):
                assert dev.slot[table[t // B] * B + t % B] == (salt, toks[t], t)
            dev.write(slots, salt, toks, p)
            live[rid] = (table, toks, salt)
        elif op < 0.6:
            rid = rng.choice(list(live))
            table, toks, salt = live[rid]
            try:
                s = c.append(rid, rng.randrange(6))
            except OutOfBlocks:
                continue
            toks.append(c.requests[rid]["tokens"][-1])
            table[:] = c.requests[rid]["blocks"]
            dev.write([s], salt, toks, len(toks) - 1)
        elif op < 0.8:
            c.commit(rng.choice(list(live)))
        else:
            rid = rng.choice(list(live))
            c.release(rid)
            del live[rid]
        # conservation and reference counts
        in_use = set(b for tab, _, _ in live.values() for b in tab)
        free, evictable, cached = c.stats()
        assert free + evictable + len(in_use) == NB
        for b in range(NB):
            assert c.ref[b] == sum(tab.count(b) for tab, _, _ in live.values())
        # two live requests share a block only where their contents agree
        owner = {}
        for rid, (tab, toks, salt) in live.items():
            for i, b in enumerate(tab):
                if b in owner:
                    o = owner[b]
                    ot = live[o][1]
                    n = min(len(ot), len(toks), (i + 1) * B) - i * B
                    assert live[o][2] == salt and ot[i * B:i * B + n] == toks[i * B:i * B + n]
                owner[b] = rid


def test_chain_hash_salt_isolates_tenants():
    c = ChainHashPrefixCache(64, 4)
    toks = list(range(17))
    rid, _, _, _ = c.admit(toks, salt=1)
    c.commit(rid)
    assert c.admit(toks, salt=2)[2] == 0        # other tenant: no reuse
    assert c.admit(toks, salt=1)[2] == 16       # same tenant: 4 whole blocks
    assert c.admit(toks[:16], salt=1)[2] == 12  # all cached: the last block is recomputed


def test_chain_hash_eviction_order_and_capacity():
    c = ChainHashPrefixCache(4, 2)
    a, _, _, _ = c.admit([1, 2, 3, 4])       # blocks 0, 1
    c.commit(a)
    c.release(a)                               # tail first: 1 then 0 become evictable
    assert c.stats() == (2, 2, 2)
    b, tb, p, _ = c.admit([9, 9, 8, 8, 7, 7])  # needs 3: free 2, 3 then evicts block 1
    assert p == 0 and tb == [2, 3, 1]
    c.release(b)                               # never published: back to the free list, tail first
    assert c.stats() == (3, 1, 1)
    _, tc, p, _ = c.admit([1, 2, 5])           # block 0 ([1, 2]) is still cached
    assert p == 2 and tc == [0, 1]
    with pytest.raises(OutOfBlocks):
        c.admit([5, 5, 5, 5, 5])               # 3 blocks needed, 2 free, block 0 in use
    assert c.stats() == (2, 0, 1)
