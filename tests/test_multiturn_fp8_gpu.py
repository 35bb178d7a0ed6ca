"""Multi-turn conversations over an fp8 e4m3 KV cache, end to end: each
turn's prefix is every earlier turn (page A §03: the longer the cached
prefix, the less prefill; page A §04: new KV joins the cache after each
request), matched by the C++ prefix cache; the new user message is appended
(quantized) and suffix-prefilled, then a few reply tokens are decoded one by
one. Every output is checked against the oracle's full recompute over the
quantized K/V of the whole conversation (tolerance 2e-2 for fp8 KV)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import prefix_reuse_amd as pkv
import workloads
from _helpers import TOL, report
from prefix_reuse_amd.prefix_index import PrefixCache

pytestmark = pytest.mark.gpu

H_Q, H_KV, D, B, NB = 16, 4, 128, 32, 1024
VOCAB, MAX_POS = 1000, 8192
K_SCALE, V_SCALE = 6.0 / 448, 6.0 / 448  # the rows stay within +-6


def tables(seed):
    g = torch.Generator().manual_seed(seed)
    emb = {w: torch.randn(VOCAB, H_KV, D, generator=g).clamp_(-3, 3) for w in "kv"}
    pos = {w: (0.5 * torch.randn(MAX_POS, H_KV, D, generator=g)).clamp_(-2, 2) for w in "kv"}
    return emb, pos


def rows(emb, pos, tokens, start, end):
    t = torch.tensor(tokens[start:end], dtype=torch.long)
    p = torch.arange(start, end)
    return tuple((emb[w][t] + pos[w][p]).float() for w in "kv")


def oracle_pools(emb, pos, tokens):
    """Quantized logical pools of the whole conversation (identity table)."""
    n = len(tokens)
    nblk = -(-n // B)
    k, v = rows(emb, pos, tokens, 0, n)
    out = []
    for x, sc in ((k, K_SCALE), (v, V_SCALE)):
        codes = np.full((nblk * B, H_KV, D), workloads.fp8_nan_code, np.uint8)
        codes[:n] = oracle.e4m3fn_quantize(x.numpy(), sc)
        out.append(codes.reshape(nblk, B, H_KV, D))
    return out[0], out[1], np.arange(nblk)[None, :]


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("q_dtype", [torch.bfloat16, torch.float16])
def test_multiturn_fp8_conversations(q_dtype, split):
    """split: each turn's suffix prefill through pkv_suffix_prefill_attn_split
    (one request at a time: the case it is for)."""
    dev = torch.device("cuda")
    emb, pos = tables(91)
    rng = np.random.default_rng(13)
    kc, vc = pkv.empty_caches(NB, B, H_KV, D, torch.float8_e4m3fn, dev)
    kc.view(torch.uint8).fill_(workloads.fp8_nan_code)
    vc.view(torch.uint8).fill_(workloads.fp8_nan_code)
    pc = PrefixCache(NB, B)
    scale = D ** -0.5
    system = rng.integers(0, VOCAB, 300).tolist()  # a system prompt every conversation starts with
    convs = [list(system) for _ in range(3)]
    reused = computed = 0
    for turn in range(4):
        for ci, conv in enumerate(convs):
            before = len(conv)
            conv += rng.integers(0, VOCAB, int(rng.integers(40, 160))).tolist()  # the new user message
            rid, table, p, slots = pc.admit(conv)
            n = len(conv)
            # every earlier turn is cached up to its last whole block; on the
            # first turn the later conversations reuse the system prompt's blocks
            want = (before // B) * B if turn > 0 or ci > 0 else 0
            assert p == want and len(slots) == n - p, (turn, ci, p, want)
            reused += p
            computed += n - p
            k, v = rows(emb, pos, conv, p, n)
            pkv.append(k.to(dev), v.to(dev), torch.tensor(slots, dtype=torch.int64, device=dev), kc, vc,
                       K_SCALE, V_SCALE)
            g = torch.Generator().manual_seed(100 * turn + ci)
            q = torch.randn(n - p, H_Q, D, generator=g).to(q_dtype)
            bt = torch.zeros(1, 256, dtype=torch.int32)
            bt[0, :len(table)] = torch.tensor(table, dtype=torch.int32)
            prefill = pkv.suffix_prefill_attn_split if split else pkv.suffix_prefill_attn
            out = prefill(q.to(dev), kc, vc, bt.to(dev), torch.tensor([p], dtype=torch.int32, device=dev),
                          torch.tensor([n - p], dtype=torch.int32, device=dev), scale,
                          k_scale=K_SCALE, v_scale=V_SCALE)
            torch.cuda.synchronize()
            lk, lv, ident = oracle_pools(emb, pos, conv)
            ref = oracle.suffix_prefill_attention(q.double().numpy(), lk, lv, ident, np.array([p]),
                                                  np.array([n - p]), scale, fp8=True, k_scale=K_SCALE,
                                                  v_scale=V_SCALE)
            print(f"turn {turn} conversation {ci}: {n} tokens, {p} reused", flush=True)
            assert report(f"t{turn} c{ci} prefill", out.double().cpu().numpy(), ref, q_dtype, TOL["fp8"]) <= 1.0
            # a short reply, decoded token by token
            for _ in range(3):
                tok = int(rng.integers(0, VOCAB))
                slot = pc.append(rid, tok)
                conv.append(tok)
                n = len(conv)
                k, v = rows(emb, pos, conv, n - 1, n)
                pkv.append(k.to(dev), v.to(dev), torch.tensor([slot], dtype=torch.int64, device=dev), kc, vc,
                           K_SCALE, V_SCALE)
            table = pc.block_table(rid)
            bt = torch.zeros(1, 256, dtype=torch.int32)
            bt[0, :len(table)] = torch.tensor(table, dtype=torch.int32)
            qd = torch.randn(1, H_Q, D, generator=g).to(q_dtype)
            out = pkv.decode_attn(qd.to(dev), kc, vc, bt.to(dev), torch.tensor([n], dtype=torch.int32, device=dev),
                                  scale, k_scale=K_SCALE, v_scale=V_SCALE)
            torch.cuda.synchronize()
            lk, lv, ident = oracle_pools(emb, pos, conv)
            ref = oracle.decode_attention(qd.double().numpy(), lk, lv, ident, np.array([n]), scale, fp8=True,
                                          k_scale=K_SCALE, v_scale=V_SCALE)
            assert report(f"t{turn} c{ci} decode", out.double().cpu().numpy(), ref, q_dtype, TOL["fp8"]) <= 1.0
            pc.commit(rid)
            pc.release(rid)
    assert reused > 2 * computed  # most of every later turn came from the cache
