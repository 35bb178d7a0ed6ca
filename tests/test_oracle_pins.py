"""Pins of the CPU oracle against what the pages and the mathematics fix.

CPU only. Each test ties an oracle function to something other than itself:
figures the pages print (tests/golden/page_figures.json), a library routine
(torch's fp8 codec, torch's scaled_dot_product_attention), closed forms, brute
force on tiny inputs, and invariants the pages state (scattered blocks read as
one sequence; reuse does not change the output; past K, V never change).
"""
import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = json.loads((Path(__file__).parent / "golden" / "page_figures.json").read_text())


# ---------------------------------------------------------------------------
# KV size closed form
# ---------------------------------------------------------------------------
def test_kv_bytes_per_token_matches_page_figure():
    g = GOLDEN["kv_bytes_per_token_llama3_8b_fp16"]
    got = oracle.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["dtype_bytes"])
    assert got == g["value_kib"] * 1024 == 131072


def test_kv_bytes_100k_context_exact_and_page_rounding():
    g = GOLDEN["kv_bytes_100k_context_gib_as_printed"]
    per_tok = oracle.kv_bytes_per_token(32, 8, 128, 2)
    total = per_tok * g["tokens"]
    assert total == 13_107_200_000
    # the page's 12.8 is the KiB count / 10^6, i.e. a decimal/binary unit mix
    assert total / 1024 / 1e6 == pytest.approx(g["value"])
    assert total / 2**30 == pytest.approx(12.207, abs=1e-3)


def test_kv_bytes_fp8_halves_fp16_and_long_context_total():
    fp16 = oracle.kv_bytes_per_token(32, 8, 128, 2)
    fp8 = oracle.kv_bytes_per_token(32, 8, 128, 1)
    assert fp8 / fp16 == GOLDEN["fp8_vs_fp16_memory_ratio"]["value"]
    assert fp8 * 8 * 100_000 == 52_428_800_000  # batch 8 x 100k tokens, 32 layers


def test_kv_bytes_llama2_70b_with_kv_heads():
    g = GOLDEN["llama2_70b_kv_per_token_kb"]
    per_tok = oracle.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["dtype_bytes"])
    assert per_tok == 327_680
    assert round(per_tok / 1000) == g["value_kb"]
    assert per_tok * 4096 / 1e9 == pytest.approx(g["per_request_4096_gb"], abs=0.05)


def test_kv_bytes_agree_with_allocated_tensor_sizes():
    # a Llama-3-8B-shaped cache for one token in every layer, in the layout the
    # workloads use, counted by torch
    b = 16
    per_layer = torch.empty(1, b, 8, 128, dtype=torch.float16, device="meta")
    bytes_per_token = 2 * 32 * per_layer.numel() * per_layer.element_size() // b
    assert bytes_per_token == oracle.kv_bytes_per_token(32, 8, 128, 2)
    c5 = workloads.config5_long_context_fp8(num_layers=32)
    assert c5.kv_read_bytes_per_layer() * 32 == oracle.kv_bytes_per_token(32, 8, 128, 1) * 8 * 100_000


def test_block_counts_of_page_examples():
    g = GOLDEN["sixty_token_request_blocks_b16"]
    assert math.ceil(g["tokens"] / g["block_size"]) == g["blocks"]
    case = workloads.config1_tiny_decode()
    # 17, 33, 60, 100 tokens take 2, 3, 4, 7 blocks: 16 of the 64-block pool
    used = {int(case.block_tables[s, j]) for s, n in enumerate(case.context_lens.tolist())
            for j in range(math.ceil(n / 16))}
    assert len(used) == 16
    c5 = workloads.config5_long_context_fp8(num_layers=1)
    assert c5.block_tables.shape == (8, 3125)


# ---------------------------------------------------------------------------
# fp8 e4m3fn codec
# ---------------------------------------------------------------------------
def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.nanmax(ours) == 448.0 and np.nanmin(np.abs(ours[ours != 0])) == 2.0 ** -9
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def _torch_quantize(x: np.ndarray, scale: float) -> np.ndarray:
    y = torch.from_numpy(np.asarray(x, np.float32)) / torch.tensor(scale, dtype=torch.float32)
    y = y.clamp(-448.0, 448.0)  # torch maps overflow to NaN; the rule here saturates
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_quantize_matches_torch_on_random_values():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(200_000) * s for s in (0.01, 1.0, 30.0, 300.0)]).astype(np.float32)
    for scale in (1.0, 0.37, 4.5 / 448):
        assert np.array_equal(oracle.e4m3fn_quantize(x, scale), _torch_quantize(x, scale))


def test_fp8_quantize_every_midpoint_and_grid_point():
    grid = oracle.e4m3fn_decode(np.arange(127))
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    vals = np.concatenate([grid.astype(np.float32), mids, -mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(1000))]).astype(np.float32)
    assert np.array_equal(oracle.e4m3fn_quantize(vals, 1.0), _torch_quantize(vals, 1.0))
    # ties go to the even code: midpoint of codes 1 and 2 -> 2, of 2 and 3 -> 2
    assert oracle.e4m3fn_quantize(np.float32(1.5 * 2 ** -9), 1.0) == 2
    assert oracle.e4m3fn_quantize(np.float32(2.5 * 2 ** -9), 1.0) == 2


def test_fp8_quantize_saturates_and_keeps_nan():
    q = oracle.e4m3fn_quantize(np.array([447.9, 448, 463.9, 464, 465, 1e9, np.inf, -1e9, np.nan], np.float32), 1.0)
    assert q.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F]


def test_fp8_quantize_divides_in_float32():
    # x / scale rounded to float32 before rounding to fp8: pick x where the
    # float64 quotient and the float32 quotient fall on opposite sides of a tie
    x = np.float32(1.0625) * np.float32(3.0)
    scale = np.float32(3.0)
    assert np.float32(x) / scale == np.float32(1.0625)
    assert oracle.e4m3fn_quantize(np.array([x]), float(scale))[0] == _torch_quantize(np.array([x]), float(scale))[0]


# ---------------------------------------------------------------------------
# append and gather
# ---------------------------------------------------------------------------
def _tiny_pool(seed=0, nb=6, b=4, h=2, d=3):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((nb, b, h, d)), rng.standard_normal((nb, b, h, d))


def test_append_round_trip_and_untouched_slots():
    kc, vc = _tiny_pool()
    rng = np.random.default_rng(1)
    k = rng.standard_normal((5, 2, 3))
    v = rng.standard_normal((5, 2, 3))
    slots = np.array([7, -1, 0, 23, 12])
    k2, v2 = oracle.append(kc, vc, k, v, slots)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(k2[s // 4, s % 4], k[i]) and np.array_equal(v2[s // 4, s % 4], v[i])
    written = {int(s) for s in slots if s >= 0}
    for s in range(24):
        if s not in written:
            assert np.array_equal(k2[s // 4, s % 4], kc[s // 4, s % 4])
            assert np.array_equal(v2[s // 4, s % 4], vc[s // 4, s % 4])
    # inputs untouched (write-once: the caller's arrays are not modified)
    assert not np.shares_memory(k2, kc)


def test_append_fp8_stores_quantized_codes():
    kc = np.zeros((2, 4, 1, 8), np.uint8)
    vc = np.zeros((2, 4, 1, 8), np.uint8)
    k = np.linspace(-3, 3, 8, dtype=np.float32).reshape(1, 1, 8)
    v = -k
    k2, v2 = oracle.append(kc, vc, k, v, np.array([5]), fp8=True, k_scale=0.5, v_scale=2.0)
    assert np.array_equal(k2[1, 1, 0], _torch_quantize(k[0, 0], 0.5))
    assert np.array_equal(v2[1, 1, 0], _torch_quantize(v[0, 0], 2.0))


def test_gather_brute_force():
    kc, _ = _tiny_pool(nb=8, b=4)
    table = np.array([5, 2, 7, 0])
    g = oracle.gather(kc, table, 13)
    for t in range(13):
        assert np.array_equal(g[t], kc[table[t // 4], t % 4])


# ---------------------------------------------------------------------------
# decode attention
# ---------------------------------------------------------------------------
def _scalar_decode(q, kc, vc, table, n, scale, group):
    """Independent brute force: pure Python loops with math.exp."""
    b = kc.shape[1]
    hq, d = q.shape
    out = [[0.0] * d for _ in range(hq)]
    for h in range(hq):
        g = h // group
        scores = []
        for t in range(n):
            row = kc[table[t // b], t % b, g]
            scores.append(scale * sum(float(q[h, i]) * float(row[i]) for i in range(d)))
        mx = max(scores)
        w = [math.exp(s - mx) for s in scores]
        z = sum(w)
        for i in range(d):
            out[h][i] = sum(w[t] * float(vc[table[t // b], t % b, g, i]) for t in range(n)) / z
    return np.array(out)


def _np(t):
    return t.double().numpy()


def test_decode_matches_scalar_brute_force_on_config1():
    case = workloads.config1_tiny_decode()
    kc, vc = oracle.append(_np(case.k_pool), _np(case.v_pool), _np(case.k_new), _np(case.v_new),
                           case.slot_mapping.numpy())
    bt = case.block_tables.numpy()
    lens = case.context_lens.numpy()
    out = oracle.decode_attention(_np(case.q), kc, vc, bt, lens, case.scale)
    for s in range(case.num_seqs):
        ref = _scalar_decode(_np(case.q)[s], kc, vc, bt[s], int(lens[s]), case.scale, 2)
        np.testing.assert_allclose(out[s], ref, rtol=1e-12, atol=1e-12)


def test_decode_closed_form_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(3)
    nb, b, h, d, n = 9, 16, 2, 8, 70
    kc = np.repeat(rng.standard_normal((1, 1, h, d)), nb * b, axis=0).reshape(nb, b, h, d)
    vc = rng.standard_normal((nb, b, h, d))
    table = rng.permutation(nb)
    q = rng.standard_normal((1, 4, d))
    out = oracle.decode_attention(q, kc, vc, table[None], np.array([n]), 0.3)
    vals = vc[table[np.arange(n) // b], np.arange(n) % b]  # [n, h, d]
    for hh in range(4):
        np.testing.assert_allclose(out[0, hh], vals[:, hh // 2].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_decode_closed_forms_constant_v_single_key_and_sharp_softmax():
    rng = np.random.default_rng(4)
    nb, b, h, d = 4, 16, 1, 8
    kc = rng.standard_normal((nb, b, h, d))
    vc = np.broadcast_to(np.arange(d, dtype=np.float64), (nb, b, h, d)).copy()
    q = rng.standard_normal((1, 1, d))
    out = oracle.decode_attention(q, kc, vc, np.array([[2, 0, 3, 1]]), np.array([50]), 1.0)
    np.testing.assert_allclose(out[0, 0], np.arange(d), rtol=1e-12)
    vc = rng.standard_normal((nb, b, h, d))
    out = oracle.decode_attention(q, kc, vc, np.array([[3, 1, 0, 2]]), np.array([1]), 1.0)
    np.testing.assert_array_equal(out[0, 0], vc[3, 0, 0])
    # one key aligned with q and a huge scale: the output is that key's value
    kc2 = kc.copy()
    kc2[1, 5, 0] = q[0, 0] * 3
    out = oracle.decode_attention(q, kc2, vc, np.array([[3, 1, 0, 2]]), np.array([40]), 1e3)
    np.testing.assert_allclose(out[0, 0], vc[1, 5, 0], rtol=1e-9)


def test_decode_zero_length_gives_zero_row():
    kc, vc = _tiny_pool()
    out = oracle.decode_attention(np.ones((1, 2, 3)), kc, vc, np.array([[0, 1]]), np.array([0]), 1.0)
    assert np.array_equal(out, np.zeros((1, 2, 3)))


def test_decode_invariant_under_physical_block_permutation():
    case = workloads.make_decode_case(11, [37, 64, 5], 8, 2, 16, 16, torch.float32)
    kc, vc = _np(case.k_pool), _np(case.v_pool)
    bt, lens = case.block_tables.numpy(), case.context_lens.numpy() - 1
    q = _np(case.q)
    base = oracle.decode_attention(q, kc, vc, bt, lens, case.scale)
    perm = np.random.default_rng(5).permutation(kc.shape[0])  # new position of each block
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    out = oracle.decode_attention(q, kc2, vc2, perm[bt], lens, case.scale)
    assert np.array_equal(out, base)


def test_decode_shared_prefix_blocks_equal_private_copies():
    case = workloads.make_decode_case(12, [40, 70, 33], 4, 2, 16, 16, torch.float32,
                                      shared_prefix_tokens=35)
    kc, vc = _np(case.k_pool), _np(case.v_pool)
    bt = case.block_tables.numpy().copy()
    lens = case.context_lens.numpy() - 1
    assert len({tuple(bt[s, :2]) for s in range(3)}) == 1  # two aliased blocks
    base = oracle.decode_attention(_np(case.q), kc, vc, bt, lens, case.scale)
    # give every sequence its own copy of the shared blocks
    extra_k, extra_v = [], []
    nb = kc.shape[0]
    for s in range(1, 3):
        for j in range(2):
            extra_k.append(kc[bt[s, j]])
            extra_v.append(vc[bt[s, j]])
            bt[s, j] = nb + len(extra_k) - 1
    kc2 = np.concatenate([kc, np.stack(extra_k)])
    vc2 = np.concatenate([vc, np.stack(extra_v)])
    out = oracle.decode_attention(_np(case.q), kc2, vc2, bt, lens, case.scale)
    assert np.array_equal(out, base)


def test_decode_gqa_grouping_is_consecutive():
    # With H_q=4, H_kv=2, heads 0,1 read KV head 0 and heads 2,3 read KV head 1:
    # make the two KV heads' values constant and different.
    rng = np.random.default_rng(9)
    kc = rng.standard_normal((2, 16, 2, 4))
    vc = np.zeros((2, 16, 2, 4))
    vc[:, :, 0] = 1.0
    vc[:, :, 1] = 2.0
    out = oracle.decode_attention(rng.standard_normal((1, 4, 4)), kc, vc, np.array([[1, 0]]),
                                  np.array([20]), 0.5)
    np.testing.assert_allclose(out[0, :, 0], [1, 1, 2, 2])


# ---------------------------------------------------------------------------
# suffix prefill
# ---------------------------------------------------------------------------
def test_prefill_without_prefix_matches_library_causal_attention():
    case = workloads.make_prefill_case(21, [0, 0], [37, 20], 4, 2, 16, 16, torch.float32)
    kc, vc = oracle.append(_np(case.k_pool), _np(case.v_pool), _np(case.k_new), _np(case.v_new),
                           case.slot_mapping.numpy())
    out = oracle.suffix_prefill_attention(_np(case.q_suffix), kc, vc, case.block_tables.numpy(),
                                          case.prefix_lens.numpy(), case.suffix_lens.numpy(), case.scale)
    base = 0
    for r, s in enumerate(case.suffix_lens.tolist()):
        q = torch.from_numpy(_np(case.q_suffix)[base:base + s]).permute(1, 0, 2)  # [H, S, d]
        k = torch.from_numpy(_np(case.k_new)[base:base + s]).permute(1, 0, 2)
        v = torch.from_numpy(_np(case.v_new)[base:base + s]).permute(1, 0, 2)
        k = k.repeat_interleave(2, dim=0)
        v = v.repeat_interleave(2, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True,
                                                               scale=case.scale)[0].permute(1, 0, 2)
        np.testing.assert_allclose(out[base:base + s], ref.numpy(), rtol=1e-10, atol=1e-12)
        base += s


def _full_vs_suffix(prefix, suffix, d=16, hq=2, hkv=1, seed=31):
    """Run the same request as P=prefix,S=suffix and as P=0,S=prefix+suffix."""
    n = prefix + suffix
    full = workloads.make_prefill_case(seed, [0], [n], hq, hkv, d, 16, torch.float32)
    kc, vc = oracle.append(_np(full.k_pool), _np(full.v_pool), _np(full.k_new), _np(full.v_new),
                           full.slot_mapping.numpy())
    q = _np(full.q_suffix)
    ref = oracle.suffix_prefill_attention(q, kc, vc, full.block_tables.numpy(), np.array([0]),
                                          np.array([n]), full.scale)
    got = oracle.suffix_prefill_attention(q[prefix:], kc, vc, full.block_tables.numpy(),
                                          np.array([prefix]), np.array([suffix]), full.scale)
    return ref[prefix:], got


def test_prefix_reuse_equals_full_recompute_2000_1900():
    g = GOLDEN["prefix_reuse_2000_1900"]
    ref, got = _full_vs_suffix(g["cached_tokens"], g["prefilled_tokens"])
    assert got.shape[0] == g["request_tokens"] - g["cached_tokens"]
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_prefix_reuse_what_day_is_it_example():
    g = GOLDEN["what_day_is_it"]
    ref, got = _full_vs_suffix(g["shared_prefix"], g["second_request_computed"], d=8)
    assert got.shape[0] == 1
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)


def test_prefill_last_row_equals_decode():
    # the last suffix row sees exactly the whole context, like a decode query
    case = workloads.make_prefill_case(41, [23, 9], [6, 17], 4, 2, 16, 16, torch.float32)
    kc, vc = oracle.append(_np(case.k_pool), _np(case.v_pool), _np(case.k_new), _np(case.v_new),
                           case.slot_mapping.numpy())
    out = oracle.suffix_prefill_attention(_np(case.q_suffix), kc, vc, case.block_tables.numpy(),
                                          case.prefix_lens.numpy(), case.suffix_lens.numpy(), case.scale)
    last_rows = np.cumsum(case.suffix_lens.numpy()) - 1
    q = _np(case.q_suffix)[last_rows]
    dec = oracle.decode_attention(q, kc, vc, case.block_tables.numpy(),
                                  (case.prefix_lens + case.suffix_lens).numpy(), case.scale)
    np.testing.assert_allclose(out[last_rows], dec, rtol=0, atol=1e-14)


def test_chatbot_prefill_saving_arithmetic():
    g = GOLDEN["chatbot_shared_system_prompt"]
    without = g["requests"] * g["prompt_tokens"]
    with_reuse = g["prompt_tokens"]  # the prompt once, reused 999 times
    assert without == g["prefill_tokens_without_reuse"]
    assert round(100 * (1 - with_reuse / without)) >= g["saving_percent"]


# ---------------------------------------------------------------- grouped (shared-prefix) batches
# The cascade decode is checked on the GPU against decode_attention on grouped
# batches; these pins fix what those batches must be: members of a group read
# their shared prefix through the same physical blocks (page A §03: a common
# prefix is stored once), and reading it through aliased blocks gives exactly
# what private copies of those blocks give (page A §02: scattered blocks are read
# as one logical sequence).
def _grouped(seed, groups, dtype=torch.float32, hq=4, hkv=2, d=16, b=16):
    case = workloads.make_grouped_decode_case(seed, groups, hq, hkv, d, b, dtype)
    kc, vc = oracle.append(_np(case.k_pool), _np(case.v_pool), _np(case.k_new), _np(case.v_new),
                           case.slot_mapping.numpy())
    return case, kc, vc


GROUPINGS = [
    [([40, 70, 33], 32)],                          # one group, two shared blocks
    [([40, 70, 33], 32), ([5], 0), ([100, 90], 64)],
    [([20, 50], 48), ([0, 17], 16), ([16, 33], 16)],  # members shorter than / equal to the prefix, an empty one
]


@pytest.mark.parametrize("groups", GROUPINGS)
def test_grouped_batches_alias_their_shared_blocks(groups):
    case, _, _ = _grouped(77, groups)
    gs, sl, bt = case.meta["group_starts"].numpy(), case.meta["shared_lens"].numpy(), case.block_tables.numpy()
    b = case.block_size
    assert gs[0] == 0 and gs[-1] == case.num_seqs and (np.diff(gs) >= 0).all()
    for g in range(len(gs) - 1):
        members = range(gs[g], gs[g + 1])
        assert len({int(sl[s]) for s in members}) == 1  # one shared length per group, whole blocks
        n = int(sl[gs[g]]) // b
        assert int(sl[gs[g]]) % b == 0
        for s in members:
            assert (bt[s, :n] == bt[gs[g], :n]).all()
    # no block is shared across groups
    for g in range(len(gs) - 1):
        for h in range(g + 1, len(gs) - 1):
            a = {int(x) for s in range(gs[g], gs[g + 1]) for x in bt[s, :(int(case.context_lens[s]) + b - 1) // b]}
            c = {int(x) for s in range(gs[h], gs[h + 1]) for x in bt[s, :(int(case.context_lens[s]) + b - 1) // b]}
            assert not a & c


@pytest.mark.parametrize("groups", GROUPINGS)
def test_aliased_prefix_equals_private_copies(groups):
    case, kc, vc = _grouped(78, groups)
    bt, ctx = case.block_tables.numpy().copy(), case.context_lens.numpy()
    ref = oracle.decode_attention(_np(case.q), kc, vc, bt, ctx, case.scale)
    # give every member after the first its own copy of each shared block
    gs, sl = case.meta["group_starts"].numpy(), case.meta["shared_lens"].numpy()
    kcs, vcs = [kc], [vc]
    nb = kc.shape[0]
    for g in range(len(gs) - 1):
        n = int(sl[gs[g]]) // case.block_size
        for s in range(gs[g] + 1, gs[g + 1]):
            for j in range(n):
                kcs.append(kc[bt[s, j]][None]); vcs.append(vc[bt[s, j]][None])
                bt[s, j] = nb
                nb += 1
    got = oracle.decode_attention(_np(case.q), np.concatenate(kcs), np.concatenate(vcs), bt, ctx, case.scale)
    assert np.array_equal(got, ref)
