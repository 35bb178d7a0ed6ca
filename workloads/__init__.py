"""Seeded synthetic inputs for paged-KV attention with prefix reuse.

This module only builds inputs: block pools, block tables, lengths, slot
mappings and N(0,1) values in the shapes of the workloads the source pages
describe. It holds none of the attention arithmetic, and both the HIP path and
the CPU oracle consume what it returns.

Conventions
-----------
* Caches are returned in the *logical* layout ``[num_blocks, B, H_kv, d]``:
  the row of a token at logical position t of sequence s sits at
  ``[block_tables[s, t // B], t % B]`` (page "PagedAttention과 RadixAttention으로
  LLM KV 캐시 최적화", section 02: a per-request block table maps logical
  blocks onto scattered physical blocks of 16 or 32 tokens).
* Slots that hold no live token are filled with NaN (fp8 code 0x7F), so a
  kernel that reads a slot it should not read produces NaN.
* Block-table columns past a sequence's last block point at a dedicated poison
  block (all NaN) at the end of the pool: reading one is in bounds but shows.
* ``context_lens`` count the newest token (it is appended, then attended).
* One ``torch.Generator`` seeded with ``1000 + config index`` draws, in order,
  lengths, the block permutation, then values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

__all__ = [
    "DecodeCase", "PrefillCase", "LongContextFp8Case",
    "make_decode_case", "make_prefill_case",
    "config1_tiny_decode", "config2_llama_decode", "config3_shared_prefix_decode",
    "config4_suffix_prefill", "next_turn_suffix_prefill", "config5_long_context_fp8",
    "fp8_nan_code",
]

fp8_nan_code = 0x7F


@dataclass
class DecodeCase:
    name: str
    dtype: torch.dtype              # q / out / appended-row dtype
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q: torch.Tensor                 # [num_seqs, H_q, d]
    k_pool: torch.Tensor            # logical [NB, B, H_kv, d], pre-append state
    v_pool: torch.Tensor
    block_tables: torch.Tensor      # int32 [num_seqs, max_blocks]
    context_lens: torch.Tensor      # int32 [num_seqs], post-append
    k_new: torch.Tensor             # [T, H_kv, d], rows to append
    v_new: torch.Tensor
    slot_mapping: torch.Tensor      # int64 [T]
    scale: float
    shared_blocks: int = 0          # leading table columns aliased by every sequence
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return self.q.shape[0]

    @property
    def num_blocks(self) -> int:
        return self.k_pool.shape[0]

    def kv_read_bytes(self) -> int:
        """Logical K+V bytes one decode pass reads: every live token of every
        sequence, for every KV head, K and V."""
        el = self.k_pool.element_size()
        return int(self.context_lens.long().sum()) * 2 * self.num_kv_heads * self.head_dim * el

    def unique_kv_read_bytes(self) -> int:
        """K+V bytes of distinct physical slots read (aliased prefix blocks once)."""
        b = self.block_size
        seen = set()
        total = 0
        for s in range(self.num_seqs):
            n = int(self.context_lens[s])
            for j in range((n + b - 1) // b):
                blk = int(self.block_tables[s, j])
                used = min(b, n - j * b)
                key = blk
                if key in seen:
                    continue
                seen.add(key)
                total += used
        return total * 2 * self.num_kv_heads * self.head_dim * self.k_pool.element_size()


@dataclass
class PrefillCase:
    name: str
    dtype: torch.dtype
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_suffix: torch.Tensor          # [sum S_r, H_q, d]
    k_pool: torch.Tensor            # logical [NB, B, H_kv, d]; suffix slots NaN
    v_pool: torch.Tensor
    block_tables: torch.Tensor      # int32 [R, max_blocks]
    prefix_lens: torch.Tensor       # int32 [R]
    suffix_lens: torch.Tensor       # int32 [R]
    k_new: torch.Tensor             # [sum S_r, H_kv, d] suffix K rows
    v_new: torch.Tensor
    slot_mapping: torch.Tensor      # int64 [sum S_r]
    scale: float
    meta: dict = field(default_factory=dict)

    def flops(self) -> int:
        """Multiply-adds x 2 of QK^T and PV over unmasked (row, key) pairs only."""
        pairs = 0
        for p, s in zip(self.prefix_lens.tolist(), self.suffix_lens.tolist()):
            pairs += p * s + s * (s + 1) // 2
        return 4 * self.head_dim * self.num_q_heads * pairs


def _randn(g: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)


def _poison_value(dtype: torch.dtype):
    return float("nan")


def _layout_sequences(g, lens, block_size, extra_free_blocks=0, shared=None):
    """Assign physical blocks. Returns (block_tables, num_blocks, poison_block).

    ``shared``: optional (num_shared_blocks,) -> the first columns of every
    table alias the same physical blocks."""
    nseq = len(lens)
    nblk_seq = [(n + block_size - 1) // block_size for n in lens]
    n_shared = 0 if shared is None else shared
    private = [max(nb - n_shared, 0) for nb in nblk_seq]  # a member may end inside the shared blocks
    used = n_shared + sum(private)
    pool = used + extra_free_blocks
    perm = torch.randperm(pool, generator=g)
    poison = pool  # one extra all-NaN block after the pool proper
    max_blocks = max(max(nblk_seq) if nseq else 1, n_shared)  # every table holds the shared blocks
    bt = torch.full((nseq, max(max_blocks, 1)), poison, dtype=torch.int32)
    cursor = 0
    shared_ids = perm[:n_shared]
    cursor = n_shared
    for s in range(nseq):
        if n_shared:
            bt[s, :n_shared] = shared_ids.to(torch.int32)
        k = private[s]
        bt[s, n_shared:n_shared + k] = perm[cursor:cursor + k].to(torch.int32)
        cursor += k
    return bt, pool + 1, poison


def _fill_pool(g, num_blocks, block_size, hkv, d, dtype):
    k = _randn(g, (num_blocks, block_size, hkv, d), dtype)
    v = _randn(g, (num_blocks, block_size, hkv, d), dtype)
    return k, v


def _live_mask(bt, lens, num_blocks, block_size):
    """Bool [num_blocks, B]: True where some sequence keeps a token."""
    live = torch.zeros(num_blocks, block_size, dtype=torch.bool)
    for s, n in enumerate(lens):
        for j in range((n + block_size - 1) // block_size):
            used = min(block_size, n - j * block_size)
            live[int(bt[s, j]), :used] = True
    return live


def _slot(bt_row, t, block_size) -> int:
    return int(bt_row[t // block_size]) * block_size + t % block_size


def make_decode_case(seed: int, lens: List[int], num_q_heads: int, num_kv_heads: int, head_dim: int,
                     block_size: int, dtype: torch.dtype, name: str = "decode",
                     extra_free_blocks: int = 0, shared_prefix_tokens: int = 0,
                     scale: Optional[float] = None, lens_given: bool = True,
                     g: Optional[torch.Generator] = None) -> DecodeCase:
    """A decode batch: every sequence has ``lens[s]`` tokens after appending its
    newest one. Tokens 0 .. len-2 are already cached; token len-1 is appended.

    ``shared_prefix_tokens``: the first ``shared_prefix_tokens // B`` full
    blocks of every table alias the same physical blocks, and the remaining
    ``shared_prefix_tokens % B`` prefix tokens are identical private copies at
    the start of each sequence's first private block (only full blocks can be
    shared: a block is matched as a whole)."""
    if g is None:
        g = torch.Generator().manual_seed(seed)
    n_shared = shared_prefix_tokens // block_size
    tail = shared_prefix_tokens % block_size
    bt, nb, poison = _layout_sequences(g, lens, block_size, extra_free_blocks, n_shared)
    nseq = len(lens)
    q = _randn(g, (nseq, num_q_heads, head_dim), dtype)
    k_pool, v_pool = _fill_pool(g, nb, block_size, num_kv_heads, head_dim, dtype)
    if shared_prefix_tokens:
        k_tail = _randn(g, (tail, num_kv_heads, head_dim), dtype)
        v_tail = _randn(g, (tail, num_kv_heads, head_dim), dtype)
        for s in range(nseq):
            for t in range(n_shared * block_size, shared_prefix_tokens):
                blk, off = divmod(_slot(bt[s], t, block_size), block_size)
                k_pool[blk, off] = k_tail[t - n_shared * block_size]
                v_pool[blk, off] = v_tail[t - n_shared * block_size]
    k_new = _randn(g, (nseq, num_kv_heads, head_dim), dtype)
    v_new = _randn(g, (nseq, num_kv_heads, head_dim), dtype)
    # poison everything that is not a live, already-cached token; the shared
    # blocks hold the whole shared prefix, and a sequence that ends inside
    # them has its newest token there already (nothing to append)
    in_shared = [0 < n <= n_shared * block_size for n in lens]
    pre_lens = [n if sh else max(n - 1, 0) for n, sh in zip(lens, in_shared)]
    live = _live_mask(bt, pre_lens, nb, block_size)
    if n_shared:
        live[bt[0, :n_shared].long()] = True
    k_pool[~live] = _poison_value(dtype)
    v_pool[~live] = _poison_value(dtype)
    slots = torch.tensor([_slot(bt[s], lens[s] - 1, block_size) if lens[s] > 0 and not in_shared[s] else -1
                          for s in range(nseq)], dtype=torch.int64)
    return DecodeCase(
        name=name, dtype=dtype, block_size=block_size, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, q=q, k_pool=k_pool, v_pool=v_pool,
        block_tables=bt, context_lens=torch.tensor(lens, dtype=torch.int32),
        k_new=k_new, v_new=v_new, slot_mapping=slots,
        scale=(1.0 / math.sqrt(head_dim)) if scale is None else scale,
        shared_blocks=n_shared, meta={"poison_block": poison, "seed": seed})


def make_grouped_decode_case(seed: int, groups: List[tuple], num_q_heads: int, num_kv_heads: int,
                             head_dim: int, block_size: int, dtype: torch.dtype,
                             name: str = "grouped-decode") -> DecodeCase:
    """Several groups of sequences, each group sharing its own prefix blocks:
    ``groups`` is a list of (lens, shared_prefix_tokens) as for
    make_decode_case. The groups' pools are laid side by side (block ids
    offset), so blocks are shared within a group and never across groups.
    meta["group_starts"] ([G+1]) and meta["shared_lens"] (per sequence, the
    aliased whole blocks in tokens) describe the grouping."""
    parts = [make_decode_case(seed * 1000 + i, list(lens), num_q_heads, num_kv_heads, head_dim, block_size,
                              dtype, shared_prefix_tokens=shared)
             for i, (lens, shared) in enumerate(groups)]
    width = max(c.block_tables.shape[1] for c in parts)
    offset, tables, starts, shared_lens = 0, [], [0], []
    for c, (lens, shared) in zip(parts, groups):
        bt = torch.full((c.num_seqs, width), c.meta["poison_block"], dtype=torch.int32)
        bt[:, :c.block_tables.shape[1]] = c.block_tables
        tables.append(bt + offset)
        starts.append(starts[-1] + c.num_seqs)
        shared_lens += [(shared // block_size) * block_size] * c.num_seqs
        offset += c.num_blocks
    slots, base = [], 0
    for c in parts:
        slots.append(torch.where(c.slot_mapping >= 0, c.slot_mapping + base * block_size, c.slot_mapping))
        base += c.num_blocks
    return DecodeCase(
        name=name, dtype=dtype, block_size=block_size, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, q=torch.cat([c.q for c in parts]), k_pool=torch.cat([c.k_pool for c in parts]),
        v_pool=torch.cat([c.v_pool for c in parts]), block_tables=torch.cat(tables),
        context_lens=torch.cat([c.context_lens for c in parts]), k_new=torch.cat([c.k_new for c in parts]),
        v_new=torch.cat([c.v_new for c in parts]), slot_mapping=torch.cat(slots), scale=parts[0].scale,
        meta={"group_starts": torch.tensor(starts, dtype=torch.int32),
              "shared_lens": torch.tensor(shared_lens, dtype=torch.int32), "seed": seed})


def make_prefill_case(seed: int, prefix_lens: List[int], suffix_lens: List[int], num_q_heads: int,
                      num_kv_heads: int, head_dim: int, block_size: int, dtype: torch.dtype,
                      name: str = "prefill", extra_free_blocks: int = 0,
                      scale: Optional[float] = None) -> PrefillCase:
    """Requests whose first ``prefix_lens[r]`` tokens are cached (matched prefix)
    and whose next ``suffix_lens[r]`` tokens are new: their K, V rows are
    returned in ``k_new``/``v_new`` with the slots to append them to."""
    g = torch.Generator().manual_seed(seed)
    lens = [p + s for p, s in zip(prefix_lens, suffix_lens)]
    bt, nb, poison = _layout_sequences(g, lens, block_size, extra_free_blocks)
    total = sum(suffix_lens)
    q = _randn(g, (total, num_q_heads, head_dim), dtype)
    k_pool, v_pool = _fill_pool(g, nb, block_size, num_kv_heads, head_dim, dtype)
    k_new = _randn(g, (total, num_kv_heads, head_dim), dtype)
    v_new = _randn(g, (total, num_kv_heads, head_dim), dtype)
    live = _live_mask(bt, list(prefix_lens), nb, block_size)
    k_pool[~live] = _poison_value(dtype)
    v_pool[~live] = _poison_value(dtype)
    slots = []
    for r, (p, s) in enumerate(zip(prefix_lens, suffix_lens)):
        slots += [_slot(bt[r], t, block_size) for t in range(p, p + s)]
    return PrefillCase(
        name=name, dtype=dtype, block_size=block_size, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, q_suffix=q, k_pool=k_pool, v_pool=v_pool,
        block_tables=bt, prefix_lens=torch.tensor(prefix_lens, dtype=torch.int32),
        suffix_lens=torch.tensor(suffix_lens, dtype=torch.int32), k_new=k_new, v_new=v_new,
        slot_mapping=torch.tensor(slots, dtype=torch.int64),
        scale=(1.0 / math.sqrt(head_dim)) if scale is None else scale,
        meta={"poison_block": poison, "seed": seed})


# ---------------------------------------------------------------------------
# The five workloads (Llama-3-8B geometry: 32 Q heads, 8 KV heads, d=128, from
# page "PagedAttention과 RadixAttention으로 LLM KV 캐시 최적화" section 01)
# ---------------------------------------------------------------------------
def config1_tiny_decode() -> DecodeCase:
    """4 sequences, H_q=4, H_kv=2, d=64, fp32, B=16, lengths {17, 33, 60, 100}
    (60 tokens need only 4 blocks, section 02), a 64-block pool in random order."""
    lens = [17, 33, 60, 100]
    used = sum((n + 15) // 16 for n in lens)
    return make_decode_case(1001, lens, 4, 2, 64, 16, torch.float32, name="tiny-decode-fp32",
                            extra_free_blocks=64 - used, scale=0.125)


def config2_llama_decode() -> DecodeCase:
    """Batch 64, 32/8 heads, d=128, fp16, B=16, lengths uniform in [512, 4096]."""
    g = torch.Generator().manual_seed(1002)
    lens = torch.randint(512, 4097, (64,), generator=g).tolist()
    return make_decode_case(1002, lens, 32, 8, 128, 16, torch.float16,
                            name="llama3-8b-decode-b64-fp16", g=g)


def config3_shared_prefix_decode() -> DecodeCase:
    """256 sequences sharing a 1,000-token prefix (31 aliased 32-token blocks +
    8 copied tail tokens) plus 50..500 private tokens, 32/8 heads, d=128, bf16,
    B=32 (page "KV Cache 완전 정리", RadixAttention: 1,000 chat requests with one
    1,000-token system prompt)."""
    g = torch.Generator().manual_seed(1003)
    suffix = torch.randint(50, 501, (256,), generator=g).tolist()
    lens = [1000 + s for s in suffix]
    return make_decode_case(1003, lens, 32, 8, 128, 32, torch.bfloat16,
                            name="shared-prefix-decode-256x1000-bf16", shared_prefix_tokens=1000, g=g)


def config4_suffix_prefill() -> PrefillCase:
    """16 requests, 1,900 cached prefix tokens + 100 new suffix tokens each
    (page "PagedAttention과 RadixAttention…" section 03: a 2,000-token request
    with 1,900 cached prefills 100), 32/8 heads, d=128, bf16, B=16, a
    2,000-block pool in random order."""
    return make_prefill_case(1004, [1900] * 16, [100] * 16, 32, 8, 128, 16, torch.bfloat16,
                             name="suffix-prefill-16x(1900+100)-bf16")


def next_turn_suffix_prefill() -> PrefillCase:
    """One conversation's next turn: one request, 8,000 cached tokens (every
    earlier turn) + 100 new ones (page "KV Cache에 대해 알아보자" section 5,
    third limit: each turn of a multi-turn conversation carries all earlier
    turns, whose K and V are cached), 32/8 heads, d=128, bf16, B=16."""
    return make_prefill_case(1006, [8000], [100], 32, 8, 128, 16, torch.bfloat16,
                             name="suffix-prefill-1x(8000+100)-bf16")


# ---------------------------------------------------------------------------
# Config 5: long-context fp8 decode. Too large to build on the host, so values
# are drawn on the device, chunk by chunk, from seeds derived from the layer and
# sequence; the same chunk can be re-drawn later for a sampled oracle check.
# ---------------------------------------------------------------------------
@dataclass
class LongContextFp8Case:
    name: str
    num_layers: int
    num_seqs: int
    context_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    block_tables: torch.Tensor      # int32 [num_seqs, context_len / B], shared by all layers
    num_blocks: int                 # per-layer pool size (+1 poison block)
    base_seed: int = 1005

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def raw_kv(self, layer: int, seq: int, device, which: str) -> torch.Tensor:
        """Underlying fp32 K (which='k') or V ('v') rows [context_len, H_kv, d]
        of one sequence in one layer, ~N(0,1), drawn on ``device``."""
        off = 0 if which == "k" else 1
        g = torch.Generator(device=device).manual_seed(
            self.base_seed * 1_000_003 + (layer * 64 + seq) * 2 + off)
        return torch.randn(self.context_len, self.num_kv_heads, self.head_dim,
                           generator=g, device=device, dtype=torch.float32)

    def raw_q(self, layer: int, device) -> torch.Tensor:
        g = torch.Generator(device=device).manual_seed(self.base_seed * 7919 + layer)
        return torch.randn(self.num_seqs, self.num_q_heads, self.head_dim, generator=g,
                           device=device, dtype=torch.float32).to(torch.bfloat16)

    def raw_new(self, layer: int, device, which: str) -> torch.Tensor:
        g = torch.Generator(device=device).manual_seed(self.base_seed * 104729 + layer * 2
                                                       + (0 if which == "k" else 1))
        return torch.randn(self.num_seqs, self.num_kv_heads, self.head_dim, generator=g,
                           device=device, dtype=torch.float32).to(torch.bfloat16)

    def slots(self, seq: int, t0: int, t1: int) -> torch.Tensor:
        t = torch.arange(t0, t1)
        return (self.block_tables[seq].long()[t // self.block_size] * self.block_size
                + t % self.block_size)

    def kv_read_bytes_per_layer(self) -> int:
        return self.num_seqs * self.context_len * 2 * self.num_kv_heads * self.head_dim


def config5_long_context_fp8(num_layers: int = 32, num_seqs: int = 8,
                             context_len: int = 100_000) -> LongContextFp8Case:
    """Batch 8 at 100,000-token contexts, 32 layers, 32/8 heads, d=128, fp8
    e4m3 KV with one fp32 scale per layer per K/V, B=32; one block table per
    sequence serves every layer (page A section 02 gives a table per request)."""
    bsz = 32
    g = torch.Generator().manual_seed(1005)
    nblk = (context_len + bsz - 1) // bsz
    pool = nblk * num_seqs
    perm = torch.randperm(pool, generator=g).to(torch.int32)
    bt = perm.view(num_seqs, nblk).clone()
    return LongContextFp8Case(name="long-context-fp8-decode-8x100k-32L", num_layers=num_layers,
                              num_seqs=num_seqs, context_len=context_len, num_q_heads=32,
                              num_kv_heads=8, head_dim=128, block_size=bsz, block_tables=bt,
                              num_blocks=pool + 1)
