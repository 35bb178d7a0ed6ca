"""Plain CPU oracle for attention over a paged KV cache with prefix reuse.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call this
module: it is used by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``. It shares no code with the HIP path.

Everything here is float64 NumPy written for readability, not speed. Each
function cites the passage of the source pages it follows:

* page A: "PagedAttention과 RadixAttention으로 LLM KV 캐시 최적화"
  (aitrends.kr, AI-written summary), sections 01-06.
* page B: "KV Cache 완전 정리 — PagedAttention vs RadixAttention, SGLang이
  빠른 이유" (cell-devlog), sections "KV 캐시가 뭔가", "PagedAttention",
  "RadixAttention", "FP8 KV 캐시".
* page C: "KV Cache에 대해 알아보자 (Feat. Attention)" (chooblog), sections
  1 (attention and the KV cache), 3 (prefill vs decode), 4 (memory size).

Logical cache layout used by every function below: ``cache[block, offset,
kv_head, dim]``; a token at logical position t of a sequence lives in
physical block ``block_table[t // B]`` at offset ``t % B`` (page A, section 02:
the block table maps logical blocks to scattered physical blocks that the
kernel reads as one contiguous sequence). How the GPU path lays these blocks
out in memory is its own business; tests hand this module logical views.

Parity status of each function (how it is pinned, in tests/test_oracle_pins.py):

* kv_bytes_per_token .......... pinned: the 128 KiB/token figure of page A §01.
* e4m3fn_decode ............... pinned: all 256 codes vs torch.float8_e4m3fn.
* e4m3fn_quantize ............. pinned: vs torch's RNE conversion after clamping,
                                 plus hand-checked ties, subnormals, saturation.
* append ...................... pinned: write-once round trip, untouched slots.
* gather ...................... pinned: permutation of physical blocks, brute force.
* decode_attention ............ pinned: scalar brute force, closed forms (mean of V,
                                 constant V, single key), library SDPA.
* suffix_prefill_attention .... pinned: P=0 vs library causal SDPA; prefix reuse
                                 equals full recompute (page A §03 2,000/1,900).
"""
from __future__ import annotations


import numpy as np

__all__ = [
    "kv_bytes_per_token",
    "E4M3FN_MAX",
    "e4m3fn_decode",
    "e4m3fn_quantize",
    "append",
    "gather",
    "decode_attention",
    "suffix_prefill_attention",
]


# --------------------------------------------------------------------------
# KV size (page C §4 formula; page A §01 Llama-3-8B example)
# --------------------------------------------------------------------------
def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """Bytes of K and V cache one token occupies: 2 (K and V) x layers x KV heads
    x head dim x element size (page C §4; the head count is the KV head count,
    as in page A §01 where 32 layers, 8 KV heads, d=128, FP16 give ~128 KiB)."""
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


# --------------------------------------------------------------------------
# FP8 e4m3 codec (page B, "FP8 KV 캐시": the cache may be stored as fp8_e4m3)
# --------------------------------------------------------------------------
# The pages name the format only as "fp8_e4m3". Reading: the OCP E4M3FN encoding
# (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, the
# all-ones code S.1111.111 is NaN, largest finite magnitude 448).
E4M3FN_MAX = 448.0


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each e4m3fn byte as float64, from the bit-field definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = np.ldexp(1.0 + man / 8.0, exp - 7)
    subnormal = np.ldexp(man / 8.0, -6)
    val = np.where(exp == 0, subnormal, normal) * sign
    val = np.where((exp == 0xF) & (man == 0x7), np.nan, val)
    return val


# codes 0x00 .. 0x7E: every non-negative finite value, strictly increasing
_GRID = e4m3fn_decode(np.arange(127))


def e4m3fn_quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """Quantize real values to e4m3fn codes: y = x / scale computed as an IEEE
    float32 division, then rounded to the nearest e4m3fn value with ties going
    to the even code (the code's last bit is the mantissa's last bit), and
    saturated to +-448 (reading of page B "FP8 KV 캐시": the stored value times
    the per-tensor scale stands for x). NaN stays NaN (code 0x7F).

    The rounding is done against the explicit list of the 127 non-negative
    finite e4m3fn values, which ``e4m3fn_decode`` gives in increasing order."""
    y = (np.asarray(x, dtype=np.float32) / np.float32(scale)).astype(np.float64)
    nan = np.isnan(y)
    a = np.abs(np.where(nan, 0.0, y))
    hi = np.clip(np.searchsorted(_GRID, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - _GRID[lo]
    d_hi = _GRID[hi] - a
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a >= E4M3FN_MAX, 0x7E, code)
    code = code | np.where(np.signbit(y) & ~nan, 0x80, 0)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# Append (page C §3: decode adds the new token's K and V to the cache;
# page A §02: the slot is chosen by the block manager)
# --------------------------------------------------------------------------
def append(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray, v: np.ndarray,
           slot_mapping: np.ndarray, fp8: bool = False, k_scale: float = 1.0,
           v_scale: float = 1.0):
    """Expected caches after writing token i's K and V rows into flat slot
    ``slot_mapping[i]`` (slot = physical block * B + offset); negative slots are
    skipped. Caches are logical [num_blocks, B, H_kv, d]; for an fp8 cache they
    hold uint8 codes and rows are quantized with ``e4m3fn_quantize``. Returns
    new arrays; the inputs are not modified. Slots not named keep their bytes
    (past K and V never change, page C §1)."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    nb, bsz = kc.shape[0], kc.shape[1]
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0 or slot >= nb * bsz:
            continue
        blk, off = divmod(int(slot), bsz)
        if fp8:
            kc[blk, off] = e4m3fn_quantize(k[i], k_scale)
            vc[blk, off] = e4m3fn_quantize(v[i], v_scale)
        else:
            kc[blk, off] = k[i]
            vc[blk, off] = v[i]
    return kc, vc


# --------------------------------------------------------------------------
# Gather (page A §02: physically scattered blocks, e.g. 7, 1, 3, are read in
# logical order through the block table)
# --------------------------------------------------------------------------
def gather(cache: np.ndarray, block_table_row: np.ndarray, length: int,
           fp8: bool = False, scale: float = 1.0) -> np.ndarray:
    """Contiguous float64 copy [length, H_kv, d] of one sequence's cached rows.
    For an fp8 cache the codes are decoded and multiplied by the scale."""
    bsz = cache.shape[1]
    t = np.arange(length)
    blocks = np.asarray(block_table_row)[t // bsz].astype(np.int64)
    rows = cache[blocks, t % bsz]
    if fp8:
        return e4m3fn_decode(rows) * float(scale)
    return rows.astype(np.float64)


def _softmax_attend(q_row: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q K^T * scale) V for one query row (page C §1 equation, with
    scale = 1/sqrt(d_k) passed in). The max is subtracted before exp; this
    does not change the value."""
    s = scale * (keys @ q_row)
    p = np.exp(s - s.max())
    p = p / p.sum()
    return p @ values


# --------------------------------------------------------------------------
# Decode (page C §3: the new token's Q attends to every cached K, V;
# page C §4 / page A §01: grouped-query attention with fewer KV heads)
# --------------------------------------------------------------------------
def decode_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                     block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                     fp8: bool = False, k_scale: float = 1.0, v_scale: float = 1.0,
                     seqs=None, heads=None) -> np.ndarray:
    """out[s, h] = softmax(scale * q[s,h] . K_s^T) V_s over the context_lens[s]
    cached tokens of sequence s, for query head h reading KV head h // G with
    G = H_q / H_kv (reading: consecutive query heads share a KV head). A
    sequence with length 0 gives a zero row. ``seqs``/``heads`` restrict the
    work to a sample; other rows are NaN."""
    num_seqs, hq, d = q.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    out = np.full((num_seqs, hq, d), np.nan)
    for s in (range(num_seqs) if seqs is None else seqs):
        n = int(context_lens[s])
        if n <= 0:
            out[s] = 0.0
            continue
        kc = gather(k_cache, block_tables[s], n, fp8, k_scale)
        vc = gather(v_cache, block_tables[s], n, fp8, v_scale)
        for h in (range(hq) if heads is None else heads):
            g = h // group
            out[s, h] = _softmax_attend(q[s, h].astype(np.float64), kc[:, g, :], vc[:, g, :], scale)
    return out


# --------------------------------------------------------------------------
# Suffix-only prefill (page A §03: with the longest matched prefix cached, only
# the unmatched suffix goes through the model; page C §3: prefill handles all
# new tokens at once, each attending causally)
# --------------------------------------------------------------------------
def suffix_prefill_attention(q_suffix: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                             block_tables: np.ndarray, prefix_lens: np.ndarray,
                             suffix_lens: np.ndarray, scale: float, fp8: bool = False,
                             k_scale: float = 1.0, v_scale: float = 1.0,
                             rows=None) -> np.ndarray:
    """For request r with P_r cached prefix tokens and S_r new suffix tokens
    (whose K, V are already in the cache at positions P_r .. P_r+S_r-1), suffix
    row i of query head h attends to key positions 0 .. P_r + i inclusive.
    q_suffix and the result are [sum_r S_r, H_q, d], packed request by request.
    ``rows`` optionally restricts the work to a list of packed row indices."""
    total, hq, d = q_suffix.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    out = np.full((total, hq, d), np.nan)
    wanted = None if rows is None else set(int(x) for x in rows)
    base = 0
    for r in range(len(prefix_lens)):
        p, sl = int(prefix_lens[r]), int(suffix_lens[r])
        if sl > 0 and (wanted is None or any(base <= x < base + sl for x in wanted)):
            kc = gather(k_cache, block_tables[r], p + sl, fp8, k_scale)
            vc = gather(v_cache, block_tables[r], p + sl, fp8, v_scale)
            for i in range(sl):
                if wanted is not None and base + i not in wanted:
                    continue
                n = p + i + 1  # keys 0 .. P + i inclusive
                for h in range(hq):
                    g = h // group
                    out[base + i, h] = _softmax_attend(q_suffix[base + i, h].astype(np.float64),
                                                       kc[:n, g, :], vc[:n, g, :], scale)
        base += sl
    return out
