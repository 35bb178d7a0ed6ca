"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/*.h declares, and rejects bad arguments with a
status code and a message before launching anything."""
import ctypes
import re
from pathlib import Path

import pytest

import prefix_reuse_amd as pkv
from prefix_reuse_amd import PkvTensor

HEADERS = sorted((Path(__file__).resolve().parent.parent / "include").glob("*.h"))

F32, F16, BF16, FP8, I32, I64 = range(6)
FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = "\n".join(h.read_text() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"pkv_append", "pkv_decode_attn", "pkv_suffix_prefill_attn", "pkv_decode_workspace_bytes",
            "pkv_last_error", "pkv_abi_version", "pkv_pc_admit", "pkv_radix_match"} <= set(names)
    for n in names:
        assert hasattr(pkv.lib, n), n


def test_abi_version():
    assert pkv.abi_version() == 6


def T(shape, dtype, strides=None, ptr=FAKE):
    t = PkvTensor()
    t.data = ptr
    t.dtype = dtype
    t.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, strides)):
        t.shape[i] = s
        t.stride[i] = st
    return t


def caches(nb=8, h=2, b=16, d=64, dt=F16):
    return T([nb, h, b, d], dt), T([nb, h, d, b], dt)


def R(x):
    return ctypes.byref(x) if x is not None else None


def decode(q, kc, vc, bt, cl, out, ws=None, ws_bytes=0, scale=0.125, ks=1.0, vs=1.0):
    return pkv.lib.pkv_decode_attn(R(q), R(kc), R(vc), R(bt), R(cl), scale, ks, vs, ws, ws_bytes, R(out), None)


def err():
    return pkv.lib.pkv_last_error().decode()


def test_decode_rejects_null_descriptor():
    kc, vc = caches()
    rc = decode(None, kc, vc, T([2, 4], I32), T([2], I32), T([2, 4, 64], F16))
    assert rc == 1 and "q" in err()


def test_element_count_overflow_is_rejected():
    """Extents whose product overflows 64 bits fail validation (status SHAPE)
    instead of wrapping around into a plausible size."""
    kc, vc = caches()
    huge = T([2 ** 40, 2 ** 40, 64], F16, strides=[2 ** 46, 64, 1])
    rc = decode(huge, kc, vc, T([2, 4], I32), T([2], I32), T([2, 4, 64], F16))
    assert rc == 3 and "overflows" in err()


def test_decode_rejects_group_mismatch():
    kc, vc = caches(h=3)
    rc = decode(T([2, 4, 64], F16), kc, vc, T([2, 4], I32), T([2], I32), T([2, 4, 64], F16))
    assert rc == 5 and "multiple" in err()


def test_decode_rejects_dtype_mismatch():
    kc, vc = caches(dt=BF16)
    rc = decode(T([2, 4, 64], F16), kc, vc, T([2, 4], I32), T([2], I32), T([2, 4, 64], F16))
    assert rc == 2
    kc, vc = caches(dt=FP8)
    rc = decode(T([2, 4, 64], F32), kc, vc, T([2, 4], I32), T([2], I32), T([2, 4, 64], F32))
    assert rc == 2 and "fp8" in err()


def test_decode_rejects_unsupported_head_dim_and_block():
    kc, vc = caches(d=96)
    assert decode(T([2, 4, 96], F16), kc, vc, T([2, 4], I32), T([2], I32), T([2, 4, 96], F16)) == 5
    kc, vc = caches(b=8)
    assert decode(T([2, 4, 64], F16), kc, vc, T([2, 4], I32), T([2], I32), T([2, 4, 64], F16)) == 5


def test_decode_rejects_wrong_cache_layout():
    kc, _ = caches()
    vc_wrong = T([8, 2, 16, 64], F16)  # V given in the K layout
    assert decode(T([2, 4, 64], F16), kc, vc_wrong, T([2, 4], I32), T([2], I32), T([2, 4, 64], F16)) == 3
    kc_strided = T([8, 2, 16, 64], F16, strides=[4096, 2048, 64, 1])  # not contiguous
    _, vc = caches()
    assert decode(T([2, 4, 64], F16), kc_strided, vc, T([2, 4], I32), T([2], I32), T([2, 4, 64], F16)) == 4


def test_decode_rejects_bad_tables_and_lengths():
    kc, vc = caches()
    assert decode(T([2, 4, 64], F16), kc, vc, T([2, 4], I64), T([2], I32), T([2, 4, 64], F16)) == 2
    assert decode(T([2, 4, 64], F16), kc, vc, T([3, 4], I32), T([2], I32), T([2, 4, 64], F16)) == 3
    assert decode(T([2, 4, 64], F16), kc, vc, T([2, 4], I32), T([2], I64), T([2, 4, 64], F16)) == 2


def test_decode_rejects_misaligned_rows():
    kc, vc = caches()
    q = T([2, 4, 64], F16, ptr=FAKE + 2)
    assert decode(q, kc, vc, T([2, 4], I32), T([2], I32), T([2, 4, 64], F16)) == 4


def test_decode_rejects_missing_workspace():
    need = pkv.decode_workspace_bytes(1, 4, 2, 64, 4096, 16)
    assert need > 0
    kc, vc = caches()
    rc = decode(T([1, 4, 64], F16), kc, vc, T([1, 4096], I32), T([1], I32), T([1, 4, 64], F16))
    assert rc == 6 and "workspace" in err()
    rc = decode(T([1, 4, 64], F16), kc, vc, T([1, 4096], I32), T([1], I32), T([1, 4, 64], F16),
                ws=FAKE, ws_bytes=need - 1)
    assert rc == 6


def test_workspace_size_formula(monkeypatch):
    assert pkv.decode_workspace_bytes(0, 4, 3, 64, 4, 16) == 0  # 4 % 3 != 0
    monkeypatch.setenv("PKV_DECODE_WAVES", "64")
    # 64 waves over 8 KV heads -> 8 per head; slots = 8 + S; plus 2 ints per sequence
    assert pkv.decode_workspace_bytes(5, 32, 8, 128, 3125, 32) == (8 + 5) * 32 * 130 * 4 + 5 * 8
    # 40 query heads over 2 KV heads: G = 20 needs 2 head chunks -> 4 units, 16 waves each
    assert pkv.decode_workspace_bytes(3, 40, 2, 64, 10, 16) == (16 + 3) * 40 * 66 * 4 + 3 * 8


def test_append_rejects_bad_arguments():
    kc, vc = caches()
    k = T([3, 2, 64], F16)
    slots = T([3], I64)
    f = pkv.lib.pkv_append
    assert f(R(k), R(k), R(T([4], I64)), R(kc), R(vc), 1.0, 1.0, None) == 3
    assert f(R(k), R(k), R(T([3], F32)), R(kc), R(vc), 1.0, 1.0, None) == 2
    assert f(R(T([3, 2, 64], BF16)), R(T([3, 2, 64], BF16)), R(slots), R(kc), R(vc), 1.0, 1.0, None) == 2
    k8, v8 = caches(dt=FP8)
    assert f(R(k), R(k), R(slots), R(k8), R(v8), 0.0, 1.0, None) == 3  # scale must be > 0
    assert f(R(T([3, 4, 64], F16)), R(T([3, 4, 64], F16)), R(slots), R(kc), R(vc), 1.0, 1.0, None) == 3


def test_prefill_rejects_bad_arguments():
    kc, vc = caches()
    f = pkv.lib.pkv_suffix_prefill_attn
    q = T([10, 4, 64], F16)
    ok_bt, pl, sl = T([2, 4], I32), T([2], I32), T([2], I32)
    assert f(R(T([10, 4, 64], F32)), R(kc), R(vc), R(ok_bt), R(pl), R(sl), 0.1, 1.0, 1.0, R(T([10, 4, 64], F32)), None) == 2
    assert f(R(q), R(kc), R(vc), R(ok_bt), R(pl), R(T([3], I32)), 0.1, 1.0, 1.0, R(q), None) == 3
    assert f(R(q), R(kc), R(vc), R(T([2, 4], I32)), R(pl), R(sl), 0.1, 1.0, 1.0, R(T([9, 4, 64], F16)), None) == 3
    assert f(R(q), R(kc), R(vc), R(ok_bt), R(pl), R(sl), float("nan"), 1.0, 1.0, R(q), None) == 3


def test_prefill_split_workspace(monkeypatch):
    """The key-split prefill's workspace: none for a batch whose row tiles
    fill the CUs or under PKV_PREFILL_SPLITS=1; parts * total * H_q * (d + 2)
    floats under a forced count; a call with too small a workspace is
    refused before anything is launched."""
    ws = pkv.lib.pkv_suffix_prefill_workspace_bytes
    assert ws(1600, 16, 32, 8, 128, 125, 16) == 0           # the 16 x (1,900 + 100) batch: 200 work-groups
    assert ws(10, 1, 32, 7, 128, 100, 16) == 0              # 32 % 7 != 0
    monkeypatch.setenv("PKV_PREFILL_SPLITS", "1")
    assert ws(100, 1, 32, 8, 128, 600, 16) == 0
    monkeypatch.setenv("PKV_PREFILL_SPLITS", "5")
    assert ws(100, 1, 32, 8, 128, 600, 16) == 5 * 100 * 32 * 130 * 4
    assert ws(10, 2, 4, 2, 64, 4, 16) == 5 * 10 * 4 * 66 * 4
    kc, vc = caches()
    f = pkv.lib.pkv_suffix_prefill_attn_split
    q, bt, pl, sl = T([10, 4, 64], F16), T([2, 4], I32), T([2], I32), T([2], I32)
    assert f(R(q), R(kc), R(vc), R(bt), R(pl), R(sl), 0.1, 1.0, 1.0, None, 0, R(q), None) == 6
    assert "workspace" in err()
    need = ws(10, 2, 4, 2, 64, 4, 16)
    assert f(R(q), R(kc), R(vc), R(bt), R(pl), R(sl), 0.1, 1.0, 1.0, FAKE, need - 1, R(q), None) == 6
    assert f(R(q), R(kc), R(vc), R(bt), R(pl), R(sl), 0.1, 1.0, 1.0, FAKE + 8, need, R(q), None) == 4  # alignment
    assert f(R(T([10, 4, 64], F32)), R(kc), R(vc), R(bt), R(pl), R(sl), 0.1, 1.0, 1.0, FAKE, need,
             R(T([10, 4, 64], F32)), None) == 2


def test_scale_and_table_limits_are_checked():
    """scale * k_scale * log2(e) must be finite; block tables hold at most 2^24
    entries per row (so every position fits in 32 bits); a batch must hold
    fewer than 2^31 32-token chunks."""
    kc, vc = caches()
    args = (T([2, 4, 64], F16), kc, vc, T([2, 4], I32), T([2], I32), T([2, 4, 64], F16))
    assert decode(*args, scale=float("inf")) == 3 and "finite" in err()
    k8, v8 = caches(dt=FP8)
    assert decode(T([2, 4, 64], F16), k8, v8, T([2, 4], I32), T([2], I32), T([2, 4, 64], F16), scale=3e38,
                  ks=10.0) == 3 and "overflows" in err()
    wide = T([2, 2 ** 24 + 1], I32)
    assert decode(T([2, 4, 64], F16), kc, vc, wide, T([2], I32), T([2, 4, 64], F16)) == 3 and "wide" in err()
    many = 2 ** 14
    rc = decode(T([many, 4, 64], F16), kc, vc, T([many, 2 ** 24], I32), T([many], I32), T([many, 4, 64], F16))
    assert rc == 3 and "chunks" in err()
    f = pkv.lib.pkv_suffix_prefill_attn
    q = T([10, 4, 64], F16)
    assert f(R(q), R(kc), R(vc), R(T([2, 2 ** 24 + 1], I32)), R(T([2], I32)), R(T([2], I32)), 0.1, 1.0, 1.0,
             R(q), None) == 3


def test_empty_batches_are_accepted_without_launch():
    kc, vc = caches()
    assert decode(T([0, 4, 64], F16), kc, vc, T([0, 4], I32), T([0], I32), T([0, 4, 64], F16)) == 0
    f = pkv.lib.pkv_append
    assert f(R(T([0, 2, 64], F16)), R(T([0, 2, 64], F16)), R(T([0], I64)), R(kc), R(vc), 1.0, 1.0, None) == 0


def cascade(q, kc, vc, bt, cl, gs, sl, out, ws=None, ws_bytes=0):
    return pkv.lib.pkv_cascade_decode_attn(R(q), R(kc), R(vc), R(bt), R(cl), R(gs), R(sl), 0.125, 1.0, 1.0,
                                           ws, ws_bytes, R(out), None)


def test_cascade_rejects_bad_arguments():
    kc, vc = caches()
    q, out = T([3, 4, 64], F16), T([3, 4, 64], F16)
    bt, cl, gs, sl = T([3, 8], I32), T([3], I32), T([2], I32), T([3], I32)
    assert cascade(T([3, 4, 64], F32), *caches(dt=F32), bt, cl, gs, sl, T([3, 4, 64], F32)) == 2  # matrix cores
    assert cascade(q, kc, vc, bt, cl, T([2], I64), sl, out) == 2
    assert cascade(q, kc, vc, bt, cl, gs, T([2], I32), out) == 3          # one shared length per sequence
    assert cascade(q, kc, vc, bt, cl, T([0], I32), sl, out) == 3          # group_starts needs an entry
    need = pkv.cascade_workspace_bytes(3, 4, 2, 64)
    assert need > pkv.decode_workspace_bytes(3, 4, 2, 64, 8, 16)
    rc = cascade(q, kc, vc, bt, cl, gs, sl, out, ws=FAKE, ws_bytes=need - 1)
    assert rc == 6 and "cascade workspace" in err()


def test_cascade_workspace_size_formula(monkeypatch):
    monkeypatch.setenv("PKV_DECODE_WAVES", "64")
    monkeypatch.setenv("PKV_CASCADE_SPLITS", "3")
    dec = pkv.decode_workspace_bytes(5, 32, 8, 128, 100, 32)
    assert pkv.cascade_workspace_bytes(5, 32, 8, 128) == (dec + 15) // 16 * 16 + 3 * 5 * 32 * 130 * 4


def step(q, kn, vn, kc, vc, bt, cl, out, ws=None, ws_bytes=0, scale=0.125, ks=1.0, vs=1.0):
    return pkv.lib.pkv_decode_step_attn(R(q), R(kn), R(vn), R(kc), R(vc), R(bt), R(cl), scale, ks, vs, ws, ws_bytes,
                                        R(out), None)


def test_decode_step_rejects_bad_new_rows():
    kc, vc = caches()
    q, out, bt, cl = T([2, 4, 64], F16), T([2, 4, 64], F16), T([2, 4], I32), T([2], I32)
    good = T([2, 2, 64], F16)
    assert step(q, None, good, kc, vc, bt, cl, out) == 1 and "k_new" in err()
    assert step(q, good, None, kc, vc, bt, cl, out) == 1 and "v_new" in err()
    assert step(q, T([2, 2, 64], F32), good, kc, vc, bt, cl, out) == 2 and "cache dtype" in err()
    assert step(q, T([3, 2, 64], F16), T([3, 2, 64], F16), kc, vc, bt, cl, out) == 3
    assert step(q, T([2, 2, 64], F16), T([2, 1, 64], F16), kc, vc, bt, cl, out) == 3
    assert step(q, T([2, 2, 64], F16, ptr=FAKE + 2), good, kc, vc, bt, cl, out) == 4
    # an fp8 cache takes the rows in the q dtype, quantized like pkv_append
    kc8, vc8 = caches(dt=FP8)
    assert step(q, good, good, kc8, vc8, bt, cl, out) == 6  # rows accepted; no workspace given
    assert step(T([2, 4, 64], BF16), good, good, kc8, vc8, bt, cl, T([2, 4, 64], BF16)) == 2 and "q dtype" in err()


def test_missing_library_fails_loudly(tmp_path):
    """Without libpkv.so the package refuses to import: there is no CPU path to
    fall back to."""
    import shutil
    import subprocess
    import sys

    pkg = tmp_path / "prefix_reuse_amd"
    pkg.mkdir()
    src = Path(pkv.__file__).parent
    for f in src.glob("*.py"):
        shutil.copy(f, pkg / f.name)  # the package without its built library
    import os

    env = {k: v for k, v in os.environ.items() if k != "PKV_LIBRARY"}
    res = subprocess.run([sys.executable, "-c", "import prefix_reuse_amd"], cwd=tmp_path, capture_output=True,
                         text=True, timeout=120, env=env)
    assert res.returncode != 0
    assert "ImportError" in res.stderr and "There is no CPU fallback" in res.stderr


def test_noalloc_decode_rejects_a_batch_beyond_its_scratch_before_launch():
    """pkv_decode_attn_noalloc keeps its partial results in a fixed 32 MiB
    device array; a batch that needs more is refused on the host."""
    kc, vc = caches(h=8, d=128)
    s = 4000
    rc = pkv.lib.pkv_decode_attn_noalloc(R(T([s, 32, 128], F16)), R(kc), R(vc), R(T([s, 4], I32)), R(T([s], I32)),
                                         0.1, 1.0, 1.0, R(T([s, 32, 128], F16)), None)
    assert rc == 6 and "scratch" in err()
