#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X.

One step = one serving step of the decode workload in one call
(pkv_decode_step_attn): the newest token's K and V of every sequence go into
the cache and each query attends to the whole cache, as pkv_append followed
by pkv_decode_attn would do. Workload: batch 64, 32 query / 8 KV heads, head
dim 128, fp16 KV, 16-token blocks, context lengths uniform in [512, 4096],
physical blocks shuffled (Llama-3-8B-shaped single layer).

Printed as one JSON line:
  value      decode KV-read GB/s = K+V bytes the step must read / step time
  roofline   the decode call's own duration (HIP events on its stream)
             against the HBM peak; traffic from rocprofv3 counters when they
             match the current kernel sources (else null)
  step_roofline  the same for the step's one call (the value's own kernels)
  suffix_prefill  the same for the suffix-prefill workload (16 requests x
             1,900 cached + 100 new tokens, bf16): TFLOP/s against bf16 MFMA
             peak, timed cold (inputs evicted) and warm
  suffix_prefill_fp8_kv  the same workload over an fp8 e4m3fn cache
  suffix_prefill_next_turn  one conversation's next turn (1 request, 8,000
             cached + 100 new tokens), the key-split call against the plain one
  shared_prefix_decode  256 sequences on one 1,000-token shared prefix
             (cascade decode), GB/s of unique KV bytes against the HBM peak
  long_context_fp8  8 sequences x 100,000 tokens x 32 layers with an fp8
             e4m3fn cache: append + decode for every layer per step, GB/s of
             KV read, and one layer's decode call against the HBM peak
  cpu_baseline    the CPU oracle timed on this host's cores (one core, and N worker
             processes) on the decode, suffix-prefill and long-context workloads
  measured_peaks  ceilings this GPU reaches with probe kernels (stream read, 4 KiB
             tile gather, bf16 MFMA loop, and the shader clock under that loop);
             each roofline also gives its fraction of the measured ceiling
  clocks_rocm_smi  rocm-smi's clock readout, sampled while the decode step runs

Inputs are synthetic (seeded N(0,1)), resident in HBM before timing starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak
# the device code and the launch planning behind every profiled kernel
KERNEL_SOURCES = [f"prefix_reuse_amd/csrc/{f}" for f in (
    "pkv_decode.hip", "pkv_decode_body.hpp", "pkv_prefill.hip", "pkv_prefill_body.hpp", "pkv_cascade.hip",
    "pkv_device.hpp", "pkv_internal.hpp", "pkv_append.hip", "pkv_api.hip")]


def sources_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update((ROOT / f).read_bytes())
    return h.hexdigest()[:16]


def load_traffic(name: str, files) -> dict | None:
    """Counter-based HBM traffic per launch, if it was taken on these sources."""
    p = ROOT / "profiles" / f"{name}_traffic.json"
    if not p.exists():
        return None
    rec = json.loads(p.read_text())
    if rec.get("sources_hash") != sources_hash(files):
        return None
    return rec


def warm_clocks(torch, fn, seconds=0.5):
    """Untimed launches for a fixed wall time, so that the timed region does
    not start on a GPU still raising its clocks."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def smi_clocks(torch, fn, limit_s=20.0):
    """Clocks as rocm-smi reports them (`--showclocks --json`), sampled in a
    child process while fn runs back to back; None if the tool is missing or
    prints no JSON."""
    try:
        proc = subprocess.Popen(["rocm-smi", "--showclocks", "--json"], stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t0 = time.perf_counter()
    while proc.poll() is None and time.perf_counter() - t0 < limit_s:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    try:
        text, _ = proc.communicate(timeout=max(1.0, limit_s - (time.perf_counter() - t0)))
    except subprocess.TimeoutExpired:
        proc.kill()
        proc.communicate()
        return None
    i = text.find("{")
    if proc.returncode != 0 or i < 0:
        return None
    try:
        return json.loads(text[i:])
    except ValueError:
        return None


def time_launches(torch, stream, fn, n) -> float:
    """Average milliseconds per launch of fn over n back-to-back launches,
    from HIP events recorded on the launch stream around the whole region."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def decode_setup(torch, pkv, workloads, dev):
    case = workloads.config2_llama_decode()
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, dev)
    t = {
        "case": case, "kc": kc, "vc": vc,
        "q": case.q.to(dev), "bt": case.block_tables.to(dev), "cl": case.context_lens.to(dev),
        "k_new": case.k_new.to(dev), "v_new": case.v_new.to(dev), "slots": case.slot_mapping.to(dev),
    }
    t["out"] = torch.empty_like(t["q"])
    need = pkv.decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                      case.block_tables.shape[1], case.block_size)
    t["ws"] = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
    pkv.append(t["k_new"], t["v_new"], t["slots"], kc, vc)  # the newest token, as a step does
    torch.cuda.synchronize()
    return t


def prefill_setup(torch, pkv, workloads, dev):
    case = workloads.config4_suffix_prefill()
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, dev)
    t = {
        "case": case, "kc": kc, "vc": vc, "q": case.q_suffix.to(dev), "bt": case.block_tables.to(dev),
        "pl": case.prefix_lens.to(dev), "sl": case.suffix_lens.to(dev),
        "k_new": case.k_new.to(dev), "v_new": case.v_new.to(dev), "slots": case.slot_mapping.to(dev),
    }
    t["out"] = torch.empty_like(t["q"])
    # the suffix K/V go into the cache first, as in the pages' flow (the slots
    # hold the pool's NaN poison until then)
    pkv.append(t["k_new"], t["v_new"], t["slots"], kc, vc)
    torch.cuda.synchronize()
    return t


def next_turn_setup(torch, pkv, workloads, dev):
    """One conversation's next turn (one request, 8,000 cached + 100 new
    tokens), with the key-split call's workspace."""
    case = workloads.next_turn_suffix_prefill()
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, dev)
    t = {"case": case, "kc": kc, "vc": vc, "q": case.q_suffix.to(dev), "bt": case.block_tables.to(dev),
         "pl": case.prefix_lens.to(dev), "sl": case.suffix_lens.to(dev)}
    t["out"] = torch.empty_like(t["q"])
    pkv.append(case.k_new.to(dev), case.v_new.to(dev), case.slot_mapping.to(dev), kc, vc)
    need = pkv.suffix_prefill_workspace_bytes(case.q_suffix.shape[0], 1, case.num_q_heads, case.num_kv_heads,
                                              case.head_dim, case.block_tables.shape[1], case.block_size)
    t["ws"] = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    t["ws_bytes"] = need
    torch.cuda.synchronize()
    return t


def run_next_turn_split(pkv, t):
    c = t["case"]
    pkv.suffix_prefill_attn_split(t["q"], t["kc"], t["vc"], t["bt"], t["pl"], t["sl"], c.scale, out=t["out"],
                                  workspace=t["ws"])


def run_next_turn_plain(pkv, t):
    c = t["case"]
    pkv.suffix_prefill_attn(t["q"], t["kc"], t["vc"], t["bt"], t["pl"], t["sl"], c.scale, out=t["out"])


def prefill_fp8_setup(torch, pkv, workloads, dev):
    """The same suffix-prefill workload over an fp8 e4m3fn cache: every cached
    row and every suffix row is quantized through pkv_append (scale = amax/448
    for K and for V); q and the output stay bf16."""
    import numpy as np

    case = workloads.config4_suffix_prefill()
    nb, b, h, d = case.k_pool.shape
    kc, vc = pkv.empty_caches(nb, b, h, d, torch.float8_e4m3fn, dev)
    kc.view(torch.uint8).fill_(workloads.fp8_nan_code)
    vc.view(torch.uint8).fill_(workloads.fp8_nan_code)
    live = (~torch.isnan(case.k_pool[:, :, 0, 0].float())).nonzero()
    slots = torch.cat([live[:, 0] * b + live[:, 1], case.slot_mapping]).to(dev)
    rows = {w: torch.cat([pool[live[:, 0], live[:, 1]], new]).to(dev)
            for w, pool, new in (("k", case.k_pool, case.k_new), ("v", case.v_pool, case.v_new))}
    sc = {w: float(np.float32(rows[w].float().abs().max().item()) / np.float32(448.0)) for w in rows}
    pkv.append(rows["k"], rows["v"], slots, kc, vc, sc["k"], sc["v"])
    t = {"case": case, "kc": kc, "vc": vc, "q": case.q_suffix.to(dev), "bt": case.block_tables.to(dev),
         "pl": case.prefix_lens.to(dev), "sl": case.suffix_lens.to(dev), "ks": sc["k"], "vs": sc["v"]}
    t["out"] = torch.empty_like(t["q"])
    del rows
    torch.cuda.synchronize()
    return t


def run_prefill_fp8_call(pkv, t):
    c = t["case"]
    pkv.suffix_prefill_attn(t["q"], t["kc"], t["vc"], t["bt"], t["pl"], t["sl"], c.scale, out=t["out"],
                            k_scale=t["ks"], v_scale=t["vs"])


def long_context_setup(torch, pkv, workloads, dev, num_layers=32):
    """Per-layer fp8 caches of the long-context workload, every token quantized
    through pkv_append from N(0,1) rows drawn on the device (scale = amax/448
    per layer for K and for V)."""
    import numpy as np

    case = workloads.config5_long_context_fp8(num_layers=num_layers)
    n = case.context_len
    layers = []
    for layer in range(num_layers):
        kc, vc = pkv.empty_caches(case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim,
                                  torch.float8_e4m3fn, dev)
        kc.view(torch.uint8).fill_(workloads.fp8_nan_code)
        vc.view(torch.uint8).fill_(workloads.fp8_nan_code)
        amax = {"k": 0.0, "v": 0.0}
        for sq in range(case.num_seqs):
            for w in amax:
                amax[w] = max(amax[w], float(case.raw_kv(layer, sq, dev, w).abs().max().item()))
        ks = float(np.float32(amax["k"]) / np.float32(448.0))
        vs = float(np.float32(amax["v"]) / np.float32(448.0))
        for sq in range(case.num_seqs):
            pkv.append(case.raw_kv(layer, sq, dev, "k"), case.raw_kv(layer, sq, dev, "v"),
                       case.slots(sq, 0, n).to(dev), kc, vc, ks, vs)
        layers.append({"kc": kc, "vc": vc, "ks": ks, "vs": vs, "q": case.raw_q(layer, dev),
                       "k_new": case.raw_new(layer, dev, "k"), "v_new": case.raw_new(layer, dev, "v")})
    t = {"case": case, "layers": layers, "bt": case.block_tables.to(dev),
         "cl": torch.full((case.num_seqs,), n, dtype=torch.int32, device=dev),
         "last_slots": torch.cat([case.slots(sq, n - 1, n) for sq in range(case.num_seqs)]).to(dev)}
    t["out"] = torch.empty_like(layers[0]["q"])
    need = pkv.decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                      case.block_tables.shape[1], case.block_size)
    t["ws"] = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    return t


def run_long_context_decode(pkv, t, lay):
    c = t["case"]
    pkv.decode_attn(lay["q"], lay["kc"], lay["vc"], t["bt"], t["cl"], c.scale, out=t["out"],
                    k_scale=lay["ks"], v_scale=lay["vs"], workspace=t["ws"])


def run_long_context_step(pkv, t):
    """One decode step of the whole model's attention: per layer, write the
    newest token's K, V (position 99,999, quantized to fp8) and attend over all
    100,000, in one call."""
    c = t["case"]
    for lay in t["layers"]:
        pkv.decode_step_attn(lay["q"], lay["k_new"], lay["v_new"], lay["kc"], lay["vc"], t["bt"], t["cl"], c.scale,
                             out=t["out"], k_scale=lay["ks"], v_scale=lay["vs"], workspace=t["ws"])


def run_decode_call(pkv, t):
    c = t["case"]
    pkv.decode_attn(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], c.scale, out=t["out"], workspace=t["ws"])


def run_decode_step(pkv, t):
    """A whole decode step in one call: append each sequence's newest K, V and
    attend over its full context."""
    c = t["case"]
    pkv.decode_step_attn(t["q"], t["k_new"], t["v_new"], t["kc"], t["vc"], t["bt"], t["cl"], c.scale, out=t["out"],
                         workspace=t["ws"])


def shared_prefix_setup(torch, pkv, workloads, dev):
    """256 sequences on one 1,000-token system prompt (31 aliased 32-token
    blocks), bf16: one group for the cascade decode."""
    case = workloads.config3_shared_prefix_decode()
    kc, vc = pkv.caches_from_logical(case.k_pool, case.v_pool, dev)
    pkv.append(case.k_new.to(dev), case.v_new.to(dev), case.slot_mapping.to(dev), kc, vc)
    t = {"case": case, "kc": kc, "vc": vc, "q": case.q.to(dev), "bt": case.block_tables.to(dev),
         "cl": case.context_lens.to(dev),
         "gs": torch.tensor([0, case.num_seqs], dtype=torch.int32, device=dev),
         "sl": torch.full((case.num_seqs,), case.shared_blocks * case.block_size, dtype=torch.int32, device=dev)}
    t["out"] = torch.empty_like(t["q"])
    need = max(pkv.cascade_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim),
               pkv.decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                          case.block_tables.shape[1], case.block_size))
    t["ws"] = torch.zeros(need, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    return t


def run_cascade_call(pkv, t):
    c = t["case"]
    pkv.cascade_decode_attn(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], t["gs"], t["sl"], c.scale, out=t["out"],
                            workspace=t["ws"])


def run_prefill_call(pkv, t):
    c = t["case"]
    pkv.suffix_prefill_attn(t["q"], t["kc"], t["vc"], t["bt"], t["pl"], t["sl"], c.scale, out=t["out"])


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as written, on this host's cores. It runs before
# anything touches the GPU, so that its worker processes fork from a process
# with no GPU state. Each leg is timed on one core (BLAS limited to one
# thread) and over N worker processes (one BLAS thread each), N = the cores
# this process may use, at most 16 (one GPU's share of the host).
# ---------------------------------------------------------------------------
_CPU = {}  # the work of the leg being timed, inherited by the forked workers


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _run_units(units):
    fn = _CPU["fn"]
    work = 0.0
    for u in units:
        work += fn(u)
    return work


def _time_oracle(fn, units, seconds, max_procs):
    """(1-core work/s, N-process work/s, N, details). fn(unit) runs the oracle
    on one unit of the leg and returns the unit's work (bytes or FLOP)."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    _CPU["fn"] = fn
    # one core: units in order until `seconds` of work
    done, work, t0 = 0, 0.0, time.perf_counter()
    with threadpool_limits(1):
        while True:
            work += fn(units[done % len(units)])
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
    t1 = time.perf_counter() - t0
    rate1 = work / t1
    # N processes, each on about `seconds` worth of units
    n = max(1, min(max_procs, len(os.sched_getaffinity(0))))
    per = max(1, int(round(done * 1.0)))
    batches = [[units[(w * per + i) % len(units)] for i in range(per)] for w in range(n)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(n, initializer=_one_blas_thread) as pool:
        works = pool.map(_run_units, batches, chunksize=1)
    tn = time.perf_counter() - t0
    return rate1, sum(works) / tn, n, {"units_one_core": done, "seconds_one_core": round(t1, 2),
                                       "units_per_process": per, "seconds_n_procs": round(tn, 2)}


def cpu_baselines(seconds=4.0, max_procs=16) -> dict:
    """The oracle on the three timed workloads: the Llama decode (KV GB/s),
    the suffix prefill (TFLOP/s) and one layer of the long-context fp8 decode
    (GB/s, extrapolated to the 32-layer step's rate: every layer costs the
    same)."""
    import numpy as np
    import torch

    import oracle
    import workloads

    out = {}
    # --- Llama-3-8B-shaped decode: one unit = one sequence's decode --------
    case = workloads.config2_llama_decode()
    kc, vc = oracle.append(case.k_pool.double().numpy(), case.v_pool.double().numpy(), case.k_new.double().numpy(),
                           case.v_new.double().numpy(), case.slot_mapping.numpy())
    q, bt, cl = case.q.double().numpy(), case.block_tables.numpy(), case.context_lens.numpy()
    per_tok = 2 * case.num_kv_heads * case.head_dim * case.k_pool.element_size()

    def dec_unit(s):
        oracle.decode_attention(q, kc, vc, bt, cl, case.scale, seqs=[s])
        return float(cl[s]) * per_tok

    r1, rn, n, det = _time_oracle(dec_unit, list(range(case.num_seqs)), seconds, max_procs)
    out["decode"] = {"value": round(rn / 1e9, 4), "unit": "GB/s", "cores": n, "one_core": round(r1 / 1e9, 4),
                     "details": det,
                     "sample": "float64 NumPy oracle decode of the 64-sequence Llama-3-8B-shaped batch (fp16 KV), "
                               "one unit = one sequence, KV bytes counted as in the GPU metric; the oracle's "
                               "append (a copy of the whole pool) is done once beforehand and not timed"}
    del kc, vc
    # --- suffix prefill: one unit = one suffix row (all 32 heads) ----------
    pc = workloads.config4_suffix_prefill()
    kc, vc = oracle.append(pc.k_pool.double().numpy(), pc.v_pool.double().numpy(), pc.k_new.double().numpy(),
                           pc.v_new.double().numpy(), pc.slot_mapping.numpy())
    qs, pbt = pc.q_suffix.double().numpy(), pc.block_tables.numpy()
    pl, sl = pc.prefix_lens.numpy(), pc.suffix_lens.numpy()
    starts = np.concatenate([[0], np.cumsum(sl)[:-1]])

    def row_flops(row):
        r = int(np.searchsorted(starts, row, side="right") - 1)
        return 4.0 * pc.head_dim * pc.num_q_heads * (int(pl[r]) + (row - int(starts[r])) + 1)

    def pre_unit(row):
        oracle.suffix_prefill_attention(qs, kc, vc, pbt, pl, sl, pc.scale, rows=[row])
        return row_flops(row)

    rng = np.random.default_rng(11)
    rows = rng.permutation(int(sl.sum())).tolist()
    r1, rn, n, det = _time_oracle(pre_unit, rows, seconds, max_procs)
    out["suffix_prefill"] = {"value": round(rn / 1e12, 6), "unit": "TFLOP/s", "cores": n,
                             "one_core": round(r1 / 1e12, 6), "details": det,
                             "sample": "float64 NumPy oracle suffix prefill of the 16 x (1,900 + 100) bf16 workload, "
                                       "one unit = one suffix row (32 heads, all its visible keys), rows in seeded "
                                       "random order, FLOP counted as in the GPU metric"}
    del kc, vc
    # --- long-context fp8: one unit = one sequence of one layer ------------
    lc = workloads.config5_long_context_fp8()
    n_tok, b, h, d = lc.context_len, lc.block_size, lc.num_kv_heads, lc.head_dim
    g = torch.Generator().manual_seed(lc.base_seed)
    codes = {}
    for w in ("k", "v"):
        x = torch.randn(n_tok, h, d, generator=g)
        sc = float(np.float32(x.abs().max().item()) / np.float32(448.0))
        codes[w] = ((x / sc).to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(n_tok // b, b, h, d), sc)
        del x
    ql = torch.randn(1, lc.num_q_heads, d, generator=g).to(torch.bfloat16).double().numpy()
    ident = np.arange(n_tok // b)[None, :]

    def long_unit(_):
        oracle.decode_attention(ql, codes["k"][0], codes["v"][0], ident, np.array([n_tok]), lc.scale, fp8=True,
                                k_scale=codes["k"][1], v_scale=codes["v"][1])
        return float(n_tok) * 2 * h * d  # fp8: one byte per element

    r1, rn, n, det = _time_oracle(long_unit, list(range(lc.num_seqs)), seconds, min(max_procs, lc.num_seqs))
    out["long_context_fp8"] = {"value": round(rn / 1e9, 4), "unit": "GB/s", "cores": n,
                               "one_core": round(r1 / 1e9, 4), "details": det, "extrapolated": True,
                               "step_seconds_extrapolated": round(lc.kv_read_bytes_per_layer() * lc.num_layers / rn, 1),
                               "sample": "float64 NumPy oracle decode of one 100,000-token sequence of one layer "
                                         "(fp8 e4m3fn codes of N(0,1) rows quantized with scale amax/448, drawn "
                                         "on the host), 32 query heads; the 8-sequence, 32-layer step costs 256 "
                                         "such units, so its time is extrapolated from this rate"}
    del codes
    primary = out["decode"]
    return {
        "value": primary["value"], "unit": "GB/s", "cores": primary["cores"], "kind": "oracle",
        "sample": primary["sample"], "one_core": primary["one_core"],
        "cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
        "legs": {"suffix_prefill": out["suffix_prefill"], "long_context_fp8": out["long_context_fp8"]},
        "decode_details": primary["details"],
    }


def ingest_profile(name: str, trace_dir: str, fetch_dir: str, write_dir: str, kernel_regex: str,
                   command: str, last: int = 20) -> None:
    """Summarise rocprofv3 csv output (a kernel-trace --stats run and two
    --pmc runs, FETCH_SIZE then WRITE_SIZE) into profiles/<name>.md and
    profiles/<name>_traffic.json. Counters are calibrated by the 1 GiB device
    copy that `--only` runs end with: factor = true bytes / counter bytes."""
    import csv
    import re

    rx = re.compile(kernel_regex)

    def find(d, suffix):
        hits = sorted(Path(d).rglob(f"*{suffix}"))
        if not hits:
            raise FileNotFoundError(f"no *{suffix} under {d}")
        return hits[0]

    stats = list(csv.DictReader(open(find(trace_dir, "kernel_stats.csv"))))
    # the measured launches: the last `last` dispatches of each matched kernel
    trace = list(csv.DictReader(open(find(trace_dir, "kernel_trace.csv"))))
    by_kernel = {}
    for r in sorted(trace, key=lambda r: int(r["Start_Timestamp"])):
        if rx.search(r["Kernel_Name"]):
            by_kernel.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    measured_ns = sum(sum(v[-last:]) / len(v[-last:]) for v in by_kernel.values())
    lines = [f"# {name}", "", "rocprofv3 summaries (MI355X, gfx950). Commands, run from /tmp with TMPDIR=/tmp:", "",
             "```", command, "```", "", "## Kernel trace (--kernel-trace --stats)", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    total_avg_ns = 0.0
    for r in stats:
        short = r["Name"][:110]
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                     f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} |")
        if rx.search(r["Name"]):
            total_avg_ns += float(r["AverageNs"])
    counters = {}
    for label, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = list(csv.DictReader(open(find(d, "counter_collection.csv"))))
        copy = [r for r in rows if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) >= 65536]
        copy_kib = float(copy[-1]["Counter_Value"]) if copy else float("nan")
        factor = (1 << 20) / copy_kib  # the copy moves 1 GiB = 2^20 KiB each way
        per = {}
        for r in rows:
            if rx.search(r["Kernel_Name"]):
                per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        counters[label] = (factor, copy_kib, {k: sum(v) / len(v) for k, v in per.items()})
    lines += ["", "## HBM traffic (--pmc, one counter per run)", "",
              "Calibration: the same counter over a plain 1 GiB device-to-device copy.", "",
              "| counter | copy reads as KiB | factor | kernel | KiB per dispatch (raw) | MB per dispatch (calibrated) |",
              "|---|---|---|---|---|---|"]
    total_bytes = 0.0
    parts = {}
    for label, (factor, copy_kib, per) in counters.items():
        for k, v in per.items():
            mb = v * factor * 1024 / 1e6
            total_bytes += v * factor * 1024
            parts[f"{label}:{k[:60]}"] = round(v * factor * 1024)
            lines.append(f"| {label} | {copy_kib:.0f} | {factor:.3f} | `{k[:60]}` | {v:.0f} | {mb:.2f} |")
    lines += ["", "## Measured launches", "",
              f"Average over the last {last} launches of each matched kernel (the ones after the clock warm-up, "
              f"as timed in the benchmark): {measured_ns/1e3:.2f} us per launch (sum over the matched kernels); "
              f"over all launches, warm-up included: {total_avg_ns/1e3:.2f} us.", "",
              f"Sum over the matched kernels: HBM traffic {total_bytes/1e6:.2f} MB per launch.", ""]
    (ROOT / "profiles").mkdir(exist_ok=True)
    (ROOT / "profiles" / f"{name}.md").write_text("\n".join(lines))
    rec = {"name": name, "kernel_regex": kernel_regex, "sources_hash": sources_hash(KERNEL_SOURCES),
           "avg_launch_us": round(measured_ns / 1e3, 3), "avg_launch_us_all": round(total_avg_ns / 1e3, 3),
           "bytes_per_launch": round(total_bytes),
           "parts": parts, "command": command}
    (ROOT / "profiles" / f"{name}_traffic.json").write_text(json.dumps(rec, indent=1) + "\n")
    print(f"wrote profiles/{name}.md and profiles/{name}_traffic.json")


def time_cold(torch, stream, fn, n, scrub, write=False):
    """Milliseconds per launch of fn when it starts on cold caches: each launch
    follows a 1 GiB scrub (four times the 256 MB MALL) on the same stream, so
    nothing the previous launch left in L2 or the MALL survives. The scrubs are
    timed alone and subtracted: scrub and launch run back to back as in the
    warm timing, so no launch is timed in isolation (an isolated launch adds
    ~10 us of dispatch latency that back-to-back launches hide). The scrub
    reads the 1 GiB, leaving the caches full of clean lines; with write=True it
    writes them instead, and the launch also pays for writing back the scrub's
    dirty lines it evicts."""

    def scrub_once(i):
        if write:
            scrub.fill_(i & 0xFF)
        else:
            scrub.sum(dtype=torch.int64)

    def region(with_fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            scrub_once(i)
            if with_fn:
                fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1)

    region(True)  # warm-up of both kernels
    best = None
    for _ in range(3):  # three rounds of (scrubs alone, scrubs + launches); the smallest difference wins
        t_s = region(False)
        t_sf = region(True)
        d = (t_sf - t_s) / n
        best = d if best is None else min(best, d)
    return best


def measured_peaks(torch, dev, stream) -> dict:
    """Ceilings this device reaches with the probe kernels of libpkv_peak.so:
    a streaming read of 4 GiB, random whole 4 KiB tiles (the decode's access
    pattern) over 2 GiB, and back-to-back bf16 32x32x16 matrix products on
    every SIMD. Each is the best of several timed launches (HIP events on the
    launch stream)."""
    import ctypes

    lib = ctypes.CDLL(str(ROOT / "prefix_reuse_amd" / "libpkv_peak.so"))
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.pkv_peak_stream_read.argtypes = [vp, i64, vp, i32, vp]
    lib.pkv_peak_tile_gather.argtypes = [vp, i64, vp, i32, vp, i32, vp]
    lib.pkv_peak_mfma_bf16.argtypes = [i32, i32, vp, vp, vp]
    for f in (lib.pkv_peak_stream_read, lib.pkv_peak_tile_gather, lib.pkv_peak_mfma_bf16):
        f.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    hs = stream.cuda_stream

    def best(fn, reps=8):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = fn()
            e1.record(stream)
            e1.synchronize()
            assert rc == 0, f"probe launch failed ({rc})"
            t.append(e0.elapsed_time(e1))
        return min(t)

    out = {}
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    ms = best(lambda: lib.pkv_peak_stream_read(buf.data_ptr(), buf.numel(), sink.data_ptr(), cus * 16, hs))
    out["stream_read_gbs"] = round(buf.numel() / (ms * 1e-3) / 1e9, 1)
    tiles = (2 << 30) // 4096
    ids = torch.randperm(tiles, device=dev).to(torch.int32)
    ms = best(lambda: lib.pkv_peak_tile_gather(buf.data_ptr(), tiles, ids.data_ptr(), tiles, sink.data_ptr(),
                                               cus * 8, hs))
    out["tile_gather_4k_gbs"] = round(tiles * 4096 / (ms * 1e-3) / 1e9, 1)
    del buf, ids
    torch.cuda.empty_cache()
    blocks, iters = cus * 4, 4000
    clock = torch.zeros(2, dtype=torch.int64, device=dev)
    ms = best(lambda: lib.pkv_peak_mfma_bf16(blocks, iters, sink.data_ptr(), clock.data_ptr(), hs), reps=5)
    flops = blocks * 4 * 4 * iters * 32768
    out["mfma_bf16_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
    cycles, ticks = (int(x) for x in clock.cpu().tolist())  # the last launch's first wave
    if ticks > 0:
        # shader clock under full matrix load, and the MFMA rate it allows
        # (1,024 FLOP per cycle per SIMD, 4 SIMDs per CU)
        ghz = cycles / (ticks * 10.0)
        out["shader_clock_ghz_under_mfma"] = round(ghz, 3)
        out["mfma_bf16_tflops_at_that_clock"] = round(cus * 4 * 1024 * ghz * 1e9 / 1e12, 1)
    out["probe"] = ("libpkv_peak.so: 4 GiB streamed once with 16-byte loads; 524,288 random 4 KiB tiles of a "
                    "2 GiB buffer, one wave per tile, 8 waves per CU; 16 waves per CU each issuing "
                    f"{4 * iters} v_mfma_f32_32x32x16_bf16 in 4 independent chains; best of several launches")
    return out


def with_measured(roof: dict, peak) -> dict:
    """Add the fraction of the measured ceiling next to the spec fraction."""
    if peak:
        roof["measured_peak"] = peak
        roof["frac_of_measured"] = round(roof["achieved"] / peak, 4)
    return roof


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-long-context", action="store_true")
    ap.add_argument("--no-shared-prefix", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-ceiling probes")
    ap.add_argument("--only", choices=["decode", "step", "prefill", "prefill_fp8", "turn", "long", "shared"],
                    default=None,
                    help="run only this kernel's launches (for profiler runs)")
    ap.add_argument("--ingest-profile", nargs=5, metavar=("NAME", "TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "KERNEL_REGEX"),
                    help="summarise rocprofv3 csv output into profiles/ (no GPU needed)")
    ap.add_argument("--profile-command", default="", help="command text recorded with --ingest-profile")
    ap.add_argument("--ingest-last", type=int, default=20, help="measured launches per kernel in the trace")
    args = ap.parse_args()
    if args.ingest_profile:
        ingest_profile(*args.ingest_profile, command=args.profile_command, last=args.ingest_last)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    cpu = None
    if args.only is None and not args.no_cpu_baseline:
        cpu = cpu_baselines()  # before the GPU is touched: its workers fork from this process

    import torch

    import prefix_reuse_amd as pkv
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.only is not None:
        setup = {"decode": decode_setup, "step": decode_setup, "prefill": prefill_setup,
                 "prefill_fp8": prefill_fp8_setup, "turn": next_turn_setup, "long": long_context_setup,
                 "shared": shared_prefix_setup}[args.only]
        call = {"decode": run_decode_call, "step": run_decode_step, "prefill": run_prefill_call,
                "prefill_fp8": run_prefill_fp8_call, "turn": run_next_turn_split,
                "long": lambda pkv, t: run_long_context_decode(pkv, t, t["layers"][0]),
                "shared": run_cascade_call}[args.only]
        t = setup(torch, pkv, workloads, dev) if args.only != "long" else setup(torch, pkv, workloads, dev, 1)
        for _ in range(args.warmup):
            call(pkv, t)
        warm_clocks(torch, lambda: call(pkv, t))
        for _ in range(args.steps):  # the last `steps` launches are the measured ones
            call(pkv, t)
        torch.cuda.synchronize()
        # a plain copy of known size, to calibrate the memory counters
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "measured_launches": args.steps, "copy_bytes": 1 << 30}))
        return 0

    peaks = {} if args.no_peaks else measured_peaks(torch, dev, stream)
    hbm_meas = peaks.get("stream_read_gbs")
    mfma_meas = peaks.get("mfma_bf16_tflops")

    # ---------------- decode step: append + decode, one call ----------------
    t = decode_setup(torch, pkv, workloads, dev)
    case = t["case"]

    def step():
        run_decode_step(pkv, t)

    def step_two_calls():
        pkv.append(t["k_new"], t["v_new"], t["slots"], t["kc"], t["vc"])
        run_decode_call(pkv, t)

    for _ in range(args.warmup):
        step()
    warm_clocks(torch, step)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    kv_bytes = case.kv_read_bytes()
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9

    clocks = smi_clocks(torch, step)
    # the same step as two calls (pkv_append, then pkv_decode_attn)
    two_ms = time_launches(torch, stream, step_two_calls, args.steps)
    # the decode call alone (its two kernels), back to back on its stream
    dec_ms = time_launches(torch, stream, lambda: run_decode_call(pkv, t), args.steps)
    dec_gbs = kv_bytes / (dec_ms * 1e-3) / 1e9
    traffic = load_traffic("decode_llama3_8b_b64_fp16", KERNEL_SOURCES)
    step_traffic = load_traffic("decode_step_llama3_8b_b64_fp16", KERNEL_SOURCES)
    roofline = {
        "kernel": "pkv_decode_attn (decode_kernel + decode_combine_kernel)",
        "bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
        "traffic": None if traffic is None else traffic["bytes_per_launch"],
        "avg_launch_us": round(dec_ms * 1e3, 2), "algorithmic_bytes_per_launch": kv_bytes,
    }
    with_measured(roofline, hbm_meas)
    if peaks:
        roofline["frac_of_measured_tile_gather"] = round(dec_gbs / peaks["tile_gather_4k_gbs"], 4)

    result = {
        "metric": "decode KV-read GB/s (% HBM peak) + suffix-prefill TFLOP/s (% MFMA), 1 GPU",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "llama3-8b-shaped decode step: append 1 token/seq + paged decode attention "
                               "(pkv_decode_step_attn, one call)",
                   "batch": case.num_seqs, "q_heads": case.num_q_heads, "kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "block_size": case.block_size, "kv_dtype": "fp16",
                   "context_lens": "uniform [512, 4096], seed 1002", "kv_bytes_per_step": kv_bytes,
                   "tokens_per_step": case.num_seqs},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(case.num_seqs / (ms_per_step * 1e-3), 1),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "step_as_two_calls_us": round(two_ms * 1e3, 2),
        "roofline": roofline,
        "step_roofline": with_measured({
            "kernel": "pkv_decode_step_attn (decode_kernel in its step form + decode_combine_kernel)",
            "bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4),
            "traffic": None if step_traffic is None else step_traffic["bytes_per_launch"],
            "avg_launch_us": round(ms_per_step * 1e3, 2), "algorithmic_bytes_per_launch": kv_bytes}, hbm_meas),
        "measured_peaks": peaks or None,
        "clocks_rocm_smi": None if clocks is None else {
            "sampled": "rocm-smi --showclocks --json, run while the decode step ran back to back",
            "reading": clocks},
    }

    # ---------------- suffix prefill: append suffix + prefill ----------------
    if not args.no_prefill:
        del t
        torch.cuda.empty_cache()
        p = prefill_setup(torch, pkv, workloads, dev)
        pc = p["case"]
        for _ in range(args.warmup):
            run_prefill_call(pkv, p)
        warm_clocks(torch, lambda: run_prefill_call(pkv, p))
        warm_ms = time_launches(torch, stream, lambda: run_prefill_call(pkv, p), args.steps)
        # cold: back-to-back launches rotating over four copies of the inputs (~600 MB, more than twice the
        # 256 MB MALL), so each launch finds its KV cache, q and out evicted by the other copies' traffic
        copies = [p] + [dict(p, kc=p["kc"].clone(), vc=p["vc"].clone(), q=p["q"].clone(),
                             out=torch.empty_like(p["out"])) for _ in range(3)]
        rot = iter(range(1 << 30))
        rot_call = lambda: run_prefill_call(pkv, copies[next(rot) % len(copies)])
        for _ in range(8):
            rot_call()
        cold_ms = time_launches(torch, stream, rot_call, max(4 * (args.steps // 4), 20))
        del copies
        torch.cuda.empty_cache()
        scrub = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
        rcold_ms = time_cold(torch, stream, lambda: run_prefill_call(pkv, p), max(10, args.steps // 5), scrub)
        wcold_ms = time_cold(torch, stream, lambda: run_prefill_call(pkv, p), max(10, args.steps // 5), scrub, True)
        del scrub
        pre_ms = cold_ms  # the headline: caches cold, as a prefill after other work finds them
        flops = pc.flops()
        tflops = flops / (pre_ms * 1e-3) / 1e12
        warm_tflops = flops / (warm_ms * 1e-3) / 1e12
        ptraffic = load_traffic("prefill_16x1900p100_bf16", KERNEL_SOURCES)
        result["suffix_prefill"] = {
            "metric": "suffix-prefill TFLOP/s", "value": round(tflops, 2), "unit": "TFLOP/s",
            "timing": "cold: back-to-back launches rotating over four copies of the inputs (KV cache, q, out; "
                      "~600 MB), so no launch finds its inputs in L2 or the 256 MB MALL",
            "config": {"workload": "16 requests x (1,900 cached + 100 new tokens), 32/8 heads, d=128, bf16, B=16",
                       "flop_per_launch": flops, "suffix_tokens": int(pc.suffix_lens.sum())},
            "roofline": with_measured({"kernel": "prefill_kernel", "bound": "mfma", "achieved": round(tflops, 2),
                                       "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                       "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                                       "traffic": None if ptraffic is None else ptraffic["bytes_per_launch"],
                                       "avg_launch_us": round(pre_ms * 1e3, 2)}, mfma_meas),
            "warm": {"value": round(warm_tflops, 2), "avg_launch_us": round(warm_ms * 1e3, 2),
                     "frac": round(warm_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "timing": "back to back: the 131 MB of KV stays in the 256 MB MALL between launches"},
            "cold_after_read_scrub": {
                "value": round(flops / (rcold_ms * 1e-3) / 1e12, 2), "avg_launch_us": round(rcold_ms * 1e3, 2),
                "frac": round(flops / (rcold_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                "timing": "each launch follows a 1 GiB scrub read (scrubs timed alone and subtracted; includes the "
                          "switch between the two kernels)"},
            "cold_after_write_scrub": {
                "value": round(flops / (wcold_ms * 1e-3) / 1e12, 2), "avg_launch_us": round(wcold_ms * 1e3, 2),
                "frac": round(flops / (wcold_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                "timing": "each launch follows a 1 GiB scrub write (scrubs timed alone and subtracted): the launch "
                          "also pays for writing back the scrub's dirty lines it evicts from L2 and the MALL"},
            "suffix_tokens_per_s": round(int(pc.suffix_lens.sum()) / (pre_ms * 1e-3), 1),
        }
        # the pages' flow: append the suffix K/V, then the prefill
        flow_ms = time_launches(torch, stream, lambda: (pkv.append(p["k_new"], p["v_new"], p["slots"], p["kc"], p["vc"]),
                                                        run_prefill_call(pkv, p)), args.steps)
        result["suffix_prefill"]["append_then_prefill_us"] = round(flow_ms * 1e3, 2)
        del p
        torch.cuda.empty_cache()
        # the same prefill over an fp8 e4m3fn cache (multi-turn with an fp8 KV cache)
        p8 = prefill_fp8_setup(torch, pkv, workloads, dev)
        for _ in range(args.warmup):
            run_prefill_fp8_call(pkv, p8)
        warm_clocks(torch, lambda: run_prefill_fp8_call(pkv, p8))
        f8_ms = time_launches(torch, stream, lambda: run_prefill_fp8_call(pkv, p8), args.steps)
        f8_tflops = flops / (f8_ms * 1e-3) / 1e12
        f8traffic = load_traffic("prefill_16x1900p100_fp8", KERNEL_SOURCES)
        result["suffix_prefill_fp8_kv"] = {
            "metric": "suffix-prefill TFLOP/s, fp8 KV cache", "value": round(f8_tflops, 2), "unit": "TFLOP/s",
            "config": {"workload": "16 requests x (1,900 cached + 100 new tokens), 32/8 heads, d=128, fp8 e4m3fn "
                                   "K/V (per-tensor scales), bf16 q/out, B=16", "flop_per_launch": flops},
            "roofline": with_measured({"kernel": "prefill_kernel (fp8 cache)", "bound": "mfma",
                                       "achieved": round(f8_tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(f8_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                                       "traffic": None if f8traffic is None else f8traffic["bytes_per_launch"],
                                       "avg_launch_us": round(f8_ms * 1e3, 2)}, mfma_meas),
            "timing": "back to back",
        }
        del p8
        torch.cuda.empty_cache()

        # one conversation's next turn: the key-split call against the plain one
        nt = next_turn_setup(torch, pkv, workloads, dev)
        nflops = nt["case"].flops()
        for _ in range(args.warmup):
            run_next_turn_split(pkv, nt)
            run_next_turn_plain(pkv, nt)
        warm_clocks(torch, lambda: run_next_turn_split(pkv, nt))
        ns_ms = time_launches(torch, stream, lambda: run_next_turn_split(pkv, nt), args.steps)
        np_ms = time_launches(torch, stream, lambda: run_next_turn_plain(pkv, nt), args.steps)
        ns_tflops = nflops / (ns_ms * 1e-3) / 1e12
        ntraffic = load_traffic("prefill_next_turn_1x8000p100_bf16", KERNEL_SOURCES)
        result["suffix_prefill_next_turn"] = {
            "metric": "suffix-prefill TFLOP/s, one conversation's next turn", "value": round(ns_tflops, 2),
            "unit": "TFLOP/s",
            "config": {"workload": "1 request x (8,000 cached + 100 new tokens), 32/8 heads, d=128, bf16, B=16 "
                                   "(pkv_suffix_prefill_attn_split)", "flop_per_launch": nflops,
                       "workspace_bytes": nt["ws_bytes"]},
            "split_us": round(ns_ms * 1e3, 2), "plain_us": round(np_ms * 1e3, 2),
            "plain_tflops": round(nflops / (np_ms * 1e-3) / 1e12, 2),
            "roofline": with_measured({"kernel": "prefill_split_kernel + prefill_merge_kernel", "bound": "mfma",
                                       "achieved": round(ns_tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(ns_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                                       "traffic": None if ntraffic is None else ntraffic["bytes_per_launch"],
                                       "avg_launch_us": round(ns_ms * 1e3, 2)}, mfma_meas),
            "timing": "back to back",
        }
        del nt
        torch.cuda.empty_cache()

    # ---------------- shared-prefix decode: cascade vs plain ----------------
    if not args.no_shared_prefix:
        torch.cuda.empty_cache()
        sp = shared_prefix_setup(torch, pkv, workloads, dev)
        sc = sp["case"]
        casc = lambda: run_cascade_call(pkv, sp)
        plain = lambda: run_decode_call(pkv, sp)
        for _ in range(args.warmup):
            casc()
            plain()
        warm_clocks(torch, casc, 0.3)
        c_ms = time_launches(torch, stream, casc, args.steps)
        p_ms = time_launches(torch, stream, plain, args.steps)
        ub, lb = sc.unique_kv_read_bytes(), sc.kv_read_bytes()
        straffic = load_traffic("cascade_shared_prefix_256x1000_bf16", KERNEL_SOURCES)
        result["shared_prefix_decode"] = {
            "metric": "shared-prefix decode KV-read GB/s (unique bytes)", "value": round(ub / (c_ms * 1e-3) / 1e9, 1),
            "unit": "GB/s",
            "config": {"workload": "256 sequences sharing a 1,000-token system prompt (31 aliased 32-token blocks) "
                                   "+ 50..500 private tokens, 32/8 heads, d=128, bf16, B=32",
                       "unique_kv_bytes": ub, "logical_kv_bytes": lb},
            "cascade_us": round(c_ms * 1e3, 2), "plain_decode_us": round(p_ms * 1e3, 2),
            "plain_decode_unique_gbs": round(ub / (p_ms * 1e-3) / 1e9, 1),
            # the K/V bytes the step attends to (shared blocks counted once per sequence), per second
            "logical_kv_gbs": round(lb / (c_ms * 1e-3) / 1e9, 1),
            "tokens_per_s": round(sc.num_seqs / (c_ms * 1e-3), 1),  # one decoded token per sequence
            "roofline": with_measured({"kernel": "pkv_cascade_decode_attn (shared part + decode_kernel + combine)",
                                       "bound": "hbm", "achieved": round(ub / (c_ms * 1e-3) / 1e9, 1),
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": round(ub / (c_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                       "traffic": None if straffic is None else straffic["bytes_per_launch"],
                                       "avg_launch_us": round(c_ms * 1e3, 2), "algorithmic_bytes_per_launch": ub},
                                      hbm_meas),
        }
        del sp
        torch.cuda.empty_cache()

    # ---------------- long-context fp8 decode: 32 layers per step ----------------
    if not args.no_long_context:
        torch.cuda.empty_cache()
        lt = long_context_setup(torch, pkv, workloads, dev)
        lc = lt["case"]
        lsteps = max(3, args.steps // 10)
        for _ in range(max(1, args.warmup // 5)):
            run_long_context_step(pkv, lt)
        warm_clocks(torch, lambda: run_long_context_step(pkv, lt), 0.3)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(lsteps):
            run_long_context_step(pkv, lt)
        e1.record(stream)
        torch.cuda.synchronize()
        lms = e0.elapsed_time(e1) / lsteps
        lbytes = lc.kv_read_bytes_per_layer() * lc.num_layers
        layers = lt["layers"]
        it = iter(range(1 << 30))
        lay_ms = time_launches(torch, stream, lambda: run_long_context_decode(pkv, lt, layers[next(it) % len(layers)]),
                               lc.num_layers * lsteps)
        lay_gbs = lc.kv_read_bytes_per_layer() / (lay_ms * 1e-3) / 1e9
        ltraffic = load_traffic("decode_long_context_8x100k_fp8", KERNEL_SOURCES)
        result["long_context_fp8"] = {
            "metric": "long-context fp8 decode KV-read GB/s", "value": round(lbytes / (lms * 1e-3) / 1e9, 1),
            "unit": "GB/s", "ms_per_step": round(lms, 4), "steps": lsteps,
            "tokens_per_s": round(lc.num_seqs / (lms * 1e-3), 1),
            "config": {"workload": "8 sequences x 100,000 tokens, 32 layers, 32/8 heads, d=128, fp8 e4m3fn KV "
                                   "(per-layer K/V scales), bf16 q/out, B=32; step = append newest token + "
                                   "decode, every layer", "kv_bytes_per_step": lbytes},
            "roofline": with_measured({"kernel": "pkv_decode_attn on one layer (decode_kernel + decode_combine_kernel)",
                                       "bound": "hbm", "achieved": round(lay_gbs, 1), "peak": HBM_PEAK_GBS,
                                       "unit": "GB/s", "frac": round(lay_gbs / HBM_PEAK_GBS, 4),
                                       "traffic": None if ltraffic is None else ltraffic["bytes_per_launch"],
                                       "avg_launch_us": round(lay_ms * 1e3, 2),
                                       "algorithmic_bytes_per_launch": lc.kv_read_bytes_per_layer()}, hbm_meas),
        }
        del lt
        torch.cuda.empty_cache()

    if cpu is not None:
        result["cpu_baseline"] = cpu

    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
