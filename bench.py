"""Benchmark: the DSA attention layer's hot path on one MI355X, at the pages' shapes.

Timed step (the headline): c2, speculative-verify decode at 128K context -- 64 requests x 6 query
rows (causal drafts at positions 131,066..131,071), 64-token pages under a random page
permutation, a 4-layer group in the pages' full/shared pattern: layer 0 full (index-K store of
the step's tokens, q quantise, fused indexer logits + top-2048, sparse MLA), layers 1-3 shared
(sparse MLA reusing layer 0's top-k tensor).  Every layer has its own 5.5 GB latent cache; the
full layer its own 1.1 GB index-K cache.  Inputs are seeded synthetic N(0,1) / U(0,1) at the
pages' shapes, generated in HBM before timing.

  value    = query tokens / s of the full layer (384 rows / the full layer's time in the step)
  roofline = the step's dominant kernel (largest share of the step's time), its algorithmic
             bytes per launch / its mean event-timed launch duration, against 8 TB/s

Also measured, each as its own section: c0 (1 request at 4K), c1 (32 requests at 8K-32K), c3
(1 request at 1M), the 1K..1M single-request sweep -- these with at least 2 GB of cache copies
rotated per iteration so the 256 MB last-level cache cannot serve the reads -- and c4 (8192-row
chunked prefill on a 65,536-token prefix); the plain indexer-logits call for the index-K
read rate; the MXFP4 index-K variant, the MTP draft iteration, the fused norm + RoPE store and
the 1M-token chunked prefill; the oracle timed on the host per stage.

Prints one JSON line.  --gpus N > 1 exits: the library has no multi-GPU path.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA layer query-tokens/s at 128K ctx; indexer-cache HBM GB/s (% of peak)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense fp8 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
STATS_FILE = os.path.join(ROOT, "profiles", "kernel_stats.json")
MLA_BYTES_PER_ROW = 2048 * 656 + 64 * 576 * 2 + 64 * 512 * 2 + 2048 * 4   # 1,490,944 B
MLA_FLOPS_PER_ROW = 2 * 64 * 2048 * (576 + 512)                            # 285,212,672
LN_EPS, THETA, SM, TOPK = 1e-6, 10000.0, 1.0 / 16.0, 2048
ROTATE_BYTES = 2 << 30          # cache copies rotated per iteration for workloads under 1 GB
PREFILL_LOGITS_BUDGET = 4 << 30   # logits scratch per indexer launch in the 1M chunked prefill
# per token of the fused store: kv latent + k_pe (576 bf16), index key (128 bf16), 64 query rope
# parts read and written (64 x 64 bf16 each way), the 656-B record, the 132-B index entry, req + pos
FUSED_STORE_BYTES_PER_TOKEN = 576 * 2 + 128 * 2 + 2 * 64 * 64 * 2 + 656 + 132 + 8
SECTIONS = ("c2", "c0", "c1", "c3", "sweep", "c4", "mxfp4", "mtp", "fused_store", "prefill1m", "copy")
# file stem of each section's summaries under profiles/: the workload it covers
PROFILE_STEMS = {"c2": "c2_verify_128k", "c0": "c0_tiny_decode_4k", "c1": "c1_decode_batch_8k_32k",
                 "c3": "c3_long_context_1m", "c4": "c4_chunked_prefill_8192_on_64k", "sweep": "decode_ctx_sweep_1k_1m",
                 "mxfp4": "c2_verify_128k_mxfp4_index", "mtp": "c2_mtp_draft_round",
                 "fused_store": "fused_norm_rope_store_8192", "prefill1m": "chunked_prefill_1m"}

_IDX_SRC = ["sparse_attention_store_amd/csrc/k_indexer.hip", "sparse_attention_store_amd/csrc/dsa_device.hpp",
            "sparse_attention_store_amd/csrc/dsa_internal.h"]
_MLA_SRC = ["sparse_attention_store_amd/csrc/k_mla.hip", "sparse_attention_store_amd/csrc/dsa_device.hpp",
            "sparse_attention_store_amd/csrc/dsa_internal.h"]
_STORE_SRC = ["sparse_attention_store_amd/csrc/k_store.hip", "sparse_attention_store_amd/csrc/dsa_device.hpp",
              "sparse_attention_store_amd/csrc/dsa_internal.h"]
_TOPK_SRC = ["sparse_attention_store_amd/csrc/k_topk.hip", "sparse_attention_store_amd/csrc/dsa_device.hpp",
             "sparse_attention_store_amd/csrc/dsa_internal.h"]


def kernel_sources(name):
    """The source files a kernel (as rocprofv3 names it) is built from."""
    for key, src in (("k_logits_decode", _IDX_SRC), ("k_sparse_mla", _MLA_SRC), ("k_mla_", _MLA_SRC),
                     ("k_fused_norm", _STORE_SRC), ("k_index_k_store", _STORE_SRC), ("k_latent_store", _STORE_SRC),
                     ("k_quant_fp8", _STORE_SRC), ("k_filt", _TOPK_SRC), ("k_init", _TOPK_SRC), ("k_hist", _TOPK_SRC),
                     ("k_select", _TOPK_SRC), ("k_final", _TOPK_SRC), ("k_range", _TOPK_SRC),
                     ("k_row_topk", _TOPK_SRC)):
        if key in name:
            return src
    return None


def indexer_bytes(ctx, rows, key_bytes=132):
    """Algorithmic bytes of one indexer-logits launch: every visible key once (FP8: 128 B + a
    4-B scale; MXFP4: 64 B + four 1-B scales), the page-table entries, and per row the fp8
    query, its scales and head weights."""
    import numpy as np
    L = np.asarray(ctx, dtype=np.int64)
    return int((key_bytes * L + 4 * ((L + 63) // 64)).sum() + rows * (32 * 128 + 32 * 4 + 32 * 4))


def filter_pass_bytes(ctx, rows_per_req, sample_step=16):
    """Algorithmic bytes of the fused call's filter pass: the keys of every page but the sampled
    ones (one in sample_step, scored by the sample pass), the page-table entries, per row the
    query, scales and weights, and the sampled pages' stored scores it reads back instead."""
    import numpy as np
    L = np.asarray(ctx, dtype=np.int64)
    pages = (L + 63) // 64
    sampled = (pages + sample_step - 1) // sample_step
    rows = rows_per_req * len(L)
    return int(((pages - sampled) * 8448 + 4 * pages + rows_per_req * sampled * 64 * 4).sum()
               + rows * (32 * 128 + 32 * 4 + 32 * 4))


def source_digest(files):
    """sha256 over the kernel sources a measurement was taken with."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _load(path):
    try:
        with open(path) as fh:
            return json.load(fh)
    except (OSError, ValueError):
        return {}


def measured_traffic(section, kernel):
    """HBM bytes per launch of `kernel` in a section of this benchmark, from the committed
    rocprofv3 counter summary: FETCH_SIZE x fetch_factor + WRITE_SIZE x write_factor (KiB per
    dispatch; the factors make a plain 1 GiB copy read and write 1 GiB).  None when there is no
    summary or the kernel's sources changed since it was taken."""
    t = _load(TRAFFIC_FILE)
    k = t.get("sections", {}).get(section, {}).get(kernel)
    if not k or source_digest(k["sources"]) != k["source_sha256"]:
        return None
    return int(round((k["fetch_kib"] * t["fetch_factor"] + k["write_kib"] * t["write_factor"]) * 1024))


def profiled_us(section, kernel):
    """Mean duration (us) of `kernel` in a section, from the committed rocprofv3 kernel trace;
    None when absent or the kernel's sources changed since."""
    k = _load(STATS_FILE).get("sections", {}).get(section, {}).get(kernel)
    if not k or source_digest(k["sources"]) != k["source_sha256"]:
        return None
    return k["avg_us"]


# ----------------------------------------------------------------------------- counter summaries
def _kname(raw):
    """A kernel's name as rocprofv3 prints it, without return type, namespaces and arguments."""
    for junk in ("(anonymous namespace)::", "void ", "dsa::"):
        raw = raw.replace(junk, "")
    return raw.split("(")[0].strip()


def _read_csv(path):
    import csv
    with open(path) as fh:
        return list(csv.DictReader(fh))


def write_traffic(section, fetch_csv, write_csv, command):
    """Merges two rocprofv3 --pmc runs of `bench.py --configs <section> --copy-probe`
    (FETCH_SIZE, then WRITE_SIZE) into TRAFFIC_FILE: per kernel the median KiB per dispatch, and
    the factors that make the 1 GiB device copy read and write 1 GiB."""
    import statistics

    def per_kernel(path):
        vals = {}
        for r in _read_csv(path):
            vals.setdefault(_kname(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_csv), per_kernel(write_csv)
    gib_kib = float(1 << 20)
    copy_f = max(v for n, vs in fetch.items() if "copyBuffer" in n for v in vs)
    copy_w = max(v for n, vs in write.items() if "copyBuffer" in n for v in vs)
    out = _load(TRAFFIC_FILE) or {"sections": {}}
    out["about"] = ("HBM traffic per dispatch of the benchmark's kernels by section, from rocprofv3 --pmc FETCH_SIZE "
                    "and WRITE_SIZE (KiB per dispatch, median over the section's dispatches); fetch_factor and "
                    "write_factor make a 1 GiB device copy read and write 1 GiB")
    out.update({"copy_fetch_kib": copy_f, "copy_write_kib": copy_w, "fetch_factor": gib_kib / copy_f,
                "write_factor": gib_kib / copy_w})
    sec = {"command": command}
    for k in fetch:
        src = kernel_sources(k)
        if src and k in write:
            sec[k] = {"fetch_kib": statistics.median(fetch[k]), "write_kib": statistics.median(write[k]),
                      "dispatches": len(fetch[k]), "sources": src, "source_sha256": source_digest(src)}
    out["sections"][section] = sec
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    lines = [f"HBM traffic per dispatch, section {section} of bench.py (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)",
             "", "Command (one run per counter):"] + ["  " + c for c in command.split(" ;; ")] + [
             "", f"Calibration: a 1 GiB device copy reads {copy_f:.0f} KiB (factor {gib_kib / copy_f:.4f}) and writes "
                 f"{copy_w:.0f} KiB (factor {gib_kib / copy_w:.4f}); the MB below are scaled by these factors.", "",
             f"{'kernel':<56} {'dispatches':>10} {'fetch MB':>10} {'write MB':>10}"]
    for k, v in sorted(sec.items(), key=lambda kv: -kv[1]["fetch_kib"] if isinstance(kv[1], dict) else 0):
        if isinstance(v, dict):
            lines.append(f"{k[:56]:<56} {v['dispatches']:>10} {v['fetch_kib'] * 1024 * gib_kib / copy_f / 1e6:>10.2f} "
                         f"{v['write_kib'] * 1024 * gib_kib / copy_w / 1e6:>10.2f}")
    with open(os.path.join(ROOT, "profiles", f"{PROFILE_STEMS.get(section, section)}_hbm_traffic.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return sec


def write_stats(section, stats_csv, command, title):
    """Merges a rocprofv3 --kernel-trace --stats summary (kernel_stats.csv) of `bench.py --configs
    <section>` into STATS_FILE and writes profiles/<section>_kernel_stats.txt."""
    rows = _read_csv(stats_csv)
    out = _load(STATS_FILE) or {"sections": {}}
    sec = {"command": command}
    lines = [title, "", "Command:", "  " + command, "",
             f"{'kernel':<64} {'calls':>7} {'avg us':>9} {'min us':>9} {'max us':>9}"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = _kname(r["Name"])
        avg, mn, mx = float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3
        lines.append(f"{name[:64]:<64} {int(r['Calls']):>7} {avg:>9.2f} {mn:>9.2f} {mx:>9.2f}")
        src = kernel_sources(name)
        if src:
            sec[name] = {"calls": int(r["Calls"]), "avg_us": avg, "min_us": mn, "max_us": mx, "sources": src,
                         "source_sha256": source_digest(src)}
    out["sections"][section] = sec
    with open(STATS_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    with open(os.path.join(ROOT, "profiles", f"{PROFILE_STEMS.get(section, section)}_kernel_stats.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return sec


def write_counters(section, csvs, command, title):
    """Summarises rocprofv3 --pmc runs of one section (comma-separated counter_collection.csv
    files, one per pass, each with GRBM_GUI_ACTIVE) into profiles/<stem>_counters.txt: per
    kernel, over all its dispatches, the busy fractions of the MFMA and VALU units, LDS activity
    and bank conflicts, wave wait fractions and instruction counts.  Chip constants: 8 XCDs of
    32 CUs, 4 SIMDs per CU; GRBM_GUI_ACTIVE is summed over the XCDs."""
    import collections
    xcd, cus, simds = 8, 256, 1024
    tot = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for path in csvs.split(","):
        seen = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in _read_csv(path):
            name = _kname(r["Kernel_Name"])
            seen[name][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[(name, path)].add(r["Dispatch_Id"])
        for name, cs in seen.items():
            gui = cs.pop("GRBM_GUI_ACTIVE", 0.0)
            for c, v in cs.items():
                tot[name][c] += v
                tot[name]["gui:" + c] += gui      # the pass's own cycles, for its counters' ratios
    lines = [title, "", "Command (one run per pass, counters as listed):"] + ["  " + c for c in command.split(" ;; ")]
    lines += ["", "Per kernel, summed over its dispatches; busy fractions are of all SIMDs (MFMA, VALU) or CUs (LDS)",
              "over the kernel's active cycles (GRBM_GUI_ACTIVE / 8 XCDs).  conflict/access = bank-conflict cycles",
              "per conflict-free LDS cycle.  wait/active = share of wave-cycles waiting / issuing.", ""]

    def ratio(m, c, scale):
        g = m.get("gui:" + c, 0.0) / xcd
        return m[c] / (g * scale) if c in m and g else None

    for name, m in sorted(tot.items(), key=lambda kv: -max(v for c, v in kv[1].items() if c.startswith("gui:"))):
        n = max(len(d) for (k, _), d in disp.items() if k == name)
        cyc = max(v for c, v in m.items() if c.startswith("gui:")) / xcd
        parts = [f"{name}", f"  dispatches {n}, active {cyc / 2.4e3 / n:.1f} us per dispatch at 2.4 GHz"]
        mf, va = ratio(m, "SQ_VALU_MFMA_BUSY_CYCLES", simds), ratio(m, "SQ_ACTIVE_INST_VALU", simds / 4)
        ld = ratio(m, "SQ_LDS_IDX_ACTIVE", cus)
        f = []
        if mf is not None:
            f.append(f"MFMA busy {100 * mf:.1f}%")
        if va is not None:
            f.append(f"VALU {100 * va:.1f}% (SQ_ACTIVE_INST_VALU x 4 cycles / SIMD-cycles)")
        if ld is not None:
            conf = m.get("SQ_LDS_BANK_CONFLICT", 0.0)
            f.append(f"LDS active {100 * ld:.1f}%, conflict/access {conf / max(1.0, m['SQ_LDS_IDX_ACTIVE'] - conf):.3f}")
        if "SQ_WAVE_CYCLES" in m:
            wc = m["SQ_WAVE_CYCLES"]
            f.append(f"wave-cycles: wait {100 * m.get('SQ_WAIT_ANY', 0) / wc:.0f}%, wait on dependency "
                     f"{100 * m.get('SQ_WAIT_INST_ANY', 0) / wc:.0f}%, issuing {100 * m.get('SQ_ACTIVE_INST_ANY', 0) / wc:.0f}%")
        if "SQ_INSTS_VALU" in m:
            f.append("instructions per dispatch: " + ", ".join(
                f"{c[9:].lower()} {m[c] / n:.3g}" for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
                                                           "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD") if c in m))
        lines += parts + ["  " + x for x in f] + [""]
    path = os.path.join(ROOT, "profiles", f"{PROFILE_STEMS.get(section, section)}_counters.txt")
    with open(path, "w") as fh:
        fh.write("\n".join(lines))
    return path


# ----------------------------------------------------------------------------- GPU timing helpers
class Timer:
    """Per-stage GPU durations from HIP events on the stream the library runs on.  A spin kernel
    queued first keeps the device busy while the host enqueues the iterations, so host-side call
    overhead does not show as idle time between events."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def _spin_for(self, host_us_per_iter, n):
        self.torch.cuda._sleep(int(min(1.5 * n * host_us_per_iter + 200.0, 5e5) * 2000))   # ~2 GHz shader clock

    def _host_us(self, make, i):
        t = self.torch
        t.cuda.synchronize()
        h0 = time.perf_counter()
        for _, f in make(i):
            f()
        us = (time.perf_counter() - h0) * 1e6
        t.cuda.synchronize()
        return us

    def stages(self, make, n, warmup):
        """make(i) -> [(name, fn), ...] for iteration i.  Returns ({name: median us}, median
        total us) over n iterations timed with an event between stages, and the mean us of an
        iteration timed without intermediate events (kernel-only layer time)."""
        import numpy as np
        t = self.torch
        for i in range(warmup):
            for _, f in make(i):
                f()
        host = self._host_us(make, warmup)
        names = [nm for nm, _ in make(0)]
        ev = [[t.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(n)]
        self._spin_for(host, n)
        for i in range(n):
            fs = make(warmup + 1 + i)
            ev[i][0].record(self.stream)
            for j, (_, f) in enumerate(fs):
                f()
                ev[i][j + 1].record(self.stream)
        t.cuda.synchronize()
        per = {nm: float(np.median([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(n)])) * 1e3
               for j, nm in enumerate(names)}
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        self._spin_for(host, n)
        e0.record(self.stream)
        for i in range(n):
            for _, f in make(warmup + 1 + n + i):
                f()
        e1.record(self.stream)
        t.cuda.synchronize()
        return per, e0.elapsed_time(e1) / n * 1e3

    def calls(self, fn, n):
        """Mean us per call of fn(i), n calls back to back."""
        t = self.torch
        fn(0)
        host = self._host_us(lambda i: [("f", lambda: fn(i))], 1)
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        self._spin_for(host, n)
        e0.record(self.stream)
        for i in range(n):
            fn(2 + i)
        e1.record(self.stream)
        t.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3


def frac(gbps):
    return round(gbps / HBM_PEAK_GBPS, 4)


class Rotation:
    """At least `min_bytes` of independent copies of a layer's index-K and latent caches, each with
    its own page table (the same logical content, disjoint pages of one pool); iteration i reads
    copy i mod N, so a copy has left the last-level cache by the time it is read again."""

    def __init__(self, torch, dsa, D, min_bytes=ROTATE_BYTES):
        P = D.w.num_pages
        foot = P * (dsa.INDEX_PAGE_BYTES + dsa.LATENT_PAGE_BYTES)
        self.n = max(1, math.ceil(min_bytes / foot))
        self.bytes = self.n * foot
        self.index = torch.empty((self.n * P, dsa.INDEX_PAGE_BYTES), dtype=torch.uint8, device="cuda")
        self.latent = torch.empty((self.n * P, dsa.LATENT_PAGE_BYTES), dtype=torch.uint8, device="cuda")
        for i in range(self.n):
            self.index[i * P:(i + 1) * P].copy_(D.index_cache[0])
            self.latent[i * P:(i + 1) * P].copy_(D.latent_cache[0])
        self.pages = [dsa.Pages(D.pages.page_table + i * P, self.n * P) for i in range(self.n)]
        torch.cuda.synchronize()

    def at(self, i):
        return self.pages[i % self.n]


def layer_stages(dsa, D, pages, icache, lcache, prefill=False):
    """One full layer as the library's calls: store, quantise, fused indexer + top-k, sparse MLA."""
    mla = dsa.dsa_sparse_mla_prefill if prefill else dsa.dsa_sparse_mla_decode
    return [("store", lambda: dsa.dsa_index_k_store(D.k_new, D.rows, pages, icache, LN_EPS, THETA)),
            ("quant", lambda: dsa.dsa_quant_fp8(D.q_idx, D.q8, D.qs)),
            ("indexer_topk", lambda: dsa.dsa_indexer_topk(D.q8, D.qs, D.w_head, D.rows, pages, icache, D.logits,
                                                          TOPK, D.idx, D.ws_topk)),
            ("mla", lambda: mla(D.q_mla[0], D.rows, pages, lcache, D.idx, D.out[0], D.lse[0], D.ws_mla, SM))]


def measure_layer(torch, dsa, timer, w, n, warmup, rotate=True, prefill=False):
    """Full-layer stages of workload w (latent layer 0 only), with cache rotation when the
    workload's caches fit the last-level cache; plus the plain indexer-logits call."""
    import numpy as np
    from sparse_attention_store_amd.workload import DeviceLayer
    D = DeviceLayer(w, latent_layers=[0])
    rot = Rotation(torch, dsa, D) if rotate else None
    if rot is not None:       # the rotation pool replaces the layer's own caches
        del D.index_cache[0], D.latent_cache[0]
        D.index_cache[0], D.latent_cache[0] = None, None
        icache, lcache, pages_at = rot.index, rot.latent, rot.at
    else:
        icache, lcache, pages_at = D.index_cache[0], D.latent_cache[0], (lambda i: D.pages)
    torch.cuda.synchronize()
    per, layer_us = timer.stages(lambda i: layer_stages(dsa, D, pages_at(i), icache, lcache, prefill), n, warmup)
    logits_us = timer.calls(lambda i: dsa.dsa_indexer_logits(D.q8, D.qs, D.w_head, D.rows, pages_at(i), icache,
                                                             D.logits), n)
    R = w.R
    ib = indexer_bytes(w.ctx, R)
    mb = MLA_BYTES_PER_ROW * R
    res = {
        "rows": R, "requests": w.B, "ctx_min": int(w.ctx.min()), "ctx_max": int(w.ctx.max()),
        "ctx_mean": float(np.mean(w.ctx)),
        "rotation": ({"copies": rot.n, "bytes": rot.bytes} if rot else None),
        "stage_us_median": {k: round(v, 2) for k, v in per.items()},
        "full_layer_us": round(layer_us, 2),
        "query_tokens_per_s": R / (layer_us * 1e-6),
        "index_k": {"algorithmic_bytes": ib, "plain_logits_us": round(logits_us, 2),
                    "plain_logits_GBps": round(ib / (logits_us * 1e-6) / 1e9, 1),
                    "plain_logits_frac": frac(ib / (logits_us * 1e-6) / 1e9),
                    "fused_indexer_topk_GBps": round(ib / (per["indexer_topk"] * 1e-6) / 1e9, 1),
                    "fused_indexer_topk_frac": frac(ib / (per["indexer_topk"] * 1e-6) / 1e9)},
        "mla": {"algorithmic_bytes": mb, "us": round(per["mla"], 2),
                "GBps": round(mb / (per["mla"] * 1e-6) / 1e9, 1), "frac_hbm": frac(mb / (per["mla"] * 1e-6) / 1e9),
                "TFLOPs": round(MLA_FLOPS_PER_ROW * R / (per["mla"] * 1e-6) / 1e12, 1)},
    }
    del D, rot
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- oracle (CPU) timing
def _omp_threads(n=None):
    """Sets (n given) and returns the OpenMP thread count of the oracle's runtime."""
    import ctypes
    gomp = ctypes.CDLL("libgomp.so.1")
    if n is not None:
        gomp.omp_set_num_threads(int(n))
    return int(gomp.omp_get_max_threads())


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def oracle_stage_times(w, rows, n_layers=1):
    """The oracle (as it stands) on the given rows of workload w, per stage: store of the rows'
    own keys, q quantisation, indexer logits, top-k, sparse MLA per layer.  The rows' requests get
    a compact page pool; their index-K caches and the selected latent records are built outside
    the timed part (the caches' state before the step).  Seconds per stage."""
    import numpy as np
    import dsa_inputs as gi
    import oracle as orc
    rows = np.asarray(rows)
    reqs = np.unique(w.row_req[rows])
    local = {int(b): i for i, b in enumerate(reqs)}
    npg = [(int(w.ctx[b]) + 63) // 64 for b in reqs]
    pt = np.zeros((len(reqs), max(npg)), np.int32)
    off = 0
    for i, n in enumerate(npg):
        pt[i, :n] = np.arange(off, off + n)
        off += n
    icache = np.zeros((off, 8448), np.uint8)
    for b in reqs:
        L = int(w.ctx[b])
        k = gi.normal_bf16(w.seed, gi.T_RAW_K, int(w.token_base[b]) * 128, L * 128).reshape(L, 128)
        orc.index_k_store(k, np.full(L, local[int(b)], np.int32), np.arange(L, dtype=np.int32), pt, icache)
    req = np.array([local[int(b)] for b in w.row_req[rows]], np.int32)
    pos = w.row_pos[rows].astype(np.int32)
    gr = w.row0 + rows
    knew = np.stack([gi.normal_bf16(w.seed, gi.T_RAW_K, (int(w.token_base[w.row_req[r]]) + int(w.row_pos[r])) * 128, 128)
                     for r in rows])
    q = np.stack([gi.normal_bf16(w.seed, gi.T_IDX_Q, int(r) * 32 * 128, 32 * 128) for r in gr])
    wt = np.stack([gi.uniform_f32(w.seed, gi.T_W, int(r) * 32, 32, gi.w_scale()) for r in gr])
    t = {}
    t0 = time.perf_counter()
    orc.index_k_store(knew, req, pos, pt, icache)
    t["store"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    q8, qs = orc.quant_fp8(q.reshape(-1, 128))
    t["quant"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    lg = orc.indexer_logits(q8.reshape(-1, 32, 128), qs.reshape(-1, 32), wt, req, pos, pt, icache)
    t["logits"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    idx, _ = orc.topk(lg, pos, TOPK)
    t["topk"] = time.perf_counter() - t0
    del lg
    t["mla"] = 0.0
    for l in range(n_layers):
        qm = np.stack([gi.normal_bf16(w.seed, gi.T_MLA_Q, (l * w.rows_total + int(r)) * 64 * 576, 64 * 576)
                       for r in gr]).reshape(-1, 64, 576)
        lcache = np.zeros((off, 64 * 656), np.uint8)
        for i, b in enumerate(reqs):
            sel = np.unique(idx[req == i]).astype(np.int64)
            sel = sel[sel >= 0]
            kv = gi.normal_bf16_at(w.seed, gi.T_LATENT0 + l,
                                   ((int(w.token_base[b]) + sel)[:, None] * 576 + np.arange(576)[None, :]).ravel())
            orc.latent_store(kv.reshape(-1, 576), np.full(len(sel), i, np.int32), sel.astype(np.int32), pt, lcache)
        t0 = time.perf_counter()
        orc.sparse_mla(qm, req, pos, pt, lcache, idx, SM)
        t["mla" if l == 0 else f"mla_shared{l}"] = time.perf_counter() - t0
    return t


def cpu_baselines(threads):
    """The oracle per stage on the pages' configs: c0, c1, c3 in full (c0 also on one thread), c2 on
    4 of its 64 requests and c4 on 256 of its 8192 rows (the batch times scaled by rows and
    labelled extrapolated)."""
    import numpy as np
    import dsa_inputs as gi

    def summary(w, rows, n_layers=1, scale=1.0, label="full"):
        t0 = time.perf_counter()
        t = oracle_stage_times(w, rows, n_layers)
        wall = time.perf_counter() - t0
        full = sum(v for k, v in t.items() if not k.startswith("mla_shared"))
        out = {"rows": len(rows), "sample": label, "stage_s": {k: round(v, 4) for k, v in t.items()},
               "full_layer_s": round(full, 4), "query_tokens_per_s": len(rows) / full,
               "threads_busy": min(threads, len(rows)), "wall_s_with_setup": round(wall, 1)}
        if scale != 1.0:
            out["extrapolated_batch_full_layer_s"] = round(full * scale, 3)
        return out

    res = {"cpu": cpu_model(), "nproc": os.cpu_count(), "omp_threads": threads}
    w0 = gi.config(0)
    res["c0"] = summary(w0, np.arange(w0.R))
    _omp_threads(1)
    res["c0_one_thread"] = summary(w0, np.arange(w0.R))
    _omp_threads(threads)
    w1 = gi.config(1)
    res["c1"] = summary(w1, np.arange(w1.R))
    w2 = gi.config(2)
    r2 = np.where(np.isin(w2.row_req, [0, 21, 42, 63]))[0]
    res["c2"] = summary(w2, r2, n_layers=4, scale=w2.R / len(r2), label="4 of 64 requests (24 rows), extrapolated")
    w3 = gi.config(3)
    res["c3"] = summary(w3, np.arange(w3.R))
    w4 = gi.config(4)
    r4 = np.linspace(0, w4.R - 1, 256).astype(np.int64)
    res["c4"] = summary(w4, r4, scale=w4.R / 256, label="256 of 8192 rows, extrapolated")
    return res


# ----------------------------------------------------------------------------- sections
def measured_references(torch, dsa, timer, D, n):
    """Reference rates measured on this device for the access patterns of the two hot kernels:
    a streaming read of the step's index-K cache (the indexer's scan) and a gather of the 656-B
    latent records at the positions the step's top-k selected (the sparse MLA's reads), both by
    the library's probe kernels."""
    sink = torch.empty(dsa.PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    cache = D.index_cache[0]
    read_b = cache.numel()
    read_us = timer.calls(lambda i: dsa.dsa_probe_stream_read(cache, sink), n)
    # physical record index of every selected position: page id * 64 + position within the page
    pt = D.pages.page_table.long()
    req = D.rows.req.long()[:, None].expand_as(D.idx)
    sel = D.idx.long()
    ok = sel >= 0
    phys = pt[req, torch.where(ok, sel, 0) >> 6] * 64 + (torch.where(ok, sel, 0) & 63)
    ids = phys[ok].to(torch.int32).contiguous()
    pool = D.latent_cache[0]
    gather_b = ids.numel() * 656
    gather_us = timer.calls(lambda i: dsa.dsa_probe_gather_records(pool, 656, ids, sink), n)
    return {"stream_read": {"about": "dsa_probe_stream_read over the step's index-K cache (one full layer)",
                            "bytes": read_b, "us": round(read_us, 2),
                            "GBps": round(read_b / (read_us * 1e-6) / 1e9, 1),
                            "frac_of_nominal": frac(read_b / (read_us * 1e-6) / 1e9)},
            "record_gather": {"about": "dsa_probe_gather_records: the 656-B latent records at the step's selected "
                                       "positions (one sparse-MLA launch's reads), each read whole",
                              "records": int(ids.numel()), "bytes": gather_b, "us": round(gather_us, 2),
                              "GBps": round(gather_b / (gather_us * 1e-6) / 1e9, 1),
                              "frac_of_nominal": frac(gather_b / (gather_us * 1e-6) / 1e9)}}


def run_c2(torch, dsa, timer, a, stream):
    """The timed step: one c2 layer group per step (K steps after W warm-up steps)."""
    import numpy as np
    import dsa_inputs as gi
    from sparse_attention_store_amd.workload import DeviceLayer
    w = gi.config(2)
    t0 = time.time()
    D = DeviceLayer(w)
    print(f"[bench] c2 ready in {time.time() - t0:.1f} s: {w.B} requests x {w.rows_per_req} rows, ctx {int(w.ctx[0])}, "
          f"{w.num_pages} pages, {len(D.layers)} layers", file=sys.stderr, flush=True)
    names = ["store", "quant", "indexer_topk"] + [f"mla{l}" for l in D.layers]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        dsa.dsa_index_k_store(D.k_new, D.rows, D.pages, D.index_cache[0], LN_EPS, THETA)
        mark(1)
        dsa.dsa_quant_fp8(D.q_idx, D.q8, D.qs)
        mark(2)
        D.indexer_topk(0)     # fused indexer logits + top-2048
        mark(3)
        for j, l in enumerate(D.layers):
            D.mla(l)          # layer 0 full, later layers shared: same idx tensor
            mark(4 + j)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(a.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(a.steps):
        step(evs[s])
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / a.steps
    per = {n: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(a.steps)])) * 1e3
           for i, n in enumerate(names)}
    full_us = per["store"] + per["quant"] + per["indexer_topk"] + per["mla0"]
    shared_us = float(np.mean([per[f"mla{l}"] for l in D.layers[1:]]))
    R = w.R
    # the plain indexer-logits call (every score written): the index-K read rate of §8(d)
    logits_us = timer.calls(lambda i: dsa.dsa_indexer_logits(D.q8, D.qs, D.w_head, D.rows, D.pages, D.index_cache[0],
                                                             D.logits), a.steps)
    ib = indexer_bytes(w.ctx, R)
    mla_b = MLA_BYTES_PER_ROW * R
    mla_launch_us = float(np.mean([per[f"mla{l}"] for l in D.layers]))
    mla_total = sum(per[f"mla{l}"] for l in D.layers)
    filt_us = profiled_us("c2", "k_logits_decode<6, 2, 0>")
    filt_b = filter_pass_bytes(w.ctx, w.rows_per_req)
    roof_mla = {"kernel": f"k_sparse_mla_stream (dsa_sparse_mla_decode, {R} rows, k=2048)", "bound": "hbm",
                "achieved": round(mla_b / (mla_launch_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": frac(mla_b / (mla_launch_us * 1e-6) / 1e9), "traffic": measured_traffic("c2", "k_sparse_mla_stream"),
                "algorithmic_bytes_per_launch": mla_b, "avg_launch_us": round(mla_launch_us, 2),
                "mfma_TFLOPs": round(MLA_FLOPS_PER_ROW * R / (mla_launch_us * 1e-6) / 1e12, 1),
                "share_of_step": round(mla_total / (ms_step * 1e3), 3)}
    roof_idx = {"kernel": "dsa_indexer_topk (fused indexer + top-k, all its kernels)", "bound": "hbm",
                "achieved": round(ib / (per["indexer_topk"] * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": frac(ib / (per["indexer_topk"] * 1e-6) / 1e9), "traffic": None,
                "algorithmic_bytes_per_launch": ib, "avg_launch_us": round(per["indexer_topk"], 2),
                "share_of_step": round(per["indexer_topk"] / (ms_step * 1e3), 3)}
    ref = measured_references(torch, dsa, timer, D, a.steps)
    # the same kernels against those measured rates: the MLA's 656-B record reads per second
    # against the record gather, the plain logits' index-K reads against the streaming read
    mla_rec_gbps = R * 2048 * 656 / (mla_launch_us * 1e-6) / 1e9
    roof_mla["records_GBps"] = round(mla_rec_gbps, 1)
    roof_mla["frac_of_measured_gather"] = round(mla_rec_gbps / ref["record_gather"]["GBps"], 4)
    dominant = roof_mla if mla_total >= per["indexer_topk"] else roof_idx
    out = {
        "value": R / (full_us * 1e-6), "ms_per_step": ms_step,
        "roofline": dominant,
        "c2": {
            "rows": R, "requests": w.B, "ctx": int(w.ctx[0]), "layers": len(D.layers),
            "full_layer_us": round(full_us, 2), "shared_layer_us": round(shared_us, 2),
            "group_us": round(ms_step * 1e3, 2),
            "full_layer_query_tokens_per_s": R / (full_us * 1e-6),
            "shared_layer_query_tokens_per_s": R / (shared_us * 1e-6),
            "group_query_tokens_per_s": R / (ms_step * 1e-3),
            "group_query_token_layers_per_s": R * len(D.layers) / (ms_step * 1e-3),
            "stage_us_mean": {k: round(v, 2) for k, v in per.items()},
            "index_k": {
                "algorithmic_bytes": ib,
                "plain_logits": {"kernel": "k_logits_decode<6, 0, 0> (dsa_indexer_logits)", "us": round(logits_us, 2),
                                 "GBps": round(ib / (logits_us * 1e-6) / 1e9, 1),
                                 "frac": frac(ib / (logits_us * 1e-6) / 1e9),
                                 "frac_of_measured_read": round(ib / (logits_us * 1e-6) / 1e9
                                                                / ref["stream_read"]["GBps"], 4),
                                 "traffic": measured_traffic("c2", "k_logits_decode<6, 0, 0>")},
                "fused_call": {"kernel": "dsa_indexer_topk (all its kernels)", "us": round(per["indexer_topk"], 2),
                               "GBps": roof_idx["achieved"], "frac": roof_idx["frac"]},
                "filter_pass": {"kernel": "k_logits_decode<6, 2, 0> (rocprofv3 trace, committed profile)",
                                "us": filt_us, "algorithmic_bytes": filt_b,
                                "GBps": round(filt_b / (filt_us * 1e-6) / 1e9, 1) if filt_us else None,
                                "frac": frac(filt_b / (filt_us * 1e-6) / 1e9) if filt_us else None,
                                "traffic": measured_traffic("c2", "k_logits_decode<6, 2, 0>")},
            },
            "roofline_mla": roof_mla,
            "roofline_indexer": roof_idx,
            "measured_reference_rates": ref,
        },
        "_layer": D,
    }
    return out


def run_mxfp4(torch, dsa, timer, D, a):
    import numpy as np
    w = D.w
    idx_fp8 = D.idx.clone()
    mx = D.build_mxfp4_index(0)
    logits_us = timer.calls(lambda i: dsa.dsa_indexer_logits_mxfp4(D.q8, D.qs, D.w_head, D.rows, D.pages, mx, D.logits),
                            a.steps)
    topk_us = timer.calls(lambda i: dsa.dsa_indexer_topk_mxfp4(D.q8, D.qs, D.w_head, D.rows, D.pages, mx, D.logits,
                                                               TOPK, D.idx, D.ws_topk), a.steps)
    a8, a4 = idx_fp8.cpu().numpy(), D.idx.cpu().numpy()
    overlap = float(np.mean([len(np.intersect1d(x[x >= 0], y[y >= 0])) / max(1, int((x >= 0).sum()))
                             for x, y in zip(a8, a4)]))
    mxb = indexer_bytes(w.ctx, w.R, key_bytes=68)
    del mx
    D.idx.copy_(idx_fp8)
    return {"about": "the same keys in the MXFP4 index-K format (68 B/token); indexer on it, c2 workload",
            "logits_us": round(logits_us, 2), "algorithmic_bytes_per_launch": mxb,
            "logits_GBps": round(mxb / (logits_us * 1e-6) / 1e9, 1), "logits_frac": frac(mxb / (logits_us * 1e-6) / 1e9),
            "indexer_topk_us": round(topk_us, 2), "topk_overlap_with_fp8": round(overlap, 4)}


def run_fused_store(torch, dsa, timer, a, stream):
    import dsa_inputs as gi
    fw = gi.config(4)
    nf, cs = fw.R, stream.cuda_stream
    fkv = torch.empty((nf, gi.KV_A_WIDTH), dtype=torch.int16, device="cuda")
    fg = torch.empty(512, dtype=torch.int16, device="cuda")
    fk = torch.empty((nf, 128), dtype=torch.int16, device="cuda")
    fq = torch.empty((nf, 64, 576), dtype=torch.int16, device="cuda")
    for t_id, buf in ((gi.T_KV_A, fkv), (gi.T_GAMMA, fg), (gi.T_RAW_K, fk), (gi.T_MLA_Q, fq)):
        gi.dev_normal_bf16(fw.seed, t_id, 0, buf.numel(), buf.data_ptr(), cs)
    flat = torch.zeros((fw.num_pages, 41984), dtype=torch.uint8, device="cuda")
    fidx = torch.zeros((fw.num_pages, 8448), dtype=torch.uint8, device="cuda")
    frows = dsa.Rows(torch.from_numpy(fw.row_req).cuda(), torch.from_numpy(fw.row_pos).cuda(), int(fw.row_pos.max()), 1)
    fpages = dsa.Pages(torch.from_numpy(fw.page_table).cuda(), fw.num_pages)
    fkv_c = fkv[:, 2048:].contiguous()
    us = timer.calls(lambda i: dsa.dsa_fused_norm_rope_store(fkv[:, 2048:], frows, fpages, flat, index_cache=fidx,
                                                             k_idx=fk, gamma=fg, q_pe=fq[:, :, 512:]), a.steps)
    sep_us = timer.calls(lambda i: (dsa.dsa_latent_store(fkv_c, frows, fpages, flat),
                                    dsa.dsa_index_k_store(fk, frows, fpages, fidx, LN_EPS, THETA)), a.steps)
    b = FUSED_STORE_BYTES_PER_TOKEN * nf + 512 * 2
    gbps = b / (us * 1e-6) / 1e9
    return {"about": "RMSNorm + RoPE + 656-B latent record + 132-B index-K entry + in-place query rope rotation for "
                     "the 8192-token chunk of the chunked prefill (65,536-token prefix)",
            "kernel": "k_fused_norm_rope_store", "us": round(us, 2), "algorithmic_bytes_per_launch": b,
            "GBps": round(gbps, 1), "frac_of_peak": frac(gbps),
            "traffic": measured_traffic("fused_store", "k_fused_norm_rope_store"),
            "separate_latent_and_index_stores_us": round(sep_us, 2)}


def run_prefill1m(torch, dsa, stream):
    """One 1,048,576-token prompt prefilled in 32 chunks of 32,768 rows over one full layer's
    caches: per chunk the store of its index keys, q quantisation, the indexer + top-2048 in row
    chunks (4 GiB of logits scratch per launch) and the sparse MLA over its rows."""
    import numpy as np
    import dsa_inputs as gi
    from sparse_attention_store_amd.workload import DeviceLayer
    pw = gi.config(5)
    n_chunk_rows = pw.extra["chunk"]
    pbase, cp = None, []
    for c in range((pw.R + n_chunk_rows - 1) // n_chunk_rows):
        wc = gi.prefill_chunk(pw, c)
        Lc = DeviceLayer(wc, latent_layers=[0], logits_budget_bytes=PREFILL_LOGITS_BUDGET, caches_from=pbase)
        pbase = pbase or Lc
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        dsa.dsa_index_k_store(Lc.k_new, Lc.rows, Lc.pages, Lc.index_cache[0], LN_EPS, THETA)
        dsa.dsa_quant_fp8(Lc.q_idx, Lc.q8, Lc.qs)
        ev[1].record(stream)
        Lc.indexer_topk(0)
        ev[2].record(stream)
        Lc.mla(0)
        ev[3].record(stream)
        torch.cuda.synchronize()
        cp.append([ev[i].elapsed_time(ev[i + 1]) for i in range(3)])
        if Lc is not pbase:
            del Lc
    del pbase
    torch.cuda.empty_cache()
    cp = np.array(cp)                                           # ms: store + quant, indexer + top-k, MLA
    ppos = pw.row_pos.astype(np.int64)
    score_flops = int(((ppos + 1) * (ppos + 1 > 2048)).sum()) * 32 * 128 * 2
    mla_flops = int(np.minimum(ppos + 1, 2048).sum()) * 2 * 64 * (576 + 512)
    idx_s, mla_s = cp[:, 1].sum() / 1e3, cp[:, 2].sum() / 1e3
    return {"about": "one 1,048,576-token prompt prefilled in 32 chunks of 32,768 rows, one full layer: store + q "
                     "quantisation, indexer + top-2048 in row chunks (4 GiB logits scratch per launch), sparse MLA; "
                     "the indexer's scoring FLOPs are the rows' visible keys x 32 heads x 128 dims x 2",
            "chunks": int(len(cp)), "chunk_rows": int(n_chunk_rows), "logits_budget_bytes": PREFILL_LOGITS_BUDGET,
            "layer_ms": round(float(cp.sum()), 2), "store_quant_ms": round(float(cp[:, 0].sum()), 2),
            "indexer_topk_ms": round(float(cp[:, 1].sum()), 2), "sparse_mla_ms": round(float(cp[:, 2].sum()), 2),
            "indexer_scoring_flops": score_flops, "indexer_TFLOPs": round(score_flops / idx_s / 1e12, 1),
            "indexer_frac_of_fp8_peak": round(score_flops / idx_s / 1e12 / FP8_PEAK_TFLOPS, 4),
            "mla_flops": mla_flops, "mla_TFLOPs": round(mla_flops / mla_s / 1e12, 1),
            "mla_frac_of_bf16_peak": round(mla_flops / mla_s / 1e12 / BF16_PEAK_TFLOPS, 4),
            "chunk_ms_first_middle_last": [round(float(cp[i].sum()), 2) for i in (0, len(cp) // 2, len(cp) - 1)]}


def run_c4(torch, dsa, timer, a):
    """8192-row chunked prefill on a 65,536-token prefix (the footprint exceeds 1 GB: no rotation)."""
    import numpy as np
    import dsa_inputs as gi
    w = gi.config(4)
    res = measure_layer(torch, dsa, timer, w, max(5, a.steps // 2), 2, rotate=False, prefill=True)
    pos = w.row_pos.astype(np.int64)
    score_flops = int((pos + 1).sum()) * 32 * 128 * 2
    mla_flops = MLA_FLOPS_PER_ROW * w.R
    st = res["stage_us_median"]
    res["indexer_topk_TFLOPs"] = round(score_flops / (st["indexer_topk"] * 1e-6) / 1e12, 1)
    res["indexer_topk_frac_fp8"] = round(res["indexer_topk_TFLOPs"] / FP8_PEAK_TFLOPS, 4)
    res["plain_logits_TFLOPs"] = round(score_flops / (res["index_k"]["plain_logits_us"] * 1e-6) / 1e12, 1)
    res["plain_logits_frac_fp8"] = round(res["plain_logits_TFLOPs"] / FP8_PEAK_TFLOPS, 4)
    res["mla_TFLOPs"] = round(mla_flops / (st["mla"] * 1e-6) / 1e12, 1)
    res["mla_frac_fp8"] = round(res["mla_TFLOPs"] / FP8_PEAK_TFLOPS, 4)
    res["mla_frac_bf16"] = round(res["mla_TFLOPs"] / BF16_PEAK_TFLOPS, 4)
    res["scoring_flops"], res["mla_flops"] = score_flops, mla_flops
    return res


def run_copy(torch):
    """A plain 2 GiB device copy (read + write counted): the achievable streaming rate beside the
    nominal peak."""
    x = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    e0.record()
    for _ in range(n):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    del x, y
    torch.cuda.empty_cache()
    gbps = 2 * (2 << 30) / (us * 1e-6) / 1e9
    return {"about": "torch device copy of 2 GiB, bytes read + written per second", "GBps": round(gbps, 1),
            "frac_of_nominal": frac(gbps)}


def run_read(torch):
    """A plain streaming read: torch's sum over 2 GiB of fp32 (bytes read per second), the practical
    read rate beside the nominal peak (the indexer's index-K scan is a read of this kind)."""
    x = torch.ones((2 << 30) // 4, dtype=torch.float32, device="cuda")
    for _ in range(2):
        s = x.sum()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    e0.record()
    for _ in range(n):
        s = x.sum()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    assert abs(float(s) - x.numel()) <= 1e-3 * x.numel()
    del x
    torch.cuda.empty_cache()
    gbps = (2 << 30) / (us * 1e-6) / 1e9
    return {"about": "torch sum over 2 GiB of fp32, bytes read per second", "GBps": round(gbps, 1),
            "frac_of_nominal": frac(gbps)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--configs", default=",".join(SECTIONS),
                    help="comma list of sections: " + ",".join(SECTIONS) + " (the JSON line needs c2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true", help="also run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("SECTION", "FETCH_CSV", "WRITE_CSV", "COMMAND"),
                    help="merge two rocprofv3 --pmc counter files of one section into the traffic summary")
    ap.add_argument("--write-stats", nargs=4, metavar=("SECTION", "STATS_CSV", "COMMAND", "TITLE"),
                    help="merge a rocprofv3 --stats kernel summary of one section into the stats summary")
    ap.add_argument("--write-counters", nargs=4, metavar=("SECTION", "CSVS", "COMMANDS", "TITLE"),
                    help="summarise rocprofv3 --pmc passes (comma-separated counter csv files) of one section")
    a = ap.parse_args()
    if a.write_counters:
        print(write_counters(*a.write_counters))
        return
    if a.write_traffic:
        print(json.dumps(write_traffic(*a.write_traffic), indent=1))
        return
    if a.write_stats:
        print(json.dumps(write_stats(*a.write_stats), indent=1))
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    secs = [s for s in a.configs.split(",") if s]
    bad = [s for s in secs if s not in SECTIONS]
    if bad:
        sys.exit(f"unknown section(s) {bad}; choose from {SECTIONS}")

    import numpy as np
    import torch

    import dsa_inputs as gi
    from sparse_attention_store_amd import dsa

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream)
    out = {"metric": METRIC, "value": None, "unit": "query-tokens/s", "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "fp8 (index-K scores, MLA QK) + bf16 (MLA PV), fp32 accumulation",
           "data": "synthetic (seeded N(0,1) keys/latents/queries, U(0,1)/sqrt(32) head weights)",
           "config": {"workload": "c2 speculative verify: 64 requests x 6 rows, ctx 131072, page 64, 4-layer group "
                                  "(1 full + 3 shared), top-2048",
                      "value_def": "query tokens / s of the full layer (store + quant + fused indexer/top-k + "
                                   "sparse MLA); ms_per_step is the 4-layer group"}}
    if a.copy_probe:
        x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        del x, y
    D = None
    if "c2" in secs:
        r = run_c2(torch, dsa, timer, a, stream)
        D = r.pop("_layer")
        out.update(r)
        print(f"[bench] c2 full layer {r['c2']['full_layer_us']:.1f} us, group {r['ms_per_step'] * 1e3:.1f} us",
              file=sys.stderr, flush=True)
        if "mxfp4" in secs:
            out["mxfp4_index"] = run_mxfp4(torch, dsa, timer, D, a)
            out["mxfp4_index"]["full_layer_us"] = round(
                out["c2"]["stage_us_mean"]["store"] + out["c2"]["stage_us_mean"]["quant"] +
                out["mxfp4_index"]["indexer_topk_us"] + out["c2"]["stage_us_mean"]["mla0"], 2)
        if "mtp" in secs:
            n_mtp = max(3, a.steps // 4)
            carry = timer.calls(lambda i: D.mtp_draft_round(carry=True, steps=5), n_mtp)
            plain = timer.calls(lambda i: D.mtp_draft_round(carry=False, steps=5), n_mtp)
            out["mtp_draft_round"] = {
                "about": "one MTP draft iteration: 5 steps x 64 rows (one per request), indexer + top-k + sparse "
                         "MLA per step; the carry reuses step 0's top-k in steps 1-4",
                "with_carry_us": round(carry, 2), "without_carry_us": round(plain, 2),
                "indexer_read_bytes_saved": 4 * indexer_bytes(D.w.ctx, 0)}
        del D
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    n_cfg = max(50, a.steps)
    cfgs = {}
    for cid in (0, 1, 3):
        if f"c{cid}" in secs:
            w = gi.config(cid)
            cfgs[f"c{cid}"] = measure_layer(torch, dsa, timer, w, n_cfg, 10)
            print(f"[bench] c{cid}: full layer {cfgs[f'c{cid}']['full_layer_us']:.1f} us", file=sys.stderr, flush=True)
    if "sweep" in secs:
        sweep = []
        for e in range(10, 21):
            w = gi.make_decode(f"sweep_{1 << e}", gi.SEED_BASE + 50, [1 << e])
            r = measure_layer(torch, dsa, timer, w, n_cfg, 10)
            r["ctx"] = 1 << e
            sweep.append(r)
        cfgs["sweep"] = sweep
        print("[bench] sweep done", file=sys.stderr, flush=True)
    if "c4" in secs:
        cfgs["c4"] = run_c4(torch, dsa, timer, a)
        print(f"[bench] c4: full layer {cfgs['c4']['full_layer_us']:.1f} us", file=sys.stderr, flush=True)
    if cfgs:
        out["configs"] = cfgs
    if "fused_store" in secs:
        out["fused_norm_rope_store"] = run_fused_store(torch, dsa, timer, a, stream)
    if "prefill1m" in secs:
        out["chunked_prefill_1m"] = run_prefill1m(torch, dsa, stream)
        print(f"[bench] chunked prefill 1M: layer {out['chunked_prefill_1m']['layer_ms']:.1f} ms", file=sys.stderr,
              flush=True)
    if "copy" in secs:
        out["hbm_measured_copy"] = run_copy(torch)
        out["hbm_measured_read"] = run_read(torch)
    if not a.no_cpu_baseline and "c2" in secs:
        print("[bench] timing the oracle on host cores", file=sys.stderr, flush=True)
        threads = _omp_threads()
        base = cpu_baselines(threads)
        c2b = base["c2"]
        out["cpu_baseline"] = {
            "value": c2b["query_tokens_per_s"], "unit": "query-tokens/s", "cores": c2b["threads_busy"],
            "kind": "oracle",
            "sample": f"c2 full layer (store + quant + logits + top-k + sparse MLA) on 4 of 64 requests (24 rows at "
                      f"ctx 131072), {c2b['full_layer_s']:.1f} s; {threads} OpenMP threads over rows, "
                      f"{base['cpu']}"}
        out["cpu_baseline_configs"] = base
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
