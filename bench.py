#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X.

A *step* is one pass of the hot path over one synthetic batch: the
once-per-batch plan, then for each of ``--layers`` layers (each with its own
K/V pools, so the 256 MB last-level cache cannot serve a layer from the
previous one) the store of the step's new K/V rows and the attention call.

The headline workload is the bf16 decode batch (B=64, 32 q / 8 kv heads,
d=128, page 16, cached lengths U[512,4096]); ``value`` is its KV-read
throughput: K+V bytes attended per step / step time.  The extend (prefill),
long-context decode and 8-bit decode workloads are reported in
``secondary`` with their own roofline figures.

Prints ONE JSON line.  Inputs are resident in HBM before timing starts.

Timing: ``ms_per_step`` spans the K timed steps (two events around them).
Inside each step the stores of all layers are issued first and the attention
calls of all layers follow back to back, bracketed by one event pair; the
``roofline`` launch duration is that bracket divided by the layer count.  A
decode attention call is the split-KV kernel followed by its merge kernel,
so its duration is the sum of both kernels' times in a kernel trace.

Two helper modes feed the ``traffic`` field of ``roofline``:
``--copy-calibration`` runs a plain copy kernel of known size (1 GiB read,
1 GiB written) for a counter run, and ``--ingest-counters`` turns the
rocprofv3 ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` CSV files of a workload
and of that copy into ``profiles/traffic_<workload>.json``.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode KV-read GB/s (% of HBM peak); extend TFLOP/s (% of MFMA peak)"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "flashattention_paged_kv_amd", "csrc")

KERNEL_SOURCES = {
    "decode_n4_bf16": ["decode_bf16.hip", "decode_stream.h", "decode_merge.h", "plan.hip", "device_common.h"],
    "decode_bf16": ["decode_bf16.hip", "decode_stream.h", "decode_merge.h", "plan.hip", "device_common.h"],
    "long_decode_bf16": ["decode_bf16.hip", "decode_stream.h", "decode_merge.h", "plan.hip", "device_common.h"],
    "single_decode_bf16": ["decode_bf16.hip", "decode_stream.h", "decode_merge.h", "plan.hip", "device_common.h"],
    "decode_fp8": ["decode_fp8.hip", "decode_stream.h", "decode_merge.h", "plan.hip", "device_common.h"],
    "decode_int8": ["decode_fp8.hip", "decode_stream.h", "decode_merge.h", "plan.hip", "device_common.h"],
    "extend_bf16": ["extend_bf16.hip", "lds_dma.h", "plan.hip", "device_common.h"],
    "extend_fp8": ["extend_fp8.hip", "lds_dma.h", "plan.hip", "device_common.h"],
    "sparse_decode_bf16": ["decode_bf16.hip", "decode_stream.h", "decode_merge.h", "plan.hip", "device_common.h",
                           "block_sparse.hip"],
    "sparse_decode_fp8": ["decode_fp8.hip", "decode_stream.h", "decode_merge.h", "plan.hip", "device_common.h",
                          "block_sparse.hip"],
}


def source_hash(workload: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[workload]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_counters(workload: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, or None when
    the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != source_hash(workload):
        return None
    return t.get("traffic_bytes_per_launch")


# Kernels that make up one attention call of each workload, as rocprofv3 names them.
CALL_KERNELS = {
    "decode_bf16": ("decode_bf16_kernel", "decode_merge"),
    "long_decode_bf16": ("decode_bf16_kernel", "decode_merge"),
    "single_decode_bf16": ("decode_bf16_kernel", "decode_merge"),
    "decode_fp8": ("decode_fp8_kernel", "decode_merge"),
    "decode_int8": ("decode_fp8_kernel", "decode_merge"),
    "decode_n4_bf16": ("decode_bf16_kernel", "decode_merge"),
    "extend_bf16": ("extend_bf16_kernel",),
    "extend_fp8": ("extend_fp8_kernel",),
    "sparse_decode_bf16": ("decode_bf16_kernel", "decode_merge"),
    "sparse_decode_fp8": ("decode_fp8_kernel", "decode_merge"),
}
COPY_BYTES = 1 << 30


def _counter_per_dispatch(path: str, counter: str):
    """{kernel substring match -> (dispatches, average value)} from a rocprofv3 counter CSV."""
    import collections
    import csv
    per = collections.defaultdict(float)
    names = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
    return per, names


def _avg_for(per, names, needle):
    vals = [v for d, v in per.items() if needle in names[d]]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {needle!r} in the counter file")
    return len(vals), sum(vals) / len(vals)


def ingest_counters(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, commands):
    """Scale the kernels' FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what the
    same counters read for the plain 1 GiB copy, and store bytes per attention call."""
    cf, cn = _counter_per_dispatch(copy_fetch_csv, "FETCH_SIZE")
    cw, cwn = _counter_per_dispatch(copy_write_csv, "WRITE_SIZE")
    # the copy is the only kernel with a 1 GiB footprint: take the largest dispatches
    copy_fetch = max(cf.values()) * 1024.0
    copy_write = max(cw.values()) * 1024.0
    fetch_factor, write_factor = copy_fetch / COPY_BYTES, copy_write / COPY_BYTES
    kf, kfn = _counter_per_dispatch(fetch_csv, "FETCH_SIZE")
    kw, kwn = _counter_per_dispatch(write_csv, "WRITE_SIZE")
    kernels = {}
    total = 0.0
    for k in CALL_KERNELS[workload]:
        nf, f = _avg_for(kf, kfn, k)
        nw, w = _avg_for(kw, kwn, k)
        fb, wb = f * 1024.0 / fetch_factor, w * 1024.0 / write_factor
        kernels[k] = {"dispatches": [nf, nw], "fetch_kib": round(f, 1), "write_kib": round(w, 1),
                      "fetch_bytes": round(fb), "write_bytes": round(wb)}
        total += fb + wb
    out = {"workload": workload, "source_sha": source_hash(workload), "kernels": kernels,
           "copy_calibration": {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                                "fetch_factor": round(fetch_factor, 4), "write_factor": round(write_factor, 4)},
           "traffic_bytes_per_launch": round(total), "commands": commands}
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


SIMDS = 1024  # MI355X: 256 CUs x 4 SIMDs
SQ_ENGINES = 32  # the SQ cycle counters add up over 32 shader engines (8 XCDs x 4)


def summarize_sq_counters(workload, csv_paths, commands):
    """Per-dispatch averages of the SQ counters in rocprofv3 --pmc CSV files for
    the workload's main kernel, with derived utilisations, written to
    profiles/<kernel>.sq_counters.<workload>.txt."""
    import collections
    import csv
    kernel = CALL_KERNELS[workload][0]
    avg = {}
    dispatches = 0
    for path in csv_paths:
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        with open(path) as f:
            for r in csv.DictReader(f):
                if kernel in r["Kernel_Name"]:
                    per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
        if not per:
            raise SystemExit(f"no dispatch of {kernel} in {path}")
        dispatches = len(per)
        for name in {k for v in per.values() for k in v}:
            avg[name] = sum(v.get(name, 0.0) for v in per.values()) / len(per)
    lines = [f"SQ counters of {kernel}, workload {workload} ({dispatches} dispatches averaged per pass)",
             f"source sha {source_hash(workload)}", "", "commands:"] + [f"  {c}" for c in commands] + ["", "per dispatch:"]
    lines += [f"  {k:32s} {v:14.6g}" for k, v in sorted(avg.items())]
    cyc = avg.get("SQ_CYCLES", 0.0) / SQ_ENGINES  # kernel cycles
    if cyc > 0:
        lines += ["", "derived (kernel cycles = SQ_CYCLES / 32 shader engines; per SIMD = / 1024 SIMDs):",
                  f"  kernel cycles                          {cyc:14.6g}"]
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            lines.append(f"  matrix cores busy (share of SIMD time)  {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / SIMDS / cyc:14.3f}")
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg and avg.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            lines.append(f"  MFMA busy cycles with VALU co-issue     "
                         f"{avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / avg['SQ_VALU_MFMA_BUSY_CYCLES']:14.3f}")
        if "SQ_INSTS_VALU" in avg:
            lines.append(f"  VALU instructions per SIMD cycle        {avg['SQ_INSTS_VALU'] / SIMDS / cyc:14.4f}")
        if "SQ_INSTS_VALU_TRANS_F32" in avg and "SQ_INSTS_MFMA" in avg:
            lines.append(f"  VALU instructions per MFMA              {avg['SQ_INSTS_VALU'] / avg['SQ_INSTS_MFMA']:14.2f}")
            lines.append(f"  transcendental instructions per MFMA    "
                         f"{avg['SQ_INSTS_VALU_TRANS_F32'] / avg['SQ_INSTS_MFMA']:14.2f}")
    if avg.get("SQ_INSTS_LDS"):
        lines.append(f"  LDS bank-conflict cycles per LDS instr  {avg.get('SQ_LDS_BANK_CONFLICT', 0.0) / avg['SQ_INSTS_LDS']:14.3f}")
    path = os.path.join(PROFILES, f"{kernel}.sq_counters.{workload}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(workload, stats_csv, bench_log, command):
    """profiles/<kernel>.<workload>.txt from a rocprofv3 --kernel-trace --stats
    run of bench.py: the library kernels' call counts and durations, and the
    bench line of the same run."""
    import csv
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            name = r["Name"]
            if "pkv::" not in name:
                continue  # torch's own set-up kernels
            rows.append((name, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(key=lambda t: -t[1] * t[2])
    with open(bench_log) as f:
        line = json.loads([x for x in f if x.startswith("{")][-1])
    roof = line["roofline"]
    call = [t for t in rows if any(k in t[0] for k in CALL_KERNELS[workload])]
    kernel = CALL_KERNELS[workload][0]
    out = [f"# rocprofv3 kernel trace: {kernel} on the {workload} workload", "",
           "Command (repo root on one MI355X; TMPDIR=/tmp):", f"  {command}", "",
           "Library kernels (from the kernel_stats.csv of that run; torch set-up kernels omitted):", "",
           f"  {'kernel':58s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s} {'share':>7s}"]
    for name, calls, avg, mn, mx, pct in rows:
        short = name.split("(")[0]
        out.append(f"  {short[:58]:58s} {calls:6d} {avg:9.2f} {mn:9.2f} {mx:9.2f} {pct:6.1f}%")
    total = 0.0
    seen = set()
    for k in CALL_KERNELS[workload]:
        for name, calls, avg, *_ in call:
            if k in name and name not in seen:
                seen.add(name)
                total += avg
    unit = roof["unit"]
    work = roof.get("algorithmic_bytes_per_launch") or roof.get("algorithmic_flops_per_launch")
    out += ["", f"One attention call = {' + '.join(CALL_KERNELS[workload])}: sum of averages {total:.2f} us.",
            f"The same run's bench line (HIP events around the attention block, per call): avg_launch_us "
            f"{roof['avg_launch_us']}, achieved {roof['achieved']} {unit} = {100 * roof['frac']:.1f}% of "
            f"{roof['peak']} {unit}.",
            f"Algorithmic work per call: {work} " + ("bytes (K+V read)" if unit == "GB/s" else "flops (4*d*Hq per unmasked pair)"),
            f"Step time in that run: {line['ms_per_step']} ms ({line['config'].get('layers_per_step')} layers/step).",
            f"Kernel sources sha {source_hash(workload)}."]
    path = os.path.join(PROFILES, f"{kernel}.{workload}.txt")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def copy_calibration():
    """A plain streaming kernel of known size: 1 GiB read once, 1 GiB written once."""
    import torch
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "kernel": "torch.neg (bf16 elementwise)"}), flush=True)


# ---------------------------------------------------------------- oracle timing (cpu_baseline)
def _rows_host(pool, rows):
    """Pool rows [L, Hkv, d] of one request, copied to the host: float32 for
    bf16 pools (exact), the raw codes for 8-bit pools."""
    import torch
    t = pool[rows]
    return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy()


def _q_host(q):
    import torch
    return (q.float() if q.dtype == torch.bfloat16 else q).cpu().numpy()


def time_oracle(units, budget_s):
    """Run ``units`` (an iterator of (prepare, run, work) triples: prepare
    copies a unit's inputs to the host and is not timed, run is one oracle
    call) until ``budget_s`` seconds of oracle time are spent.  Returns
    (work done, oracle seconds, units run)."""
    done, spent, n = 0, 0.0, 0
    for prepare, run, work in units:
        args = prepare()
        t0 = time.perf_counter()
        run(*args)
        spent += time.perf_counter() - t0
        done += work
        n += 1
        if spent >= budget_s:
            break
    return done, spent, n


def _cycle(seq):
    while True:
        for x in seq:
            yield x


# ---------------------------------------------------------------- workloads
KV_DTYPE_NAMES = {"bf16": "bf16", "fp8": "fp8_e4m3", "int8": "int8 q/k (sage), fp8_e4m3 v"}


class DecodeRunner:
    def __init__(self, name, layers, torch, pkv, workloads):
        self.torch, self.pkv = torch, pkv
        spec = workloads.SPECS[name]
        self.spec = spec
        self.fp8 = spec.dtype in ("fp8", "int8")  # the 8-bit Sage path (E4M3, or INT8 Q/K)
        self.qk_codes = "int8" if spec.dtype == "int8" else "e4m3"
        self.db = workloads.make_device_batch(spec, seed=0, layers=layers)
        lay = self.db.layout
        self.layers = layers
        kv_dtype = pkv.PKV_SAGE_INT8 if spec.dtype == "int8" else pkv.PKV_FP8_E4M3
        kw = dict(kv_dtype=kv_dtype, q_block=spec.q_block, k_block=spec.k_block) if self.fp8 else {}
        self.q_len = int(lay.new_lens[0])  # new tokens per request
        self.params = pkv.Params(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                                 max_kv_len=lay.req_to_token.shape[1], decode_q_len=self.q_len, **kw)
        ws_bytes, sc_bytes = pkv.workspace_size(self.params, pkv.PKV_DECODE, spec.batch)
        self.ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        self.scratch = torch.empty(max(sc_bytes, 16), dtype=torch.uint8, device="cuda")
        rows = spec.batch * self.q_len
        self.out = [torch.empty((rows, spec.num_q_heads, spec.head_dim), dtype=torch.bfloat16, device="cuda")
                    for _ in range(layers)]
        self.lse = torch.empty((rows, spec.num_q_heads), dtype=torch.float32, device="cuda")
        esize = 1 if self.fp8 else 2
        tokens = int(lay.seq_lens.astype("int64").sum())
        self.kv_bytes_per_layer = tokens * spec.num_kv_heads * spec.head_dim * 2 * esize
        self.work_per_step = self.kv_bytes_per_layer * layers

    def pre(self):
        """The once-per-step work: the plan and every layer's K/V store."""
        pkv, db = self.pkv, self.db
        self.plan = pkv.plan_metadata(self.params, pkv.PKV_DECODE, db.seq_lens, workspace=self.ws)
        for l in range(self.layers):
            pkv.kv_store(self.params, db.k_pools[l], db.v_pools[l], db.k_new[l], db.v_new[l], db.new_slots)

    plan_per_layer = False  # --plan-per-layer: re-plan before every layer (the pattern the plan replaces)

    def attn(self):
        """Every layer's attention call, back to back."""
        pkv, db = self.pkv, self.db
        for l in range(self.layers):
            if self.plan_per_layer:
                self.plan = pkv.plan_metadata(self.params, pkv.PKV_DECODE, db.seq_lens, workspace=self.ws)
            pkv.attn_decode(self.params, db.q, db.k_pools[l], db.v_pools[l], db.req_to_token, db.seq_lens, self.plan,
                            scratch=self.scratch, out=self.out[l], lse=self.lse,
                            sfq=db.sfq, sfk=db.sfk, sfv=db.sfv)

    def describe(self):
        s = self.spec
        lo, hi = s.prefix
        cached = f"{lo}" if lo == hi else f"U[{lo},{hi}]"
        return {"workload": s.name, "batch": s.batch, "num_q_heads": s.num_q_heads, "num_kv_heads": s.num_kv_heads,
                "head_dim": s.head_dim, "page_size": s.page_size,
                "cached_len": f"{cached} + {self.q_len} new token{'s' if self.q_len > 1 else ''}",
                "kv_dtype": KV_DTYPE_NAMES[s.dtype], "layers_per_step": self.layers,
                "kv_bytes_per_layer": self.kv_bytes_per_layer}

    def roofline(self, avg_launch_s, workload):
        achieved = self.kv_bytes_per_layer / avg_launch_s / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic_from_counters(workload),
                "kernel": " + ".join(CALL_KERNELS[workload]),
                "algorithmic_bytes_per_launch": self.kv_bytes_per_layer,
                "avg_launch_us": round(avg_launch_s * 1e6, 2)}

    def _oracle_units(self, oracle):
        """One unit per request of layer 0: all heads of its new-token rows."""
        db, spec = self.db, self.spec
        lay = db.layout
        q = _q_host(db.q)
        sc = [t.cpu().numpy() for t in (db.sfq, db.sfk, db.sfv)] if self.fp8 else None
        esize = 1 if self.fp8 else 2
        nq = self.q_len

        def unit(b):
            L = int(lay.seq_lens[b])
            rows = db.req_to_token[b, :L].long()
            prepare = lambda: (_rows_host(db.k_pools[0], rows), _rows_host(db.v_pools[0], rows))
            rtt = np.arange(L)[None]
            if self.fp8:
                run = lambda K, V: oracle.sage_decode(q[b:b + 1], K, V, rtt, [L], sc[0][b:b + 1], sc[1][b:b + 1],
                                                      sc[2][b:b + 1], k_block=spec.k_block, qk_codes=self.qk_codes)
            else:
                run = lambda K, V: oracle.paged_attention(q[b * nq:(b + 1) * nq], K, V, rtt, [L], [0, nq])
            return prepare, run, L * spec.num_kv_heads * spec.head_dim * 2 * esize

        return (unit(b) for b in _cycle(range(spec.batch)))

    def cpu_baseline(self, budget_s, oracle):
        """The fp64 oracle on layer 0 of the same batch, request by request
        (each request's rows gathered on the device and copied to the host
        untimed) until ``budget_s`` seconds of oracle time are spent."""
        spec = self.spec
        done, dt, n = time_oracle(self._oracle_units(oracle), budget_s)
        return {"value": round(done / dt / 1e9, 4), "unit": "GB/s", "seconds": round(dt, 2),
                "sample": f"layer 0 of {spec.name}: {n} request-attentions ({n / spec.batch:.2f} passes over "
                          f"the {spec.batch}-request batch), all {spec.num_q_heads} heads, fp64"}


class SparseDecodeRunner(DecodeRunner):
    """Block-sparse decode: once per batch the compacted page table of the
    listed blocks (and its sfK), then the plan over the selected lengths; the
    attention calls run on that table.  Work per layer = K+V bytes of the
    selected keys."""

    def __init__(self, name, layers, torch, pkv, workloads):
        super().__init__(name, layers, torch, pkv, workloads)
        lay, spec = self.db.layout, self.spec
        bs = spec.sparse_block
        sel = 0
        for b in range(spec.batch):
            L = int(lay.seq_lens[b])
            for k in lay.blk_indices[lay.blk_indptr[b]:lay.blk_indptr[b + 1]]:
                sel += max(0, min(bs, L - int(k) * bs))
        self.selected_tokens = sel
        esize = 1 if self.fp8 else 2
        self.kv_bytes_per_layer = sel * spec.num_kv_heads * spec.head_dim * 2 * esize
        self.work_per_step = self.kv_bytes_per_layer * layers

    def pre(self):
        """The once-per-step work: every layer's K/V store, the sparse tables and the plan."""
        pkv, db = self.pkv, self.db
        for l in range(self.layers):
            pkv.kv_store(self.params, db.k_pools[l], db.v_pools[l], db.k_new[l], db.v_new[l], db.new_slots)
        self.srtt, self.slens, self.ssfk = pkv.block_sparse_table(
            self.params, db.seq_lens, db.req_to_token, db.blk_indptr, db.blk_indices, self.spec.sparse_block,
            sfk=db.sfk)
        self.plan = pkv.plan_metadata(self.params, pkv.PKV_DECODE, self.slens, workspace=self.ws)

    def attn(self):
        pkv, db = self.pkv, self.db
        for l in range(self.layers):
            pkv.attn_decode(self.params, db.q, db.k_pools[l], db.v_pools[l], self.srtt, self.slens, self.plan,
                            scratch=self.scratch, out=self.out[l], lse=self.lse,
                            sfq=db.sfq, sfk=self.ssfk, sfv=db.sfv)

    def describe(self):
        d = super().describe()
        d.update({"block_size": self.spec.sparse_block, "density": self.spec.density,
                  "selected_tokens": self.selected_tokens})
        return d

    def _oracle_units(self, oracle):
        """One unit per (request, kv head) of layer 0: that head's query heads
        over the request's listed blocks (a whole 40-head request of this
        workload takes the 8-bit oracle tens of seconds)."""
        db, spec = self.db, self.spec
        lay = db.layout
        q = _q_host(db.q)
        sc = [t.cpu().numpy() for t in (db.sfq, db.sfk, db.sfv)] if self.fp8 else None
        bs = spec.sparse_block
        esize = 1 if self.fp8 else 2
        G = spec.num_q_heads // spec.num_kv_heads

        def unit(b, g):
            L = int(lay.seq_lens[b])
            rows = db.req_to_token[b, :L].long()
            blocks = lay.blk_indices[lay.blk_indptr[b]:lay.blk_indptr[b + 1]]
            ip = [0, len(blocks)]
            rtt = np.arange(L)[None]
            hs = slice(g * G, (g + 1) * G)
            prepare = lambda: (_rows_host(db.k_pools[0][:, g:g + 1], rows), _rows_host(db.v_pools[0][:, g:g + 1], rows))
            if self.fp8:
                run = lambda K, V: oracle.block_sparse_sage_decode(q[b:b + 1, hs], K, V, rtt, [L], ip, blocks, bs,
                                                                   sc[0][b:b + 1, hs], sc[1][b:b + 1, g:g + 1],
                                                                   sc[2][b:b + 1, g:g + 1], spec.k_block,
                                                                   qk_codes=self.qk_codes)
            else:
                run = lambda K, V: oracle.block_sparse_decode(q[b:b + 1, hs], K, V, rtt, [L], ip, blocks, bs)
            sel = sum(max(0, min(bs, L - int(k) * bs)) for k in blocks)
            return prepare, run, sel * spec.head_dim * 2 * esize

        order = [(b, g) for b in range(spec.batch) for g in range(spec.num_kv_heads)]
        return (unit(b, g) for b, g in _cycle(order))

    def cpu_baseline(self, budget_s, oracle):
        """The fp64 block-sparse oracle on layer 0, request by request, until
        ``budget_s`` seconds of oracle time are spent."""
        spec = self.spec
        done, dt, n = time_oracle(self._oracle_units(oracle), budget_s)
        return {"value": round(done / dt / 1e9, 4), "unit": "GB/s", "seconds": round(dt, 2),
                "sample": f"layer 0 of {spec.name}: {n} (request, kv head) attentions over the request's "
                          f"listed blocks ({n / spec.num_kv_heads:.2f} requests' worth, all heads), fp64"}


class ExtendRunner:
    def __init__(self, name, layers, torch, pkv, workloads):
        self.torch, self.pkv = torch, pkv
        spec = workloads.SPECS[name]
        self.spec = spec
        self.fp8 = spec.dtype == "fp8"
        self.db = workloads.make_device_batch(spec, seed=0, layers=layers)
        lay = self.db.layout
        self.layers = layers
        kw = dict(kv_dtype=pkv.PKV_FP8_E4M3, q_block=1, k_block=spec.k_block) if self.fp8 else {}
        self.params = pkv.Params(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size,
                                 max_kv_len=lay.req_to_token.shape[1], **kw)
        self.total_q = lay.total_q
        ws_bytes, _ = pkv.workspace_size(self.params, pkv.PKV_EXTEND, spec.batch, self.total_q)
        self.ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        self.out = [torch.empty((self.total_q, spec.num_q_heads, spec.head_dim), dtype=torch.bfloat16, device="cuda")
                    for _ in range(layers)]
        self.lse = torch.empty((self.total_q, spec.num_q_heads), dtype=torch.float32, device="cuda")
        n = lay.new_lens.astype("int64")
        p = lay.prefix_lens.astype("int64")
        pairs = int((n * p + n * (n + 1) // 2).sum())  # unmasked (query, key) pairs per head
        self.flops_per_layer = 4 * spec.head_dim * spec.num_q_heads * pairs
        # context only: the same rows against all of their request's keys, no causal mask
        self.dense_equivalent_flops = 4 * spec.head_dim * spec.num_q_heads * int((n * (n + p)).sum())
        self.work_per_step = self.flops_per_layer * layers

    def pre(self):
        """The once-per-step work: the plan and every layer's K/V store."""
        pkv, db = self.pkv, self.db
        self.plan = pkv.plan_metadata(self.params, pkv.PKV_EXTEND, db.seq_lens, db.cu_seqlens_q,
                                      total_q=self.total_q, workspace=self.ws)
        for l in range(self.layers):
            pkv.kv_store(self.params, db.k_pools[l], db.v_pools[l], db.k_new[l], db.v_new[l], db.new_slots)

    def attn(self):
        """Every layer's attention call, back to back."""
        pkv, db = self.pkv, self.db
        for l in range(self.layers):
            pkv.attn_extend(self.params, db.q, db.k_pools[l], db.v_pools[l], db.req_to_token, db.seq_lens,
                            db.cu_seqlens_q, self.plan, out=self.out[l], lse=self.lse,
                            sfq=db.sfq, sfk=db.sfk, sfv=db.sfv)

    def describe(self):
        s = self.spec
        return {"workload": s.name, "batch": s.batch, "num_q_heads": s.num_q_heads, "num_kv_heads": s.num_kv_heads,
                "head_dim": s.head_dim, "page_size": s.page_size, "prefix_len": f"U{list(s.prefix)}",
                "new_len": f"U{list(s.new)}", "total_q": self.total_q, "layers_per_step": self.layers,
                "kv_dtype": "fp8_e4m3" if self.fp8 else "bf16", "flops_per_layer": self.flops_per_layer,
                "dense_equivalent_flops_per_layer": self.dense_equivalent_flops}

    def roofline(self, avg_launch_s, workload):
        achieved = self.flops_per_layer / avg_launch_s / 1e12
        peak = PEAK_FP8_TFLOPS if self.fp8 else PEAK_BF16_TFLOPS  # the contraction's own dtype
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_from_counters(workload),
                "kernel": "extend_fp8_kernel" if self.fp8 else "extend_bf16_kernel",
                "algorithmic_flops_per_launch": self.flops_per_layer, "avg_launch_us": round(avg_launch_s * 1e6, 2)}

    def _oracle_units(self, oracle):
        """bf16: one unit per request of layer 0 (every new-token row, all
        heads).  8-bit: one unit per new-token row (all heads over its
        visible keys, through the decode form of the formula), since the
        oracle's per-row loop makes a whole request take minutes."""
        db, spec = self.db, self.spec
        lay = db.layout
        q = _q_host(db.q)
        d, hq = spec.head_dim, spec.num_q_heads
        cu = lay.cu_seqlens_q
        if not self.fp8:
            def unit(b):
                L, n = int(lay.seq_lens[b]), int(cu[b + 1] - cu[b])
                rows = db.req_to_token[b, :L].long()
                prepare = lambda: (_rows_host(db.k_pools[0], rows), _rows_host(db.v_pools[0], rows))
                run = lambda K, V: oracle.paged_attention(q[cu[b]:cu[b + 1]], K, V, np.arange(L)[None], [L], [0, n])
                p = L - n
                return prepare, run, 4 * d * hq * (n * p + n * (n + 1) // 2)
            return (unit(b) for b in _cycle(range(spec.batch)))
        sfq, sfk, sfv = (t.cpu().numpy() for t in (db.sfq, db.sfk, db.sfv))

        def row_unit(b, t):
            L, n = int(lay.seq_lens[b]), int(cu[b + 1] - cu[b])
            vis = L - n + (t - int(cu[b])) + 1
            rows = db.req_to_token[b, :vis].long()
            prepare = lambda: (_rows_host(db.k_pools[0], rows), _rows_host(db.v_pools[0], rows))
            run = lambda K, V: oracle.sage_decode(q[t:t + 1], K, V, np.arange(vis)[None], [vis], sfq[t:t + 1],
                                                  sfk[b:b + 1], sfv[b:b + 1], spec.k_block)
            return prepare, run, 4 * d * hq * vis

        order = [(b, t) for b in range(spec.batch) for t in range(int(cu[b]), int(cu[b + 1]), 97)]
        return (row_unit(b, t) for b, t in _cycle(order))

    def cpu_baseline(self, budget_s, oracle):
        spec = self.spec
        done, dt, n = time_oracle(self._oracle_units(oracle), budget_s)
        what = (f"{n} requests (every new-token row, all {spec.num_q_heads} heads)" if not self.fp8 else
                f"{n} new-token rows (every 97th row of each request, all {spec.num_q_heads} heads over its "
                "visible keys)")
        return {"value": round(done / dt / 1e12, 6), "unit": "TFLOP/s", "seconds": round(dt, 2),
                "sample": f"layer 0 of {spec.name}: {what}, fp64; unmasked flops"}


RUNNERS = {"decode_bf16": DecodeRunner, "long_decode_bf16": DecodeRunner, "single_decode_bf16": DecodeRunner,
           "decode_fp8": DecodeRunner, "decode_int8": DecodeRunner,
           "decode_n4_bf16": DecodeRunner, "extend_bf16": ExtendRunner, "extend_fp8": ExtendRunner,
           "sparse_decode_bf16": SparseDecodeRunner, "sparse_decode_fp8": SparseDecodeRunner}
UNITS = {"decode_bf16": "GB/s", "long_decode_bf16": "GB/s", "single_decode_bf16": "GB/s", "decode_fp8": "GB/s",
         "decode_int8": "GB/s", "decode_n4_bf16": "GB/s",
         "extend_bf16": "TFLOP/s", "extend_fp8": "TFLOP/s", "sparse_decode_bf16": "GB/s", "sparse_decode_fp8": "GB/s"}
DEFAULT_LAYERS = {"decode_bf16": 4, "long_decode_bf16": 2, "single_decode_bf16": 4, "decode_fp8": 4, "decode_int8": 4, "decode_n4_bf16": 4, "extend_bf16": 4,
                  "extend_fp8": 4, "sparse_decode_bf16": 2, "sparse_decode_fp8": 2}


def capture(runner, torch):
    """The step as two HIP graphs (plan + stores, then the attention calls),
    captured once after an eager run on a side stream; replays reuse every
    buffer, as a serving loop does for its decode steps."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        runner.pre()
        runner.attn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g_pre, g_attn = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_pre):
        runner.pre()
    with torch.cuda.graph(g_attn):
        runner.attn()
    torch.cuda.synchronize()
    return g_pre.replay, g_attn.replay


def measure(name, steps, warmup, layers, torch, pkv, workloads, graph=False):
    runner = RUNNERS[name](name, layers or DEFAULT_LAYERS[name], torch, pkv, workloads)
    pre, attn = runner.pre, runner.attn
    for _ in range(warmup):
        pre()
        attn()
    torch.cuda.synchronize()
    if graph:
        pre, attn = capture(runner, torch)
        for _ in range(warmup):
            pre()
            attn()
    torch.cuda.synchronize()
    # one event pair per step around the attention block (all layers back to back):
    # every event record adds a few microseconds of queue gap, so none sit between launches
    blocks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        pre()
        blocks[i][0].record()
        attn()
        blocks[i][1].record()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    avg_launch_s = sum(a.elapsed_time(b) for a, b in blocks) / (steps * runner.layers) / 1e3
    scale = 1e9 if UNITS[name] == "GB/s" else 1e12
    value = runner.work_per_step / (ms / 1e3) / scale
    return runner, ms, value, runner.roofline(avg_launch_s, name)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


def cpu_baseline_of(runner, budget_s):
    """The oracle timed on the host cores on a bounded sample of the runner's workload."""
    import oracle
    cb = runner.cpu_baseline(budget_s, oracle)
    cb.update({"cores": _blas_threads(), "kind": "oracle"})
    return cb


def single_thread_baselines(runner, budget_s):
    """The oracle with its BLAS pool limited to one thread: on the headline
    batch (same sample rule) and on the tiny decode and extend batches (whole
    batch per call, repeated until the budget is spent)."""
    from threadpoolctl import threadpool_limits

    import oracle
    import workloads
    out = {}
    with threadpool_limits(limits=1):
        cb = runner.cpu_baseline(budget_s, oracle)
        cb.update({"cores": 1, "kind": "oracle"})
        out[runner.spec.name] = cb
        for name in ("tiny_decode", "tiny_extend"):
            hb = workloads.make_host_batch(workloads.SPECS[name], 0)
            lay, spec = hb.layout, hb.layout.spec
            q, kp, vp = (workloads.round_bf16(x) for x in (hb.q, hb.k_pool, hb.v_pool))
            n = lay.new_lens.astype("int64")
            p = lay.prefix_lens.astype("int64")
            if spec.mode == "decode":
                work, unit = int(lay.seq_lens.astype("int64").sum()) * spec.num_kv_heads * spec.head_dim * 2 * 2, "GB/s"
            else:
                work, unit = 4 * spec.head_dim * spec.num_q_heads * int((n * p + n * (n + 1) // 2).sum()), "TFLOP/s"
            run = lambda: oracle.paged_attention(q, kp, vp, lay.req_to_token, lay.seq_lens, lay.cu_seqlens_q)
            done, dt, calls = time_oracle(((lambda: (), run, work) for _ in iter(int, 1)), budget_s)
            scale = 1e9 if unit == "GB/s" else 1e12
            out[name] = {"value": round(done / dt / scale, 6), "unit": unit, "seconds": round(dt, 2),
                         "calls": calls, "us_per_call": round(dt / calls * 1e6, 1), "cores": 1, "kind": "oracle",
                         "sample": f"the whole {name} batch per call, fp64"}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_bf16", choices=sorted(RUNNERS))
    ap.add_argument("--layers", type=int, default=0, help="layers (distinct K/V pools) per step")
    ap.add_argument("--secondary", default="extend_bf16,long_decode_bf16,decode_fp8,decode_n4_bf16,extend_fp8,"
                                           "sparse_decode_bf16,sparse_decode_fp8,single_decode_bf16,decode_int8",
                    help="comma list of workloads reported under 'secondary' ('' for none)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--cpu-budget-secondary", type=float, default=3.0,
                    help="seconds of oracle work for each secondary workload's and each single-thread cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step as captured HIP graphs (plan + stores, then the attention calls) "
                         "instead of launching every kernel from Python")
    ap.add_argument("--copy-calibration", action="store_true", help="run only the 1 GiB copy (counter calibration)")
    ap.add_argument("--plan-per-layer", action="store_true",
                    help="decode: plan before every layer instead of once per batch (for comparison only)")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from rocprofv3 --pmc CSV files (host only)")
    ap.add_argument("--commands", default="", help="with --ingest-counters: the profiler commands, ' ;; '-separated")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("STATS_CSV", "BENCH_LOG"),
                    help="write profiles/<kernel>.<workload>.txt from a rocprofv3 --kernel-trace --stats run (host only)")
    ap.add_argument("--summarize-sq-counters", nargs="+", metavar="CSV",
                    help="write profiles/<kernel>.sq_counters.<workload>.txt from rocprofv3 --pmc CSV files (host only)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.workload, *args.summarize_trace, command=args.commands)
        return
    if args.summarize_sq_counters:
        summarize_sq_counters(args.workload, args.summarize_sq_counters,
                              [c.strip() for c in args.commands.split(";;") if c.strip()])
        return
    if args.ingest_counters:
        ingest_counters(args.workload, *args.ingest_counters,
                        commands=[c.strip() for c in args.commands.split(";;") if c.strip()])
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the path shards by request or kv head with no exchange)"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch

    import flashattention_paged_kv_amd as pkv
    import workloads

    pkv.load_library()  # fails loudly when the HIP library is missing
    graph = args.graph
    DecodeRunner.plan_per_layer = args.plan_per_layer
    runner, ms, value, roof = measure(args.workload, args.steps, args.warmup, args.layers, torch, pkv, workloads,
                                      graph=graph)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": UNITS[args.workload], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": {"fp8": "fp8_e4m3", "int8": "int8/fp8_e4m3"}.get(runner.spec.dtype, "bf16"),
        "data": "synthetic", "config": runner.describe(),
        "launch": ("hip_graph" if graph else "eager") + (", plan per layer" if args.plan_per_layer else ""),
        "roofline": roof,
    }
    secondary = {}
    for name in [s for s in args.secondary.split(",") if s and s != args.workload]:
        try:
            r2, ms2, v2, roof2 = measure(name, max(args.steps // 2, 5), max(args.warmup // 2, 2), 0, torch, pkv,
                                         workloads, graph=graph)
            secondary[name] = {"value": round(v2, 2), "unit": UNITS[name], "ms_per_step": round(ms2, 4),
                               "config": r2.describe(), "roofline": roof2}
            if not args.no_cpu_baseline:
                secondary[name]["cpu_baseline"] = cpu_baseline_of(r2, args.cpu_budget_secondary)
            del r2
        except Exception as e:  # a workload whose kernel is missing is reported, not hidden
            secondary[name] = {"error": f"{type(e).__name__}: {e}"}
        torch.cuda.empty_cache()
    if secondary:
        line["secondary"] = secondary
    if not args.no_cpu_baseline:
        cb = cpu_baseline_of(runner, args.cpu_budget)
        if args.workload == "decode_bf16":
            cb["single_thread"] = single_thread_baselines(runner, args.cpu_budget_secondary)
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
