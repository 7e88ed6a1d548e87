"""Throughput of the Kamera reuse operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--also A,B,...]

A step is one call of the workload's entry point (one fused launch covering
every layer and stream) over one batch of seeded synthetic input already
resident in HBM.  The default (headline) workload is the reorder shape: GQA,
36 layers, 8 KV heads x 128, 32 chunks x 2048 tokens (a 65,536-token context)
placed in a seeded order, rank-32 orbit patches on K and V, written into a
paged pool of 16-token pages -- the reuse configuration with the most bytes
(19.8 GB per call).  The single-frame (GQA, 28 layers, one 1024-token chunk),
sliding-window survival (m = 0, 64 chunks) and MLA (576-wide joint row, 16
chunks x 4096 tokens, 64-token pages) configurations are measured in the same
run, with the same fields, and reported inside the line as other_configs.
Workloads whose working set fits in the 256 MB Infinity Cache rotate over
enough independent input and pool sets (> 1.5 GB) that every step reads HBM.

Printed: one JSON line.  ``value`` is reconstructed-KV GB/s (canonical rows
read + pool rows written) over the whole timed region; ``roofline`` gives the
algorithmic bytes (rows + patch factors + index data) per launch over the
average launch time, against the 8 TB/s HBM peak; ``copy_ceiling`` gives what
a plain 16-byte copy of the same rows reaches (libkamera_probe.so: in the
kernel's own block pattern and walk order, in ascending address order, and as
one flat stream; plus hipMemcpyAsync device-to-device), and
``frac_of_copy_ceiling`` the kernel's rate over the first of them;
``cpu_baseline`` is the CPU oracle timed on this host's cores on a sample of
the same inputs.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBPS = 8000.0
METRIC = ("reconstructed KV GB/s (read+write) and % of HBM peak; "
          "µs per 1K-token chunk")
KERNEL_SRC = os.path.join(HERE, "position_invariant_kv_amd", "csrc", "kamera.hip")
ATTN_SRC = os.path.join(HERE, "position_invariant_kv_amd", "csrc", "kamera_attn.hip")
KERNEL_COMMON = os.path.join(HERE, "position_invariant_kv_amd", "csrc", "kamera_common.h")
TRAFFIC_FILE = os.path.join(HERE, "profiles", "hbm_traffic.json")
CAL_BYTES = 1 << 30  # calibration copy: 1 GiB read + 1 GiB written
# the headline: the reorder workload (GQA, 36 layers, 8 KV heads x 128, 32
# chunks x 2048 tokens, rank-32 orbit patches, 16-token pages), the reuse
# configuration with the most bytes; the other reuse configurations are
# measured in the same run and reported inside the same line
DEFAULT_WORKLOAD = "reorder_recall_rank32"
OTHER_CONFIGS = ("gqa_single_frame_reuse", "sliding_window_survival", "mla_reuse")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--also", default=",".join(OTHER_CONFIGS),
                    help="comma-separated reuse workloads reported inside the line as other_configs "
                         "(empty: the headline workload only)")
    ap.add_argument("--sets", type=int, default=0, help="rotated input sets (0: enough for 1.5 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--walk-orders", action="store_true",
                    help="print the copy-probe rate of the workload's pages in page-table and in page-id "
                         "order (paged workloads) and exit")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output dirs (FETCH_SIZE, WRITE_SIZE) of this "
                         "bench into profiles/hbm_traffic.json and exit")
    return ap.parse_args()


def kernel_digest(workload: str = "") -> str:
    """Digest of the measured kernels' sources (kamera.hip, or kamera_attn.hip
    for the decode workloads, and the helpers they include)."""
    h = hashlib.sha256(open(ATTN_SRC if workload.startswith("decode_") else KERNEL_SRC, "rb").read())
    h.update(open(KERNEL_COMMON, "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    if they were taken on a different kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_sha256_16") != kernel_digest(workload):
        return None
    return ent.get("hbm_bytes_per_launch")


def host_threads() -> int:
    """Host threads the CPU baseline uses: the CPUs this process may run on,
    at most 16 (one GPU's share of a GPU machine's host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w, inp, budget_s: float, threads: int):
    """Time the CPU oracle (as it stands) on a sample of the same inputs.

    The unit of work is one (output chunk, layer) block over every stream: the
    oracle's reconstruct() on that chunk's rows of that layer, written into a
    pool of the chunk's own pages (paged: its page-table row renumbered
    0..ceil(T/P)-1 in the same relative order; contiguous: offset 0).  A sample
    of units spread evenly over the call is copied to the host first (not
    timed); then `threads` host threads each run their share of the sample
    round robin, single-threaded each (BLAS limited to one thread; NumPy
    releases the GIL inside its array loops), until `budget_s` of wall time
    has passed.  The rate is reconstructed-KV bytes (rows read + written) of
    the finished units over the wall time."""
    import threading

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import kamera_oracle as ko
    from workloads import bits

    lay = ko.Layout(1, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim, w.rope_base, w.num_streams,
                    w.rope_style)
    if w.op in ("relocate", "relocate_patch"):
        ids, ds = list(range(w.n_chunks)), ko.deltas_relocate(inp["delta"].tolist())
    elif w.op == "reorder":
        ids = inp["perm"].tolist()
        ds = ko.deltas_reorder(ids, inp["base_pos"], w.n_tokens)
    else:
        ids = inp["chunk_ids"].tolist()
        ds = ko.deltas_recall(ids, inp["target_pos"].tolist())
    units = [(i, l) for i in range(w.n_chunks) for l in range(w.num_layers)]
    nsample = min(len(units), 2 * threads)
    sample = [units[(k * len(units)) // nsample] for k in range(nsample)]
    pt = None if inp["page_table"] is None else inp["page_table"].cpu().numpy()
    T, F, P = w.n_tokens, w.row_width, w.page_size
    work = []
    for i, l in sample:
        c = ids[i]
        src = [bits(x[c, l])[None, None] for x in inp["src"]]
        u = None if inp["u"] is None else [bits(x[c, l])[None, None] for x in inp["u"]]
        v = None if inp["v"] is None else [bits(x[c, l])[None, None] for x in inp["v"]]
        if P:
            row = pt[i]
            local = np.argsort(np.argsort(row, kind="stable"), kind="stable")[None].astype(np.int64)
            pools = [np.zeros((1, len(row) * P, F), np.uint16) for _ in src]
            work.append((src, u, v, ds[i], pools, local, None))
        else:
            pools = [np.zeros((1, T, F), np.uint16) for _ in src]
            work.append((src, u, v, ds[i], pools, None, [0]))
    done = [0] * threads
    stop = time.perf_counter() + budget_s

    def run(t):
        with threadpool_limits(limits=1):
            k = t
            while time.perf_counter() < stop:
                src, u, v, d, pools, local, off = work[k % len(work)]
                ko.reconstruct(lay, src, [0], [d], pools, P, local, off, u, v)
                done[t] += 1
                k += threads

    t0 = time.perf_counter()
    pool = [threading.Thread(target=run, args=(t,)) for t in range(threads)]
    for th in pool:
        th.start()
    for th in pool:
        th.join()
    el = time.perf_counter() - t0
    nunits = sum(done)
    unit_kv = 2 * 2 * w.num_streams * T * F
    return {"value": round(nunits * unit_kv / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{nunits} (output chunk, layer) blocks of {w.name} ({T} tokens x {F} features x "
                      f"{w.num_streams} stream(s) each, from {nsample} distinct blocks spread over the call), "
                      f"float64 NumPy oracle, {el:.1f} s wall on {threads} host thread(s)"}


def _counter_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def ingest_counters(fetch_dir, write_dir, workload):
    """Per-launch HBM bytes of the Kamera kernel from FETCH_SIZE / WRITE_SIZE runs.

    Both counters are in KiB per dispatch.  Each is scaled by what it reads for
    the calibration copy this bench runs (an elementwise bitwise_not that reads
    and writes exactly CAL_BYTES), then averaged over the Kamera dispatches.
    """
    from workloads import by_name, decode_by_name, make_varlen_inputs, varlen_by_name
    decode = workload.startswith("decode_")
    varlen = workload.startswith("varlen_")
    w = decode_by_name(workload) if decode else (varlen_by_name(workload) if varlen else by_name(workload))
    # the dominant kernel of one call: the reuse kernel, or for decode the fused
    # attention kernel (with the patch), never the pool comparison's
    if decode:
        # a context of reused entries alone runs the entries' kernel; with
        # pooled tokens, one launch covers both (the mixed kernel)
        mla = w.base.num_streams == 1
        if w.pool_tokens:
            tags = ["attn_mla_mixed_kernel<true," if mla else "attn_mfma_mixed_kernel<128, true,"]
        else:
            tags = ["attn_mla_kernel<true, false," if mla else "attn_mfma_kernel<128, true, false,"]
    else:
        tags = ["relocate"]
    out = {"workload": workload, "kernel_sha256_16": kernel_digest(workload), "calibration_bytes": CAL_BYTES}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == name]
        copy = [float(r["Counter_Value"]) for r in rows if "bitwise_not" in r["Kernel_Name"]]
        knames = sorted({r["Kernel_Name"].split("::", 1)[-1].split("(")[0]
                         for r in rows if any(t in r["Kernel_Name"] for t in tags)})
        k_kib, nk = 0.0, 0
        for t in tags:
            kern = [float(r["Counter_Value"]) for r in rows if t in r["Kernel_Name"]]
            if not kern:
                raise SystemExit(f"{d}: no {name} rows for {t}")
            k_kib += sum(kern) / len(kern)
            nk += len(kern)
        if not copy:
            raise SystemExit(f"{d}: no {name} rows for the calibration copy")
        c_kib = sum(copy) / len(copy)
        scale = CAL_BYTES / (c_kib * 1024.0)
        out[name.lower() + "_kib_per_dispatch"] = round(k_kib, 1)
        out["calibration_" + name.lower() + "_kib"] = round(c_kib, 1)
        out[name.lower() + "_scale"] = round(scale, 4)
        out[name.lower() + "_bytes"] = int(k_kib * 1024.0 * scale)
        out["kernel"] = knames
        out["dispatches"] = nk
    out["hbm_bytes_per_launch"] = out["fetch_size_bytes"] + out["write_size_bytes"]
    out["algorithmic_bytes_per_launch"] = (w.layer_bytes() if decode else
                                           make_varlen_inputs(w, index_only=True)["algorithmic_bytes"] if varlen
                                           else w.algorithmic_bytes())
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        rec = {}
    rec[workload] = out
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps(out))


def cpu_baseline_form(fw, inp, target, budget_s: float):
    """Time the patch-formation oracle (as it stands) on whole blocks of the same inputs."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import kamera_oracle as ko
    from oracle import patch_oracle as po
    from workloads import bits

    b = fw.base
    lay = ko.Layout(b.num_layers, b.num_heads, b.head_dim, b.rope_offset, b.rope_dim, b.rope_base,
                    b.num_streams, b.rope_style)
    deltas = inp["delta"].cpu().tolist()
    P = fw.views
    order = [(i, l, s) for i in range(b.n_chunks) for l in range(b.num_layers) for s in range(b.num_streams)]
    done, t_cpu = 0, 0.0
    with threadpool_limits(limits=1):
        while t_cpu < budget_s and done < len(order):
            i, l, s = order[(done * 7919) % len(order)]
            cb = bits(inp["src"][s][i, l])
            if P == 1:
                tb = bits(target[s][i, l])
                t0 = time.perf_counter()
                po.form_patch_bits(cb, tb, deltas[i], lay, s == 0, fw.rank)
            else:
                tb = np.stack([bits(target[s][i * P + v, l]) for v in range(P)])
                t0 = time.perf_counter()
                po.form_orbit_patch_bits(cb, tb, deltas[i], lay, s == 0, fw.rank)
            t_cpu += time.perf_counter() - t0
            done += 1
    per_block = 2 * (1 + P) * b.n_tokens * b.row_width
    what = "deficit + SVD" if P == 1 else f"mean deficit over {P} views + SVD"
    return {"value": round(done * per_block / t_cpu / 1e9, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} (chunk, layer, stream) blocks of {fw.name} ({b.n_tokens} x {b.row_width}), "
                      f"float64 NumPy {what}, {t_cpu:.1f} s, 1 thread"}


def bench_form(args):
    """Patch formation (kamera_form_patch, or kamera_form_orbit_patch for a
    workload with several views) on a formation workload."""
    import torch

    import position_invariant_kv_amd as kam
    from workloads import form_by_name, make_form_inputs

    fw = form_by_name(args.workload)
    b = fw.base
    torch.cuda.set_device(0)
    inp = make_form_inputs(fw, "cuda")
    lay = kam.Layout(b.num_layers, b.num_heads, b.head_dim, b.rope_offset, b.rope_dim, b.rope_base,
                     b.num_streams, b.rope_style)
    n, L, T, F, S = b.n_chunks, b.num_layers, b.n_tokens, b.row_width, b.num_streams
    P = fw.views
    # KV(B|A) for the benchmark: R(delta) canon + signal, written by this library's
    # relocate_patch into [L][n*P*T][F] (view v of chunk i at chunk index
    # i * P + v) and viewed as [n*P][L][T][F]
    pools = [torch.empty((L, n * P * T, F), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    for vw in range(P):
        dv = inp["delta"] if P == 1 else inp["delta"][:, vw].contiguous()
        uv = inp["u_sig"] if P == 1 else [x.view(n, P, L, T, -1)[:, vw].contiguous() for x in inp["u_sig"]]
        kam.relocate_patch(lay, inp["src"], dv, uv, inp["v_sig"], pools,
                           dst_offset=(torch.arange(n, dtype=torch.int64, device="cuda") * P + vw) * T)
    target = [p.view(L, n * P, T, F).permute(1, 0, 2, 3) for p in pools]
    del inp["u_sig"], inp["v_sig"]
    u = [torch.empty((n, L, T, fw.rank), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    v = [torch.empty((n, L, F, fw.rank), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    stream = torch.cuda.current_stream()
    if P == 1:
        call = kam.prepare_form_patch(lay, inp["src"], target, inp["delta"], u, v, inp["omega"],
                                      oversample=fw.oversample, power_iters=fw.power_iters, stream=stream)
    else:
        call = kam.prepare_form_orbit_patch(lay, inp["src"], target, inp["delta"], u, v, inp["omega"],
                                            oversample=fw.oversample, power_iters=fw.power_iters, stream=stream)
    steps, warmup = args.steps, args.warmup
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    alg = fw.method_bytes()
    achieved = alg / (ms * 1e-3) / 1e9
    impl = fw.implementation_bytes()
    flops = fw.sketch_flops()
    out = {
        "metric": "patch formation: canonical + KV(B|A) rows consumed, GB/s (deficit + randomized truncated SVD)",
        "value": round(fw.row_bytes() / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "storage_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": fw.name, "family": b.family, "layers": L, "kv_heads": b.num_heads,
                   "head_dim": b.head_dim, "chunks": n, "tokens_per_chunk": T, "rank": fw.rank,
                   "oversample": fw.oversample, "power_iters": fw.power_iters, "blocks": fw.blocks,
                   "views": P},
        "us_per_block": round(ms * 1e3 / fw.blocks, 3),
        "roofline": {
            "bound": "hbm",
            "kernel": "whole call (deficit, sketch, orthonormalization, eigen and factor kernels)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": alg,
            "algorithmic_bytes": "the method's own data: canonical rows and KV(B|A) rows read once, factors "
                                 "written once",
        },
        # the products with the deficit on the matrix cores, against the bf16 dense peak
        "mfma": {"flops_per_launch": flops, "achieved_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
                 "peak_TFLOPs": 2500.0, "frac": round(flops / (ms * 1e-3) / 2.5e15, 4),
                 "note": "2q + 2 products of each T x F block with k = m + p columns, 2 T F k flops each; "
                         "the kernels run them as two or three bf16 products (high and low parts)"},
        # what this implementation moves: the deficit's bf16 high and low parts written once, read 2q + 1
        # times (one view: the first product forms it) or 2q + 2 times
        "implementation": {"bytes_per_launch": impl, "GBps": round(impl / (ms * 1e-3) / 1e9, 2),
                           "frac_of_hbm_peak": round(impl / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_form(fw, inp, target, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline_decode(dw, inp, budget_s: float):
    """Time the decode-attention oracle (as it stands) on whole layers of the same inputs."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attention_oracle as ao
    from oracle import kamera_oracle as ko
    from workloads import bits

    b = dw.base
    lay = ko.Layout(1, b.num_heads, b.head_dim, b.rope_offset, b.rope_dim, b.rope_base, b.num_streams,
                    b.rope_style)
    se = inp["seq_entries"].cpu().numpy()
    ids = inp["chunk_ids"].cpu().tolist()
    deltas = inp["delta"].cpu().tolist()
    done, t_cpu = 0, 0.0
    with threadpool_limits(limits=1):
        while t_cpu < budget_s and done < b.num_layers:
            layer = (done * 7) % b.num_layers
            canon = [bits(x[:, layer:layer + 1]) for x in inp["src"]]
            patch = ([bits(x[:, layer:layer + 1]) for x in inp["u"]], [bits(x[:, layer:layer + 1]) for x in inp["v"]])
            q = ko.bf16_bits_to_f64(bits(inp["q"][layer]))
            pool = None
            if dw.pool_tokens:
                pool = ([bits(x[layer:layer + 1]) for x in inp["pool"]], dw.pool_page,
                        inp["block_table"].cpu().numpy(), inp["pool_tokens"].cpu().numpy())
            t0 = time.perf_counter()
            ao.decode_attention_f64(lay, 0, canon, patch, se, ids, deltas, q, dw.num_q_heads, dw.scale, pool=pool)
            t_cpu += time.perf_counter() - t0
            done += 1
    return {"value": round(done * dw.layer_bytes() / t_cpu / 1e9, 5), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{done} layer(s) of {dw.name} ({dw.context_tokens()} context tokens, "
                      f"{dw.num_q_heads} query heads), float64 NumPy oracle, {t_cpu:.1f} s, 1 thread"}


def bench_decode(args):
    """Decode attention over a reused context, relocated and patched on read
    (kamera_decode_attention): one step is every layer's attention for one
    new token of every sequence."""
    import torch

    import position_invariant_kv_amd as kam
    from workloads import decode_by_name, make_decode_inputs

    dw = decode_by_name(args.workload)
    b = dw.base
    torch.cuda.set_device(0)
    inp = make_decode_inputs(dw, "cuda")
    S = b.num_streams
    lay = kam.Layout(b.num_layers, b.num_heads, b.head_dim, b.rope_offset, b.rope_dim, b.rope_base, S,
                     b.rope_style)
    L, B, Hq, D, Dv = b.num_layers, dw.num_seqs, dw.num_q_heads, b.head_dim, dw.value_dim
    stream = torch.cuda.current_stream()
    outs = torch.empty((L, B, Hq, Dv), dtype=torch.float32, device="cuda")
    lses = torch.empty((L, B, Hq), dtype=torch.float32, device="cuda")
    pooled = dict(pool=inp["pool"], block_table=inp["block_table"], pool_tokens=inp["pool_tokens"],
                  pool_page_size=dw.pool_page) if dw.pool_tokens else {}
    # one workspace for every layer's call (they run in order on one stream)
    E = inp["chunk_ids"].numel()
    need = (kam.decode_attention_paged_workspace_bytes(lay, Hq, E, b.n_tokens, B, dw.pool_pages * dw.pool_page)
            if dw.pool_tokens else kam.decode_attention_workspace_bytes(lay, Hq, E, b.n_tokens))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    calls = [kam.prepare_decode_attention(lay, l, inp["src"], inp["q"][l], inp["seq_entries"], inp["chunk_ids"],
                                          inp["delta"], outs[l], scale=dw.scale, lse=lses[l], u=inp["u"],
                                          v=inp["v"], workspace=ws, stream=stream, **pooled) for l in range(L)]
    steps, warmup = args.steps, args.warmup

    def step():
        for c in calls:
            c()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    layer_us = ms * 1e3 / L
    achieved = dw.layer_bytes() / (layer_us * 1e-6) / 1e9
    kv_bytes = 2 * S * dw.context_tokens() * b.row_width * B * L

    # the two-step path for comparison: kamera_relocate_patch writes the whole
    # reused context (every layer) into a pool once, then every step reads the
    # pool with plain attention (delta = 0, no patch)
    n, T, F = inp["chunk_ids"].numel(), b.n_tokens, b.row_width
    ids64 = inp["chunk_ids"].to(torch.int64)
    pool = [torch.empty((L, n * T, F), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    sel_src = [x[ids64] for x in inp["src"]]
    sel_u = [x[ids64].contiguous() for x in inp["u"]]
    sel_v = [x[ids64].contiguous() for x in inp["v"]]
    reuse = kam.prepare_relocate_patch(lay, sel_src, inp["delta"], sel_u, sel_v, pool,
                                       dst_offset=torch.arange(n, dtype=torch.int64, device="cuda") * T,
                                       stream=stream)
    pool_store = [p.view(L, n, T, F).permute(1, 0, 2, 3) for p in pool]
    zero = torch.zeros(n, dtype=torch.int64, device="cuda")
    ids_pool = torch.arange(n, dtype=torch.int32, device="cuda")
    seq_pool = torch.tensor([0, n], dtype=torch.int32, device="cuda")
    plain = [kam.prepare_decode_attention(lay, l, pool_store, inp["q"][l], seq_pool, ids_pool, zero, outs[l],
                                          scale=dw.scale, lse=lses[l], workspace=ws, stream=stream, **pooled)
             for l in range(L)] if B == 1 else []
    reuse()
    for c in plain:
        c()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(5):
        reuse()
    ev1.record(stream)
    torch.cuda.synchronize()
    reuse_ms = ev0.elapsed_time(ev1) / 5
    pool_ms = None
    if plain:
        ev0.record(stream)
        for _ in range(steps):
            for c in plain:
                c()
        ev1.record(stream)
        torch.cuda.synchronize()
        pool_ms = ev0.elapsed_time(ev1) / steps
    del pool, sel_src, pool_store
    # HBM-counter calibration copy (see the reuse leg): reads and writes CAL_BYTES
    ca = torch.empty(CAL_BYTES, dtype=torch.uint8, device="cuda")
    cb = torch.empty(CAL_BYTES, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        torch.bitwise_not(ca, out=cb)
    torch.cuda.synchronize()
    del ca, cb
    out = {
        "metric": "decode attention over a reused context, relocated on read: context KV GB/s read",
        "value": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "storage_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": dw.name, "family": b.family, "layers": L, "kv_heads": b.num_heads,
                   "q_heads": Hq, "head_dim": D, "value_dim": Dv, "sequences": B,
                   "context_tokens": dw.context_tokens(),
                   "chunks": b.n_chunks, "tokens_per_chunk": T, "rank": b.rank,
                   "pooled_tokens": dw.pool_tokens, "pool_page": dw.pool_page if dw.pool_tokens else None},
        "us_per_layer": round(layer_us, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": (("attn_mla_mixed_kernel" if S == 1 else "attn_mfma_mixed_kernel") if dw.pool_tokens
                         else ("attn_mla_kernel" if S == 1 else "attn_mfma_kernel"))
                      + " + attn_combine_kernel (one call per layer)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(dw.name),
            "algorithmic_bytes_per_launch": dw.layer_bytes(),
        },
        "two_step": {"reuse_into_pool_ms": round(reuse_ms, 4),
                     "attention_over_pool_ms_per_step": None if pool_ms is None else round(pool_ms, 4),
                     "first_step_ms": None if pool_ms is None else round(reuse_ms + pool_ms, 4)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(dw, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


HOST_LINK_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction (published rate)


def bench_host(args):
    """Recall from a canonical store in pinned host memory
    (kamera_relocate_patch_host): one step recalls the workload's chunks (every
    layer and stream) over the host link into the paged pool."""
    import torch

    import position_invariant_kv_amd as kam
    from workloads import RECALL_CONFIG, make_inputs

    from dataclasses import replace
    w = replace(RECALL_CONFIG, name="recall_host_rank32", n_chunks=8, n_store=16)
    torch.cuda.set_device(0)
    inp = make_inputs(w, "cuda")
    lay = kam.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim, w.rope_base,
                     w.num_streams, w.rope_style)
    host = [x.cpu().pin_memory() for x in inp["src"]]
    del inp["src"]
    sel = inp["chunk_ids"].long()
    u = [x[sel].contiguous() for x in inp["u"]]
    v = [x[sel].contiguous() for x in inp["v"]]
    delta = inp["target_pos"].contiguous()
    ids = inp["chunk_ids"].cpu().tolist()
    stream = torch.cuda.current_stream()
    copy_stream = torch.cuda.Stream()
    call = kam.prepare_relocate_patch_host(lay, host, ids, delta, inp["pool"], u=u, v=v, page_size=w.page_size,
                                           page_table=inp["page_table"], slots=2, copy_stream=copy_stream,
                                           stream=stream)
    steps, warmup = min(args.steps, 10), min(args.warmup, 2)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    host_bytes = 2 * w.num_streams * w.num_layers * w.n_tokens * w.row_width * w.n_chunks
    # the link's own rate here: one chunk's rows, pinned host -> device, repeated
    chunk = host[0][0]
    dev = torch.empty(chunk.shape, dtype=chunk.dtype, device="cuda")
    for _ in range(2):
        dev.copy_(chunk, non_blocking=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(8):
        dev.copy_(chunk, non_blocking=True)
    ev1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 8 * chunk.numel() * 2 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    achieved = host_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "recall from a pinned host store: canonical rows delivered over the host link, GB/s",
        "value": round(achieved, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "storage_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "family": w.family, "layers": w.num_layers, "kv_heads": w.num_heads,
                   "head_dim": w.head_dim, "recalled_chunks": w.n_chunks, "stored_chunks": w.n_store,
                   "tokens_per_chunk": w.n_tokens, "rank": w.rank, "page_size": w.page_size, "slots": 2},
        "roofline": {
            "bound": "host_link",
            "kernel": "hipMemcpy2DAsync H2D (copy stream) overlapped with relocate_patch_lds_kernel",
            "achieved": round(achieved, 2),
            "peak": HOST_LINK_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HOST_LINK_PEAK_GBPS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": host_bytes,
        },
        "host_copy_ceiling_GBps": round(copy_gbps, 2),
    }
    print(json.dumps(out), flush=True)


def bench_host_varlen(args):
    """Recall of variable-length chunks from a pinned host store
    (kamera_relocate_patch_host_varlen): one step recalls the workload's
    chunks (every layer and stream) over the host link into the paged pool."""
    import torch

    import position_invariant_kv_amd as kam
    from workloads import make_varlen_inputs, varlen_by_name

    vw = varlen_by_name(args.workload)
    w = vw.base
    torch.cuda.set_device(0)
    inp = make_varlen_inputs(vw, "cuda")
    lay = kam.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim, w.rope_base,
                     w.num_streams, w.rope_style)
    host = [x.cpu().pin_memory() for x in inp["src"]]
    del inp["src"]
    ids = list(inp["out_ids"])
    lengths = inp["lengths"]
    ro = inp["row_offset"].cpu().tolist()
    u = [torch.cat([x[ro[c]:ro[c] + w.num_layers * lengths[c]] for c in ids]).contiguous() for x in inp["u"]]
    sel = torch.tensor(ids, dtype=torch.long, device="cuda")
    v = [x[sel].contiguous() for x in inp["v"]]
    delta = inp["target_pos"].contiguous()
    stream = torch.cuda.current_stream()
    copy_stream = torch.cuda.Stream()
    call = kam.prepare_relocate_patch_host_varlen(lay, host, ro, lengths, vw.max_tokens, ids, delta, inp["pool"],
                                                  u=u, v=v, page_size=w.page_size, page_table=inp["page_table"],
                                                  slots=2, copy_stream=copy_stream, stream=stream)
    steps, warmup = min(args.steps, 10), min(args.warmup, 2)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    tok = sum(inp["out_lengths"])
    host_bytes = 2 * w.num_streams * w.num_layers * tok * w.row_width
    # the link's own rate here: the longest recalled chunk's rows, pinned host -> device, repeated
    c = max(ids, key=lambda k: lengths[k])
    chunk = host[0][ro[c]:ro[c] + w.num_layers * lengths[c]]
    dev = torch.empty(chunk.shape, dtype=chunk.dtype, device="cuda")
    for _ in range(2):
        dev.copy_(chunk, non_blocking=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(8):
        dev.copy_(chunk, non_blocking=True)
    ev1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 8 * chunk.numel() * 2 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    achieved = host_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "recall from a pinned host store: canonical rows delivered over the host link, GB/s",
        "value": round(achieved, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "storage_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": vw.name, "family": w.family, "layers": w.num_layers, "kv_heads": w.num_heads,
                   "head_dim": w.head_dim, "recalled_chunks": w.n_chunks, "stored_chunks": w.n_store,
                   "tokens": tok, "tokens_per_chunk_range": list(vw.len_range), "rank": w.rank,
                   "page_size": w.page_size, "slots": 2},
        "roofline": {
            "bound": "host_link",
            "kernel": "hipMemcpyAsync H2D (copy stream) overlapped with relocate_patch_lds_kernel",
            "achieved": round(achieved, 2),
            "peak": HOST_LINK_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HOST_LINK_PEAK_GBPS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": host_bytes,
        },
        "host_copy_ceiling_GBps": round(copy_gbps, 2),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_varlen(vw, inp, budget_s: float):
    """The oracle (reconstruct_varlen) on whole output chunks of the same inputs, single thread.

    Each sampled chunk's rows are copied to the host (not timed) and the oracle
    writes them into a pool of that chunk's size (contiguous), so the host
    never holds the whole store.
    """
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import kamera_oracle as ko
    from workloads import bits

    w = vw.base
    lay = ko.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim,
                    w.rope_base, w.num_streams, w.rope_style)
    ids = list(inp["out_ids"])
    lengths = inp["lengths"]
    ro = inp["row_offset"].cpu().tolist()
    if w.op == "recall":
        ds = ko.deltas_recall(ids, inp["target_pos"].tolist())
    else:
        ds = ko.deltas_relocate(inp["delta"].tolist())
    done, tok, el = 0, 0, 0.0
    with threadpool_limits(limits=1):
        while el < budget_s and done < 100000:
            i = done % len(ids)
            c = ids[i]
            T = lengths[c]
            rows = slice(ro[c], ro[c] + w.num_layers * T)
            src = [bits(x[rows]) for x in inp["src"]]
            u = None if inp["u"] is None else [bits(x[rows]) for x in inp["u"]]
            v = None if inp["v"] is None else [bits(x[c:c + 1]) for x in inp["v"]]
            pools = [np.zeros((w.num_layers, T, w.row_width), dtype=np.uint16) for _ in inp["src"]]
            t0 = time.perf_counter()
            ko.reconstruct_varlen(lay, src, [0], [T], [0], [ds[i]], pools, 0, dst_offset=[0], u=u, v=v)
            el += time.perf_counter() - t0
            done += 1
            tok += T
    kv = 2 * 2 * w.num_streams * w.num_layers * tok * w.row_width
    return {"value": round(kv / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} output chunk(s) of {vw.name} ({tok} tokens, all {w.num_layers} layers x "
                      f"{w.num_streams} streams each) into a contiguous pool of the chunk's size, float64 "
                      f"NumPy oracle, {el:.1f} s of oracle time (host copies of the rows not timed), 1 thread"}


def bench_varlen(args):
    """Variable-length chunks: one packed store, kamera_recall_varlen / kamera_relocate_patch_varlen.

    The store (~10 GB) is far larger than the Infinity Cache, so one input set
    suffices; a step is one call over every chunk of the workload."""
    import torch

    import position_invariant_kv_amd as kam
    from workloads import make_varlen_inputs, varlen_by_name

    vw = varlen_by_name(args.workload)
    w = vw.base
    torch.cuda.set_device(0)
    inp = make_varlen_inputs(vw, "cuda")
    lay = kam.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim,
                     w.rope_base, w.num_streams, w.rope_style)
    stream = torch.cuda.current_stream()
    kw = dict(u=inp["u"], v=inp["v"], page_size=w.page_size, page_table=inp["page_table"],
              dst_offset=inp["dst_offset"], canon_pos=inp["canon_pos"], stream=stream)
    if w.op == "recall":
        call = kam.prepare_recall_varlen(lay, inp["src"], inp["row_offset"], inp["n_tokens"], inp["max_tokens"],
                                         inp["chunk_ids"], inp["target_pos"], inp["pool"], **kw)
    else:
        call = kam.prepare_relocate_patch_varlen(lay, inp["src"], inp["row_offset"], inp["n_tokens"],
                                                 inp["max_tokens"], inp["delta"], inp["pool"], **kw)
    steps, warmup = min(args.steps, 20), min(args.warmup, 3)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps

    tok = sum(inp["out_lengths"])
    kv = 2 * 2 * w.num_streams * w.num_layers * tok * w.row_width
    nbytes = kv // 2
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b.copy_(a)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(5):
        b.copy_(a)
    ev1.record(stream)
    torch.cuda.synchronize()
    copy_ms = ev0.elapsed_time(ev1) / 5
    del a, b
    ca = torch.empty(CAL_BYTES, dtype=torch.uint8, device="cuda")
    cb = torch.empty(CAL_BYTES, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        torch.bitwise_not(ca, out=cb)
    torch.cuda.synchronize()
    del ca, cb

    alg = inp["algorithmic_bytes"]
    achieved = alg / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(kv / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "storage_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": vw.name, "family": w.family, "op": w.op + "_varlen", "layers": w.num_layers,
                   "kv_heads": w.num_heads, "head_dim": w.head_dim, "rope_dim": w.rope_dim,
                   "chunks": w.n_chunks, "tokens": tok, "tokens_per_chunk_range": list(vw.len_range),
                   "rank": w.rank, "page_size": w.page_size},
        "hbm_frac": round(achieved / HBM_PEAK_GBPS, 4),
        "us_per_1k_tokens": round(ms * 1e3 / (tok / 1024), 3),
        "copy_ceiling_GBps": round(2 * nbytes / (copy_ms * 1e-3) / 1e9, 1),
        "roofline": {
            "bound": "hbm",
            "kernel": "relocate_patch_lds_kernel" if w.rank > 0 else "relocate_rows_kernel",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(vw.name),
            "algorithmic_bytes_per_launch": alg,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_varlen(vw, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters, args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the Kamera operator is measured on a single "
              "MI355X; --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    if args.workload.startswith("form_"):
        bench_form(args)
        return
    if args.workload.startswith("decode_"):
        bench_decode(args)
        return
    if args.workload == "recall_host_rank32":
        bench_host(args)
        return
    if args.workload == "varlen_recall_host_rank32":
        bench_host_varlen(args)
        return
    if args.workload.startswith("varlen_"):
        bench_varlen(args)
        return

    from workloads import by_name

    if args.walk_orders:
        print(json.dumps(walk_orders(by_name(args.workload), args.steps)), flush=True)
        return
    head = bench_reuse(by_name(args.workload), args.steps, args.warmup, args)
    others = []
    for name in [x for x in args.also.split(",") if x and x != args.workload]:
        # the other reuse configs: same contract, more steps for the short ones
        try:
            others.append(bench_reuse(by_name(name), max(args.steps, 100), max(args.warmup, 5), args))
        except Exception as e:  # one failed config must not lose the headline line
            others.append({"config": {"workload": name}, "error": f"{type(e).__name__}: {e}"})
    if others:
        head["other_configs"] = others
    print(json.dumps(head), flush=True)


def _walk_blocks(w, inp, nbytes_of, ptr_of, order="kernel"):
    """The blocks a call of workload w moves, in the order its kernel walks
    them: (source byte offset, destination byte offset) pairs relative to the
    lowest source and destination tensor addresses, and the block size.

    A block is one page of one (output chunk, layer, stream) (paged pools) or
    one chunk's rows of one layer and stream (contiguous pools).  The walk
    mirrors the library's choice: a paged call whose workgroups stay inside
    one page walks the pages in ascending page-id order (the m = 0 kernel:
    layer, then stream, then page; the patch kernel: stream, then layer, then
    page), every other call walks output chunk and stream, then layer, then the
    chunk's own pages.  order="table" or "page" forces one of the two walks
    (paged pools only; "page" nests layers and streams as the kernel of the
    workload's rank would)."""
    import numpy as np

    S, L, T, F, P, n = w.num_streams, w.num_layers, w.n_tokens, w.row_width, w.page_size, w.n_chunks
    if w.op in ("relocate", "relocate_patch"):
        ids = list(range(n))
    else:
        ids = (inp["perm"] if w.op == "reorder" else inp["chunk_ids"]).tolist()
    src0 = min(ptr_of(t) for t in inp["src"])
    dst0 = min(ptr_of(t) for t in inp["pool"])
    rows = T * F * 2                                      # bytes of one chunk's rows of one layer
    pool_layer = inp["pool"][0].stride(0) * 2
    blocks = []
    if P:
        ppc = w.pages_per_chunk
        pt = inp["page_table"].cpu().numpy()
        page = P * F * 2
        if w.rank == 0:
            by_page = (P * F) % (8 * 256 * 2) == 0        # two 16-byte vectors per thread, whole pages
        else:
            segs = (F // 64)
            win = max(k for k in (1, 2, 3, 4) if segs % k == 0)
            tpg = min(-(-4 // win), -(-T // 32))
            by_page = P % (32 * tpg) == 0
        entries = [(i, j) for i in range(n) for j in range(ppc)]
        if order != "kernel":
            by_page = order == "page"
        if by_page:
            order = sorted(range(len(entries)), key=lambda e: (int(pt[e // ppc, e % ppc]), e))
            outer = [(l, s) for l in range(L) for s in range(S)] if w.rank == 0 else \
                [(l, s) for s in range(S) for l in range(L)]
            walk = [(i, j, l, s) for (l, s) in outer for e in order for (i, j) in [entries[e]]]
        else:
            walk = [(i, j, l, s) for i in range(n) for s in range(S) for l in range(L) for j in range(ppc)]
        for i, j, l, s in walk:
            sb = ptr_of(inp["src"][s]) - src0 + ((ids[i] * L + l) * T + j * P) * F * 2
            db = ptr_of(inp["pool"][s]) - dst0 + l * pool_layer + int(pt[i, j]) * page
            blocks.append((sb, db))
        size = page
        if T % P:
            raise ValueError("the copy pattern assumes whole pages")
    else:
        off = inp["dst_offset"].cpu().tolist()
        for i in range(n):
            for s in range(S):
                for l in range(L):
                    sb = ptr_of(inp["src"][s]) - src0 + (ids[i] * L + l) * rows
                    db = ptr_of(inp["pool"][s]) - dst0 + l * pool_layer + off[i] * F * 2
                    blocks.append((sb, db))
        size = rows
    src_bytes = max(ptr_of(t) + nbytes_of(t) for t in inp["src"]) - src0
    dst_bytes = max(ptr_of(t) + nbytes_of(t) for t in inp["pool"]) - dst0
    for sb, db in blocks:
        assert 0 <= sb and sb + size <= src_bytes and 0 <= db and db + size <= dst_bytes
    return np.array(blocks, dtype=np.int64).reshape(-1, 2), size, (src0, src_bytes), (dst0, dst_bytes)


def copy_ceilings(w, sets, steps):
    """Copy-probe rates (GB/s, bytes read + written) for the rows one call moves:
    walk: the kernel's own blocks in its walk order; ascending: the same blocks
    with both sides in ascending address order; plain: the same number of
    bytes as one flat stream per side (no offset table).  Each rotates over
    the input sets like the kernel's timed steps."""
    import torch

    from position_invariant_kv_amd.probe import CopyProbe

    ptr_of = lambda t: int(t.data_ptr())
    nbytes_of = lambda t: t.numel() * t.element_size()
    probes = {"walk": [], "ascending": [], "plain": []}
    moved = 0
    for inp in sets:
        blk, size, (s0, sbytes), (d0, dbytes) = _walk_blocks(w, inp, nbytes_of, ptr_of)
        moved = 2 * len(blk) * size
        so = torch.from_numpy(blk[:, 0].copy()).cuda()
        do = torch.from_numpy(blk[:, 1].copy()).cuda()
        sa = torch.sort(so).values.contiguous()
        da = torch.sort(do).values.contiguous()
        probes["walk"].append(CopyProbe((s0, sbytes), (d0, dbytes), len(blk), size, so, do))
        probes["ascending"].append(CopyProbe((s0, sbytes), (d0, dbytes), len(blk), size, sa, da))
        # plain: the first bytes of the source tensors into the first bytes of
        # the pool tensors, one sequential stream per side (blocks of 32 KiB)
        per = len(blk) * size // len(inp["src"])
        plain, plain_bytes = [], 0
        for x, y in zip(inp["src"], inp["pool"]):
            nb = min(per, nbytes_of(x), nbytes_of(y)) // 32768
            plain.append(CopyProbe((ptr_of(x), nbytes_of(x)), (ptr_of(y), nbytes_of(y)), nb, 32768))
            plain_bytes += 2 * nb * 32768
        probes["plain"].append(plain)
        probes.setdefault("_keep", []).append((so, do, sa, da))
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for name in ("walk", "ascending", "plain"):
        calls = probes[name]

        def one(k):
            c = calls[k % len(calls)]
            for x in (c if isinstance(c, list) else [c]):
                x(stream)

        for k in range(3):
            one(k)
        torch.cuda.synchronize()
        ev0.record(stream)
        for k in range(steps):
            one(k)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / steps
        b = moved if name != "plain" else plain_bytes
        out[name + "_GBps"] = round(b / (ms * 1e-3) / 1e9, 1)
    return out


def walk_orders(w, steps: int) -> dict:
    """Copy-probe rates (GB/s, bytes read + written) of one paged workload's
    blocks walked in page-table order (output chunk and stream, then layer,
    then the chunk's pages) and in ascending page-id order (per layer and
    stream, the pages by id), each with one and two 16-byte vectors per
    thread: the ceiling each walk order leaves a kernel."""
    import torch

    from position_invariant_kv_amd.probe import CopyProbe
    from workloads import make_inputs

    if not w.page_size:
        raise SystemExit("--walk-orders needs a paged workload")
    inp = make_inputs(w, "cuda")
    ptr_of = lambda t: int(t.data_ptr())
    nbytes_of = lambda t: t.numel() * t.element_size()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for order in ("table", "page"):
        blk, size, s, d = _walk_blocks(w, inp, nbytes_of, ptr_of, order)
        so = torch.from_numpy(blk[:, 0].copy()).cuda()
        do = torch.from_numpy(blk[:, 1].copy()).cuda()
        for vpt in (1, 2):
            pr = CopyProbe(s, d, len(blk), size, so, do, vpt)
            for _ in range(3):
                pr(stream)
            torch.cuda.synchronize()
            ev0.record(stream)
            for _ in range(steps):
                pr(stream)
            ev1.record(stream)
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1) / steps
            out[f"{order}_order_vpt{vpt}_GBps"] = round(2 * len(blk) * size / (ms * 1e-3) / 1e9, 1)
    return {"workload": w.name, "block_bytes": size, "blocks": len(blk), "steps": steps, **out}


def memcpy_ceiling(w, nsets, steps):
    """hipMemcpyAsync device-to-device (torch copy_ of contiguous bytes) of the
    call's row bytes, rotated over enough buffer pairs to read HBM."""
    import torch
    nbytes = w.kv_bytes() // 2
    pairs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda"),
              torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(nsets)]
    stream = torch.cuda.current_stream()
    for k in range(len(pairs) + 2):
        pairs[k % len(pairs)][1].copy_(pairs[k % len(pairs)][0])
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for k in range(steps):
        pairs[k % len(pairs)][1].copy_(pairs[k % len(pairs)][0])
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    del pairs
    torch.cuda.empty_cache()
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def bench_reuse(w, steps: int, warmup: int, args) -> dict:
    """One reuse workload: K timed calls of its entry point (one fused launch
    per call over every layer and stream) on inputs resident in HBM, with its
    copy ceilings and the CPU oracle baseline.  Workloads small enough for the
    256 MB Infinity Cache rotate over enough independent input and pool sets
    (> 1.5 GB) that every call reads HBM; their cache-resident rate (one set)
    is reported apart as warm_mall_resident."""
    import torch

    import position_invariant_kv_amd as kam
    from workloads import make_inputs

    print(f"[bench] {w.name}: generating inputs", file=sys.stderr, flush=True)
    torch.cuda.set_device(0)
    base = make_inputs(w, "cuda")
    set_bytes = w.kv_bytes() + w.factor_bytes()
    nsets = args.sets or max(1, min(16, math.ceil(1.5e9 / set_bytes)))
    sets = [base]
    for k in range(1, nsets):
        s = dict(base)
        s["src"] = [t.clone() for t in base["src"]]
        s["pool"] = [t.clone() for t in base["pool"]]
        if base["u"] is not None:
            s["u"] = [t.clone() for t in base["u"]]
            s["v"] = [t.clone() for t in base["v"]]
        sets.append(s)

    lay = kam.Layout(w.num_layers, w.num_heads, w.head_dim, w.rope_offset, w.rope_dim,
                     w.rope_base, w.num_streams, w.rope_style)
    stream = torch.cuda.current_stream()

    def prepare(inp):
        kw = dict(page_size=w.page_size, page_table=inp["page_table"], dst_offset=inp["dst_offset"],
                  canon_pos=inp["canon_pos"], stream=stream)
        if w.op == "relocate":
            return kam.prepare_relocate(lay, inp["src"], inp["delta"], inp["pool"], **kw)
        if w.op == "relocate_patch":
            return kam.prepare_relocate_patch(lay, inp["src"], inp["delta"], inp["u"], inp["v"], inp["pool"], **kw)
        if w.op == "reorder":
            return kam.prepare_reorder(lay, inp["src"], inp["perm"], inp["base_pos"], inp["pool"],
                                       u=inp["u"], v=inp["v"], **kw)
        return kam.prepare_recall(lay, inp["src"], inp["chunk_ids"], inp["target_pos"], inp["pool"],
                                  u=inp["u"], v=inp["v"], **kw)

    # one prepared (validated, marshalled) call per input set: a step is then
    # a single library call, a few microseconds of host time
    calls = [prepare(x) for x in sets]

    def timed(k_steps, rotate=True):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for k in range(k_steps):
            calls[k % nsets if rotate else 0]()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / k_steps

    print(f"[bench] {w.name}: timing {steps} steps", file=sys.stderr, flush=True)
    for k in range(warmup):
        calls[k % nsets]()
    torch.cuda.synchronize()
    ms = timed(steps)
    warm = None
    if nsets > 1:
        for _ in range(3):
            calls[0]()
        torch.cuda.synchronize()
        warm_ms = timed(max(steps, 100), rotate=False)
    ceil = copy_ceilings(w, sets, max(steps, 20))
    ceil["memcpy_d2d_GBps"] = memcpy_ceiling(w, nsets, max(steps, 20))
    # HBM-counter calibration copy: one elementwise kernel that reads and writes
    # exactly CAL_BYTES each (bitwise_not over uint8), recognisable by name in
    # rocprofv3 counter runs
    ca = torch.empty(CAL_BYTES, dtype=torch.uint8, device="cuda")
    cb = torch.empty(CAL_BYTES, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        torch.bitwise_not(ca, out=cb)
    torch.cuda.synchronize()
    del ca, cb

    kv_gbps = w.kv_bytes() / (ms * 1e-3) / 1e9
    alg = w.algorithmic_bytes()
    achieved = alg / (ms * 1e-3) / 1e9
    tokens = w.n_chunks * w.n_tokens
    out = {
        "metric": METRIC,
        "value": round(kv_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "storage_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "family": w.family, "op": w.op, "layers": w.num_layers,
                   "kv_heads": w.num_heads, "head_dim": w.head_dim, "rope_dim": w.rope_dim,
                   "chunks": w.n_chunks, "tokens_per_chunk": w.n_tokens, "rank": w.rank,
                   "page_size": w.page_size, "rotated_input_sets": nsets},
        "hbm_frac": round(achieved / HBM_PEAK_GBPS, 4),
        "us_per_1k_tokens": round(ms * 1e3 / (tokens / 1024), 3),
        "roofline": {
            "bound": "hbm",
            "kernel": "relocate_patch_lds_kernel" if w.rank > 0 else "relocate_rows_kernel",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(w.name),
            "algorithmic_bytes_per_launch": alg,
        },
        "copy_ceiling": ceil,
        "frac_of_copy_ceiling": round(achieved / ceil["walk_GBps"], 4),
    }
    if nsets > 1:
        out["warm_mall_resident"] = {
            "ms_per_step": round(warm_ms, 6),
            "achieved_GBps": round(alg / (warm_ms * 1e-3) / 1e9, 2),
            "note": "one input set reused every step: the rows stay in the Infinity Cache (MALL); "
                    "not an HBM figure"}
    del calls, sets
    if not args.no_cpu_baseline:
        print(f"[bench] {w.name}: CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, base, args.cpu_seconds, host_threads())
        if w.n_chunks * w.num_layers * w.n_tokens <= 1 << 15:
            out["cpu_baseline_one_core"] = cpu_baseline(w, base, args.cpu_seconds, 1)
    del base
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
