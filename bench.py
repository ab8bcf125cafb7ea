#!/usr/bin/env python3
"""Benchmark of one verification round on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
ancestor-masked tree attention for one layer, the exit law and TEV's exit-node
and bonus-token draws with one uniform pair per request -- one call of
tev_verify_round (or, with --separate, tev_tree_attn + tev_exit_law +
tev_sample).  The default workload is the Qwen3-4B-shaped round:
1 request, B = 64 tree nodes (root included), V = 151936 bf16 logits, 32/8
heads of dim 128 over a 4096-token KV prefix.

Timing: every step reads a different copy of its inputs from a ring larger
than the 256 MB Infinity Cache, so every step reads its inputs from HBM.  The
timed loop replays graphs that each hold G consecutive rounds on distinct
copies (as nodes of a captured decode step would run them; G = 11 by
default), so graph launches are not charged once per round; the rate with one
graph launch per round is reported beside it.  The timed region is bracketed by a device synchronisation and HIP
events on the stream the graphs are launched on.  The duration of each of the
round's three launches (for the roofline of the dominant one) comes from HIP
events that tev_verify_round_timed records at its launch boundaries; the
separate calls are timed by graph replays of each call alone (context).

The CPU baseline is the fp64 oracle timed on this host's cores on whole
rounds of the same workload (bounded to about 10 s of CPU work).

Prints one JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "verified tree nodes/sec (tree-attn + exit-law + TEV) at B=64,V=152k; % HBM peak"
CSRC = os.path.join(ROOT, "draft_tree_verification_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvent:
    """A HIP event without the system-scope release fence (timing enabled)."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            h = ctypes.CDLL("libamdhip64.so")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            HipEvent._hip = h
        ev = ctypes.c_void_p()
        if HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(ev), HipEvent.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.cuda_event = ev.value

    @staticmethod
    def elapsed_us(a: "HipEvent", b: "HipEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        if HipEvent._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a.cuda_event),
                                             ctypes.c_void_p(b.cuda_event)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1e3


# The sources the round's three kernels (vocabulary pass, attention, tail) are
# compiled from; counters stored for them stay valid while these are unchanged.
ROUND_SOURCES = ("exit_law.hip", "exit_law_dev.h", "round.hip", "tev_internal.h",
                 "tree_attn.hip", "tree_attn_dev.h", "wave_ops.h")


def kernel_source_hash() -> str:
    """Hash of the code the round's kernels are compiled from, comments and
    blank space left out (a comment edit does not change what was counted)."""
    h = hashlib.sha256()
    for f in ROUND_SOURCES:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(f.encode() + " ".join(src.split()).encode())
    return h.hexdigest()[:16]


def algorithmic_work(wl):
    """Bytes and FLOPs the method must move / compute per round (the dense
    work of masked sibling pairs is not counted)."""
    import numpy as np
    from tests import workloads as W
    e = 2 if wl.dtype == "bf16" else 4
    kv = 2 * wl.R * wl.Hkv * (wl.P + wl.B) * wl.D * e
    q = wl.R * wl.B * wl.Hq * wl.D * e
    out = wl.R * wl.B * wl.Hq * wl.D * 4
    flops = 0
    for r in range(wl.R):
        d = W.depths_of(wl.parents[r])
        flops += 4 * wl.Hq * wl.D * int(np.sum(wl.P + d + 1))
    logits = wl.R * wl.B * wl.V * e
    return {"attn_bytes": kv + q + out, "attn_flops": flops, "exit_law_bytes": logits,
            "sample_bytes": wl.R * min(wl.V, 8192) * e}


def cpu_baseline(wl, budget_s: float = 10.0):
    """The oracle as it stands, whole rounds of the same workload."""
    import numpy as np
    import oracle
    threads = oracle.max_threads(0)
    u1 = np.ascontiguousarray(wl.uniforms[:, :1, :])
    rounds, t0 = 0, time.perf_counter()
    while True:
        oracle.tree_attn(wl.q, wl.k, wl.v, wl.dtype, wl.parents, wl.P, wl.scale)
        el = oracle.exit_law(wl.logits, wl.dtype, wl.parents, wl.tokens, wl.inv_temperature)
        oracle.sample(wl.logits, wl.dtype, wl.parents, wl.tokens, el.exit_mass, u1, wl.inv_temperature)
        rounds += 1
        el_t = time.perf_counter() - t0
        if el_t >= budget_s or rounds >= 500:
            break
    nodes = rounds * wl.R * wl.B
    return {"value": nodes / el_t, "unit": "nodes/s", "cores": threads, "kind": "oracle",
            "sample": f"{rounds} whole round(s) of the {wl.name} workload (attention + exit law "
                      f"+ one draw per request), {el_t:.1f} s, fp64, {threads} OpenMP threads"}


def oracle_rows_us(wl, pd_uni, exit_nodes, n_layers, P_c, zrows, loss_w, tb_args, budget_s=2.0):
    """The oracle of each widened row, timed on the host on the same inputs as
    the GPU call beside it (repeated up to budget_s, at least once)."""
    import numpy as np
    import oracle

    def timed(fn):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s or n >= 20:
                return el / n * 1e6

    out = {"tev_predraw": timed(lambda: oracle.predraw(wl.logits, wl.dtype, wl.parents, wl.tokens, pd_uni,
                                                       wl.inv_temperature))}
    kv_shape = (n_layers, wl.R, wl.Hkv, P_c + wl.B, wl.D)
    kk = np.zeros(kv_shape, np.uint16 if wl.dtype == "bf16" else np.float32)
    out["tev_commit_kv"] = timed(lambda: oracle.commit_kv(kk, kk, wl.parents, exit_nodes, P_c))
    del kk
    if zrows is not None and loss_w is not None:
        out["tev_exit_loss"] = timed(lambda: oracle.exit_loss(zrows, wl.dtype, wl.parents, wl.tokens, loss_w))
    if tb_args is not None:
        z, dt, K, B, roots, modes = tb_args
        if modes == 1:
            out["tev_build_tree"] = timed(lambda: oracle.build_tree(z, dt, K, B, roots))
        else:
            out["tev_build_tree_modes"] = timed(lambda: oracle.build_tree_modes(z, dt, K, B, roots))
    return {k: round(v, 1) for k, v in out.items()}


def load_traffic(config: str, src_hash: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != src_hash:
        return None
    return t


COPY_BYTES = 512 << 20   # calibration copy for the HBM byte counters


def summarize_counters(config: str, fetch_db: str, write_db: str):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of every kernel of a
    --counters run, scaled by what the same counter reads for the calibration
    copy (COPY_BYTES read and COPY_BYTES written), into
    profiles/traffic_<config>.json, tagged with the kernel source hash."""
    import sqlite3
    from collections import defaultdict

    def per_kernel(db, counter):
        con = sqlite3.connect(db)
        rows = con.execute("select kernel_name, dispatch_id, value from counters_collection "
                           "where counter_name = ?", (counter,)).fetchall()
        acc = defaultdict(lambda: defaultdict(float))
        for name, disp, val in rows:
            acc[name][disp] += val
        return {k: sum(v.values()) / len(v) for k, v in acc.items()}, \
               {k: max(v.values()) for k, v in acc.items()}

    fetch, fetch_max = per_kernel(fetch_db, "FETCH_SIZE")
    write, write_max = per_kernel(write_db, "WRITE_SIZE")
    copy_k = max((k for k in fetch_max if "copy" in k.lower()), key=lambda k: fetch_max[k])
    f_fetch = COPY_BYTES / (fetch_max[copy_k] * 1024.0)
    f_write = COPY_BYTES / (write_max[copy_k] * 1024.0)
    short = lambda k: k.replace("void ", "").replace("tev::(anonymous namespace)::", "").split("(")[0].split("<")[0]
    out = {"kernel_source_hash": kernel_source_hash(), "workload": config,
           "calibration": {"kernel": short(copy_k), "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                           "fetch_kib": fetch_max[copy_k], "write_kib": write_max[copy_k],
                           "fetch_factor": f_fetch, "write_factor": f_write},
           "kernels": {}}
    for k in fetch:
        if not short(k).startswith("k_"):
            continue
        fb = fetch[k] * 1024.0 * f_fetch
        wb = write.get(k, 0.0) * 1024.0 * f_write
        out["kernels"][short(k)] = {"fetch_kib": fetch[k], "write_kib": write.get(k), "fetch_bytes": fb,
                                    "write_bytes": wb, "bytes_per_launch": fb + wb}
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


N_XCD = 8                 # XCDs of one MI355X (GRBM_GUI_ACTIVE is summed over them)
N_SIMD = 256 * 4          # SIMDs of one MI355X


def summarize_pmc(config: str, dbs):
    """Per-launch counters of a --counters run (several rocprofv3 --pmc
    databases, one pass each), with the calibration copy's readings, into
    profiles/pmc_<config>.json; derived: MFMA busy fraction, MFMA FLOP and
    rate, LDS bytes read, HBM bytes by FETCH_SIZE (scaled by the copy) and by
    the L2's read requests and misses."""
    import sqlite3
    from collections import defaultdict
    # per database: a counter's rows of one dispatch (one per XCD or shader
    # engine) are summed, then averaged over the dispatches; a counter that
    # several passes collect (GRBM_GUI_ACTIVE, say) is averaged over them
    per_db = []
    for db in dbs:
        acc = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
        con = sqlite3.connect(db)
        for name, disp, ctr, val in con.execute(
                "select kernel_name, dispatch_id, counter_name, value from counters_collection"):
            acc[name][ctr][disp] += val
        per_db.append(acc)

    def combine(reduce_dispatches):
        vals = defaultdict(lambda: defaultdict(list))
        for acc in per_db:
            for k, cs in acc.items():
                for c, d in cs.items():
                    vals[k][c].append(reduce_dispatches(list(d.values())))
        return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}

    short = lambda k: k.replace("void ", "").replace("tev::(anonymous namespace)::", "").split("(")[0]
    mean = combine(lambda v: sum(v) / len(v))
    # the calibration copy is the largest dispatch of the copy kernel (the
    # same kernel also moves the run's small inputs)
    peak = combine(max)
    copy_k = max((k for k in peak if "copy" in k.lower()), key=lambda k: peak[k].get("FETCH_SIZE", 0.0),
                 default=None)
    cal = peak.get(copy_k, {}) if copy_k else {}
    out = {"kernel_source_hash": kernel_source_hash(), "workload": config, "calibration_kernel": short(copy_k or ""),
           "calibration_bytes": COPY_BYTES, "calibration": cal, "kernels": {}}
    for k, c in mean.items():
        sk = short(k)
        if not sk.startswith("k_"):
            continue
        d = {"counters": c}
        if "GRBM_GUI_ACTIVE" in c:
            cyc = c["GRBM_GUI_ACTIVE"] / N_XCD
            d["cycles"] = cyc
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                d["mfma_busy_frac"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD)
            if "SQ_LDS_IDX_ACTIVE" in c:
                d["lds_active_frac"] = c["SQ_LDS_IDX_ACTIVE"] / (cyc * 256)
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)
        if mops:
            d["mfma_flop"] = mops * 512
        if "SQ_INSTS_LDS_LOAD_BANDWIDTH" in c:
            d["lds_read_bytes"] = c["SQ_INSTS_LDS_LOAD_BANDWIDTH"] * 64
        if c.get("SQ_WAVE_CYCLES"):
            # shares of the waves' resident cycles (all in quad-cycles):
            # waiting on a dependency (s_waitcnt, barrier), waiting to issue
            # (the unit or the issue slot taken), issuing
            wc = c["SQ_WAVE_CYCLES"]
            d["wave_state"] = {n: c[f"SQ_{n.upper()}"] / wc for n in
                               ("wait_any", "wait_inst_any", "active_inst_any", "active_inst_valu",
                                "active_inst_lds", "active_inst_vmem", "wait_inst_lds")
                               if f"SQ_{n.upper()}" in c}
        if "FETCH_SIZE" in c and cal.get("FETCH_SIZE"):
            d["fetch_bytes"] = c["FETCH_SIZE"] * COPY_BYTES / cal["FETCH_SIZE"]
        if "WRITE_SIZE" in c and cal.get("WRITE_SIZE"):
            d["write_bytes"] = c["WRITE_SIZE"] * COPY_BYTES / cal["WRITE_SIZE"]
        if "TCC_EA0_RDREQ_sum" in c and cal.get("TCC_EA0_RDREQ_sum"):
            d["fetch_bytes_by_rdreq"] = c["TCC_EA0_RDREQ_sum"] * COPY_BYTES / cal["TCC_EA0_RDREQ_sum"]
        if "TCC_MISS_sum" in c and cal.get("TCC_MISS_sum"):
            d["fetch_bytes_by_l2_miss"] = c["TCC_MISS_sum"] * COPY_BYTES / cal["TCC_MISS_sum"]
        out["kernels"][sk] = d
    path = os.path.join(ROOT, "profiles", f"pmc_{config}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def summarize_trace(db: str):
    """Per-kernel durations of a rocprofv3 --kernel-trace database (the
    kernels view: end - start of every dispatch), as the markdown table the
    kernel-trace summaries under profiles/ hold: calls, total, average,
    median and minimum in microseconds, and each kernel's share of the total."""
    import sqlite3
    import statistics
    from collections import defaultdict
    con = sqlite3.connect(db)
    cols = [r[1] for r in con.execute("pragma table_info(kernels)")]
    ki = cols.index("kernel_name") if "kernel_name" in cols else cols.index("name")
    si, ei = cols.index("start"), cols.index("end")
    dur = defaultdict(list)
    for row in con.execute("select * from kernels"):
        dur[row[ki]].append((row[ei] - row[si]) / 1000.0)
    total = sum(sum(v) for v in dur.values())
    print("| kernel | calls | total (us) | average (us) | median (us) | min (us) | share |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for k, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{k[:70]}` | {len(v)} | {sum(v):.1f} | {sum(v) / len(v):.3f} | "
              f"{statistics.median(v):.3f} | {min(v):.3f} | {100 * sum(v) / total:.1f}% |")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_single_thread(wl_main, budget_s: float = 20.0):
    """The oracle on one thread: whole rounds of the tiny and the main
    workload, and the exit law alone on every workload (the 32-request one
    on its first four requests), each timed once."""
    import numpy as np
    import oracle
    from tests import workloads as W
    out = {"threads": 1}

    def one_round(wl):
        u1 = np.ascontiguousarray(wl.uniforms[:, :1, :])
        t0 = time.perf_counter()
        oracle.tree_attn(wl.q, wl.k, wl.v, wl.dtype, wl.parents, wl.P, wl.scale, nthreads=1)
        el = oracle.exit_law(wl.logits, wl.dtype, wl.parents, wl.tokens, wl.inv_temperature, nthreads=1)
        oracle.sample(wl.logits, wl.dtype, wl.parents, wl.tokens, el.exit_mass, u1, wl.inv_temperature,
                      nthreads=1)
        return time.perf_counter() - t0

    t_start = time.perf_counter()
    rounds = {}
    for wl in (W.make_config("tiny", n_uniform=1), wl_main):
        dt = one_round(wl)
        rounds[wl.name] = {"s_per_round": round(dt, 4), "nodes_per_s": round(wl.R * wl.B / dt, 2)}
    out["round"] = rounds
    exit_law = {}
    for name in ("tiny", "qwen3_4b", "qwen3_8b_wide", "mixture", "batched"):
        if time.perf_counter() - t_start > budget_s:
            break
        wl = W.make_config(name, n_uniform=1, with_attention=False,
                           requests=4 if name == "batched" else None)
        t0 = time.perf_counter()
        oracle.exit_law(wl.logits, wl.dtype, wl.parents, wl.tokens, wl.inv_temperature, nthreads=1)
        dt = time.perf_counter() - t0
        exit_law[name] = {"rows": wl.R * wl.B, "s": round(dt, 4), "rows_per_s": round(wl.R * wl.B / dt, 1)}
    out["exit_law"] = exit_law
    out["note"] = ("one OpenMP thread; the round is attention + exit law + one draw per request; "
                   "the 32-request workload's exit law on its first 4 requests")
    return out


def timed_graphs(torch, stream, graphs, n_rounds, G, ring):
    """Replay graphs of G rounds (then one-round graphs) for exactly n_rounds,
    an event pair around each replay: (mean us per round, list of us per round
    of each G-round replay)."""
    per = []
    evs = []
    full, rest = divmod(n_rounds, G)
    with torch.cuda.stream(stream):
        e_all0 = torch.cuda.Event(enable_timing=True)
        e_all1 = torch.cuda.Event(enable_timing=True)
        e_all0.record(stream)
        for i in range(full):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            graphs["multi"][i % len(graphs["multi"])].replay()
            b.record(stream)
            evs.append((a, b))
        for i in range(rest):
            graphs["single"][(full * G + i) % ring].replay()
        e_all1.record(stream)
    torch.cuda.synchronize()
    for a, b in evs:
        per.append(a.elapsed_time(b) * 1e3 / G)
    return e_all0.elapsed_time(e_all1) * 1e3 / n_rounds, per


def percentiles(xs):
    import numpy as np
    if not xs:
        return None
    q = np.percentile(np.asarray(xs), [10, 50, 90])
    return {"p10": round(float(q[0]), 3), "median": round(float(q[1]), 3), "p90": round(float(q[2]), 3),
            "n": len(xs)}


def measure_workload(name, steps, ring_bytes, log_prefix="[bench]"):
    """Round time, launch intervals and roofline fractions of tev_verify_round
    on one named workload (graphs of consecutive rounds on distinct input
    copies, as for the headline workload)."""
    import numpy as np
    import torch
    from draft_tree_verification_amd import tev
    from tests import workloads as W
    t_gen = time.perf_counter()
    wl = W.make_config(name, n_uniform=1)
    gen_s = time.perf_counter() - t_gen

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    base = dict(lg=to_dev(wl.logits), q=to_dev(wl.q), k=to_dev(wl.k), v=to_dev(wl.v),
                par=tev.to_device_i32(wl.parents), tok=tev.to_device_i32(wl.tokens),
                uni=torch.from_numpy(np.ascontiguousarray(wl.uniforms[:, :1, :])).cuda())
    slot_bytes = sum(t.numel() * t.element_size() for t in base.values())
    ring = max(1, min(64, int(np.ceil(ring_bytes / slot_bytes))))
    slots = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(ring - 1)]
    R, B, V = wl.R, wl.B, wl.V
    ws = torch.zeros(tev.tev_verify_round_workspace_bytes(R, B, V, wl.Hq, wl.Hkv, wl.D, wl.P),
                     dtype=torch.uint8, device="cuda")
    out = tev.tev_verify_round(base["q"], base["k"], base["v"], base["lg"], base["par"], base["tok"],
                               base["uni"], wl.P, wl.scale, wl.inv_temperature, workspace=ws)

    def step(s, events=None):
        tev.tev_verify_round(s["q"], s["k"], s["v"], s["lg"], s["par"], s["tok"], s["uni"], wl.P, wl.scale,
                             wl.inv_temperature, out=out, events=events)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    G = max(1, min(11, ring))
    graphs = {"single": [], "multi": []}
    with torch.cuda.stream(stream):
        for s in slots:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(s)
            graphs["single"].append(g)
        for j in range(max(1, ring // G)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for t in range(G):
                    step(slots[(j * G + t) % ring])
            graphs["multi"].append(g)
        for i in range(2):
            graphs["multi"][i % len(graphs["multi"])].replay()
    torch.cuda.synchronize()
    mean_us, per = timed_graphs(torch, stream, graphs, steps, G, ring)
    ev = [[HipEvent() for _ in range(4)] for _ in range(max(4, min(steps, 2 * ring)) + 2)]
    with torch.cuda.stream(stream):
        for i, row in enumerate(ev):
            step(slots[i % ring], events=row)
    torch.cuda.synchronize()
    names = ("k_vocab", "k_round_attn", "k_round_tail")
    phase = {nm: float(np.mean([HipEvent.elapsed_us(row[j], row[j + 1]) for row in ev[2:]]))
             for j, nm in enumerate(names)}
    work = algorithmic_work(wl)
    attn_hbm = work["attn_bytes"] / HBM_PEAK_GBS > work["attn_flops"] / MFMA_BF16_PEAK_TFLOPS / 1e3
    vg = work["exit_law_bytes"] / (phase["k_vocab"] * 1e-6) / 1e9
    if attn_hbm:
        a = work["attn_bytes"] / (phase["k_round_attn"] * 1e-6) / 1e9
        attn = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4)}
    else:
        a = work["attn_flops"] / (phase["k_round_attn"] * 1e-6) / 1e12
        attn = {"bound": "mfma", "achieved": round(a, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(a / MFMA_BF16_PEAK_TFLOPS, 4)}
    res = {"requests": R, "nodes_per_request": B, "vocab": V, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
           "head_dim": wl.D, "kv_prefix": wl.P, "ring_copies": ring, "rounds": steps,
           "us_per_round": round(mean_us, 3), "round_us": percentiles(per),
           "nodes_per_s": round(R * B / (mean_us * 1e-6), 1),
           "launch_us": {k: round(v, 3) for k, v in phase.items()},
           "vocab": {"bytes": work["exit_law_bytes"], "achieved_gbs": round(vg, 1),
                     "frac_hbm": round(vg / HBM_PEAK_GBS, 4)},
           "attention": dict(attn, bytes=work["attn_bytes"], flops=work["attn_flops"]),
           "inputs": wl.digests()}
    log(f"{log_prefix} {name}: {mean_us:.2f} us per round ({R * B / mean_us:.3f} M nodes/s), launches "
        + ", ".join(f"{k} {v:.2f}" for k, v in phase.items()) + f" us (inputs generated in {gen_s:.1f} s)")
    del graphs, slots, base, out, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def verifier_stage(budgets, n_layers=36, iters=100):
    """TEV's decision (exit node + bonus, one draw) against predraw-and-follow
    (B node draws + walk), each followed by the cache commit of the accepted
    path over an n_layers cache, on the Qwen3-4B-shaped round at several node
    budgets (both after the same exit law)."""
    import numpy as np
    import torch
    from draft_tree_verification_amd import tev
    from tests import workloads as W
    res = {}
    stream = torch.cuda.Stream()
    for B in budgets:
        wl = W.make_qwen_budget(B)
        lg0 = torch.from_numpy(np.ascontiguousarray(wl.logits).view(np.int16)).view(torch.bfloat16).cuda()
        ring = max(1, min(33, int(np.ceil(1.2e9 / (lg0.numel() * 2)))))
        lgs = [lg0] + [lg0.clone() for _ in range(ring - 1)]
        par, tok = tev.to_device_i32(wl.parents), tev.to_device_i32(wl.tokens)
        uni = torch.from_numpy(np.ascontiguousarray(wl.uniforms[:, :1, :])).cuda()
        pd_uni = torch.from_numpy((np.random.default_rng(7).integers(0, 1 << 24, size=(1, 1, B))
                                   * 2.0 ** -24).astype(np.float32)).cuda()
        el = tev.tev_exit_law(lg0, par, tok, wl.inv_temperature)
        draws = tev.tev_sample(lg0, par, tok, el.workspace, uni, wl.inv_temperature)
        pd = tev.tev_predraw(lg0, par, tok, el.workspace, pd_uni, wl.inv_temperature)
        kc = torch.zeros((n_layers, 1, wl.Hkv, wl.P + B, wl.D), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        exit_nodes = draws[0][:, 0].contiguous()
        new_len = torch.empty((1,), dtype=torch.int32, device="cuda")
        calls = {
            "tev_sample": lambda j: tev.tev_sample(lgs[j % ring], par, tok, el.workspace, uni, wl.inv_temperature,
                                                   out=draws),
            "tev_predraw": lambda j: tev.tev_predraw(lgs[j % ring], par, tok, el.workspace, pd_uni,
                                                     wl.inv_temperature, out=pd),
            "tev_commit_kv": lambda j: tev.tev_commit_kv(kc, vc, par, exit_nodes, wl.P, out=new_len),
        }
        G = 11
        us = {}
        for name, fn in calls.items():
            gs = []
            with torch.cuda.stream(stream):
                for j in range(max(1, ring // G)):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=stream):
                        for t in range(G):
                            fn(j * G + t)
                    gs.append(g)
                for i in range(2):
                    gs[i % len(gs)].replay()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            reps = max(1, iters // G)
            with torch.cuda.stream(stream):
                a.record(stream)
                for i in range(reps):
                    gs[i % len(gs)].replay()
                b.record(stream)
            torch.cuda.synchronize()
            us[name] = a.elapsed_time(b) / (reps * G) * 1e3
            del gs
        tev_stage = us["tev_sample"] + us["tev_commit_kv"]
        pd_stage = us["tev_predraw"] + us["tev_commit_kv"]
        res[f"B={B}"] = {"tev_sample_us": round(us["tev_sample"], 3), "tev_predraw_us": round(us["tev_predraw"], 3),
                         "tev_commit_kv_us": round(us["tev_commit_kv"], 3),
                         "tev_stage_us": round(tev_stage, 3), "predraw_stage_us": round(pd_stage, 3),
                         "tev_reduction": round(1.0 - tev_stage / pd_stage, 4)}
        log(f"[bench] verifier stage at B={B}: TEV {tev_stage:.2f} us vs predraw {pd_stage:.2f} us "
            f"({100 * (1 - tev_stage / pd_stage):.1f}% lower; commit over {n_layers} layers)")
        del lgs, kc, vc, el, draws, pd
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    res["note"] = ("both after the same tev_exit_law; decision (one draw per request) plus the cache "
                   f"commit over {n_layers} layers of the 32/8-head, 4096-prefix cache; Qwen3-4B-shaped "
                   "round cut at each node budget")
    return res


def device_peaks():
    """Context: a 1 GiB device copy (read + write), a 1 GiB read (sum), and
    a bf16 8192^3 GEMM, on this GPU."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    f = src.view(torch.float32)
    a = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda")

    def t(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    copy_s = t(lambda: dst.copy_(src), 10)
    read_s = t(lambda: f.sum(), 10)
    gemm_s = t(lambda: torch.matmul(a, b), 10)
    # the qwen3_4b logit bytes (64 x 151936 bf16): a read of that size alone,
    # over 16 distinct copies so that every read comes from HBM
    small = src[: 16 * (64 * 151936 * 2)].view(torch.bfloat16).view(16, 64 * 151936)
    ring = iter(range(1 << 30))
    small_s = t(lambda: small[next(ring) % 16].sum(dtype=torch.float32), 160)
    out = {"copy_1gib_gbs": round(2 * n / copy_s / 1e9, 1), "read_1gib_gbs": round(n / read_s / 1e9, 1),
           "read_qwen3_4b_logits_gbs": round(64 * 151936 * 2 / small_s / 1e9, 1),
           "gemm_bf16_8192_tflops": round(2 * 8192 ** 3 / gemm_s / 1e12, 1),
           "note": "torch copy_ (bytes read + written), torch sum of f32 (bytes read), torch sum of one "
                   "19.45 MB bf16 tensor of 16 (the qwen3_4b logit bytes; launch gaps included), "
                   "torch.matmul bf16; context for the 8 TB/s and 2.5 PFLOP/s spec peaks"}
    del src, dst, a, b, small
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="qwen3_4b")
    ap.add_argument("--ring-bytes", type=float, default=1.2e9,
                    help="total size of the ring of input copies (defeats the 256 MB MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--call-iters", type=int, default=100)
    ap.add_argument("--rounds-per-graph", type=int, default=11,
                    help="rounds captured back to back in one graph for the timed loop")
    ap.add_argument("--counters", type=int, default=0,
                    help="counter-collection mode: replay this many one-round graphs and one "
                         "calibration copy of a known size, then exit (run under rocprofv3 --pmc)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc "
                         "databases (FETCH_SIZE run, WRITE_SIZE run) of a --counters run")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DB",
                    help="write profiles/pmc_<workload>.json from the rocprofv3 --pmc databases "
                         "(one per counter pass) of a --counters run")
    ap.add_argument("--summarize-trace", metavar="DB",
                    help="print the per-kernel duration table of a rocprofv3 --kernel-trace database")
    ap.add_argument("--separate", action="store_true",
                    help="time the three calls tev_tree_attn, tev_exit_law, tev_sample instead of tev_verify_round")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads, the verifier-stage comparison and the device peaks")
    args = ap.parse_args()

    if args.summarize_counters:
        summarize_counters(args.config, *args.summarize_counters)
        return
    if args.summarize_pmc:
        summarize_pmc(args.config, args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the verification stage "
              "runs on a single device; the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from draft_tree_verification_amd import tev
    from tests import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    wl = W.make_config(args.config, n_uniform=1)
    log(f"[bench] workload {wl.name}: {wl.meta['description']} (generated in "
        f"{time.perf_counter() - t_gen:.1f} s)")
    R, B, V = wl.R, wl.B, wl.V

    def to_dev(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()

    base = dict(lg=to_dev(wl.logits), q=to_dev(wl.q), k=to_dev(wl.k), v=to_dev(wl.v),
                par=tev.to_device_i32(wl.parents), tok=tev.to_device_i32(wl.tokens),
                uni=torch.from_numpy(np.ascontiguousarray(wl.uniforms[:, :1, :])).cuda())
    slot_bytes = sum(t.numel() * t.element_size() for t in base.values())
    ring = max(1, min(64, int(np.ceil(args.ring_bytes / slot_bytes))))
    slots = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(ring - 1)]
    log(f"[bench] {slot_bytes / 1e6:.1f} MB of inputs per round, ring of {ring} copies "
        f"({ring * slot_bytes / 1e9:.2f} GB)")

    ws_e = torch.zeros(tev.tev_exit_law_workspace_bytes(R, B, V), dtype=torch.uint8, device="cuda")
    ws_a = torch.zeros(max(1, tev.tev_tree_attn_workspace_bytes(R, B, wl.Hq, wl.Hkv, wl.D, wl.P)),
                       dtype=torch.uint8, device="cuda")
    out_attn = torch.empty((R, B, wl.Hq, wl.D), dtype=torch.float32, device="cuda")
    el_out = tev.ExitLawResult(*[torch.empty((R, B), dtype=torch.float32, device="cuda") for _ in range(3)],
                               torch.empty((R,), dtype=torch.float32, device="cuda"), ws_e)
    draws = (torch.empty((R, 1), dtype=torch.int32, device="cuda"),
             torch.empty((R, 1), dtype=torch.int32, device="cuda"))

    def call_attn(s):
        tev.tev_tree_attn(s["q"], s["k"], s["v"], s["par"], wl.P, wl.scale, workspace=ws_a, out=out_attn)

    def call_exit(s):
        tev.tev_exit_law(s["lg"], s["par"], s["tok"], wl.inv_temperature, out=el_out)

    def call_sample(s):
        tev.tev_sample(s["lg"], s["par"], s["tok"], ws_e, s["uni"], wl.inv_temperature, out=draws)

    # Predraw-and-follow (the pages' baseline verifier): one uniform per node
    pd_uni = torch.from_numpy((np.random.default_rng(7).integers(0, 1 << 24, size=(R, 1, B))
                               * 2.0 ** -24).astype(np.float32)).cuda()
    pd_out = (torch.empty((R, 1, B), dtype=torch.int32, device="cuda"),
              torch.empty((R, 1), dtype=torch.int32, device="cuda"),
              torch.empty((R, 1), dtype=torch.int32, device="cuda"))

    def call_predraw(s):
        tev.tev_predraw(s["lg"], s["par"], s["tok"], ws_e, pd_uni, wl.inv_temperature, out=pd_out)

    def step_separate(s):
        call_attn(s)
        call_exit(s)
        call_sample(s)

    ws_r = torch.zeros(tev.tev_verify_round_workspace_bytes(R, B, V, wl.Hq, wl.Hkv, wl.D, wl.P),
                       dtype=torch.uint8, device="cuda")
    round_out = tev.RoundResult(out_attn, el_out.rho, el_out.reach, el_out.exit_mass, el_out.coverage,
                                draws[0], draws[1], ws_r)

    def step_round(s):
        tev.tev_verify_round(s["q"], s["k"], s["v"], s["lg"], s["par"], s["tok"], s["uni"], wl.P,
                             wl.scale, wl.inv_temperature, out=round_out)

    step = step_separate if args.separate else step_round

    # eager check of one round before capture
    step(slots[0])
    torch.cuda.synchronize()
    cov = float(el_out.coverage[0])
    assert np.isfinite(cov), "exit law returned a non-finite coverage"
    log(f"[bench] eager round ok: coverage {cov:.4f}, exit node {int(draws[0][0, 0])}, "
        f"bonus {int(draws[1][0, 0])}")

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def capture(fn):
        graphs = []
        with torch.cuda.stream(stream):
            for s in slots:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    fn(s)
                graphs.append(g)
        torch.cuda.synchronize()
        return graphs

    g_step = capture(step)
    if args.counters:
        with torch.cuda.stream(stream):
            for i in range(args.counters):
                g_step[i % ring].replay()
            # calibration: a device copy of exactly COPY_BYTES (read once, written once)
            src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
            dst = torch.empty_like(src)
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] counters run: {args.counters} rounds and one {COPY_BYTES >> 20} MiB copy")
        return
    # Graphs of G consecutive rounds (distinct ring slots): as nodes of a
    # captured decode step would run them, without one graph launch per round.
    G = max(1, min(args.rounds_per_graph, ring))
    n_multi = ring // G
    g_multi = []
    with torch.cuda.stream(stream):
        for j in range(n_multi):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for t in range(G):
                    step(slots[j * G + t])
            g_multi.append(g)
    torch.cuda.synchronize()
    log(f"[bench] captured {len(g_step)} one-round graphs and {n_multi} graphs of {G} rounds")

    def run_steps(n):
        """Exactly n rounds: graphs of G rounds, then one-round graphs."""
        full, rest = divmod(n, G)
        for i in range(full):
            g_multi[i % n_multi].replay()
        for i in range(rest):
            g_step[(full * G + i) % ring].replay()

    with torch.cuda.stream(stream):
        run_steps(args.warmup)
    torch.cuda.synchronize()

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            fn(n)
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_per_step = timed(run_steps, args.steps)
    value = R * B / (ms_per_step * 1e-3)
    # spread: one event pair around each G-round graph replay of a second pass
    _, per_round = timed_graphs(torch, stream, {"multi": g_multi, "single": g_step}, args.steps, G, ring)
    round_pct = percentiles(per_round)
    log(f"[bench] {ms_per_step * 1e3:.2f} us per round -> {value / 1e6:.3f} M nodes/s"
        + (f" (per-graph median {round_pct['median']:.2f}, p10 {round_pct['p10']:.2f}, p90 {round_pct['p90']:.2f})"
           if round_pct else ""))
    ms_single = timed(lambda n: [g_step[i % ring].replay() for i in range(n)], args.steps)
    log(f"[bench] {ms_single * 1e3:.2f} us per round with one graph launch per round")

    # Launch durations of the round: tev_verify_round_timed records four HIP
    # events at its launch boundaries.  The events skip the system-scope fence
    # of a default event (which would add a cache flush to every boundary), so
    # each interval is the launch plus its dispatch gap.  Rounds are enqueued
    # back to back (the host runs ahead of the GPU), then read.
    n_phase = max(args.call_iters, 2 * ring)
    ev = [[HipEvent() for _ in range(4)] for _ in range(n_phase + 6)]
    with torch.cuda.stream(stream):
        for i, row in enumerate(ev):
            sl = slots[i % ring]
            tev.tev_verify_round(sl["q"], sl["k"], sl["v"], sl["lg"], sl["par"], sl["tok"], sl["uni"],
                                 wl.P, wl.scale, wl.inv_temperature, out=round_out, events=row)
    torch.cuda.synchronize()
    names = ("k_vocab", "k_round_attn", "k_round_tail")
    phase_us = {nm: float(np.mean([HipEvent.elapsed_us(row[j], row[j + 1]) for row in ev[6:]]))
                for j, nm in enumerate(names)}
    log("[bench] round launches (us): " + ", ".join(f"{k} {v:.2f}" for k, v in phase_us.items()))

    # per-call durations of the separate calls: graphs of G consecutive calls
    # on distinct ring slots, as the round itself is timed
    per_call = {}
    call_exit(slots[0])   # a filled exit-law workspace for the draw calls
    for name, fn in (("tev_tree_attn", call_attn), ("tev_exit_law", call_exit), ("tev_sample", call_sample),
                     ("tev_predraw", call_predraw)):
        gs = []
        with torch.cuda.stream(stream):
            for j in range(n_multi):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for t in range(G):
                        fn(slots[j * G + t])
                gs.append(g)
            for i in range(2):
                gs[i % n_multi].replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        reps = max(1, args.call_iters // G)
        with torch.cuda.stream(stream):
            a.record(stream)
            for i in range(reps):
                gs[i % n_multi].replay()
            b.record(stream)
        torch.cuda.synchronize()
        per_call[name] = a.elapsed_time(b) / (reps * G) * 1e3   # us
        del gs
    log(f"[bench] per call (us): " + ", ".join(f"{k} {v:.2f}" for k, v in per_call.items()))

    # cache commit of the drawn exit node's root path over a 36-layer cache of
    # the workload's kv layout (the depth of a Qwen3-4B target); in place, so
    # repeated commits keep permuting rows inside the tree region
    # (the prefix rows are never touched: past 4 GB of cache the prefix is left
    # out, P = 0, and the same rows move)
    n_layers = 36
    esz_kv = base["k"].element_size()
    P_c = wl.P if 2 * n_layers * R * wl.Hkv * (wl.P + B) * wl.D * esz_kv <= (4 << 30) else 0
    kc = torch.zeros((n_layers, R, wl.Hkv, P_c + B, wl.D), dtype=base["k"].dtype, device="cuda")
    vc = torch.zeros_like(kc)
    exit_nodes = draws[0][:, 0].contiguous()
    new_len = torch.empty((R,), dtype=torch.int32, device="cuda")

    def call_commit(s):
        tev.tev_commit_kv(kc, vc, s["par"], exit_nodes, P_c, out=new_len)

    gs = []
    with torch.cuda.stream(stream):
        for j in range(n_multi):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for t in range(G):
                    call_commit(slots[j * G + t])
            gs.append(g)
        for i in range(2):
            gs[i % n_multi].replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    reps = max(1, args.call_iters // G)
    with torch.cuda.stream(stream):
        a.record(stream)
        for i in range(reps):
            gs[i % n_multi].replay()
        b.record(stream)
    torch.cuda.synchronize()
    per_call["tev_commit_kv"] = a.elapsed_time(b) / (reps * G) * 1e3
    del gs, kc, vc
    log(f"[bench] tev_commit_kv ({n_layers} layers, prefix {P_c}): {per_call['tev_commit_kv']:.2f} us")

    # the exit-guided draft-tree loss on the workload's own draft rows, weighted
    # by the exit masses the exit law just produced (loss alone, then with the
    # gradient), graphs of consecutive calls over a ring of draft-row copies
    exit_loss = None
    tree_build = None
    loss_w_host = None
    tb_args = None
    try:
        zrows = W.draft_rows(wl.name)
    except KeyError:
        zrows = None
    if zrows is not None:
        H = zrows.shape[1]
        z0 = to_dev(zrows)
        zring = [z0] + [z0.clone() for _ in range(max(1, min(64, int(np.ceil(
            args.ring_bytes / (z0.numel() * z0.element_size()))))) - 1)]
        el_w = el_out.exit_mass.clone()
        loss_w_host = el_w.cpu().numpy()
        ws_l = torch.empty(tev.tev_exit_loss_workspace_bytes(R, B, H, V), dtype=torch.uint8, device="cuda")
        lo = tev.ExitLossResult(torch.empty(1, dtype=torch.float32, device="cuda"),
                                torch.empty((R, H), dtype=torch.float32, device="cuda"),
                                torch.empty((R, H), dtype=torch.float32, device="cuda"), None, ws_l)
        lo_g = tev.ExitLossResult(lo.loss, lo.row_lse, lo.row_weight,
                                  torch.empty((R, H, V), dtype=torch.float32, device="cuda"), ws_l)
        exit_loss = {"rows": R * H, "vocab": V, "copies": len(zring)}
        esz = z0.element_size()
        for name, o, nbytes in (("loss", lo, R * H * V * esz), ("loss_and_grad", lo_g, R * H * V * (2 * esz + 4))):
            def fn(j, o=o):
                tev.tev_exit_loss(zring[j % len(zring)], base["par"], base["tok"], el_w, out=o)
            gs = []
            with torch.cuda.stream(stream):
                for j in range(n_multi):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=stream):
                        for t in range(G):
                            fn(j * G + t)
                    gs.append(g)
                for i in range(2):
                    gs[i % n_multi].replay()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            reps = max(1, args.call_iters // G)
            with torch.cuda.stream(stream):
                a.record(stream)
                for i in range(reps):
                    gs[i % n_multi].replay()
                b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / (reps * G) * 1e3
            del gs
            gbs = nbytes / (us * 1e-6) / 1e9
            exit_loss[name] = {"us": round(us, 3), "bytes": nbytes, "achieved_gbs": round(gbs, 1),
                               "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        exit_loss["loss_value"] = float(lo.loss[0])
        log(f"[bench] tev_exit_loss over {R * H} draft rows: loss {exit_loss['loss']['us']:.2f} us, "
            f"loss + grad {exit_loss['loss_and_grad']['us']:.2f} us "
            f"({exit_loss['loss_and_grad']['achieved_gbs']:.0f} GB/s)")
        del zring

    # the tree builder on the workload's own draft rows (B tokens kept per
    # position, up to 128; the mixture's 8 draft modes through the merged heap)
    try:
        zb, nmodes = W.draft_rows(wl.name), 1
    except KeyError:
        zb, nmodes = (W.draft_rows_modes(wl.name), 8) if wl.name == "mixture" else (None, 0)
    if zb is not None:
        zb0 = to_dev(zb)
        zbring = [zb0] + [zb0.clone() for _ in range(max(1, min(64, int(np.ceil(
            args.ring_bytes / (zb0.numel() * zb0.element_size()))))) - 1)]
        Kb = min(B, 128)
        roots = base["tok"][:, 0].contiguous()
        tb_args = (zb, wl.dtype, Kb, B, wl.tokens[:, 0].copy(), nmodes)
        if nmodes == 1:
            tb = tev.tev_build_tree(zb0, Kb, B, roots)

            def fn_tb(j):
                tev.tev_build_tree(zbring[j % len(zbring)], Kb, B, out=tb)
        else:
            tb = tev.tev_build_tree_modes(zb0, Kb, B, None, roots)

            def fn_tb(j):
                tev.tev_build_tree_modes(zbring[j % len(zbring)], Kb, B, None, out=tb)
        gs = []
        with torch.cuda.stream(stream):
            for j in range(n_multi):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for t in range(G):
                        fn_tb(j * G + t)
                gs.append(g)
            for i in range(2):
                gs[i % n_multi].replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        reps = max(1, args.call_iters // G)
        with torch.cuda.stream(stream):
            a.record(stream)
            for i in range(reps):
                gs[i % n_multi].replay()
            b.record(stream)
        torch.cuda.synchronize()
        tb_us = a.elapsed_time(b) / (reps * G) * 1e3
        del gs, zbring
        rows = zb.shape[0] * nmodes * zb.shape[-2]
        tree_build = {"us": round(tb_us, 3), "modes": nmodes, "K": Kb, "B": B, "rows": rows, "vocab": V,
                      "call": "tev_build_tree" if nmodes == 1 else "tev_build_tree_modes"}
        log(f"[bench] {tree_build['call']} over {rows} draft rows (K={Kb}, B={B}): {tb_us:.2f} us")

    work = algorithmic_work(wl)
    attn_hbm_bound = work["attn_bytes"] / HBM_PEAK_GBS > work["attn_flops"] / MFMA_BF16_PEAK_TFLOPS / 1e3

    def attn_roof(us):
        gbs = work["attn_bytes"] / (us * 1e-6) / 1e9
        tfs = work["attn_flops"] / (us * 1e-6) / 1e12
        if attn_hbm_bound:
            return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4)}
        return {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4)}

    def vocab_roof(us):
        gbs = work["exit_law_bytes"] / (us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}

    kernels = {
        "k_vocab": dict(us=round(phase_us["k_vocab"], 3), bytes=work["exit_law_bytes"],
                        **vocab_roof(phase_us["k_vocab"])),
        "k_round_attn": dict(us=round(phase_us["k_round_attn"], 3), bytes=work["attn_bytes"],
                             flops=work["attn_flops"], **attn_roof(phase_us["k_round_attn"]),
                             note="attention workgroups + the reach workgroup of each request, which also "
                                  "makes the request's draws (at most four per request)"),
        "k_round_tail": {"us": round(phase_us["k_round_tail"], 3),
                         "note": "the attention split combine (no launch without prefix splits); draw "
                                 "workgroups only with more than four draws per request"},
        "separate_calls_us": {k: round(v, 3) for k, v in per_call.items()},
        "verifier_decision_us": {"tev_sample (exit node + bonus)": round(per_call["tev_sample"], 3),
                                 "tev_predraw (B node draws + walk)": round(per_call["tev_predraw"], 3),
                                 "tev_commit_kv (36 layers)": round(per_call["tev_commit_kv"], 3),
                                 "tev stage (sample + commit)": round(per_call["tev_sample"]
                                                                      + per_call["tev_commit_kv"], 3),
                                 "predraw stage (predraw + commit)": round(per_call["tev_predraw"]
                                                                           + per_call["tev_commit_kv"], 3),
                                 "note": "both after the same tev_exit_law; one draw per request"},
        "tev_exit_loss": exit_loss,
        "tev_build_tree": tree_build,
    }
    dominant = max(("k_vocab", "k_round_attn"), key=phase_us.get)
    roof = dict(kernels[dominant])
    for k_ in ("us", "bytes", "flops", "note"):
        roof.pop(k_, None)
    roof["kernel"] = dominant
    roof["launch_us"] = round(phase_us[dominant], 3)
    src_hash = kernel_source_hash()
    traffic = load_traffic(wl.name, src_hash)
    tk = traffic.get("kernels", {}).get(dominant) if traffic else None
    roof["traffic"] = round(tk["bytes_per_launch"]) if tk else None

    extra = {}
    if not args.no_extra:
        del slots, g_step, g_multi
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        extra["verifier_stage"] = verifier_stage((32, 64, 128))
        extra["device_peaks"] = device_peaks()
        log(f"[bench] device peaks: {extra['device_peaks']}")
        wls = {}
        for name, st_ in (("qwen3_8b_wide", 50), ("mixture", 50), ("batched", 10)):
            wls[name] = measure_workload(name, min(args.steps, st_), args.ring_bytes)
        extra["workloads"] = wls

    cpu = None
    rows_cpu = {}
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        cpu = cpu_baseline(wl, args.cpu_seconds)
        cpu["cpu_model"] = cpu_model()
        log(f"[bench] oracle: {cpu['value']:.1f} nodes/s on {cpu['cores']} threads ({cpu['cpu_model']})")
        rows_cpu = oracle_rows_us(wl, pd_uni.cpu().numpy(), exit_nodes.cpu().numpy(), n_layers, P_c,
                                  zrows, loss_w_host, tb_args)
        log("[bench] oracle per widened call (us): " + ", ".join(f"{k} {v:.0f}" for k, v in rows_cpu.items()))
        if not args.no_extra:
            import oracle
            n_thr = oracle.max_threads(0)
            cpu["single_thread"] = oracle_single_thread(wl)
            oracle.max_threads(n_thr)
            log(f"[bench] oracle on one thread: {cpu['single_thread']}")

    # The widened rows: GPU time, algorithmic bytes, what bounds them and the
    # host oracle's time for the same call.
    esz_l = 2 if wl.dtype == "bf16" else 4
    nc = (V + 4095) // 4096
    depth_mean = float(np.mean([W.depths_of(p).mean() for p in wl.parents]))
    widened = {
        "tev_predraw": {"us": per_call["tev_predraw"], "bound": "latency",
                        "bytes": int(R * B * (nc * 24 + 4096 * esz_l))},
        "tev_commit_kv": {"us": per_call["tev_commit_kv"], "bound": "latency",
                          "bytes": int(4 * n_layers * R * wl.Hkv * (depth_mean + 1) * wl.D * esz_kv)},
    }
    if exit_loss is not None:
        widened["tev_exit_loss"] = {"us": exit_loss["loss"]["us"], "bound": "hbm",
                                    "bytes": exit_loss["loss"]["bytes"]}
        widened["tev_exit_loss (with gradient)"] = {"us": exit_loss["loss_and_grad"]["us"], "bound": "hbm",
                                                    "bytes": exit_loss["loss_and_grad"]["bytes"]}
    if tree_build is not None:
        widened[tree_build["call"]] = {"us": tree_build["us"], "bound": "latency",
                                       "bytes": int(tree_build["rows"] * V * esz_l)}
    for k_, e in widened.items():
        e["us"] = round(e["us"], 3)
        e["achieved_gbs"] = round(e["bytes"] / (e["us"] * 1e-6) / 1e9, 1)
        e["frac_hbm"] = round(e["achieved_gbs"] / HBM_PEAK_GBS, 4)
        base_k = k_.split(" ")[0]
        if base_k in rows_cpu and k_ == base_k:
            e["oracle_cpu_us"] = rows_cpu[base_k]

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "nodes/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded; shapes of the pages' Qwen3 workloads)",
        "config": {"workload": wl.name, "requests": R, "nodes_per_request": B, "vocab": V,
                   "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": wl.D, "kv_prefix": wl.P,
                   "draws_per_request": 1, "ring_copies": ring, "graph": True,
                   "call": "tev_tree_attn + tev_exit_law + tev_sample" if args.separate
                   else "tev_verify_round", "rounds_per_graph": G},
        "ms_per_step_one_graph_per_round": round(ms_single, 6),
        "round_us": round_pct,
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "widened_calls": widened,
        **extra,
        "kernel_source_hash": src_hash,
        "inputs": wl.digests(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
