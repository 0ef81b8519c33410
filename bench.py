"""Benchmark of the PolyKV shared-pool hot path on one MI355X.

One step = one pass of the whole hot path over one synthetic workload: write-once
compression of the fp16 K and V of every layer into the pool (compress_k + compress_v),
then D decode steps of all agents against that pool (one attend_shared launch each).
Inputs (fp16 K/V and the queries of all D decode steps) are resident in HBM before timing.

Every launch goes to one explicit stream; HIP events recorded on that stream bracket each
compress launch and each step's run of D back-to-back decode launches (average decode
launch = that interval / D). Three identical copies of the pool are used in turn, so each decode launch reads a
copy that at least two pool-sized streams have passed through the 256 MB Infinity Cache
since it was last touched: it comes from HBM (--warm uses a single copy). Decode launches
right after a 1 GiB write (cold caches and address translations) are timed separately and
reported beside the main figures.

Prints ONE JSON line. value = whole-job agent-tokens/s = agents * D / (compress time +
D * decode time), from the event times. Also reported: compress GB/s and decode GB/s over
algorithmic bytes, each as a fraction of the 8 TB/s HBM peak, a roofline object for the
decode kernel, and the CPU oracle timed on a bounded sample (cpu_baseline).
"""

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "shared-pool decode agent-tokens/s + compress GB/s, % of HBM peak"


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--config", default="3", help="workload index or name (default: the 4K Llama-3-8B pool)")
    p.add_argument("--decode-steps", type=int, default=None, help="decode launches per step (default: the workload's)")
    p.add_argument("--path", choices=["auto", "valu", "mfma"], default="auto")
    p.add_argument("--warm", action="store_true", help="one pool copy, left in the caches between launches")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--chunk-tokens", type=int, default=512,
                   help="prefill chunk size for the append figure")
    p.add_argument("--tail-tokens", type=int, default=None,
                   help="private fp16 tail per agent for the tail-merge figure (default: the decode steps)")
    p.add_argument("--cpu-sample-layers", type=int, default=None)
    p.add_argument("--mode", choices=["bench", "profile", "copy", "summarize"], default="bench",
                   help="profile: a few launches for rocprofv3 and no JSON; copy: a 1 GiB device copy "
                        "for counter calibration; summarize: write profiles/ from rocprofv3 output")
    # summarize: rocprofv3 output directories and the exact commands that produced them
    p.add_argument("--trace-dir")
    p.add_argument("--trace-cmd", default="")
    p.add_argument("--fetch-dir")
    p.add_argument("--fetch-cmd", default="")
    p.add_argument("--write-dir")
    p.add_argument("--write-cmd", default="")
    p.add_argument("--calib-fetch-dir")
    p.add_argument("--calib-write-dir")
    p.add_argument("--calib-cmds", default="")
    p.add_argument("--workload", help="workload name the summaries are filed under")
    p.add_argument("--only", default="", help="comma-separated profile names to write (default: all found)")
    p.add_argument("--sq-dirs", default="", help="comma-separated rocprofv3 --pmc output directories of SQ counters")
    p.add_argument("--sq-cmds", default="", help="the commands that made --sq-dirs, one per line")
    return p.parse_args()


# Product kernels as they appear in rocprofv3 traces: (profile name, part of the demangled
# kernel name, the source files its code comes from).
KERNELS = (
    ("attend_mfma", "k_attend_mfma<", ("attend_mfma.hip", "lds_dma.h", "polykv_internal.h")),
    ("attend_valu", "k_attend_valu<", ("attend.hip", "polykv_internal.h")),
    ("attend_tail", "k_attend_tail<", ("attend_tail.hip", "polykv_internal.h")),
    ("compress_k", "k_compress_k(", ("compress.hip", "codec.h", "polykv_internal.h")),
    ("compress_v", "k_compress_v_mfma<", ("compress.hip", "codec.h", "polykv_internal.h")),
    ("compress_kv", "k_compress_kv<", ("compress.hip", "codec.h", "polykv_internal.h")),
    ("compress_v_valu", "k_compress_v<", ("compress.hip", "codec.h", "polykv_internal.h")),
    ("dequant_k", "k_dequant_k", ("dequant.hip", "polykv_internal.h")),
    ("dequant_v", "k_dequant_v<", ("dequant.hip", "polykv_internal.h")),
    ("project_store", ", 0>(polykv::(anonymous namespace)::PjArgs)", ("project.hip", "codec.h", "lds_dma.h", "polykv_internal.h")),
    ("project_pool", ", 1>(polykv::(anonymous namespace)::PjArgs)", ("project.hip", "codec.h", "lds_dma.h", "polykv_internal.h")),
)
SOURCES = {name: files for name, _, files in KERNELS}


def _src_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "agent_q8_quant_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel, workload):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    sha = _src_sha(SOURCES[kernel])
    for line in open(path):
        f = line.split()
        if len(f) == 4 and not line.startswith("#") and f[0] == kernel and f[1] == workload:
            return int(f[3]) if f[2] == sha else None
    return None


def _csv_rows(d, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit("no %s under %s" % (suffix, d))
    return list(csv.DictReader(open(files[0])))


def _kernel_of(name):
    for prof, key, _ in KERNELS:
        if key in name and "polykv" in name:
            return prof
    return None


def _counter(d, counter):
    """{profile name: {grid: [per-dispatch value]}} of one PMC counter."""
    out = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        prof = _kernel_of(r["Kernel_Name"])
        if prof:
            out.setdefault(prof, {}).setdefault(r["Grid_Size"], {}).setdefault(r["Dispatch_Id"], 0.0)
            out[prof][r["Grid_Size"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: {g: list(v.values()) for g, v in gr.items()} for k, gr in out.items()}


def summarize(args):
    """Write profiles/<kernel>_<workload>.txt and profiles/hbm_traffic.txt from rocprofv3
    output: kernel-trace durations per launch grid, and FETCH_SIZE / WRITE_SIZE per dispatch
    scaled by what the same counters read for a 1 GiB device copy. Every figure written here
    comes from the given directories; the source hash is computed from the current files."""
    import statistics
    wl = args.workload
    prof_dir = os.path.join(ROOT, "profiles")
    fscale = wscale = None
    if args.calib_fetch_dir and args.calib_write_dir:
        cf = [float(r["Counter_Value"]) for r in _csv_rows(args.calib_fetch_dir, "counter_collection.csv")
              if r["Counter_Name"] == "FETCH_SIZE" and "copyBuffer" in r["Kernel_Name"]]
        cw = [float(r["Counter_Value"]) for r in _csv_rows(args.calib_write_dir, "counter_collection.csv")
              if r["Counter_Name"] == "WRITE_SIZE" and "copyBuffer" in r["Kernel_Name"]]
        kib = float(1 << 20)  # 1 GiB in KiB
        fscale, wscale = kib / statistics.mean(cf), kib / statistics.mean(cw)
        with open(os.path.join(prof_dir, "hbm_counter_calibration_copy_1GiB.txt"), "w") as f:
            f.write("# HBM counter calibration: 1 GiB device-to-device copy\n\n")
            f.write("Commands (repository root, one MI355X):\n%s\n\n" % args.calib_cmds)
            f.write("Kernel __amd_rocclr_copyBuffer, 1 GiB read + 1 GiB written per dispatch, %d dispatches.\n" % len(cf))
            f.write("FETCH_SIZE per dispatch: %.0f KiB -> scale %.4f (1048576 KiB actually read)\n" % (statistics.mean(cf), fscale))
            f.write("WRITE_SIZE per dispatch: %.0f KiB -> scale %.4f (1048576 KiB actually written)\n" % (statistics.mean(cw), wscale))
    else:
        for line in open(os.path.join(prof_dir, "hbm_counter_calibration_copy_1GiB.txt")):
            if line.startswith("FETCH_SIZE per dispatch"):
                fscale = float(line.split("scale")[1].split()[0])
            if line.startswith("WRITE_SIZE per dispatch"):
                wscale = float(line.split("scale")[1].split()[0])
    trace = {}
    names = {}
    for r in _csv_rows(args.trace_dir, "kernel_trace.csv"):
        prof = _kernel_of(r["Kernel_Name"])
        if not prof:
            continue
        g = "%s x %s x %s" % (r["Grid_Size_X"], r["Grid_Size_Y"], r["Grid_Size_Z"])
        trace.setdefault(prof, {}).setdefault(g, []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
        names[prof] = r["Kernel_Name"]
    fetch = _counter(args.fetch_dir, "FETCH_SIZE") if args.fetch_dir else {}
    write = _counter(args.write_dir, "WRITE_SIZE") if args.write_dir else {}
    only = set(filter(None, args.only.split(",")))
    traffic_path = os.path.join(prof_dir, "hbm_traffic.txt")
    table = {}
    if os.path.exists(traffic_path):
        for line in open(traffic_path):
            f = line.split()
            if len(f) == 4 and not line.startswith("#") and f[0] in SOURCES:
                table[(f[0], f[1])] = line.rstrip("\n")
    for prof in sorted(trace):
        if only and prof not in only:
            continue
        sha = _src_sha(SOURCES[prof])
        lines = ["# %s on %s (rocprofv3, one MI355X)" % (prof, wl), "",
                 "Kernel: %s" % names[prof],
                 "Source: %s under agent_q8_quant_amd/csrc (sha256 prefix %s)" % (", ".join(SOURCES[prof]), sha), "",
                 "## Kernel trace (durations, per launch grid)",
                 "Command (repository root):", "  " + args.trace_cmd]
        for g, d in sorted(trace[prof].items(), key=lambda kv: -len(kv[1])):
            sd = statistics.pstdev(d) if len(d) > 1 else 0.0
            lines.append("grid %s: calls %d, average %.2f us, median %.2f us, min %.2f us, max %.2f us, std %.2f us"
                         % (g, len(d), statistics.mean(d), statistics.median(d), min(d), max(d), sd))
        if prof in fetch and prof in write:
            # the grid launched most often in the counter runs is the workload-sized one
            gf = max(fetch[prof], key=lambda g: len(fetch[prof][g]))
            gw = max(write[prof], key=lambda g: len(write[prof][g]))
            fk, wk = statistics.mean(fetch[prof][gf]), statistics.mean(write[prof][gw])
            total = int(round(fk * 1024 * fscale + wk * 1024 * wscale))
            lines += ["", "## HBM traffic per dispatch (PMC, one counter per run; grid size %s)" % gf,
                      "Commands (repository root):", "  " + args.fetch_cmd, "  " + args.write_cmd,
                      "FETCH_SIZE %.0f KiB raw x %.4f = %.2f MB read   (%d dispatches)" % (fk, fscale, fk * 1024 * fscale / 1e6, len(fetch[prof][gf])),
                      "WRITE_SIZE %.0f KiB raw x %.4f = %.2f MB written (%d dispatches)" % (wk, wscale, wk * 1024 * wscale / 1e6, len(write[prof][gw])),
                      "Total HBM bytes per dispatch: %d" % total,
                      "Scales from hbm_counter_calibration_copy_1GiB.txt."]
            key = (prof, wl if prof != "attend_tail" else wl + "_tail%s" % args.tail_tokens)
            table[key] = "%s %s %s %d" % (key[0], key[1], sha, total)
        name = "%s_%s.txt" % (prof, wl)
        with open(os.path.join(prof_dir, name), "w") as f:
            f.write("\n".join(lines) + "\n")
        print("wrote profiles/%s" % name)
    with open(traffic_path, "w") as f:
        f.write("# kernel workload source_sha256_prefix hbm_bytes_per_dispatch (FETCH_SIZE+WRITE_SIZE, copy-calibrated)\n")
        for k in sorted(table):
            f.write(table[k] + "\n")
    print("wrote profiles/hbm_traffic.txt")


def summarize_sq(args):
    """profiles/sq_counters_<workload>.txt: per kernel, the mean per dispatch of every SQ
    counter found in the --sq-dirs runs (the grid launched most often), and the shares
    derived from them."""
    import statistics
    vals = {}
    for d in filter(None, args.sq_dirs.split(",")):
        per = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            prof = _kernel_of(r["Kernel_Name"])
            if not prof:
                continue
            key = (prof, r["Counter_Name"], r["Grid_Size"])
            per.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
            per[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
        grids = {}
        for (prof, cn, g), dv in per.items():
            grids.setdefault(prof, {}).setdefault(g, len(dv))
        for (prof, cn, g), dv in per.items():
            gbest = max(grids[prof], key=lambda x: grids[prof][x])
            if g == gbest:
                vals.setdefault(prof, {})[cn] = statistics.mean(dv.values())
    if not vals:
        raise SystemExit("no product kernels in --sq-dirs")
    counters = sorted({c for v in vals.values() for c in v})
    lines = ["# SQ counters per dispatch, %s shapes (rocprofv3, one MI355X)" % args.workload, "",
             "Commands (repository root), one pass each:"]
    lines += ["  " + c for c in args.sq_cmds.splitlines() if c.strip()]
    lines += ["", "Each kernel's figures are the mean over its dispatches of the launch grid it ran most",
              "often. GRBM_GUI_ACTIVE is summed over the 8 XCDs: cycles = GRBM_GUI_ACTIVE / 8.",
              "Derived: per-wave counts = SQ_INSTS_* / SQ_WAVES; VALU active = SQ_ACTIVE_INST_VALU x 4 /",
              "(1024 SIMDs x cycles), the wave-cycles spent in vector instructions per SIMD cycle (the",
              "counter runs per wave, so overlapping waves can take it past 100%); MFMA busy =",
              "SQ_VALU_MFMA_BUSY_CYCLES / (1024 x cycles); LDS bank-conflict share =",
              "SQ_LDS_BANK_CONFLICT / (SQ_ACTIVE_INST_LDS + SQ_LDS_BANK_CONFLICT).",
              "Source hashes: as in the kernel's own summary file of this workload.", ""]
    derived = ("VALU/wave", "MFMA/wave", "LDS/wave", "SALU/wave", "VALU active", "MFMA busy", "LDS conflict share")
    lines.append("| kernel | " + " | ".join(derived) + " |")
    lines.append("|---" * (len(derived) + 1) + "|")
    for prof in sorted(vals):
        v = vals[prof]
        cyc = v.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        waves = v.get("SQ_WAVES", 0.0)
        def per_wave(c):
            return "%.0f" % (v[c] / waves) if c in v and waves else "-"
        def share(x):
            return "%.0f%%" % (100.0 * x) if x is not None else "-"
        valu = v["SQ_ACTIVE_INST_VALU"] * 4 / (1024 * cyc) if "SQ_ACTIVE_INST_VALU" in v and cyc else None
        mfma = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * cyc) if "SQ_VALU_MFMA_BUSY_CYCLES" in v and cyc else None
        lds = None
        if "SQ_LDS_BANK_CONFLICT" in v and "SQ_ACTIVE_INST_LDS" in v and v["SQ_ACTIVE_INST_LDS"] + v["SQ_LDS_BANK_CONFLICT"] > 0:
            lds = v["SQ_LDS_BANK_CONFLICT"] / (v["SQ_ACTIVE_INST_LDS"] + v["SQ_LDS_BANK_CONFLICT"])
        lines.append("| %s | %s | %s | %s | %s | %s | %s | %s |" % (
            prof, per_wave("SQ_INSTS_VALU"), per_wave("SQ_INSTS_MFMA"), per_wave("SQ_INSTS_LDS"),
            per_wave("SQ_INSTS_SALU"), share(valu), share(mfma), share(lds)))
    lines += ["", "Raw means per dispatch:", "", "| kernel | " + " | ".join(counters) + " |",
              "|---" * (len(counters) + 1) + "|"]
    for prof in sorted(vals):
        lines.append("| %s | " % prof + " | ".join("%.0f" % vals[prof][c] if c in vals[prof] else "-"
                                                   for c in counters) + " |")
    name = "sq_counters_%s.txt" % args.workload
    with open(os.path.join(ROOT, "profiles", name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote profiles/%s" % name)


def cpu_baseline(cfg, n_layers_sample, n_steps_sample):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    from workloads import gen_k_layer, gen_q_step, gen_v_layer
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    c32, b32 = oracle.codebook_fp32()
    tc = td = ta = 0.0
    qs = [gen_q_step(cfg, s) for s in range(n_steps_sample)]
    for l in range(n_layers_sample):
        k, v = gen_k_layer(cfg, l), gen_v_layer(cfg, l)
        t = time.perf_counter()
        pool = oracle.compress_pool(k, v, b32)
        tc += time.perf_counter() - t
        t = time.perf_counter()
        kh, vh = oracle.dequant_pool(pool, c32)
        td += time.perf_counter() - t
        for q in qs:
            t = time.perf_counter()
            oracle.shared_pool_decode(q[l:l + 1], kh[None], vh[None], cfg.gqa, cfg.softmax_scale)
            ta += time.perf_counter() - t
    n, ns = n_layers_sample, n_steps_sample
    L, D = cfg.n_layers, cfg.decode_steps
    job = (tc + td) / n * L + ta / (n * ns) * L * D
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": cfg.n_agents * D / job, "unit": "agent-tokens/s",
            "cores": int(blas_threads), "kind": "oracle",
            "sample": "%d of %d layers, %d of %d decode steps: oracle compress + per-token dequant "
                      "of those layers, then those steps' attention; job time = L/n * (compress + "
                      "dequant) + L*D/(n*s) * attention" % (n, L, ns, D),
            "seconds_measured": round(tc + td + ta, 2),
            "compress_GBps": (cfg.kv_elems * 4 + _analytic(cfg)) / ((tc / n) * L) / 1e9,
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model,
            "host": platform.node()}


def _analytic(cfg):
    d = cfg.head_dim
    return cfg.n_layers * cfg.n_kv_heads * cfg.n_tokens * (d + 2 * (d // 32) + 3 * d // 8 + 2)


def main():
    args = _parse()
    if args.mode == "summarize":
        if args.trace_dir:
            summarize(args)
        if args.sq_dirs:
            summarize_sq(args)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(the pool would shard by KV head, with no collective between GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch
    import agent_q8_quant_amd as pk
    from workloads import config_by_name, gen_k_layer, gen_q_step, gen_v_layer

    if not os.path.exists(os.path.join(ROOT, "agent_q8_quant_amd", "libpolykv.so")):
        from agent_q8_quant_amd.build import build
        build()
    dev = torch.device("cuda", 0)

    if args.mode == "copy":
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("copy of 1 GiB done x3", flush=True)
        return

    cfg = config_by_name(args.config)
    D = args.decode_steps if args.decode_steps is not None else cfg.decode_steps
    path = {"auto": pk.POLYKV_PATH_AUTO, "valu": pk.POLYKV_PATH_VALU, "mfma": pk.POLYKV_PATH_MFMA}[args.path]
    lay = pk.polykv_pool_layout(cfg.n_layers, cfg.n_kv_heads, cfg.head_dim, cfg.n_tokens)

    print("bench: generating %s" % cfg.name, file=sys.stderr, flush=True)
    k = torch.empty((cfg.n_layers, cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim), dtype=torch.float16, device=dev)
    v = torch.empty_like(k)
    for l in range(cfg.n_layers):
        k[l].copy_(torch.from_numpy(gen_k_layer(cfg, l)))
        v[l].copy_(torch.from_numpy(gen_v_layer(cfg, l)))
    qshape = (cfg.n_layers, cfg.n_agents, cfg.n_q_heads, cfg.head_dim)
    q = torch.empty((D,) + qshape, dtype=torch.float32, device=dev)
    for s in range(D):
        q[s].copy_(torch.from_numpy(gen_q_step(cfg, s)))
    out = torch.empty(qshape, dtype=torch.float32, device=dev)
    ws_bytes = pk.polykv_attend_workspace_bytes(lay, cfg.n_agents, cfg.gqa)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    n_pools = 1 if args.warm else 3
    pools = [torch.zeros(lay.total_bytes, dtype=torch.uint8, device=dev) for _ in range(n_pools)]
    stream = torch.cuda.Stream(device=dev)
    # Private tails for the tail-merge figure: every agent's own fp16 K/V after n_tail
    # decode steps, [agent][layer][kv head][token][dim]; copies used in turn like the pools.
    n_tail = args.tail_tokens if args.tail_tokens is not None else D
    tail_shape = (cfg.n_agents, cfg.n_layers, cfg.n_kv_heads, n_tail, cfg.head_dim)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260427)
    tails = [(torch.randn(tail_shape, generator=gen, dtype=torch.float16, device=dev),
              torch.randn(tail_shape, generator=gen, dtype=torch.float16, device=dev))
             for _ in range(n_pools)] if n_tail > 0 else []
    tail_len = torch.full((cfg.n_agents,), n_tail, dtype=torch.int32, device=dev)
    lse = torch.empty((cfg.n_layers, cfg.n_agents, cfg.n_q_heads), dtype=torch.float32, device=dev)
    # Prefill chunks for the append figure: the same context cut into --chunk-tokens pieces
    chunk = max(1, min(args.chunk_tokens, cfg.n_tokens))
    cuts = list(range(0, cfg.n_tokens, chunk)) + [cfg.n_tokens]
    chunks = [(a, b, k[:, :, a:b, :].contiguous(), v[:, :, a:b, :].contiguous()) for a, b in zip(cuts[:-1], cuts[1:])]
    torch.cuda.synchronize()

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def decode(p, s):
        pk.polykv_attend_shared_path(pools[p], lay, q[s], out, cfg.n_agents, cfg.gqa,
                                     cfg.softmax_scale, path, workspace=ws, stream=stream)

    def one_step(j, rec):
        # The step compresses into pool j % n and decodes from the others in turn, so each
        # decode launch reads a pool that at least two pool-sized reads have passed since
        # (nothing of it is left in the 256 MB Infinity Cache); all copies are identical.
        pw = j % n_pools
        e = [ev()]
        pk.polykv_compress_kv(k, v, pools[pw], lay, stream=stream)
        e.append(ev())
        # the D decode launches back to back, one event pair around them: an event between
        # launches would add its own packet's time to every launch
        for s in range(D):
            decode((pw + 1 + s) % n_pools, s)
        e.append(ev())
        rec.append(e)

    stream2 = torch.cuda.Stream(device=dev)

    def append_all(i, fused=True, two_streams=False):
        # The whole context, chunk by chunk, into pool copy i (it ends up identical). Chunk
        # boundaries are multiples of 32 tokens, so consecutive chunks touch disjoint plane
        # groups and may run concurrently: with two_streams the odd chunks go to a second
        # stream, joined to the first before and after.
        if two_streams:
            e = torch.cuda.Event()
            e.record(stream)
            stream2.wait_event(e)
        for n, (a, b, kc, vc) in enumerate(chunks):
            st = stream2 if (two_streams and n % 2) else stream
            if fused:
                pk.polykv_append_kv(kc, vc, pools[i % n_pools], lay, a, stream=st)
            else:
                pk.polykv_append_k(kc, pools[i % n_pools], lay, a, stream=st)
                pk.polykv_append_v(vc, pools[i % n_pools], lay, a, stream=st)
        if two_streams:
            e = torch.cuda.Event()
            e.record(stream2)
            stream.wait_event(e)

    # Fused K/V projection + compression (prefill): one layer's input rows x [T][hidden] and
    # the two projection weights [H*d][hidden], seeded normals (random weights, as no
    # checkpoint is used); hidden = the model's width (query heads x head_dim).
    hidden = cfg.n_q_heads * cfg.head_dim
    proj = None
    if cfg.head_dim in (64, 128) and hidden % 64 == 0:
        px = torch.randn((cfg.n_tokens, hidden), generator=gen, device=dev).to(torch.float16)
        pwk = (torch.randn((cfg.n_kv_heads * cfg.head_dim, hidden), generator=gen, device=dev) / hidden ** 0.5).to(torch.float16)
        pwv = (torch.randn((cfg.n_kv_heads * cfg.head_dim, hidden), generator=gen, device=dev) / hidden ** 0.5).to(torch.float16)
        pk_tmp = torch.empty((cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim), dtype=torch.float16, device=dev)
        pv_tmp = torch.empty_like(pk_tmp)
        proj = (px, pwk, pwv, pk_tmp, pv_tmp)

    def project_fused(i):
        px, pwk, pwv, _, _ = proj
        for l in range(cfg.n_layers):
            pk.polykv_project_compress(px, pwk, pwv, pools[i % n_pools], lay, l, 0, stream=stream)

    def project_unfused(i):
        px, pwk, pwv, kt, vt = proj
        for l in range(cfg.n_layers):
            pk.polykv_project_kv(px, pwk, pwv, kt, vt, cfg.n_kv_heads, cfg.head_dim, stream=stream)
            pk.polykv_append_kv(kt, vt, pools[i % n_pools], lay, 0, layer_begin=l, layer_count=1, stream=stream)

    def dequant(i, which):
        # pool copy i -> fp16 K or V (into the compress inputs, which are not needed again)
        if which == "k":
            pk.polykv_dequant_k(pools[i % n_pools], lay, k, stream=stream)
        else:
            pk.polykv_dequant_v(pools[i % n_pools], lay, v, stream=stream)

    def tail_merge(i):
        tk, tv = tails[i % len(tails)]
        pk.polykv_attend_tail_merge(lay, q[0], out, lse, tk, tv, tail_len, cfg.n_agents, cfg.gqa,
                                    cfg.softmax_scale, stream=stream)

    with torch.cuda.stream(stream):
        if args.mode == "profile":
            for j in range(n_pools + max(1, args.steps)):
                one_step(j, [])
            if tails:
                pk.polykv_attend_shared_lse(pools[0], lay, q[0], out, lse, cfg.n_agents, cfg.gqa,
                                            cfg.softmax_scale, path, workspace=ws, stream=stream)
                for i in range(2 * n_pools):
                    tail_merge(i)
            # the single-kind compress kernels over the whole pool (appends run them on
            # smaller ranges: left out here, so that their statistics stay the one-shot ones)
            for i in range(n_pools + max(1, args.steps)):
                pk.polykv_compress_k(k, pools[i % n_pools], lay, stream=stream)
                pk.polykv_compress_v(v, pools[i % n_pools], lay, stream=stream)
            if proj is not None:
                project_fused(0)
                px, pwk, pwv, kt, vt = proj
                for l in range(cfg.n_layers):
                    pk.polykv_project_kv(px, pwk, pwv, kt, vt, cfg.n_kv_heads, cfg.head_dim, stream=stream)
            if cfg.head_dim in (64, 128):
                for i in range(2 * n_pools):
                    pk.polykv_compress_v(v, pools[i % n_pools], lay, stream=stream, path=pk.POLYKV_PATH_VALU)
            for i in range(2 * n_pools):
                dequant(i, "k")
                dequant(i, "v")
            stream.synchronize()
            print("profile run done: %d steps x (2 compress + %d decode) launches"
                  % (n_pools + args.steps, D), flush=True)
            return
        for j in range(max(args.warmup, n_pools)):  # every pool copy written before timing
            one_step(j, [])
        stream.synchronize()
        print("bench: warmup done, timing %d steps" % args.steps, file=sys.stderr, flush=True)
        rec = []
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for j in range(args.steps):
            one_step(j, rec)
        stream.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0

        # Secondary figure: one step's D decode launches captured in a HIP graph and replayed
        # (the same kernels and pools as the eager launches above, without host work per
        # launch; every kernel has run eagerly before the capture)
        graph_ev, graph_us, graph_err = [], None, None
        try:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                for s in range(D):
                    decode((1 + s) % n_pools, s)
            gr.replay()
            for _ in range(3):
                e0 = ev()
                gr.replay()
                e1 = ev()
                graph_ev.append((e0, e1))
            stream.synchronize()
            graph_us = sorted(a.elapsed_time(b) * 1e3 / D for a, b in graph_ev)[1]
            del gr
        except RuntimeError as exc:  # a secondary figure: report why it is missing
            stream.synchronize()
            graph_err = str(exc)[:200]

        # Secondary figures: single decode launches right after evicting the 256 MB Infinity
        # Cache with 1 GiB of other traffic, outside the events: a 1 GiB read (the pool then
        # comes from HBM), and a 1 GiB write (which also leaves that cache full of dirty
        # lines that the decode's reads force back to HBM).
        cold_us = {"read": [], "write": []}
        if not args.warm:
            flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
            flush32 = flush.view(torch.int32)
            sink = torch.zeros(1, dtype=torch.int64, device=dev)
            for s in range(8):
                kind = "read" if s % 2 == 0 else "write"
                if kind == "read":
                    sink += flush32.sum(dtype=torch.int64)
                else:
                    flush.add_(1)
                e0 = ev()
                decode(0, s % D)
                e1 = ev()
                cold_us[kind].append((e0, e1))
            stream.synchronize()
            cold_us = {k: [a.elapsed_time(b) * 1e3 for a, b in v] for k, v in cold_us.items()}
            del flush, flush32, sink

        # Secondary figure: the private-tail merge after the pool decode (lse exported).
        tail_ev = []
        if tails:
            pk.polykv_attend_shared_lse(pools[0], lay, q[0], out, lse, cfg.n_agents, cfg.gqa,
                                        cfg.softmax_scale, path, workspace=ws, stream=stream)
            for i in range(n_pools + 16):
                e0 = ev()
                tail_merge(i)
                e1 = ev()
                if i >= n_pools:
                    tail_ev.append((e0, e1))
            stream.synchronize()

        # Secondary figure: keys and values compressed by their own launches, one after the
        # other (the same pool bytes as the one-launch compress of the timed steps).
        sep_ev = []
        for i in range(n_pools + 6):
            e0 = ev()
            pk.polykv_compress_k(k, pools[i % n_pools], lay, stream=stream)
            e1 = ev()
            pk.polykv_compress_v(v, pools[i % n_pools], lay, stream=stream)
            e2 = ev()
            if i >= n_pools:
                sep_ev.append((e0, e1, e2))
        stream.synchronize()

        # Secondary figure: the value compress with the rotation on the vector ALU instead of
        # the matrix cores (the same pool bytes up to boundary codes), for the kernel choice.
        cvv_ev = []
        if cfg.head_dim in (64, 128):
            for i in range(n_pools + 6):
                e0 = ev()
                pk.polykv_compress_v(v, pools[i % n_pools], lay, stream=stream, path=pk.POLYKV_PATH_VALU)
                e1 = ev()
                if i >= n_pools:
                    cvv_ev.append((e0, e1))
            stream.synchronize()
            for i in range(n_pools):  # the pools hold the matrix-core compress again
                pk.polykv_compress_v(v, pools[i], lay, stream=stream)
            stream.synchronize()

        # Secondary figure: the same compression as prefill chunks appended one at a time:
        # keys and values of a chunk in one launch, the chunks alternating over two streams;
        # the same on one stream; and keys and values in two launches on one stream.
        app_ev = {"two": [], "one": [], "separate": []}
        for name, fused, two in (("two", True, True), ("one", True, False), ("separate", False, False)):
            for i in range(n_pools + 6):
                e0 = ev()
                append_all(i, fused, two)
                e1 = ev()
                if i >= n_pools:
                    app_ev[name].append((e0, e1))
        torch.cuda.synchronize()

        # Secondary figure: the K/V projection of every layer with the compression fused in,
        # against the projection written as fp16 and then appended by the one-launch key +
        # value append (the same pool bytes), and against the library GEMM alone.
        # The pools end up holding the projected cache; nothing after this reads them.
        pj_ev = {"fused": [], "unfused": [], "library": []}
        if proj is not None:
            px, pwk, pwv, _, _ = proj
            # [2 H d][hidden] row-major, as the kernel reads it: x W^T with W^T a transposed
            # view (the library's faster layout for this shape), one 2-D GEMM per layer
            w_kv = torch.cat([pwk, pwv])

            def project_library(i):
                for l in range(cfg.n_layers):
                    torch.matmul(px, w_kv.t())
            # the three in turn, three rounds, so that the chip's state (clock, temperature)
            # weighs on each alike
            runs = (("fused", project_fused), ("unfused", project_unfused), ("library", project_library))
            for _, fn in runs:
                fn(0)
            for i in range(3):
                for name, fn in runs:
                    e0 = ev()
                    fn(i)
                    e1 = ev()
                    pj_ev[name].append((e0, e1))
            stream.synchronize()

        # Secondary figure: dequantisation of a pool back to fp16 K and V. It runs last,
        # because it overwrites the compress inputs.
        dq_ev = {"k": [], "v": []}
        for which in ("k", "v"):
            for i in range(n_pools + 12):
                e0 = ev()
                dequant(i, which)
                e1 = ev()
                if i >= n_pools:
                    dq_ev[which].append((e0, e1))
        stream.synchronize()

        # Achievable-bandwidth reference: a plain device copy of one pool copy into another
        # buffer (read + write of the pool's bytes), the source rotating like the decode's
        cp_dst = torch.empty_like(pools[0])
        cp_ev = []
        with torch.cuda.stream(stream):
            for i in range(n_pools + 12):
                e0 = ev()
                cp_dst.copy_(pools[i % n_pools])
                e1 = ev()
                if i >= n_pools:
                    cp_ev.append((e0, e1))
        stream.synchronize()
        del cp_dst
        # and a plain read: a library reduction over one pool copy (as int64 words), the
        # source rotating the same way
        rd_ev = []
        with torch.cuda.stream(stream):
            for i in range(n_pools + 12):
                e0 = ev()
                pools[i % n_pools].view(torch.int64).sum()
                e1 = ev()
                if i >= n_pools:
                    rd_ev.append((e0, e1))
        stream.synchronize()

    step_ms = [r[0].elapsed_time(r[-1]) for r in rec]
    ckv_ms = [r[0].elapsed_time(r[1]) for r in rec]
    at_ms = [r[1].elapsed_time(r[2]) / D for r in rec]
    step_s = sum(step_ms) / len(step_ms) / 1e3
    t_ckv = sum(ckv_ms) / len(ckv_ms) / 1e3
    t_at = sum(at_ms) / len(at_ms) / 1e3
    t_ck = sum(a.elapsed_time(b) for a, b, _ in sep_ev) / len(sep_ev) / 1e3
    t_cv = sum(b.elapsed_time(c) for _, b, c in sep_ev) / len(sep_ev) / 1e3

    analytic = lay.analytic_bytes
    fp16_bytes = cfg.kv_elems * 2
    q_bytes = cfg.n_layers * cfg.n_agents * cfg.n_q_heads * cfg.head_dim * 4
    compress_bytes = 2 * fp16_bytes + analytic
    decode_bytes = analytic + 2 * q_bytes
    compress_gbps = compress_bytes / t_ckv / 1e9
    decode_gbps = decode_bytes / t_at / 1e9
    workload = cfg.name
    chosen = pk.polykv_attend_path(lay, cfg.n_agents, cfg.gqa) if path == pk.POLYKV_PATH_AUTO else path
    kname = "attend_mfma" if chosen == pk.POLYKV_PATH_MFMA else "attend_valu"
    traffic = _traffic(kname, workload)
    result = {
        "metric": METRIC,
        "value": cfg.n_agents * D / step_s,
        "unit": "agent-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8+u3 pool; fp32 accumulate" + (" (fp16 MFMA operands)" if chosen == pk.POLYKV_PATH_MFMA else ""),
        "data": "synthetic",
        "config": {"workload": workload, "layers": cfg.n_layers, "kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "tokens": cfg.n_tokens, "agents": cfg.n_agents,
                   "gqa": cfg.gqa, "decode_steps": D, "v_dist": cfg.v_dist,
                   "cache": ("warm: one pool copy" if args.warm else
                             "3 identical pool copies used in turn: each decode reads a copy that "
                             ">= 2 pool-sized reads have passed since (not in the Infinity Cache)"),
                   "path": kname},
        "roofline": {"kernel": kname, "bound": "hbm", "achieved": decode_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": decode_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": decode_bytes,
                     "avg_launch_us": t_at * 1e6},
        "decode_agent_tokens_per_s": cfg.n_agents / t_at,
        "decode_GBps": decode_gbps, "decode_frac_hbm": decode_gbps / HBM_PEAK_GBPS,
        "compress_GBps": compress_gbps, "compress_frac_hbm": compress_gbps / HBM_PEAK_GBPS,
        "compress_us": t_ckv * 1e6,
        "compress_kernel": "compress_kv (keys and values in one launch)",
        "compress_traffic": _traffic("compress_kv", workload),
        "compress_separate": {
            "us": {"k": t_ck * 1e6, "v": t_cv * 1e6},
            "GBps": {"k": (fp16_bytes + cfg.kv_elems + cfg.kv_elems // 16) / t_ck / 1e9,
                     "v": (fp16_bytes + cfg.kv_elems * 3 // 8
                           + cfg.n_layers * cfg.n_kv_heads * cfg.n_tokens * 2) / t_cv / 1e9},
            "GBps_both": compress_bytes / (t_ck + t_cv) / 1e9},
        "wall_ms_per_step": wall / args.steps * 1e3,
    }
    result["decode_graph"] = {"what": "one step's decode launches captured in a HIP graph, replayed (median of 3)",
                              "us_per_launch": graph_us}
    if graph_err:
        result["decode_graph"]["error"] = graph_err
    if cold_us["read"]:
        result["decode_us_after_1GiB_read"] = cold_us["read"]
        result["decode_us_after_1GiB_write"] = cold_us["write"]
    if tail_ev:
        t_tail = sum(a.elapsed_time(b) for a, b in tail_ev) / len(tail_ev) / 1e3
        # fp16 tail K and V, q read, out read + written, lse read + written
        lse_bytes = cfg.n_layers * cfg.n_agents * cfg.n_q_heads * 4
        tail_bytes = 2 * 2 * cfg.n_agents * cfg.n_layers * cfg.n_kv_heads * n_tail * cfg.head_dim \
            + 3 * q_bytes + 2 * lse_bytes
        result["tail_merge"] = {"kernel": "attend_tail", "tail_tokens_per_agent": n_tail,
                                "us": t_tail * 1e6, "GBps": tail_bytes / t_tail / 1e9,
                                "frac_hbm": tail_bytes / t_tail / 1e9 / HBM_PEAK_GBPS,
                                "algorithmic_bytes_per_launch": tail_bytes,
                                "traffic": _traffic("attend_tail", "%s_tail%d" % (workload, n_tail))}
    if cvv_ev:
        t_vv = sum(a.elapsed_time(b) for a, b in cvv_ev) / len(cvv_ev) / 1e3
        vbytes = fp16_bytes + cfg.kv_elems * 3 // 8 + cfg.n_layers * cfg.n_kv_heads * cfg.n_tokens * 2
        result["compress_v_vector_alu"] = {
            "kernel": "compress_v (rotation on the vector ALU)", "us": t_vv * 1e6,
            "GBps": vbytes / t_vv / 1e9, "frac_hbm": vbytes / t_vv / 1e9 / HBM_PEAK_GBPS,
            "vs_matrix_core_us": t_cv * 1e6}
    t_app = {n: sum(a.elapsed_time(b) for a, b in ev_) / len(ev_) / 1e3 for n, ev_ in app_ev.items()}
    result["append"] = {"kernels": ["compress_kv"], "chunk_tokens": chunk, "chunks": len(chunks),
                        "streams": 2, "us": t_app["two"] * 1e6,
                        "GBps": compress_bytes / t_app["two"] / 1e9,
                        "frac_hbm": compress_bytes / t_app["two"] / 1e9 / HBM_PEAK_GBPS,
                        "algorithmic_bytes": compress_bytes,
                        "one_stream": {"us": t_app["one"] * 1e6,
                                       "frac_hbm": compress_bytes / t_app["one"] / 1e9 / HBM_PEAK_GBPS},
                        "separate_launches_one_stream": {
                            "kernels": ["compress_k", "compress_v"], "us": t_app["separate"] * 1e6,
                            "frac_hbm": compress_bytes / t_app["separate"] / 1e9 / HBM_PEAK_GBPS}}
    if pj_ev["fused"]:
        def med_s(evs):  # median over the rounds, seconds
            t = sorted(a.elapsed_time(b) for a, b in evs)
            return t[len(t) // 2] / 1e3
        t_f = med_s(pj_ev["fused"])
        t_u = med_s(pj_ev["unfused"])
        flops = 2.0 * cfg.n_layers * cfg.n_tokens * hidden * 2 * cfg.n_kv_heads * cfg.head_dim
        result["project_compress"] = {
            "kernel": "project (fused)", "hidden": hidden, "layers": cfg.n_layers,
            "us_fused": t_f * 1e6, "us_unfused": t_u * 1e6,
            "us_library_gemm_only": med_s(pj_ev["library"]) * 1e6,
            "roofline": {"bound": "mfma", "achieved": flops / t_f / 1e12, "peak": 2500.0,
                         "unit": "TFLOP/s", "frac": flops / t_f / 1e12 / 2500.0},
            "flops": flops}
    t_dk = sum(a.elapsed_time(b) for a, b in dq_ev["k"]) / len(dq_ev["k"]) / 1e3
    t_dv = sum(a.elapsed_time(b) for a, b in dq_ev["v"]) / len(dq_ev["v"]) / 1e3
    # algorithmic bytes: the pool's K (or V) region read, fp16 K (or V) written
    dk_bytes = cfg.kv_elems + cfg.kv_elems // 16 + fp16_bytes
    dv_bytes = cfg.kv_elems * 3 // 8 + cfg.n_layers * cfg.n_kv_heads * cfg.n_tokens * 2 + fp16_bytes
    result["dequant"] = {
        "kernels": ["dequant_k", "dequant_v"], "us": {"k": t_dk * 1e6, "v": t_dv * 1e6},
        "GBps": {"k": dk_bytes / t_dk / 1e9, "v": dv_bytes / t_dv / 1e9},
        "frac_hbm": {"k": dk_bytes / t_dk / 1e9 / HBM_PEAK_GBPS, "v": dv_bytes / t_dv / 1e9 / HBM_PEAK_GBPS},
        "algorithmic_bytes_per_launch": {"k": dk_bytes, "v": dv_bytes},
        "traffic": {"k": _traffic("dequant_k", workload), "v": _traffic("dequant_v", workload)}}
    t_cp = sum(a.elapsed_time(b) for a, b in cp_ev) / len(cp_ev) / 1e3
    result["device_copy_reference"] = {
        "what": "torch copy of one pool copy (read + write), sources rotating like the decode",
        "bytes": 2 * lay.total_bytes, "us": t_cp * 1e6, "GBps": 2 * lay.total_bytes / t_cp / 1e9,
        "frac_hbm": 2 * lay.total_bytes / t_cp / 1e9 / HBM_PEAK_GBPS}
    t_rd = sum(a.elapsed_time(b) for a, b in rd_ev) / len(rd_ev) / 1e3
    result["device_read_reference"] = {
        "what": "torch int64 sum over one pool copy (read only), sources rotating like the decode",
        "bytes": lay.total_bytes, "us": t_rd * 1e6, "GBps": lay.total_bytes / t_rd / 1e9,
        "frac_hbm": lay.total_bytes / t_rd / 1e9 / HBM_PEAK_GBPS}
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        n = args.cpu_sample_layers or cfg.n_layers
        result["cpu_baseline"] = cpu_baseline(cfg, n, max(1, min(D, 32)))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
