#!/usr/bin/env python3
"""SSA forward throughput on one MI355X.

One step = the whole hot path over one batch of synthetic input: the block
build (keys, stable radix sort, segments) followed by the forward pass
(pooling, compressed attention with top-k, selected-block attention, window
attention, gated sum).  Inputs are resident in HBM before timing starts.

Workload: 131072 surface-band voxel tokens of a seeded union of 12 primitives
on a 1024^3 grid; 16 query / 16 key-value heads, head dim 64, bfloat16;
m_cmp = 4, m_win = 8, top-k = 16 (the 128k-token setting of the Direct3D-S2
summary page, "Experiments").  ``--workload 4`` times the grouped-head
workload instead (262144 tokens, 32 query / 2 key-value heads, head dim 32),
for its kernel profile; ``--workload 5`` times a training step (block build,
forward that saves its log-sum-exps, backward giving dq, dk, dv and the gate
gradients for a seeded output gradient) on the varlen batch of 8 sequences.

Prints one JSON line (rank 0, N = 1 only).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# the timed workload (default) and the grouped-head workload, which
# ``--workload 4`` times for its kernel profile
WORKLOADS = {
    3: dict(name="ssa-fwd-1024^3-12prims-131072tok-h16-d64-bf16", tag="131072tok",
            metric="SSA fwd tokens/s and TFLOP/s at 131072 voxel tokens; % bf16 MFMA peak"),
    4: dict(name="ssa-fwd-1024^3-16prims-262144tok-h32kv2-d32-bf16", tag="262144tok",
            metric="SSA fwd tokens/s and TFLOP/s at 262144 voxel tokens, 32 query / 2 key-value heads; "
                   "% bf16 MFMA peak"),
    5: dict(name="ssa-fwd+bwd-varlen-8seq-469315tok-h16-d64-bf16", tag="varlen",
            metric="SSA fwd+bwd (dq, dk, dv, dgates given dout) tokens/s and TFLOP/s on the varlen batch of "
                   "8 sequences; % bf16 MFMA peak"),
}
TRAIN_WORKLOADS = (5,)
WORKLOAD_ID = 3
CALIB_BYTES = 1 << 30       # plain-copy calibration size for the HBM byte counters
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "spatial_sparse_attention_ssa_amd", "csrc")
# the source file of each timed kernel (with the shared header, its content
# hash tells whether stored counter readings still describe the kernel)
KERNEL_SOURCES = {
    "cmp_mfma_kernel": "ssa_attn_cmp.hip",
    "topk_fixup_kernel": "ssa_attn_cmp.hip",
    "probe_select_kernel": "ssa_attn_cmp.hip",
    "win_mfma_kernel": "ssa_attn_win.hip",
    "sel_combine_kernel": "ssa_attn_sel.hip",
    "sel_group_kernel": "ssa_attn_sel.hip",
    "pool_kernel": "ssa_pool.hip",
    "gqa_cmp_kernel": "ssa_attn_gqa.hip",
    "gqa_topk_kernel": "ssa_attn_gqa.hip",
    "gqa_seq_kmax_kernel": "ssa_attn_gqa.hip",
    "cmp_dq_mfma_kernel": "ssa_bwd_mfma.hip",
    "cmp_dkv_mfma_kernel": "ssa_bwd_mfma.hip",
    "kv_grad_mfma_kernel": "ssa_bwd_mfma.hip",
    "win_dq_mfma_kernel": "ssa_bwd_mfma.hip",
    "win_dkv_mfma_kernel": "ssa_bwd_mfma.hip",
    "rows_prep_kernel": "ssa_bwd_mfma.hip",
}


def kernel_source_hash(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "ssa_internal.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_path(kernel: str, wid: int = WORKLOAD_ID) -> str:
    return os.path.join(PROFILES, f"{kernel}_{WORKLOADS[wid]['tag']}_traffic.json")


def stored_traffic(kernel: str, wid: int = WORKLOAD_ID):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or the kernel's source changed since."""
    path = traffic_path(kernel, wid)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return rec.get("traffic_bytes")


def mfma_path(kernel: str, wid: int = WORKLOAD_ID) -> str:
    return os.path.join(PROFILES, f"{kernel}_{WORKLOADS[wid]['tag']}_mfma.json")


def stored_mfma(kernel: str, wid: int = WORKLOAD_ID):
    """MFMA counter figures of `kernel` from the committed summary (busy share
    of SIMD cycles, executed bf16 MFMA TFLOP per launch, implied clock), or
    None when there is none or the kernel's source changed since."""
    path = mfma_path(kernel, wid)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return {k: rec[k] for k in ("mfma_busy_frac", "executed_tflop", "executed_tflops", "clock_ghz", "launches")}


def pool_bytes(wl, nb: int) -> float:
    """Algorithmic HBM bytes of the pooling kernel: every token's K and V row
    read once (gathered through perm, 4 B per token), pooled rows written."""
    row = wl.h_kv * wl.head_dim * 2
    return wl.n_tokens * (2 * row + 4) + 2 * nb * row


def summarize_counters(fetch_csv: str, write_csv: str, stats_csv: str | None, commands: dict, wid: int):
    """Turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (each with
    --copy-calibration) into per-kernel HBM bytes per launch; writes
    profiles/<kernel>_<tokens>tok_traffic.json and prints a markdown table."""
    import csv
    from collections import defaultdict

    def load(path, counter):
        per = defaultdict(list)
        copy_vals = []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                name, val = r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0
                if "copyBuffer" in name:
                    copy_vals.append(val)
                for k in KERNEL_SOURCES:
                    if f"::{k}" in name or f" {k}" in name or name.startswith(k):
                        per[k].append(val)
        return per, max(copy_vals)

    fetch, copy_f = load(fetch_csv, "FETCH_SIZE")
    write, copy_w = load(write_csv, "WRITE_SIZE")
    ff, fw = CALIB_BYTES / copy_f, CALIB_BYTES / copy_w
    avg_ns = {}
    if stats_csv:
        with open(stats_csv) as fh:
            for r in csv.DictReader(fh):
                for k in KERNEL_SOURCES:
                    if f"::{k}" in r["Name"]:
                        avg_ns[k] = float(r["AverageNs"])
    print(f"calibration: 1 GiB copy read {copy_f / 2**20:.1f} MiB by FETCH_SIZE (x{ff:.3f}), "
          f"wrote {copy_w / 2**20:.1f} MiB by WRITE_SIZE (x{fw:.3f})")
    print("| kernel | FETCH MB/launch (scaled) | WRITE MB/launch (scaled) | HBM MB/launch | avg us | GB/s |")
    print("|---|---|---|---|---|---|")
    for k in KERNEL_SOURCES:
        if k not in fetch or k not in write:
            continue
        fb = sum(fetch[k]) / len(fetch[k]) * ff
        wb = sum(write[k]) / len(write[k]) * fw
        us = avg_ns.get(k, float("nan")) / 1e3
        print(f"| {k} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} | {us:.1f} | {(fb + wb) / (us * 1e3):.0f} |")
        rec = {"kernel": k, "workload": WORKLOADS[wid]["name"], "source_sha256": kernel_source_hash(k),
               "fetch_bytes": fb, "write_bytes": wb, "traffic_bytes": fb + wb,
               "fetch_factor": ff, "write_factor": fw, "launches": len(fetch[k]), "commands": commands}
        with open(traffic_path(k, wid), "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")


def algorithmic_flops(wl, blocks, topk, torch):
    """Sum over (token, head) of 4 * D * (blocks in its sequence + tokens in its
    selected blocks + tokens in its window), with the actual sizes."""
    dev = blocks.perm.device
    h = blocks.trimmed()
    blk_off = h["blk_off"].to(dev).long()
    win_off = h["win_off"].to(dev).long()
    seq_blk_off = h["seq_blk_off"].to(dev).long()
    n = wl.n_tokens
    cu = torch.as_tensor(wl.cu_seqlens, device=dev).long()
    seq_of_tok = torch.bucketize(torch.arange(n, device=dev), cu[1:], right=True)
    nb_seq = (seq_blk_off[1:] - seq_blk_off[:-1])[seq_of_tok].double()          # [N]
    win_size = (win_off[1:] - win_off[:-1])
    win_sizes_sorted = torch.repeat_interleave(win_size, win_size)
    n_win = torch.empty(n, dtype=torch.long, device=dev)
    n_win[blocks.perm.long()] = win_sizes_sorted
    blk_size = blk_off[1:] - blk_off[:-1]
    sel = topk.long()                                                           # [N, Hkv, k]
    n_sel = torch.where(sel >= 0, blk_size[sel.clamp(min=0)], torch.zeros_like(sel)).sum(-1)  # [N, Hkv]
    G = wl.h_q // wl.h_kv
    D = wl.head_dim
    f_cmp = 4.0 * D * wl.h_q * nb_seq.sum().item()
    f_sel = 4.0 * D * G * n_sel.double().sum().item()
    f_win = 4.0 * D * wl.h_q * n_win.double().sum().item()
    return dict(cmp=f_cmp, sel=f_sel, win=f_win, total=f_cmp + f_sel + f_win,
                mean_sel_tokens=n_sel.double().mean().item(), mean_win_tokens=n_win.double().mean().item(),
                nb=int(h["counts"][0]), nw=int(h["counts"][1]))


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES",
                 "GRBM_GUI_ACTIVE")
N_SIMD = 256 * 4            # MI355X: 256 compute units of 4 SIMDs
N_XCC = 8


def summarize_mfma(pmc_csv: str, wid: int, command: str = ""):
    """Counter-based MFMA utilisation per attention kernel from one rocprofv3
    --pmc run of MFMA_COUNTERS: executed bf16 MFMA flops (512 per MOPS unit),
    the MFMA pipe's busy share of all SIMD cycles (cycles per XCC from
    GRBM_GUI_ACTIVE), and the clock those cycles imply; prints a markdown
    table and the time-weighted utilisation, and writes
    profiles/<kernel>_<tokens>tok_mfma.json for the kernels it knows."""
    import csv
    import re
    from collections import defaultdict

    per = defaultdict(lambda: defaultdict(list))
    dur = defaultdict(list)
    with open(pmc_csv) as fh:
        for r in csv.DictReader(fh):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
            name = re.sub(r"[<(].*", "", name).split("::")[-1]
            per[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                dur[name].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    print("| kernel | launches | avg us | executed MFMA TFLOP | executed TFLOP/s | % of 2.5 PF | "
          "MFMA busy % of SIMD cycles | implied clock GHz |")
    print("|---|---|---|---|---|---|---|---|")
    tw_busy, tw_t = 0.0, 0.0
    for name, c in per.items():
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [])
        if not mops or max(mops) == 0:
            continue
        avg = lambda k: sum(c[k]) / len(c[k])
        t = sum(dur[name]) / len(dur[name])
        flops = 512.0 * avg("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        cycles = avg("GRBM_GUI_ACTIVE") / N_XCC
        busy = avg("SQ_VALU_MFMA_BUSY_CYCLES") / (cycles * N_SIMD)
        tw_busy += busy * t
        tw_t += t
        print(f"| {name} | {len(c['GRBM_GUI_ACTIVE'])} | {t * 1e6:.1f} | {flops / 1e12:.3f} | "
              f"{flops / t / 1e12:.0f} | {100 * flops / t / 1e12 / PEAK_BF16_TFLOPS:.1f} | {100 * busy:.1f} | "
              f"{cycles / t / 1e9:.2f} |")
        if name in KERNEL_SOURCES:
            rec = {"kernel": name, "workload": WORKLOADS[wid]["name"], "source_sha256": kernel_source_hash(name),
                   "mfma_busy_frac": busy, "executed_tflop": flops / 1e12, "executed_tflops": flops / t / 1e12,
                   "clock_ghz": cycles / t / 1e9, "launches": len(c["GRBM_GUI_ACTIVE"]),
                   "counters": list(MFMA_COUNTERS), "command": command}
            with open(mfma_path(name, wid), "w") as fh:
                json.dump(rec, fh, indent=1)
                fh.write("\n")
    if tw_t:
        print(f"\ntime-weighted MFMA busy share over these kernels: {100 * tw_busy / tw_t:.1f} %")


MEMPATH_COUNTERS = ("TA_TA_BUSY", "TA_DATA_STALLED_BY_TC_CYCLES", "TCP_TCC_READ_REQ", "TCP_TOTAL_CACHE_ACCESSES",
                    "TCP_PENDING_STALL_CYCLES", "TCP_TCC_READ_REQ_LATENCY", "TCC_HIT", "TCC_MISS", "GRBM_GUI_ACTIVE",
                    "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VMEM", "SQ_INSTS_VMEM_RD")
N_CU = 256


def summarize_mempath(pmc_csv: str, grid: int = 0):
    """Memory-path counters per SSA kernel from one rocprofv3 --pmc run of
    MEMPATH_COUNTERS: the texture addresser's busy share and its share stalled
    by the cache (both over cycles x 256 compute units), the L2 hit rate, the
    mean L1-to-L2 read latency in cycles, the L1's pending-request stall share,
    and vector-memory read instructions per launch; prints a markdown table.
    With `grid`, only the launches of that many threads are counted (one
    size of a sweep)."""
    import csv
    import re
    from collections import defaultdict

    per = defaultdict(lambda: defaultdict(list))
    dur = defaultdict(list)
    with open(pmc_csv) as fh:
        for r in csv.DictReader(fh):
            m = re.search(r"ssa::\(anonymous namespace\)::(\w+)", r["Kernel_Name"])
            if not m or (grid and int(r["Grid_Size"]) != grid):
                continue
            per[m.group(1)][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                dur[m.group(1)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    print("| kernel | launches | avg us | TA busy % | TA stalled by cache % | L2 hit % | L2 read latency (cycles) | "
          "L1 pending-stall % | VMEM read insts |")
    print("|---|---|---|---|---|---|---|---|---|")
    for name, c in per.items():
        avg = lambda k: sum(c[k]) / len(c[k])
        t = sum(dur[name]) / len(dur[name])
        if not grid and t < 50e-6:
            continue
        cu_cycles = avg("GRBM_GUI_ACTIVE") / N_XCC * N_CU
        hits, miss = avg("TCC_HIT"), avg("TCC_MISS")
        req = avg("TCP_TCC_READ_REQ")
        lat = avg("TCP_TCC_READ_REQ_LATENCY") / req if req else 0.0
        print(f"| {name} | {len(c['GRBM_GUI_ACTIVE'])} | {t * 1e6:.1f} | {100 * avg('TA_TA_BUSY') / cu_cycles:.0f} | "
              f"{100 * avg('TA_DATA_STALLED_BY_TC_CYCLES') / cu_cycles:.0f} | {100 * hits / max(hits + miss, 1):.0f} | "
              f"{lat:.0f} | {100 * avg('TCP_PENDING_STALL_CYCLES') / cu_cycles:.0f} | {avg('SQ_INSTS_VMEM_RD'):.3g} |")


def build_bytes(n: int, nb: int, nw: int, batch: int) -> float:
    """Algorithmic HBM bytes of the block build: coordinates read (12 B per
    token), the permutation written (4 B per token), the segment offsets and
    the sequence offsets."""
    return 16.0 * n + 4.0 * (nb + nw + 2) + 8.0 * (batch + 1)


def build_sweep(torch, ssa, dev, reps: int = 20):
    """Block build time against the token count, 2^17 .. 2^24 tokens of
    uniformly random voxels of a 1024^3 grid (one sequence; duplicates are
    legal tokens), m_cmp = 4, m_win = 8: the build's HBM fraction shows only
    at sizes far above one shape's 131072 tokens."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(17)
    points = []
    for lg in range(17, 25):
        n = 1 << lg
        coords = torch.randint(0, 1024, (n, 3), generator=gen, device=dev, dtype=torch.int32)
        cu = torch.tensor([0, n], dtype=torch.int32, device=dev)
        b = ssa.build_blocks(coords, cu, 1024, 4, 8, sync=True)
        nb, nw = int(b.struct.nb), int(b.struct.nw)
        geo = ssa._binding.SsaGeometry(1024, 4, 8, 0)
        ws_bytes = int(ssa._binding.lib().ssa_build_blocks_workspace(n, 1, ctypes.byref(geo)))
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        for _ in range(3):
            ssa.build_blocks(coords, cu, 1024, 4, 8, sync=False, workspace=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            ssa.build_blocks(coords, cu, 1024, 4, 8, sync=False, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        by = build_bytes(n, nb, nw, 1)
        gbs = by / (us * 1e-6) / 1e9
        points.append({"n_tokens": n, "nb": nb, "nw": nw, "us": us, "algorithmic_bytes": by, "GB/s": gbs,
                       "hbm_frac": gbs / PEAK_HBM_GBS})
        print(f"[build sweep] N=2^{lg}: {us:.1f} us, {gbs:.0f} GB/s", file=sys.stderr, flush=True)
        del coords, b, ws
    return points


def host_description() -> dict:
    """CPU model, numpy version and BLAS build of this host (for the baseline)."""
    import numpy as np
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info() if i.get("user_api") == "blas"]
        blas = ", ".join(libs) or blas
    except Exception:
        pass
    return {"cpu_model": model, "numpy": np.__version__, "blas": blas}


CPU_ROW_STRIDE = 16   # the oracle runs every 16th token (all heads) of the workload


def cpu_baseline(wl, train: bool = False):
    """Time the float64 oracle (test infrastructure) on the host's cores: the
    block build and pooling once in this process, then every head of every
    CPU_ROW_STRIDE-th token (input order) over one worker process per core,
    one BLAS thread each (with ``train`` also those rows' backward).  The
    step time is stated as build + pooling + CPU_ROW_STRIDE x the sampled
    rows' time, since the rows are independent and equally distributed."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from oracle import parallel
    workers = parallel.default_workers()
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        ob = oracle.build_blocks(wl.coords, wl.cu_seqlens, wl.grid_res, wl.m_cmp, wl.m_win)
        kbar = oracle.pool_blocks(wl.k, ob, wl.dtype)
        vbar = oracle.pool_blocks(wl.v, ob, wl.dtype)
        t_fixed = time.perf_counter() - t0
    toks = range(0, wl.n_tokens, CPU_ROW_STRIDE)
    rows = [(t, h) for t in toks for h in range(wl.h_q)]
    tf = {}
    parallel.forward_rows(wl, ob, rows, kbar=kbar, vbar=vbar, workers=workers, timing=tf)
    t_rows = tf["rows_s"]
    if train:
        dout = np.ones(wl.q.shape, np.float32)
        tb = {}
        parallel.backward_rows(wl, dout, ob, rows, workers=workers, timing=tb)
        t_rows += tb["rows_s"]
    t_step = t_fixed + CPU_ROW_STRIDE * t_rows
    what = "forward + backward" if train else "forward"
    return {
        "value": wl.n_tokens / t_step,
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"float64 numpy oracle over {workers} worker processes (one BLAS thread each): block build + "
                   f"pooling of all {wl.n_tokens} tokens once ({t_fixed:.1f} s, one process), then the {what} of "
                   f"all {wl.h_q} heads of every {CPU_ROW_STRIDE}th token, {len(rows)} (token, head) rows, timed "
                   f"in full ({t_rows:.1f} s); step time = build + pooling + {CPU_ROW_STRIDE} x rows = "
                   f"{t_step:.0f} s"),
        "host": host_description(),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="only summarise two rocprofv3 --pmc runs into profiles/*_traffic.json")
    ap.add_argument("--kernel-stats", help="rocprofv3 --stats kernel_stats.csv for the summary")
    ap.add_argument("--summarize-mempath", metavar="PMC_CSV",
                    help="print the memory-path counter table of one rocprofv3 --pmc run of MEMPATH_COUNTERS")
    ap.add_argument("--mempath-grid", type=int, default=0,
                    help="with --summarize-mempath: only launches of this many threads")
    ap.add_argument("--summarize-mfma", metavar="PMC_CSV",
                    help="only summarise a rocprofv3 --pmc run of the MFMA counters into a markdown table")
    ap.add_argument("--build-sweep", action="store_true",
                    help="only time the block build at 2^17 .. 2^24 random voxel tokens (one JSON line)")
    ap.add_argument("--workload", type=int, default=WORKLOAD_ID, choices=sorted(WORKLOADS),
                    help="3: the 131072-token workload (default); 4: the grouped-head 262144-token "
                         "workload, for its kernel profile; 5: forward + backward on the varlen batch")
    args = ap.parse_args()
    wid = args.workload
    if args.summarize_counters:
        extra = "" if wid == WORKLOAD_ID else f" --workload {wid}"
        cmds = {c.lower(): f"rocprofv3 --pmc {c} --output-format csv -d <dir> -o run -- python bench.py "
                           f"--steps 1 --warmup 1 --no-cpu-baseline --copy-calibration{extra}"
                for c in ("FETCH_SIZE", "WRITE_SIZE")}
        cmds = {"fetch": cmds["fetch_size"], "write": cmds["write_size"]}
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.kernel_stats, cmds, wid)
        return
    if args.summarize_mempath:
        summarize_mempath(args.summarize_mempath, args.mempath_grid)
        return
    if args.summarize_mfma:
        extra = "" if wid == WORKLOAD_ID else f" --workload {wid}"
        summarize_mfma(args.summarize_mfma, wid,
                       f"rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} --output-format csv -d <dir> -o run -- "
                       f"python bench.py --steps 1 --warmup 1 --no-cpu-baseline{extra}")
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import spatial_sparse_attention_ssa_amd as ssa
    from workloads import make_workload

    dev = torch.device("cuda:0")
    if args.build_sweep:
        pts = build_sweep(torch, ssa, dev)
        print(json.dumps({"metric": "block build time and algorithmic HBM GB/s against the token count",
                          "unit": "us", "higher_is_better": False, "data": "synthetic",
                          "config": {"workload": "uniform random voxels of a 1024^3 grid, one sequence",
                                     "m_cmp": 4, "m_win": 8},
                          "points": pts}), flush=True)
        return
    wl = make_workload(wid)
    bf = torch.bfloat16
    up = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    coords, cu = up(wl.coords, torch.int32), up(wl.cu_seqlens, torch.int32)
    q, k, v, gates = up(wl.q, bf), up(wl.k, bf), up(wl.v, bf), up(wl.gates, bf)

    # reference run for the work counts (untimed)
    blocks0 = ssa.build_blocks(coords, cu, wl.grid_res, wl.m_cmp, wl.m_win, sync=True)
    res0 = ssa.forward(blocks0, q, k, v, gates, wl.topk, return_topk=True)
    torch.cuda.synchronize()
    work = algorithmic_flops(wl, blocks0, res0["topk"], torch)

    # buffers for the timed loop: async build (nb unknown on the host)
    blocks_async = ssa.build_blocks(coords, cu, wl.grid_res, wl.m_cmp, wl.m_win, sync=False)
    ws_fwd = torch.empty(ssa.forward_workspace_bytes(blocks_async, q, k, wl.topk), dtype=torch.uint8,
                         device=dev)
    out = torch.empty_like(q)

    train = wid in TRAIN_WORKLOADS
    if train:
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 * wid + 4)
        dout = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32).to(bf)
        ws_bwd = torch.empty(ssa.backward_workspace_bytes(blocks0, q, k, wl.topk), dtype=torch.uint8, device=dev)

    def step():
        if not train:
            b = ssa.build_blocks(coords, cu, wl.grid_res, wl.m_cmp, wl.m_win, sync=False)
            ssa.forward(b, q, k, v, gates, wl.topk, out=out, workspace=ws_fwd)
            return
        # the backward's workspace is sized from the block count, so the
        # training step builds with the counts synced
        b = ssa.build_blocks(coords, cu, wl.grid_res, wl.m_cmp, wl.m_win, sync=True)
        saved = ssa.forward_train(b, q, k, v, gates, wl.topk, workspace=ws_fwd)
        ssa.backward(b, q, k, v, gates, saved, dout, workspace=ws_bwd)

    if args.copy_calibration:
        # a plain copy of known size whose source is not cache-resident: its
        # FETCH_SIZE / WRITE_SIZE counter readings calibrate the same counters
        # of the SSA kernels
        src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device=dev)
        evict = torch.ones(CALIB_BYTES, dtype=torch.uint8, device=dev)   # pushes src out of the caches
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, evict, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step (event), wall {wall_ms / args.steps:.3f} ms/step",
          file=sys.stderr, flush=True)

    # per-kernel times: HIP events recorded by the library around each kernel
    # it launches on this stream (same kernels, same workspace)
    stage_sum = {}
    reps = max(3, min(args.steps, 10))
    for _ in range(reps):
        st = {}
        b = ssa.build_blocks(coords, cu, wl.grid_res, wl.m_cmp, wl.m_win, sync=False)
        ssa.forward(b, q, k, v, gates, wl.topk, out=out, workspace=ws_fwd, stage_times=st)
        if train:
            saved = ssa.forward_train(blocks0, q, k, v, gates, wl.topk, workspace=ws_fwd)
            bst = {}
            ssa.backward(blocks0, q, k, v, gates, saved, dout, workspace=ws_bwd, stage_times=bst)
            st.update({"bwd:" + name: ms for name, ms in bst.items()})
        for name, ms in st.items():
            stage_sum[name] = stage_sum.get(name, 0.0) + ms
    stage_ms = {name: ms / reps for name, ms in stage_sum.items()}
    # block build alone
    eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    eb0.record()
    for _ in range(reps):
        ssa.build_blocks(coords, cu, wl.grid_res, wl.m_cmp, wl.m_win, sync=False)
    eb1.record()
    torch.cuda.synchronize()
    build_ms = eb0.elapsed_time(eb1) / reps

    n = wl.n_tokens
    if not train:
        # roofline of the compressed-attention kernel, which does the
        # compressed branch's algorithmic flops (the largest kernel)
        dom = "gqa_cmp_kernel" if "gqa_cmp_kernel" in stage_ms else "cmp_mfma_kernel"
        achieved = work["cmp"] / (stage_ms[dom] * 1e-3) / 1e12
        total_flops = work["total"]
    else:
        # backward algorithmic work: per (query head, key) pair of every branch
        # 8 D flops (dP = dO V^T, dq = dS K, dk = dS^T q, dv = P^T dO); the
        # pooled-row gradient kernel does the compressed branch's dk and dv
        # part, 4 D per pair (its recomputed S and dP are not counted)
        dom = "bwd:cmp_dkv_mfma_kernel"
        achieved = work["cmp"] / (stage_ms[dom] * 1e-3) / 1e12
        total_flops = 3.0 * work["total"]
    tflops = total_flops / (ms_step * 1e-3) / 1e12
    pool_gbs = pool_bytes(wl, work["nb"]) / (stage_ms["pool_kernel"] * 1e-3) / 1e9
    bp_bytes = build_bytes(n, work["nb"], work["nw"], wl.batch) + pool_bytes(wl, work["nb"])
    bp_gbs = bp_bytes / ((build_ms + stage_ms["pool_kernel"]) * 1e-3) / 1e9

    line = {
        "metric": WORKLOADS[wid]["metric"],
        "value": n / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[wid]["name"], "n_tokens": n,
                   "grid_res": wl.grid_res, "h_q": wl.h_q, "h_kv": wl.h_kv, "head_dim": wl.head_dim,
                   "m_cmp": wl.m_cmp, "m_win": wl.m_win, "topk": wl.topk, "parallelism": "none"},
        "tflops": tflops,
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "algorithmic_tflop_per_step": total_flops / 1e12,
        "work": {k2: work[k2] for k2 in ("cmp", "sel", "win", "mean_sel_tokens", "mean_win_tokens", "nb", "nw")},
        "build_ms": build_ms,
        "stage_ms": stage_ms,
        "pool_hbm": {"achieved": pool_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": pool_gbs / PEAK_HBM_GBS,
                     "bytes": pool_bytes(wl, work["nb"])},
        "build_pool_hbm": {"achieved": bp_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": bp_gbs / PEAK_HBM_GBS,
                           "bytes": bp_bytes},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": stored_traffic(dom.split(":")[-1], wid),
                     # the same kernel's rocprofv3 MFMA counters (SQ_VALU_MFMA_BUSY_CYCLES, ...) from the
                     # committed summary, while its source is unchanged
                     "mfma_counters": stored_mfma(dom.split(":")[-1], wid)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, train=train)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
