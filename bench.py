"""Benchmark: 131,072-token 1B-shape ARMT forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1b_s128]
    python bench.py --all-workloads      # diag + seq on every benchmark workload
    python bench.py --group-sweep        # grouped kernels vs wave width k
    python bench.py --logit-drift        # LM-head logits: diag vs seq vs oracle per segment count
    python bench.py --full-attention     # full-attention Llama comparator vs diagonal ARMT, 4K..131K
    python bench.py --batch-sweep        # B independent sequences per node, B = 1..8
    python bench.py --backward           # grouped vs node-by-node backward (fp32; 1B shape in bf16)

A step is one full forward of the workload (all S + L - 1 diagonal waves, every
kernel of every node) over a synthetic sequence that is resident in HBM before
timing starts.  The headline value is tokens/s of the diagonal schedule
(input tokens S*T per forward), over K forwards bracketed by synchronisations.
The same number of sequential-schedule forwards is timed next for the
diagonal-vs-sequential ratio the pages quote (abstract on the paper page: 1.8x
at 131,072 tokens, another GPU).  Each forward is also timed alone with HIP
events on the library's stream, for the median and the minimum.

Extra fields:
  roofline      the grouped gate/up GEMM (the largest kernel, about half of all
                FLOPs): algorithmic FLOPs of its launches divided by their
                summed durations, from HIP events recorded around every launch
                on the library's stream during a timed pass, against the bf16
                dense MFMA peak of 2.5 PFLOP/s; traffic = HBM bytes per launch
                from the committed FETCH_SIZE / WRITE_SIZE counters
                (profiles/pmc_<workload>.json);
  gemm_util     the same for all four grouped GEMMs together;
  kernels       every kernel: time per forward, FLOP/s and algorithmic GB/s,
                each against its peak; from the counter record, HBM bytes per
                launch and their rate over the measured launch time, and the
                matrix-core / vector-ALU busy fractions;
  launches      kernel and graph launches per forward, diagonal vs sequential;
  cpu_baseline  the CPU oracle timed on a bounded sample (first nodes of
                segment 0) on this host.
Weights and inputs are random (seeded) of the ARMT shapes; no checkpoint.
"""

import argparse
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PEAK_F32_TFLOPS = 157.3   # fp32 vector, published (packed fp32 counted)
METRIC = "tokens/s, 131K-token 1B-shape ARMT forward (diag vs seq); GEMM MFMA util %"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="1b_s128")
    ap.add_argument("--roofline-kernel", default="gate_up")
    ap.add_argument("--no-seq", action="store_true", help="skip the sequential-schedule timing")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--gemm-rows", type=int, default=0,
                    help="rows per GEMM tile / 16 (0: the library's choice)")
    ap.add_argument("--profile-only", action="store_true",
                    help="only the diagonal forward (for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only a plain 256 MiB device-to-device copy, three times (to calibrate the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    ap.add_argument("--all-workloads", action="store_true",
                    help="time diagonal and sequential forwards of every benchmark workload, one JSON "
                         "line each")
    ap.add_argument("--group-sweep", action="store_true",
                    help="grouped GEMM and attention throughput against the wave width k (1B shapes)")
    ap.add_argument("--logit-drift", action="store_true",
                    help="LM-head logits of the last segment against the segment count: diagonal vs "
                         "sequential vs the CPU oracle, one JSON line per count, plus the LM head's "
                         "throughput over the whole sequence")
    ap.add_argument("--drift-segments", type=int, default=8,
                    help="largest segment count of --logit-drift (the oracle runs this many segments)")
    ap.add_argument("--full-attention", action="store_true",
                    help="full-attention Llama comparator against the diagonal ARMT forward at 4K..131K "
                         "tokens (1B shape): time, speed-up and workspace memory, one JSON line per length")
    ap.add_argument("--batch-sweep", action="store_true",
                    help="diagonal forward of B = 1, 2, 4, 8 independent 32-segment sequences per node "
                         "(1B shape): total tokens/s against the batch size")
    ap.add_argument("--backward", action="store_true",
                    help="grouped backward (reversed diagonal waves) against the node-by-node backward on an "
                         "fp32 workload and on the 1B shape in bf16: time per forward + backward, one JSON line "
                         "per workload and schedule")
    ap.add_argument("--trace-summary", metavar="DB",
                    help="print per-kernel tables of a rocprofv3 --kernel-trace database (rocpd SQLite) "
                         "of --profile-only forwards (--forwards N in it); no GPU needed")
    ap.add_argument("--forwards", type=int, default=5, help="forwards in the traced run (--trace-summary)")
    ap.add_argument("--pmc-summary", action="store_true",
                    help="print the committed counter record of --workload as a table; no GPU needed")
    ap.add_argument("--pmc-record", metavar="DIR",
                    help="write profiles/pmc_<workload>.json, the per-kernel counter record, from the CSV "
                         "output of rocprofv3 --pmc passes under DIR (pmc_* over bench.py --profile-only, "
                         "calib_FETCH_SIZE / calib_WRITE_SIZE over --copy-calibration); no GPU needed")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# shared helpers
# ---------------------------------------------------------------------------

def to_dev(a, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev, torch.bfloat16).contiguous()


def build(inp, cfg, dev, layers=None, gemm_rows=0):
    """Device weights and a model of the first `layers` layers of `inp`."""
    from long_context_recurrent_amd import armt as C
    from long_context_recurrent_amd.model import ArmtModel, make_config
    L = layers or cfg.n_layers
    w = {k: to_dev(v[:L], dev) for k, v in inp.weights.items()}
    w.update(g_attn=to_dev(inp.g_attn[:L], dev), g_mlp=to_dev(inp.g_mlp[:L], dev),
             mem_emb=to_dev(inp.mem_emb, dev))
    ccfg = make_config(L, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                       cfg.ffn_hidden, cfg.seg_len, cfg.n_mem, cfg.d_key, cfg.dtype)
    model = ArmtModel(ccfg, w)
    if gemm_rows:
        model.set_option(C.ARMT_OPT_GEMM_ROWS, gemm_rows)
    return model


def node_gflop(cfg):
    return sum(cfg.node_flops().values()) / 1e9


class Runner:
    """Times forwards of one model on its stream."""

    def __init__(self, model, x, n_segments):
        import torch
        from long_context_recurrent_amd import armt as C
        self.C, self.torch = C, torch
        self.model, self.x, self.S = model, x, n_segments
        self.out = model.alloc_outputs(n_segments)

    def run(self, schedule, k):
        fn = self.C.armt_forward_diagonal if schedule == "diagonal" else self.C.armt_forward_sequential
        for _ in range(k):
            fn(self.model.handle, self.x, self.S, None, None, self.out[0], self.out[1], self.out[2])

    def timed(self, schedule, steps, warmup):
        """(mean seconds per forward over `steps` forwards bracketed by
        synchronisations, [per-forward seconds from HIP events])."""
        torch, st = self.torch, self.model.stream
        self.run(schedule, warmup)
        torch.cuda.synchronize()
        st.synchronize()
        a = time.perf_counter()
        self.run(schedule, steps)
        st.synchronize()
        torch.cuda.synchronize()
        mean = (time.perf_counter() - a) / steps
        each = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            self.run(schedule, 1)
            e1.record(st)
            e1.synchronize()
            each.append(e0.elapsed_time(e1) * 1e-3)
        return mean, each

    def kernel_stats(self, forwards):
        C, stats = self.C, {}
        for kname in C.KERNELS:
            self.model.set_option(C.ARMT_OPT_TIME_KERNEL, C.KERNELS.index(kname))
            self.run("diagonal", forwards)
            stats[kname] = self.model.kernel_stats()
            self.model.set_option(C.ARMT_OPT_TIME_KERNEL, -1)
        return stats


def launches(cfg, S, L):
    """Kernel and graph launches per forward of both schedules."""
    per_node = 9 if cfg.dtype == "bf16" else 10
    return {"diagonal": {"graph_launches": S + L - 1, "kernels": per_node * (S + L - 1)},
            "sequential": {"graph_launches": S * L, "kernels": per_node * S * L},
            "kernels_per_wave": per_node}


def timing_summary(mean, each, tokens):
    return {"ms_mean": mean * 1e3, "ms_median": statistics.median(each) * 1e3, "ms_min": min(each) * 1e3,
            "tokens_per_s_median": tokens / statistics.median(each)}


def kernel_summary(v, forwards, kernel=None, workload=None, rec=None):
    """Per-kernel figures from HIP-event timing: time per forward, algorithmic
    FLOP/s against the bf16 MFMA peak and algorithmic bytes/s against HBM;
    with a current counter record, the HBM bytes the counters measured per
    launch over the same launch time, and the matrix-core busy fraction."""
    sec = v["ms"] * 1e-3
    tf = v["flops"] / sec / 1e12 if sec else 0.0
    gbs = v["bytes"] / sec / 1e9 if sec else 0.0
    out = {"us_per_forward": v["ms"] * 1e3 / forwards, "launches_per_forward": v["launches"] // forwards,
           "tflops": tf, "frac_mfma_bf16": tf / PEAK_BF16_TFLOPS, "gb_s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS}
    if kernel is not None and rec is not None:
        tb = measured_traffic(kernel, workload, rec)
        if tb is not None and v["launches"]:
            per_launch_s = sec / v["launches"]
            out.update(traffic_bytes_per_launch=tb, traffic_gb_s=tb / per_launch_s / 1e9,
                       traffic_frac_hbm=tb / per_launch_s / 1e9 / PEAK_HBM_GBS,
                       traffic_over_algorithmic=tb * v["launches"] / v["bytes"] if v["bytes"] else None)
        mu = counter_value(kernel, workload, "MfmaUtil", rec)
        if mu is not None:
            out["mfma_busy_counter"] = mu / 100.0
        vb = counter_value(kernel, workload, "VALUBusy", rec)
        if vb is not None:
            out["valu_busy_counter"] = vb / 100.0
    return out


PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {"mem_read": "memory_mfma.hip", "qkv": "gemm_bf16.hip", "attn": "attention.hip",
                  "o_proj": "gemm_bf16.hip", "mlp_norm": "memory.hip", "gate_up": "gemm_bf16.hip",
                  "down": "gemm_bf16.hip", "mem_keys": "memory_mfma.hip", "mem_update": "memory_mfma.hip"}
EPI_KERNEL = {1: "qkv", 3: "gate_up"}     # gemm_bf16_kernel<RB, EPI>; EPI 2 (residual) is O-proj or down


def _source_sha(kernel):
    import hashlib
    with open(os.path.join(ROOT, "long_context_recurrent_amd", "csrc", KERNEL_SOURCES[kernel]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def pmc_record(workload):
    """The committed per-kernel counter record of a workload (None if absent)."""
    path = os.path.join(PROFILE_DIR, f"pmc_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        return json.load(f)


def measured_traffic(kernel, workload, rec=None):
    """HBM bytes per launch of ``kernel`` from the committed FETCH_SIZE /
    WRITE_SIZE counters of this workload, scaled by the copy-kernel
    calibration stored with them; None when there is no record or the
    kernel's source changed since the counters were taken."""
    rec = rec if rec is not None else pmc_record(workload)
    k = (rec or {}).get("kernels", {}).get(kernel)
    if not k or "FETCH_SIZE" not in k or "WRITE_SIZE" not in k:
        return None
    if k.get("source_sha256") != _source_sha(kernel):
        log(f"counter record for {kernel} is stale (kernel source changed); reporting null")
        return None
    cal = rec["calibration"]
    return (k["FETCH_SIZE"] * cal["FETCH_SIZE_factor"] + k["WRITE_SIZE"] * cal["WRITE_SIZE_factor"]) * 1024.0


def counter_value(kernel, workload, counter, rec=None):
    """Average per-dispatch value of a collected counter (None if absent or stale)."""
    rec = rec if rec is not None else pmc_record(workload)
    k = (rec or {}).get("kernels", {}).get(kernel)
    if not k or counter not in k or k.get("source_sha256") != _source_sha(kernel):
        return None
    return k[counter]


def _pmc_label(name, resid_seen):
    """Forward kernel of a dispatch from its kernel name; the residual GEMMs
    alternate O-proj, down within every wave."""
    if "gemm_bf16_kernel<" in name:
        epi = int(name.split("gemm_bf16_kernel<", 1)[1].split(">", 1)[0].split(",")[1])
        if epi == 2:
            return ("o_proj", "down")[resid_seen % 2]
        return EPI_KERNEL.get(epi)
    for key, k in (("memread_norm", "mem_read"), ("attn_bf16_kernel", "attn"), ("rmsnorm_kernel", "mlp_norm"),
                   ("memkeys", "mem_keys"), ("memupdate", "mem_update")):
        if key in name:
            return k
    return None


def write_pmc_record(args):
    """Per-kernel counter record of one profiled forward: every
    DIR/pmc_*/run_counter_collection.csv (rocprofv3 --pmc passes over
    ``bench.py --profile-only``) averaged per dispatch for each forward
    kernel, and the factors that make FETCH_SIZE / WRITE_SIZE read the true
    byte count of a plain 256 MiB copy (DIR/calib_*)."""
    import csv
    d = args.pmc_record
    out = {"workload": args.workload, "kernels": {}, "calibration": {"copy_bytes": 64 * 1024 * 1024 * 4}}
    sums = {}
    passes = sorted(p for p in os.listdir(d) if p.startswith("pmc_") and os.path.isdir(os.path.join(d, p)))
    for p in passes:
        with open(os.path.join(d, p, "run_counter_collection.csv"), newline="") as f:
            rows = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
        by_dispatch = {}
        for r in rows:
            by_dispatch.setdefault(int(r["Dispatch_Id"]), []).append(r)
        resid = 0
        for did in sorted(by_dispatch):
            rs = by_dispatch[did]
            k = _pmc_label(rs[0]["Kernel_Name"], resid)
            if "gemm_bf16_kernel<" in rs[0]["Kernel_Name"] and k in ("o_proj", "down"):
                resid += 1
            if k is None:
                continue
            for r in rs:
                acc = sums.setdefault(k, {}).setdefault(r["Counter_Name"], [0.0, 0])
                acc[0] += float(r["Counter_Value"])
                acc[1] += 1
    for k, ctrs in sums.items():
        rec = {c: v[0] / v[1] for c, v in ctrs.items()}
        rec["dispatches"] = max(v[1] for v in ctrs.values())
        rec["source"] = KERNEL_SOURCES[k]
        rec["source_sha256"] = _source_sha(k)
        out["kernels"][k] = rec
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        path = os.path.join(d, f"calib_{ctr}", "run_counter_collection.csv")
        if not os.path.exists(path):
            continue
        with open(path, newline="") as f:
            crows = [r for r in csv.DictReader(f) if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == ctr]
        kib = sum(float(r["Counter_Value"]) for r in crows) / len(crows)
        out["calibration"][f"{ctr}_kib"] = kib
        out["calibration"][f"{ctr}_factor"] = round(out["calibration"]["copy_bytes"] / 1024.0 / kib, 4)
    out["commands"] = [
        "cd /tmp && export TMPDIR=/tmp",
        "timeout -s KILL 150 rocprofv3 --pmc <COUNTERS> --output-format csv -d DIR/pmc_<NAME> -o run -- "
        "python3 /root/repo/bench.py --steps 1 --warmup 0 --profile-only   (one pass per counter set: "
        + "; ".join(p[4:] for p in passes) + ")",
        "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/calib_FETCH_SIZE -o run -- "
        "python3 /root/repo/bench.py --copy-calibration   (and WRITE_SIZE into DIR/calib_WRITE_SIZE)",
        f"python3 bench.py --workload {args.workload} --pmc-record DIR",
    ]
    path = os.path.join(PROFILE_DIR, f"pmc_{args.workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    log(f"wrote {path}: kernels {sorted(out['kernels'])}")


def trace_summary(db_path, forwards):
    """Markdown tables from a rocprofv3 --kernel-trace database: every forward
    kernel's dispatches summed by logical kernel (the residual GEMMs split into
    O-proj and down by their order in each wave) and by instantiation."""
    import sqlite3
    cur = sqlite3.connect(db_path).cursor()
    rows = list(cur.execute("select dispatch_id, name, duration from kernels order by dispatch_id"))
    per_kernel, per_name, resid = {}, {}, 0
    for _, name, dur in rows:
        short = name.replace("armt::", "").replace("void ", "")
        a = per_name.setdefault(short, [0, 0.0, float("inf"), 0.0])
        a[0] += 1
        a[1] += dur
        a[2] = min(a[2], dur)
        a[3] = max(a[3], dur)
        k = _pmc_label(name, resid)
        if "gemm_bf16_kernel<" in name and k in ("o_proj", "down"):
            resid += 1
        if k is not None:
            b = per_kernel.setdefault(k, [0, 0.0])
            b[0] += 1
            b[1] += dur
    out = ["| kernel | calls | total ms | ms / forward | avg us / call |", "|:--|--:|--:|--:|--:|"]
    total = 0.0
    for k in KERNEL_SOURCES:
        if k in per_kernel:
            n, t = per_kernel[k]
            total += t
            out.append(f"| {k} | {n} | {t / 1e6:.1f} | {t / 1e6 / forwards:.2f} | {t / n / 1e3:.1f} |")
    out.append(f"| sum | | {total / 1e6:.1f} | {total / 1e6 / forwards:.2f} | |")
    out += ["", "| kernel (instantiation) | calls | total ms | avg us | min us | max us |",
            "|:--|--:|--:|--:|--:|--:|"]
    for short, (n, t, lo, hi) in sorted(per_name.items(), key=lambda kv: -kv[1][1]):
        out.append(f"| {short} | {n} | {t / 1e6:.1f} | {t / n / 1e3:.1f} | {lo / 1e3:.1f} | {hi / 1e3:.1f} |")
    return "\n".join(out)


def pmc_markdown(workload):
    """Markdown table of the committed counter record: per kernel the
    matrix-core busy fraction (MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES /
    (GRBM_GUI_ACTIVE x SIMDs)), the vector-ALU busy fraction (VALUBusy =
    SQ_ACTIVE_INST_VALU / (GRBM_GUI_ACTIVE x CUs)), the LDS bank-conflict
    stall fraction, the counted bf16 MFMA FLOPs (SQ_INSTS_VALU_MFMA_MOPS_BF16 x
    512) and the calibrated HBM bytes per dispatch."""
    rec = pmc_record(workload)
    cal = rec["calibration"]
    out = ["| kernel | dispatches | MFMA busy | VALU busy | LDS bank-conflict stall | MFMA GFLOP / dispatch "
           "| HBM read MB / dispatch | HBM write MB / dispatch | HBM MB / dispatch |",
           "|:--|--:|--:|--:|--:|--:|--:|--:|--:|"]
    for k in KERNEL_SOURCES:
        v = rec["kernels"].get(k)
        if not v:
            continue
        rd = v.get("FETCH_SIZE", 0) * cal["FETCH_SIZE_factor"] * 1024 / 1e6
        wr = v.get("WRITE_SIZE", 0) * cal["WRITE_SIZE_factor"] * 1024 / 1e6
        fl = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) * 512 / 1e9
        out.append(f"| {k} | {v['dispatches']} | {v.get('MfmaUtil', 0):.1f}% | {v.get('VALUBusy', 0):.1f}% | "
                   f"{v.get('LDSBankConflict', 0):.1f}% | {fl:.1f} | {rd:.1f} | {wr:.1f} | {rd + wr:.1f} |")
    # where the waves' resident cycles go (SQ_WAVE_CYCLES split into issuing,
    # waiting on a counter or barrier, and ready but not issued) and the mean
    # occupancy, when those passes are in the record
    if any("SQ_WAIT_INST_ANY" in v for v in rec["kernels"].values()):
        out += ["", "| kernel | waves / dispatch | mean occupancy (waves per CU) | issuing | waiting on a counter "
                "or barrier | ready, not issued |", "|:--|--:|--:|--:|--:|--:|"]
        for k in KERNEL_SOURCES:
            v = rec["kernels"].get(k)
            if not v or "SQ_WAIT_INST_ANY" not in v or not v.get("SQ_WAVE_CYCLES"):
                continue
            wc = v["SQ_WAVE_CYCLES"]
            out.append(f"| {k} | {v.get('SQ_WAVES', 0):.0f} | {v.get('MeanOccupancyPerCU', 0):.1f} | "
                       f"{100 * v['SQ_ACTIVE_INST_ANY'] / wc:.0f}% | {100 * v['SQ_WAIT_ANY'] / wc:.0f}% | "
                       f"{100 * v['SQ_WAIT_INST_ANY'] / wc:.0f}% |")
    return "\n".join(out)


def host_cpu():
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except Exception:
        pass
    return {"os_cpu_count": os.cpu_count(), "model": model,
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def roofline_mfma(achieved_tflops):
    """Roofline object of a contraction-bound path against the bf16 peak."""
    return {"bound": "mfma", "achieved": achieved_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved_tflops / PEAK_BF16_TFLOPS, "traffic": None}


def oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
    except Exception:
        return os.cpu_count()


def cpu_baseline(inp, seconds):
    """The oracle as it stands, on this host: nodes in sequential order
    (segment 0 through every layer, then segment 1, ...), each layer carrying
    its own memory state, until about `seconds` of CPU work; tokens/s =
    T / (L * mean node time), i.e. one segment through every layer."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
    except Exception:
        cores = os.cpu_count()
    cfg = inp.cfg
    o = oracle.Oracle(inp)
    A = [np.zeros((cfg.d_model, cfg.d_key)) for _ in range(cfg.n_layers)]
    z = [np.zeros(cfg.d_key) for _ in range(cfg.n_layers)]
    done, a = 0, time.perf_counter()
    for s in range(cfg.n_segments):
        h = o.node_input(s)
        for l in range(cfg.n_layers):
            h, A[l], z[l] = o.node(l, h, A[l], z[l])
            done += 1
            if time.perf_counter() - a > seconds:
                break
        if time.perf_counter() - a > seconds:
            break
    segs = (done + cfg.n_layers - 1) // cfg.n_layers
    el = time.perf_counter() - a
    per_node = el / done
    value = cfg.seg_len / (per_node * cfg.n_layers)
    log(f"cpu oracle: {done} nodes in {el:.1f}s -> {value:.1f} tokens/s")
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle", "host": host_cpu(),
            "sample": f"{done} node(s) of segments 0..{segs - 1} in sequential order ({cfg.seg_len + cfg.n_mem} rows each, "
                      f"float64 NumPy, BLAS threads = {cores}) in {el:.1f}s; "
                      f"tokens/s = T / (L * mean node time)"}


# ---------------------------------------------------------------------------
# modes
# ---------------------------------------------------------------------------

def headline(args, dev):
    from armt_inputs import get_config, make_inputs
    cfg = get_config(args.workload)
    t0 = time.time()
    inp = make_inputs(cfg)
    log(f"inputs drawn in {time.time() - t0:.1f}s")
    model = build(inp, cfg, dev, gemm_rows=args.gemm_rows)
    x = to_dev(inp.x, dev)
    S, T, L = cfg.n_segments, cfg.seg_len, cfg.n_layers
    tokens = S * T
    r = Runner(model, x, S)

    log(f"warmup {args.warmup}, timing {args.steps} diagonal forwards of {args.workload}")
    diag_s, diag_each = r.timed("diagonal", args.steps, args.warmup)
    log(f"diagonal: {diag_s * 1e3:.1f} ms/forward, {tokens / diag_s:.0f} tokens/s "
        f"(median {statistics.median(diag_each) * 1e3:.1f}, min {min(diag_each) * 1e3:.1f} ms)")
    if args.profile_only:
        return
    seq_s = seq_each = None
    if not args.no_seq:
        seq_s, seq_each = r.timed("sequential", args.steps, 1)
        log(f"sequential: {seq_s * 1e3:.1f} ms/forward, {tokens / seq_s:.0f} tokens/s")

    nfwd = max(1, min(args.steps, 3))
    kstats = r.kernel_stats(nfwd)
    rk = kstats[args.roofline_kernel]
    achieved = rk["flops"] / (rk["ms"] * 1e-3) / 1e12
    prec = pmc_record(args.workload)
    traffic = measured_traffic(args.roofline_kernel, args.workload, prec)
    gemm = [kstats[k] for k in ("qkv", "o_proj", "gate_up", "down")]
    g_flops = sum(k["flops"] for k in gemm)
    g_ms = sum(k["ms"] for k in gemm)
    for k, v in kstats.items():
        tf = v["flops"] / (v["ms"] * 1e-3) / 1e12 if v["ms"] else 0.0
        gbs = v["bytes"] / (v["ms"] * 1e-3) / 1e9 if v["ms"] else 0.0
        log(f"  {k:10s} {v['ms'] / max(v['launches'], 1) * 1e3:9.1f} us/launch  {tf:7.1f} TFLOP/s  {gbs:7.0f} GB/s")

    cpu = None if args.no_cpu else cpu_baseline(inp, args.cpu_seconds)
    res = {
        "metric": METRIC,
        "value": tokens / diag_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": diag_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) weights of the 1B ARMT shape)",
        "config": {"workload": args.workload, "n_layers": L, "d_model": cfg.d_model,
                   "heads": f"{cfg.n_heads}/{cfg.n_kv_heads}x{cfg.head_dim}", "ffn": cfg.ffn_hidden,
                   "seg_len": T, "n_mem": cfg.n_mem, "n_segments": S, "tokens": tokens, "batch": 1,
                   "waves": S + L - 1},
        "diagonal": timing_summary(diag_s, diag_each, tokens),
        "sequential": None if seq_s is None else dict(
            timing_summary(seq_s, seq_each, tokens), value=tokens / seq_s, unit="tokens/s",
            ms_per_step=seq_s * 1e3, diag_speedup=seq_s / diag_s),
        "launches": launches(cfg, S, L),
        "roofline": {"kernel": args.roofline_kernel, "bound": "mfma", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "launches": rk["launches"],
                     "avg_launch_us": rk["ms"] / max(rk["launches"], 1) * 1e3},
        "gemm_util": {"achieved": g_flops / (g_ms * 1e-3) / 1e12, "unit": "TFLOP/s",
                      "frac": g_flops / (g_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "kernels": {k: kernel_summary(v, nfwd, k, args.workload, prec) for k, v in kstats.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    model.close()


def all_workloads(args, dev):
    """Diagonal and sequential forwards of every benchmark workload (the
    oracle-sized ones excluded), one JSON line each."""
    import gc
    import torch
    from armt_inputs import get_config, make_inputs
    for names in (["1b_s32", "1b_s128"], ["3b_t512", "3b_t1024", "3b_t2048"]):
        inp = make_inputs(get_config(names[-1]))    # the longest X of the group; row prefixes serve the rest
        for name in names:
            cfg = get_config(name)
            S, T, L = cfg.n_segments, cfg.seg_len, cfg.n_layers
            model = build(inp, cfg, dev)
            x = to_dev(inp.x[:S * T], dev)
            r = Runner(model, x, S)
            d_mean, d_each = r.timed("diagonal", args.steps, args.warmup)
            s_mean, s_each = r.timed("sequential", args.steps, 1)
            line = {"workload": name, "tokens": S * T, "waves": S + L - 1,
                    "node_gflop": node_gflop(cfg),
                    "diagonal": timing_summary(d_mean, d_each, S * T),
                    "sequential": timing_summary(s_mean, s_each, S * T),
                    "diag_speedup": s_mean / d_mean,
                    "tflops_diagonal": node_gflop(cfg) * S * L / d_mean / 1e3,
                    "launches": launches(cfg, S, L)}
            log(f"{name}: diag {d_mean * 1e3:.1f} ms, seq {s_mean * 1e3:.1f} ms, x{s_mean / d_mean:.2f}")
            print(json.dumps(line), flush=True)
            model.close()
            del model, x, r
            gc.collect()
            torch.cuda.empty_cache()
        del inp
        gc.collect()


def logit_drift(args, dev):
    """Relative logit drift against the number of segments processed, in the
    manner of the pages' Table 2 (Pith review: falsifier and referee report):
    for S = 1 .. S_max the logits of segment S - 1 from a diagonal and a
    sequential forward of S segments, and from the float64 oracle run over the
    same S segments (random weights of the workload's shape, synthetic V)."""
    import numpy as np
    import torch
    import oracle
    from armt_inputs import get_config, make_head, make_inputs
    cfg = get_config(args.workload)
    S_max, T, L = args.drift_segments, cfg.seg_len, cfg.n_layers
    inp = make_inputs(cfg, n_segments=max(S_max, cfg.n_segments))
    w_lm, g = make_head(cfg)
    V = w_lm.shape[0]
    model = build(inp, cfg, dev)
    dw, dg = to_dev(w_lm, dev), to_dev(g, dev)
    x = to_dev(inp.x, dev)

    # LM head throughput over the workload's whole output (S * T rows)
    S = cfg.n_segments
    y, _, _ = model.forward(x[:S * T].contiguous(), "diagonal")
    lg = torch.empty(S * T, V, dtype=torch.float32, device=dev)
    st = model.stream
    model.logits(y, dg, dw, out=lg)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(3):
        model.logits(y, dg, dw, out=lg, sync=False)
    e1.record(st)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / 3
    flops = 2.0 * S * T * V * cfg.d_model
    head = {"rows": S * T, "vocab": V, "ms": ms, "tflops": flops / ms / 1e9,
            "frac_mfma_bf16": flops / ms / 1e9 / PEAK_BF16_TFLOPS}
    cpu = None
    if not args.no_cpu:
        # the oracle's LM head (float64) on the first rows of the same output
        rows = min(S * T, 4096)
        yh = y[:rows].to(torch.float64).cpu().numpy()
        a = time.perf_counter()
        oracle.logits(yh, g, w_lm, cfg.dtype, cfg.rms_eps)
        el = time.perf_counter() - a
        cpu = {"value": rows / el, "unit": "rows/s", "cores": oracle_threads(), "kind": "oracle",
               "host": host_cpu(), "sample": f"final norm + LM head of {rows} of {S * T} rows (V={V}, float64 "
                                              f"NumPy) in {el:.2f}s"}
        log(f"cpu oracle LM head: {rows} rows in {el:.2f}s")
    log(f"LM head over {S * T} rows, V={V}: {ms:.2f} ms, {head['tflops']:.0f} TFLOP/s")
    print(json.dumps({"workload": args.workload, "lm_head": head, "roofline": roofline_mfma(head["tflops"]),
                      "rows_per_s": S * T / (ms * 1e-3), "cpu_baseline": cpu}), flush=True)
    del lg, y

    o = oracle.Oracle(inp)
    A, z = o.initial_state()
    for s in range(S_max):
        xs = x[:(s + 1) * T].contiguous()
        out = {}
        for sched in ("diagonal", "sequential"):
            y, _, _ = model.forward(xs, sched)
            out[sched] = model.logits(y[s * T:].contiguous(), dg, dw).clone()
        t0 = time.time()
        h = o.node_input(s)
        for l in range(L):
            h, A[l], z[l] = o.node(l, h, A[l], z[l])
        ref = oracle.logits(o.R(h[:T]), g, w_lm, cfg.dtype, cfg.rms_eps)
        got = out["diagonal"].to(torch.float64).cpu().numpy()
        diff = out["diagonal"] - out["sequential"]
        line = {"workload": args.workload, "segments": s + 1, "tokens": (s + 1) * T, "vocab": V,
                "rows_compared": T,
                "diag_vs_seq": {"rel_l2": float(torch.linalg.vector_norm(diff) /
                                                torch.linalg.vector_norm(out["sequential"])),
                                "max_abs": float(diff.abs().max()),
                                "bitwise_equal": bool(torch.equal(out["diagonal"], out["sequential"]))},
                "gpu_vs_oracle": {"rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
                                  "max_abs": float(np.abs(got - ref).max()),
                                  "max_abs_ref": float(np.abs(ref).max()),
                                  "argmax_agree": float(np.mean(got.argmax(1) == ref.argmax(1)))},
                "oracle_s": time.time() - t0}
        log(f"S={s + 1}: diag vs seq {line['diag_vs_seq']['rel_l2']:.1e}, "
            f"vs oracle {line['gpu_vs_oracle']['rel_l2']:.2e} (oracle {line['oracle_s']:.0f}s)")
        print(json.dumps(line), flush=True)
    model.close()


def full_attention(args, dev):
    """The pages' comparator (paper page, abstract; Pith review, Figure 1 and
    Table 1): the same Llama-shaped layers with no memory over the whole
    sequence as one causal window, against the diagonal ARMT forward over the
    same tokens in 1,024-token segments.  Random weights of the 1B shape."""
    import gc
    import torch
    from armt_inputs import get_config, make_inputs
    from long_context_recurrent_amd import armt as C
    from long_context_recurrent_amd.model import FullAttentionModel
    cfg = get_config("1b_s128")
    T, L, d = cfg.seg_len, cfg.n_layers, cfg.d_model
    inp = make_inputs(cfg)
    x_all = to_dev(inp.x, dev)
    w = {k: to_dev(inp.weights[k], dev) for k in ("w_qkv", "w_o", "w_gate", "w_up", "w_down")}
    w.update(g_attn=to_dev(inp.g_attn, dev), g_mlp=to_dev(inp.g_mlp, dev))
    armt = build(inp, cfg, dev)
    ccfg = armt.cfg
    armt_ws = armt.ws_bytes
    per_layer = cfg.node_flops()
    blk = 2 * d * (cfg.qkv_dim + cfg.n_heads * cfg.head_dim + 3 * cfg.ffn_hidden)   # GEMM FLOPs per token

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        each = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            each.append(e0.elapsed_time(e1) * 1e-3)
        return statistics.median(each), min(each)

    cpu = None
    if not args.no_cpu:
        # the oracle's full-attention forward (float64) on 1,024 tokens through
        # 2 of the 16 layers; tokens/s scaled by 2/16 (at 1,024 tokens the
        # products dominate, so the scaling holds there; longer windows cost
        # the oracle more per token)
        import numpy as np
        import oracle
        Ls, Ns = 2, 1024
        sub = inp.__class__(cfg=cfg.with_(n_layers=Ls, n_segments=1), x=inp.x[:Ns], mem_emb=inp.mem_emb,
                            weights={k: v[:Ls] for k, v in inp.weights.items()}, g_attn=inp.g_attn[:Ls],
                            g_mlp=inp.g_mlp[:Ls])
        a = time.perf_counter()
        oracle.llama_forward(sub, n_tokens=Ns)
        el = time.perf_counter() - a
        cpu = {"value": Ns / el * Ls / L, "unit": "tokens/s", "cores": oracle_threads(), "kind": "oracle",
               "host": host_cpu(), "sample": f"full-attention forward of {Ns} tokens through {Ls} of {L} layers "
                                              f"(float64 NumPy) in {el:.1f}s; tokens/s scaled by {Ls}/{L}"}
        log(f"cpu oracle full attention: {Ns} tokens x {Ls} layers in {el:.1f}s")
    for N in (4096, 8192, 16384, 32768, 65536, 131072):
        S = N // T
        x = x_all[:N]
        full = FullAttentionModel(ccfg, w, N)
        y = torch.empty(N, d, dtype=torch.bfloat16, device=dev)
        t_full, t_full_min = timed(lambda: full.forward(x, out=y, sync=False), max(1, min(args.steps, 3)))
        full_ws = full.ws_bytes
        full.close()
        del full
        out = armt.alloc_outputs(S)
        t_armt, t_armt_min = timed(lambda: armt.forward(x, "diagonal", out=out, sync=False),
                                   max(1, min(args.steps, 3)))
        flops_full = N * blk * L + L * 4 * (N * (N + 1) / 2) * cfg.head_dim * cfg.n_heads
        flops_armt = sum(per_layer.values()) * S * L
        line = {"workload": "1b", "tokens": N, "segments_armt": S,
                "full_attention": {"ms": t_full * 1e3, "ms_min": t_full_min * 1e3, "tokens_per_s": N / t_full,
                                   "tflops": flops_full / t_full / 1e12, "workspace_bytes": full_ws},
                "armt_diagonal": {"ms": t_armt * 1e3, "ms_min": t_armt_min * 1e3, "tokens_per_s": N / t_armt,
                                  "tflops": flops_armt / t_armt / 1e12, "workspace_bytes": armt_ws},
                "speedup_armt_over_full": t_full / t_armt,
                "workspace_ratio_full_over_armt": full_ws / armt_ws,
                "roofline": dict(roofline_mfma(flops_full / t_full / 1e12), path="full attention forward"),
                "cpu_baseline": cpu if N == 4096 else None}
        log(f"N={N}: full attention {t_full * 1e3:.1f} ms ({line['full_attention']['tflops']:.0f} TFLOP/s), "
            f"ARMT diagonal {t_armt * 1e3:.1f} ms, x{t_full / t_armt:.2f}; workspace "
            f"{full_ws / 2**30:.2f} vs {armt_ws / 2**30:.2f} GiB")
        print(json.dumps(line), flush=True)
        del y, out
        gc.collect()
        torch.cuda.empty_cache()
    armt.close()


def batch_sweep(args, dev):
    """B independent sequences of 32 segments (1B shape) in one batched
    handle: the grouped kernels see P layers x B sequences per launch."""
    import gc
    import numpy as np
    import torch
    from armt_inputs import get_config, make_batch_x, make_inputs
    from long_context_recurrent_amd.model import ArmtModel
    cfg = get_config("1b_s32")
    S, T, L = cfg.n_segments, cfg.seg_len, cfg.n_layers
    inp = make_inputs(cfg)
    base = build(inp, cfg, dev)
    w, ccfg = base.weights, base.cfg
    xs_all = make_batch_x(cfg, inp, 8)
    base.close()
    # a batch adds no arithmetic of its own: the oracle's forward rate is the
    # headline's (per sequence, one node at a time)
    cpu = None if args.no_cpu else cpu_baseline(inp, args.cpu_seconds)
    for B in (1, 2, 4, 8):
        model = ArmtModel(ccfg, w, batch=B)
        x = to_dev(np.ascontiguousarray(xs_all[:B]) if B > 1 else xs_all[0], dev)
        out = model.alloc_outputs(S)
        run = lambda: model.forward(x, "diagonal", out=out, sync=False)
        run()
        torch.cuda.synchronize()
        each = []
        for _ in range(max(1, min(args.steps, 3))):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            e1.synchronize()
            each.append(e0.elapsed_time(e1) * 1e-3)
        t = statistics.median(each)
        tokens = B * S * T
        tf = node_gflop(cfg) * S * L * B / t / 1e3
        line = {"workload": "1b_s32", "batch": B, "tokens": tokens, "ms": t * 1e3, "tokens_per_s": tokens / t,
                "tflops": tf, "workspace_bytes": model.ws_bytes, "roofline": roofline_mfma(tf),
                "cpu_baseline": cpu if B == 1 else None}
        log(f"B={B}: {t * 1e3:.1f} ms, {tokens / t:.0f} tokens/s, {line['tflops']:.0f} TFLOP/s")
        print(json.dumps(line), flush=True)
        model.close()
        del model, x, out
        gc.collect()
        torch.cuda.empty_cache()


def backward_bench(args, dev):
    """Forward + backward: the grouped backward over the reversed diagonal
    waves against the node-by-node backward in reverse segment-major order
    (same results, bitwise), on an 8-layer fp32 workload (vector-ALU kernels)
    and on the 1B shape in bf16 (16 layers, 32 segments; matrix cores)."""
    from armt_inputs import get_config
    fp32 = get_config("tiny_fp32").with_(name="fp32_l8_s32", n_layers=8, d_model=256, n_heads=4, n_kv_heads=2,
                                         head_dim=64, ffn_hidden=512, seg_len=128, n_mem=8, n_segments=32)
    one_b = get_config("1b_s128").with_(name="1b_bf16_s32", n_segments=32)
    backward_workload(args, dev, fp32, cpu_segments=fp32.n_segments, cpu_layers=None,
                      kernels="fp32 vector ALU (no packed fp32, no matrix cores)", peak=PEAK_F32_TFLOPS, bound="alu")
    backward_workload(args, dev, one_b, cpu_segments=2, cpu_layers=2,
                      kernels="bf16 matrix cores (fp32 operands as bf16 pairs; attention operands bf16)",
                      peak=PEAK_BF16_TFLOPS, bound="mfma")


def backward_workload(args, dev, cfg, cpu_segments, cpu_layers, kernels, peak, bound):
    import gc
    import numpy as np
    import torch
    from armt_inputs import make_inputs
    from long_context_recurrent_amd import armt as C
    from long_context_recurrent_amd.model import ArmtModel, WEIGHT_FIELDS, make_config
    S, T, L = cfg.n_segments, cfg.seg_len, cfg.n_layers
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    inp = make_inputs(cfg)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    w = {k: f(v) for k, v in inp.weights.items()}
    w.update(g_attn=f(inp.g_attn), g_mlp=f(inp.g_mlp), mem_emb=f(inp.mem_emb))
    ccfg = make_config(L, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn_hidden, T, cfg.n_mem,
                       dtype=cfg.dtype)
    model = ArmtModel(ccfg, w)
    x = f(inp.x)
    dy = torch.randn(x.shape, device=dev).to(dt)
    ws_bytes = C.armt_backward_workspace_size(model.handle, S)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
    ws_ptr = (ws.data_ptr() + 255) // 256 * 256
    grads = {k: torch.empty(w[k].shape, dtype=torch.float32, device=dev) for k in WEIGHT_FIELDS}
    gw = C.armt_weights(*[grads[k].data_ptr() for k in WEIGHT_FIELDS])
    dx = torch.empty(x.shape, dtype=torch.float32, device=dev)
    dA0 = torch.empty(L, cfg.d_model, 64, device=dev)
    dz0 = torch.empty(L, 64, device=dev)
    st = model.stream
    results = {}
    for sched, code in (("diagonal", 0), ("sequential", 1)):
        run = lambda: C.armt_backward(model.handle, code, x, S, None, None, dy, None, None, dx, dA0, dz0, gw,
                                      ws_ptr, ws_bytes)
        run()
        st.synchronize()
        each = []
        for _ in range(max(1, min(args.steps, 3))):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            run()
            e1.record(st)
            e1.synchronize()
            each.append(e0.elapsed_time(e1) * 1e-3)
        results[sched] = (statistics.median(each), dx.clone())
    y_t = statistics.median([timed_forward(model, x) for _ in range(3)])
    same = bool(torch.equal(results["diagonal"][1], results["sequential"][1]))
    # algorithmic work of forward + backward: every product of the forward has
    # two in the backward (input and weight gradients; for attention dV, dP,
    # dQ and dK), so three times the forward's FLOPs; the recomputation of
    # the forward inside the backward is not counted
    flops = 3 * node_gflop(cfg) * 1e9 * S * L
    cpu = None if args.no_cpu else grad_cpu_baseline(inp, cpu_segments, cpu_layers)
    for sched in ("diagonal", "sequential"):
        t = results[sched][0]
        achieved = flops / t / 1e12
        line = {"workload": cfg.name, "dtype": cfg.dtype, "schedule": sched, "tokens": S * T,
                "ms_forward_plus_backward": t * 1e3, "tokens_per_s": S * T / t,
                "ms_forward_alone": y_t * 1e3, "bitwise_equal_schedules": same,
                "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                             "frac": achieved / peak, "traffic": None,
                             "work": "3 x forward FLOPs (forward + input and weight gradients)"},
                "cpu_baseline": cpu if sched == "diagonal" else None, "kernels": kernels}
        log(f"{cfg.name} {sched}: forward + backward {t * 1e3:.1f} ms ({S * T / t:.0f} tokens/s, "
            f"{achieved:.2f} TFLOP/s); forward alone {y_t * 1e3:.1f} ms")
        print(json.dumps(line), flush=True)
    log(f"{cfg.name}: grouped backward speed-up {results['sequential'][0] / results['diagonal'][0]:.2f}x")
    model.close()
    del model, ws, grads, w, x, dy, dx
    gc.collect()
    torch.cuda.empty_cache()


def grad_cpu_baseline(inp, n_seg, n_layers=None):
    """The gradient oracle (float64 autograd) on the first `n_seg` segments
    (and, if given, the first `n_layers` layers) of the workload: tokens/s of
    forward + backward on the host, scaled to all layers by the layer
    count."""
    import numpy as np
    from oracle import armt_grad
    import torch
    cores = torch.get_num_threads()   # autograd's CPU kernels run on torch's thread pool
    cfg = inp.cfg
    L = cfg.n_layers
    Ls = L if n_layers is None else n_layers
    rows = n_seg * cfg.seg_len
    sub = inp.__class__(cfg=cfg.with_(n_segments=n_seg, n_layers=Ls), x=inp.x[:rows], mem_emb=inp.mem_emb,
                        weights={k: v[:Ls] for k, v in inp.weights.items()}, g_attn=inp.g_attn[:Ls],
                        g_mlp=inp.g_mlp[:Ls])
    rng = np.random.default_rng(0)
    dy = rng.standard_normal((rows, cfg.d_model))
    dA = np.zeros((Ls, cfg.d_model, cfg.d_key))
    dz = np.zeros((Ls, cfg.d_key))
    a = time.perf_counter()
    armt_grad.vjp(sub, None, None, dy, dA, dz)
    el = time.perf_counter() - a
    value = rows / el * Ls / L
    log(f"cpu gradient oracle: {n_seg} segment(s) x {Ls} layer(s) in {el:.1f}s -> {value:.1f} tokens/s")
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle", "host": host_cpu(),
            "sample": f"forward + backward of the first {n_seg} of {cfg.n_segments} segments through "
                      f"{Ls} of {L} layers by float64 autograd ({rows} tokens) in {el:.1f}s; "
                      f"tokens/s scaled by {Ls}/{L}"}


def timed_forward(model, x):
    import torch
    st = model.stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    model.forward(x, "diagonal", sync=False)
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e-3


def group_sweep(args, dev):
    """Grouped GEMM and attention throughput against the wave width k: a
    model of the first k layers of the 1B shape, run diagonally over 32 k
    segments, so all but 2(k - 1) of its 33k - 1 waves have exactly k nodes."""
    import numpy as np
    from armt_inputs import get_config, make_inputs
    base = get_config("1b_s128")
    inp = make_inputs(base)
    T = base.seg_len
    for k in (1, 2, 4, 8, 16):
        S = 32 * k
        reps = -(-S * T // inp.x.shape[0])
        xs = np.concatenate([inp.x] * reps)[:S * T] if reps > 1 else inp.x[:S * T]
        model = build(inp, base, dev, layers=k)
        r = Runner(model, to_dev(xs, dev), S)
        r.run("diagonal", 1)
        stats = r.kernel_stats(1)
        gemm = [stats[n] for n in ("qkv", "o_proj", "gate_up", "down")]
        gf, gms = sum(v["flops"] for v in gemm), sum(v["ms"] for v in gemm)
        at = stats["attn"]
        line = {"k": k, "n_segments": S, "waves": S + k - 1, "full_width_waves": S - k + 1,
                "gemm_tflops": gf / (gms * 1e-3) / 1e12,
                "attn_tflops": at["flops"] / (at["ms"] * 1e-3) / 1e12,
                "per_kernel_tflops": {n: stats[n]["flops"] / (stats[n]["ms"] * 1e-3) / 1e12
                                      for n in ("qkv", "o_proj", "gate_up", "down", "attn")}}
        log(f"k={k:2d}: GEMM {line['gemm_tflops']:.0f} TFLOP/s, attention {line['attn_tflops']:.0f} TFLOP/s")
        print(json.dumps(line), flush=True)
        model.close()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    if args.pmc_record:
        write_pmc_record(args)
        return
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.forwards))
        return
    if args.pmc_summary:
        print(pmc_markdown(args.workload))
        return
    import torch

    if args.copy_calibration:
        a = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied {a.numel() * 4} bytes x3")
        return
    dev = torch.device("cuda:0")
    if args.all_workloads:
        all_workloads(args, dev)
    elif args.logit_drift:
        logit_drift(args, dev)
    elif args.full_attention:
        full_attention(args, dev)
    elif args.batch_sweep:
        batch_sweep(args, dev)
    elif args.backward:
        backward_bench(args, dev)
    elif args.group_sweep:
        group_sweep(args, dev)
    else:
        headline(args, dev)


if __name__ == "__main__":
    main()
