"""Benchmark: 131,072-token 1B-shape ARMT forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1b_s128]

A step is one full forward of the workload (all S + L - 1 diagonal waves, every
kernel of every node) over a synthetic sequence that is resident in HBM before
timing starts.  The headline value is tokens/s of the diagonal schedule
(input tokens S*T per forward).  The same number of sequential-schedule
forwards is timed next for the diagonal-vs-sequential ratio the pages quote
(abstract on the paper page: 1.8x at 131,072 tokens, another GPU).

Extra fields:
  roofline      the grouped gate/up GEMM (the largest kernel, about half of all
                FLOPs): algorithmic FLOPs of its launches divided by their
                summed durations, from HIP events recorded around every launch
                on the library's stream during a timed pass, against the bf16
                dense MFMA peak of 2.5 PFLOP/s;
  gemm_util     the same for all four grouped GEMMs together;
  cpu_baseline  the CPU oracle timed on a bounded sample (first nodes of
                segment 0) on this host.
Weights and inputs are random (seeded) of the 1B ARMT shape; no checkpoint.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


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
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import numpy as np
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

    from armt_inputs import get_config, make_inputs
    from long_context_recurrent_amd import armt as C
    from long_context_recurrent_amd.model import ArmtModel, make_config

    cfg = get_config(args.workload)
    dev = torch.device("cuda:0")
    t0 = time.time()
    inp = make_inputs(cfg)
    log(f"inputs drawn in {time.time() - t0:.1f}s")

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev, torch.bfloat16).contiguous()

    w = {k: t(v) for k, v in inp.weights.items()}
    w.update(g_attn=t(inp.g_attn), g_mlp=t(inp.g_mlp), mem_emb=t(inp.mem_emb))
    x = t(inp.x)
    ccfg = make_config(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                       cfg.ffn_hidden, cfg.seg_len, cfg.n_mem, cfg.d_key, cfg.dtype)
    model = ArmtModel(ccfg, w)
    if args.gemm_rows:
        model.set_option(C.ARMT_OPT_GEMM_ROWS, args.gemm_rows)
    S, T, L = cfg.n_segments, cfg.seg_len, cfg.n_layers
    tokens = S * T
    out = model.alloc_outputs(S)
    st = model.stream

    def run(schedule, k):
        fn = C.armt_forward_diagonal if schedule == "diagonal" else C.armt_forward_sequential
        for _ in range(k):
            fn(model.handle, x, S, None, None, out[0], out[1], out[2])

    def timed(schedule, steps, warmup):
        run(schedule, warmup)
        torch.cuda.synchronize()
        st.synchronize()
        a = time.perf_counter()
        run(schedule, steps)
        st.synchronize()
        torch.cuda.synchronize()
        return (time.perf_counter() - a) / steps

    log(f"warmup {args.warmup}, timing {args.steps} diagonal forwards of {args.workload}")
    diag_s = timed("diagonal", args.steps, args.warmup)
    log(f"diagonal: {diag_s * 1e3:.1f} ms/forward, {tokens / diag_s:.0f} tokens/s")
    if args.profile_only:
        return
    seq_s = None
    if not args.no_seq:
        seq_s = timed("sequential", args.steps, 1)
        log(f"sequential: {seq_s * 1e3:.1f} ms/forward, {tokens / seq_s:.0f} tokens/s")

    # per-kernel durations from HIP events on the library's stream
    kstats = {}
    for kname in C.KERNELS:
        kid = C.KERNELS.index(kname)
        model.set_option(C.ARMT_OPT_TIME_KERNEL, kid)
        run("diagonal", max(1, min(args.steps, 3)))
        kstats[kname] = model.kernel_stats()
        model.set_option(C.ARMT_OPT_TIME_KERNEL, -1)
    rk = kstats[args.roofline_kernel]
    achieved = rk["flops"] / (rk["ms"] * 1e-3) / 1e12
    traffic = measured_traffic(args.roofline_kernel, args.workload)
    gemm = [kstats[k] for k in ("qkv", "o_proj", "gate_up", "down")]
    g_flops = sum(k["flops"] for k in gemm)
    g_ms = sum(k["ms"] for k in gemm)
    for k, v in kstats.items():
        tf = v["flops"] / (v["ms"] * 1e-3) / 1e12 if v["ms"] else 0.0
        gbs = v["bytes"] / (v["ms"] * 1e-3) / 1e9 if v["ms"] else 0.0
        log(f"  {k:10s} {v['ms'] / max(v['launches'], 1) * 1e3:9.1f} us/launch  {tf:7.1f} TFLOP/s  {gbs:7.0f} GB/s")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(inp, args.cpu_seconds)

    res = {
        "metric": "tokens/s, 131K-token 1B-shape ARMT forward (diag vs seq); GEMM MFMA util %",
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
        "sequential": None if seq_s is None else {
            "value": tokens / seq_s, "unit": "tokens/s", "ms_per_step": seq_s * 1e3,
            "diag_speedup": seq_s / diag_s},
        "roofline": {"kernel": args.roofline_kernel, "bound": "mfma", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "launches": rk["launches"],
                     "avg_launch_us": rk["ms"] / max(rk["launches"], 1) * 1e3},
        "gemm_util": {"achieved": g_flops / (g_ms * 1e-3) / 1e12, "unit": "TFLOP/s",
                      "frac": g_flops / (g_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "kernels": {k: kernel_summary(v, max(1, min(args.steps, 3))) for k, v in kstats.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    model.close()


def kernel_summary(v, forwards):
    """Per-kernel figures from HIP-event timing: time per forward, algorithmic
    FLOP/s against the bf16 MFMA peak and algorithmic bytes/s against HBM."""
    sec = v["ms"] * 1e-3
    tf = v["flops"] / sec / 1e12 if sec else 0.0
    gbs = v["bytes"] / sec / 1e9 if sec else 0.0
    return {"us_per_forward": v["ms"] * 1e3 / forwards, "launches_per_forward": v["launches"] // forwards,
            "tflops": tf, "frac_mfma_bf16": tf / PEAK_BF16_TFLOPS, "gb_s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS}


TRAFFIC_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {"gate_up": "gemm_bf16.hip", "down": "gemm_bf16.hip", "qkv": "gemm_bf16.hip",
                  "o_proj": "gemm_bf16.hip", "attn": "attention.hip"}


def measured_traffic(kernel, workload):
    """Average HBM bytes per launch of ``kernel`` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE record of this workload, scaled by the copy-kernel
    calibration factors stored with it; None when there is no record or the
    kernel's source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(TRAFFIC_DIR, f"traffic_{kernel}_{workload}.json")
    src = KERNEL_SOURCES.get(kernel)
    if not (src and os.path.exists(path)):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(os.path.join(ROOT, "long_context_recurrent_amd", "csrc", src), "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if rec.get("source_sha256") != digest:
        log(f"traffic record for {kernel} is stale (kernel source changed); reporting null")
        return None
    return (rec["fetch_kib_per_dispatch"] * rec["fetch_factor"]
            + rec["write_kib_per_dispatch"] * rec["write_factor"]) * 1024.0


def cpu_baseline(inp, seconds):
    """The oracle as it stands, on this host: nodes of segment 0, layer by
    layer, until about `seconds` of CPU work; tokens/s = T / (L * mean node
    time), i.e. one segment through every layer."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
    except Exception:
        cores = os.cpu_count()
    cfg = inp.cfg
    o = oracle.Oracle(inp)
    A = np.zeros((cfg.d_model, cfg.d_key))
    z = np.zeros(cfg.d_key)
    h = o.node_input(0)
    done, a = 0, time.perf_counter()
    while done < cfg.n_layers:
        h, _, _ = o.node(done, h, A, z)
        done += 1
        if time.perf_counter() - a > seconds:
            break
    el = time.perf_counter() - a
    per_node = el / done
    value = cfg.seg_len / (per_node * cfg.n_layers)
    log(f"cpu oracle: {done} nodes in {el:.1f}s -> {value:.1f} tokens/s")
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} node(s) of segment 0 (layers 0..{done - 1}, {cfg.seg_len + cfg.n_mem} rows each, "
                      f"float64 NumPy) in {el:.1f}s; tokens/s = T / (L * mean node time)"}


if __name__ == "__main__":
    main()
