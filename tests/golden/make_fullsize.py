"""Write the oracle's full-length reference samples for the benchmark workloads.

    python tests/golden/make_fullsize.py 1b          # 1b_s128, and 1b_s32 as its first 32 segments
    python tests/golden/make_fullsize.py 3b_t512     # (also 3b_t1024, 3b_t2048)

Test infrastructure: this script calls only ``oracle/`` (the float64 CPU
oracle) and ``armt_inputs/`` (the seeded input generator).  It runs every node
of the (segment, layer) grid from the zero memory state (the workloads'
stated initial state), in wave order -- the diagonal order, which the oracle's
own tests show gives results bitwise equal to the segment-major order -- with
the independent nodes of a wave spread over worker processes.  Each worker
calls ``oracle.Oracle.node``; nothing here does the model's arithmetic.

What it keeps (``tests/golden/fullsize_<workload>.npz``), for a GPU run to
be compared against:

* ``rows_seg`` / ``rows``: output rows 0..ROWS-1 of the middle and the last
  segment (bf16 bit patterns: the oracle's output is rounded to bf16);
* ``sketch``: every segment's whole output summarised as y_s R_sk [T, 2]
  (R_sk from ``armt_inputs.make_sketch``), so every output row is covered;
* ``A_rows``: every 16th row of each layer's final A_l; ``A_sketch``:
  A_lᵀ R_sk per layer (covers every element); ``z``: every layer's final z_l;
* ``A_norm``: the Frobenius norm of every A_l.

A JSON sidecar records the command, the SHA-256 of the oracle and input
sources it ran, the host and the wall time.  ``--spread-full`` reruns the
workload with the same oracle under a 3e-6 relative jitter before every
rounding (an equally valid accumulation order, seeded per node) and adds how
far that run lands from the stored one -- per segment (``spread``) and per
layer of the final state (``spread_A_rows``, ``spread_A_sketch``,
``spread_z``): how closely any implementation that is not bitwise the oracle
can be expected to agree.  (``--spread N`` does the same for the first N
segments only, in one process.)  Progress is checkpointed (under
``--ckpt``, default /tmp/armt_fullsize_ckpt) so an interrupted run resumes.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))

ROWS = 48           # output rows kept per sampled segment
A_STRIDE = 16       # every A_STRIDE-th row of each A_l is kept

RUNS = {            # run name -> (workload drawn, workloads written with their segment count)
    "1b": ("1b_s128", [("1b_s32", 32), ("1b_s128", 128)]),
    "3b_t512": ("3b_t512", [("3b_t512", 128)]),
    "3b_t1024": ("3b_t1024", [("3b_t1024", 64)]),
    "3b_t2048": ("3b_t2048", [("3b_t2048", 32)]),
}

_O = None           # the oracle object (the main process's, or each worker's)
_SHM = []           # shared-memory segments a worker has attached


def sha256(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def source_digests() -> dict:
    return {rel: sha256(os.path.join(ROOT, rel))
            for rel in ("oracle/armt_oracle.py", "armt_inputs/__init__.py")}


JITTER_EPS = 3e-6
JITTER_SEED = 123
_JIT = None         # (R, Rs) of the oracle object before jitter wrappers, when jittering
_JRNG = None        # random stream of the node being run (jitter mode)


def _set_jitter(o):
    """Wrap the oracle's two rounding functions so that every value is
    multiplied by (1 + JITTER_EPS * N(0, 1)) just before it is rounded -- an
    equally valid order of the fp32 accumulations.  The random stream is
    reset per node (seeded by the node's (segment, layer)), so results do not
    depend on which worker runs which node."""
    global _JIT
    import numpy as np
    _JIT = (o.R, o.Rs)

    def jitter(f):
        def g(x):
            x = np.asarray(x, dtype=np.float64)
            return f(x * (1.0 + JITTER_EPS * _JRNG.standard_normal(x.shape)))
        return g

    o.R, o.Rs = jitter(o.R), jitter(o.Rs)


def _node(job):
    global _JRNG
    s, l, h, A, z = job[:5]
    if _JIT is not None:
        import numpy as np
        _JRNG = np.random.default_rng([JITTER_SEED, s, l])
    if h is None:
        h = _O.node_input(s)
    return _O.node(l, h, A, z)


def _share(inputs, release):
    """Move the input arrays into shared memory so spawned workers map them
    instead of holding copies.  Returns (segments to keep alive, a picklable
    description the workers rebuild the inputs from)."""
    from multiprocessing import shared_memory

    import numpy as np

    keep, desc = [], {}

    def put(key, a):
        a = np.ascontiguousarray(a)
        shm = shared_memory.SharedMemory(create=True, size=max(a.nbytes, 1))
        np.ndarray(a.shape, a.dtype, buffer=shm.buf)[...] = a
        keep.append(shm)
        desc[key] = (shm.name, a.shape, a.dtype.str)

    put("x", inputs.x)
    put("mem_emb", inputs.mem_emb)
    put("g_attn", inputs.g_attn)
    put("g_mlp", inputs.g_mlp)
    for name in list(inputs.weights):
        put("w:" + name, inputs.weights[name])
        if release:
            inputs.weights[name] = None      # drop the caller's copy as soon as it is shared
    return keep, (inputs.cfg, desc)


def _attach(shared, jitter=False):
    """Worker initializer: rebuild the inputs over the shared arrays."""
    from multiprocessing import shared_memory

    import numpy as np

    import oracle
    from armt_inputs import ArmtInputs

    global _O, _SHM
    cfg, desc = shared
    _SHM, arrays = [], {}
    for key, (name, shape, dt) in desc.items():
        shm = shared_memory.SharedMemory(name=name)
        _SHM.append(shm)
        arrays[key] = np.ndarray(shape, np.dtype(dt), buffer=shm.buf)
    weights = {k[2:]: v for k, v in arrays.items() if k.startswith("w:")}
    _O = oracle.Oracle(ArmtInputs(cfg, arrays["x"], arrays["mem_emb"], weights,
                                  arrays["g_attn"], arrays["g_mlp"]))
    if jitter:
        _set_jitter(_O)


def run_waves(inputs, workers: int, on_output, ckpt_path: str | None = None, n_segments=None,
              snap_after=(), log=print, release=False, jitter=False):
    """Run the oracle's nodes wave by wave from the zero state; call
    ``on_output(s, y_s)`` with each segment's output rows y_s = R(h[:T]) of
    the last layer.  Returns the final (A, z) lists and a dict
    {k: (A, z)} of the state after the first k segments for each k in
    ``snap_after`` (layer l's state after segment k - 1 is its state once
    node (k - 1, l) has run).  With ``ckpt_path`` the pending activations and
    state are saved every few waves and a matching checkpoint is resumed.
    ``release`` lets the runner drop the caller's weight arrays once they are
    in shared memory (the caller must not use ``inputs`` afterwards)."""
    import multiprocessing as mp

    import numpy as np

    import oracle

    global _O, _JIT
    cfg = inputs.cfg
    _O = oracle.Oracle(inputs)
    _JIT = None
    if jitter:
        _set_jitter(_O)
    T = cfg.seg_len
    L = inputs.weights["w_qkv"].shape[0]
    S = n_segments or inputs.x.shape[0] // cfg.seg_len
    T = cfg.seg_len
    A, z = _O.initial_state()
    pending = {}                 # (s, l) -> output h of node (s, l), awaiting (s, l + 1)
    snaps = {k: ([None] * L, [None] * L) for k in snap_after}
    start = 0
    if ckpt_path and os.path.exists(ckpt_path):
        ck = np.load(ckpt_path, allow_pickle=False)
        if int(ck["S"]) == S and int(ck["L"]) == L and str(ck["digest"]) == json.dumps(source_digests()):
            start = int(ck["wave"])
            A = [ck["A"][l].astype(np.float64) for l in range(L)]
            z = [ck["z"][l].astype(np.float64) for l in range(L)]
            for key in ck["pending_keys"]:
                s, l = int(key[0]), int(key[1])
                pending[(s, l)] = ck[f"h_{s}_{l}"]
            log(f"resumed at wave {start} of {S + L - 1}")
    pool, shm = None, []
    if workers > 1:
        # spawned workers (a forked child of a process that has run torch's
        # or OpenBLAS's thread pools can deadlock) over shared input arrays
        shm, shared = _share(inputs, release)
        pool = mp.get_context("spawn").Pool(workers, initializer=_attach, initargs=(shared, jitter))
    t0 = time.time()
    try:
        for i, wave in enumerate(oracle.waves(L, S)):
            if i < start:
                continue
            jobs = [(s, l, None if l == 0 else pending.pop((s, l - 1)), A[l], z[l]) for (s, l) in wave]
            results = pool.map(_node, jobs, chunksize=1) if pool else [_node(j) for j in jobs]
            for (s, l), (h, An, zn) in zip(wave, results):
                A[l], z[l] = An, zn
                if s + 1 in snaps:
                    snaps[s + 1][0][l], snaps[s + 1][1][l] = An, zn
                if l == L - 1:
                    on_output(s, (_JIT[0] if _JIT else _O.R)(h[:T]))
                else:
                    pending[(s, l)] = h
            done = i + 1
            if done % 4 == 0 or done == S + L - 1:
                el = time.time() - t0
                log(f"wave {done}/{S + L - 1}  {el:.0f}s", flush=True)
            if ckpt_path and (done % 8 == 0) and done < S + L - 1:
                _save_ckpt(ckpt_path, S, L, done, A, z, pending, snaps, on_output)
    finally:
        if pool:
            pool.close()
            pool.join()
        for seg in shm:
            seg.close()
            seg.unlink()
    return A, z, snaps


def _save_ckpt(path, S, L, wave, A, z, pending, snaps, on_output):
    import numpy as np
    arrays = {"S": S, "L": L, "wave": wave, "digest": json.dumps(source_digests()),
              "A": np.stack(A), "z": np.stack(z),
              "pending_keys": np.array(sorted(pending), dtype=np.int64).reshape(-1, 2)}
    for (s, l), h in pending.items():
        arrays[f"h_{s}_{l}"] = h
    for k, (As, zs) in snaps.items():
        for l in range(L):
            if As[l] is not None:
                arrays[f"snapA_{k}_{l}"] = As[l]
                arrays[f"snapz_{k}_{l}"] = zs[l]
    extra = getattr(on_output, "state", None)
    if extra is not None:
        arrays.update(extra())
    tmp = path + ".tmp.npz"
    np.savez(tmp, **arrays)
    os.replace(tmp, path)


class Collector:
    """Keeps what the golden files hold from each segment's output rows."""

    def __init__(self, cfg, S, sample_segments, sketch):
        import numpy as np
        self.sk = np.asarray(sketch, dtype=np.float64)
        self.sketch = np.zeros((S, cfg.seg_len, self.sk.shape[1]), dtype=np.float32)
        self.sample_segments = sorted(set(sample_segments))
        self.rows = {}
        self.seen = np.zeros(S, dtype=bool)

    def __call__(self, s, y):
        import numpy as np
        self.sketch[s] = (y @ self.sk).astype(np.float32)
        if s in self.sample_segments:
            self.rows[s] = bf16_bits(y[:ROWS])
        self.seen[s] = True

    def state(self):
        import numpy as np
        out = {"col_sketch": self.sketch, "col_seen": self.seen}
        for s, r in self.rows.items():
            out[f"col_rows_{s}"] = r
        return out

    def restore(self, path):
        import numpy as np
        if not os.path.exists(path):
            return
        ck = np.load(path, allow_pickle=False)
        if "col_sketch" in ck and ck["col_sketch"].shape == self.sketch.shape:
            self.sketch[:] = ck["col_sketch"]
            self.seen[:] = ck["col_seen"]
            for s in self.sample_segments:
                if f"col_rows_{s}" in ck:
                    self.rows[s] = ck[f"col_rows_{s}"]


def bf16_bits(y):
    """Bit patterns of values that are exactly bf16 (the oracle rounded them)."""
    import numpy as np
    b = np.asarray(y, dtype=np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "output rows are not bf16 values"
    return (b >> 16).astype(np.uint16)


def write_golden(path, S, segs, col, A, z, sketch, meta):
    import numpy as np
    A = np.stack(A).astype(np.float32)              # the oracle stores the state in float32
    z = np.stack(z).astype(np.float32)
    assert col.seen[:S].all(), "not every segment produced its output"
    np.savez_compressed(
        path,
        n_segments=np.int64(S),
        rows_seg=np.array(segs, dtype=np.int64),
        rows=np.stack([col.rows[s] for s in segs]),
        sketch=col.sketch[:S],
        A_rows=A[:, ::A_STRIDE, :],
        A_sketch=np.einsum("ldk,dw->lkw", A.astype(np.float64), np.asarray(sketch, np.float64)).astype(np.float32),
        A_norm=np.linalg.norm(A.astype(np.float64).reshape(A.shape[0], -1), axis=1),
        z=z,
    )
    with open(path[:-4] + ".json", "w") as f:
        json.dump(meta, f, indent=1)
        f.write("\n")


def self_spread(inputs, n_segments, eps=3e-6, seed=123, log=print):
    """The oracle's own sensitivity to rounding order: the same oracle with
    every stored value multiplied by (1 + eps * N(0, 1)) just before it is
    rounded -- an equally valid order of the fp32 accumulations, eps about
    the relative error of a long fp32 sum -- run from the zero state through
    the first ``n_segments`` segments.  Returns each segment's output rows
    (R(h[:T]) of the last layer); a GPU result cannot be expected to agree
    with the float64 oracle more closely than this run does."""
    import numpy as np

    import oracle

    o = oracle.Oracle(inputs)
    rng = np.random.default_rng(seed)
    R, Rs = o.R, o.Rs

    def jitter(f):
        def g(x):
            x = np.asarray(x, dtype=np.float64)
            return f(x * (1.0 + eps * rng.standard_normal(x.shape)))
        return g

    o.R, o.Rs = jitter(R), jitter(Rs)
    A, z = o.initial_state()
    T, L = inputs.cfg.seg_len, inputs.weights["w_qkv"].shape[0]
    out = []
    for s in range(n_segments):
        t0 = time.time()
        h = o.node_input(s)
        for l in range(L):
            h, A[l], z[l] = o.node(l, h, A[l], z[l])
        out.append(R(h[:T]))
        log(f"spread: segment {s} in {time.time() - t0:.0f}s", flush=True)
    return out


def add_spread(name, n_segments, out_dir):
    """Store, in an existing golden file, the relative L2 between the
    jittered oracle's sketch and the stored sketch for its first segments."""
    import numpy as np
    from armt_inputs import get_config, make_inputs, make_sketch
    path = os.path.join(out_dir, f"fullsize_{name}.npz")
    g = dict(np.load(path, allow_pickle=False))
    cfg = get_config(name)
    inp = make_inputs(cfg, n_segments=n_segments)
    sk = make_sketch(cfg).astype(np.float64)
    ys = self_spread(inp, n_segments)
    spread = np.array([np.linalg.norm(y @ sk - g["sketch"][s]) / np.linalg.norm(g["sketch"][s])
                       for s, y in enumerate(ys)])
    g["spread"] = spread
    np.savez_compressed(path, **g)
    with open(path[:-4] + ".json") as f:
        meta = json.load(f)
    meta["spread"] = {"segments": n_segments, "eps": 3e-6, "seed": 123, "sketch_rel_l2": [float(v) for v in spread],
                      "command": f"python tests/golden/make_fullsize.py {name} --spread {n_segments}"}
    with open(path[:-4] + ".json", "w") as f:
        json.dump(meta, f, indent=1)
        f.write("\n")
    print(f"[{name}] spread of the first {n_segments} segments: {np.array2string(spread, precision=4)}", flush=True)


def add_spread_full(run, workers, out_dir, ckpt_dir):
    """Run a whole workload (or the 1B pair) again with the jittered oracle
    and store, in each of its golden files, how far that run lands from the
    stored one: per segment (sketch relative L2, ``spread``), and per layer
    for the final state (``spread_A_rows``, ``spread_A_sketch``,
    ``spread_z``)."""
    import numpy as np
    from armt_inputs import get_config, make_inputs, make_sketch
    drawn, outputs = RUNS[run]
    cfg = get_config(drawn)
    S = cfg.n_segments
    inp = make_inputs(cfg)
    sk64 = make_sketch(cfg).astype(np.float64)
    sketches = np.zeros((S, cfg.seg_len, sk64.shape[1]))

    def on_output(s, y):
        sketches[s] = y @ sk64

    t0 = time.time()
    A, z, snaps = run_waves(inp, workers, on_output, os.path.join(ckpt_dir, f"{run}_jitter.npz"),
                            snap_after=[s_out for _, s_out in outputs if s_out < S], release=True, jitter=True)
    wall = time.time() - t0

    def rel(a, b):
        return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))

    for name, s_out in outputs:
        path = os.path.join(out_dir, f"fullsize_{name}.npz")
        g = dict(np.load(path, allow_pickle=False))
        A_out, z_out = (A, z) if s_out == S else snaps[s_out]
        Aj = np.stack(A_out).astype(np.float32).astype(np.float64)
        zj = np.stack(z_out).astype(np.float32).astype(np.float64)
        L = Aj.shape[0]
        g["spread"] = np.array([rel(sketches[s], g["sketch"][s]) for s in range(s_out)])
        g["spread_A_rows"] = np.array([rel(Aj[l, ::A_STRIDE], g["A_rows"][l]) for l in range(L)])
        g["spread_A_sketch"] = np.array([rel(Aj[l].T @ sk64, g["A_sketch"][l]) for l in range(L)])
        g["spread_z"] = np.array([rel(zj[l], g["z"][l]) for l in range(L)])
        np.savez_compressed(path, **g)
        with open(path[:-4] + ".json") as f:
            meta = json.load(f)
        meta["spread"] = {"eps": JITTER_EPS, "seed": JITTER_SEED, "segments": s_out,
                          "max_segment": float(g["spread"].max()),
                          "max_layer_A_rows": float(g["spread_A_rows"].max()),
                          "max_layer_A_sketch": float(g["spread_A_sketch"].max()),
                          "max_layer_z": float(g["spread_z"].max()),
                          "command": f"python tests/golden/make_fullsize.py {run} --spread-full",
                          "wall_s": round(wall, 1)}
        with open(path[:-4] + ".json", "w") as f:
            json.dump(meta, f, indent=1)
            f.write("\n")
        print(f"[{name}] spread: segments max {g['spread'].max():.3e}, A rows max {g['spread_A_rows'].max():.3e}, "
              f"A sketch max {g['spread_A_sketch'].max():.3e}, z max {g['spread_z'].max():.3e}", flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("run", choices=sorted(RUNS) + ["1b_s32", "1b_s128"])
    ap.add_argument("--spread-full", action="store_true",
                    help="instead: rerun the whole workload with the jittered oracle and add its distance "
                         "from the stored run (per segment and per layer) to the golden files")
    ap.add_argument("--spread", type=int, default=0,
                    help="instead: add the jittered oracle's spread over the first N segments to an "
                         "existing golden file of this workload")
    ap.add_argument("--workers", type=int, default=4, help="worker processes (nodes of a wave in parallel)")
    ap.add_argument("--blas-threads", type=int, default=2, help="BLAS threads per worker")
    ap.add_argument("--ckpt", default="/tmp/armt_fullsize_ckpt")
    ap.add_argument("--out", default=HERE)
    args = ap.parse_args(argv)
    for var in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = str(args.blas_threads)
    sys.path.insert(0, ROOT)
    if args.spread:
        add_spread(args.run, args.spread, args.out)
        return
    if args.spread_full:
        os.makedirs(args.ckpt, exist_ok=True)
        add_spread_full(args.run, args.workers, args.out, args.ckpt)
        return
    from armt_inputs import get_config, make_inputs, make_sketch

    drawn, outputs = RUNS[args.run]
    cfg = get_config(drawn)
    S = cfg.n_segments
    t0 = time.time()
    inp = make_inputs(cfg)
    sketch = make_sketch(cfg)
    print(f"[{args.run}] inputs drawn in {time.time() - t0:.1f}s", flush=True)
    samples = []
    for _, s_out in outputs:
        samples += [s_out // 2, s_out - 1]
    col = Collector(cfg, S, samples, sketch)
    os.makedirs(args.ckpt, exist_ok=True)
    ckpt = os.path.join(args.ckpt, f"{args.run}.npz")
    col.restore(ckpt)

    def on_output(s, y):
        col(s, y)

    on_output.state = col.state
    t_run = time.time()
    A, z, snaps = run_waves(inp, args.workers, on_output, ckpt,
                            snap_after=[s_out for _, s_out in outputs if s_out < S], release=True)
    wall = time.time() - t_run
    host = {"cpu": platform.processor() or platform.machine(), "cpu_count": os.cpu_count(),
            "workers": args.workers, "blas_threads": args.blas_threads}
    digests = source_digests()
    for name, s_out in outputs:
        A_out, z_out = (A, z) if s_out == S else snaps[s_out]
        meta = {"workload": name, "n_segments": s_out, "drawn_as": drawn, "seed": 0,
                "initial_state": "zero", "rows_per_sample": ROWS, "A_row_stride": A_STRIDE,
                "sampled_segments": [s_out // 2, s_out - 1],
                "command": f"python tests/golden/make_fullsize.py {args.run}",
                "sources_sha256": digests, "host": host, "wall_s_full_run": round(wall, 1)}
        write_golden(os.path.join(args.out, f"fullsize_{name}.npz"), s_out, [s_out // 2, s_out - 1],
                     col, A_out, z_out, sketch, meta)
        print(f"[{args.run}] wrote fullsize_{name}.npz", flush=True)
    if os.path.exists(ckpt):
        os.remove(ckpt)


if __name__ == "__main__":
    main()
