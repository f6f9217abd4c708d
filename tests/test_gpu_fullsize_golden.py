"""Full-length GPU parity against the oracle: the benchmark workloads run from
the zero state through every segment (diagonal schedule, captured graphs, the
library's own GEMM tile choice -- the launch configuration the benchmark
times) and compared with the float64 oracle's results for the same seeded
inputs, stored by tests/golden/make_fullsize.py (which calls only the oracle
and the input generator):

* output rows 0..47 of the middle and of the last segment;
* a sketch y_s R_sk [T, 2] of every segment's whole output (R_sk a fixed
  Gaussian matrix from the input generator), so every output row of every
  segment takes part;
* every layer's final memory state: every 16th row of A_l, A_l^T R_sk (every
  element), the Frobenius norm of A_l, and z_l;
* for the 32-segment 1B workload, the LM-head logits of the last segment's
  sampled rows end to end (the GPU's own y through the GPU head against the
  oracle's y through the oracle's head) -- the pages' drift measurement at
  32,768 tokens (skill page "Diagonal Batching for Recurrent Memory
  Transformers", the results after Practical Guidance; Pith review, referee
  report on Table 2).

The bar is the stated one for bf16 workloads: relative L2 <= 2e-2 on the
sampled rows, on every segment's output sketch, on all segments together and
on the state of every layer and of all layers together -- or twice the
oracle's own spread there where that exceeds the bar: the distance between
the stored oracle run and the same oracle rerun with a 3e-6 relative jitter
before every rounding, an equally valid accumulation order
(make_fullsize.py --spread-full; pooled over segments or layers for the
aggregate checks).  The schedule is a reordering of the same
recurrence (Pith review of arXiv 2506.05229, "What carries the argument"),
so the last segments carry the full depth of the recurrence.
"""

import gc
import json
import os
import sys
import time

import numpy as np
import pytest
import torch

import oracle
from armt_inputs import get_config, make_head, make_inputs, make_sketch

from gpu_util import build_model, rel_l2, to_device, to_np, tol

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
WORKLOADS = ["1b_s32", "1b_s128", "3b_t512", "3b_t1024", "3b_t2048"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _check(name, got, ref, bar, results):
    e = rel_l2(got, ref)
    results[name] = e
    say(f"  {name}: rel L2 {e:.2e} (bound {bar:.2e})")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert e <= bar, f"{name}: rel L2 {e:.3e} > {bar}"


def _pooled_spread(spreads, refs):
    """The oracle's spread over several parts together (relative L2 of the
    concatenation), from each part's relative spread and its reference."""
    num = sum((float(sp) * np.linalg.norm(r)) ** 2 for sp, r in zip(spreads, refs))
    den = sum(np.linalg.norm(r) ** 2 for r in refs)
    return float(np.sqrt(num / den))


@pytest.mark.parametrize("name", WORKLOADS)
def test_fullsize_against_oracle(name):
    path = os.path.join(GOLDEN, f"fullsize_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} has not been written (tests/golden/make_fullsize.py)")
    g = np.load(path, allow_pickle=False)
    cfg = get_config(name)
    S, T, L, bar = cfg.n_segments, cfg.seg_len, cfg.n_layers, tol(cfg)
    assert int(g["n_segments"]) == S
    t0 = time.time()
    inp = make_inputs(cfg)
    say(f"[{name}] inputs drawn in {time.time() - t0:.1f}s")
    model = build_model(inp)
    x = to_device(inp.x, cfg)
    y, A, z = model.forward(x, "diagonal")
    torch.cuda.synchronize()
    say(f"[{name}] diagonal forward of {S} segments done")
    assert torch.isfinite(y).all() and torch.isfinite(A).all() and torch.isfinite(z).all()
    res = {}

    # sampled rows of the middle and the last segment
    rows = _bits_to_f64(g["rows"])
    for i, s in enumerate(g["rows_seg"]):
        s = int(s)
        _check(f"y segment {s} rows 0..{rows.shape[1] - 1}", to_np(y[s * T:s * T + rows.shape[1]]), rows[i],
               bar, res)
    # every segment through the sketch (fp32 product on the device; its own
    # rounding is ~1e-6, far inside the bar)
    sk = torch.from_numpy(make_sketch(cfg)).to(y.device)
    ysk = (y.float() @ sk).double().cpu().numpy().reshape(S, T, -1)
    ref_sk = g["sketch"].astype(np.float64)
    per_seg = np.array([rel_l2(ysk[s], ref_sk[s]) for s in range(S)])
    res["sketch per segment max"] = float(per_seg.max())
    say(f"  sketch of every segment: max rel L2 {per_seg.max():.2e} (segment {int(per_seg.argmax())}), "
        f"first {per_seg[0]:.2e}, last {per_seg[-1]:.2e}")
    # Each segment within the bar -- or, for the first segments, within twice
    # the oracle's own spread where that exceeds it: the stored "spread" is
    # how far the same oracle moves under a 3e-6 relative jitter before every
    # rounding (an equally valid accumulation order); the first segments
    # after the zero state are the most sensitive to it, and one can move by
    # more than the bar (3b_t1024 segment 3: 2.6e-2).
    spread = g["spread"] if "spread" in g else np.zeros(0)
    if len(spread):
        say("  oracle spread of the first segments: " + " ".join(f"{v:.2e}" for v in spread))
    for s_ in range(S):
        bound = max(bar, 2.0 * spread[s_]) if s_ < len(spread) else bar
        assert per_seg[s_] <= bound, f"segment {s_}: sketch rel L2 {per_seg[s_]:.3e} > {bound:.3e}"
    # all segments together: the bar, or twice the oracle's pooled spread
    # where the spread of every segment is stored
    agg = bar
    if len(spread) == S:
        agg = max(bar, 2.0 * _pooled_spread(spread, ref_sk))
    _check("sketch of all segments", ysk, ref_sk, agg, res)
    del ysk

    # final memory state of every layer
    An, zn = to_np(A), to_np(z)
    a_rows = g["A_rows"].astype(np.float64)
    stride = An.shape[1] // a_rows.shape[1]
    z_ref = g["z"].astype(np.float64)
    a_bound, z_bound = bar, bar
    if "spread_A_rows" in g:
        a_bound = max(bar, 2.0 * _pooled_spread(g["spread_A_rows"], a_rows))
        z_bound = max(bar, 2.0 * _pooled_spread(g["spread_z"], z_ref))
    _check("A every 16th row (all layers)", An[:, ::stride], a_rows, a_bound, res)
    _check("z (all layers)", zn, z_ref, z_bound, res)
    # every layer's state: within the bar, or within twice the oracle's own
    # spread for that layer where that exceeds the bar (stored spread_*)
    a_sk = np.einsum("ldk,dw->lkw", An, make_sketch(cfg).astype(np.float64))
    per_layer = {
        "A_rows": [rel_l2(An[l, ::stride], a_rows[l]) for l in range(L)],
        "A_sketch": [rel_l2(a_sk[l], g["A_sketch"][l]) for l in range(L)],
        "z": [rel_l2(zn[l], g["z"][l]) for l in range(L)],
    }
    for key, errs in per_layer.items():
        sp = g[f"spread_{key}"] if f"spread_{key}" in g else np.zeros(L)
        worst = int(np.argmax(errs))
        res[f"{key} worst layer"] = float(errs[worst])
        say(f"  {key} per layer: worst layer {worst} rel L2 {errs[worst]:.2e} (oracle spread there "
            f"{sp[worst]:.2e}), median {float(np.median(errs)):.2e}")
        for l in range(L):
            bound = max(bar, 2.0 * float(sp[l]))
            assert np.isfinite(errs[l]) and errs[l] <= bound, \
                f"layer {l} {key}: rel L2 {errs[l]:.3e} > {bound:.3e} (oracle spread {sp[l]:.3e})"
    # the Frobenius norm moves by at most the relative L2 of the whole state,
    # whose oracle spread the sampled rows' spread stands for
    norm_err = np.abs(np.linalg.norm(An.reshape(L, -1), axis=1) / g["A_norm"] - 1.0)
    res["A norm max rel diff"] = float(norm_err.max())
    say(f"  Frobenius norm of A_l: max rel diff {norm_err.max():.2e} (layer {int(norm_err.argmax())})")
    sp_rows = g["spread_A_rows"] if "spread_A_rows" in g else np.zeros(L)
    for l in range(L):
        bound = max(bar, 2.0 * float(sp_rows[l]))
        assert norm_err[l] <= bound, f"layer {l}: Frobenius norm rel diff {norm_err[l]:.3e} > {bound:.3e}"

    if name == "1b_s32":
        # logits of the last segment's sampled rows, end to end
        w_lm, gf = make_head(cfg, gain_std=0.1)
        s_last = int(g["rows_seg"][-1])
        nrow = rows.shape[1]
        lg = model.logits(y[s_last * T:s_last * T + nrow].contiguous(), to_device(gf, cfg), to_device(w_lm, cfg))
        ref = oracle.logits(rows[-1], gf, w_lm, "bf16", cfg.rms_eps)
        _check(f"logits segment {s_last} rows 0..{nrow - 1} (32,768 tokens, end to end)", to_np(lg), ref, bar, res)
        agree = float(np.mean(to_np(lg).argmax(1) == ref.argmax(1)))
        say(f"  argmax agreement {agree:.3f}")
    say(f"[{name}] " + json.dumps({k: float(f"{v:.3e}") for k, v in res.items()}))
    model.close()
    del model, x, y, A, z, inp
    gc.collect()
    torch.cuda.empty_cache()
