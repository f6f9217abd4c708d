"""Full-size GPU parity: the five benchmark workloads at their real shapes, run
through the C ABI in the launch configuration the benchmark times (diagonal
schedule, graphs on, the library's own GEMM tile choice).

The oracle cannot run a whole 131,072-token forward, so it checks outputs it
can compute one by one:

* every segment-token row of segment 0 through all layers and the per-layer
  state after segment 0 (a GPU run with S = 1), starting from a non-zero
  state so the memory read is exercised;
* prefix rows of segment 1 through all layers from the oracle's own state
  after segment 0 (the recurrence across segments at every layer);
* for the larger 3B segmentations, prefix rows of segment 0 and the layer-0
  state after one full node;
* the LM head over all 131,072 output rows of the 1B run: segment 0's logits
  end to end, and sampled rows of the last segment through the head alone.

Causal attention makes the first r rows of a node independent of the rest, so
prefix rows are exact samples (oracle ``Oracle.node(..., rows=r)``).
At any size, properties that must hold exactly: diagonal == sequential
bitwise; a shorter sequence gives a bitwise prefix of a longer one's output
(the schedule is a reordering of the same recurrence: Pith review of arXiv
2506.05229, "What carries the argument"); all outputs finite.
"""

import gc
import sys
import time

import numpy as np
import pytest
import torch

import oracle
from armt_inputs import get_config, make_head, make_inputs, make_state

from gpu_util import build_model, rel_l2, state_to_device, to_device, to_np, tol

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]

ROWS = 48          # prefix rows sampled per segment


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _oracle_segment(o, s, A, z, rows=None):
    """Segment s through every layer; A, z lists of per-layer state (updated
    in place when rows is None).  Returns the last layer's output rows."""
    h = o.node_input(s)
    for l in range(len(A)):
        h, An, zn = o.node(l, h, A[l], z[l], rows=rows)
        if rows is None:
            A[l], z[l] = An, zn
    return h


def _check(name, got, ref, bar):
    e = rel_l2(got, ref)
    say(f"  {name}: rel L2 {e:.2e}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert e <= bar, f"{name}: rel L2 {e:.3e} > {bar}"


def _check_state(A_gpu, z_gpu, A_ref, z_ref, A0, z0, bar, layers):
    """The state after segment 0 and, separately, its increment over the
    initial state (the initial state is large, so the update would hide in a
    check of the state alone)."""
    Ag, zg = to_np(A_gpu), to_np(z_gpu)
    Ar, zr = np.stack(A_ref), np.stack(z_ref)
    ls = list(layers)
    _check("A after segment 0", Ag[ls], Ar, bar)
    _check("z after segment 0", zg[ls], zr, bar)
    _check("A increment over segment 0", Ag[ls] - A0[ls], Ar - A0[ls], bar)
    _check("z increment over segment 0", zg[ls] - z0[ls], zr - z0[ls], bar)
    for l in ls[:: max(1, len(ls) // 3)]:
        i = ls.index(l)
        _check(f"A[{l}] increment", Ag[l] - A0[l], Ar[i] - A0[l], bar)


def _run(model, x, S, A0, z0, schedule="diagonal"):
    dA0, dz0 = state_to_device(A0, z0)
    return model.forward(x[:S * model.cfg.seg_len].contiguous(), schedule, dA0, dz0)


def _release(model):
    model.close()
    gc.collect()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# 1B shape: S = 128 (131,072 tokens) and S = 32 share weights and input rows
# ---------------------------------------------------------------------------

def test_1b_fullsize():
    cfg = get_config("1b_s128")
    t0 = time.time()
    inp = make_inputs(cfg)
    A0, z0 = make_state(cfg)
    say(f"[1b] inputs drawn in {time.time() - t0:.1f}s")
    model = build_model(inp)
    x = to_device(inp.x, cfg)
    T, S, L, bar = cfg.seg_len, cfg.n_segments, cfg.n_layers, tol(cfg)

    y128, A128, z128 = _run(model, x, S, A0, z0)
    say("[1b] S=128 diagonal done")
    for t in (y128, A128, z128):
        assert torch.isfinite(t).all()
    ys, As, zs = _run(model, x, S, A0, z0, "sequential")
    assert torch.equal(ys, y128) and torch.equal(As, A128) and torch.equal(zs, z128), \
        "sequential and diagonal differ at S=128"
    del ys, As, zs
    y32, _, _ = _run(model, x, 32, A0, z0)
    assert torch.equal(y32, y128[:32 * T]), "S=32 output is not a prefix of the S=128 output"
    y1, A1, z1 = _run(model, x, 1, A0, z0)
    assert torch.equal(y1, y128[:T])
    say("[1b] schedule properties hold; oracle segment 0 (16 full nodes)")

    o = oracle.Oracle(inp)
    A, z = o.initial_state(A0, z0)
    t0 = time.time()
    h = _oracle_segment(o, 0, A, z)
    say(f"[1b] oracle segment 0 in {time.time() - t0:.1f}s")
    _check("y segment 0 (all rows)", to_np(y1), oracle.round_bf16(h[:T]), bar)
    _check_state(A1, z1, A, z, A0, z0, bar, range(L))
    h1 = _oracle_segment(o, 1, A, z, rows=ROWS)
    _check(f"y segment 1 rows 0..{ROWS - 1}", to_np(y128[T:T + ROWS]), oracle.round_bf16(h1), bar)
    # LM head (V = 32,000) in the benchmark's launch configuration: the
    # logits of all 131,072 rows at once (fp32, 16.8 GB), sampled against the
    # oracle's head on the oracle's own segment-0 rows (end to end) and on the
    # GPU's y rows of the last segment (the head alone)
    w_lm, g = make_head(cfg, gain_std=0.1)
    dw, dg = to_device(w_lm, cfg), to_device(g, cfg)
    lg = model.logits(y128, dg, dw)
    assert torch.isfinite(lg).all()
    _check("logits segment 0 (all rows, end to end)", to_np(lg[:T]),
           oracle.logits(oracle.round_bf16(h[:T]), g, w_lm, "bf16", cfg.rms_eps), bar)
    last = slice((S - 1) * T, (S - 1) * T + ROWS)
    _check(f"logits segment {S - 1} rows 0..{ROWS - 1} (head only)", to_np(lg[last]),
           oracle.logits(to_np(y128[last]), g, w_lm, "bf16", cfg.rms_eps), bar)
    del lg
    del x, y1, A1, z1
    _release(model)


# ---------------------------------------------------------------------------
# 3B shape: 65,536 tokens as 128 x 512, 64 x 1024, 32 x 2048 (same weights)
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def inputs_3b():
    cfg = get_config("3b_t512")
    t0 = time.time()
    inp = make_inputs(cfg)
    say(f"[3b] inputs drawn in {time.time() - t0:.1f}s")
    yield inp
    del inp
    gc.collect()


@pytest.mark.parametrize("name", ["3b_t512", "3b_t1024", "3b_t2048"])
def test_3b_fullsize(inputs_3b, name):
    cfg = get_config(name)
    inp = inputs_3b
    # same weights and token rows; only the segmentation differs
    assert inp.x.shape == (cfg.n_segments * cfg.seg_len, cfg.d_model)
    inp = type(inp)(cfg, inp.x, inp.mem_emb, inp.weights, inp.g_attn, inp.g_mlp)
    A0, z0 = make_state(cfg)
    model = build_model(inp)
    x = to_device(inp.x, cfg)
    T, S, bar = cfg.seg_len, cfg.n_segments, tol(cfg)

    y, A_, z_ = _run(model, x, S, A0, z0)
    say(f"[{name}] S={S} diagonal done")
    for t in (y, A_, z_):
        assert torch.isfinite(t).all()
    ys, As, zs = _run(model, x, S, A0, z0, "sequential")
    assert torch.equal(ys, y) and torch.equal(As, A_) and torch.equal(zs, z_), \
        "sequential and diagonal differ"
    del ys, As, zs
    y1, A1, z1 = _run(model, x, 1, A0, z0)
    assert torch.equal(y1, y[:T])

    o = oracle.Oracle(inp)
    A, z = o.initial_state(A0, z0)
    t0 = time.time()
    if name == "3b_t512":
        h = _oracle_segment(o, 0, A, z)
        say(f"[{name}] oracle segment 0 in {time.time() - t0:.1f}s")
        _check("y segment 0 (all rows)", to_np(y1), oracle.round_bf16(h[:T]), bar)
        _check_state(A1, z1, A, z, A0, z0, bar, range(cfg.n_layers))
        h1 = _oracle_segment(o, 1, A, z, rows=ROWS)
        _check(f"y segment 1 rows 0..{ROWS - 1}", to_np(y[T:T + ROWS]), oracle.round_bf16(h1), bar)
    else:
        h = _oracle_segment(o, 0, A, z, rows=ROWS)
        say(f"[{name}] oracle segment 0 prefix in {time.time() - t0:.1f}s")
        _check(f"y segment 0 rows 0..{ROWS - 1}", to_np(y[:ROWS]), oracle.round_bf16(h), bar)
        _, Al, zl = o.node(0, o.node_input(0), A[0], z[0])
        _check_state(A1, z1, [Al], [zl], A0, z0, bar, [0])
    del x, y1, A1, z1
    _release(model)
