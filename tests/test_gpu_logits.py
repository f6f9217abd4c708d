"""GPU parity of the LM head (armt_logits: final RMSNorm + vocabulary
projection, fp32 logits) through the C ABI against the CPU oracle.

The pages compare final logits between the sequential and the diagonal
schedule (Pith review of arXiv 2506.05229: falsifier, and the referee report
on Table 2's relative logit drift).  Here the two schedules give bitwise equal
y, hence bitwise equal logits; against the oracle the bars are those of the
forward (relative L2 1e-4 fp32, 2e-2 bf16).  Shapes cover ragged row and
vocabulary tiles, several workspace chunks (L * (T + M) rows each) and a
non-unit final gain.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from armt_inputs import get_config, make_head, make_inputs
from long_context_recurrent_amd import armt as C

from gpu_util import build_model, rel_l2, to_device, to_np, tol

pytestmark = pytest.mark.gpu

TINY = get_config("tiny_fp32")
SMALL = get_config("small_bf16")
MID64 = SMALL.with_(name="mid_hd64", n_layers=3, d_model=512, n_heads=8, n_kv_heads=2, head_dim=64,
                    ffn_hidden=1536, seg_len=200, n_mem=16, n_segments=5)
MID128 = SMALL.with_(name="mid_hd128", n_layers=3, d_model=768, n_heads=6, n_kv_heads=2, head_dim=128,
                     ffn_hidden=1280, seg_len=120, n_mem=8, n_segments=4)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("cfg,vocab", [(TINY, 100), (SMALL, 1000), (MID64, 1304), (MID128, 520)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_logits_parity(cfg, vocab):
    say(f"[logits] {cfg.name} V={vocab}")
    inp = make_inputs(cfg)
    w_lm, g = make_head(cfg, vocab, gain_std=0.1)
    model = build_model(inp)
    x = to_device(inp.x, cfg)
    yd, _, _ = [t.clone() for t in model.forward(x, "diagonal")]
    ys, _, _ = model.forward(x, "sequential")
    assert torch.equal(yd, ys)
    dw, dg = to_device(w_lm, cfg), to_device(g, cfg)
    ld = model.logits(yd, dg, dw)
    ls = model.logits(ys, dg, dw)
    assert torch.equal(ld, ls), "logits of the two schedules differ"
    rows = yd.shape[0]
    assert ld.shape == (rows, vocab) and ld.dtype == torch.float32
    assert rows > cfg.n_layers * cfg.n, "the test must span several workspace chunks"
    # the head alone, on the GPU's own y
    y_gpu = to_np(yd)
    ref_head = oracle.logits(y_gpu, g, w_lm, cfg.dtype, cfg.rms_eps)
    e_head = rel_l2(to_np(ld), ref_head)
    # the whole path: oracle forward, then the oracle's head
    y_ref, _, _ = oracle.forward_sequential(inp)
    ref_all = oracle.logits(y_ref, g, w_lm, cfg.dtype, cfg.rms_eps)
    e_all = rel_l2(to_np(ld), ref_all)
    say(f"  rel L2 head-only {e_head:.2e}, end to end {e_all:.2e}")
    assert e_head <= tol(cfg) and e_all <= tol(cfg)
    # per-row bar too (no row may hide behind the others)
    lg = to_np(ld)
    for r in range(0, rows, max(1, rows // 16)):
        assert rel_l2(lg[r], ref_head[r]) <= tol(cfg)
    # the normalised rows of the last chunk stay in the workspace
    chunk = cfg.n_layers * cfg.n
    last = rows - (rows - 1) // chunk * chunk
    normed = model.view("normed", shape=(last, cfg.d_model))
    R = oracle.round_bf16 if cfg.dtype == "bf16" else (lambda v: v)
    b_ref = R(oracle.rms_norm(y_gpu[rows - last:], g, cfg.rms_eps))
    assert rel_l2(to_np(normed), b_ref) <= (1e-6 if cfg.dtype == "f32" else 4e-3)


def test_logits_single_row_and_repeat_calls():
    cfg = SMALL.with_(n_segments=2)
    inp = make_inputs(cfg)
    w_lm, g = make_head(cfg, 64)
    model = build_model(inp)
    y, _, _ = model.forward(to_device(inp.x, cfg), "diagonal")
    dw, dg = to_device(w_lm, cfg), to_device(g, cfg)
    full = model.logits(y, dg, dw).clone()
    one = model.logits(y[5:6].contiguous(), dg, dw)
    assert torch.equal(one[0], full[5]), "a row's logits must not depend on the other rows"
    again = model.logits(y, dg, dw)
    assert torch.equal(again, full)


def test_logits_argument_errors():
    cfg = SMALL.with_(n_segments=1)
    inp = make_inputs(cfg)
    model = build_model(inp)
    y, _, _ = model.forward(to_device(inp.x, cfg), "diagonal")
    w_lm, g = make_head(cfg, 64)
    dw, dg = to_device(w_lm, cfg), to_device(g, cfg)
    out = torch.empty(y.shape[0], 64, dtype=torch.float32, device=y.device)
    lib = C.load_library()
    h = model.handle
    assert lib.armt_logits(h, y.data_ptr(), 0, dg.data_ptr(), dw.data_ptr(), 64, out.data_ptr()) == -1
    assert lib.armt_logits(h, y.data_ptr(), y.shape[0], dg.data_ptr(), dw.data_ptr(), 0, out.data_ptr()) == -1
    assert lib.armt_logits(h, None, y.shape[0], dg.data_ptr(), dw.data_ptr(), 64, out.data_ptr()) == -1
    assert lib.armt_logits(h, y.data_ptr(), y.shape[0], dg.data_ptr(), dw.data_ptr(), 60, out.data_ptr()) == -2
    assert "multiple of 8" in C.armt_last_error()
    assert lib.armt_logits(None, y.data_ptr(), 1, dg.data_ptr(), dw.data_ptr(), 64, out.data_ptr()) == -1
    # the handle still works after rejected calls
    got = model.logits(y, dg, dw)
    assert torch.isfinite(got).all()
