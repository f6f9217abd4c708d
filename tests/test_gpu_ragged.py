"""GPU parity of any-length sequences (armt_forward_*_tokens): the last
segment may be shorter than T.  Through the C ABI against the oracle's
``n_tokens`` runs; bars as for the forward (relative L2 1e-4 fp32, 2e-2
bf16); diagonal == sequential bitwise; the token-count calls with a multiple
of T bitwise equal to the segment-count calls; the captured graphs serve full
and short calls alike.
"""

import sys
import time

import numpy as np
import pytest
import torch

import oracle
from armt_inputs import get_config, make_inputs, make_state
from long_context_recurrent_amd import armt as C

from gpu_util import build_model, rel_l2, state_to_device, to_device, to_np, tol

pytestmark = pytest.mark.gpu

TINY = get_config("tiny_fp32")
SMALL = get_config("small_bf16")
MID64 = SMALL.with_(name="mid_hd64", n_layers=3, d_model=512, n_heads=8, n_kv_heads=2, head_dim=64,
                    ffn_hidden=1536, seg_len=200, n_mem=16, n_segments=5)
MID128 = SMALL.with_(name="mid_hd128", n_layers=3, d_model=768, n_heads=6, n_kv_heads=2, head_dim=128,
                     ffn_hidden=1280, seg_len=120, n_mem=8, n_segments=4)
MID32 = SMALL.with_(name="mid_hd32", n_layers=2, d_model=256, n_heads=8, n_kv_heads=4, head_dim=32,
                    ffn_hidden=512, seg_len=150, n_mem=5, n_segments=3)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [(TINY, 3 * 16 + 1), (TINY, 2 * 16 + 9), (TINY, 5), (SMALL, 16 * 128 - 91), (SMALL, 1),
         (SMALL, 3 * 128 + 64), (MID64, 4 * 200 + 17), (MID128, 3 * 120 + 119), (MID32, 2 * 150 + 1)]


@pytest.mark.parametrize("cfg,N", CASES, ids=lambda v: getattr(v, "name", str(v)))
@pytest.mark.parametrize("state", ["zero", "given"])
def test_ragged_parity(cfg, N, state):
    say(f"[ragged] {cfg.name} N={N} state={state}")
    inp = make_inputs(cfg)
    assert N <= inp.x.shape[0]
    A0, z0 = make_state(cfg) if state == "given" else (None, None)
    y_ref, A_ref, z_ref = oracle.forward_sequential(inp, A0, z0, n_tokens=N)
    model = build_model(inp)
    x = to_device(inp.x[:N], cfg)
    dA0, dz0 = state_to_device(A0, z0)
    yd, Ad, zd = [t.clone() for t in model.forward(x, "diagonal", dA0, dz0, by_tokens=True)]
    assert yd.shape == (N, cfg.d_model)
    e = (rel_l2(to_np(yd), y_ref), rel_l2(to_np(Ad), A_ref), rel_l2(to_np(zd), z_ref))
    say(f"  rel L2 y={e[0]:.2e} A={e[1]:.2e} z={e[2]:.2e}")
    assert max(e) <= tol(cfg)
    # the short segment's own rows, and its state increment over the previous state
    T = cfg.seg_len
    tail = slice((N - 1) // T * T, N)
    assert rel_l2(to_np(yd[tail]), y_ref[tail]) <= tol(cfg)
    if A0 is not None:
        An = to_np(Ad)
        for l in range(cfg.n_layers):
            assert rel_l2(An[l] - A0[l], A_ref[l] - A0[l]) <= tol(cfg)
    ys, As, zs = model.forward(x, "sequential", dA0, dz0, by_tokens=True)
    assert torch.equal(ys, yd) and torch.equal(As, Ad) and torch.equal(zs, zd)


def test_token_count_calls_equal_segment_calls_and_share_graphs():
    cfg = MID64
    inp = make_inputs(cfg)
    model = build_model(inp)
    T, S = cfg.seg_len, cfg.n_segments
    x = to_device(inp.x, cfg)
    ref = [t.clone() for t in model.forward(x, "diagonal", by_tokens=False)]
    got = model.forward(x, "diagonal", by_tokens=True)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    # a short call, then a full one through the same graphs, then the short again
    N = (S - 1) * T + 3
    xs = x[:N].contiguous()
    short = [t.clone() for t in model.forward(xs, "diagonal")]
    again = model.forward(x, "diagonal")
    for a, b in zip(ref, again):
        assert torch.equal(a, b), "a short call left state behind in the graphs"
    short2 = model.forward(xs, "diagonal")
    for a, b in zip(short, short2):
        assert torch.equal(a, b)
    # earlier segments do not see the short last one
    assert torch.equal(short[0][:(S - 1) * T], ref[0][:(S - 1) * T])
    # direct launches agree with the graphs
    model.set_option(C.ARMT_OPT_GRAPHS, 0)
    direct = model.forward(xs, "sequential")
    for a, b in zip(short, direct):
        assert torch.equal(a, b)


def test_token_count_errors():
    cfg = SMALL.with_(n_segments=2)
    inp = make_inputs(cfg)
    model = build_model(inp)
    x = to_device(inp.x, cfg)
    y, A, z = model.alloc_outputs(2)
    lib = C.load_library()
    h = model.handle
    assert lib.armt_forward_diagonal_tokens(h, x.data_ptr(), 0, None, None, y.data_ptr(), A.data_ptr(),
                                            z.data_ptr()) == -1
    assert lib.armt_forward_sequential_tokens(h, x.data_ptr(), -5, None, None, y.data_ptr(), A.data_ptr(),
                                              z.data_ptr()) == -1
    assert lib.armt_forward_diagonal_tokens(None, x.data_ptr(), 10, None, None, y.data_ptr(), A.data_ptr(),
                                            z.data_ptr()) == -1
    assert lib.armt_forward_diagonal_tokens(h, None, 10, None, None, y.data_ptr(), A.data_ptr(),
                                            z.data_ptr()) == -1
    model.forward(x[:100].contiguous(), "diagonal")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_ragged_1b():
    """1B shape, 1,324 tokens (a full segment and a 300-token one), from a
    non-zero state: every output row and the state against the oracle; and
    131,072 - 500 tokens: the first 127 segments bitwise equal to the full
    run's, all outputs finite."""
    cfg = get_config("1b_s128")
    t0 = time.time()
    inp = make_inputs(cfg)
    A0, z0 = make_state(cfg)
    say(f"[ragged 1b] inputs drawn in {time.time() - t0:.1f}s")
    model = build_model(inp)
    x = to_device(inp.x, cfg)
    T, bar = cfg.seg_len, tol(cfg)
    dA0, dz0 = state_to_device(A0, z0)
    N = T + 300
    y, A, z = [t.clone() for t in model.forward(x[:N].contiguous(), "diagonal", dA0, dz0)]
    t0 = time.time()
    y_ref, A_ref, z_ref = oracle.forward_sequential(inp, A0, z0, n_tokens=N)
    say(f"[ragged 1b] oracle in {time.time() - t0:.1f}s")
    for name, got, ref in (("y", y, y_ref), ("y short segment", y[T:], y_ref[T:]), ("A", A, A_ref),
                           ("z", z, z_ref)):
        e = rel_l2(to_np(got), ref)
        say(f"  {name}: rel L2 {e:.2e}")
        assert e <= bar
    An = to_np(A)
    e = rel_l2(An - A0, A_ref - A0)
    say(f"  A increment: rel L2 {e:.2e}")
    assert e <= bar
    Nl = cfg.n_segments * T - 500
    yl, Al, zl = model.forward(x[:Nl].contiguous(), "diagonal")
    assert torch.isfinite(yl).all() and torch.isfinite(Al).all() and torch.isfinite(zl).all()
    yf, _, _ = model.forward(x, "diagonal")
    assert torch.equal(yl[:127 * T], yf[:127 * T])
    ys, As, zs = model.forward(x[:Nl].contiguous(), "sequential")
    assert torch.equal(ys, yl) and torch.equal(As, Al) and torch.equal(zs, zl)
    model.close()
