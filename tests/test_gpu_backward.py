"""GPU parity of the backward pass (armt_backward, fp32 handles) against the
gradient oracle (PyTorch autograd over a float64 restatement of the forward,
pinned to finite differences): the gradients of <y, dy> + <A_out, dA_out> +
<z_out, dz_out> with respect to x, A0, z0 and all twelve weight tensors,
relative L2 <= 1e-4 each; the grouped (reversed diagonal waves) and the
node-by-node backward bitwise equal.  The shapes run from a single node to the
timed backward workload itself (8 layers, 32 segments of 128 + 8 tokens).
"""

import sys

import numpy as np
import pytest
import torch

from oracle import armt_grad
from armt_inputs import get_config, make_inputs, make_state
from long_context_recurrent_amd import armt as C
from long_context_recurrent_amd.model import ArmtModel, WEIGHT_FIELDS, backward

from gpu_util import build_model, rel_l2, to_device, to_np

pytestmark = pytest.mark.gpu

TINY = get_config("tiny_fp32")
CASES = [
    TINY.with_(name="bw_l2_s3", n_layers=2, n_segments=3, seg_len=5, n_mem=3, d_model=64, n_heads=2, n_kv_heads=1,
               head_dim=32, ffn_hidden=64),
    TINY.with_(name="bw_l3_s4", n_layers=3, n_segments=4, seg_len=16, n_mem=4, d_model=128, n_heads=4,
               n_kv_heads=2, head_dim=32, ffn_hidden=192),
    TINY.with_(name="bw_l1_s1", n_layers=1, n_segments=1, seg_len=7, n_mem=2, d_model=64, n_heads=1, n_kv_heads=1,
               head_dim=64, ffn_hidden=128),
    # head dimension 128 (two elements per lane in the attention backward),
    # 64 x 64 GEMM tiles, a node longer than one 64-key lane sweep
    TINY.with_(name="bw_hd128", n_layers=4, n_segments=3, seg_len=200, n_mem=8, d_model=256, n_heads=2,
               n_kv_heads=1, head_dim=128, ffn_hidden=512),
    # the timed backward workload (8 layers, 32 segments of 128 + 8 tokens)
    TINY.with_(name="bw_bench", n_layers=8, d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn_hidden=512,
               seg_len=128, n_mem=8, n_segments=32),
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("state", ["zero", "given"])
def test_backward_parity(cfg, state):
    say(f"[backward] {cfg.name} state={state}")
    inp = make_inputs(cfg)
    if state == "given":
        A0, z0 = make_state(cfg)
        A0 = (A0 / 64.0).astype(np.float32)
    else:
        A0, z0 = None, None
    rng = np.random.default_rng(5)
    dy = rng.standard_normal(inp.x.shape).astype(np.float32)
    dA = (rng.standard_normal((cfg.n_layers, cfg.d_model, cfg.d_key)) * 1e-3).astype(np.float32)
    dz = (rng.standard_normal((cfg.n_layers, cfg.d_key)) * 1e-3).astype(np.float32)
    dx_r, dA0_r, dz0_r, dp_r = armt_grad.vjp(inp, A0, z0, dy, dA, dz)

    model = build_model(inp)
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x = to_device(inp.x, cfg)
    got = {}
    for sched in ("diagonal", "sequential"):
        got[sched] = backward(model, x, dev(dy), dev(A0), dev(z0), dev(dA), dev(dz), schedule=sched)
    dxd, dA0d, dz0d, gd = got["diagonal"]
    dxs, dA0s, dz0s, gs = got["sequential"]
    assert torch.equal(dxd, dxs) and torch.equal(dA0d, dA0s) and torch.equal(dz0d, dz0s)
    for k in WEIGHT_FIELDS:
        assert torch.equal(gd[k], gs[k]), f"d{k}: diagonal and sequential backward differ"
    errs = {"x": rel_l2(to_np(dxd), dx_r), "A0": rel_l2(to_np(dA0d), dA0_r), "z0": rel_l2(to_np(dz0d), dz0_r)}
    for k in WEIGHT_FIELDS:
        errs[k] = rel_l2(to_np(gd[k]), dp_r[k])
    say("  rel L2 " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= 1e-4, f"d{k}: rel L2 {v:.3e}"
    # the handle's forward is untouched by the backward
    y1 = model.forward(x, "diagonal")[0].clone()
    model2 = build_model(inp)
    assert torch.equal(y1, model2.forward(x, "diagonal")[0])


SMALL = get_config("small_bf16")
BF16_CASES = [
    SMALL.with_(name="bw16_l2_s3", n_layers=2, n_segments=3, seg_len=64, n_mem=8, d_model=256, n_heads=4,
                n_kv_heads=2, head_dim=64, ffn_hidden=512),
    SMALL.with_(name="bw16_l3_s4_hd128", n_layers=3, n_segments=4, seg_len=100, n_mem=16, d_model=256, n_heads=2,
                n_kv_heads=1, head_dim=128, ffn_hidden=768),
]


def _bf16_case(cfg, state):
    inp = make_inputs(cfg)
    if state == "given":
        A0, z0 = make_state(cfg)
        A0 = (A0 / 64.0).astype(np.float32)
    else:
        A0, z0 = None, None
    rng = np.random.default_rng(5)
    # dy is given in bf16: the oracle sees the same (exactly representable) values
    dy = torch.from_numpy(rng.standard_normal(inp.x.shape).astype(np.float32)).to(torch.bfloat16)
    dA = (rng.standard_normal((cfg.n_layers, cfg.d_model, cfg.d_key)) * 1e-3).astype(np.float32)
    dz = (rng.standard_normal((cfg.n_layers, cfg.d_key)) * 1e-3).astype(np.float32)
    return inp, A0, z0, dy, dA, dz


@pytest.mark.parametrize("cfg", BF16_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("state", ["zero", "given"])
def test_backward_bf16_parity(cfg, state):
    """bf16 handles: the recording forward is the bf16 forward and each node
    is differentiated in fp32 with the weights widened, so the gradients differ
    from the float64 gradient of the unrounded forward by the bf16 forward's
    own error and the bf16 operands of attention; bar 2e-2 relative L2 (the
    bf16 forward's bar)."""
    say(f"[backward bf16] {cfg.name} state={state}")
    inp, A0, z0, dy, dA, dz = _bf16_case(cfg, state)
    dx_r, dA0_r, dz0_r, dp_r = armt_grad.vjp(inp, A0, z0, dy.float().numpy(), dA, dz)
    model = build_model(inp)
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x = to_device(inp.x, cfg)
    got = {sched: backward(model, x, dy.cuda(), dev(A0), dev(z0), dev(dA), dev(dz), schedule=sched)
           for sched in ("diagonal", "sequential")}
    dxd, dA0d, dz0d, gd = got["diagonal"]
    dxs, dA0s, dz0s, gs = got["sequential"]
    assert dxd.dtype == torch.float32 and all(gd[k].dtype == torch.float32 for k in WEIGHT_FIELDS)
    assert torch.equal(dxd, dxs) and torch.equal(dA0d, dA0s) and torch.equal(dz0d, dz0s)
    for k in WEIGHT_FIELDS:
        assert torch.equal(gd[k], gs[k]), f"d{k}: diagonal and sequential backward differ"
    errs = {"x": rel_l2(to_np(dxd), dx_r), "A0": rel_l2(to_np(dA0d), dA0_r), "z0": rel_l2(to_np(dz0d), dz0_r)}
    for k in WEIGHT_FIELDS:
        errs[k] = rel_l2(to_np(gd[k]), dp_r[k])
    say("  rel L2 " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= 2e-2, f"d{k}: rel L2 {v:.3e}"


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_backward_bf16_1b_layer_shape():
    """The 1B layer shape (d 2048, 32/8 heads of 64, F 8192, 1024 + 16 rows),
    2 layers x 2 segments from a non-zero state: every gradient against the
    float64 oracle (bar 2e-2), grouped == node-by-node bitwise."""
    cfg = get_config("1b_s128").with_(n_layers=2, n_segments=2)
    say(f"[backward bf16 1B shape] L={cfg.n_layers} S={cfg.n_segments}")
    inp, A0, z0, dy, dA, dz = _bf16_case(cfg, "given")
    dx_r, dA0_r, dz0_r, dp_r = armt_grad.vjp(inp, A0, z0, dy.float().numpy(), dA, dz)
    model = build_model(inp)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x = to_device(inp.x, cfg)
    got = {sched: backward(model, x, dy.cuda(), dev(A0), dev(z0), dev(dA), dev(dz), schedule=sched)
           for sched in ("diagonal", "sequential")}
    dxd, dA0d, dz0d, gd = got["diagonal"]
    dxs, dA0s, dz0s, gs = got["sequential"]
    assert torch.equal(dxd, dxs) and torch.equal(dA0d, dA0s) and torch.equal(dz0d, dz0s)
    for k in WEIGHT_FIELDS:
        assert torch.equal(gd[k], gs[k])
    errs = {"x": rel_l2(to_np(dxd), dx_r), "A0": rel_l2(to_np(dA0d), dA0_r), "z0": rel_l2(to_np(dz0d), dz0_r)}
    for k in WEIGHT_FIELDS:
        errs[k] = rel_l2(to_np(gd[k]), dp_r[k])
    say("  rel L2 " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= 2e-2, f"d{k}: rel L2 {v:.3e}"


def test_backward_argument_errors():
    cfg = CASES[0]
    inp = make_inputs(cfg)
    model = build_model(inp)
    lib = C.load_library()
    n = C.armt_backward_workspace_size(model.handle, cfg.n_segments)
    assert n > 0
    with pytest.raises(C.ArmtError):
        C.armt_backward_workspace_size(model.handle, 0)
    bmodel = ArmtModel(model.cfg, model.weights, batch=2)
    with pytest.raises(C.ArmtError) as e:
        C.armt_backward_workspace_size(bmodel.handle, 1)
    assert e.value.code == -2
    assert lib.armt_backward(None, 0, 1, 1, None, None, 1, None, None, 1, 1, 1, None, 1, 1) == -1
    with pytest.raises(ValueError):
        backward(model, x=to_device(inp.x, cfg).to(torch.bfloat16), dy=to_device(inp.x, cfg))
