"""GPU parity at the edges of what the library accepts: the smallest node
(one token, one memory token), the most memory tokens (64), the longest bf16
node (T + M = 4096), the narrowest bf16 model (d = 128, 4:1 grouped-query
heads of 32), the largest fp32 node and width (T + M = 2048, d = 1024), and
bf16 widths whose column-chunk counts (3, 9, 23) the memory read handles with
wait counts computed at run time.
Each against the oracle (relative L2 1e-4 fp32, 2e-2 bf16, from a given
non-zero state so the memory read is exercised), diagonal == sequential
bitwise.
"""

import sys
import time

import pytest
import torch

import oracle
from armt_inputs import get_config, make_inputs, make_state

from gpu_util import build_model, rel_l2, state_to_device, to_device, to_np, tol

pytestmark = pytest.mark.gpu

SMALL = get_config("small_bf16")
TINY = get_config("tiny_fp32")

EDGES = [
    SMALL.with_(name="one_token", n_layers=2, d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn_hidden=512,
                seg_len=1, n_mem=1, n_segments=5),
    SMALL.with_(name="mem64", n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64, ffn_hidden=512,
                seg_len=64, n_mem=64, n_segments=3),
    SMALL.with_(name="n4096", n_layers=2, d_model=256, n_heads=4, n_kv_heads=1, head_dim=64, ffn_hidden=512,
                seg_len=4032, n_mem=64, n_segments=2),
    SMALL.with_(name="d128_gqa4", n_layers=3, d_model=128, n_heads=4, n_kv_heads=1, head_dim=32, ffn_hidden=256,
                seg_len=100, n_mem=3, n_segments=4),
    TINY.with_(name="f32_n2048_d1024", n_layers=1, d_model=1024, n_heads=8, n_kv_heads=4, head_dim=128,
               ffn_hidden=1024, seg_len=2000, n_mem=48, n_segments=2),
    # bf16 widths outside the memory read's fixed-count instantiations (3, 9
    # and 23 column chunks of 128: wait counts taken at run time)
    SMALL.with_(name="d384_chunks3", n_layers=2, d_model=384, n_heads=6, n_kv_heads=2, head_dim=64, ffn_hidden=768,
                seg_len=100, n_mem=8, n_segments=3),
    SMALL.with_(name="d1152_chunks9", n_layers=2, d_model=1152, n_heads=18, n_kv_heads=6, head_dim=64,
                ffn_hidden=1024, seg_len=64, n_mem=16, n_segments=3),
    SMALL.with_(name="d2944_chunks23", n_layers=2, d_model=2944, n_heads=46, n_kv_heads=2, head_dim=64,
                ffn_hidden=512, seg_len=32, n_mem=8, n_segments=2),
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("cfg", EDGES, ids=lambda c: c.name)
def test_edge_parity(cfg):
    say(f"[edge] {cfg.name} L={cfg.n_layers} d={cfg.d_model} n={cfg.n} S={cfg.n_segments} {cfg.dtype}")
    inp = make_inputs(cfg)
    A0, z0 = make_state(cfg)
    t0 = time.time()
    y_ref, A_ref, z_ref = oracle.forward_sequential(inp, A0, z0)
    say(f"  oracle {time.time() - t0:.1f}s")
    model = build_model(inp)
    x = to_device(inp.x, cfg)
    dA0, dz0 = state_to_device(A0, z0)
    yd, Ad, zd = [t.clone() for t in model.forward(x, "diagonal", dA0, dz0)]
    e = (rel_l2(to_np(yd), y_ref), rel_l2(to_np(Ad), A_ref), rel_l2(to_np(zd), z_ref),
         rel_l2(to_np(Ad) - A0, A_ref - A0))
    say(f"  rel L2 y={e[0]:.2e} A={e[1]:.2e} z={e[2]:.2e} dA={e[3]:.2e}")
    assert max(e) <= tol(cfg)
    ys, As, zs = model.forward(x, "sequential", dA0, dz0)
    assert torch.equal(ys, yd) and torch.equal(As, Ad) and torch.equal(zs, zd)
