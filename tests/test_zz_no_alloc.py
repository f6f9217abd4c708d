"""armt_forward_diagonal_noalloc -- the diagonal forward for callers that
cannot allocate, whose workspace is the library's static device scratch --
against a handle's armt_forward_diagonal on the same inputs, through the C
ABI: two calls in a row on each workload (the second with fewer segments, so
it runs over what the first left in the scratch), from a given initial state
and from zeros.  Bar: the stated parity tolerance (1e-4 fp32, 2e-2 bf16
relative L2); the two differ only in where the RoPE table is computed."""

import numpy as np
import pytest
import torch

from armt_inputs import get_config, make_inputs, make_state
from long_context_recurrent_amd import armt as C
from long_context_recurrent_amd.model import WEIGHT_FIELDS

from gpu_util import build_model, rel_l2, state_to_device, to_device, to_np, tol

pytestmark = pytest.mark.gpu

TINY = get_config("tiny_fp32")
SMALL = get_config("small_bf16")
MID64 = SMALL.with_(name="mid_hd64", n_layers=3, d_model=512, n_heads=8, n_kv_heads=2, head_dim=64,
                    ffn_hidden=1536, seg_len=200, n_mem=16, n_segments=5)


def _noalloc(model, x, S, A0, z0):
    L, B = model.cfg.n_layers, 1
    d, dk = model.cfg.d_model, model.cfg.d_key
    y = torch.empty(S * model.cfg.seg_len, d, dtype=model.dtype, device=x.device)
    A = torch.empty(L, d, dk, dtype=torch.float32, device=x.device)
    z = torch.empty(L, dk, dtype=torch.float32, device=x.device)
    w = C.armt_weights(*[model.weights[k].data_ptr() for k in WEIGHT_FIELDS])
    st = torch.cuda.current_stream(x.device)
    C.armt_forward_diagonal_noalloc(model.cfg, w, x, S, A0, z0, y, A, z, st)
    st.synchronize()
    return y, A, z


@pytest.mark.parametrize("cfg", [TINY, SMALL, MID64], ids=lambda c: c.name)
@pytest.mark.parametrize("state", ["zero", "given"])
def test_noalloc_matches_handle_forward(cfg, state):
    inp = make_inputs(cfg)
    model = build_model(inp)
    A0, z0 = make_state(cfg) if state == "given" else (None, None)
    dA0, dz0 = state_to_device(A0, z0)
    x = to_device(inp.x, cfg)
    T, S = cfg.seg_len, cfg.n_segments
    for s_call in (S, max(1, S // 2)):
        xs = x[:s_call * T].contiguous()
        ref = [t.clone() for t in model.forward(xs, "diagonal", dA0, dz0)]
        got = _noalloc(model, xs, s_call, dA0, dz0)
        for name, a, b in zip(("y", "A", "z"), got, ref):
            e = rel_l2(to_np(a), to_np(b))
            print(f"{cfg.name} S={s_call} {state} {name}: rel L2 {e:.2e} bitwise={torch.equal(a, b)}", flush=True)
            assert torch.isfinite(a).all()
            assert e <= tol(cfg), f"{name}: {e:.3e}"
    model.close()


def test_noalloc_rejects_models_beyond_the_scratch():
    big = get_config("1b_s32")
    inp = make_inputs(SMALL)
    model = build_model(inp)
    bcfg = C.armt_config(big.n_layers, big.d_model, big.n_heads, big.n_kv_heads, big.head_dim, big.ffn_hidden,
                         big.seg_len, big.n_mem, big.d_key, C.ARMT_BF16, 1e-5, 1e4, 1e-6)
    w = C.armt_weights(*[model.weights[k].data_ptr() for k in WEIGHT_FIELDS])
    x = torch.zeros(big.seg_len, big.d_model, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(C.ArmtError) as e:
        C.armt_forward_diagonal_noalloc(bcfg, w, x, 1, None, None, x, x, x, None)
    assert e.value.code == C.ARMT_E_WORKSPACE and "scratch" in str(e.value)
    model.close()
