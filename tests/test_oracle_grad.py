"""Pins of the gradient oracle (oracle.armt_grad): its forward equals the
NumPy oracle's, and its autograd vector-Jacobian product equals central
finite differences of that forward on a tiny fp32 workload (brute force,
float64)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import armt_grad
from armt_inputs import get_config, make_inputs, make_state

CFG = get_config("tiny_fp32").with_(n_layers=2, n_segments=3, seg_len=5, n_mem=3, d_model=64, n_heads=2,
                                    n_kv_heads=1, head_dim=32, ffn_hidden=64)


def _torch_params(inp):
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
    p = {k: t(v) for k, v in inp.weights.items()}
    p.update(g_attn=t(inp.g_attn), g_mlp=t(inp.g_mlp), mem_emb=t(inp.mem_emb))
    return p


def test_torch_forward_equals_numpy_oracle():
    inp = make_inputs(CFG)
    A0, z0 = make_state(CFG)
    y, A, z = armt_grad.forward_torch(CFG, torch.tensor(inp.x, dtype=torch.float64), _torch_params(inp),
                                      torch.tensor(A0, dtype=torch.float64), torch.tensor(z0, dtype=torch.float64))
    y_ref, A_ref, z_ref = oracle.forward_sequential(inp, A0, z0)
    # the NumPy oracle stores the state in float32 after every update; this
    # restatement keeps it in float64, so they agree to float32 rounding
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(y.numpy(), y_ref) < 1e-6
    assert rel(A.numpy(), A_ref) < 1e-6
    assert rel(z.numpy(), z_ref) < 1e-6


def test_vjp_against_finite_differences():
    inp = make_inputs(CFG)
    A0, z0 = make_state(CFG)
    A0 = A0 / 64.0                                                # keep the read of moderate size
    rng = np.random.default_rng(11)
    dy = rng.standard_normal(inp.x.shape)
    dA = rng.standard_normal(A0.shape) * 1e-3
    dz = rng.standard_normal(z0.shape) * 1e-3
    dx, dA0, dz0, dp = armt_grad.vjp(inp, A0, z0, dy, dA, dz)
    params = _torch_params(inp)
    x = torch.tensor(inp.x, dtype=torch.float64)
    A0t, z0t = torch.tensor(A0, dtype=torch.float64), torch.tensor(z0, dtype=torch.float64)

    def loss():
        with torch.no_grad():
            y, A, z = armt_grad.forward_torch(CFG, x, params, A0t, z0t)
            return float((y.numpy() * dy).sum() + (A.numpy() * dA).sum() + (z.numpy() * dz).sum())

    def fd(t, idx, eps=1e-6):
        old = t[idx].item()
        t[idx] = old + eps
        lp = loss()
        t[idx] = old - eps
        lm = loss()
        t[idx] = old
        return (lp - lm) / (2 * eps)

    checks = [("x", x, dx), ("A0", A0t, dA0), ("z0", z0t, dz0)] + [(k, params[k], dp[k]) for k in armt_grad.PARAM_NAMES]
    for name, t, g in checks:
        flat = t.view(-1)
        picks = rng.choice(flat.numel(), size=min(4, flat.numel()), replace=False)
        for i in picks:
            idx = np.unravel_index(int(i), tuple(t.shape))
            want = fd(t, idx)
            got = g[idx]
            assert abs(got - want) <= 1e-5 * max(1.0, abs(want)), f"{name}{idx}: autograd {got} vs fd {want}"
