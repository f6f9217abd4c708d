"""Gradients of the ARMT forward, for the backward pass: PyTorch autograd over
a float64 restatement of the forward in ``armt_oracle`` (fp32 workloads: no
rounding points).

TEST INFRASTRUCTURE ONLY, like ``armt_oracle``: only the test suite and the
benchmark's CPU-baseline leg may import it.  It shares no code with the HIP
library.

The forward below takes the same steps as ``armt_oracle.Oracle.node`` in the
same order (memory read, attention block, MLP block, memory write; the
sequential order of nodes, which the pages show gives the same recurrence as
any order of the diagonal waves: Pith review of arXiv 2506.05229, "What
carries the argument").  It is written with torch operations so that
``torch.autograd`` differentiates it; its values are pinned to the NumPy
oracle and its gradients to central finite differences (tests marked "not
gpu").

The loss whose gradient is returned is the inner product of the outputs with
given output gradients, <y, dy> + <A_out, dA_out> + <z_out, dz_out>, so the
result is the vector-Jacobian product the backward computes.
"""

from __future__ import annotations

import math

import numpy as np
import torch

__all__ = ["PARAM_NAMES", "forward_torch", "vjp"]

PARAM_NAMES = ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "g_attn", "g_mlp",
               "w_mq", "w_mk", "w_mv", "w_beta", "mem_emb")


def _phi(u):
    return torch.where(u > 0, u + 1.0, torch.exp(torch.clamp(u, max=0.0)))


def _rms(h, g, eps):
    return h / torch.sqrt((h * h).mean(-1, keepdim=True) + eps) * g


def _rope(x, theta):
    n, _, hd = x.shape
    half = hd // 2
    inv = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / hd)
    ang = torch.arange(n, dtype=torch.float64)[:, None] * inv[None, :]
    cos, sin = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return torch.cat([a * cos - b * sin, b * cos + a * sin], dim=-1)


def _attention(Q, K, V):
    n, H, hd = Q.shape
    G = K.shape[1]
    rep = H // G
    mask = torch.triu(torch.ones(n, n, dtype=torch.bool), diagonal=1)
    outs = []
    for j in range(H):
        s = (Q[:, j, :] @ K[:, j // rep, :].T) / math.sqrt(hd)
        s = s.masked_fill(mask, float("-inf"))
        outs.append(torch.softmax(s, dim=1) @ V[:, j // rep, :])
    return torch.stack(outs, dim=1).reshape(n, H * hd)


def forward_torch(cfg, x, params, A0, z0):
    """x [S*T, d]; params: name -> tensor ([L, ...] stacked; mem_emb [M, d]);
    A0 [L, d, d_k], z0 [L, d_k].  Returns (y, A_out, z_out)."""
    L = params["w_qkv"].shape[0]
    T, M, H, G, hd = cfg.seg_len, cfg.n_mem, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    S = x.shape[0] // T
    A = [A0[l] for l in range(L)]
    z = [z0[l] for l in range(L)]
    ys = []
    for s in range(S):
        h = torch.cat([x[s * T:(s + 1) * T], params["mem_emb"]], dim=0)
        n = h.shape[0]
        for l in range(L):
            # memory read
            q = _phi(h @ params["w_mq"][l].T)
            h = h + (q @ A[l].T) / (q @ z[l] + cfg.mem_eps)[:, None]
            # attention block
            a = _rms(h, params["g_attn"][l], cfg.rms_eps)
            qkv = a @ params["w_qkv"][l].T
            Q = _rope(qkv[:, :H * hd].reshape(n, H, hd), cfg.rope_theta)
            K = _rope(qkv[:, H * hd:(H + G) * hd].reshape(n, G, hd), cfg.rope_theta)
            V = qkv[:, (H + G) * hd:].reshape(n, G, hd)
            h = h + _attention(Q, K, V) @ params["w_o"][l].T
            # MLP block
            b = _rms(h, params["g_mlp"][l], cfg.rms_eps)
            gate = b @ params["w_gate"][l].T
            up = b @ params["w_up"][l].T
            h = h + (gate * torch.sigmoid(gate) * up) @ params["w_down"][l].T
            # memory write from the memory-token rows
            Y = h[T:]
            k = _phi(Y @ params["w_mk"][l].T)
            v = Y @ params["w_mv"][l].T
            beta = torch.sigmoid(Y @ params["w_beta"][l])
            vbar = (k @ A[l].T) / (k @ z[l] + cfg.mem_eps)[:, None]
            A[l] = A[l] + (beta[:, None] * (v - vbar)).T @ k
            z[l] = z[l] + k.sum(0)
        ys.append(h[:T])
    return torch.cat(ys, dim=0), torch.stack(A), torch.stack(z)


def vjp(inputs, A0, z0, dy, dA_out, dz_out):
    """Gradients of <y, dy> + <A_out, dA_out> + <z_out, dz_out> with respect
    to x, A0, z0 and every parameter, as float64 NumPy arrays:
    (dx, dA0, dz0, {name: d_param})."""
    cfg = inputs.cfg
    L = inputs.weights["w_qkv"].shape[0]
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    x = t(inputs.x)
    params = {name: t(inputs.weights[name]) for name in inputs.weights}
    params["g_attn"] = t(inputs.g_attn)
    params["g_mlp"] = t(inputs.g_mlp)
    params["mem_emb"] = t(inputs.mem_emb)
    A0t = t(np.zeros((L, cfg.d_model, cfg.d_key)) if A0 is None else A0)
    z0t = t(np.zeros((L, cfg.d_key)) if z0 is None else z0)
    y, A, z = forward_torch(cfg, x, params, A0t, z0t)
    loss = (y * torch.as_tensor(dy, dtype=torch.float64)).sum() \
        + (A * torch.as_tensor(dA_out, dtype=torch.float64)).sum() \
        + (z * torch.as_tensor(dz_out, dtype=torch.float64)).sum()
    names = list(PARAM_NAMES)
    grads = torch.autograd.grad(loss, [x, A0t, z0t] + [params[k] for k in names])
    g = [gr.detach().numpy() for gr in grads]
    return g[0], g[1], g[2], dict(zip(names, g[3:]))
