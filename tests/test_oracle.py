"""Pins of the CPU oracle against things other than itself (CPU only).

* bf16 rounding against torch's float32 -> bfloat16 conversion;
* phi, sigmoid, SiLU, RMSNorm against torch's library routines;
* RoPE against rotation by complex multiplication, plus norm preservation,
  identity at position 0 and dependence of scores on relative position only;
* causal GQA attention against torch's scaled_dot_product_attention;
* the memory read/write against closed forms derived by hand;
* a zero-memory node against a block built from torch's library routines;
* order invariances: diagonal == sequential bitwise, wave shuffles, resume
  from a saved state (Pith review: the schedule is a pure reordering that keeps
  the recurrence; skill page, Practical Guidance: exact recurrence).
"""

import dataclasses
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from armt_inputs import get_config, make_inputs, make_state


# ---------------------------------------------------------------- rounding

def test_round_bf16_matches_torch():
    rng = np.random.default_rng(1)
    vals = [rng.standard_normal(20000).astype(np.float32),
            (rng.standard_normal(5000) * 1e30).astype(np.float32),
            (rng.standard_normal(5000) * 1e-38).astype(np.float32),    # subnormal range
            np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, -3.3895314e38, 3.4e38,
                      np.inf, -np.inf, 1e-45, -1e-45], dtype=np.float32)]
    # exact ties: 1 + 2^-8 (+odd multiples) sit halfway between bf16 neighbours
    ties = np.array([1 + k * 2.0 ** -8 for k in range(1, 64, 2)], dtype=np.float32)
    vals.append(ties)
    vals.append(-ties)
    x = np.concatenate(vals)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    assert np.isnan(oracle.round_bf16(np.array([np.nan])))[0]


def test_round_bf16_is_direct_from_float64():
    # 1 + 2^-8 + 2^-40 is above the tie, so it rounds up; going through float32
    # first would land exactly on the tie and round to even (down).
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -40])
    assert oracle.round_bf16(x)[0] == 1 + 2.0 ** -7


# ---------------------------------------------------------------- elementwise

def test_phi_sigmoid_silu_against_torch():
    u = np.linspace(-30, 30, 4001)
    t = torch.from_numpy(u)
    # elu(u) + 1 = (exp(u) - 1) + 1 cancels for u << 0: compare absolutely there
    np.testing.assert_allclose(oracle.phi(u), (F.elu(t) + 1).numpy(), rtol=1e-15, atol=2e-16)
    np.testing.assert_allclose(oracle.sigmoid(u), torch.sigmoid(t).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(oracle.silu(u), F.silu(t).numpy(), rtol=1e-14, atol=1e-300)
    assert np.all(oracle.phi(u) > 0)


def test_rms_norm_against_torch():
    rng = np.random.default_rng(2)
    h = rng.standard_normal((7, 96)) * 3
    g = rng.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(h), (96,), weight=torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.rms_norm(h, g, 1e-5), ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- RoPE

@pytest.mark.parametrize("hd", [32, 64, 128])
def test_rope_complex_rotation(hd):
    rng = np.random.default_rng(3)
    n, nh, theta = 37, 3, 10000.0
    x = rng.standard_normal((n, nh, hd))
    got = oracle.rope(x, theta)
    half = hd // 2
    # pair (i, i + hd/2) as the complex number x_i + 1j * x_{i+hd/2}, rotated
    # by e^{1j * pos * theta^(-2i/hd)}
    c = x[..., :half] + 1j * x[..., half:]
    freq = np.power(theta, -np.arange(0, hd, 2) / hd)
    rot = np.exp(1j * np.outer(np.arange(n), freq))[:, None, :]
    r = c * rot
    ref = np.concatenate([r.real, r.imag], axis=-1)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(4)
    n, hd = 50, 64
    x = rng.standard_normal((n, 2, hd))
    y = oracle.rope(x, 10000.0)
    # norm preserved per (pos, head); position 0 untouched
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    np.testing.assert_array_equal(y[0], x[0])
    # scores depend on relative position only: q, k fixed vectors at all positions
    q = np.broadcast_to(rng.standard_normal(hd), (n, 1, hd)).copy()
    k = np.broadcast_to(rng.standard_normal(hd), (n, 1, hd)).copy()
    sc = oracle.rope(q, 10000.0)[:, 0] @ oracle.rope(k, 10000.0)[:, 0].T
    for m in range(n - 1):
        for j in range(n - 1):
            assert abs(sc[m + 1, j + 1] - sc[m, j]) < 1e-10


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("H,G,hd,n", [(2, 2, 32, 20), (4, 2, 64, 33), (6, 2, 128, 17), (8, 8, 16, 1)])
def test_attention_against_sdpa(H, G, hd, n):
    rng = np.random.default_rng(5)
    Q = rng.standard_normal((n, H, hd))
    K = rng.standard_normal((n, G, hd))
    V = rng.standard_normal((n, G, hd))
    got = oracle.causal_gqa_attention(Q, K, V)
    q = torch.from_numpy(Q).transpose(0, 1)                       # [H, n, hd]
    k = torch.from_numpy(K).transpose(0, 1).repeat_interleave(H // G, dim=0)
    v = torch.from_numpy(V).transpose(0, 1).repeat_interleave(H // G, dim=0)
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True)  # [H, n, hd]
    ref = ref.transpose(0, 1).reshape(n, H * hd).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- memory, closed forms

EPS = 1e-6


def _kappa(a):
    return a + 1.0 if a > 0 else math.exp(a)


@pytest.mark.parametrize("a,b,c", [(0.7, -1.3, 2.5), (-0.4, 0.9, -2.0), (1e-3, 5.0, 5.0)])
def test_memory_closed_forms(a, b, c):
    """d = 2, d_k = 1; W_mk = W_mq = [[1, 0]] (keys see only the first
    coordinate); W_mv = I; w_beta = 0 so beta = 1/2 exactly; kappa = phi(a)."""
    wk = np.array([[1.0, 0.0]])
    wv = np.eye(2)
    wb = np.zeros(2)
    A0 = np.zeros((2, 1))
    z0 = np.zeros(1)
    kap = _kappa(a)
    # a read from the zero state is exactly zero
    h = np.array([[a, 4.0]])
    np.testing.assert_array_equal(oracle.mem_read(h, wk, A0, z0, EPS), h)
    # first write y = (a, b): A1 = 1/2 (a, b)^T kappa, z1 = kappa
    A1, z1 = oracle.mem_write(np.array([[a, b]]), wk, wv, wb, A0, z0, EPS)
    np.testing.assert_allclose(A1, 0.5 * kap * np.array([[a], [b]]), rtol=1e-15)
    np.testing.assert_allclose(z1, [kap], rtol=1e-15)
    # read with key kappa: h + 1/2 (a, b) kappa^2 / (kappa^2 + eps)
    r = oracle.mem_read(h, wk, A1, z1, EPS)
    np.testing.assert_allclose(r, h + 0.5 * np.array([[a, b]]) * kap ** 2 / (kap ** 2 + EPS), rtol=1e-14)
    # second write y2 = (a, c): same key, the stored value is corrected
    vbar = 0.5 * np.array([a, b]) * kap ** 2 / (kap ** 2 + EPS)
    A2, z2 = oracle.mem_write(np.array([[a, c]]), wk, wv, wb, A1, z1, EPS)
    np.testing.assert_allclose(A2, A1 + 0.5 * kap * (np.array([[a], [c]]) - vbar[:, None]), rtol=1e-14)
    np.testing.assert_allclose(z2, [2 * kap], rtol=1e-15)
    # two tokens in one write both see the pre-update state
    e, f = -0.25, 1.75
    kap2 = _kappa(e)
    A3, z3 = oracle.mem_write(np.array([[a, c], [e, f]]), wk, wv, wb, A1, z1, EPS)
    vbar2 = 0.5 * np.array([a, b]) * kap * kap2 / (kap2 * kap + EPS)
    want = (A1 + 0.5 * kap * (np.array([[a], [c]]) - vbar[:, None])
            + 0.5 * kap2 * (np.array([[e], [f]]) - vbar2[:, None]))
    np.testing.assert_allclose(A3, want, rtol=1e-14)
    np.testing.assert_allclose(z3, [2 * kap + kap2], rtol=1e-15)


def test_memory_gate_and_retrieval():
    """With the gate saturated (beta -> 1) one write makes the memory return the
    written value for that key; with beta = 0 (w_beta -> -inf) A is unchanged
    while z still accumulates the key."""
    rng = np.random.default_rng(6)
    d, dk = 5, 3
    wk = np.abs(rng.standard_normal((dk, d)))
    wv = rng.standard_normal((d, d))
    y = np.abs(rng.standard_normal((1, d)))
    A0, z0 = np.zeros((d, dk)), np.zeros(dk)
    big = 1e3 * np.ones(d)                      # y > 0, so y . w_beta -> +inf
    A1, z1 = oracle.mem_write(y, wk, wv, big, A0, z0, EPS)
    k = oracle.phi(y @ wk.T)
    v = y @ wv.T
    np.testing.assert_allclose(A1, v.T @ k, rtol=1e-14)
    np.testing.assert_allclose(z1, k[0], rtol=1e-15)
    # retrieval with the same key feature returns v (up to eps)
    got = (k @ A1.T) / (k @ z1 + EPS)[:, None]
    np.testing.assert_allclose(got, v, rtol=1e-6)
    A2, z2 = oracle.mem_write(y, wk, wv, -big, A1, z1, EPS)
    np.testing.assert_array_equal(A2, A1)
    np.testing.assert_allclose(z2, 2 * k[0], rtol=1e-15)


# ---------------------------------------------------------------- whole node

def _torch_block(inp, l, h):
    """Memory-free Llama block from torch library routines (float64)."""
    c = inp.cfg
    H, G, hd, n = c.n_heads, c.n_kv_heads, c.head_dim, h.shape[0]
    W = {k: torch.from_numpy(v[l].astype(np.float64)) for k, v in inp.weights.items()}
    h = torch.from_numpy(h)
    a = F.rms_norm(h, (c.d_model,), weight=torch.from_numpy(inp.g_attn[l].astype(np.float64)), eps=c.rms_eps)
    qkv = F.linear(a, W["w_qkv"])
    q = qkv[:, :H * hd].reshape(n, H, hd)
    k = qkv[:, H * hd:(H + G) * hd].reshape(n, G, hd)
    v = qkv[:, (H + G) * hd:].reshape(n, G, hd)
    half = hd // 2
    freq = c.rope_theta ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    rot = torch.polar(torch.ones(n, half, dtype=torch.float64),
                      torch.outer(torch.arange(n, dtype=torch.float64), freq))[:, None, :]

    def rope(x):
        z = torch.complex(x[..., :half], x[..., half:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)
    q, k = rope(q), rope(k)
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                       is_causal=True, enable_gqa=True)
    h = h + F.linear(o.transpose(0, 1).reshape(n, H * hd), W["w_o"])
    b = F.rms_norm(h, (c.d_model,), weight=torch.from_numpy(inp.g_mlp[l].astype(np.float64)), eps=c.rms_eps)
    h = h + F.linear(F.silu(F.linear(b, W["w_gate"])) * F.linear(b, W["w_up"]), W["w_down"])
    return h.numpy()


def test_zero_memory_node_is_llama_block():
    cfg = get_config("tiny_fp32").with_(n_heads=4, n_kv_heads=2)     # exercise GQA
    inp = make_inputs(cfg)
    o = oracle.Oracle(inp)
    h_in = o.node_input(0)
    zA, zz = np.zeros((cfg.d_model, cfg.d_key)), np.zeros(cfg.d_key)
    for l in range(cfg.n_layers):
        h, A, z = o.node(l, h_in, zA, zz)
        ref = _torch_block(inp, l, np.asarray(h_in, dtype=np.float64))
        np.testing.assert_allclose(h, ref, rtol=1e-11, atol=1e-11)
        # and the write from the zero state equals the closed form
        y = h[cfg.seg_len:]
        k = oracle.phi(y @ inp.weights["w_mk"][l].astype(np.float64).T)
        v = y @ inp.weights["w_mv"][l].astype(np.float64).T
        beta = 1 / (1 + np.exp(-(y @ inp.weights["w_beta"][l].astype(np.float64))))
        np.testing.assert_allclose(A, (beta[:, None] * v).T @ k, rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(z, k.sum(0), rtol=1e-6)
        h_in = h


def test_prefix_rows_equal_full_node():
    """Causal attention and row-wise steps make the first r output rows depend
    only on the first r input rows (used for sampled checks at full size)."""
    cfg = get_config("small_bf16")
    inp = make_inputs(cfg, n_segments=2)
    A0, z0 = make_state(cfg)
    o = oracle.Oracle(inp)
    h_in = o.node_input(1)
    full, _, _ = o.node(2, h_in, A0[2], z0[2])
    part, _, _ = o.node(2, h_in, A0[2], z0[2], rows=40)
    np.testing.assert_allclose(part, full[:40], rtol=0, atol=2 ** -7 * np.abs(full[:40]).max())
    assert np.mean(part == full[:40]) > 0.99


# ---------------------------------------------------------------- order invariances

@pytest.mark.parametrize("name", ["tiny_fp32", "small_bf16"])
def test_diagonal_equals_sequential_bitwise(name):
    inp = make_inputs(get_config(name))
    ys, As, zs = oracle.forward_sequential(inp)
    yd, Ad, zd = oracle.forward_diagonal(inp)
    yx, Ax, zx = oracle.forward_diagonal(inp, shuffle_seed=11)
    for a, b, c in [(ys, yd, yx), (As, Ad, Ax), (zs, zd, zx)]:
        np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(a, c)
    assert np.all(np.isfinite(ys)) and np.abs(ys).max() > 0


@pytest.mark.parametrize("name", ["tiny_fp32", "small_bf16"])
def test_split_resume_bitwise(name):
    cfg = get_config(name)
    inp = make_inputs(cfg)
    S, T = cfg.n_segments, cfg.seg_len
    S1 = S // 2 + 1
    A0, z0 = make_state(cfg)
    y, A, z = oracle.forward_diagonal(inp, A0, z0)
    first = dataclasses.replace(inp, x=inp.x[:S1 * T])
    second = dataclasses.replace(inp, x=inp.x[S1 * T:])
    y1, A1, z1 = oracle.forward_sequential(first, A0, z0)
    y2, A2, z2 = oracle.forward_diagonal(second, A1.astype(np.float32), z1.astype(np.float32))
    np.testing.assert_array_equal(np.concatenate([y1, y2]), y)
    np.testing.assert_array_equal(A2, A)
    np.testing.assert_array_equal(z2, z)


def test_memory_carries_information_across_segments():
    """Segment 1's output depends on segment 0's tokens only through (A, z)."""
    cfg = get_config("tiny_fp32")
    inp = make_inputs(cfg)
    T = cfg.seg_len
    y, _, _ = oracle.forward_sequential(inp)
    x2 = inp.x.copy()
    x2[:T] += 1.0
    y2, _, _ = oracle.forward_sequential(dataclasses.replace(inp, x=x2))
    assert not np.allclose(y[T:2 * T], y2[T:2 * T])
    # with the memory disabled (w_mq = 0 gives q = 1, but A = 0 keeps the read
    # at zero only if nothing is written: zero the value path and the gate)
    w = dict(inp.weights)
    w["w_mv"] = np.zeros_like(w["w_mv"])
    w["w_beta"] = np.full_like(w["w_beta"], -1e4)
    ya, _, _ = oracle.forward_sequential(dataclasses.replace(inp, weights=w))
    yb, _, _ = oracle.forward_sequential(dataclasses.replace(inp, weights=w, x=x2))
    np.testing.assert_array_equal(ya[T:], yb[T:])


def test_storage_precision_of_bf16_workloads():
    """Stored values of a bf16 workload: branch activations are bf16 values,
    the residual stream and the state are float32 values, y is the stream
    rounded to bf16 (the reading of "bf16 activations with fp32 accumulate")."""
    cfg = get_config("small_bf16").with_(n_layers=2, n_segments=2)
    inp = make_inputs(cfg)
    o = oracle.Oracle(inp)
    A0, z0 = make_state(cfg)
    tr = {}
    h, A, z = o.node(0, o.node_input(0), A0[0], z0[0], trace=tr)

    def is_bf16(a):
        return np.array_equal(oracle.round_bf16(a), a)

    def is_f32(a):
        return np.array_equal(np.asarray(a, np.float32).astype(np.float64), a)

    for k in ("a_attn", "Q", "K", "V", "O", "a_mlp", "U"):
        assert is_bf16(tr[k]), k
    for k in ("h_read", "h_attn", "h_out"):
        assert is_f32(tr[k]), k
        assert not is_bf16(tr[k]), f"{k} should carry more than bf16 precision"
    assert is_f32(A) and is_f32(z)
    y, _, _ = oracle.forward_sequential(inp, A0, z0)
    assert is_bf16(y)
    # y is the last layer's stream rounded once: recompute segment 0 by hand
    h0 = o.node_input(0)
    for l in range(cfg.n_layers):
        h0, _, _ = o.node(l, h0, A0[l], z0[l])
    np.testing.assert_array_equal(y[:cfg.seg_len], oracle.round_bf16(h0[:cfg.seg_len]))


@pytest.mark.parametrize("name,bar_y,bar_state", [("tiny_fp32", 1e-6, 1e-6), ("small_bf16", 2e-3, 1e-4)])
def test_oracle_own_rounding_error_is_far_below_the_parity_bars(name, bar_y, bar_state):
    """The same oracle run with float32 arithmetic stays within 1/100 (fp32
    workload, bar 1e-4) and 1/10 (bf16 workload, bar 2e-2; its gap comes from
    bf16 rounding decisions flipping) of the parity bars of the float64
    oracle, so the oracle's own rounding cannot decide a parity test."""
    cfg = get_config(name)
    inp = make_inputs(cfg)
    A0, z0 = make_state(cfg)
    ref = oracle.forward_sequential(inp, A0, z0)
    with oracle.working_precision(np.float32):
        low = oracle.forward_sequential(inp, A0, z0)
    assert all(a.dtype == np.float32 for a in low)
    again = oracle.forward_sequential(inp, A0, z0)      # back in float64, unchanged
    for a, b in zip(ref, again):
        assert a.dtype == np.float64
        np.testing.assert_array_equal(a, b)

    def rel(a, b):
        return np.linalg.norm(a.astype(np.float64) - b) / np.linalg.norm(b)
    assert rel(low[0], ref[0]) < bar_y
    assert rel(low[1], ref[1]) < bar_state
    assert rel(low[2], ref[2]) < bar_state


# ---------------------------------------------------------------------------
# LM head (final RMSNorm + vocabulary projection)
# ---------------------------------------------------------------------------

def test_logits_unit_vector_geometry():
    """With eps = 0 the normalised row is sqrt(d) * y / |y|_2 (RMSNorm puts
    every row on the sphere of radius sqrt(d)); a 3-4-5 row makes it exact:
    sqrt(2) * (0.6, 0.8)."""
    y = np.array([[3.0, 4.0], [-6.0, 8.0]])
    eye = np.eye(2)
    out = oracle.logits(y, np.ones(2), eye, eps=0.0)
    np.testing.assert_allclose(out[0], math.sqrt(2) * np.array([0.6, 0.8]), rtol=1e-15)
    np.testing.assert_allclose(out[1], math.sqrt(2) * np.array([-0.6, 0.8]), rtol=1e-15)
    rng = np.random.default_rng(5)
    y = rng.standard_normal((7, 48)) * rng.uniform(0.1, 10.0, (7, 1))
    out = oracle.logits(y, np.ones(48), np.eye(48), eps=0.0)
    want = math.sqrt(48) * y / np.linalg.norm(y, axis=1, keepdims=True)
    np.testing.assert_allclose(out, want, rtol=1e-13)
    # eps > 0 shrinks every row by sqrt(ms / (ms + eps)) exactly
    eps = 0.25
    ms = np.mean(y * y, axis=1, keepdims=True)
    np.testing.assert_allclose(oracle.logits(y, np.ones(48), np.eye(48), eps=eps),
                               want * np.sqrt(ms / (ms + eps)), rtol=1e-13)


def test_logits_head_orientation_and_gain():
    """Rows of w_lm are vocabulary entries: a one-hot / two-hot head picks (sums)
    coordinates of the normalised row, so a transposed head fails; the gain
    scales coordinates before the head."""
    y = np.array([[3.0, 4.0]])
    b = math.sqrt(2) * np.array([0.6, 0.8])
    w = np.array([[0.0, 1.0], [1.0, 0.0], [1.0, 1.0]])      # V = 3, d = 2
    out = oracle.logits(y, np.ones(2), w, eps=0.0)
    assert out.shape == (1, 3)
    np.testing.assert_allclose(out[0], [b[1], b[0], b[0] + b[1]], rtol=1e-15)
    out = oracle.logits(y, np.array([2.0, -0.5]), w, eps=0.0)
    np.testing.assert_allclose(out[0], [-0.5 * b[1], 2 * b[0], 2 * b[0] - 0.5 * b[1]], rtol=1e-15)


def test_logits_scale_invariance_and_row_independence():
    rng = np.random.default_rng(6)
    y = rng.standard_normal((5, 64))
    g = 1 + 0.1 * rng.standard_normal(64)
    w = 0.02 * rng.standard_normal((40, 64))
    base = oracle.logits(y, g, w, eps=0.0)
    np.testing.assert_allclose(oracle.logits(37.0 * y, g, w, eps=0.0), base, rtol=1e-12, atol=1e-15)
    for r in range(5):
        np.testing.assert_allclose(oracle.logits(y[r:r + 1], g, w, eps=0.0)[0], base[r], rtol=1e-13, atol=1e-15)


def test_logits_bf16_rounds_the_normalised_row_only():
    """bf16 workloads store the normalised row in bf16 (round to nearest even,
    checked against torch's conversion); the product itself is not rounded."""
    y = np.array([[1.0, 2.0, 2.0]])                          # |y| = 3
    b = math.sqrt(3) * np.array([1.0, 2.0, 2.0]) / 3.0
    b16 = torch.tensor(b).to(torch.bfloat16).to(torch.float64).numpy()
    assert not np.array_equal(b16, b)
    out = oracle.logits(y, np.ones(3), np.eye(3), dtype="bf16", eps=0.0)
    np.testing.assert_array_equal(out[0], b16)
    w = np.array([[1.0 / 3.0, 1.0 / 7.0, 1.0]])
    out = oracle.logits(y, np.ones(3), w, dtype="bf16", eps=0.0)
    assert out[0, 0] == pytest.approx(b16[0] / 3.0 + b16[1] / 7.0 + b16[2], rel=1e-15)


# ---------------------------------------------------------------------------
# full-attention comparator (Llama block stack over one causal window)
# ---------------------------------------------------------------------------

def test_llama_forward_against_torch_block_stack():
    """fp32 workload (no rounding points): the comparator over 80 positions is
    the layers' torch-built blocks applied in turn, y = the last stream."""
    cfg = get_config("tiny_fp32").with_(n_heads=4, n_kv_heads=2, n_segments=5)
    inp = make_inputs(cfg)
    y = oracle.llama_forward(inp)
    assert y.shape == (80, cfg.d_model)
    h = inp.x.astype(np.float64)
    for l in range(cfg.n_layers):
        h = _torch_block(inp, l, h)
    np.testing.assert_allclose(y, h, rtol=1e-11, atol=1e-11)


def test_llama_forward_causal_prefix_and_zero_memory_node():
    cfg = get_config("small_bf16").with_(n_segments=3)
    inp = make_inputs(cfg)
    full = oracle.llama_forward(inp)
    part = oracle.llama_forward(inp, rows=57)
    assert part.shape == (57, cfg.d_model)
    np.testing.assert_array_equal(part, oracle.llama_forward(inp, n_tokens=57))
    assert np.mean(part == full[:57]) > 0.99          # BLAS blocking aside, the same rows
    np.testing.assert_allclose(part, full[:57], rtol=0, atol=2 ** -7 * np.abs(full[:57]).max())
    # one segment of the recurrent model from the zero state is the comparator
    # over that segment's rows followed by the memory rows (the read of a zero
    # memory adds exactly 0); its y is the comparator's first T rows
    T = cfg.seg_len
    y_armt, _, _ = oracle.forward_sequential(inp, n_segments=1)
    mixed = dataclasses.replace(inp, x=np.concatenate([inp.x[:T], inp.mem_emb]))
    np.testing.assert_array_equal(oracle.llama_forward(mixed)[:T], y_armt)


# ---------------------------------------------------------------------------
# any sequence length: a short last segment
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,t", [("tiny_fp32", 1), ("tiny_fp32", 9), ("small_bf16", 37)])
def test_short_last_segment_is_a_segment_of_its_own_length(name, t):
    """n_tokens = (S-1) T + t: the first S-1 segments are exactly the (S-1)-segment
    run, and the last is one segment of a model with seg_len = t (same weights)
    started from the state the first S-1 segments leave."""
    cfg = get_config(name).with_(n_segments=3)
    T = cfg.seg_len
    inp = make_inputs(cfg)
    A0, z0 = make_state(cfg)
    N = 2 * T + t
    y, A, z = oracle.forward_sequential(inp, A0, z0, n_tokens=N)
    assert y.shape == (N, cfg.d_model)
    y2, A2, z2 = oracle.forward_sequential(inp, A0, z0, n_segments=2)
    np.testing.assert_array_equal(y[:2 * T], y2)
    short = dataclasses.replace(inp, cfg=cfg.with_(seg_len=t, n_segments=1), x=inp.x[2 * T:N])
    y3, A3, z3 = oracle.forward_sequential(short, A2.astype(np.float32), z2.astype(np.float32))
    np.testing.assert_array_equal(y[2 * T:], y3)
    np.testing.assert_array_equal(A, A3)
    np.testing.assert_array_equal(z, z3)
    # and the schedule is still a pure reordering
    for shuffle in (None, 3):
        yd, Ad, zd = oracle.forward_diagonal(inp, A0, z0, n_tokens=N, shuffle_seed=shuffle)
        np.testing.assert_array_equal(yd, y)
        np.testing.assert_array_equal(Ad, A)
        np.testing.assert_array_equal(zd, z)
