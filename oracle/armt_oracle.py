"""Plain CPU oracle for the diagonal-batching forward of a layer-level recurrent
memory transformer (ARMT).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run this module.  It shares no code
with the HIP library: it is NumPy on the host, float64 by default, slow and
written to be read against the pages:

  * paper page "Diagonal Batching Unlocks Parallelism in Recurrent Memory
    Transformers for Long Contexts" (abstract);
  * skill page "Diagonal Batching for Recurrent Memory Transformers" (Core
    Concept, Implementation, Practical Guidance);
  * Pith review of arXiv 2506.05229 ("What carries the argument", "Extended
    reading notes", referee report, assumptions, Figures 1-6);
  * Pith verdict record for arXiv 2506.05229 (skeptic_critique.concrete_test).

The pages define the schedule exactly and name the model family (ARMT, an
associative-memory PRMT) but print none of its layer or memory equations.  The
node below follows the plainest reading the rest supports: a Llama-shaped block
(RMSNorm, RoPE, grouped-query causal attention, SwiGLU, no biases) whose input
first reads a per-layer associative memory (A_l, z_l) with phi = elu + 1 keys,
and whose memory-token outputs then update that memory with a gated delta rule.
Every such reading is listed with the design notes of this repository.

Precision: arithmetic in float64.  For bf16 workloads (bf16 weights and
activations, fp32 accumulation) the branch activations are rounded to
bfloat16 (round to nearest even, directly from float64) where they are stored:
each RMSNorm output, Q/K after RoPE and V, the attention output and the SwiGLU
product.  The residual stream -- the node's hidden state h, which accumulates
the memory read and every branch output across layers -- is stored in float32
(after the memory read and after each residual add), and the output y is that
stream rounded once to bfloat16.  (With a bfloat16 residual stream the rounding
noise alone compounds with depth: two equally valid bf16 implementations then
differ by ~2e-2 relative L2 after 28 layers of the 3B shape.)  The memory state
(A, z) is stored in float32 after every update.  For fp32 workloads every value
stays in float64.

Pins (tests marked "not gpu"): the oracle rerun in float32 arithmetic
(``working_precision``) stays far inside the parity bars of the float64 run;
schedule brute force and Lemma 3.1; the RMT
counter-example of the Pith verdict; diagonal == sequential order bitwise and
wave-shuffle invariance; split (resume) invariance; hand-derived closed forms of
the memory read and write; the zero-memory node against torch's library
routines (rms_norm, scaled_dot_product_attention, silu, linear); RoPE against
complex rotation plus its norm and relative-position invariants; bf16 rounding
against torch's conversion; phi against torch's elu; the logits' closed forms
(permutation and one-hot heads, constant rows, gain and scale behaviour); the
full-attention comparator against a block stack built from torch's library
routines, its causal prefix property, and equality with a zero-memory node.  No function here is
"parity unpinned" with respect to the stated reading; the reading itself (the
ARMT memory equations) cannot be pinned to the authors' model, which the pages
do not print.
"""

from __future__ import annotations

import contextlib
import math

import numpy as np

# Working precision of every arithmetic step.  float64 always, except inside
# ``working_precision`` (used by the tests to bound the oracle's own rounding
# error by rerunning it in float32).
_WP = np.float64


@contextlib.contextmanager
def working_precision(dtype):
    """Run the oracle's arithmetic in ``dtype`` inside this block."""
    global _WP
    old, _WP = _WP, np.dtype(dtype).type
    try:
        yield
    finally:
        _WP = old

__all__ = [
    "waves", "round_bf16", "phi", "sigmoid", "silu", "rms_norm", "rope",
    "causal_gqa_attention", "mem_read", "mem_write", "node",
    "forward_sequential", "forward_diagonal", "Oracle", "working_precision",
    "logits", "llama_forward",
]


# ---------------------------------------------------------------------------
# Schedule
# ---------------------------------------------------------------------------

def waves(n_layers: int, n_segments: int):
    """Diagonal enumeration of the (segment, layer) grid.

    Wave i holds every node (s, l) with s + l = i, 0 <= s < S, 0 <= l < L; there
    are S + L - 1 waves (Pith review, "What carries the argument" and "Core
    claim", Lemma 3.1; skill page, Implementation: positions with constant
    segment + layer can run in parallel).  Nodes inside a wave are listed by
    increasing layer.
    """
    out = []
    for i in range(n_segments + n_layers - 1):
        wave = []
        for l in range(n_layers):
            s = i - l
            if 0 <= s < n_segments:
                wave.append((s, l))
        out.append(wave)
    return out


# ---------------------------------------------------------------------------
# Element-wise definitions
# ---------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as
    float64.  bfloat16 keeps 8 significant bits and float32's exponent range;
    values beyond its largest finite value become +-inf."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    # quantum of the 8-bit significand, floored at the smallest subnormal 2**-133
    q_exp = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x, -q_exp)), q_exp)   # np.rint: half to even
    big = np.abs(r) > 3.3895313892515355e38             # largest finite bf16
    r = np.where(big, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x).astype(_WP)


def _identity(x):
    return np.asarray(x, dtype=_WP)


def _round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(_WP)


def phi(u):
    """Feature map of the associative memory, elu(u) + 1: u + 1 for u > 0, else
    exp(u).  Strictly positive, so memory denominators stay positive."""
    u = np.asarray(u, dtype=_WP)
    return np.where(u > 0, u + 1.0, np.exp(np.minimum(u, 0.0))).astype(_WP)


def sigmoid(u):
    u = np.asarray(u, dtype=_WP)
    e = np.exp(-np.abs(u))
    return np.where(u >= 0, 1.0 / (1.0 + e), e / (1.0 + e)).astype(_WP)


def silu(u):
    return np.asarray(u, dtype=_WP) * sigmoid(u)


def rms_norm(h, g, eps):
    """h / sqrt(mean(h^2) + eps) * g over the last axis (Llama RMSNorm)."""
    h = np.asarray(h, dtype=_WP)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return (h / np.sqrt(ms + _WP(eps)) * np.asarray(g, dtype=_WP)).astype(_WP)


def rope(x, theta):
    """Rotary position embedding on x [n, heads, hd], positions 0..n-1.

    Half-split pairing: coordinate i is paired with i + hd/2 and the pair is
    rotated by angle pos * theta**(-2i/hd) (Llama convention)."""
    x = np.asarray(x, dtype=_WP)
    n, _, hd = x.shape
    half = hd // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / hd)
    ang = np.arange(n, dtype=np.float64)[:, None] * inv_freq[None, :]     # [n, half]
    cos = np.cos(ang).astype(_WP)[:, None, :]
    sin = np.sin(ang).astype(_WP)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def causal_gqa_attention(Q, K, V):
    """softmax(Q K^T / sqrt(hd) + causal mask) V per query head.

    Q [n, H, hd], K and V [n, G, hd]; query head j reads key/value head
    j // (H/G) (contiguous groups).  Returns [n, H*hd].  Each node attends only
    over its own n rows (segment tokens then memory tokens)."""
    n, H, hd = Q.shape
    G = K.shape[1]
    rep = H // G
    out = np.empty((n, H, hd), dtype=_WP)
    mask = np.triu(np.ones((n, n), dtype=bool), k=1)
    for j in range(H):
        kv = j // rep
        s = (Q[:, j, :] @ K[:, kv, :].T) / _WP(math.sqrt(hd))
        s = np.where(mask, -np.inf, s)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, j, :] = p @ V[:, kv, :]
    return out.reshape(n, H * hd)


# ---------------------------------------------------------------------------
# Associative memory (read, gated delta-rule write)
# ---------------------------------------------------------------------------

def mem_read(h, w_mq, A, z, eps):
    """Read of the layer's associative memory, added to the residual stream.

    q = phi(h W_mq^T) [rows, d_k];  r = (q A^T) / (q . z + eps);  return h + r.
    A is [d, d_k], z is [d_k].  From the zero state the read is exactly 0."""
    h = np.asarray(h, dtype=_WP)
    q = phi(h @ np.asarray(w_mq, dtype=_WP).T)
    num = q @ np.asarray(A, dtype=_WP).T
    den = q @ np.asarray(z, dtype=_WP) + _WP(eps)
    return h + num / den[:, None]


def mem_write(y_mem, w_mk, w_mv, w_beta, A, z, eps):
    """Gated delta-rule update of (A, z) from the memory-token outputs.

    k_m = phi(y_m W_mk^T), v_m = y_m W_mv^T, beta_m = sigmoid(y_m . w_beta);
    vbar_m = (k_m A^T) / (k_m . z + eps) is what the pre-update memory returns
    for k_m; then A += sum_m beta_m (v_m - vbar_m) k_m^T and z += sum_m k_m.
    All tokens of one write see the pre-update state.  Returns new (A, z)."""
    y = np.asarray(y_mem, dtype=_WP)
    A = np.asarray(A, dtype=_WP)
    z = np.asarray(z, dtype=_WP)
    k = phi(y @ np.asarray(w_mk, dtype=_WP).T)                 # [M, d_k]
    v = y @ np.asarray(w_mv, dtype=_WP).T                      # [M, d]
    beta = sigmoid(y @ np.asarray(w_beta, dtype=_WP))          # [M]
    vbar = (k @ A.T) / (k @ z + _WP(eps))[:, None]             # [M, d]
    A_new = A + ((beta[:, None] * (v - vbar)).T @ k)           # [d, d_k]
    z_new = z + k.sum(axis=0)
    return A_new, z_new


# ---------------------------------------------------------------------------
# One node of the grid and the two schedules
# ---------------------------------------------------------------------------

class Oracle:
    """Holds a workload's weights (float64 copies are made per layer on use)
    and runs nodes.  ``inputs`` is an ``armt_inputs.ArmtInputs``-like object
    with fields cfg, x, mem_emb, weights (name -> [L, ...]), g_attn, g_mlp."""

    def __init__(self, inputs):
        self.inp = inputs
        self.cfg = inputs.cfg
        self.dtype = _WP
        bf = self.cfg.dtype == "bf16"
        self.R = round_bf16 if bf else _identity         # branch activations
        self.Rs = _round_f32 if bf else _identity        # residual stream
        self.n_tokens = inputs.x.shape[0]                # sequence length (run() sets it)

    def w(self, name, l):
        return np.asarray(self.inp.weights[name][l], dtype=self.dtype)

    def seg_tokens(self, s):
        """Tokens of segment s: T, or fewer in a short last segment."""
        T = self.cfg.seg_len
        return min(T, self.n_tokens - s * T)

    def node_input(self, s, prev=None):
        """Layer-0 input of segment s: its T token rows (fewer in a short last
        segment), then the M memory token rows; deeper layers take the
        previous layer's node output."""
        if prev is not None:
            return prev
        T = self.cfg.seg_len
        x = np.asarray(self.inp.x[s * T:s * T + self.seg_tokens(s)], dtype=self.dtype)
        return np.concatenate([x, np.asarray(self.inp.mem_emb, dtype=self.dtype)], axis=0)

    def node(self, l, h_in, A, z, rows=None, trace=None):
        """Node (s, l): memory read, attention block, MLP block, memory write.

        Returns (h_out, A_new, z_new).  With ``rows`` = r < n only the first r
        rows are computed (causal attention makes them independent of later
        rows) and the memory write is skipped (A_new, z_new are None).  A dict
        passed as ``trace`` receives the intermediate values by name."""
        c, Rs = self.cfg, self.Rs
        h = np.asarray(h_in, dtype=self.dtype)
        n_in = h.shape[0]
        if rows is not None:
            h = h[:rows]
        # 1. memory read
        h = Rs(mem_read(h, self.w("w_mq", l), A, z, c.mem_eps))
        if trace is not None:
            trace.update(h_read=h)
        # 2-3. attention and MLP blocks
        h = self.block(l, h, trace)
        if rows is not None:
            return h, None, None
        # 4. memory write from the memory-token rows (the node's last M rows)
        A_new, z_new = mem_write(h[n_in - c.n_mem:], self.w("w_mk", l), self.w("w_mv", l),
                                 self.w("w_beta", l), A, z, c.mem_eps)
        return h, _round_f32(A_new), _round_f32(z_new)

    def block(self, l, h, trace=None):
        """Layer l's Llama-shaped block on the residual stream h [n, d] (rows
        are positions 0..n-1): pre-norm causal GQA attention with RoPE, then
        a pre-norm SwiGLU MLP, each added to the stream."""
        c, R, Rs = self.cfg, self.R, self.Rs
        H, G, hd = c.n_heads, c.n_kv_heads, c.head_dim
        n = h.shape[0]
        # attention block
        a = R(rms_norm(h, self.inp.g_attn[l], c.rms_eps))
        qkv = a @ self.w("w_qkv", l).T
        Q = qkv[:, :H * hd].reshape(n, H, hd)
        K = qkv[:, H * hd:(H + G) * hd].reshape(n, G, hd)
        V = qkv[:, (H + G) * hd:].reshape(n, G, hd)
        Q = R(rope(Q, c.rope_theta))
        K = R(rope(K, c.rope_theta))
        V = R(V)
        O = R(causal_gqa_attention(Q, K, V))
        h = Rs(h + O @ self.w("w_o", l).T)
        h_attn = h
        # MLP block
        b = R(rms_norm(h, self.inp.g_mlp[l], c.rms_eps))
        U = R(silu(b @ self.w("w_gate", l).T) * (b @ self.w("w_up", l).T))
        h = Rs(h + U @ self.w("w_down", l).T)
        if trace is not None:
            trace.update(a_attn=a, Q=Q, K=K, V=V, O=O, h_attn=h_attn, a_mlp=b, U=U, h_out=h)
        return h

    def initial_state(self, A0=None, z0=None):
        c = self.cfg
        L = self.inp.weights["w_qkv"].shape[0]
        A = [np.zeros((c.d_model, c.d_key), dtype=_WP) if A0 is None else _round_f32(A0[l]) for l in range(L)]
        z = [np.zeros(c.d_key, dtype=_WP) if z0 is None else _round_f32(z0[l]) for l in range(L)]
        return A, z

    def run(self, order, n_segments, A0=None, z0=None, n_tokens=None):
        """Run the nodes in ``order`` (a list of (s, l)); every node's inputs
        must already have been produced.  Returns (Y, A, z) with Y [N, d] the
        last layer's segment-token rows (N = S*T, or ``n_tokens`` with a short
        last segment) and A [L, d, d_k], z [L, d_k]."""
        c = self.cfg
        L = self.inp.weights["w_qkv"].shape[0]
        T = c.seg_len
        self.n_tokens = n_segments * T if n_tokens is None else n_tokens
        A, z = self.initial_state(A0, z0)
        out = {}
        Y = np.zeros((self.n_tokens, c.d_model), dtype=_WP)
        for (s, l) in order:
            prev = None if l == 0 else out.pop((s, l - 1))
            h, A[l], z[l] = self.node(l, self.node_input(s, prev), A[l], z[l])
            if l == L - 1:
                ts = self.seg_tokens(s)
                Y[s * T:s * T + ts] = self.R(h[:ts])      # output: the stream, stored once
            else:
                out[(s, l)] = h
        return Y, np.stack(A), np.stack(z)


def _segments(inputs, n_segments, n_tokens):
    T = inputs.cfg.seg_len
    if n_tokens is not None:
        return -(-n_tokens // T)
    return n_segments or inputs.x.shape[0] // T


def forward_sequential(inputs, A0=None, z0=None, n_segments=None, n_tokens=None):
    """Segment-major order: for s: for l: node(s, l) -- the L*S sequential
    steps of the baseline schedule (Pith review, Figure 3).  ``n_tokens``
    runs the first n_tokens rows of x as ceil(n_tokens / T) segments, the
    last one shorter if T does not divide n_tokens."""
    o = Oracle(inputs)
    L = inputs.weights["w_qkv"].shape[0]
    S = _segments(inputs, n_segments, n_tokens)
    order = [(s, l) for s in range(S) for l in range(L)]
    return o.run(order, S, A0, z0, n_tokens)


def forward_diagonal(inputs, A0=None, z0=None, n_segments=None, shuffle_seed=None, n_tokens=None):
    """Wave order: for each diagonal s + l = i, all its nodes (Pith review,
    "What carries the argument").  ``shuffle_seed`` permutes the nodes inside
    every wave, which must not change any result."""
    o = Oracle(inputs)
    L = inputs.weights["w_qkv"].shape[0]
    S = _segments(inputs, n_segments, n_tokens)
    rng = None if shuffle_seed is None else np.random.default_rng(shuffle_seed)
    order = []
    for wave in waves(L, S):
        wave = list(wave)
        if rng is not None:
            rng.shuffle(wave)
        order.extend(wave)
    return o.run(order, S, A0, z0, n_tokens)


def node(inputs, l, h_in, A, z, rows=None):
    """Convenience wrapper: one node of layer l."""
    return Oracle(inputs).node(l, h_in, A, z, rows)


def logits(y, g_final, w_lm, dtype="f32", eps=1e-5):
    """Final RMSNorm and LM head over output rows y [rows, d]: the logits the
    pages compare between the sequential and the diagonal schedule (Pith
    review: falsifier, and the referee report on Table 2's relative logit
    drift).  The normalised row is a branch activation like the block's own
    norm outputs, so bf16 workloads store it rounded to bf16; the product
    accumulates in the working precision and is not rounded."""
    R = round_bf16 if dtype == "bf16" else _identity
    b = R(rms_norm(y, g_final, eps))
    return b @ np.asarray(w_lm, dtype=_WP).T


def llama_forward(inputs, n_tokens=None, rows=None):
    """Full-attention comparator: the same layers' Llama-shaped blocks, with no
    memory, run over the whole sequence as one causal window (positions
    0..N-1) -- the standard-transformer baseline the paper page's abstract
    and the Pith review's Figure 1 compare against.  The stream is stored like
    the recurrent model's (float32 for bf16 workloads) and y = R(h) of the last
    layer.  ``rows`` = r computes only the first r positions, which causal
    attention makes independent of the rest."""
    o = Oracle(inputs)
    L = inputs.weights["w_qkv"].shape[0]
    N = inputs.x.shape[0] if n_tokens is None else n_tokens
    r = N if rows is None else min(rows, N)
    h = o.Rs(np.asarray(inputs.x[:r], dtype=o.dtype))
    for l in range(L):
        h = o.block(l, h)
    return o.R(h)

