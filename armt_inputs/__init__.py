"""Seeded synthetic inputs for the ARMT diagonal-batching forward.

This module is shared by the tests, the benchmark and the CPU oracle's tests.
It holds the workload shapes and a deterministic random generator, and none of
the model's arithmetic: it draws numbers and stores them in the activation
dtype, nothing else.

Workloads (shapes of the 1B/3B Llama-style ARMT models the paper evaluates; the
abstract on the paper page quotes the 131,072-token single-sequence setting,
and the Pith review's Figure 1 caption the 1,024-token segment):

    name          L   d     H/G/hd     F     T     M   S    dtype
    tiny_fp32     2   64    2/2/32     128   16    4   4    f32
    small_bf16    4   256   4/4/64     1024  128   8   16   bf16
    1b_s32        16  2048  32/8/64    8192  1024  16  32   bf16
    1b_s128       16  2048  32/8/64    8192  1024  16  128  bf16
    3b_t512       28  3072  24/8/128   8192  512   16  128  bf16
    3b_t1024      28  3072  24/8/128   8192  1024  16  64   bf16
    3b_t2048      28  3072  24/8/128   8192  2048  16  32   bf16

Draw recipe (seed 0 unless a test says otherwise).  Every tensor has its own
PCG64 stream keyed by ``SeedSequence([seed, index])``; the index is the
tensor's place in this fixed order:

    0  X      [S*T, d]            N(0, 1)      token embeddings of the sequence
    1  E_mem  [M, d]              N(0, 1)      memory-token embeddings
    then for layer l = 0..L-1, index 2 + 9*l + j with j =
    0  W_qkv  [(H+2G)*hd, d]      N(0, 0.02)   rows: Q heads, then K heads, then V heads
    1  W_o    [d, H*hd]           N(0, 0.02)
    2  W_g    [F, d]              N(0, 0.02)
    3  W_u    [F, d]              N(0, 0.02)
    4  W_d    [d, F]              N(0, 0.02)
    5  W_mq   [d_k, d]            N(0, 0.02)
    6  W_mk   [d_k, d]            N(0, 0.02)
    7  W_mv   [d, d]              N(0, 0.02)
    8  w_b    [d]                 N(0, 0.02)
    RMSNorm gains g_attn, g_mlp [L, d] are 1.

Optional non-zero initial memory state (for resume tests), index 2 + 9*L:
    A0 [L, d, d_k] = 128 * N(0, 1);  z0 [L, d_k] = 16 * U(1, 2)   (float32)
    (scaled so that a memory read from it is of the order of the residual
    stream: q.z is about 64*24 and q A^T about 8*128)

Batches of independent sequences: sequence 0 is X above; sequence b >= 1 is
drawn at index 5 + 9*L + b, N(0, 1), same shape; its optional initial state
is ``make_state(cfg, seed=b)``.

LM head (final RMSNorm + vocabulary projection after the last layer; the
pages give no vocabulary size, so V is synthetic, ``HEAD_VOCAB``):
    index 3 + 9*L: W_lm [V, d] N(0, 0.02);  index 4 + 9*L: g_final [d] =
    1 + gain_std * N(0, 1) (gain_std 0 by default: gains of 1, like the layers').

Sketch for sampled full-length checks (no part of the model): index 1,000,003:
    R_sk [d, 2] N(0, 1) float32; a segment's output rows y_s [T, d] are
    summarised as y_s R_sk [T, 2], so a check over every segment stays small.

Matrices are stored row-major as [out_features, in_features].  Values are
drawn in float32 and, for bf16 workloads, rounded once to bfloat16 so that the
GPU path and the oracle consume the same numbers.
"""

from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

__all__ = ["ArmtConfig", "CONFIGS", "get_config", "ArmtInputs", "make_inputs",
           "make_state", "make_head", "make_batch_x", "make_sketch", "HEAD_VOCAB", "WEIGHT_NAMES"]


@dataclasses.dataclass(frozen=True)
class ArmtConfig:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_hidden: int
    seg_len: int
    n_mem: int
    n_segments: int
    d_key: int = 64
    dtype: str = "bf16"          # "bf16" or "f32": activations and weights
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    mem_eps: float = 1e-6

    @property
    def n(self) -> int:          # rows per node: segment tokens then memory tokens
        return self.seg_len + self.n_mem

    @property
    def qkv_dim(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def tokens(self) -> int:
        return self.n_segments * self.seg_len

    def with_(self, **kw) -> "ArmtConfig":
        return dataclasses.replace(self, **kw)

    def node_flops(self) -> dict:
        """Algorithmic FLOPs of one (segment, layer) node, by step.

        Matrix products count 2*m*n*k; causal attention counts the lower
        triangle including the diagonal (n*(n+1)/2 score entries per head) for
        both QK^T and PV.  Element-wise work is not counted.
        """
        n, d, F, dk, M = self.n, self.d_model, self.ffn_hidden, self.d_key, self.n_mem
        H, hd = self.n_heads, self.head_dim
        tri = n * (n + 1) // 2
        return {
            "mem_read": 2 * n * d * dk * 2,
            "qkv": 2 * n * d * self.qkv_dim,
            "attn": 2 * 2 * tri * hd * H,
            "o_proj": 2 * n * (H * hd) * d,
            "gate_up": 2 * n * d * (2 * F),
            "down": 2 * n * F * d,
            "mem_write": 2 * M * d * (2 * dk + d + 1) + 2 * M * dk * d,
        }


CONFIGS = {
    c.name: c for c in [
        ArmtConfig("tiny_fp32", 2, 64, 2, 2, 32, 128, 16, 4, 4, dtype="f32"),
        ArmtConfig("small_bf16", 4, 256, 4, 4, 64, 1024, 128, 8, 16),
        ArmtConfig("1b_s32", 16, 2048, 32, 8, 64, 8192, 1024, 16, 32),
        ArmtConfig("1b_s128", 16, 2048, 32, 8, 64, 8192, 1024, 16, 128),
        ArmtConfig("3b_t512", 28, 3072, 24, 8, 128, 8192, 512, 16, 128),
        ArmtConfig("3b_t1024", 28, 3072, 24, 8, 128, 8192, 1024, 16, 64),
        ArmtConfig("3b_t2048", 28, 3072, 24, 8, 128, 8192, 2048, 16, 32),
    ]
}


def get_config(name: str) -> ArmtConfig:
    return CONFIGS[name]


WEIGHT_NAMES = ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "w_mq", "w_mk", "w_mv", "w_beta")


def _shapes(cfg: ArmtConfig) -> dict:
    d, F, dk = cfg.d_model, cfg.ffn_hidden, cfg.d_key
    return {
        "w_qkv": (cfg.qkv_dim, d), "w_o": (d, cfg.n_heads * cfg.head_dim),
        "w_gate": (F, d), "w_up": (F, d), "w_down": (d, F),
        "w_mq": (dk, d), "w_mk": (dk, d), "w_mv": (d, d), "w_beta": (d,),
    }


def _draw(seed: int, index: int, shape, std: float) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, index])))
    out = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype; returned as float32 values."""
    if dtype == "f32":
        return a
    import torch
    t = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32)
    return t.numpy()


@dataclasses.dataclass
class ArmtInputs:
    """Stacked weights and inputs, all float32 numpy arrays holding values that
    are exactly representable in ``cfg.dtype``."""
    cfg: ArmtConfig
    x: np.ndarray                 # [S*T, d]
    mem_emb: np.ndarray           # [M, d]
    weights: dict                 # name -> [L, ...]
    g_attn: np.ndarray            # [L, d]
    g_mlp: np.ndarray             # [L, d]


def make_inputs(cfg: ArmtConfig, seed: int = 0, n_segments: int | None = None,
                layers: int | None = None, threads: int | None = None) -> ArmtInputs:
    """Draw the inputs of ``cfg`` (see the module docstring for the recipe).

    ``n_segments`` overrides S.  X is filled sequentially from its stream, so
    a shorter draw is a row prefix of a longer one.
    ``layers`` draws only the first ``layers`` layers' weights (same values as
    the full draw for those layers).
    """
    S = cfg.n_segments if n_segments is None else n_segments
    L = cfg.n_layers if layers is None else layers
    d, T, M = cfg.d_model, cfg.seg_len, cfg.n_mem
    shapes = _shapes(cfg)
    jobs = [("x", 0, (S * T, d), 1.0), ("mem_emb", 1, (M, d), 1.0)]
    for l in range(L):
        for j, name in enumerate(WEIGHT_NAMES):
            jobs.append(((name, l), 2 + 9 * l + j, shapes[name], 0.02))
    threads = threads or min(16, os.cpu_count() or 1)

    def run(job):
        key, idx, shape, std = job
        return key, _to_storage(_draw(seed, idx, shape, std), cfg.dtype)

    with _cf.ThreadPoolExecutor(threads) as ex:
        results = dict(ex.map(run, jobs))
    weights = {}
    for name in WEIGHT_NAMES:
        weights[name] = np.stack([results[(name, l)] for l in range(L)])
    ones = np.ones((L, d), dtype=np.float32)
    return ArmtInputs(cfg, results["x"], results["mem_emb"], weights, ones, ones.copy())


def make_state(cfg: ArmtConfig, seed: int = 0, layers: int | None = None):
    """A non-zero initial memory state (A0 [L, d, d_k], z0 [L, d_k], float32)."""
    L = cfg.n_layers if layers is None else layers
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2 + 9 * cfg.n_layers])))
    A0 = (128.0 * rng.standard_normal((L, cfg.d_model, cfg.d_key))).astype(np.float32)
    z0 = (16.0 * rng.uniform(1.0, 2.0, (L, cfg.d_key))).astype(np.float32)
    return A0, z0


# Synthetic vocabulary sizes of the LM head per workload (multiples of 8; the
# small ones leave ragged output tiles).
HEAD_VOCAB = {"tiny_fp32": 100, "small_bf16": 1000, "1b_s32": 32000, "1b_s128": 32000,
              "3b_t512": 32000, "3b_t1024": 32000, "3b_t2048": 32000}


def make_head(cfg: ArmtConfig, vocab: int | None = None, seed: int = 0, gain_std: float = 0.0):
    """LM-head weights (W_lm [V, d], g_final [d]) in the storage dtype."""
    V = HEAD_VOCAB.get(cfg.name, 1000) if vocab is None else vocab
    L = cfg.n_layers
    w_lm = _to_storage(_draw(seed, 3 + 9 * L, (V, cfg.d_model), 0.02), cfg.dtype)
    g = np.ones(cfg.d_model, dtype=np.float32)
    if gain_std:
        g = g + np.float32(gain_std) * _draw(seed, 4 + 9 * L, (cfg.d_model,), 1.0)
    return w_lm, _to_storage(g.astype(np.float32), cfg.dtype)


def make_batch_x(cfg: ArmtConfig, inputs: "ArmtInputs", batch: int, seed: int = 0) -> np.ndarray:
    """Token embeddings of ``batch`` independent sequences, [B, S*T, d]:
    sequence 0 is ``inputs.x``, the others are drawn as the recipe says."""
    rows, d = inputs.x.shape
    out = np.empty((batch, rows, d), dtype=np.float32)
    out[0] = inputs.x
    for b in range(1, batch):
        out[b] = _to_storage(_draw(seed, 5 + 9 * cfg.n_layers + b, (rows, d), 1.0), cfg.dtype)
    return out



SKETCH_INDEX = 1_000_003


def make_sketch(cfg: ArmtConfig, width: int = 2, seed: int = 0) -> np.ndarray:
    """A fixed Gaussian matrix [d, width] (float32) used to summarise output
    rows for the full-length checks; it is test data, not a model weight."""
    return _draw(seed, SKETCH_INDEX, (cfg.d_model, width), 1.0)
