"""GPU parity of the full-attention comparator (armt_llama_*: the recurrent
model's Llama-shaped blocks, no memory, one causal window over the whole
sequence -- the baseline of the paper page's abstract and the Pith review's
Figure 1) through the C ABI against the oracle's ``llama_forward``.

Bars as for the recurrent forward (relative L2 1e-4 fp32, 2e-2 bf16).  Causal
attention makes the first r outputs independent of later tokens, so at full
length (131,072 tokens of the 1B shape) the oracle checks prefix rows, and
shorter runs must give bitwise prefixes of longer ones.
"""

import gc
import sys
import time

import numpy as np
import pytest
import torch

import oracle
from armt_inputs import get_config, make_head, make_inputs
from long_context_recurrent_amd import armt as C
from long_context_recurrent_amd.model import FullAttentionModel, make_config

from gpu_util import build_model, rel_l2, to_device, to_np, tol

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


def build_full(inp, max_tokens, device="cuda"):
    c = inp.cfg
    L = inp.weights["w_qkv"].shape[0]
    ccfg = make_config(L, c.d_model, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn_hidden,
                       c.seg_len, c.n_mem, c.d_key, c.dtype, c.rms_eps, c.rope_theta, c.mem_eps)
    w = {k: to_device(inp.weights[k], c, device) for k in ("w_qkv", "w_o", "w_gate", "w_up", "w_down")}
    w["g_attn"] = to_device(inp.g_attn, c, device)
    w["g_mlp"] = to_device(inp.g_mlp, c, device)
    return FullAttentionModel(ccfg, w, max_tokens)


@pytest.mark.parametrize("cfg,N", [(TINY, 64), (TINY, 37), (SMALL, 2048), (SMALL, 1000), (MID64, 1000),
                                   (MID128, 480), (MID32, 450)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_full_attention_parity(cfg, N):
    say(f"[full attention] {cfg.name} N={N}")
    inp = make_inputs(cfg)
    assert inp.x.shape[0] >= N
    model = build_full(inp, max_tokens=inp.x.shape[0])
    x = to_device(inp.x[:N], cfg)
    y = model.forward(x)
    t0 = time.time()
    ref = oracle.llama_forward(inp, n_tokens=N)
    e = rel_l2(to_np(y), ref)
    say(f"  rel L2 {e:.2e} (oracle {time.time() - t0:.1f}s)")
    assert e <= tol(cfg)
    yn = to_np(y)
    for r in (0, N // 3, N - 1):
        assert rel_l2(yn[r], ref[r]) <= tol(cfg), f"row {r}"
    # a second call on the same handle gives the same bits
    assert torch.equal(model.forward(x), y)


def test_full_attention_prefix_and_lengths():
    """Every position depends only on positions at or before it, and the GEMM
    tile height never changes a result: a shorter run is a bitwise prefix of a
    longer one, whatever the lengths (ragged against every tile size)."""
    cfg = MID64
    inp = make_inputs(cfg)
    N = inp.x.shape[0]
    model = build_full(inp, max_tokens=N)
    x = to_device(inp.x, cfg)
    full = model.forward(x).clone()
    for n in (1, 63, 64, 129, 777):
        part = model.forward(x[:n].contiguous())
        assert torch.equal(part, full[:n]), f"prefix of length {n} differs"
    for rb in (4, 9, 13, 14):
        model.set_option(C.ARMT_OPT_GEMM_ROWS, rb)
        assert torch.equal(model.forward(x), full), f"GEMM rows {16 * rb} changed the result"


def test_full_attention_logits_and_errors():
    cfg = SMALL
    inp = make_inputs(cfg)
    model = build_full(inp, max_tokens=600)
    x = to_device(inp.x[:600], cfg)
    y = model.forward(x)
    w_lm, g = make_head(cfg, 1000, gain_std=0.1)
    lg = model.logits(y, to_device(g, cfg), to_device(w_lm, cfg))
    ref = oracle.logits(to_np(y), g, w_lm, cfg.dtype, cfg.rms_eps)
    assert rel_l2(to_np(lg), ref) <= tol(cfg)
    lib = C.load_library()
    h = model.handle
    assert lib.armt_llama_forward(h, x.data_ptr(), 601, y.data_ptr()) == -1
    assert lib.armt_llama_forward(h, x.data_ptr(), 0, y.data_ptr()) == -1
    assert lib.armt_forward_diagonal(h, x.data_ptr(), 1, None, None, y.data_ptr(), y.data_ptr(),
                                     y.data_ptr()) == -1
    assert "full-attention" in C.armt_last_error()
    rec = build_model(make_inputs(SMALL.with_(n_segments=1)))
    assert lib.armt_llama_forward(rec.handle, x.data_ptr(), 10, y.data_ptr()) == -1
    # still usable
    assert torch.equal(model.forward(x), y)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_full_attention_1b_131k():
    """The 1B shape over 131,072 tokens, as the benchmark runs it: the first
    48 positions against the oracle; the first 16,384 positions bitwise equal
    to a 16,384-token run; everything finite."""
    cfg = get_config("1b_s128")
    t0 = time.time()
    inp = make_inputs(cfg)
    say(f"[full attention 1b] inputs drawn in {time.time() - t0:.1f}s")
    N = cfg.n_segments * cfg.seg_len
    model = build_full(inp, max_tokens=N)
    x = to_device(inp.x, cfg)
    t0 = time.time()
    y = model.forward(x)
    say(f"[full attention 1b] N={N} forward in {time.time() - t0:.2f}s")
    assert torch.isfinite(y).all()
    short = model.forward(x[:16384].contiguous())
    assert torch.equal(short, y[:16384])
    ref = oracle.llama_forward(inp, n_tokens=N, rows=48)
    e = rel_l2(to_np(y[:48]), ref)
    say(f"  rows 0..47: rel L2 {e:.2e}")
    assert e <= tol(cfg)
    model.close()
    del model, x, y, short
    gc.collect()
    torch.cuda.empty_cache()
