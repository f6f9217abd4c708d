"""Torch-facing wrapper around the C ABI: owns the workspace and output
buffers of one libarmt handle.  torch provides device memory and streams only;
the forward runs entirely in libarmt.so."""

from __future__ import annotations

import torch

from . import armt as _c

WEIGHT_FIELDS = ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "g_attn", "g_mlp",
                 "w_mq", "w_mk", "w_mv", "w_beta", "mem_emb")


def make_config(n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_hidden, seg_len, n_mem,
                d_key=64, dtype="bf16", rms_eps=1e-5, rope_theta=10000.0, mem_eps=1e-6):
    return _c.armt_config(n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_hidden, seg_len,
                          n_mem, d_key, _c.ARMT_BF16 if dtype == "bf16" else _c.ARMT_F32,
                          rms_eps, rope_theta, mem_eps)


BLOCK_FIELDS = WEIGHT_FIELDS[:7]     # w_qkv .. g_mlp: all the full-attention comparator uses


class _Handle:
    """Common part of the two handle kinds: weights kept referenced (the
    library borrows them), the workspace, the stream."""

    def _setup(self, cfg, weights: dict, fields, stream, ws_bytes_fn):
        self.cfg = cfg
        self.dtype = torch.bfloat16 if cfg.dtype == _c.ARMT_BF16 else torch.float32
        self.weights = {}
        for k in fields:
            t = weights[k]
            if not (t.is_cuda and t.is_contiguous() and t.dtype == self.dtype):
                raise ValueError(f"weight {k} must be a contiguous {self.dtype} CUDA tensor")
            self.weights[k] = t
        self.device = self.weights["w_qkv"].device
        self.stream = stream if stream is not None else torch.cuda.Stream(device=self.device)
        self.ws_bytes = ws_bytes_fn()
        self.workspace = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=self.device)
        base = self.workspace.data_ptr()
        self.ws_ptr = (base + 255) // 256 * 256
        return _c.armt_weights(*[self.weights[k].data_ptr() if k in self.weights else None
                                 for k in WEIGHT_FIELDS])

    def close(self):
        if getattr(self, "handle", None):
            _c.armt_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def view(self, which: str, dtype=None, shape=None):
        return _view(self, which, dtype, shape)

    def set_option(self, option: int, value: int):
        _c.armt_set_option(self.handle, option, value)

    def logits(self, y: torch.Tensor, g_final: torch.Tensor, w_lm: torch.Tensor, out=None,
               sync: bool = True):
        """Final RMSNorm + LM head: y [rows, d], g_final [d], w_lm [V, d] (device
        tensors of the config dtype) -> fp32 logits [rows, V]."""
        c = self.cfg
        for name, t in (("y", y), ("g_final", g_final), ("w_lm", w_lm)):
            if t.dtype != self.dtype or not t.is_contiguous() or t.device != self.device:
                raise ValueError(f"{name} must be a contiguous device tensor of the config dtype")
        if y.dim() != 2 or y.shape[1] != c.d_model or g_final.shape != (c.d_model,) \
                or w_lm.dim() != 2 or w_lm.shape[1] != c.d_model:
            raise ValueError("shapes: y [rows, d], g_final [d], w_lm [vocab, d]")
        rows, vocab = y.shape[0], w_lm.shape[0]
        if out is None:
            out = torch.empty(rows, vocab, dtype=torch.float32, device=self.device)
        elif out.shape != (rows, vocab) or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 [rows, vocab] tensor")
        self.stream.wait_stream(torch.cuda.current_stream(self.device))
        _c.armt_logits(self.handle, y, rows, g_final, w_lm, vocab, out)
        if sync:
            self.stream.synchronize()
        else:
            torch.cuda.current_stream(self.device).wait_stream(self.stream)
        return out


class ArmtModel(_Handle):
    """One handle: ``weights`` maps the armt_weights field names to contiguous
    device tensors of the config dtype (kept referenced here: the library
    borrows them)."""

    def __init__(self, cfg: _c.armt_config, weights: dict, stream: torch.cuda.Stream | None = None,
                 batch: int = 1):
        self.batch = batch
        w = self._setup(cfg, weights, WEIGHT_FIELDS, stream, lambda: _c.armt_workspace_size_batched(cfg, batch))
        with torch.cuda.device(self.device):
            self.handle = _c.armt_create_batched(cfg, w, batch, self.ws_ptr, self.ws_bytes, self.stream)

    def kernel_stats(self):
        return _c.armt_kernel_stats(self.handle)

    def alloc_outputs(self, n_segments: int, n_tokens: int | None = None):
        """y [rows, d], A [L, d, d_k], z [L, d_k]; with batch B > 1:
        y [B, rows, d], A [L, B, d, d_k], z [L, B, d_k]."""
        c = self.cfg
        rows = n_segments * c.seg_len if n_tokens is None else n_tokens
        lead = () if self.batch == 1 else (self.batch,)
        y = torch.empty(*lead, rows, c.d_model, dtype=self.dtype, device=self.device)
        A = torch.empty(c.n_layers, *lead, c.d_model, c.d_key, dtype=torch.float32, device=self.device)
        z = torch.empty(c.n_layers, *lead, c.d_key, dtype=torch.float32, device=self.device)
        return y, A, z

    def forward(self, x: torch.Tensor, schedule: str = "diagonal", A0=None, z0=None, out=None,
                sync: bool = True, by_tokens: bool | None = None):
        """x [N, d] ([B, N, d] for batch B > 1) device tensor of the config
        dtype.  Returns (y, A, z) (shapes as alloc_outputs).
        N a multiple of seg_len runs through armt_forward_{diagonal,sequential};
        any other N (or by_tokens=True) through the *_tokens entry points
        (a shorter last segment)."""
        c = self.cfg
        want = 2 if self.batch == 1 else 3
        if x.dim() != want or x.shape[-1] != c.d_model or x.shape[-2] < 1 or \
                (want == 3 and x.shape[0] != self.batch):
            raise ValueError("x must be [n_tokens, d_model] ([batch, n_tokens, d_model] for batch > 1)")
        if x.dtype != self.dtype or not x.is_contiguous() or x.device != self.device:
            raise ValueError("x must be a contiguous device tensor of the config dtype")
        N = x.shape[-2]
        if by_tokens is None:
            by_tokens = N % c.seg_len != 0
        S = -(-N // c.seg_len)
        y, A, z = out if out is not None else self.alloc_outputs(S, N)
        for t in (A0, z0):
            if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
                raise ValueError("A0 / z0 must be contiguous float32 device tensors")
        if schedule not in ("diagonal", "sequential"):
            raise ValueError("schedule must be 'diagonal' or 'sequential'")
        if by_tokens:
            fn = _c.armt_forward_diagonal_tokens if schedule == "diagonal" else _c.armt_forward_sequential_tokens
            count = N
        else:
            fn = _c.armt_forward_diagonal if schedule == "diagonal" else _c.armt_forward_sequential
            count = S
        # the library's stream must see the inputs the caller's stream produced
        self.stream.wait_stream(torch.cuda.current_stream(self.device))
        fn(self.handle, x, count, A0, z0, y, A, z)
        if sync:
            self.stream.synchronize()
        else:
            torch.cuda.current_stream(self.device).wait_stream(self.stream)
        return y, A, z


def backward(model: "ArmtModel", x: torch.Tensor, dy: torch.Tensor, A0=None, z0=None, dA_out=None, dz_out=None,
             schedule: str = "diagonal"):
    """Gradients of <y, dy> + <A_out, dA_out> + <z_out, dz_out>: returns
    (dx, dA0, dz0, {weight field: gradient}).  x and dy have the model's
    dtype; every gradient is fp32."""
    c = model.cfg
    if x.dtype != model.dtype or dy.dtype != model.dtype:
        raise ValueError("x and dy must have the model's dtype")
    S = x.shape[0] // c.seg_len
    dev = model.device
    ws_bytes = _c.armt_backward_workspace_size(model.handle, S)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
    ws_ptr = (ws.data_ptr() + 255) // 256 * 256
    grads = {k: torch.empty(model.weights[k].shape, dtype=torch.float32, device=dev) for k in WEIGHT_FIELDS}
    gw = _c.armt_weights(*[grads[k].data_ptr() for k in WEIGHT_FIELDS])
    dx = torch.empty(x.shape, dtype=torch.float32, device=dev)
    dA0 = torch.empty(c.n_layers, c.d_model, c.d_key, dtype=torch.float32, device=dev)
    dz0 = torch.empty(c.n_layers, c.d_key, dtype=torch.float32, device=dev)
    model.stream.wait_stream(torch.cuda.current_stream(dev))
    _c.armt_backward(model.handle, 0 if schedule == "diagonal" else 1, x, S, A0, z0, dy, dA_out, dz_out,
                     dx, dA0, dz0, gw, ws_ptr, ws_bytes)
    model.stream.synchronize()
    del ws
    return dx, dA0, dz0, grads


class FullAttentionModel(_Handle):
    """The full-attention comparator (armt_llama_*): the block weights of the
    recurrent model's layers over one causal window of up to ``max_tokens``."""

    def __init__(self, cfg: _c.armt_config, weights: dict, max_tokens: int,
                 stream: torch.cuda.Stream | None = None):
        self.max_tokens = max_tokens
        w = self._setup(cfg, weights, BLOCK_FIELDS, stream,
                        lambda: _c.armt_llama_workspace_size(cfg, max_tokens))
        with torch.cuda.device(self.device):
            self.handle = _c.armt_llama_create(cfg, w, max_tokens, self.ws_ptr, self.ws_bytes, self.stream)

    def forward(self, x: torch.Tensor, out=None, sync: bool = True):
        """x [N, d] device tensor of the config dtype -> y [N, d]."""
        c = self.cfg
        if x.dim() != 2 or x.shape[1] != c.d_model or not 1 <= x.shape[0] <= self.max_tokens:
            raise ValueError(f"x must be [N, d_model] with 1 <= N <= {self.max_tokens}")
        if x.dtype != self.dtype or not x.is_contiguous() or x.device != self.device:
            raise ValueError("x must be a contiguous device tensor of the config dtype")
        y = out if out is not None else torch.empty_like(x)
        self.stream.wait_stream(torch.cuda.current_stream(self.device))
        _c.armt_llama_forward(self.handle, x, x.shape[0], y)
        if sync:
            self.stream.synchronize()
        else:
            torch.cuda.current_stream(self.device).wait_stream(self.stream)
        return y


def _view(self, which: str, dtype=None, shape=None):
    """Device tensor aliasing an internal workspace buffer (tests only)."""
    ptr, nbytes = _c.armt_debug_view(self.handle, which)
    off = ptr - self.workspace.data_ptr()
    raw = self.workspace[off:off + nbytes]
    dt = dtype or (torch.float32 if which in ("A", "z", "act0", "act1") else self.dtype)
    t = raw.view(dt)
    return t if shape is None else t[: _numel(shape)].view(*shape)


def _numel(shape):
    n = 1
    for s in shape:
        n *= s
    return n
