"""ctypes binding of libarmt.so with the names of include/armt.h.

Argument marshalling only: every step of the forward runs in the HIP kernels
of libarmt.so.  Device buffers are passed as torch tensors (their data_ptr()),
streams as torch.cuda.Stream or raw handles.  Each function raises ArmtError
with armt_last_error() when the library returns a non-OK status.
"""

from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "ArmtError", "armt_config", "armt_weights", "load_library", "library_path",
    "armt_workspace_size", "armt_create", "armt_workspace_size_batched", "armt_create_batched",
    "armt_forward_sequential",
    "armt_forward_diagonal", "armt_forward_diagonal_noalloc", "armt_forward_sequential_tokens", "armt_forward_diagonal_tokens", "armt_logits", "armt_llama_workspace_size", "armt_llama_create",
    "armt_llama_forward", "armt_backward_workspace_size", "armt_backward", "armt_destroy", "armt_last_error",
    "armt_wave_schedule", "armt_set_option", "armt_kernel_stats",
    "armt_debug_view", "declared_functions",
    "ARMT_F32", "ARMT_BF16", "ARMT_OPT_GRAPHS", "ARMT_OPT_TIME_KERNEL", "ARMT_OPT_GEMM_ROWS", "ARMT_OPT_DEBUG_SYNC",
    "KERNELS", "VIEWS",
]

ARMT_OK, ARMT_E_INVALID, ARMT_E_UNSUPPORTED, ARMT_E_WORKSPACE, ARMT_E_HIP = 0, -1, -2, -3, -4
ARMT_F32, ARMT_BF16 = 0, 1
ARMT_OPT_GRAPHS, ARMT_OPT_TIME_KERNEL, ARMT_OPT_GEMM_ROWS, ARMT_OPT_DEBUG_SYNC = 0, 1, 2, 3
KERNELS = ["mem_read", "attn_norm", "qkv", "attn", "o_proj", "mlp_norm", "gate_up", "down", "mem_keys", "mem_update"]
VIEWS = {"act0": 0, "act1": 1, "normed": 2, "qkv": 3, "vt": 4, "attn": 5, "swiglu": 6, "A": 7, "z": 8}

_PKG = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(_PKG), "include", "armt.h")


class ArmtError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"armt status {code}: {msg}")
        self.code = code


class armt_config(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "n_layers", "d_model", "n_heads", "n_kv_heads", "head_dim", "ffn_hidden",
        "seg_len", "n_mem", "d_key", "dtype")] + [
        ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float), ("mem_eps", ctypes.c_float)]


class armt_weights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "w_qkv", "w_o", "w_gate", "w_up", "w_down", "g_attn", "g_mlp",
        "w_mq", "w_mk", "w_mv", "w_beta", "mem_emb")]


_lib = None


def library_path() -> str:
    """The in-tree libarmt.so, or the library named by ARMT_LIBRARY (a debug
    build of the same sources, e.g. the host-sanitizer build)."""
    return os.environ.get("ARMT_LIBRARY") or os.path.join(_PKG, "libarmt.so")


def load_library():
    """Load libarmt.so from the package directory (built in-tree by
    long_context_recurrent_amd.build).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m long_context_recurrent_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sigs = {
        "armt_workspace_size": (I32, [ctypes.POINTER(armt_config), ctypes.POINTER(SZ)]),
        "armt_create": (I32, [ctypes.POINTER(armt_config), ctypes.POINTER(armt_weights), P, SZ, P,
                              ctypes.POINTER(P)]),
        "armt_workspace_size_batched": (I32, [ctypes.POINTER(armt_config), I32, ctypes.POINTER(SZ)]),
        "armt_create_batched": (I32, [ctypes.POINTER(armt_config), ctypes.POINTER(armt_weights), I32, P, SZ, P,
                                      ctypes.POINTER(P)]),
        "armt_forward_sequential": (I32, [P, P, I32, P, P, P, P, P]),
        "armt_forward_diagonal": (I32, [P, P, I32, P, P, P, P, P]),
        "armt_forward_diagonal_noalloc": (I32, [ctypes.POINTER(armt_config), ctypes.POINTER(armt_weights), P, I32,
                                                P, P, P, P, P, P]),
        "armt_forward_sequential_tokens": (I32, [P, P, ctypes.c_int64, P, P, P, P, P]),
        "armt_forward_diagonal_tokens": (I32, [P, P, ctypes.c_int64, P, P, P, P, P]),
        "armt_logits": (I32, [P, P, ctypes.c_int64, P, P, I32, P]),
        "armt_llama_workspace_size": (I32, [ctypes.POINTER(armt_config), ctypes.c_int64, ctypes.POINTER(SZ)]),
        "armt_llama_create": (I32, [ctypes.POINTER(armt_config), ctypes.POINTER(armt_weights), ctypes.c_int64,
                                    P, SZ, P, ctypes.POINTER(P)]),
        "armt_llama_forward": (I32, [P, P, ctypes.c_int64, P]),
        "armt_backward_workspace_size": (I32, [P, I32, ctypes.POINTER(SZ)]),
        "armt_backward": (I32, [P, I32, P, I32, P, P, P, P, P, P, P, P, ctypes.POINTER(armt_weights), P, SZ]),
        "armt_destroy": (None, [P]),
        "armt_last_error": (ctypes.c_char_p, []),
        "armt_wave_schedule": (I32, [I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32), I32,
                                     ctypes.POINTER(I32)]),
        "armt_set_option": (I32, [P, I32, I32]),
        "armt_kernel_stats": (I32, [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
        "armt_debug_view": (I32, [P, I32, ctypes.POINTER(P), ctypes.POINTER(SZ)]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def declared_functions(header: str = HEADER) -> list:
    """Names of the functions include/armt.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(armt_[a-z_]+)\s*\(", text)))


def _check(code: int):
    if code != ARMT_OK:
        raise ArmtError(code, load_library().armt_last_error().decode())


def _ptr(t):
    """Device pointer of a tensor (or None / int passthrough)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def armt_last_error() -> str:
    return load_library().armt_last_error().decode()


def armt_workspace_size(cfg: armt_config) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().armt_workspace_size(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def armt_create(cfg: armt_config, w: armt_weights, workspace, ws_bytes: int, stream=None):
    h = ctypes.c_void_p(0)
    _check(load_library().armt_create(ctypes.byref(cfg), ctypes.byref(w), _ptr(workspace), ws_bytes,
                                      _stream(stream), ctypes.byref(h)))
    return h.value


def armt_workspace_size_batched(cfg: armt_config, batch: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().armt_workspace_size_batched(ctypes.byref(cfg), batch, ctypes.byref(n)))
    return n.value


def armt_create_batched(cfg: armt_config, w: armt_weights, batch: int, workspace, ws_bytes: int, stream=None):
    h = ctypes.c_void_p(0)
    _check(load_library().armt_create_batched(ctypes.byref(cfg), ctypes.byref(w), batch, _ptr(workspace), ws_bytes,
                                              _stream(stream), ctypes.byref(h)))
    return h.value


def armt_forward_sequential(h, x, n_segments: int, A0, z0, y, A_out, z_out):
    _check(load_library().armt_forward_sequential(h, _ptr(x), n_segments, _ptr(A0), _ptr(z0), _ptr(y),
                                                  _ptr(A_out), _ptr(z_out)))


def armt_forward_diagonal(h, x, n_segments: int, A0, z0, y, A_out, z_out):
    _check(load_library().armt_forward_diagonal(h, _ptr(x), n_segments, _ptr(A0), _ptr(z0), _ptr(y),
                                                _ptr(A_out), _ptr(z_out)))


def armt_forward_diagonal_noalloc(cfg: armt_config, w: armt_weights, x, n_segments: int, A0, z0, y, A_out, z_out,
                                  stream=None):
    _check(load_library().armt_forward_diagonal_noalloc(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), n_segments,
                                                        _ptr(A0), _ptr(z0), _ptr(y), _ptr(A_out), _ptr(z_out),
                                                        _stream(stream)))


def armt_forward_sequential_tokens(h, x, n_tokens: int, A0, z0, y, A_out, z_out):
    _check(load_library().armt_forward_sequential_tokens(h, _ptr(x), n_tokens, _ptr(A0), _ptr(z0), _ptr(y),
                                                         _ptr(A_out), _ptr(z_out)))


def armt_forward_diagonal_tokens(h, x, n_tokens: int, A0, z0, y, A_out, z_out):
    _check(load_library().armt_forward_diagonal_tokens(h, _ptr(x), n_tokens, _ptr(A0), _ptr(z0), _ptr(y),
                                                       _ptr(A_out), _ptr(z_out)))


def armt_logits(h, y, rows: int, g_final, w_lm, vocab: int, logits):
    _check(load_library().armt_logits(h, _ptr(y), rows, _ptr(g_final), _ptr(w_lm), vocab, _ptr(logits)))


def armt_llama_workspace_size(cfg: armt_config, max_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().armt_llama_workspace_size(ctypes.byref(cfg), max_tokens, ctypes.byref(n)))
    return n.value


def armt_llama_create(cfg: armt_config, w: armt_weights, max_tokens: int, workspace, ws_bytes: int,
                      stream=None):
    h = ctypes.c_void_p(0)
    _check(load_library().armt_llama_create(ctypes.byref(cfg), ctypes.byref(w), max_tokens, _ptr(workspace),
                                            ws_bytes, _stream(stream), ctypes.byref(h)))
    return h.value


def armt_llama_forward(h, x, n_tokens: int, y):
    _check(load_library().armt_llama_forward(h, _ptr(x), n_tokens, _ptr(y)))


def armt_backward_workspace_size(h, n_segments: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().armt_backward_workspace_size(h, n_segments, ctypes.byref(n)))
    return n.value


def armt_backward(h, schedule: int, x, n_segments: int, A0, z0, dy, dA_out, dz_out, dx, dA0, dz0,
                  grads: armt_weights, workspace, ws_bytes: int):
    _check(load_library().armt_backward(h, schedule, _ptr(x), n_segments, _ptr(A0), _ptr(z0), _ptr(dy),
                                        _ptr(dA_out), _ptr(dz_out), _ptr(dx), _ptr(dA0), _ptr(dz0),
                                        ctypes.byref(grads), _ptr(workspace), ws_bytes))


def armt_destroy(h):
    if h:
        load_library().armt_destroy(h)


def armt_wave_schedule(n_layers: int, n_segments: int, cap: int | None = None):
    """Returns [(l_lo, l_hi)] per wave (host-only call)."""
    cap = n_layers + n_segments - 1 if cap is None else cap
    cap_c = max(cap, 1)
    lo = (ctypes.c_int32 * cap_c)()
    hi = (ctypes.c_int32 * cap_c)()
    nw = ctypes.c_int32(0)
    _check(load_library().armt_wave_schedule(n_layers, n_segments, lo, hi, cap, ctypes.byref(nw)))
    return [(lo[i], hi[i]) for i in range(nw.value)]


def armt_set_option(h, option: int, value: int):
    _check(load_library().armt_set_option(h, option, value))


def armt_kernel_stats(h):
    ms, fl, by = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_double(0)
    n = ctypes.c_int64(0)
    _check(load_library().armt_kernel_stats(h, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(fl),
                                            ctypes.byref(by)))
    return {"ms": ms.value, "launches": n.value, "flops": fl.value, "bytes": by.value}


def armt_debug_view(h, which):
    which = VIEWS[which] if isinstance(which, str) else which
    p = ctypes.c_void_p(0)
    n = ctypes.c_size_t(0)
    _check(load_library().armt_debug_view(h, which, ctypes.byref(p), ctypes.byref(n)))
    return p.value, n.value
