"""Host-side checks of the C ABI (no GPU compute): the library loads, exports
every function include/armt.h declares, its wave scheduler matches the
oracle's enumeration, and invalid arguments return status codes instead of
crashing."""

import ctypes
import os

import pytest

import oracle
from long_context_recurrent_amd import armt as A

LIB = A.library_path()
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libarmt.so not built")


def test_exports_every_declared_symbol():
    lib = A.load_library()
    declared = A.declared_functions()
    assert {"armt_create", "armt_forward_sequential", "armt_forward_diagonal",
            "armt_workspace_size", "armt_destroy", "armt_last_error"} <= set(declared)
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in armt.h but not exported"


@pytest.mark.parametrize("L,S", [(L, S) for L in range(1, 13) for S in range(1, 13)]
                         + [(16, 32), (16, 128), (28, 128), (28, 64), (28, 32)])
def test_native_schedule_matches_oracle(L, S):
    waves = A.armt_wave_schedule(L, S)
    ref = oracle.waves(L, S)
    assert len(waves) == len(ref) == S + L - 1
    for (lo, hi), wave in zip(waves, ref):
        assert [l for (_, l) in wave] == list(range(lo, hi + 1))


def test_schedule_errors():
    with pytest.raises(A.ArmtError) as e:
        A.armt_wave_schedule(0, 4)
    assert e.value.code == -1
    with pytest.raises(A.ArmtError):
        A.armt_wave_schedule(4, 4, cap=3)


def _cfg(**kw):
    base = dict(n_layers=2, d_model=64, n_heads=2, n_kv_heads=2, head_dim=32, ffn_hidden=128,
                seg_len=16, n_mem=4, d_key=64, dtype=A.ARMT_F32, rms_eps=1e-5, rope_theta=1e4, mem_eps=1e-6)
    base.update(kw)
    return A.armt_config(**base)


def test_workspace_size_and_config_validation():
    assert A.armt_workspace_size(_cfg()) > 0
    small = A.armt_workspace_size(_cfg(seg_len=16))
    big = A.armt_workspace_size(_cfg(seg_len=64))
    assert big > small
    cases = [
        (dict(n_layers=0), -1), (dict(d_model=96), -1), (dict(n_kv_heads=3, n_heads=2), -1),
        (dict(head_dim=16, n_heads=4), -2), (dict(d_key=32), -2), (dict(n_mem=65), -2),
        (dict(dtype=7), -1), (dict(rms_eps=0.0), -1), (dict(ffn_hidden=100), -2),
        (dict(dtype=A.ARMT_BF16, seg_len=4090, n_mem=16), -2),
        (dict(dtype=A.ARMT_BF16), -2),                                   # bf16: d_model % 128
        (dict(dtype=A.ARMT_BF16, d_model=4096, n_heads=64, head_dim=64), -2),   # bf16: d_model <= 3072
    ]
    assert A.armt_workspace_size(_cfg(dtype=A.ARMT_BF16, d_model=3072, n_heads=24, head_dim=128)) > 0
    for kw, code in cases:
        with pytest.raises(A.ArmtError) as e:
            A.armt_workspace_size(_cfg(**kw))
        assert e.value.code == code, (kw, e.value)
        assert A.armt_last_error()


def test_create_rejects_bad_arguments_before_any_gpu_work():
    lib = A.load_library()
    cfg = _cfg()
    w = A.armt_weights(*([1024] * 12))
    out = ctypes.c_void_p(0)
    # NULL workspace
    rc = lib.armt_create(ctypes.byref(cfg), ctypes.byref(w), None, 1 << 20, None, ctypes.byref(out))
    assert rc == -3 and out.value is None
    # misaligned and too small
    rc = lib.armt_create(ctypes.byref(cfg), ctypes.byref(w), 4096 + 8, 1 << 30, None, ctypes.byref(out))
    assert rc == -3
    rc = lib.armt_create(ctypes.byref(cfg), ctypes.byref(w), 4096, 16, None, ctypes.byref(out))
    assert rc == -3 and "too small" in A.armt_last_error()
    # a NULL weight pointer
    w2 = A.armt_weights(*([1024] * 11 + [0]))
    rc = lib.armt_create(ctypes.byref(cfg), ctypes.byref(w2), 4096, 1 << 30, None, ctypes.byref(out))
    assert rc == -1
    # NULL handle on the forward entry points and options
    assert lib.armt_forward_diagonal(None, 1, 1, None, None, 1, 1, 1) == -1
    assert lib.armt_forward_sequential(None, 1, 1, None, None, 1, 1, 1) == -1
    assert lib.armt_set_option(None, 0, 1) == -1
    lib.armt_destroy(None)


def test_full_attention_comparator_validation():
    """armt_llama_*: host-side validation (no GPU work): the memory fields of
    the config are ignored, the token count is bounded per dtype, and the
    workspace grows with max_tokens."""
    lib = A.load_library()
    n1 = A.armt_llama_workspace_size(_cfg(), 64)
    n2 = A.armt_llama_workspace_size(_cfg(), 128)
    assert 0 < n1 < n2
    assert A.armt_llama_workspace_size(_cfg(d_key=7, n_mem=0, seg_len=0), 64) == n1
    bf = dict(dtype=A.ARMT_BF16, d_model=2048, n_heads=32, n_kv_heads=8, head_dim=64, ffn_hidden=8192)
    assert A.armt_llama_workspace_size(_cfg(**bf), 131072) > 5e9
    cases = [
        (dict(), 0, -1), (dict(n_layers=0), 64, -1), (dict(d_model=96), 64, -1),
        (dict(head_dim=16, n_heads=4), 64, -2), (dict(), 4097, -2),
        (bf, (1 << 18) + 1, -2), (dict(d_model=8192, n_heads=64, head_dim=128), 64, -2),
        # keys of one sequence beyond 32-bit offsets: 2^18 tokens x 96 heads x 64 x 2 B
        (dict(bf, d_model=2048, n_heads=32, n_kv_heads=32), 1 << 18, -2),
    ]
    for kw, nt, code in cases:
        with pytest.raises(A.ArmtError) as e:
            A.armt_llama_workspace_size(_cfg(**kw), nt)
        assert e.value.code == code, (kw, nt, e.value)
    cfg = _cfg()
    out = ctypes.c_void_p(0)
    w = A.armt_weights(*([1024] * 7 + [0] * 5))        # memory weights may be NULL
    rc = lib.armt_llama_create(ctypes.byref(cfg), ctypes.byref(w), 64, None, 1 << 20, None, ctypes.byref(out))
    assert rc == -3 and out.value is None
    w2 = A.armt_weights(*([1024] * 6 + [0] * 6))       # g_mlp missing
    rc = lib.armt_llama_create(ctypes.byref(cfg), ctypes.byref(w2), 64, 4096, 1 << 30, None, ctypes.byref(out))
    assert rc == -1
    assert lib.armt_llama_forward(None, 1, 1, 1) == -1
    assert lib.armt_logits(None, 1, 1, 1, 1, 8, 1) == -1


def test_batched_workspace_validation():
    base = A.armt_workspace_size(_cfg())
    assert A.armt_workspace_size_batched(_cfg(), 1) == base
    assert A.armt_workspace_size_batched(_cfg(), 3) > 2 * base
    for bad in (0, -2, 1025):
        with pytest.raises(A.ArmtError) as e:
            A.armt_workspace_size_batched(_cfg(), bad)
        assert e.value.code == -1
    lib = A.load_library()
    cfg = _cfg()
    w = A.armt_weights(*([1024] * 12))
    out = ctypes.c_void_p(0)
    assert lib.armt_create_batched(ctypes.byref(cfg), ctypes.byref(w), 0, 4096, 1 << 30, None, ctypes.byref(out)) == -1
    assert lib.armt_create_batched(ctypes.byref(cfg), ctypes.byref(w), 2, None, 1 << 30, None, ctypes.byref(out)) == -3


def test_noalloc_forward_rejects_before_any_gpu_work():
    """armt_forward_diagonal_noalloc validates its config and weights and
    rejects a model whose workspace exceeds the static scratch, with a
    message, before it touches the device."""
    lib = A.load_library()
    w = A.armt_weights(*([1024] * 12))
    assert lib.armt_forward_diagonal_noalloc(None, ctypes.byref(w), 1, 1, None, None, 1, 1, 1, None) == -1
    cfg = _cfg()
    assert lib.armt_forward_diagonal_noalloc(ctypes.byref(cfg), None, 1, 1, None, None, 1, 1, 1, None) == -1
    w2 = A.armt_weights(*([1024] * 11 + [0]))
    assert lib.armt_forward_diagonal_noalloc(ctypes.byref(cfg), ctypes.byref(w2), 1, 1, None, None, 1, 1, 1,
                                             None) == -1
    big = _cfg(n_layers=16, d_model=2048, n_heads=32, n_kv_heads=8, head_dim=64, ffn_hidden=8192,
               seg_len=1024, n_mem=16, dtype=A.ARMT_BF16)
    assert A.armt_workspace_size(big) > 64 << 20
    rc = lib.armt_forward_diagonal_noalloc(ctypes.byref(big), ctypes.byref(w), 1, 1, None, None, 1, 1, 1, None)
    assert rc == -3 and "scratch" in A.armt_last_error()
