"""CPU checks of the full-length reference samples (tests/golden/fullsize_*.npz)
and of the script that writes them from the oracle.

* The script's wave runner (nodes of a wave in worker processes, each calling
  the oracle's own node) gives results bitwise equal to the oracle's
  segment-major forward, and its state snapshots equal the state of shorter
  runs -- so the stored samples are the oracle's results, not a second
  implementation's.
* Every stored file was written by the oracle and input sources now in the
  tree (their SHA-256 is recorded beside it) and has the workload's shapes.
"""

import json
import os

import numpy as np
import pytest

import oracle
from armt_inputs import get_config, make_inputs, make_sketch

from golden import make_fullsize as mf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
WORKLOADS = ["1b_s32", "1b_s128", "3b_t512", "3b_t1024", "3b_t2048"]


def test_wave_runner_matches_segment_major_oracle(tmp_path):
    cfg = get_config("small_bf16").with_(n_segments=6)
    inp = make_inputs(cfg)
    got = {}
    A, z, snaps = mf.run_waves(inp, 2, lambda s, y: got.__setitem__(s, y), None,
                               snap_after=[3], log=lambda *a, **k: None)
    Y, A_ref, z_ref = oracle.forward_sequential(inp)
    T = cfg.seg_len
    assert sorted(got) == list(range(6))
    for s in range(6):
        assert np.array_equal(got[s], Y[s * T:(s + 1) * T]), s
    assert np.array_equal(np.stack(A), A_ref) and np.array_equal(np.stack(z), z_ref)
    _, A3, z3 = oracle.forward_sequential(inp, n_segments=3)
    assert np.array_equal(np.stack(snaps[3][0]), A3) and np.array_equal(np.stack(snaps[3][1]), z3)


def test_wave_runner_resumes_from_checkpoint(tmp_path):
    cfg = get_config("small_bf16").with_(n_segments=5)
    inp = make_inputs(cfg)
    ck = str(tmp_path / "ck.npz")
    full = {}
    A, z, _ = mf.run_waves(inp, 1, lambda s, y: full.__setitem__(s, y), None, log=lambda *a, **k: None)
    # a checkpoint is written every 8 waves (5 + 4 - 1 = 8 waves here: none
    # before the end), so write one by hand after wave 4 from a partial run
    part = {}
    A4, z4, pend = _partial(inp, 4, part)
    mf._save_ckpt(ck, 5, 4, 4, A4, z4, pend, {}, None)
    resumed = {}
    A2, z2, _ = mf.run_waves(inp, 1, lambda s, y: resumed.__setitem__(s, y), ck, log=lambda *a, **k: None)
    both = {**part, **resumed}
    for s in range(5):
        assert np.array_equal(both[s], full[s])
    assert np.array_equal(np.stack(A2), np.stack(A)) and np.array_equal(np.stack(z2), np.stack(z))


def _partial(inp, n_waves, out):
    """The runner's state after its first n_waves waves (single process)."""
    o = oracle.Oracle(inp)
    L = inp.cfg.n_layers
    T = inp.cfg.seg_len
    A, z = o.initial_state()
    pending = {}
    for i, wave in enumerate(oracle.waves(L, inp.x.shape[0] // T)):
        if i == n_waves:
            break
        for (s, l) in wave:
            h_in = o.node_input(s) if l == 0 else pending.pop((s, l - 1))
            h, A[l], z[l] = o.node(l, h_in, A[l], z[l])
            if l == L - 1:
                out[s] = o.R(h[:T])
            else:
                pending[(s, l)] = h
    return A, z, pending


def test_sketch_is_fixed_and_seeded():
    cfg = get_config("1b_s32")
    a, b = make_sketch(cfg), make_sketch(cfg)
    assert a.shape == (cfg.d_model, 2) and np.array_equal(a, b)
    assert abs(float(a.std()) - 1.0) < 0.05


@pytest.mark.parametrize("name", WORKLOADS)
def test_golden_file_matches_sources_and_shapes(name):
    path = os.path.join(GOLDEN, f"fullsize_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} not written yet (tests/golden/make_fullsize.py)")
    with open(path[:-4] + ".json") as f:
        meta = json.load(f)
    assert meta["sources_sha256"] == mf.source_digests(), \
        "the golden file was written by other oracle / input sources: rerun tests/golden/make_fullsize.py"
    cfg = get_config(name)
    g = np.load(path, allow_pickle=False)
    L, d, dk, T = cfg.n_layers, cfg.d_model, cfg.d_key, cfg.seg_len
    S = cfg.n_segments
    assert int(g["n_segments"]) == S
    assert list(g["rows_seg"]) == [S // 2, S - 1]
    assert g["rows"].shape == (2, mf.ROWS, d) and g["rows"].dtype == np.uint16
    assert g["sketch"].shape == (S, T, 2)
    assert g["A_rows"].shape == (L, d // mf.A_STRIDE, dk)
    assert g["A_sketch"].shape == (L, dk, 2)
    assert g["z"].shape == (L, dk) and g["A_norm"].shape == (L,)
    for k in ("sketch", "A_rows", "A_sketch", "z", "A_norm"):
        assert np.all(np.isfinite(g[k])), k
    # z_l is a sum of phi-keys (phi > 0): every entry positive and growing with S
    assert np.all(g["z"] > 0)
    # the oracle's own spread, where stored: one value per segment / layer,
    # finite and non-negative, with the jitter that produced it recorded
    if "spread" in g:
        assert g["spread"].ndim == 1 and 1 <= len(g["spread"]) <= S
        for k, n in (("spread", None), ("spread_A_rows", L), ("spread_A_sketch", L), ("spread_z", L)):
            if k in g:
                v = g[k]
                assert n is None or v.shape == (n,), k
                assert np.all(np.isfinite(v)) and np.all(v >= 0), k
        assert meta["spread"]["eps"] == mf.JITTER_EPS and meta["spread"]["seed"] == mf.JITTER_SEED
        if g["spread"].shape == (S,):
            assert np.isclose(g["spread"].max(), meta["spread"]["max_segment"])
    # sampled rows agree with the sketch of the same segment
    sk = make_sketch(cfg).astype(np.float64)
    rows = (g["rows"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for i, s in enumerate(g["rows_seg"]):
        np.testing.assert_allclose(rows[i] @ sk, g["sketch"][s][:mf.ROWS], rtol=1e-5, atol=1e-4)


def test_jittered_runner_is_deterministic_and_close():
    """The jittered oracle (a 3e-6 relative jitter before every rounding,
    seeded per node) gives the same result whichever worker runs a node, and
    stays close to -- but not bitwise -- the plain oracle."""
    cfg = get_config("small_bf16").with_(n_segments=4)
    inp = make_inputs(cfg)
    runs = []
    for workers in (1, 2):
        ys = {}
        A, z, _ = mf.run_waves(inp, workers, lambda s, y: ys.__setitem__(s, y), None, jitter=True,
                               log=lambda *a, **k: None)
        runs.append((ys, np.stack(A), np.stack(z)))
    (y1, A1, z1), (y2, A2, z2) = runs
    for s in y1:
        assert np.array_equal(y1[s], y2[s])
    assert np.array_equal(A1, A2) and np.array_equal(z1, z2)
    Y, A_ref, _ = oracle.forward_sequential(inp)
    T = cfg.seg_len
    y_all = np.concatenate([y1[s] for s in range(4)])
    assert not np.array_equal(y_all, Y)
    assert np.linalg.norm(y_all - Y) / np.linalg.norm(Y) < 2e-2
    assert np.linalg.norm(A1 - A_ref) / np.linalg.norm(A_ref) < 2e-2
