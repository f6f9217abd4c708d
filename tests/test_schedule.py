"""Schedule pins for the oracle's diagonal enumeration (CPU only).

The dependency rule of a layer-level recurrent model -- node (s, l) needs
(s, l-1) and (s-1, l) -- and Lemma 3.1 (S + L - 1 groups, the longest path)
are from the Pith review of arXiv 2506.05229 ("What carries the argument",
"Core claim", assumptions); the RMT counter-example from the Pith verdict
record (skeptic_critique.concrete_test).
"""

import itertools
import json
import os

import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def prmt_deps(s, l):
    """Layer-level recurrence: same segment's previous layer, previous
    segment's same layer."""
    deps = []
    if l > 0:
        deps.append((s, l - 1))
    if s > 0:
        deps.append((s - 1, l))
    return deps


def rmt_deps(s, l, L):
    """Original RMT: besides the layer stack within a segment, every layer of
    segment s consumes the memory produced by the final layer of segment s-1."""
    deps = []
    if l > 0:
        deps.append((s, l - 1))
    if s > 0:
        deps.append((s - 1, L - 1))
    return deps


def longest_path_groups(L, S, deps):
    """Earliest feasible group of every node (0-indexed) = longest dependency
    path ending at it, by brute-force relaxation in (s, l) order."""
    g = {}
    for s in range(S):
        for l in range(L):
            g[(s, l)] = 0
    changed = True
    while changed:
        changed = False
        for node in g:
            for d in deps(*node):
                if g[node] < g[d] + 1:
                    g[node] = g[d] + 1
                    changed = True
    return g


@pytest.mark.parametrize("L,S", [(L, S) for L in range(1, 13) for S in range(1, 13)])
def test_waves_brute_force(L, S):
    ws = oracle.waves(L, S)
    # S + L - 1 waves (Lemma 3.1)
    assert len(ws) == S + L - 1
    seen = {}
    for i, wave in enumerate(ws):
        assert len(wave) >= 1
        for node in wave:
            assert node not in seen, "node scheduled twice"
            seen[node] = i
    # every node exactly once
    assert set(seen) == {(s, l) for s in range(S) for l in range(L)}
    for node, i in seen.items():
        # every dependency sits in a strictly earlier wave
        for d in prmt_deps(*node):
            assert seen[d] < i
    # no two nodes of one wave depend on each other (even transitively:
    # wave members share s + l, and every edge raises s + l by one)
    for wave in ws:
        for a, b in itertools.combinations(wave, 2):
            assert b not in prmt_deps(*a) and a not in prmt_deps(*b)
    # the wave count equals the longest path, i.e. it is minimal
    g = longest_path_groups(L, S, lambda s, l: prmt_deps(s, l))
    assert max(g.values()) + 1 == len(ws)
    # and each node sits at its earliest feasible group
    for node, i in seen.items():
        assert g[node] == i


def test_special_cases():
    assert len(oracle.waves(1, 7)) == 7          # one layer: S waves
    assert len(oracle.waves(5, 1)) == 5          # one segment: L waves
    assert all(len(w) == 1 for w in oracle.waves(1, 7))
    assert all(len(w) == 1 for w in oracle.waves(5, 1))


def test_lemma31_group_counts_golden():
    with open(os.path.join(GOLDEN, "lemma31_group_counts.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        L, S = case["n_layers"], case["n_segments"]
        ws = oracle.waves(L, S)
        assert len(ws) == case["groups"]
        assert sum(len(w) for w in ws) == case["sequential_steps"]


def test_rmt_counterexample_golden():
    """The diagonal schedule must be rejected for the original RMT graph, and
    the first node it gets wrong is the printed one."""
    with open(os.path.join(GOLDEN, "rmt_counterexample.json")) as f:
        gold = json.load(f)
    L, S = gold["n_layers"], gold["n_segments"]
    diag_group = {}
    for i, wave in enumerate(oracle.waves(L, S)):
        for node in wave:
            diag_group[node] = i
    deps = lambda s, l: rmt_deps(s, l, L)  # noqa: E731
    violations = sorted(
        (diag_group[node], node) for node in diag_group
        if any(diag_group[d] >= diag_group[node] for d in deps(*node)))
    assert violations, "diagonal schedule must violate the RMT graph"
    first_group, (s, l) = violations[0]
    # printed values are 1-indexed
    assert (s + 1, l + 1) == (gold["node"]["segment"], gold["node"]["layer"])
    assert first_group + 1 == gold["diagonal_group"]
    dep = (gold["depends_on"]["segment"] - 1, gold["depends_on"]["layer"] - 1)
    assert dep in deps(s, l)
    g = longest_path_groups(L, S, deps)
    assert g[(s, l)] + 1 >= gold["earliest_group_at_least"]
    # the same grid under the layer-level rule is accepted
    for node, i in diag_group.items():
        assert all(diag_group[d] < i for d in prmt_deps(*node))
