"""Pins of the oracle's gate, compaction and fold-source resolution (CPU only)."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, parent_tree, step_inputs, tree_of

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gate_cases.json")


def _num(x):
    return float(x) if not isinstance(x, str) else float(x)


def _arr(rows):
    return np.array([[[_num(v) for v in pos] for pos in br] for br in rows], dtype=np.float64)


# ------------------------------------------------------------------ gate

@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"][:40])
def test_gate_golden_hand_worked(case):
    rho, fold = oracle.gate(_arr(case["H"]), np.array(case["parent"]), case["delta"])
    exp_rho = np.array([[_num(v) for v in row] for row in case["rho"]])
    exp_fold = np.array(case["fold"], dtype=bool)
    assert np.array_equal(fold, exp_fold)
    fin = np.isfinite(exp_rho)
    np.testing.assert_allclose(rho[fin], exp_rho[fin], rtol=1e-15, atol=0)
    assert np.array_equal(np.isinf(rho), np.isinf(exp_rho))
    assert np.array_equal(np.isnan(rho), np.isnan(exp_rho))


def test_gate_closed_form_from_generator():
    """Children are built at distance r * |parent| from their parent, so at layer 0 the
    gate's rho must be exactly the drawn r (float64 rounding aside)."""
    wl = WORKLOADS["layer-1.5b"]
    inp = step_inputs(wl.shape, wl.base_seed, 0)
    rho, _ = oracle.gate(inp["H"], inp["parent"], wl.delta)
    known = np.isfinite(inp["r"])
    assert known.sum() > 200
    np.testing.assert_allclose(rho[known], inp["r"][known], rtol=1e-12)
    # unmasked rows are fresh draws: about sqrt(2) away
    unm = inp["unmasked"]
    assert np.all((rho[unm] > 0.9) & (rho[unm] < 2.0))


def test_gate_bruteforce_python_loops():
    rng = np.random.default_rng(5)
    B1, N, D = 4, 5, 7
    H = rng.standard_normal((B1, N, D))
    H[2] = H[1] + 0.05 * rng.standard_normal((N, D))
    parent = np.array([-1, 0, 1, 1])
    delta = 0.3
    rho, fold = oracle.gate(H, parent, delta)
    for i in range(B1):
        for n in range(N):
            if i == 0:
                assert rho[i, n] == 0 and not fold[i, n]
                continue
            p = parent[i]
            a = sum((H[i, n, k] - H[p, n, k]) ** 2 for k in range(D))
            b = sum(H[p, n, k] ** 2 for k in range(D))
            r = math.sqrt(a) / math.sqrt(b)
            assert rho[i, n] == pytest.approx(r, rel=1e-14)
            assert fold[i, n] == (np.float32(r) <= np.float32(delta))


def test_gate_identical_draft_folds_everything():
    wl = WORKLOADS["tiny"]
    inp = step_inputs(wl.shape, wl.base_seed, 0, tree=wl.tree, child_law=wl.child_law)
    H = inp["H"].copy()
    H[2] = H[1]                      # d2 identical to its parent d1
    rho, fold = oracle.gate(H, inp["parent"], 0.0)
    assert np.all(rho[2] == 0) and fold[2].all()
    assert not fold[0].any()


def test_generator_fold_fraction_matches_profile():
    """Layer-0 fold fraction of the 1.5B-shape generator sits near the 72 % target."""
    wl = WORKLOADS["layer-1.5b"]
    fr = []
    for step in range(4):
        inp = step_inputs(wl.shape, wl.base_seed, step)
        _, fold = oracle.gate(inp["H"], inp["parent"], 0.1)
        fr.append(fold[1:].mean())
    assert 0.62 < np.mean(fr) < 0.82


def test_one_token_drafts_structure_and_closed_form():
    """The draft-shape sweep's law: every draft unmasks exactly one position its parent still
    had masked and keeps the parent's committed positions (so the committed sets nest along the
    tree); at layer 0 the gate's rho equals the drawn r on every other row."""
    wl = WORKLOADS["draft-shapes-1.5b"]
    sh = wl.shape
    for kind in wl.tree_sweep:
        par = tree_of(kind, sh.n_branch, wl.base_seed, 0)
        inp = step_inputs(sh, wl.base_seed, 0, child_law=wl.child_law, parent=par)
        com, unm = inp["committed"], inp["unmasked"]
        assert com[0].sum() == 17 and not unm[0].any()
        for i in range(1, sh.n_branch):
            p = par[i]
            assert unm[i].sum() == 1
            u = int(np.flatnonzero(unm[i])[0])
            assert not com[p, u]
            assert np.array_equal(com[i], com[p] | unm[i])
        rho, _ = oracle.gate(inp["H"], par, wl.delta)
        known = np.isfinite(inp["r"])
        np.testing.assert_allclose(rho[known], inp["r"][known], rtol=1e-12)
        assert np.all((rho[unm] > 0.9) & (rho[unm] < 2.0))


def test_one_token_drafts_fold_fraction_depends_on_the_tree():
    """Averaged over steps, the layer-0 fold fraction of one-token drafts lies in the 0.52-0.67
    range the SpecFold summary (§D.2) reports across drafting shapes, and deeper trees (fewer
    masked positions per draft) fold more than seven siblings of main."""
    wl = WORKLOADS["draft-shapes-1.5b"]
    sh = wl.shape
    mean = {}
    for kind in wl.tree_sweep:
        fr = []
        for step in range(12):
            par = tree_of(kind, sh.n_branch, wl.base_seed, step)
            inp = step_inputs(sh, wl.base_seed, step, child_law=wl.child_law, parent=par)
            _, fold = oracle.gate(inp["H"], par, wl.delta)
            fr.append(fold[1:].mean())
        mean[kind] = float(np.mean(fr))
        assert 0.52 <= mean[kind] <= 0.67, (kind, mean[kind])
    assert mean["chain"] > mean["star"] + 0.03


# ------------------------------------------------------------------ compaction

def test_compact_matches_flatnonzero_and_counts():
    rng = np.random.default_rng(7)
    fold = rng.random((6, 9)) < 0.6
    fold[0] = False
    rec, slot, off = oracle.compact(fold)
    np.testing.assert_array_equal(rec, np.flatnonzero(~fold.ravel()))
    inv = np.full(fold.size, -1)
    inv[rec] = np.arange(rec.size)
    np.testing.assert_array_equal(slot, inv)
    assert off[0] == 0 and off[-1] == rec.size
    for i in range(fold.shape[0]):
        seg = rec[off[i]:off[i + 1]]
        assert seg.size == np.count_nonzero(~fold[i])
        assert np.all(seg // fold.shape[1] == i)


def test_compact_all_and_none():
    fold = np.zeros((3, 4), dtype=bool)
    rec, slot, off = oracle.compact(fold)
    assert rec.size == 12 and np.array_equal(slot, np.arange(12))
    fold[1:] = True
    rec, slot, off = oracle.compact(fold)
    assert np.array_equal(rec, np.arange(4)) and list(off) == [0, 4, 4, 4]


# ------------------------------------------------------------------ fold sources

def _ancestors(parent, i):
    out = []
    while i >= 0:
        out.append(i)
        i = int(parent[i]) if i > 0 else -1
    return out


@pytest.mark.parametrize("kind", ["random", "chain", "star"])
def test_resolve_invariants(kind):
    rng = np.random.default_rng(11)
    B1, N = 9, 16
    parent = parent_tree(B1, 3, 0, kind)
    fold = rng.random((B1, N)) < 0.7
    fold[0] = False
    rec, slot, _ = oracle.compact(fold)
    src, src_slot = oracle.resolve(fold, parent, slot)
    for i in range(B1):
        anc = _ancestors(parent, i)
        for n in range(N):
            s = src[i, n]
            assert not fold[s, n]                       # the source recomputed n
            assert s in anc                             # it is i or an ancestor
            for j in anc[: anc.index(s)]:               # everything below it folded n
                assert fold[j, n]
            assert src_slot[i, n] == slot[s * N + n]
            assert rec[src_slot[i, n]] == s * N + n
    assert np.all(src[0] == 0)


def test_resolve_rejects_folded_main():
    fold = np.zeros((2, 3), dtype=bool)
    fold[0, 1] = True
    _, slot, _ = oracle.compact(fold)
    with pytest.raises(ValueError):
        oracle.resolve(fold, np.array([-1, 0]), slot)
