"""Pins of the oracle's per-row primitives and of the whole folded layer (CPU only)."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import expit, softmax

import oracle
import torch_ref
from synth import WORKLOADS, Shape, layer_weights, parent_tree, prefix_kv, step_inputs

# non-square everywhere: D=48, Hq*d=32, qkv_out=64, F=40, G=2, P=7, N=6, B=4
SMALL = Shape(5, 6, 48, 4, 2, 8, 40, 7, rms_eps=1e-6, rope_theta=500.0)


def _small_inputs(seed=0, tree="random", law="lognormal", shape=SMALL):
    w = layer_weights(shape, seed, 0, random_norm=True)
    # larger weights than the workloads so attention and FFN are far from trivial
    for k in ("w_qkv", "w_o", "w_gate_up", "w_down"):
        w[k] = w[k] * 10.0
    pk, pv = prefix_kv(shape, seed, 0)
    inp = step_inputs(shape, seed, 0, tree=tree, child_law=law)
    return w, pk, pv, inp


# ------------------------------------------------------------------ primitives

def test_rms_norm_vs_torch():
    rng = np.random.default_rng(1)
    x, w = rng.standard_normal((5, 33)), rng.standard_normal(33)
    ref = F.rms_norm(torch.tensor(x), (33,), weight=torch.tensor(w), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, w, 1e-5), ref, rtol=1e-13)


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 5, 16))
    pos = np.array([0.0, 7.0, 4099.0])[:, None]
    got = oracle.rope(x, pos, 10000.0)
    ref = torch_ref.rope_complex(torch.tensor(x), torch.tensor(pos), 10000.0).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # position 0 is the identity; the rotation preserves each pair's length
    np.testing.assert_allclose(got[0], x[0], rtol=0, atol=0)
    half = 8
    np.testing.assert_allclose(got[..., :half] ** 2 + got[..., half:] ** 2,
                               x[..., :half] ** 2 + x[..., half:] ** 2, rtol=1e-12)


def test_silu_vs_expit():
    x = np.linspace(-800, 60, 2001)
    np.testing.assert_allclose(oracle.silu(x), x * expit(x), rtol=1e-13, atol=1e-300)


def test_qkv_rows_vs_torch_linear_non_square():
    w, _, _, inp = _small_inputs(1)
    rows = inp["H"].reshape(-1, SMALL.hidden)[[0, 3, 17, 29]]
    pos = np.array([7, 10, 12, 12], dtype=np.float64)
    q, k, v = oracle.qkv_rows(rows, pos, w["ln1"], w["w_qkv"], SMALL)
    x = F.rms_norm(torch.tensor(rows), (SMALL.hidden,), weight=torch.tensor(w["ln1"], dtype=torch.float64),
                   eps=SMALL.rms_eps)
    y = F.linear(x, torch.tensor(w["w_qkv"], dtype=torch.float64))
    Hq, Hkv, d = 4, 2, 8
    qr = torch_ref.rope_complex(y[:, :Hq * d].reshape(4, Hq, d), torch.tensor(pos)[:, None], 500.0)
    kr = torch_ref.rope_complex(y[:, Hq * d:(Hq + Hkv) * d].reshape(4, Hkv, d), torch.tensor(pos)[:, None], 500.0)
    np.testing.assert_allclose(q, qr.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(k, kr.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(v, y[:, (Hq + Hkv) * d:].reshape(4, Hkv, d).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_block_bruteforce_python():
    """Pure-Python softmax attention on a tiny GQA case (Hq=4 over Hkv=2)."""
    sh = Shape(1, 3, 8, 4, 2, 4, 8, 2)
    rng = np.random.default_rng(3)
    Q, K, V = rng.standard_normal((3, 4, 4)), rng.standard_normal((3, 2, 4)), rng.standard_normal((3, 2, 4))
    pk, pv = rng.standard_normal((2, 2, 4)), rng.standard_normal((2, 2, 4))
    got = oracle.attention_block(Q, K, V, pk, pv, sh)
    for n in range(3):
        for h in range(4):
            g = h // 2
            keys = [pk[t, g] for t in range(2)] + [K[m, g] for m in range(3)]
            vals = [pv[t, g] for t in range(2)] + [V[m, g] for m in range(3)]
            s = [sum(Q[n, h, e] * kk[e] for e in range(4)) / 2.0 for kk in keys]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            tot = sum(w)
            for e in range(4):
                ref = sum(w[j] * vals[j][e] for j in range(len(w))) / tot
                assert got[n, h, e] == pytest.approx(ref, rel=1e-12, abs=1e-14)


def test_attention_block_vs_sdpa_and_scipy():
    sh = Shape(1, 6, 8, 6, 2, 16, 8, 9)
    rng = np.random.default_rng(4)
    Q, K, V = rng.standard_normal((6, 6, 16)) * 3, rng.standard_normal((6, 2, 16)), rng.standard_normal((6, 2, 16))
    pk, pv = rng.standard_normal((9, 2, 16)), rng.standard_normal((9, 2, 16))
    got = oracle.attention_block(Q, K, V, pk, pv, sh)
    ref = torch_ref.attention_sdpa(*(torch.tensor(a) for a in (Q, K, V, pk, pv))).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # GQA group of head 5 is KV head 1 (contiguous groups of 3)
    s = np.concatenate([pk[:, 1], K[:, 1]]) @ Q[2, 5] / 4.0
    o = softmax(s) @ np.concatenate([pv[:, 1], V[:, 1]])
    np.testing.assert_allclose(got[2, 5], o, rtol=1e-12)


def test_dense_branch_layer_vs_torch_library_layer():
    w, pk, pv, inp = _small_inputs(2)
    for i in range(SMALL.n_branch):
        got = oracle.dense_branch_layer(inp["H"][i], w, pk, pv, SMALL)
        ref = torch_ref.dense_layer(inp["H"][i], w, pk, pv, SMALL)
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


# ------------------------------------------------------------------ whole layer

def _rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


def test_delta_zero_is_dense_per_branch_verification():
    """[SpecFold summary, §4.3] / [review (ko), 전제와 한계]: as delta goes to 0 every draft is
    recomputed and the pass becomes dense multi-branch verification."""
    w, pk, pv, inp = _small_inputs(3)
    res = oracle.verify_layer(inp["H"], inp["parent"], w, pk, pv, 0.0, SMALL)
    assert not res["fold"].any()
    for i in range(SMALL.n_branch):
        ref = torch_ref.dense_layer(inp["H"][i], w, pk, pv, SMALL)
        np.testing.assert_allclose(res["H_out"][i], ref, rtol=1e-11, atol=1e-11)


def test_delta_infinite_closed_form():
    """Every draft row folds, so every draft inherits main's Q/K/V (attention identical to
    main's) and main's FFN output: each draft's update equals main's update."""
    w, pk, pv, inp = _small_inputs(4)
    res = oracle.verify_layer(inp["H"], inp["parent"], w, pk, pv, np.inf, SMALL)
    assert res["fold"][1:].all()
    upd = res["H_out"] - inp["H"]
    for i in range(1, SMALL.n_branch):
        np.testing.assert_allclose(upd[i], upd[0], rtol=1e-12, atol=1e-12)
    assert res["rec_rows"].size == SMALL.block


def test_identical_draft_gives_identical_output():
    w, pk, pv, inp = _small_inputs(5, tree="chain")
    H = inp["H"].copy()
    H[3] = H[2]
    res = oracle.verify_layer(H, inp["parent"], w, pk, pv, 0.1, SMALL)
    assert res["fold"][3].all()
    assert np.array_equal(res["H_out"][3], res["H_out"][2])


def test_main_branch_is_independent_of_drafts():
    w, pk, pv, inp = _small_inputs(6)
    res = oracle.verify_layer(inp["H"], inp["parent"], w, pk, pv, 0.1, SMALL)
    ref = torch_ref.dense_layer(inp["H"][0], w, pk, pv, SMALL)
    np.testing.assert_allclose(res["H_out"][0], ref, rtol=1e-11, atol=1e-11)
    H2 = inp["H"].copy()
    H2[1:] += 0.3 * np.random.default_rng(0).standard_normal(H2[1:].shape)
    res2 = oracle.verify_layer(H2, inp["parent"], w, pk, pv, 0.1, SMALL)
    np.testing.assert_allclose(res2["H_out"][0], res["H_out"][0], rtol=1e-13, atol=1e-13)


def test_locality_branch_depends_only_on_its_ancestors():
    parent = np.array([-1, 0, 0, 1, 2])     # 3 under 1, 4 under 2
    w, pk, pv, inp = _small_inputs(7)
    from synth.inputs import child_hidden  # noqa: F401  (children rebuilt below)
    H = inp["H"].copy()
    rng = np.random.default_rng(1)
    for i in range(1, 5):
        H[i] = H[parent[i]] + 0.03 * rng.standard_normal(H[i].shape)
    base = oracle.verify_layer(H, parent, w, pk, pv, 0.1, SMALL)["H_out"]
    H2 = H.copy()
    H2[2] += 0.5 * rng.standard_normal(H2[2].shape)     # perturb branch 2 (not an ancestor of 1, 3)
    H2[4] += 0.5 * rng.standard_normal(H2[4].shape)
    moved = oracle.verify_layer(H2, parent, w, pk, pv, 0.1, SMALL)["H_out"]
    for i in (0, 1, 3):
        np.testing.assert_allclose(moved[i], base[i], rtol=1e-13, atol=1e-13)
    assert _rel(moved[2], base[2]) > 1e-3


def test_relabelling_drafts_permutes_outputs():
    parent = np.array([-1, 0, 0, 1, 2])
    w, pk, pv, inp = _small_inputs(8)
    H = inp["H"].copy()
    rng = np.random.default_rng(2)
    for i in range(1, 5):
        H[i] = H[parent[i]] + 0.05 * rng.standard_normal(H[i].shape)
    perm = np.array([0, 2, 1, 4, 3])          # swaps the two subtrees; topological order kept
    new_parent = np.array([-1, 0, 0, 1, 2])   # same shape after relabelling
    a = oracle.verify_layer(H, parent, w, pk, pv, 0.1, SMALL)["H_out"]
    b = oracle.verify_layer(H[perm], new_parent, w, pk, pv, 0.1, SMALL)["H_out"]
    np.testing.assert_allclose(b, a[perm], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tree", ["random", "chain", "star"])
def test_table_inheritance_form_equals_resolved_source_form(tree):
    w, pk, pv, inp = _small_inputs(9, tree=tree)
    for delta in (0.0, 0.05, 0.1, 0.3, np.inf):
        a = oracle.verify_layer(inp["H"], inp["parent"], w, pk, pv, delta, SMALL)["H_out"]
        b = oracle.verify_layer_tables(inp["H"], inp["parent"], w, pk, pv, delta, SMALL)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tree", ["random", "chain"])
def test_parent_state_correction_equals_direct_attention(tree):
    w, pk, pv, inp = _small_inputs(10, tree=tree)
    res = oracle.verify_layer(inp["H"], inp["parent"], w, pk, pv, 0.1, SMALL)
    assert res["fold"][1:].any() and (~res["fold"][1:]).any()
    corr = oracle.folded_attention_by_correction(res["q_c"], res["k_c"], res["v_c"], res["fold"],
                                                 inp["parent"], res["src_slot"], pk, pv, SMALL)
    np.testing.assert_allclose(corr.reshape(res["attn"].shape), res["attn"], rtol=1e-9, atol=1e-10)


def test_stack_delta_infinite_closed_form_and_regating():
    sh = SMALL
    layers = []
    for l in range(3):
        w = layer_weights(sh, 21, l, random_norm=True)
        for k in ("w_qkv", "w_o", "w_gate_up", "w_down"):
            w[k] = w[k] * 10.0
        layers.append((w, *prefix_kv(sh, 21, l)))
    inp = step_inputs(sh, 21, 0)
    H, folds = oracle.stack(inp["H"], inp["parent"], layers, np.inf, sh)
    for i in range(1, sh.n_branch):
        np.testing.assert_allclose(H[i] - inp["H"][i], H[0] - inp["H"][0], rtol=1e-11, atol=1e-11)
    # at a finite threshold each layer gates on its own input: masks are not all the same
    _, folds = oracle.stack(inp["H"], inp["parent"], layers, 0.1, sh)
    assert len(folds) == 3
    assert any(not np.array_equal(folds[0], f) for f in folds[1:])


def test_tiny_workload_runs_and_folds_about_seventy_percent():
    wl = WORKLOADS["tiny"]
    w = layer_weights(wl.shape, wl.base_seed, 0)
    pk, pv = prefix_kv(wl.shape, wl.base_seed, 0)
    inp = step_inputs(wl.shape, wl.base_seed, 0, tree=wl.tree, child_law=wl.child_law)
    assert list(inp["parent"]) == [-1, 0, 1]
    res = oracle.verify_layer(inp["H"], inp["parent"], w, pk, pv, wl.delta, wl.shape)
    frac = res["fold"][1:].mean()
    assert 0.4 < frac < 0.95
    # no draft row sits within 0.02 of the threshold at layer 0
    rho = res["rho"][1:]
    assert np.all(np.abs(rho - 0.1) > 0.015)
