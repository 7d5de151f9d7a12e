"""GPU parity of the pages' attention-state correction (the comparison variant under variants/).

Folded rows take their parent's retained softmax state and replace the parent's terms at the
child's recomputed positions by the child's [SpecFold summary, App. B, §A.1], level by level
down the tree [§A.3].  The result must be the branch's exact attention: it is compared with
direct fp64 attention from the oracle on the same bf16-rounded projections, and with the
library's prefix-partial + block merge.  States are fp32 with up to P + N terms; the
correction subtracts at most N terms from a denominator that still holds at least the
prefix's, so the bound below (1e-4 relative L2, 2e-3 worst element relative to the row's
largest) leaves two orders of magnitude over the fp32 rounding of these sums.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_case import DEV, LayerCase, dev_bf16, host, rel_l2
from sparse_layer_rho_amd import specfold as sf
from synth import WORKLOADS, Shape, tree_of

pytestmark = pytest.mark.gpu

I32 = torch.int32

CASES = {
    # name: (shape, tree kind or workload, delta)
    "tiny": (None, "tiny", None),
    "layer-1.5b": (None, "layer-1.5b", None),
    "chain-B8": (Shape(9, 32, 256, 4, 2, 128, 256, 96), "chain", 0.3),
    "star-B7-d64": (Shape(8, 16, 256, 8, 2, 64, 256, 200), "star", 0.3),
    "depth4-d32": (Shape(9, 24, 128, 6, 3, 32, 192, 130), "depth4", 0.3),
    "depth3-d16-noprefix": (Shape(7, 8, 64, 4, 2, 16, 128, 0), "depth3", 0.3),
}


def _case(name):
    shape, kind, delta = CASES[name]
    if shape is None:
        case = LayerCase.workload(kind)
        return case, WORKLOADS[kind].delta
    parent = tree_of(kind, shape.n_branch, 31, 0)
    return LayerCase(shape, 31, parent=parent, tree=kind), delta


def _inputs(case, delta):
    sh = case.shape
    R = sh.n_branch * sh.block
    ref = oracle.verify_layer(case.H, case.parent, case.w, case.pk, case.pv, delta, sh)
    M = ref["rec_rows"].size
    qc, kc, vc = (np.asarray(torch.from_numpy(ref[k].astype(np.float32)).to(torch.bfloat16).float(), np.float64)
                  for k in ("q_c", "k_c", "v_c"))

    def pad(x):
        out = np.zeros((R,) + x.shape[1:], np.float32)
        out[:M] = x
        return dev_bf16(out)

    _, pk, pv = case.device()
    dev = {
        "q": pad(qc), "k": pad(kc), "v": pad(vc), "pk": pk, "pv": pv,
        "rec": torch.zeros(R, dtype=I32, device=DEV),
        "cnt": torch.tensor([M], dtype=I32, device=DEV),
        "src": torch.from_numpy(ref["src_slot"].astype(np.int32).ravel()).to(DEV),
        "fold": torch.from_numpy(ref["fold"].astype(np.uint8).ravel()).to(DEV),
    }
    dev["rec"][:M] = torch.from_numpy(ref["rec_rows"].astype(np.int32)).to(DEV)
    direct = np.empty((sh.n_branch, sh.block, sh.n_q_heads, sh.head_dim))
    for i in range(sh.n_branch):
        s = ref["src_slot"][i]
        direct[i] = oracle.attention_block(qc[s], kc[s], vc[s], case.pk, case.pv, sh)
    return ref, dev, direct.reshape(R, sh.n_q_heads, sh.head_dim)


def _run_variant(case, dev):
    from variants import correction as corr

    sh = case.shape
    R = sh.n_branch * sh.block
    state = torch.full(corr.state_shape(sh), float("nan"), device=DEV)
    out = torch.full((R, sh.n_q_heads, sh.head_dim), float("nan"), device=DEV)
    corr.attention(sh, case.parent, dev["q"], dev["k"], dev["v"], dev["rec"], dev["cnt"], dev["src"], dev["fold"],
                   dev["pk"], dev["pv"], state, out)
    torch.cuda.synchronize()
    return host(out), host(state)


@pytest.mark.parametrize("name", list(CASES))
def test_correction_equals_direct_attention(name):
    case, delta = _case(name)
    sh = case.shape
    ref, dev, direct = _inputs(case, delta)
    got, state = _run_variant(case, dev)
    assert np.isfinite(got).all()
    # the case must exercise corrections: folded draft rows whose branch recomputed something
    fold = ref["fold"]
    assert fold[1:].any() and (~fold[1:]).any()
    assert rel_l2(got, direct) < 1e-4
    scale = np.abs(direct).max(axis=-1, keepdims=True)
    assert (np.abs(got - direct) / scale).max() < 2e-3
    # every state's denominator stays positive after the subtractions
    assert (state[..., 1] > 0).all()


@pytest.mark.parametrize("name", ["layer-1.5b", "chain-B8"])
def test_correction_matches_library_merge(name):
    case, delta = _case(name)
    sh = case.shape
    R = sh.n_branch * sh.block
    _, dev, direct = _inputs(case, delta)
    got, _ = _run_variant(case, dev)
    attn = torch.full((R, sh.n_q_heads * sh.head_dim), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = sf.new_workspace(sh)
    sf.folded_attention(sh, dev["q"], dev["k"], dev["v"], dev["rec"], dev["cnt"], dev["src"], dev["pk"], dev["pv"],
                        attn, ws)
    torch.cuda.synchronize()
    lib = host(attn).reshape(R, sh.n_q_heads, sh.head_dim)
    # the library rounds its output to bf16: both sit within that rounding of the exact result
    assert rel_l2(lib, direct) < 1e-2
    assert rel_l2(got, lib) < 1e-2
