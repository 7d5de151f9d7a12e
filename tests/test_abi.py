"""The C ABI loads, exports every declared symbol, and rejects bad arguments on the host
before launching anything (CPU only: every call here fails validation, so no kernel runs)."""

import ctypes
import os
import re

import pytest

from sparse_layer_rho_amd import specfold as sf
from synth import WORKLOADS

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "specfold.h")
L = sf.lib()
FAKE = 0x10000          # aligned stand-in device address: never dereferenced by failing calls
MISALIGNED = 0x10008


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(specfold_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(sf.EXPORTS)


def test_version_status_and_stages():
    assert L.specfold_version() == 1
    for code in range(-8, 1):
        assert L.specfold_status_str(code)
    assert sf.stage_names()[0] == "gate_rmsnorm"
    assert L.specfold_last_error() == b""
    assert L.specfold_stage_name(99) is None


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workspace_bytes_positive(name):
    assert sf.workspace_bytes(WORKLOADS[name].shape) > 0


def _shape(**kw):
    base = WORKLOADS["tiny"].shape
    vals = {f: getattr(base, f) for f in ("n_branch", "block", "hidden", "n_q_heads", "n_kv_heads",
                                          "head_dim", "ffn", "prefix_len", "rms_eps", "rope_theta")}
    vals.update(kw)
    return sf.Shape(*[vals[f] for f, _ in sf.Shape._fields_])


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=24), -6), (dict(n_q_heads=3), -2), (dict(n_branch=0), -2), (dict(block=65), -6),
    (dict(n_branch=65), -6), (dict(hidden=96), -6), (dict(hidden=5184), -6), (dict(ffn=100), -6), (dict(prefix_len=-1), -2),
    (dict(rope_theta=0.0), -2),
])
def test_workspace_bytes_rejects_bad_shapes(kw, code):
    sh = _shape(**kw)
    assert L.specfold_workspace_bytes(ctypes.byref(sh)) == 0


def _parent(vals):
    arr = (ctypes.c_int32 * len(vals))(*vals)
    return ctypes.cast(arr, ctypes.c_void_p), arr


@pytest.mark.parametrize("par,code", [([0, 0, 1], -3), ([-1, 1, 1], -3), ([-1, 0, 2], -3), ([-1, 0, -1], -3)])
def test_gate_rejects_bad_tree(par, code):
    sh = _shape()
    p, keep = _parent(par)
    st = L.specfold_gate(ctypes.byref(sh), p, FAKE, 0.1, None, FAKE, FAKE * 2, None, None)
    assert st == code


def test_gate_rejects_null_misaligned_alias():
    sh = _shape()
    p, keep = _parent([-1, 0, 1])
    assert L.specfold_gate(ctypes.byref(sh), p, None, 0.1, None, FAKE, FAKE * 2, None, None) == -1
    assert L.specfold_gate(ctypes.byref(sh), p, MISALIGNED, 0.1, None, FAKE, FAKE * 2, None, None) == -4
    # rho and fold overlap
    assert L.specfold_gate(ctypes.byref(sh), p, FAKE * 8, 0.1, None, FAKE, FAKE, None, None) == -7
    assert L.specfold_gate(None, p, FAKE, 0.1, None, FAKE, FAKE * 2, None, None) == -1


def test_compact_and_resolve_validation():
    sh = _shape()
    p, keep = _parent([-1, 0, 1])
    assert L.specfold_compact(ctypes.byref(sh), FAKE, None, FAKE * 2, FAKE * 3, FAKE * 4, None, 0, None) == -1
    assert L.specfold_compact(ctypes.byref(sh), FAKE, FAKE * 2, FAKE * 2, FAKE * 3, FAKE * 4, None, 0, None) == -7
    # past 8192 rows the look-back scan needs its workspace
    big = _shape(n_branch=3, block=8193)
    need = L.specfold_compact_workspace_bytes(ctypes.byref(big))
    assert L.specfold_compact_workspace_bytes(ctypes.byref(sh)) == 0 and need >= 4 * (4 + 1)
    assert L.specfold_compact(ctypes.byref(big), FAKE, 0x100000, 0x200000, 0x300000, 0x400000, None, 0, None) == -5
    assert L.specfold_compact(ctypes.byref(big), FAKE, 0x100000, 0x200000, 0x300000, 0x400000, 0x500000,
                              need - 1, None) == -5
    assert L.specfold_compact(ctypes.byref(big), FAKE, 0x100000, 0x200000, 0x300000, 0x400000, 0x100000,
                              need, None) == -7
    assert L.specfold_resolve_sources(ctypes.byref(sh), p, FAKE, FAKE * 2, FAKE * 3, FAKE * 3, None) == -7
    bad, keep2 = _parent([-1, 5, 1])
    assert L.specfold_resolve_sources(ctypes.byref(sh), bad, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None) == -3


def test_layer_entry_points_reject_small_workspace_and_alias():
    sh = _shape()
    need = L.specfold_workspace_bytes(ctypes.byref(sh))
    ws = 0x40000000
    args = [FAKE * k for k in range(1, 11)]
    # sparse_qkv: too small a workspace
    # (H, inv_rms, rec_rows, rec_count, ln1, w_qkv, q_c, k_c, v_c)
    assert L.specfold_sparse_qkv(ctypes.byref(sh), *args[:9], ws, need - 1, None) == -5
    assert L.specfold_sparse_qkv(ctypes.byref(sh), *args[:9], None, need, None) == -5
    # q_c overlaps k_c
    assert L.specfold_sparse_qkv(ctypes.byref(sh), *args[:6], FAKE * 20, FAKE * 20, FAKE * 30, ws, need, None) == -7
    # out_proj: h_mid == H
    assert L.specfold_out_proj(ctypes.byref(sh), FAKE, FAKE * 2, FAKE * 3, FAKE * 2, ws, need, None) == -7
    # sparse_ffn: H_out == h_mid
    assert L.specfold_sparse_ffn(ctypes.byref(sh), FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, FAKE * 6,
                                 FAKE * 7, FAKE, ws, need, None) == -7


def test_verify_layer_validation():
    sh = _shape()
    need = L.specfold_workspace_bytes(ctypes.byref(sh))
    ws = 0x40000000
    p, keep = _parent([-1, 0, 1])
    w = sf.LayerWeights(*(FAKE * k for k in range(1, 7)))
    pf = sf.PrefixKV(FAKE * 8, FAKE * 9, 32, 16, 32, 16)
    H_in, H_out = 0x20000000, 0x30000000
    call = lambda **kw: L.specfold_verify_layer(
        ctypes.byref(kw.get("sh", sh)), kw.get("p", p), ctypes.byref(kw.get("w", w)), ctypes.byref(kw.get("pf", pf)),
        kw.get("H_in", H_in), 0.1, kw.get("H_out", H_out), None, None, kw.get("ws", ws), kw.get("wsb", need), None)
    assert call(H_out=H_in) == -7
    assert call(wsb=16) == -5
    bad, keep2 = _parent([-1, 0, 3])
    assert call(p=bad) == -3
    assert call(w=sf.LayerWeights(FAKE, None, FAKE, FAKE, FAKE, FAKE)) == -1
    assert call(pf=sf.PrefixKV(FAKE * 8, FAKE * 9, 33, 16, 32, 16)) == -4
    assert call(sh=_shape(block=80)) == -6


def test_head_entry_points_validation():
    sh = _shape()
    V = 1000
    need = L.specfold_head_workspace_bytes(ctypes.byref(sh), V)
    R, D = sh.n_branch * sh.block, sh.hidden
    groups = (V + 63) // 64
    assert need >= R * D * 2 + 2 * groups * R * 4
    assert L.specfold_head_workspace_bytes(ctypes.byref(sh), 0) == 0
    assert L.specfold_head_workspace_bytes(ctypes.byref(_shape(hidden=96)), V) == 0
    ws = 0x40000000
    # (H, ln_f, w_lm, vocab, token, logit, ws, ws_bytes)
    assert L.specfold_lm_head(ctypes.byref(sh), None, FAKE * 2, FAKE * 3, V, FAKE * 4, FAKE * 5, ws, need, None) == -1
    assert L.specfold_lm_head(ctypes.byref(sh), MISALIGNED, FAKE * 2, FAKE * 3, V, FAKE * 4, FAKE * 5, ws, need,
                              None) == -4
    assert L.specfold_lm_head(ctypes.byref(sh), FAKE, FAKE * 2, FAKE * 3, V, FAKE * 4, FAKE * 5, ws, need - 1,
                              None) == -5
    assert L.specfold_lm_head(ctypes.byref(sh), FAKE, FAKE * 2, FAKE * 3, 0, FAKE * 4, FAKE * 5, ws, need, None) == -2
    # token and logit overlap
    assert L.specfold_lm_head(ctypes.byref(sh), FAKE, FAKE * 2, FAKE * 3, V, FAKE * 4, FAKE * 4, ws, need, None) == -7
    # embedding: NULL table, bad vocabulary, output overlapping the table
    assert L.specfold_embed(ctypes.byref(sh), FAKE, None, V, FAKE * 2, None) == -1
    assert L.specfold_embed(ctypes.byref(sh), FAKE, FAKE * 2, 0, FAKE * 3, None) == -2
    assert L.specfold_embed(ctypes.byref(sh), FAKE, FAKE * 2, V, FAKE * 2, None) == -7


def test_correction_variant_exports_and_validates():
    """The comparison variant (variants/) loads, exports what its header declares, and its
    host-side checks reject bad trees and shapes without launching anything."""
    from variants import correction as corr

    header = os.path.join(os.path.dirname(os.path.dirname(__file__)), "variants", "correction.h")
    text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(specfold_variant_[a-z_]+)\s*\(", text)))
    assert set(names) == set(corr.EXPORTS)
    for n in names:
        assert hasattr(corr._lib, n), n
    sh = WORKLOADS["layer-1.5b"].shape
    # depth levels of a known tree
    assert corr.levels(sh, [-1, 0, 0, 1, 2, 3, 1, 0, 4]) == [0b10000110, 0b01011000, 0b100100000]
    assert corr.levels(sh, [-1, 0, 1, 2, 3, 4, 5, 6, 7]) == [1 << i for i in range(1, 9)]
    with pytest.raises(sf.SpecfoldError) as e:
        corr.levels(sh, [-1, 0, 2, 1, 2, 3, 1, 0, 4])         # par[2] = 2 is not an ancestor
    assert e.value.status == -3
    bad = sf.make_shape(sh)
    bad.head_dim = 256                                         # beyond the variant's two dims per lane
    masks = (ctypes.c_uint64 * 9)()
    n = ctypes.c_int32()
    par = (ctypes.c_int32 * 9)(-1, 0, 0, 0, 0, 0, 0, 0, 0)
    assert corr._lib.specfold_variant_correction_levels(ctypes.byref(bad), par, masks, ctypes.byref(n)) == -2
    st = corr._lib.specfold_variant_correction_fresh(ctypes.byref(sf.make_shape(sh)), None, None, None, None, None,
                                                     None, None, None, None)
    assert st == -1


def test_gate_rejects_inputs_of_1gb_and_more():
    """The gate addresses H with 32-bit offsets and reads zeros past 1 GB, so an H of 1 GB or more
    is refused before anything is launched."""
    p, keep = _parent([-1] + [0] * 63)
    big = _shape(n_branch=16, block=1 << 20, hidden=64)          # 2^24 rows, 2 GB
    edge = _shape(n_branch=64, block=65536, hidden=128)          # exactly 1 GB
    for sh in (big, edge):
        assert L.specfold_gate(ctypes.byref(sh), p, FAKE, 0.1, None, FAKE, FAKE * 4096, None, None) == -6
        # rho given but inv_rms asked for: H is read, so the limit still applies
        assert L.specfold_gate(ctypes.byref(sh), p, FAKE, 0.1, 0x100000000, 0x200000000, 0x300000000,
                               0x400000000, None) == -6
