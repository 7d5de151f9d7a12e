"""Python binding of ``libspecfold_correction.so`` (declared in ``variants/correction.h``).

Argument marshalling only; the three phases run in the variant's HIP kernels: fresh states of
the recompute rows, one correction launch per depth level of the parent tree (parents before
children), and the division acc / l.
"""

from __future__ import annotations

import ctypes
import os

import torch

from sparse_layer_rho_amd import specfold as sf

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libspecfold_correction.so")

EXPORTS = ("specfold_variant_correction_levels", "specfold_variant_correction_fresh",
           "specfold_variant_correction_level", "specfold_variant_correction_finalize")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_pS = ctypes.POINTER(sf.Shape)
_lib.specfold_variant_correction_levels.argtypes = [_pS, _P, _P, _P]
_lib.specfold_variant_correction_fresh.argtypes = [_pS, _P, _P, _P, _P, _P, _P, ctypes.POINTER(sf.PrefixKV), _P, _P]
_lib.specfold_variant_correction_level.argtypes = [_pS, _P, ctypes.c_uint64, _P, _P, _P, _P, _P, _P, _P]
_lib.specfold_variant_correction_finalize.argtypes = [_pS, _P, _P, _P]
for _name in EXPORTS:
    getattr(_lib, _name).restype = ctypes.c_int


def _check(st: int, where: str) -> None:
    if st != 0:
        raise sf.SpecfoldError(st, where)


def state_shape(shape):
    return (shape.n_branch * shape.block, shape.n_q_heads, shape.head_dim + 2)


def levels(shape, parent) -> list[int]:
    """Branch masks of depth 1, 2, ... (host-side walk of the parent map)."""
    sh = sf.make_shape(shape)
    par = sf._parent_host(parent, shape.n_branch)
    masks = (ctypes.c_uint64 * shape.n_branch)()
    n = ctypes.c_int32(0)
    _check(_lib.specfold_variant_correction_levels(ctypes.byref(sh), ctypes.c_void_p(par.data_ptr()),
                                                   ctypes.cast(masks, _P), ctypes.byref(n)),
           "specfold_variant_correction_levels")
    return [int(masks[d]) for d in range(n.value)]


def _qkv(shape, q_c, k_c, v_c):
    """Slot-indexed projections hold R rows (the kernels index them by slot < R)."""
    R, d = shape.n_branch * shape.block, shape.head_dim
    return (sf._ptr(q_c, torch.bfloat16, R * shape.n_q_heads * d, "q_c"),
            sf._ptr(k_c, torch.bfloat16, R * shape.n_kv_heads * d, "k_c"),
            sf._ptr(v_c, torch.bfloat16, R * shape.n_kv_heads * d, "v_c"))


def fresh(shape, q_c, k_c, v_c, rec_rows, rec_count, src_slot, prefix_k, prefix_v, state):
    sh = sf.make_shape(shape)
    R = shape.n_branch * shape.block
    pf = sf.prefix_view(prefix_k, prefix_v) if shape.prefix_len > 0 else sf.PrefixKV()
    st = _lib.specfold_variant_correction_fresh(
        ctypes.byref(sh), *_qkv(shape, q_c, k_c, v_c), sf._ptr(rec_rows, torch.int32, R, "rec_rows"),
        sf._ptr(rec_count, torch.int32, 1, "rec_count"), sf._ptr(src_slot, torch.int32, R, "src_slot"),
        ctypes.byref(pf), sf._ptr(state, torch.float32, R * shape.n_q_heads * (shape.head_dim + 2), "state"),
        sf._stream())
    _check(st, "specfold_variant_correction_fresh")


def level(shape, parent, mask, q_c, k_c, v_c, src_slot, fold, state):
    sh = sf.make_shape(shape)
    R = shape.n_branch * shape.block
    par = sf._parent_host(parent, shape.n_branch)
    st = _lib.specfold_variant_correction_level(
        ctypes.byref(sh), ctypes.c_void_p(par.data_ptr()), ctypes.c_uint64(mask), *_qkv(shape, q_c, k_c, v_c),
        sf._ptr(src_slot, torch.int32, R, "src_slot"),
        sf._ptr(fold, torch.uint8, R, "fold"),
        sf._ptr(state, torch.float32, R * shape.n_q_heads * (shape.head_dim + 2), "state"), sf._stream())
    _check(st, "specfold_variant_correction_level")


def finalize(shape, state, out):
    sh = sf.make_shape(shape)
    R = shape.n_branch * shape.block
    st = _lib.specfold_variant_correction_finalize(
        ctypes.byref(sh), sf._ptr(state, torch.float32, R * shape.n_q_heads * (shape.head_dim + 2), "state"),
        sf._ptr(out, torch.float32, R * shape.n_q_heads * shape.head_dim, "out"), sf._stream())
    _check(st, "specfold_variant_correction_finalize")


def attention(shape, parent, q_c, k_c, v_c, rec_rows, rec_count, src_slot, fold, prefix_k, prefix_v, state, out):
    """Attention of every row by the correction method: out fp32 [R, Hq, head_dim]."""
    fresh(shape, q_c, k_c, v_c, rec_rows, rec_count, src_slot, prefix_k, prefix_v, state)
    for mask in levels(shape, parent):
        level(shape, parent, mask, q_c, k_c, v_c, src_slot, fold, state)
    finalize(shape, state, out)
