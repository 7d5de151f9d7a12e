"""specfold_verify_layer_noalloc: the whole layer with the library's own device scratch array as
its workspace, for callers that cannot allocate.  Its output must equal specfold_verify_layer's
bit for bit (same kernels), also on a second, smaller call that finds the first call's contents
in the shared array; and it must refuse a shape whose workspace exceeds the array before
launching anything."""

import ctypes

import numpy as np
import pytest
import torch

from gpu_case import DEV, LayerCase, dev_bf16
from sparse_layer_rho_amd import specfold as sf
from synth import WORKLOADS, Shape


def test_noalloc_refuses_shapes_beyond_its_scratch():
    """Host checks only (runs without a GPU): a 14B-class layer at prefix 16384 needs more
    workspace than the array holds."""
    sh = sf.make_shape(Shape(9, 32, 5120, 40, 8, 128, 13824, 16384))
    assert sf.lib().specfold_workspace_bytes(ctypes.byref(sh)) > sf.NOALLOC_SCRATCH_BYTES
    fake = 0x10000
    w = sf.LayerWeights(*(fake * k for k in range(1, 7)))
    pf = sf.PrefixKV(fake * 8, fake * 9, 8 * 128, 128, 8 * 128, 128)
    par = (ctypes.c_int32 * 9)(-1, 0, 0, 1, 1, 2, 3, 4, 5)
    st = sf.lib().specfold_verify_layer_noalloc(ctypes.byref(sh), par, ctypes.byref(w), ctypes.byref(pf),
                                               0x20000000, 0.1, 0x30000000, None, None, None)
    assert st == -5


def _both(case, delta):
    sh = case.shape
    R, D = sh.rows, sh.hidden
    w, pk, pv = case.device()
    H_in = dev_bf16(case.H.reshape(R, D))
    out = {}
    for name in ("ws", "noalloc"):
        H_out = torch.full((R, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        st = {"rho": torch.full((R,), float("nan"), device=DEV),
              "fold": torch.full((R,), 7, dtype=torch.uint8, device=DEV),
              "rec_count": torch.full((1,), -1, dtype=torch.int32, device=DEV),
              "src_slot": torch.full((R,), -9, dtype=torch.int32, device=DEV)}
        if name == "ws":
            ws = sf.new_workspace(sh)
            ws.fill_(0xA5)
            sf.verify_layer(sh, case.parent, w, pk, pv, H_in, delta, H_out, ws, stats=st)
        else:
            sf.verify_layer_noalloc(sh, case.parent, w, pk, pv, H_in, delta, H_out, stats=st)
        torch.cuda.synchronize()
        out[name] = {"H": H_out.view(torch.int16).cpu().numpy(),
                     **{k: v.cpu().numpy() for k, v in st.items()}}
    return out


@pytest.mark.gpu
def test_noalloc_equals_verify_layer_on_two_calls_in_a_row():
    big = LayerCase.workload("layer-1.5b")
    wl = WORKLOADS["layer-1.5b"]
    small_shape = wl.shape.with_branches(4)                       # R = 128 after R = 288
    small = LayerCase(small_shape, 7)
    for case, delta in ((big, wl.delta), (small, 0.1), (small, 0.0)):
        out = _both(case, delta)
        a, b = out["ws"], out["noalloc"]
        for k in ("H", "fold", "rec_count", "src_slot"):
            assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a["rho"].view(np.int32), b["rho"].view(np.int32))
        assert np.isfinite((a["H"].view(np.uint16).astype(np.uint32) << 16).view(np.float32)).all()
        print(f"R = {case.shape.rows}, delta {delta}: M = {int(b['rec_count'][0])}, outputs bitwise equal")
