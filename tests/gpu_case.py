"""Helpers of the GPU parity tests: build a seeded layer case, run it through the C ABI,
and compare with the oracle on the same bf16-rounded inputs (upcast to float64)."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from sparse_layer_rho_amd import specfold as sf
from synth import WORKLOADS, Shape, bf16_round, layer_weights, parent_tree, prefix_kv, step_inputs

DEV = "cuda"
BAND = 1e-4           # rho within this distance of delta may legitimately flip the mask
TOL_LAYER = 2e-2      # relative L2 bound on a layer's hidden-state output


def dev_bf16(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


class LayerCase:
    """One layer's seeded inputs: parent tree, bf16 hidden states, weights and prefix cache."""

    def __init__(self, shape: Shape, base_seed: int, layer: int = 0, step: int = 0, tree="random",
                 law="lognormal", parent=None, random_norm=False, H=None, weight_scale=1.0, device_weights=None):
        self.shape = shape
        self._dev = None
        if device_weights is not None:
            # weights drawn on the device (synth.device_layer): the oracle gets their exact values
            w, pk, pv = device_weights
            self.w = {k: host(v) for k, v in w.items()}
            self.pk, self.pv = host(pk), host(pv)
            self._dev = (w, pk, pv)
        else:
            self.w = layer_weights(shape, base_seed, layer, random_norm=random_norm)
            self.pk, self.pv = prefix_kv(shape, base_seed, layer)
        if weight_scale != 1.0:
            # larger projections make the layer update O(|H|), so bf16 rounding of the output
            # stays far below the update and update-level comparisons are sharp
            for k in ("w_qkv", "w_o", "w_gate_up", "w_down"):
                self.w[k] = bf16_round(self.w[k] * np.float32(weight_scale))
        if H is None:
            inp = step_inputs(shape, base_seed, step, tree=tree, child_law=law, parent=parent)
            self.parent = inp["parent"]
            H = inp["H"]
        else:
            self.parent = np.asarray(parent, dtype=np.int32)
        self.H = bf16_round(np.asarray(H, dtype=np.float32)).astype(np.float64)

    @classmethod
    def workload(cls, name, **kw):
        wl = WORKLOADS[name]
        kw.setdefault("tree", wl.tree)
        kw.setdefault("law", wl.child_law)
        return cls(wl.shape, wl.base_seed, **kw)

    def device(self):
        if self._dev is None:
            w = {k: dev_bf16(v) for k, v in self.w.items()}
            pk, pv = dev_bf16(self.pk), dev_bf16(self.pv)
            self._dev = (w, pk, pv)
        return self._dev

    def run(self, delta, H=None, ws=None, poison=True, trace=None):
        """verify_layer on the GPU; returns host arrays."""
        sh = self.shape
        R, D = sh.n_branch * sh.block, sh.hidden
        w, pk, pv = self.device()
        H_in = dev_bf16((self.H if H is None else H).reshape(R, D))
        H_out = torch.full((R, D), float("nan"), dtype=torch.bfloat16, device=DEV) if poison else \
            torch.empty((R, D), dtype=torch.bfloat16, device=DEV)
        if ws is None:
            ws = sf.new_workspace(sh)
        stats = {"rho": torch.full((R,), float("nan"), device=DEV),
                 "fold": torch.full((R,), 7, dtype=torch.uint8, device=DEV),
                 "rec_count": torch.full((1,), -1, dtype=torch.int32, device=DEV),
                 "src_slot": torch.full((R,), -9, dtype=torch.int32, device=DEV)}
        sf.verify_layer(sh, self.parent, w, pk, pv, H_in, delta, H_out, ws, stats=stats, trace=trace)
        torch.cuda.synchronize()
        return {"H_out": host(H_out).reshape(sh.n_branch, sh.block, D),
                "H_out_bits": H_out.view(torch.int16).cpu().numpy(),
                "rho": stats["rho"].cpu().numpy().reshape(sh.n_branch, sh.block),
                "fold": stats["fold"].cpu().numpy().reshape(sh.n_branch, sh.block),
                "rec_count": int(stats["rec_count"].item()),
                "src_slot": stats["src_slot"].cpu().numpy().reshape(sh.n_branch, sh.block)}

    def check(self, delta, res, H=None, tol=TOL_LAYER):
        """Teacher-forced comparison of one GPU layer result with the oracle; returns the
        oracle result and the relative L2 error."""
        Hh = self.H if H is None else H
        rho_o, fold_o = oracle.gate(Hh, self.parent, delta)
        fold_g = res["fold"].astype(bool)
        assert set(np.unique(res["fold"])) <= {0, 1}
        with np.errstate(invalid="ignore"):
            band = np.abs(rho_o - delta) < BAND
        assert np.array_equal(fold_g[~band], fold_o[~band]), "fold mask differs outside the band"
        fin = np.isfinite(rho_o) & (rho_o > 1e-3)
        np.testing.assert_allclose(res["rho"][fin], rho_o[fin], rtol=5e-5)
        ref = oracle.verify_layer(Hh, self.parent, self.w, self.pk, self.pv, delta, self.shape, fold=fold_g)
        assert res["rec_count"] == ref["rec_rows"].size
        assert np.array_equal(res["src_slot"], ref["src_slot"])
        assert np.isfinite(res["H_out"]).all(), "unwritten or NaN output rows"
        err = rel_l2(res["H_out"], ref["H_out"])
        assert err <= tol, f"relative L2 {err:.3e} > {tol}"
        # the same bound per branch, and 5x that per row, so one wrong row cannot hide in the
        # whole tensor (a single row may sit near a softmax tie, where bf16 inputs move its
        # attention by a few percent: 2.95e-2 on one row of the R = 1088 edge shape with 8x weights)
        diff = res["H_out"] - ref["H_out"]
        per_branch = np.linalg.norm(diff, axis=(1, 2)) / np.maximum(np.linalg.norm(ref["H_out"], axis=(1, 2)), 1e-300)
        per_row = np.linalg.norm(diff, axis=2) / np.maximum(np.linalg.norm(ref["H_out"], axis=2), 1e-300)
        assert per_branch.max() <= tol, f"branch {int(per_branch.argmax())}: relative L2 {per_branch.max():.3e} > {tol}"
        assert per_row.max() <= 5 * tol, f"row {np.unravel_index(per_row.argmax(), per_row.shape)}: " \
                                         f"relative L2 {per_row.max():.3e} > {5 * tol}"
        self.last_branch_err = float(per_branch.max())
        self.last_row_err = float(per_row.max())
        # the layer update itself, H_out - H_in: within tol of the oracle's update, plus the
        # bf16 rounding of H_out (half an ulp, at most 2^-9 relative per element)
        upd_ref = ref["H_out"] - Hh
        d_upd = np.linalg.norm((res["H_out"] - Hh) - upd_ref)
        allow = tol * np.linalg.norm(upd_ref) + 2.0 ** -9 * np.linalg.norm(ref["H_out"])
        assert d_upd <= allow, f"update error {d_upd:.3e} > {allow:.3e}"
        self.last_update_err = float(d_upd / max(np.linalg.norm(upd_ref), 1e-300))
        return ref, err


def random_mask(shape: Shape, rng, p_fold=0.7):
    fold = rng.random((shape.n_branch, shape.block)) < p_fold
    fold[0] = False
    return fold


__all__ = ["LayerCase", "dev_bf16", "host", "rel_l2", "random_mask", "parent_tree", "TOL_LAYER", "BAND"]
