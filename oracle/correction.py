"""The pages' own route to a folded query's attention: correct the parent's softmax state.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[SpecFold summary, §A.1 and App. B]: a folded position starts from its parent's streaming
softmax state (running maximum, denominator and unnormalised numerator per head), removes
the parent's terms at the block positions the child recomputed and adds the child's terms
there; the result is the child's exact state.  [§A.3]: branches are visited in topological
order so the parent's state is already the corrected one.  Evaluated in float64 this must
equal direct attention (``oracle.layer.attention_block`` applied per branch).
"""

from __future__ import annotations

import numpy as np

from .layer import _f64


def folded_attention_by_correction(q_c, k_c, v_c, fold, parent, src_slot, pk, pv, shape):
    """Attention output [B+1, N, Hq, d] for every row; recomputed rows get a fresh state
    over [prefix ; own block], folded rows get their parent's state corrected."""
    q_c, k_c, v_c, pk, pv = (_f64(t) for t in (q_c, k_c, v_c, pk, pv))
    fold = np.asarray(fold, dtype=bool)
    parent = np.asarray(parent)
    B1, N = fold.shape
    Hq, Hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    group = Hq // Hkv
    scale = 1.0 / np.sqrt(d)
    states = {}
    out = np.empty((B1, N, Hq, d))
    for i in range(B1):
        Q, K, V = q_c[src_slot[i]], k_c[src_slot[i]], v_c[src_slot[i]]
        m = np.empty((N, Hq))
        l = np.empty((N, Hq))
        acc = np.empty((N, Hq, d))
        changed = np.flatnonzero(~fold[i])      # block positions the child recomputed
        for n in range(N):
            for h in range(Hq):
                g = h // group
                if not fold[i, n]:
                    s = np.concatenate([pk[:, g] @ Q[n, h], K[:, g] @ Q[n, h]]) * scale
                    vals = np.concatenate([pv[:, g], V[:, g]], axis=0)
                    mx = s.max()
                    e = np.exp(s - mx)
                    m[n, h], l[n, h], acc[n, h] = mx, e.sum(), e @ vals
                    continue
                p = int(parent[i])
                mp, lp, ap = states[p][0][n, h], states[p][1][n, h], states[p][2][n, h]
                Kp, Vp = k_c[src_slot[p]], v_c[src_slot[p]]
                s_old = (Kp[changed, g] @ Q[n, h]) * scale
                s_new = (K[changed, g] @ Q[n, h]) * scale
                mx = max(mp, s_new.max()) if changed.size else mp
                e_old, e_new = np.exp(s_old - mx), np.exp(s_new - mx)
                rescale = np.exp(mp - mx)
                m[n, h] = mx
                l[n, h] = lp * rescale - e_old.sum() + e_new.sum()
                acc[n, h] = ap * rescale - e_old @ Vp[changed, g] + e_new @ V[changed, g]
        states[i] = (m, l, acc)
        out[i] = acc / l[..., None]
    return out
