"""Table-inheritance form of the folded layer, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Structured the way [SpecFold summary, Appendix A and §A.3] describe the algorithm rather
than the way a kernel runs it: branches are visited in topological (index) order; each
branch copies its parent's projection (Q/K/V) and FFN-output tables and overwrites only the
positions it recomputes, then attends with its own tables and adds its own residual stream.
No compaction and no explicit source map.  It must agree with the resolved-source form
(``oracle.layer.verify_layer``) to float64 rounding.
"""

from __future__ import annotations

import numpy as np

from .layer import _f64, attention_block, ffn_rows, gate, qkv_rows


def verify_layer_tables(H, parent, weights, pk, pv, delta, shape, fold=None):
    H = _f64(H)
    parent = np.asarray(parent)
    B1, N, D = H.shape
    Hq, Hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    if fold is None:
        _, fold = gate(H, parent, delta)
    fold = np.asarray(fold, dtype=bool)
    pos = shape.prefix_len + np.arange(N)
    w_o = _f64(weights["w_o"])
    q_tab, k_tab, v_tab, f_tab = {}, {}, {}, {}
    out = np.empty_like(H)
    for i in range(B1):
        own = np.flatnonzero(~fold[i])           # positions this branch recomputes
        if i == 0:
            if own.size != N:
                raise ValueError("the main branch recomputes every position")
            Q, K, V = np.zeros((N, Hq, d)), np.zeros((N, Hkv, d)), np.zeros((N, Hkv, d))
            Fi = np.zeros((N, D))
        else:
            p = int(parent[i])
            Q, K, V = q_tab[p].copy(), k_tab[p].copy(), v_tab[p].copy()
            Fi = f_tab[p].copy()
        if own.size:
            q, k, v = qkv_rows(H[i][own], pos[own], weights["ln1"], weights["w_qkv"], shape)
            Q[own], K[own], V[own] = q, k, v
        a = attention_block(Q, K, V, pk, pv, shape)
        h = H[i] + a.reshape(N, -1) @ w_o.T
        if own.size:
            Fi[own] = ffn_rows(h[own], weights["ln2"], weights["w_gate_up"], weights["w_down"], shape)
        q_tab[i], k_tab[i], v_tab[i], f_tab[i] = Q, K, V, Fi
        out[i] = h + Fi
    return out
