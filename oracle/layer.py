"""Resolved-source form of one folded verification layer, step by step, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the product path.

Notation (the pages'): branch i in 0..B, 0 = main, par(i) = parent, N block positions,
R = (B+1) N flattened rows with row r = i*N + n, D hidden size, Hq/Hkv query/KV heads,
d head size, F FFN width, P shared prefix length, delta the fold threshold.

Readings where the pages are silent (each one is listed with its reason in the design notes):
* the gate sees the raw residual stream entering the layer, one gate per layer shared by
  the QKV projection and the FFN;
* no biases; RMSNorm with weight and eps; rotate-half rotary embedding at absolute position
  P + n with base ``rope_theta``; contiguous GQA groups (head h uses KV head h // (Hq/Hkv));
  score scale 1/sqrt(d); bidirectional attention of every block query over the whole prefix
  and the N block keys of its own branch;
* the attention output projection is applied densely to every row (the pages fold only QKV
  and the FFN);
* SwiGLU FFN: down(silu(gate(y)) * up(y)).
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ------------------------------------------------------------------ step 1: the gate

def gate(H, parent, delta):
    """Token-level parent-child residual gate.

    [SpecFold review (ko), "무엇과 다른가"]: per layer, branch i and position n the gate
    takes the Euclidean distance between the child's and the parent's hidden rows,
    relative to the parent row's length, and marks the position folded when that ratio
    is at most delta.  [SpecFold summary, App. B]: the main branch skips the gate and
    recomputes everything.

    Readings: the norm runs over the D hidden features; a zero parent row gives 0 when
    the child row is zero too and +inf otherwise; a NaN ratio never folds.  The fold
    decision is taken in float32 (the precision the device takes it in):
    float32(rho) <= float32(delta).

    H: [B+1, N, D].  Returns rho float64 [B+1, N] (0 for main) and fold bool [B+1, N].
    """
    H = _f64(H)
    parent = np.asarray(parent)
    B1, N, _ = H.shape
    rho = np.zeros((B1, N))
    fold = np.zeros((B1, N), dtype=bool)
    thr = np.float32(delta)
    for i in range(1, B1):
        p = int(parent[i])
        diff = H[i] - H[p]
        a = np.sum(diff * diff, axis=1)          # squared distance to the parent row
        b = np.sum(H[p] * H[p], axis=1)          # squared length of the parent row
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.sqrt(a) / np.sqrt(b)
        zero_parent = np.where(a > 0, np.inf, np.where(a == 0, 0.0, np.nan))
        rho[i] = np.where(b > 0, ratio, zero_parent)
        with np.errstate(invalid="ignore", over="ignore"):
            fold[i] = rho[i].astype(np.float32) <= thr
    return rho, fold


# ------------------------------------------------------------------ step 2: compaction

def compact(fold):
    """Global and per-branch recompute lists [SpecFold summary, App. B: the gate compacts
    recomputed indices into global and per-branch lists].

    Reading: the global list holds recompute rows in ascending row order; the per-branch
    lists are its contiguous segments ``rec_rows[branch_off[i]:branch_off[i+1]]``.

    Returns rec_rows int64 [M], row_slot int64 [R] (slot of each row in rec_rows, -1 when
    folded) and branch_off int64 [B+2].
    """
    fold = np.asarray(fold, dtype=bool)
    B1, N = fold.shape
    flat = fold.reshape(-1)
    row_slot = np.full(flat.size, -1, dtype=np.int64)
    rec = []
    for r in range(flat.size):
        if not flat[r]:
            row_slot[r] = len(rec)
            rec.append(r)
    branch_off = np.zeros(B1 + 1, dtype=np.int64)
    for i in range(B1):
        branch_off[i + 1] = branch_off[i] + int(np.count_nonzero(~fold[i]))
    return np.asarray(rec, dtype=np.int64), row_slot, branch_off


# ------------------------------------------------------------------ step 3: fold sources

def resolve(fold, parent, row_slot):
    """Fold-chain source resolution [SpecFold summary, App. B: each folded position is
    followed up its chain to the nearest ancestor that recomputed it; §A.3].

    src(i, n) = i when (i, n) is recomputed, else src(par(i), n), visiting branches in
    index (topological) order.  Returns src_branch [B+1, N] and src_slot [B+1, N], the
    slot of row src(i,n)*N + n in the recompute list.
    """
    fold = np.asarray(fold, dtype=bool)
    parent = np.asarray(parent)
    B1, N = fold.shape
    if fold[0].any():
        raise ValueError("the main branch never folds")
    src = np.empty((B1, N), dtype=np.int64)
    for i in range(B1):
        for n in range(N):
            src[i, n] = i if not fold[i, n] else src[int(parent[i]), n]
    src_slot = np.asarray(row_slot)[src * N + np.arange(N)[None, :]]
    return src, src_slot


# ------------------------------------------------------------------ per-row primitives

def rms_norm(x, w, eps):
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * _f64(w)


def rope(x, pos, theta):
    """Rotate-half rotary embedding: for j < d/2 the pair (x_j, x_{j+d/2}) is rotated by
    the angle pos * theta^(-2j/d).  ``pos`` broadcasts against ``x.shape[:-1]``."""
    x = _f64(x)
    d = x.shape[-1]
    half = d // 2
    inv_freq = float(theta) ** (-(2.0 * np.arange(half)) / d)
    ang = _f64(pos)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x):
    x = _f64(x)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def qkv_rows(h_rows, pos, ln1, w_qkv, shape):
    """RMSNorm, packed QKV projection and rotary embedding of the given rows
    [SpecFold summary, App. B: recomputed positions get RMSNorm and packed QKV projections
    with rotary embeddings].  Returns q [M,Hq,d], k [M,Hkv,d], v [M,Hkv,d]."""
    Hq, Hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    x = rms_norm(h_rows, ln1, shape.rms_eps)
    y = x @ _f64(w_qkv).T
    m = y.shape[0]
    q = y[:, : Hq * d].reshape(m, Hq, d)
    k = y[:, Hq * d: (Hq + Hkv) * d].reshape(m, Hkv, d)
    v = y[:, (Hq + Hkv) * d:].reshape(m, Hkv, d)
    pos = _f64(pos)[:, None]
    return rope(q, pos, shape.rope_theta), rope(k, pos, shape.rope_theta), v


def attention_block(Q, K, V, pk, pv, shape):
    """Exact attention of one branch block [SpecFold review (ko), "무엇과 다른가": exact with
    respect to the branch's own KV; "어떻게 쓰나": the shared prefix KV is seen by every
    branch; grouped-query attention].

    Q [N, Hq, d] are the branch's queries, K/V [N, Hkv, d] its own block keys/values,
    pk/pv [P, Hkv, d] the shared prefix.  Every query attends to all P prefix keys and all
    N block keys of its branch (no mask).  Returns [N, Hq, d].
    """
    Q, K, V, pk, pv = (_f64(t) for t in (Q, K, V, pk, pv))
    Hq, Hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    group = Hq // Hkv
    scale = 1.0 / np.sqrt(d)
    out = np.empty(Q.shape)
    for h in range(Hq):
        g = h // group
        keys = np.concatenate([pk[:, g], K[:, g]], axis=0)
        vals = np.concatenate([pv[:, g], V[:, g]], axis=0)
        s = (Q[:, h] @ keys.T) * scale
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h] = p @ vals
    return out


def ffn_rows(h_rows, ln2, w_gate_up, w_down, shape):
    """RMSNorm + SwiGLU FFN of the given rows [SpecFold summary, §A.2 and App. B: the FFN is
    position-wise and runs on recomputed rows only]."""
    F = shape.ffn
    y = rms_norm(h_rows, ln2, shape.rms_eps)
    gu = y @ _f64(w_gate_up).T
    act = silu(gu[:, :F]) * gu[:, F:]
    return act @ _f64(w_down).T


# ------------------------------------------------------------------ the layer

def verify_layer(H, parent, weights, pk, pv, delta, shape, fold=None):
    """One folded verification layer (resolved-source form).

    Steps, in the order of [SpecFold summary, App. B] and [SpecFold review (ko),
    "무엇과 다른가" / "어떻게 쓰나"]:
      1. gate -> rho, fold (``fold`` may be given to force the mask);
      2. compaction of recompute rows;
      3. fold-source resolution;
      4. RMSNorm + QKV + RoPE on recompute rows only;
      5. Q/K/V of every row taken from its source's slot (folded rows inherit);
      6. exact per-branch attention over [prefix ; own block];
      7. output projection + residual on every row (dense reading);
      8. FFN on recompute rows only;
      9. every row adds its source's FFN output to its own residual stream
         [SpecFold summary, App. B: the residual stream is never folded].
    Returns a dict with every intermediate.
    """
    H = _f64(H)
    parent = np.asarray(parent)
    B1, N, D = H.shape
    R = B1 * N
    if fold is None:
        rho, fold = gate(H, parent, delta)
    else:
        rho = None
        fold = np.asarray(fold, dtype=bool)
    rec_rows, row_slot, branch_off = compact(fold)
    src_branch, src_slot = resolve(fold, parent, row_slot)

    Hf = H.reshape(R, D)
    pos = shape.prefix_len + (rec_rows % N)
    q_c, k_c, v_c = qkv_rows(Hf[rec_rows], pos, weights["ln1"], weights["w_qkv"], shape)

    attn = np.empty((B1, N, shape.n_q_heads, shape.head_dim))
    for i in range(B1):
        sl = src_slot[i]
        attn[i] = attention_block(q_c[sl], k_c[sl], v_c[sl], pk, pv, shape)
    h_mid = Hf + attn.reshape(R, -1) @ _f64(weights["w_o"]).T

    f_c = ffn_rows(h_mid[rec_rows], weights["ln2"], weights["w_gate_up"], weights["w_down"], shape)
    H_out = h_mid + f_c[src_slot.reshape(-1)]
    return {
        "H_out": H_out.reshape(B1, N, D), "rho": rho, "fold": fold, "rec_rows": rec_rows,
        "row_slot": row_slot, "branch_off": branch_off, "src_branch": src_branch,
        "src_slot": src_slot, "q_c": q_c, "k_c": k_c, "v_c": v_c,
        "attn": attn.reshape(R, -1), "h_mid": h_mid, "f_c": f_c,
    }


def dense_branch_layer(Hb, weights, pk, pv, shape):
    """The plain (unfolded) layer on one branch block [N, D]: every position recomputed.
    Running it per branch is serialized verification [SpecFold summary, App. C]."""
    Hb = _f64(Hb)
    N = Hb.shape[0]
    pos = shape.prefix_len + np.arange(N)
    q, k, v = qkv_rows(Hb, pos, weights["ln1"], weights["w_qkv"], shape)
    a = attention_block(q, k, v, pk, pv, shape)
    h = Hb + a.reshape(N, -1) @ _f64(weights["w_o"]).T
    return h + ffn_rows(h, weights["ln2"], weights["w_gate_up"], weights["w_down"], shape)


def stack(H0, parent, layers, delta, shape):
    """Apply folded layers in sequence; every layer re-gates on its own input, so the
    per-branch divergence carried by the residual streams accumulates [SpecFold review (ko),
    "무엇과 다른가"].  ``layers`` is a list of (weights, pk, pv).  Returns (H_L, folds)."""
    H = _f64(H0)
    folds = []
    for weights, pk, pv in layers:
        res = verify_layer(H, parent, weights, pk, pv, delta, shape)
        folds.append(res["fold"])
        H = res["H_out"]
    return H, folds
