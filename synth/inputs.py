"""Workload shapes and seeded input recipes (no arithmetic of the method).

Workloads mirror the pages' setting: a denoising block of 32 positions, a main
branch plus B drafts arranged as a parent tree of depth at most 4, drafts that
add one to four newly unmasked positions where hidden states diverge strongly
and stay close to the parent elsewhere.  The closeness is drawn so that, at the
first layer, 72 % of draft rows have relative residual <= 0.1 and 88 % have
<= 0.3 -- the redundancy profile reported in the SpecFold summary (paperlayer.ai,
§3.1) and the Korean review (onedev.kr, section "어떻게 동작하나").  Model
sizes follow the 1.5B / 7B / 14B-class shapes of the evaluated model families.

Seeds: every tensor comes from ``default_rng([base_seed, step, layer, tensor_id])``.
Weights and prefix caches use ``step = 0`` so they stay fixed across the steps of
a multi-step workload; hidden states and trees use ``layer = 0``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# tensor ids inside a seed tuple
_T_LN1, _T_WQKV, _T_WO, _T_LN2, _T_WGU, _T_WDOWN, _T_PK, _T_PV = range(8)
_T_TREE, _T_MAIN, _T_CHILD = 10, 11, 12
_T_TOKENS = 13

# Log-normal law of a draft row's relative distance r (non-unmasked rows) chosen so
# that, with E[#unmasked]/N = 2.5/32, P(r <= 0.1) = 0.72 and P(r <= 0.3) = 0.88 over
# all draft rows (unmasked rows sit near sqrt(2) and never fold at delta <= 0.7).
LOGNORMAL_MU = -3.2335
LOGNORMAL_SIGMA = 1.2003

# One-token drafts (the draft-shape sweep, [SpecFold summary, §D.2]: seven one-token sibling
# drafts at depth 1 through parent-extending chains).  Main's block has 17 of its 32 positions
# committed (the parent of the summary's Figure 6 example); every draft unmasks exactly one
# position its parent still has masked and inherits the parent's committed tokens.  The
# parent-child divergence concentrates at the positions that are still masked ([SpecFold
# summary, §3.1 and §4.4]): there r is log-normal with P(r <= 0.1) = 0.20, at committed
# positions with P(r <= 0.1) = 0.85 (both with the sigma above).  A draft deeper in the tree
# has fewer masked positions, so the fold fraction depends on the tree's shape: about 0.54 for
# seven siblings of main and 0.60 averaged over a seven-deep chain, inside the 0.52-0.67 range
# the summary reports across drafting shapes.
UNMASK1_COMMITTED = 17
UNMASK1_MU_COMMITTED = -3.5466
UNMASK1_MU_MASKED = -1.2924


@dataclass(frozen=True)
class Shape:
    """Sizes of one verification layer.

    n_branch = B + 1 (main + drafts); block = N positions per branch;
    hidden = D; n_q_heads / n_kv_heads = Hq / Hkv (grouped-query attention);
    head_dim = d; ffn = F (SwiGLU width); prefix_len = P shared prefix tokens.
    """

    n_branch: int
    block: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    prefix_len: int
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0

    @property
    def rows(self) -> int:
        return self.n_branch * self.block

    @property
    def qkv_out(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def with_branches(self, n_branch: int) -> "Shape":
        return Shape(n_branch, self.block, self.hidden, self.n_q_heads, self.n_kv_heads,
                     self.head_dim, self.ffn, self.prefix_len, self.rms_eps, self.rope_theta)

    def weight_bytes_bf16(self) -> int:
        d, dq = self.hidden, self.n_q_heads * self.head_dim
        return 2 * (self.qkv_out * d + d * dq + 3 * self.ffn * d + 2 * d)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    base_seed: int
    delta: float
    layers: int = 1
    steps: int = 1
    tree: str = "random"            # "random" (depth <= 4) or "chain"
    child_law: str = "lognormal"    # "lognormal" (with unmasked rows) or "tiny"
    branch_sweep: tuple = ()
    delta_sweep: tuple = ()
    tree_sweep: tuple = ()          # tree shapes: "star", "depthK" (random, depth <= K), "chain"
    # standard deviations of the random-init projections (w_qkv, w_o, w_gate_up, w_down)
    weight_std: tuple = (0.02, 0.02, 0.02, 0.02)
    note: str = ""


WORKLOADS: dict[str, Workload] = {
    # tiny single layer: hidden 64, 4 q heads / 2 kv heads, head_dim 16, FFN 128,
    # block 8, main + 2 drafts in a chain main<-d1<-d2, prefix 16, delta 0.1, seed 0
    "tiny": Workload("tiny", Shape(3, 8, 64, 4, 2, 16, 128, 16), 0, 0.1,
                     tree="chain", child_law="tiny"),
    # one layer at 1.5B-class shape, B = 8 drafts, prefix 512
    "layer-1.5b": Workload("layer-1.5b", Shape(9, 32, 1536, 12, 2, 128, 8960, 512), 1, 0.1),
    # 28-layer stack at 1.5B-class shape, prefix 2048, 8 steps with a new tree each step.  The
    # attention projections and the down projection are drawn with std 0.0375: then a folded
    # position's branch-specific attention output moves its residual away from the parent's
    # layer after layer, so the per-branch divergence accumulates and positions leave the fold
    # set as the stack deepens (0.71 of draft rows fold at the first layer, 0.67 at the last, 0.68
    # over all 28 layers -- near the 72 % of cells over all layers that the SpecFold summary, §3.1,
    # profiles).  With std 0.02 (or 0.03) every layer's fold set is the first layer's; with 0.04
    # the fold fraction falls to 0.23 by the last layer.
    "stack-1.5b": Workload("stack-1.5b", Shape(9, 32, 1536, 12, 2, 128, 8960, 2048), 2, 0.1,
                           layers=28, steps=8, weight_std=(0.0375, 0.0375, 0.02, 0.0375)),
    # 28-layer stack at 7B-class shape, prefix 2048; attention and down projections drawn with
    # std 0.0279, where the fold fraction falls slowly as at the 1.5B shape (0.73 of draft rows
    # at the first layer, 0.64 at the last, 0.67 over the stack; 0.0275 keeps nearly the first
    # layer's fold set, 0.029 drives it to 0.21)
    "stack-7b": Workload("stack-7b", Shape(9, 32, 3584, 28, 4, 128, 18944, 2048), 3, 0.1,
                         layers=28, weight_std=(0.0279, 0.0279, 0.02, 0.0279)),
    # one layer at 14B-class shape, prefix 4096, swept over B and delta
    "sweep-14b": Workload("sweep-14b", Shape(9, 32, 5120, 40, 8, 128, 13824, 4096), 4, 0.1,
                          branch_sweep=(2, 4, 6, 8),
                          delta_sweep=(0.0, 0.01, 0.1, 0.2, 0.3, 0.5, 0.7)),
    # one layer at 1.5B-class shape with B = 7 drafts, swept over the draft tree's shape: seven
    # siblings of main (depth 1), random trees of depth <= 2, 3, 4, and a 7-deep chain
    # one-token drafts (child law "unmask1")
    "draft-shapes-1.5b": Workload("draft-shapes-1.5b", Shape(8, 32, 1536, 12, 2, 128, 8960, 512), 5, 0.1,
                                  child_law="unmask1",
                                  tree_sweep=("star", "depth2", "depth3", "depth4", "chain")),
}


def tree_of(kind: str, n_branch: int, base_seed: int, step: int) -> np.ndarray:
    """Parent map for a tree-shape name: "star", "chain", or "depthK" (random, depth <= K)."""
    if kind.startswith("depth"):
        return parent_tree(n_branch, base_seed, step, "random", max_depth=int(kind[5:]))
    return parent_tree(n_branch, base_seed, step, kind)


# ---------------------------------------------------------------- bfloat16 rounding

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (round to nearest, ties to even); return the uint16 bit patterns."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        rounded = np.where(nan, np.uint16(0x7FC0), rounded)
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array holding the bfloat16-rounded values of ``x``."""
    return bf16_bits_to_f32(bf16_bits(x))


# ---------------------------------------------------------------- draws

def _rng(base_seed: int, step: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([base_seed, step, layer, tensor_id])


def layer_weights(shape: Shape, base_seed: int, layer: int, random_norm: bool = False) -> dict:
    """Random-init weights of one layer, float32, already rounded to bfloat16.

    Linear weights are N(0, 0.02^2) in torch ``Linear.weight`` layout ([out][in]):
    w_qkv [(Hq+2Hkv)d, D] (Q heads, then K heads, then V heads), w_o [D, Hq d],
    w_gate_up [2F, D] (gate rows, then up rows), w_down [D, F].  RMSNorm weights are
    ones unless ``random_norm`` (tests use 1 + 0.1 N(0,1) so a misplaced norm weight shows).
    """
    D, F = shape.hidden, shape.ffn
    dq = shape.n_q_heads * shape.head_dim

    def lin(tid, rows, cols):
        w = _rng(base_seed, 0, layer, tid).standard_normal((rows, cols), dtype=np.float32)
        w *= np.float32(0.02)
        return bf16_round(w)

    def norm(tid):
        if not random_norm:
            return np.ones(D, dtype=np.float32)
        g = _rng(base_seed, 0, layer, tid).standard_normal(D, dtype=np.float32)
        return bf16_round(1.0 + 0.1 * g)

    return {
        "ln1": norm(_T_LN1),
        "w_qkv": lin(_T_WQKV, shape.qkv_out, D),
        "w_o": lin(_T_WO, D, dq),
        "ln2": norm(_T_LN2),
        "w_gate_up": lin(_T_WGU, 2 * F, D),
        "w_down": lin(_T_WDOWN, D, F),
    }


def device_layer(torch, shape: Shape, seed: int, device, std=(0.02, 0.02, 0.02, 0.02)):
    """Random-init weights and prefix cache of one layer drawn on the device by torch (stacks of
    28 layers hold several GB of weights, too slow to draw on the host): projections
    N(0, std^2) in ``layer_weights``' layout and order (w_qkv, w_o, w_gate_up, w_down), RMSNorm
    weights 1, prefix K and V N(0, 1), all rounded to bfloat16.  One torch generator seeded
    with ``seed`` draws them in a fixed order.  Returns (weights dict, pk, pv)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    D, F = shape.hidden, shape.ffn

    def rnd(sd, *sz):
        return (torch.randn(*sz, device=device, generator=g) * sd).to(torch.bfloat16)

    w = {"w_qkv": rnd(std[0], shape.qkv_out, D), "w_o": rnd(std[1], D, shape.n_q_heads * shape.head_dim),
         "w_gate_up": rnd(std[2], 2 * F, D), "w_down": rnd(std[3], D, F),
         "ln1": torch.ones(D, device=device, dtype=torch.bfloat16),
         "ln2": torch.ones(D, device=device, dtype=torch.bfloat16)}
    pk = rnd(1.0, shape.prefix_len, shape.n_kv_heads, shape.head_dim)
    pv = rnd(1.0, shape.prefix_len, shape.n_kv_heads, shape.head_dim)
    return w, pk, pv


def prefix_kv(shape: Shape, base_seed: int, layer: int) -> tuple[np.ndarray, np.ndarray]:
    """Shared prefix K and V caches [P, Hkv, d], N(0,1), bfloat16-rounded, taken as already
    rotary-embedded (they were written by earlier passes)."""
    sz = (shape.prefix_len, shape.n_kv_heads, shape.head_dim)
    k = _rng(base_seed, 0, layer, _T_PK).standard_normal(sz, dtype=np.float32)
    v = _rng(base_seed, 0, layer, _T_PV).standard_normal(sz, dtype=np.float32)
    return bf16_round(k), bf16_round(v)


def parent_tree(n_branch: int, base_seed: int, step: int, kind: str = "random",
                max_depth: int = 4) -> np.ndarray:
    """Parent map par[0..B]: par[0] = -1, 0 <= par[i] < i.

    "random": draft i picks its parent uniformly among earlier branches whose depth is
    below ``max_depth`` (so no branch is deeper than ``max_depth``).  "chain": par[i] = i-1.
    "star": every draft hangs off main.
    """
    par = np.full(n_branch, -1, dtype=np.int32)
    if kind == "chain":
        par[1:] = np.arange(n_branch - 1, dtype=np.int32)
        return par
    if kind == "star":
        par[1:] = 0
        return par
    rng = _rng(base_seed, step, 0, _T_TREE)
    depth = np.zeros(n_branch, dtype=np.int64)
    for i in range(1, n_branch):
        cands = [j for j in range(i) if depth[j] < max_depth]
        p = int(cands[rng.integers(len(cands))])
        par[i] = p
        depth[i] = depth[p] + 1
    return par


def step_tokens(shape: Shape, vocab: int, base_seed: int, step: int, parent) -> np.ndarray:
    """Token ids [B+1, N] of one verification step: main's block is uniform over the
    vocabulary; each draft copies its parent's block and newly unmasks 1-4 positions with
    fresh uniform tokens (the drafts' structure of the hidden-state generator, at token level)."""
    parent = np.asarray(parent, dtype=np.int64)
    B1, N = shape.n_branch, shape.block
    rng = _rng(base_seed, step, 0, _T_TOKENS)
    tok = np.empty((B1, N), dtype=np.int32)
    tok[0] = rng.integers(0, vocab, N)
    for i in range(1, B1):
        tok[i] = tok[parent[i]]
        u = int(rng.integers(1, 5))
        pos = rng.choice(N, size=min(u, N), replace=False)
        tok[i, pos] = rng.integers(0, vocab, pos.size)
    return tok


def main_hidden(shape: Shape, base_seed: int, step: int) -> np.ndarray:
    """Main branch block hidden state [N, D], N(0,1), float64."""
    return _rng(base_seed, step, 0, _T_MAIN).standard_normal((shape.block, shape.hidden))


def child_hidden(parent_rows: np.ndarray, r: np.ndarray, unmasked: np.ndarray,
                 rng: np.random.Generator) -> np.ndarray:
    """Build a draft block from its parent block.

    Newly unmasked positions get a fresh N(0,1) row.  Every other position is the
    parent's row plus a random direction scaled to ``r[n]`` times the parent row's
    Euclidean length, so the child's distance to its parent, relative to the parent's
    length, is exactly ``r[n]`` in exact arithmetic.
    """
    n, dim = parent_rows.shape
    g = rng.standard_normal((n, dim))
    fresh = rng.standard_normal((n, dim))
    plen = np.sqrt(np.sum(parent_rows * parent_rows, axis=1, keepdims=True))
    glen = np.sqrt(np.sum(g * g, axis=1, keepdims=True))
    out = parent_rows + (r[:, None] * plen) * (g / glen)
    out[unmasked] = fresh[unmasked]
    return out


def step_inputs(shape: Shape, base_seed: int, step: int, tree: str = "random",
                child_law: str = "lognormal", parent: np.ndarray | None = None) -> dict:
    """Hidden states of all branches for one verification step.

    Returns ``{"parent": int32[B+1], "H": float64[B+1, N, D], "r": float64[B+1, N],
    "unmasked": bool[B+1, N]}``; ``r`` is the drawn relative distance of each draft row
    (NaN for main and for unmasked rows).  Children are built in branch order from the
    (already built) parent block.  With ``child_law="unmask1"`` the result also holds
    ``"committed": bool[B+1, N]`` (each branch's committed positions).
    """
    B1, N = shape.n_branch, shape.block
    if parent is None:
        parent = parent_tree(B1, base_seed, step, tree)
    parent = np.asarray(parent, dtype=np.int32)
    rng = _rng(base_seed, step, 0, _T_CHILD)
    H = np.empty((B1, N, shape.hidden))
    H[0] = main_hidden(shape, base_seed, step)
    r_all = np.full((B1, N), np.nan)
    unm_all = np.zeros((B1, N), dtype=bool)
    committed = None
    if child_law == "unmask1":
        committed = np.zeros((B1, N), dtype=bool)
        committed[0, rng.choice(N, size=min(UNMASK1_COMMITTED, N), replace=False)] = True
    for i in range(1, B1):
        if child_law == "unmask1":
            p = parent[i]
            masked = np.flatnonzero(~committed[p])
            u = int(masked[rng.integers(masked.size)]) if masked.size else int(rng.integers(N))
            unmasked = np.zeros(N, dtype=bool)
            unmasked[u] = True
            committed[i] = committed[p] | unmasked
            r = np.where(committed[p], rng.lognormal(UNMASK1_MU_COMMITTED, LOGNORMAL_SIGMA, N),
                         rng.lognormal(UNMASK1_MU_MASKED, LOGNORMAL_SIGMA, N))
        elif child_law == "tiny":
            small = rng.random(N) < 0.7
            r = np.where(small, rng.uniform(0.01, 0.08, N), rng.uniform(0.15, 1.0, N))
            unmasked = np.zeros(N, dtype=bool)
        else:
            u = int(rng.integers(1, 5))
            unmasked = np.zeros(N, dtype=bool)
            unmasked[rng.choice(N, size=min(u, N), replace=False)] = True
            r = rng.lognormal(LOGNORMAL_MU, LOGNORMAL_SIGMA, N)
        H[i] = child_hidden(H[parent[i]], r, unmasked, rng)
        r_all[i] = np.where(unmasked, np.nan, r)
        unm_all[i] = unmasked
    out = {"parent": parent, "H": H, "r": r_all, "unmasked": unm_all}
    if committed is not None:
        out["committed"] = committed
    return out


def expected_fold_fraction(delta: float, n_block: int = 32) -> float:
    """Layer-0 folded fraction of draft rows implied by the log-normal law (unmasked
    rows never fold for delta < sqrt(2))."""
    if delta <= 0:
        return 0.0
    z = (math.log(delta) - LOGNORMAL_MU) / LOGNORMAL_SIGMA
    phi = 0.5 * (1.0 + math.erf(z / math.sqrt(2.0)))
    return (1.0 - 2.5 / n_block) * phi
