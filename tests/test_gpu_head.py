"""GPU parity of the steps either side of the layer stack (embedding gather, final RMSNorm,
LM head, greedy token) against the oracle.

The greedy token is an argmax: the GPU decides it on fp32 logits of bf16-rounded normalised
rows, the oracle on float64 logits.  Where a row's top two oracle logits are further apart
than twice a bound on the GPU's logit error, the tokens must be equal; elsewhere the GPU's
token must be within that bound of the maximum.  Planted maxima and planted ties (identical
weight rows) are checked exactly."""

import numpy as np
import pytest
import torch

import oracle
from gpu_case import DEV, dev_bf16
from sparse_layer_rho_amd import specfold as sf
from synth import Shape, bf16_round

pytestmark = pytest.mark.gpu


def _shape(B1, N, D):
    return Shape(B1, N, D, 4, 2, 64, 256, 0)


def _check_tokens(H, ln, W, tok_gpu, logit_gpu, eps, rows=None):
    """Compare GPU tokens with the oracle's on `rows` (all by default).  NaN logits are no
    candidates on either side; a row without candidates must give token -1 and logit NaN."""
    rows = np.arange(H.shape[0]) if rows is None else np.asarray(rows)
    xn = oracle.final_norm(H[rows], ln, eps)
    with np.errstate(invalid="ignore"):
        logits = oracle.lm_head_logits(xn, W)
    tok_o, mx = oracle.greedy_tokens(logits)
    tg = tok_gpu[rows]
    none = tok_o < 0
    assert np.array_equal(tg[none], tok_o[none]) and np.isnan(logit_gpu[rows][none]).all()
    keep = ~none
    rows, xn, logits, tok_o, mx, tg = rows[keep], xn[keep], logits[keep], tok_o[keep], mx[keep], tg[keep]
    if rows.size == 0:
        return 0.0
    nanc = np.isnan(logits)
    # bf16 rounding of xn (relative 2^-8) plus fp32 accumulation over D terms
    with np.errstate(invalid="ignore"):
        mag = np.nan_to_num(np.abs(xn) @ np.nan_to_num(np.abs(W)).T)
    bound = (2.0 ** -8 + H.shape[1] * 2.0 ** -24) * mag.max(axis=1)
    srt = np.sort(np.where(nanc, -np.inf, logits), axis=1)
    gap = srt[:, -1] - srt[:, -2] if logits.shape[1] > 1 else np.full(rows.size, np.inf)
    clear = gap > 2 * bound
    assert np.array_equal(tg[clear], tok_o[clear])
    assert ((tg >= 0) & (tg < W.shape[0])).all()
    chosen = logits[np.arange(rows.size), tg]
    assert not np.isnan(chosen).any(), "a NaN logit was chosen"
    assert (chosen >= mx - 2 * bound).all()
    assert np.all(np.abs(logit_gpu[rows] - chosen) <= bound + 1e-6)
    return clear.mean()


def test_embed_matches_oracle():
    sh = _shape(3, 8, 64)
    R, D, V = 24, 64, 1000
    rng = np.random.default_rng(0)
    E = bf16_round(rng.standard_normal((V, D)).astype(np.float32))
    tokens = rng.integers(0, V, R).astype(np.int32)
    tokens[[3, 17]] = [-1, V]                               # ids outside the vocabulary
    H = torch.empty((R, D), dtype=torch.bfloat16, device=DEV)
    sf.embed(sh, torch.from_numpy(tokens).to(DEV), dev_bf16(E), H)
    torch.cuda.synchronize()
    got = H.float().cpu().numpy()
    ref = oracle.embed(tokens, E)
    ok = ~np.isnan(ref).any(axis=1)
    assert np.array_equal(got[ok], ref[ok])
    assert np.isnan(got[~ok]).all()


@pytest.mark.parametrize("B1,N,D,V", [(3, 8, 64, 1000), (9, 32, 256, 4099), (1, 5, 128, 64)])
def test_lm_head_matches_oracle(B1, N, D, V):
    sh = _shape(B1, N, D)
    R = B1 * N
    rng = np.random.default_rng(V)
    H = bf16_round(rng.standard_normal((R, D)).astype(np.float32))
    ln = bf16_round((1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    W = bf16_round((0.02 * rng.standard_normal((V, D))).astype(np.float32))
    tok = torch.full((R,), -7, dtype=torch.int32, device=DEV)
    logit = torch.full((R,), float("nan"), device=DEV)
    ws = sf.head_workspace(sh, V)
    sf.lm_head(sh, dev_bf16(H), dev_bf16(ln), dev_bf16(W), tok, logit, ws)
    torch.cuda.synchronize()
    frac = _check_tokens(H.astype(np.float64), ln, W.astype(np.float64), tok.cpu().numpy(), logit.cpu().numpy(),
                         sh.rms_eps)
    assert frac > 0.5


def test_lm_head_planted_maxima_and_ties():
    """Row r's maximum is planted at token t_r (a scaled copy of its normalised row); for row 0
    two identical weight rows share the maximum and the lower index must win."""
    sh = _shape(2, 16, 128)
    R, D, V = 32, 128, 3000
    rng = np.random.default_rng(5)
    H = bf16_round(rng.standard_normal((R, D)).astype(np.float32))
    ln = np.ones(D, np.float32)
    W = bf16_round((0.01 * rng.standard_normal((V, D))).astype(np.float32))
    t = rng.permutation(V)[:R]
    W[t] = bf16_round((0.05 * H / np.linalg.norm(H, axis=1, keepdims=True) * np.sqrt(D)).astype(np.float32))
    W[t[0] + 1 if t[0] + 1 < V else t[0] - 1] = W[t[0]]   # planted tie for row 0
    tie = sorted([t[0], t[0] + 1 if t[0] + 1 < V else t[0] - 1])
    tok = torch.empty((R,), dtype=torch.int32, device=DEV)
    logit = torch.empty((R,), device=DEV)
    ws = sf.head_workspace(sh, V)
    sf.lm_head(sh, dev_bf16(H), dev_bf16(ln), dev_bf16(W), tok, logit, ws)
    torch.cuda.synchronize()
    got = tok.cpu().numpy()
    assert got[0] == tie[0]
    assert np.array_equal(got[1:], t[1:])


def test_lm_head_full_vocab_sampled_rows():
    """1.5B-class head: D 1536, V 151936, R 288; the oracle scores a sample of rows."""
    sh = Shape(9, 32, 1536, 12, 2, 128, 8960, 0)
    R, D, V = 288, 1536, 151936
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    W = (0.02 * torch.randn(V, D, device=DEV, generator=g)).to(torch.bfloat16)
    Hd = torch.randn(R, D, device=DEV, generator=g).to(torch.bfloat16)
    ln = torch.ones(D, dtype=torch.bfloat16, device=DEV)
    tok = torch.empty((R,), dtype=torch.int32, device=DEV)
    logit = torch.empty((R,), device=DEV)
    ws = sf.head_workspace(sh, V)
    sf.lm_head(sh, Hd, ln, W, tok, logit, ws)
    torch.cuda.synchronize()
    rows = [0, 1, 77, 150, 286, 287]
    Wh = W.float().cpu().numpy().astype(np.float64)
    _check_tokens(Hd.float().cpu().numpy().astype(np.float64), np.ones(D), Wh, tok.cpu().numpy(),
                  logit.cpu().numpy(), sh.rms_eps, rows)


def test_lm_head_vocab_in_pieces():
    """W_lm over 1 GB (D 5120, V 106000: two launches); row 0's maximum is planted in the
    second piece, row 1's in the first."""
    sh = Shape(1, 8, 5120, 40, 8, 128, 13824, 0)
    R, D, V = 8, 5120, 106000
    g = torch.Generator(device=DEV)
    g.manual_seed(13)
    W = (0.01 * torch.randn(V, D, device=DEV, generator=g)).to(torch.bfloat16)
    Hd = torch.randn(R, D, device=DEV, generator=g).to(torch.bfloat16)
    xn_dir = Hd.float() / Hd.float().norm(dim=1, keepdim=True)
    W[105900] = (0.05 * np.sqrt(D) * xn_dir[0]).to(torch.bfloat16)
    W[17] = (0.05 * np.sqrt(D) * xn_dir[1]).to(torch.bfloat16)
    ln = torch.ones(D, dtype=torch.bfloat16, device=DEV)
    tok = torch.empty((R,), dtype=torch.int32, device=DEV)
    logit = torch.empty((R,), device=DEV)
    ws = sf.head_workspace(sh, V)
    sf.lm_head(sh, Hd, ln, W, tok, logit, ws)
    torch.cuda.synchronize()
    got = tok.cpu().numpy()
    assert got[0] == 105900 and got[1] == 17
    rows = [2, 7]
    Wh = W.float().cpu().numpy().astype(np.float64)
    _check_tokens(Hd.float().cpu().numpy().astype(np.float64), np.ones(D), Wh, got, logit.cpu().numpy(),
                  sh.rms_eps, rows)


def _run_head(sh, H, ln, W):
    R = sh.n_branch * sh.block
    V = W.shape[0]
    tok = torch.full((R,), -7, dtype=torch.int32, device=DEV)
    logit = torch.full((R,), 7.0, device=DEV)
    ws = sf.head_workspace(sh, V)
    sf.lm_head(sh, dev_bf16(H), dev_bf16(ln), dev_bf16(W), tok, logit, ws)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), logit.cpu().numpy()


def test_lm_head_nan_logits_are_never_chosen():
    """NaN weight rows give a NaN logit in every row (never chosen, even where the row's maximum
    would have been); a NaN in a hidden row makes all its logits NaN (token -1, logit NaN)."""
    sh = _shape(3, 8, 128)
    R, D, V = 24, 128, 1000
    rng = np.random.default_rng(21)
    H = bf16_round(rng.standard_normal((R, D)).astype(np.float32))
    ln = np.ones(D, np.float32)
    W = bf16_round((0.02 * rng.standard_normal((V, D))).astype(np.float32))
    # row 0's maximum is planted at column 123, then that weight row gets a NaN
    W[123] = bf16_round((0.05 * H[0] / np.linalg.norm(H[0]) * np.sqrt(D)).astype(np.float32))
    W[123, 7] = np.nan
    W[[5, V - 1]] = np.nan
    H[5] = np.nan
    H[6, 17] = np.nan
    tok, logit = _run_head(sh, H, ln, W)
    assert tok[5] == -1 and tok[6] == -1 and np.isnan(logit[5]) and np.isnan(logit[6])
    assert tok[0] != 123 and not np.isin(tok, [5, V - 1, 123]).any()
    _check_tokens(H.astype(np.float64), ln.astype(np.float64), W.astype(np.float64), tok, logit, sh.rms_eps)


@pytest.mark.parametrize("V", [1, 3, 6, 4099])
def test_lm_head_last_columns_of_a_vocab_not_a_multiple_of_4(V):
    """The last V % 4 columns are scored: row 0's maximum is planted in column V - 1, row 1's in
    column V - 2 (when there is one)."""
    sh = _shape(2, 16, 128)
    R, D = 32, 128
    rng = np.random.default_rng(V)
    H = bf16_round(rng.standard_normal((R, D)).astype(np.float32))
    ln = np.ones(D, np.float32)
    W = bf16_round((0.01 * rng.standard_normal((V, D))).astype(np.float32))
    W[V - 1] = bf16_round((0.05 * H[0] / np.linalg.norm(H[0]) * np.sqrt(D)).astype(np.float32))
    if V > 1:
        W[V - 2] = bf16_round((0.05 * H[1] / np.linalg.norm(H[1]) * np.sqrt(D)).astype(np.float32))
    tok, logit = _run_head(sh, H, ln, W)
    assert tok[0] == V - 1
    if V > 1:
        assert tok[1] == V - 2
    assert ((tok >= 0) & (tok < V)).all() and np.isfinite(logit).all()
    _check_tokens(H.astype(np.float64), ln.astype(np.float64), W.astype(np.float64), tok, logit, sh.rms_eps)
