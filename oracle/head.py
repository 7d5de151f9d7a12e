"""The steps either side of the layer stack, in float64: token-embedding gather before
layer 0, and the final RMSNorm, language-model head and per-row greedy token after the last
layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the product path.

[SpecFold summary, App. B]: the folded kernels cover the transformer layers; embeddings and
the language-model head stay outside them (in PyTorch / cuBLAS on the pages).  The LM head
is not folded: every row of every branch gets its logits.  [SpecFold summary, §1]: a
verification pass scores every branch's block, so the per-row greedy token is the plain
reading of what the head produces for acceptance (readings listed in the design notes):
* the final RMSNorm has a weight vector and the layer's eps;
* no bias on the LM head; logits[r][v] = xn[r] . W_lm[v];
* the greedy token of a row is the lowest index among its maximal logits, where a NaN logit
  is no candidate at all (it is neither larger nor smaller than any other value, so it can
  never be "the maximum"); a row with no candidate (every logit NaN) has token -1 and best
  logit NaN; +inf and -inf are ordinary candidates;
* a token id outside [0, V) embeds as a row of NaN.
"""

from __future__ import annotations

import numpy as np

from .layer import rms_norm


def embed(tokens, E):
    """Rows E[tokens[r]] (float64); ids outside [0, V) give NaN rows."""
    tokens = np.asarray(tokens)
    E = np.asarray(E, dtype=np.float64)
    out = np.full(tokens.shape + (E.shape[1],), np.nan)
    ok = (tokens >= 0) & (tokens < E.shape[0])
    out[ok] = E[tokens[ok]]
    return out


def final_norm(H, ln_f, eps):
    """RMSNorm of every row with weight ln_f."""
    return rms_norm(H, ln_f, eps)


def lm_head_logits(xn, W_lm):
    """logits[r][v] = xn[r] . W_lm[v] (float64 matrix product)."""
    return np.asarray(xn, dtype=np.float64) @ np.asarray(W_lm, dtype=np.float64).T


def greedy_tokens(logits):
    """Per row: the lowest index among the maximal non-NaN logits, and that maximum; a row
    whose logits are all NaN gives token -1 and NaN."""
    logits = np.asarray(logits, dtype=np.float64)
    cand = ~np.isnan(logits)
    has = cand.any(axis=-1)
    # NaN entries become -inf for the max; a row that has candidates reaches its maximum at a
    # candidate (if that maximum is -inf, the first -inf candidate, never a former NaN)
    filled = np.where(cand, logits, -np.inf)
    mx = filled.max(axis=-1)
    tok = np.argmax((filled == mx[..., None]) & cand, axis=-1)
    tok = np.where(has, tok, -1)
    mx = np.where(has, mx, np.nan)
    return tok.astype(np.int64), mx


def verify_head(H, ln_f, W_lm, eps):
    """Final RMSNorm, LM head and greedy token of every row of H [R][D]."""
    return greedy_tokens(lm_head_logits(final_norm(H, ln_f, eps), W_lm))
