"""A plain dense transformer layer built only from torch library routines (float64, CPU).

Used by the tests as an outside pin of the oracle: with no folded position (delta = 0 on
perturbed inputs) the folded layer must reduce to this standard pre-RMSNorm GQA attention +
SwiGLU layer applied to each branch on its own.  It shares nothing with ``oracle``: the
norm is ``F.rms_norm``, projections are ``F.linear``, rotary embedding is a complex
multiplication, attention is ``F.scaled_dot_product_attention`` with the KV heads repeated
per group, and the activation is ``F.silu``.
"""

import torch
import torch.nn.functional as F

f64 = torch.float64


def t(x):
    return torch.as_tensor(x, dtype=f64)


def rope_complex(x, pos, theta):
    """Rotate-half rotary embedding as a complex product: the pair (x_j, x_{j+d/2}) is the
    complex number x_j + i x_{j+d/2}, multiplied by exp(i pos theta^(-2j/d))."""
    d = x.shape[-1]
    half = d // 2
    z = torch.complex(x[..., :half].contiguous(), x[..., half:].contiguous())
    freqs = torch.pow(torch.tensor(float(theta), dtype=f64), -2.0 * torch.arange(half, dtype=f64) / d)
    ang = pos[..., None] * freqs
    z = z * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


def attention_sdpa(q, k, v, pk, pv):
    """q [N, Hq, d]; k, v [N, Hkv, d]; pk, pv [P, Hkv, d] -> [N, Hq, d]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    keys = torch.cat([pk, k], 0).permute(1, 0, 2).repeat_interleave(G, dim=0)
    vals = torch.cat([pv, v], 0).permute(1, 0, 2).repeat_interleave(G, dim=0)
    o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], keys[None], vals[None])
    return o[0].permute(1, 0, 2)


def dense_layer(Hb, weights, pk, pv, shape):
    Hb = t(Hb)
    N, D = Hb.shape
    Hq, Hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    pos = shape.prefix_len + torch.arange(N, dtype=f64)
    x = F.rms_norm(Hb, (D,), weight=t(weights["ln1"]), eps=shape.rms_eps)
    qkv = F.linear(x, t(weights["w_qkv"]))
    q = qkv[:, : Hq * d].reshape(N, Hq, d)
    k = qkv[:, Hq * d: (Hq + Hkv) * d].reshape(N, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].reshape(N, Hkv, d)
    q = rope_complex(q, pos[:, None], shape.rope_theta)
    k = rope_complex(k, pos[:, None], shape.rope_theta)
    a = attention_sdpa(q, k, v, t(pk), t(pv)).reshape(N, Hq * d)
    h = Hb + F.linear(a, t(weights["w_o"]))
    y = F.rms_norm(h, (D,), weight=t(weights["ln2"]), eps=shape.rms_eps)
    g, u = F.linear(y, t(weights["w_gate_up"])).split(shape.ffn, dim=-1)
    return (h + F.linear(F.silu(g) * u, t(weights["w_down"]))).numpy()
