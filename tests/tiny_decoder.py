"""A small randomly initialised decoder for the step-0 loss sanity check.

Shapes follow Forge's default model (forge-studio RESEARCH.md, section 2:
vocab 4096, d_model 384, 6 heads, d_ff 1024, RMSNorm, SwiGLU, RoPE, tied
embeddings); weights are N(0, 0.02^2).  Attention is a callable supplied by
the caller (the float64 oracle on the CPU, or the HIP fa_fwd on the GPU);
everything else is plain torch.  With near-uniform logits the mean
cross-entropy of uniformly random targets sits near ln(vocab).
"""
import math

import torch


def build_weights(n_layers=2, vocab=4096, d_model=384, n_heads=6, d_ff=1024,
                  seed=0):
    g = torch.Generator("cpu").manual_seed(seed)

    def w(*shape):
        return torch.randn(shape, generator=g) * 0.02

    layers = []
    for _ in range(n_layers):
        layers.append(dict(wq=w(d_model, d_model), wk=w(d_model, d_model),
                           wv=w(d_model, d_model), wo=w(d_model, d_model),
                           w1=w(d_ff, d_model), w3=w(d_ff, d_model),
                           w2=w(d_model, d_ff)))
    return dict(emb=w(vocab, d_model), layers=layers, n_heads=n_heads)


def _rms(x, eps=1e-6):
    return x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + eps)


def step0_loss(weights, tokens, targets, attention, rope):
    """Mean cross-entropy of one forward pass.

    attention(q, k, v) -> o with q, k, v [B, H, T, dh] float32 CPU tensors;
    rope(x) -> x rotated, same shape.
    """
    emb = weights["emb"]
    H = weights["n_heads"]
    B, T = tokens.shape
    x = emb[tokens]
    D = x.shape[-1]
    dh = D // H
    for L in weights["layers"]:
        h = _rms(x)
        q = (h @ L["wq"].T).view(B, T, H, dh).transpose(1, 2)
        k = (h @ L["wk"].T).view(B, T, H, dh).transpose(1, 2)
        v = (h @ L["wv"].T).view(B, T, H, dh).transpose(1, 2)
        o = attention(rope(q.contiguous()), rope(k.contiguous()), v.contiguous())
        x = x + o.transpose(1, 2).reshape(B, T, D) @ L["wo"].T
        h = _rms(x)
        x = x + (torch.nn.functional.silu(h @ L["w1"].T) * (h @ L["w3"].T)) @ L["w2"].T
    logits = _rms(x) @ emb.T
    return torch.nn.functional.cross_entropy(
        logits.reshape(-1, logits.shape[-1]), targets.reshape(-1)).item()


def random_tokens(B, T, vocab, seed=1):
    g = torch.Generator("cpu").manual_seed(seed)
    tok = torch.randint(0, vocab, (B, T + 1), generator=g)
    return tok[:, :-1], tok[:, 1:]


LN_4096 = math.log(4096)
