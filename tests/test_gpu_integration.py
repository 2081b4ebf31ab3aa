"""Integration checks on the GPU: the torch.autograd wrapper returns exactly
fa_bwd's gradients, and a randomly initialised decoder whose attention runs
through fa_fwd starts at a cross-entropy near ln(vocab) (the pages print
8.40 for vocab 4096)."""
import math

import numpy as np
import pytest
import torch

from causal_attention_fa_amd import synth
from tests.gpu_util import dev, say
from tests.tiny_decoder import build_weights, random_tokens, step0_loss

pytestmark = pytest.mark.gpu


def test_autograd_wrapper_matches_fa_bwd():
    from causal_attention_fa_amd import fa
    w = synth.Workload("ag", "bf16", 2, 4, 2, 200, 128, window=50, softcap=20.0)
    q, k, v, do = (t.to(dev()) for t in synth.draw(w))
    say("[integration] autograd wrapper")
    qa, ka, va = (t.clone().requires_grad_() for t in (q, k, v))
    o = fa.FlashAttention.apply(qa, ka, va, w.scale, w.window, w.softcap)
    o.backward(do)
    o2, lse = fa.attention_forward(q, k, v, w.scale, w.window, 0, w.softcap)
    dq, dk, dv = fa.attention_backward(q, k, v, o2, lse, do, w.scale, w.window, 0, w.softcap)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    assert torch.equal(qa.grad, dq) and torch.equal(ka.grad, dk) and torch.equal(va.grad, dv)


def test_random_decoder_initial_loss_with_fa_fwd():
    from causal_attention_fa_amd import fa
    say("[integration] step-0 loss, attention through fa_fwd")
    B, T, vocab = 4, 256, 4096
    wts = build_weights(n_layers=2, vocab=vocab)
    tok, tgt = random_tokens(B, T, vocab)
    dh = 64
    tab = torch.from_numpy(fa.fa_rope_inv_freq(dh, 1e4)).to(dev())

    def attn(q, k, v):
        qd, kd, vd = (t.to(dev(), torch.bfloat16).contiguous() for t in (q, k, v))
        o, _ = fa.attention_forward(qd, kd, vd, 1.0 / math.sqrt(dh))
        return o.float().cpu()

    def rope(x):
        return fa.rope(x.to(dev(), torch.bfloat16).contiguous(), tab).float().cpu()

    loss = step0_loss(wts, tok, tgt, attn, rope)
    say(f"  loss {loss:.4f} vs ln V {math.log(vocab):.4f}")
    assert abs(loss - math.log(vocab)) / math.log(vocab) < 0.02
