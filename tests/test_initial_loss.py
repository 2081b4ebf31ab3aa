"""Step-0 loss of a random decoder is near ln(vocab), with the oracle as the
attention (CPU).  The pages print 8.40 for vocab 4096 and 9.65 for 16 384;
both are within 2 % of ln(vocab), the tolerance used here."""
import json
import math
import os

import numpy as np
import torch

from oracle import attention as OA
from oracle import rope as OR
from tests.tiny_decoder import build_weights, random_tokens, step0_loss

HERE = os.path.dirname(os.path.abspath(__file__))


def test_printed_values_near_ln_vocab():
    gold = json.load(open(os.path.join(HERE, "golden", "initial_loss.json")))
    for c in gold["cases"]:
        rel = abs(c["printed_loss"] - math.log(c["vocab"])) / math.log(c["vocab"])
        assert rel < gold["tolerance_rel"], c


def test_random_decoder_step0_loss_with_oracle_attention():
    B, T, vocab = 2, 64, 4096
    w = build_weights(n_layers=2, vocab=vocab)
    tok, tgt = random_tokens(B, T, vocab)
    dh = 384 // 6
    table = OR.inv_freq(dh, 1e4)

    def attn(q, k, v):
        o, _ = OA.attn_fwd(q.double().numpy(), k.double().numpy(),
                           v.double().numpy(), 1.0 / math.sqrt(dh), 0, 0.0)
        return torch.from_numpy(o).float()

    def rope(x):
        return torch.from_numpy(OR.rope(x.double().numpy(), table)).float()

    loss = step0_loss(w, tok, tgt, attn, rope)
    assert abs(loss - math.log(vocab)) / math.log(vocab) < 0.02, loss
    assert np.isfinite(loss)
