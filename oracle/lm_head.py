"""fp64 reference of the mask-view confidence producer that feeds the accept
scan (test infrastructure only).

[P4] para 3: a position is accepted when the draft view and the mask view
agree and the mask-view confidence exceeds the threshold.  The pages do not
spell out where the mask view's token and confidence come from; the reading
taken here is the usual one for masked diffusion decoding: the model's LM head
maps each row's final hidden state to vocabulary logits, the token is the
argmax and the confidence is its softmax probability.  The draft view's tokens
come from the same head applied to the draft rows (the model drafts for
itself).  Ties in the argmax go to the lower token id.
"""

from __future__ import annotations

import numpy as np

from . import reference as R


def lm_head_confidence(h_bits, w_bits):
    """Argmax token and its softmax probability per row.

    ``h_bits`` bf16 [rows, hidden] final hidden states; ``w_bits`` bf16
    [vocab, hidden], the head as an nn.Linear weight (no bias).  Logits
    z = h . W^T in fp64; token = the first index of max z; confidence =
    exp(z_max) / sum_v exp(z_v) = 1 / sum_v exp(z_v - z_max).
    Returns (token int32 [rows], confidence fp64 [rows], logits fp64 [rows, vocab]).
    """
    h = R.bf16_bits_to_f64(h_bits)
    w = R.bf16_bits_to_f64(w_bits)
    z = h @ w.T
    tok = np.argmax(z, axis=1).astype(np.int32)  # first maximum: the lower id on ties
    zmax = z[np.arange(z.shape[0]), tok]
    conf = 1.0 / np.exp(z - zmax[:, None]).sum(axis=1)
    return tok, conf, z


def verify_chain(h_draft_bits, h_mask_bits, w_bits, batch, window, threshold):
    """Draft tokens from the draft rows, mask tokens and confidences from the
    mask rows (rows grouped by sequence, ``window`` per sequence), then the
    accept scan of each sequence [P4 para 3]."""
    dtok, _, _ = lm_head_confidence(h_draft_bits, w_bits)
    mtok, conf, _ = lm_head_confidence(h_mask_bits, w_bits)
    dtok = dtok.reshape(batch, window)
    mtok = mtok.reshape(batch, window)
    conf = conf.reshape(batch, window)
    acc = np.array([R.accept_length(dtok[b], mtok[b], conf[b], threshold)
                    for b in range(batch)], np.int32)
    return dtok, mtok, conf, acc
