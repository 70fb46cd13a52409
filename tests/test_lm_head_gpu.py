"""GPU parity of the mask-view confidence producer (lm_head_confidence) and of
its chain into the accept scan.

Tokens (an argmax decided on fp32 logits on the GPU, fp64 in the oracle) must
equal the oracle's except at certified near-ties: where they differ, the
oracle's logits of the two tokens must lie within 1e-3 of each other (the
synthetic logits have standard deviation about 16; fp32 accumulation over the
hidden size moves them by far less).  Confidences: the float tolerance of the
step (max|d| <= 2e-2 max|ref|, rel-L2 <= 5e-3) and, where the tokens agree,
1e-3 relative per row.  The accept scan on the GPU's own tokens and
confidences is bit-exact against the oracle's scan of the same values.
"""

import numpy as np
import pytest

import oracle as O
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from tests import gpu_util as G  # noqa: E402

DEV = "cuda:0"
TIE_TOL = 1e-3


def _fd():
    import kv_cache_attention_flash_amd as fd
    fd.load()
    return fd


def _banner(msg):
    print(f"[lm_head] {msg}", flush=True)


def _check_rows(tok_g, conf_g, tok_o, conf_o, z, what):
    """Returns the number of certified near-ties."""
    near = 0
    for r in range(len(tok_o)):
        if int(tok_g[r]) != int(tok_o[r]):
            gap = z[r, int(tok_o[r])] - z[r, int(tok_g[r])]
            assert 0.0 <= gap <= TIE_TOL, (what, r, int(tok_g[r]), int(tok_o[r]), gap)
            near += 1
        else:
            assert abs(conf_g[r] - conf_o[r]) <= 1e-3 * conf_o[r], (what, r, conf_g[r], conf_o[r])
    G.assert_close(conf_g, conf_o, f"{what}: confidence")
    return near


@pytest.mark.parametrize("name", ["tiny_lmhead_v77", "small_lmhead_v1000"])
def test_small_heads_against_oracle(name):
    fd = _fd()
    wl = synth.LM_HEAD_WORKLOADS[name]()
    w, hd, hm = synth.lm_head_tensors(wl, DEV)
    for what, h_dev, h_bits in (("draft", hd, wl.h_draft), ("mask", hm, wl.h_mask)):
        tok, conf = fd.lm_head_confidence(h_dev, w)
        torch.cuda.synchronize()
        tok_o, conf_o, z = O.lm_head_confidence(h_bits, wl.w)
        near = _check_rows(tok.cpu().numpy(), conf.cpu().numpy().astype(np.float64), tok_o, conf_o,
                           z, f"{name} {what}")
        _banner(f"{name} {what}: {wl.rows} rows, near-ties {near}")


def test_ties_go_to_the_lower_id():
    """Duplicate weight rows give bitwise-equal logits: inside a lane pair,
    across waves of a tile and across column tiles the lower id must win."""
    fd = _fd()
    g = np.random.default_rng(7)
    hid, vocab, rows = 128, 700, 40
    w = g.standard_normal((vocab, hid)).astype(np.float32)
    w[256:512] = w[0:256]        # across column tiles
    w[512:700:2] = w[513:700:2]  # neighbours inside a tile (the even id is the lower)
    w[600:632] = w[100:132]      # a later tile repeats an earlier slice
    h = g.standard_normal((rows, hid)).astype(np.float32)
    wb, hb = synth.to_bf16_bits(w), synth.to_bf16_bits(h)
    tok, conf = fd.lm_head_confidence(G.bf16_tensor(hb, DEV), G.bf16_tensor(wb, DEV))
    torch.cuda.synchronize()
    tok_o, conf_o, z = O.lm_head_confidence(hb, wb)
    near = _check_rows(tok.cpu().numpy(), conf.cpu().numpy().astype(np.float64), tok_o, conf_o, z,
                       "ties")
    assert near == 0
    # all weight rows equal: every logit ties, token 0, confidence 1/V
    wb_eq = np.repeat(wb[:1], vocab, axis=0)
    tok, conf = fd.lm_head_confidence(G.bf16_tensor(hb, DEV), G.bf16_tensor(wb_eq, DEV))
    torch.cuda.synchronize()
    assert torch.all(tok == 0)
    assert torch.allclose(conf, torch.full_like(conf, 1.0 / vocab), rtol=1e-5, atol=0)


def test_reruns_are_bitwise_equal_and_rows_are_independent():
    fd = _fd()
    wl = synth.small_lm_head()
    w, hd, hm = synth.lm_head_tensors(wl, DEV)
    t1, c1 = fd.lm_head_confidence(hm, w)
    t2, c2 = fd.lm_head_confidence(hm.clone(), w)
    # a row computed alone equals the same row inside the batch
    t3, c3 = fd.lm_head_confidence(hm[5:6].contiguous(), w)
    torch.cuda.synchronize()
    assert torch.equal(t1, t2) and torch.equal(c1, c2)
    assert int(t3[0]) == int(t1[5]) and float(c3[0]) == float(c1[5])


def test_chain_into_the_accept_scan():
    """Draft tokens from the draft rows, mask tokens and confidences from the
    mask rows, then verify_accept: exact against the oracle's scan of the GPU's
    own tokens and confidences; the fully independent oracle chain agrees except
    where a token near-tie or a confidence within 1e-3 of the threshold decides."""
    fd = _fd()
    wl = synth.small_lm_head()
    w, hd, hm = synth.lm_head_tensors(wl, DEV)
    dt, _ = fd.lm_head_confidence(hd, w)
    mt, mc = fd.lm_head_confidence(hm, w)
    shape = (wl.batch, wl.window)
    acc = fd.verify_accept(dt.view(shape), mt.view(shape), mc.view(shape), wl.threshold)
    torch.cuda.synchronize()
    dt_h, mt_h = dt.cpu().numpy().reshape(shape), mt.cpu().numpy().reshape(shape)
    mc_h = mc.cpu().numpy().reshape(shape)
    want = [O.accept_length(dt_h[b], mt_h[b], mc_h[b], wl.threshold) for b in range(wl.batch)]
    assert acc.cpu().numpy().tolist() == want
    dtok, mtok, conf, acc_o = O.verify_chain(wl.h_draft, wl.h_mask, wl.w, wl.batch, wl.window,
                                             wl.threshold)
    for b in range(wl.batch):
        if int(acc_o[b]) == want[b]:
            continue
        k = min(int(acc_o[b]), want[b])  # first position where the two scans differ
        decided_by_tie = (int(dtok[b, k]) != int(dt_h[b, k]) or int(mtok[b, k]) != int(mt_h[b, k]))
        decided_by_thr = abs(float(conf[b, k]) - float(wl.threshold)) <= 1e-3
        assert decided_by_tie or decided_by_thr, (b, k, acc_o[b], want[b])
    _banner(f"chain: accept lengths {want} (oracle chain {acc_o.tolist()})")


def test_full_size_head_sampled():
    """512 rows through the 126464-token head at hidden 4096: 32 sampled rows
    of each view against the oracle, the chain's accept scan exact on the GPU's
    own values, and the bitwise rerun."""
    fd = _fd()
    wl = synth.llada8b_lm_head_b8()
    w, hd, hm = synth.lm_head_tensors(wl, DEV)
    h_all = torch.cat([hd, hm])
    tok, conf = fd.lm_head_confidence(h_all, w)
    tok2, conf2 = fd.lm_head_confidence(h_all, w)
    torch.cuda.synchronize()
    assert torch.equal(tok, tok2) and torch.equal(conf, conf2)
    rows = np.concatenate([np.arange(0, 512, 16), np.arange(7, 512, 16)])
    w_bits = G.bits_of(w)
    h_bits = G.bits_of(h_all)[rows]
    tok_o, conf_o, z = O.lm_head_confidence(h_bits, w_bits)
    near = _check_rows(tok.cpu().numpy()[rows], conf.cpu().numpy()[rows].astype(np.float64),
                       tok_o, conf_o, z, "full size")
    shape = (wl.batch, wl.window)
    dt, mt, mc = tok[:256].view(shape), tok[256:].view(shape), conf[256:].view(shape)
    acc = fd.verify_accept(dt.contiguous(), mt.contiguous(), mc.contiguous(), wl.threshold)
    torch.cuda.synchronize()
    dt_h, mt_h, mc_h = dt.cpu().numpy(), mt.cpu().numpy(), mc.cpu().numpy()
    want = [O.accept_length(dt_h[b], mt_h[b], mc_h[b], wl.threshold) for b in range(wl.batch)]
    assert acc.cpu().numpy().tolist() == want
    agree = float((dt_h == mt_h).mean())
    _banner(f"full size: {len(rows)} rows checked, near-ties {near}; views agree on "
            f"{agree:.2f} of positions, conf > 0.9 on {float((mc_h > 0.9).mean()):.2f}; "
            f"accept {want}")
