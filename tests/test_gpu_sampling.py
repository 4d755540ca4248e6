"""GPU parity of the temperature > 0 accept (strict rejection sampling, Orthrus paper summary
sec. 四 and Q&A) at the LM-head + consensus workload's own shape, its output law on a tiny
vocabulary, and its handling of draft ids outside the vocabulary.

Decisions that floating point takes (u q(d) < p(d), the residual race) are compared with the oracle
run on the GPU's own fp32 logits, so that both sides decide on the same operands; the logits
themselves are compared with the oracle's float64 product separately.
"""
import numpy as np
import pytest
import scipy.special as sp
import scipy.stats as st
import torch

import orthrus_round_amd as ora
import synth
from oracle import decode as Dc
from oracle import model as M
from oracle import philox as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == ora.BF16:
        t = t.to(torch.bfloat16)
    return t.to(DEV)


def state(B, ctx0=500, max_out=64):
    st_ = {k: torch.zeros(B, dtype=torch.int32, device=DEV) for k in ("anchor", "accept", "out_len", "round", "done")}
    st_["ctx"] = torch.full((B,), ctx0, dtype=torch.int32, device=DEV)
    st_["out"] = torch.full((B, max_out), -1, dtype=torch.int32, device=DEV)
    return st_


def reject(B, K, V, T, seed, seqs, zd, zt, ld, lt, d, s, max_out=64, max_ctx=1 << 30):
    ws = torch.empty(max(16, ora.rejection_workspace_bytes(B, V)), dtype=torch.uint8, device=DEV)
    ora.rejection_accept(B, K, V, T, seed, seqs, zd, zt, ld, lt, d, s["ctx"], s["anchor"], s["accept"], s["out"],
                         s["out_len"], s["round"], s["done"], max_out, max_ctx, ws)
    torch.cuda.synchronize()


def test_rejection_accept_qwen3_8b_shape():
    """Hidden 4096, 16 sequences x 32 slots, vocabulary 151936, T = 0.8; draft hidden states
    0.9 h + sqrt(0.19) N(0, 1) through the same LM head.  Drafts are the device's Gumbel-max samples
    (checked against the oracle's keys on a subset of rows), the verify call is an argmax call that
    keeps logits and logsumexp(z/T), and accept counts, committed tokens and KV lengths equal the
    oracle's rejection accept on the device's logits."""
    B, K, H, V, T, seed = 16, 32, 4096, 151936, 0.8, 99
    ht, w = synth.lmhead_inputs(4, B * K, H, V)
    hd = synth.draft_hidden(4, ht, mix=0.9)
    seqs = (np.arange(B, dtype=np.int32) * 7 + 3)
    rnds = np.arange(B, dtype=np.int32) % 3
    desc_d = ora.lmhead_desc(B * K, H, V, ora.BF16, K, ora.STREAM_DRAFT, T, seed)
    desc_t = ora.lmhead_desc(B * K, H, V, ora.BF16, K, ora.STREAM_AR, T, seed, sample=False)
    ws = torch.empty(ora.lmhead_workspace_bytes(desc_d), dtype=torch.uint8, device=DEV)
    zd = torch.empty((B * K, V), dtype=torch.float32, device=DEV)
    zt = torch.empty_like(zd)
    ld, lt = (torch.empty(B * K, dtype=torch.float32, device=DEV) for _ in range(2))
    d, t = (torch.empty(B * K, dtype=torch.int32, device=DEV) for _ in range(2))
    w_t = dev(w, ora.BF16)
    ora.lmhead_argmax(desc_d, dev(hd, ora.BF16), w_t, dev(seqs), dev(rnds), d, zd, ld, ws)
    ora.lmhead_argmax(desc_t, dev(ht, ora.BF16), w_t, dev(seqs), dev(rnds), t, zt, lt, ws)
    s = state(B)
    s["round"].copy_(dev(rnds))
    reject(B, K, V, T, seed, dev(seqs), zd, zt, ld, lt, d, s)
    dn = d.cpu().numpy().reshape(B, K)
    zdn = zd.cpu().numpy().astype(np.float64).reshape(B, K, V)
    ztn = zt.cpu().numpy().astype(np.float64).reshape(B, K, V)
    # logsumexp(z/T) of both calls against the device logits in float64
    for name, z, l in (("draft", zdn, ld), ("target", ztn, lt)):
        zz = z.reshape(B * K, V) / T
        ref = zz.max(1) + np.log(np.exp(zz - zz.max(1, keepdims=True)).sum(1))
        np.testing.assert_allclose(l.cpu().numpy(), ref, rtol=2e-6, err_msg=name)
    # the logits against the oracle's product (a subset of rows: 1.2 GB of weights per float64 chunk)
    rows = np.arange(0, B * K, 37)
    zref = hd[rows].astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(zdn.reshape(B * K, V)[rows] - zref).max() / np.abs(zref).max() <= 2e-3
    # drafts are Gumbel-max draws with the oracle's counters (within the eps_tie band of the keys)
    for i, r in enumerate(rows[:12]):
        b, slot = divmod(int(r), K)
        u = P.uniforms(seed, P.STREAM_DRAFT, slot, np.arange(V), rnds[b], seqs[b])
        key = zref[i] / T - np.log(-np.log(u))
        g, ref_id = int(dn[b, slot]), int(np.argmax(key))
        assert g == ref_id or key[ref_id] - key[g] <= 1e-4 * max(1.0, abs(key[ref_id])), (r, g, ref_id)
    acc = s["accept"].cpu().numpy()
    outn = s["out"].cpu().numpy()
    for b in range(B):
        ua = P.uniforms(seed, P.STREAM_ACCEPT, np.arange(K), 0, rnds[b], seqs[b])
        er = -np.log(P.uniforms(seed, P.STREAM_RESID, np.arange(V), 0, rnds[b], seqs[b]))
        k, em = Dc.rejection_accept(zdn[b], ztn[b], dn[b], T, ua, er)
        assert acc[b] == k, (b, acc[b], k)
        assert list(outn[b, :len(em)]) == em, b
    assert (s["ctx"].cpu().numpy() == 500 + np.minimum(acc + 1, K)).all()
    assert (s["round"].cpu().numpy() == rnds + 1).all()
    print("accepts", list(acc))


def test_rejection_kernel_output_law_tiny_vocab():
    """V = 8, 10^6 seeded sequences with one slot each, drafts drawn from q on the host: the
    device accepts with probability sum_x min(p, q) and commits tokens distributed as p
    (p = softmax(z_target/T), q = softmax(z_draft/T) from scipy)."""
    B, V, T, seed = 1_000_000, 8, 0.8, 2024
    zt1 = np.array([1.2, -0.3, 0.4, 2.0, -1.1, 0.1, 0.7, -0.6])
    zd1 = np.array([0.2, 0.9, 0.4, 1.1, -0.2, 0.8, -0.5, 0.3])
    p, q = sp.softmax(zt1 / T), sp.softmax(zd1 / T)
    g = np.random.default_rng(5)
    drafts = g.choice(V, size=B, p=q).astype(np.int32)
    zt = torch.from_numpy(np.tile(zt1.astype(np.float32), (B, 1))).to(DEV)
    zd = torch.from_numpy(np.tile(zd1.astype(np.float32), (B, 1))).to(DEV)
    lt = torch.full((B,), float(sp.logsumexp(zt1.astype(np.float32).astype(np.float64) / T)), device=DEV)
    ld = torch.full((B,), float(sp.logsumexp(zd1.astype(np.float32).astype(np.float64) / T)), device=DEV)
    s = state(B, ctx0=10, max_out=1)
    reject(B, 1, V, T, seed, dev(np.arange(B, dtype=np.int32)), zd, zt, ld, lt, dev(drafts), s, max_out=1)
    acc = s["accept"].cpu().numpy()
    out = s["out"].cpu().numpy()[:, 0]
    a = np.minimum(p, q).sum()
    assert abs(acc.mean() - a) < 4.5 * np.sqrt(a * (1 - a) / B)
    counts = np.bincount(out, minlength=V)
    chi2 = ((counts - B * p) ** 2 / (B * p)).sum()
    assert st.chi2.sf(chi2, V - 1) > 1e-4, (chi2, counts)
    assert np.array_equal(out[acc == 1], drafts[acc == 1])  # an accept commits the draft


@pytest.mark.parametrize("V", [50, 5000])
def test_rejection_rejects_out_of_range_draft_ids(V):
    """A draft id outside [0, V) is rejected at its slot without reading its logits; the slots before
    it (q = p, so always accepted) are committed and the correction is drawn from p at that slot
    (the residual has no mass).  V = 5000 spans three race chunks with a ragged last one."""
    B, K, T, seed = 3, 6, 0.8, 7
    rs = np.random.default_rng(3)
    z = rs.standard_normal((B, K, V)).astype(np.float32) * 2
    lse = sp.logsumexp(z.astype(np.float64) / T, axis=-1).astype(np.float32)
    d = rs.integers(0, V, (B, K)).astype(np.int32)
    bad_slot = [2, 0, 5]
    d[0, 2], d[1, 0], d[2, 5] = -1, V, 1 << 30
    zt = dev(z.reshape(B * K, V))
    lt = dev(lse.reshape(B * K))
    s = state(B)
    reject(B, K, V, T, seed, dev(np.arange(B, dtype=np.int32)), zt, zt, lt, lt, dev(d), s)
    acc = s["accept"].cpu().numpy()
    outn = s["out"].cpu().numpy()
    assert list(acc) == bad_slot
    for b in range(B):
        j = bad_slot[b]
        er = -np.log(P.uniforms(seed, P.STREAM_RESID, np.arange(V), 0, 0, b))
        corr = Dc.race(sp.softmax(z[b, j].astype(np.float64) / T), er)  # residual p - q = 0: drawn from p
        assert list(outn[b, :j + 1]) == list(d[b, :j]) + [corr]


# ------------------------------------------------------------------- the round's output law

MICRO = synth.ModelShape(layers=1, hidden=64, q_heads=2, kv_heads=1, head_dim=64, inter=128, vocab=8)


def _chi2_pvalue(counts, probs, min_expected=5.0):
    """Pearson chi-square p-value; cells expected below ``min_expected`` are pooled into one."""
    counts = np.asarray(counts, dtype=np.float64).ravel()
    probs = np.asarray(probs, dtype=np.float64).ravel()
    exp = counts.sum() * probs
    big = exp >= min_expected
    c = np.append(counts[big], counts[~big].sum())
    e = np.append(exp[big], exp[~big].sum())
    if e[-1] == 0:
        assert c[-1] == 0, "samples fell on cells of probability 0"
        c, e = c[:-1], e[:-1]
    return st.chi2.sf(((c - e) ** 2 / e).sum(), len(c) - 1)


def test_sampled_round_follows_the_ar_law():
    """Orthrus paper summary, sec. 四 and Q&A: with a temperature the committed tokens follow AR
    sampling's distribution.  One batch of 6000 sequences with the same prompt (each its own
    Philox stream through its sequence id) through a one-layer decoder on an 8-token vocabulary,
    block 4, T = 0.8: the first two committed tokens of the device's Orthrus rounds and of its AR
    steps both follow p(t1) p(t2 | t1) of the AR model (oracle passes, float64), and slot 0 is
    accepted with probability sum_x min(p, q)."""
    W = synth.model_weights(MICRO, cfg=21, w_std=0.2, diff_std=0.08)
    W["lm_head"] = W["lm_head"] * np.float32(0.5)
    Wt = M.Weights(W, MICRO)
    T, N = 0.8, 6000
    prompt = np.array([1, 5, 2, 0, 3], np.int32)
    cache, anchor = Dc.prefill(Wt, prompt, 16)
    p1 = sp.softmax(Dc.ar_pass(Wt, cache, [anchor])[0] / T)
    q1 = sp.softmax(Dc.draft_pass(Wt, cache, [anchor] + [MICRO.mask_id] * 3)[0] / T)
    joint = np.stack([p1[t] * sp.softmax(Dc.ar_pass(Wt, cache, [anchor, t])[1] / T) for t in range(8)])
    from orthrus_round_amd.decoder import Decoder
    dec = Decoder(W, MICRO, precision="fp32", block=4, max_batch=N, max_ctx=32)
    prompts = np.tile(prompt, (N, 1))
    toks, stt = dec.generate(prompts, 2, temperature=T, seed=123, poll_every=1, record_accepts=True)
    orth = np.zeros((8, 8))
    np.add.at(orth, (toks[:, 0], toks[:, 1]), 1)
    acc0 = float((stt.accept_hist[0] >= 1).mean())
    a = float(np.minimum(p1, q1).sum())
    assert abs(acc0 - a) < 4.5 * np.sqrt(a * (1 - a) / N), (acc0, a)
    assert _chi2_pvalue(orth.sum(1), p1) > 1e-4
    assert _chi2_pvalue(orth, joint) > 1e-4
    ar_toks, _ = dec.generate_ar(prompts, 2, temperature=T, seed=123)
    ar = np.zeros((8, 8))
    np.add.at(ar, (ar_toks[:, 0], ar_toks[:, 1]), 1)
    assert _chi2_pvalue(ar, joint) > 1e-4
    print(f"slot-0 accept {acc0:.3f} (law {a:.3f}); chi2 p orthrus {_chi2_pvalue(orth, joint):.3f}, "
          f"ar {_chi2_pvalue(ar, joint):.3f}")
