"""Pins for the oracle's temperature > 0 path: softmax with a temperature, Gumbel-max
sampling, the strict rejection accept, and the sampled round end to end.

Orthrus paper summary, sec. 四 and the Q&A: with a temperature the round uses strict rejection
sampling, so the committed tokens are distributed exactly as AR sampling's.  Every expected
distribution below is computed independently of the oracle's own softmax (scipy / torch in
float64 on logits the oracle's pinned passes produce), so a temperature dropped from the
oracle, a flipped Gumbel key or a wrong accept rule fails here.
"""
import numpy as np
import pytest
import scipy.special as sp
import scipy.stats as st
import torch

import synth
from oracle import decode as Dc
from oracle import model as M
from oracle import philox as P


def _chi2_pvalue(counts, probs, min_expected=5.0):
    """Pearson chi-square p-value of ``counts`` against ``probs``; cells whose expected count is
    below ``min_expected`` are pooled into one."""
    counts = np.asarray(counts, dtype=np.float64).ravel()
    probs = np.asarray(probs, dtype=np.float64).ravel()
    n = counts.sum()
    exp = n * probs
    big = exp >= min_expected
    c = np.append(counts[big], counts[~big].sum())
    e = np.append(exp[big], exp[~big].sum())
    if e[-1] == 0:
        assert c[-1] == 0, "samples fell on cells of probability 0"
        c, e = c[:-1], e[:-1]
    chi2 = ((c - e) ** 2 / e).sum()
    return st.chi2.sf(chi2, len(c) - 1)


# --------------------------------------------------------------------------- softmax(z / T)

@pytest.mark.parametrize("T", [0.25, 0.8, 1.0, 3.0])
def test_softmax_t_matches_independent_softmax(T):
    rs = np.random.default_rng(40)
    z = rs.standard_normal((5, 37)) * 4.0
    z[1] += 700.0  # a naive exp would overflow: the max must be subtracted
    ref_scipy = sp.softmax(z / T, axis=-1)
    ref_torch = torch.softmax(torch.from_numpy(z) / T, dim=-1).numpy()
    got = Dc.softmax_t(z, T)
    np.testing.assert_allclose(got, ref_scipy, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(got, ref_torch, rtol=1e-12, atol=1e-300)
    # closed form on two logits: p = (1, e^{d/T}) / (1 + e^{d/T})
    d = 0.9
    two = Dc.softmax_t(np.array([0.0, d]), T)
    assert two[1] == pytest.approx(1.0 / (1.0 + np.exp(-d / T)), rel=1e-14)


def test_softmax_t_float32_mode_stays_float32():
    z = np.random.default_rng(41).standard_normal(64).astype(np.float32) * 3
    got = Dc.softmax_t(z, 0.8)
    assert got.dtype == np.float32
    np.testing.assert_allclose(got, sp.softmax(z.astype(np.float64) / 0.8), rtol=2e-6, atol=1e-9)


# --------------------------------------------------------------------------- Gumbel-max draws

def _philox_rows(n, V, seed=5, stream=P.STREAM_DRAFT):
    """n independent rows of V uniforms from the oracle's generator (round = row index)."""
    return P.uniforms(seed, stream, 0, np.arange(V)[None, :], np.arange(n)[:, None], 0)


@pytest.mark.parametrize("T", [0.5, 0.8, 2.0])
def test_gumbel_sample_follows_softmax_over_t(T):
    V, N = 8, 20000
    z = np.array([1.3, -0.4, 0.2, 2.1, -1.5, 0.0, 0.9, -0.7])
    u = _philox_rows(N, V, seed=int(T * 10))
    draws = np.array([Dc.gumbel_sample(z, T, u[i]) for i in range(N)])
    counts = np.bincount(draws, minlength=V)
    assert _chi2_pvalue(counts, sp.softmax(z / T)) > 1e-4
    # the same draws are far from the distribution at another temperature and from the
    # distribution a sign-flipped Gumbel key would give (which favours low logits)
    assert _chi2_pvalue(counts, sp.softmax(z / (1.5 * T))) < 1e-6
    assert _chi2_pvalue(counts, sp.softmax(-z / T)) < 1e-12


def test_gumbel_sample_float32_mode():
    V, N = 8, 12000
    z = np.array([0.3, -1.0, 1.1, 0.2, 0.0, -0.5, 0.8, 1.6], np.float32)
    u = _philox_rows(N, V, seed=77)
    counts = np.bincount([Dc.gumbel_sample(z, 0.8, u[i]) for i in range(N)], minlength=V)
    assert _chi2_pvalue(counts, sp.softmax(z.astype(np.float64) / 0.8)) > 1e-4


def test_low_temperature_sampling_is_greedy():
    """T -> 0: softmax(z/T) tends to the one-hot of the argmax, and so must every draw.  The
    Gumbel key -ln(-ln u) lies in [-2.8, 16.6] for the generator's u in [2^-24, 1 - 2^-24], so a
    logit gap above 19.4 * T can never be overturned."""
    rs = np.random.default_rng(42)
    T = 1e-4
    u = _philox_rows(200, 50, seed=9)
    for i in range(200):
        z = rs.permutation(50) * 0.01 + rs.standard_normal() * 10  # distinct, gaps >= 0.01
        assert Dc.gumbel_sample(z, T, u[i]) == int(np.argmax(z))


def test_low_temperature_rejection_is_greedy_consensus():
    """At T -> 0 the draft view proposes its own argmax; such a draft is accepted when it equals
    the target's argmax and rejected otherwise, with the target's argmax as the correction: the
    greedy consensus rule."""
    rs = np.random.default_rng(43)
    K, V = 8, 30
    for trial in range(40):
        zt = rs.permutation(V * K).reshape(K, V) * 0.01
        zd = rs.permutation(V * K).reshape(K, V) * 0.01
        t = np.argmax(zt, axis=1)
        j = trial % (K + 1)
        d = t.copy()
        if j < K:
            d[j] = (t[j] + 1 + rs.integers(0, V - 1)) % V
            d[j + 1:] = rs.integers(0, V, K - j - 1)
        zd[np.arange(K), d] = zd.max(axis=1) + 0.05  # d is the draft view's argmax
        ua = rs.random(K) * (1 - 2 ** -24) + 2 ** -25
        k, em = Dc.rejection_accept(zd, zt, d, 1e-4, ua, rs.exponential(size=V))
        kg, emg = Dc.consensus(d, t)
        assert (k, em) == (kg, emg)


# --------------------------------------------------------------------------- rejection accept

def test_rejection_accept_probability_and_output_law():
    """One slot, many seeded trials: the slot is accepted with probability sum_x min(p, q) and the
    committed token is distributed as p (p, q computed with scipy from the logits)."""
    rs = np.random.default_rng(44)
    V, T, N = 6, 0.8, 30000
    zt, zd = rs.standard_normal((2, 1, V)) * 1.5
    p = sp.softmax(zt[0] / T)
    q = sp.softmax(zd[0] / T)
    g = np.random.default_rng(45)
    counts = np.zeros(V)
    acc = 0
    for _ in range(N):
        d = g.choice(V, p=q)
        k, em = Dc.rejection_accept(zd, zt, [d], T, g.random(1), g.exponential(size=V))
        acc += k
        counts[em[-1]] += 1
    a = np.minimum(p, q).sum()
    assert abs(acc / N - a) < 4.5 * np.sqrt(a * (1 - a) / N)
    assert _chi2_pvalue(counts, p) > 1e-4
    assert _chi2_pvalue(counts, q) < 1e-12


# --------------------------------------------------------------------------- the sampled round

MICRO = synth.ModelShape(layers=1, hidden=32, q_heads=2, kv_heads=1, head_dim=16, inter=64, vocab=8)


@pytest.fixture(scope="module")
def micro():
    """A one-layer decoder on an 8-token vocabulary whose logits spread over about 3 units, and a
    diffusion view distinct enough that slot 0 is accepted only about 70% of the time."""
    W = synth.model_weights(MICRO, cfg=21, w_std=0.2, diff_std=0.08)
    W["lm_head"] = W["lm_head"] * np.float32(0.7)
    return M.Weights(W, MICRO)


def _exact_two_token_law(Wt, prompt, T):
    """P(t1, t2) = p(t1 | prompt) p(t2 | prompt, t1), from the oracle's AR passes (pinned to the
    transformers Llama decoder) and scipy's softmax."""
    cache, anchor = Dc.prefill(Wt, prompt, len(prompt) + 4)
    p1 = sp.softmax(Dc.ar_pass(Wt, cache, [anchor])[0] / T)
    V = Wt.shape.vocab
    joint = np.zeros((V, V))
    for t1 in range(V):
        z2 = Dc.ar_pass(Wt, cache, [anchor, t1])[1]
        joint[t1] = p1[t1] * sp.softmax(z2 / T)
    return p1, joint


def test_sampled_orthrus_and_sampled_ar_follow_the_ar_law(micro):
    """Orthrus paper summary, sec. 四 and Q&A: with a temperature the committed tokens follow AR
    sampling's distribution.  Over seeded runs, the first two tokens of the sampled Orthrus
    round and of sampled AR decoding both follow p(t1) p(t2 | t1) of the AR model, and the
    first slot is accepted with probability sum_x min(p, q)."""
    Wt = micro
    T = 0.8
    prompt = np.array([1, 5, 2, 0, 3], np.int32)
    p1, joint = _exact_two_token_law(Wt, prompt, T)
    cache, anchor = Dc.prefill(Wt, prompt, 16)
    q1 = sp.softmax(Dc.draft_pass(Wt, cache, [anchor] + [MICRO.mask_id] * 3)[0] / T)
    N = 1500
    V = MICRO.vocab
    orth = np.zeros((V, V))
    ar = np.zeros((V, V))
    accepted = 0
    for s in range(N):
        res = Dc.generate(Wt, prompt, 2, block=4, temperature=T, seed=s)
        orth[res.tokens[0], res.tokens[1]] += 1
        accepted += res.rounds[0].accept >= 1
        a = Dc.generate_ar(Wt, prompt, 2, temperature=T, seed=s)
        ar[a[0], a[1]] += 1
    assert _chi2_pvalue(orth.sum(1), p1) > 1e-4
    assert _chi2_pvalue(ar.sum(1), p1) > 1e-4
    assert _chi2_pvalue(orth, joint) > 1e-4
    assert _chi2_pvalue(ar, joint) > 1e-4
    a = np.minimum(p1, q1).sum()
    assert abs(accepted / N - a) < 4.5 * np.sqrt(a * (1 - a) / N)
    # power: the draws are far from the draft view's law and, pooled, from the law at T = 1
    assert _chi2_pvalue(orth.sum(1), q1) < 1e-12
    assert _chi2_pvalue(orth + ar, _exact_two_token_law(Wt, prompt, 1.0)[1]) < 1e-6
