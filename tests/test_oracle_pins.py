"""Pins for the CPU oracle: each check ties it to something other than itself.

Library routines (numpy's Philox, torch's SDPA / rms_norm, transformers' Llama decoder),
closed forms and invariants.  All run on the CPU in seconds.
"""
import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import model as M
from oracle import philox as P
from oracle import decode as Dc


# --------------------------------------------------------------------------- Philox

def test_philox_matches_numpy_bitgenerator():
    rs = np.random.default_rng(7)
    for _ in range(20):
        key = rs.integers(0, 2**63, size=2, dtype=np.uint64)
        ctr = rs.integers(0, 2**63, size=4, dtype=np.uint64)
        bg = np.random.Philox(key=key, counter=ctr)
        ref = bg.random_raw(12)
        # numpy advances the 256-bit counter by one before each block of four words
        ctrs = []
        c = [int(x) for x in ctr]
        for _ in range(3):
            v = (c[0] | (c[1] << 64) | (c[2] << 128) | (c[3] << 192)) + 1
            c = [(v >> (64 * i)) & (2**64 - 1) for i in range(4)]
            ctrs.append(c)
        mine = P.philox4x64(np.array(ctrs, dtype=np.uint64), key).ravel()
        assert np.array_equal(ref, mine)


def test_uniform_exact_in_fp32_and_open_interval():
    w = np.array([0, 2**64 - 1, 2**41 - 1, 2**41, 12345678901234567890], dtype=np.uint64)
    u = P.words_to_uniform(w)
    assert np.all(u > 0) and np.all(u < 1)
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)
    assert u[0] == 2.0 ** -24 and u[1] == 1 - 2.0 ** -24


def test_uniforms_counter_layout_words():
    # index 4j+w must be word w of the block at counter (j, c1, c2, c3)
    u = P.uniforms(11, P.STREAM_RESID, np.arange(8), 0, 5, 3)
    words = P.philox4x64(np.array([[0, 0, 5, 3], [1, 0, 5, 3]], dtype=np.uint64), np.array([11, P.STREAM_RESID], dtype=np.uint64))
    assert np.array_equal(u, P.words_to_uniform(words.ravel()))


# --------------------------------------------------------------------------- norms, RoPE

def test_rmsnorm_matches_torch():
    x = np.random.default_rng(1).standard_normal((5, 64))
    g = np.random.default_rng(2).standard_normal(64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(M.rmsnorm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-13)


def test_rope_is_complex_rotation_and_preserves_norm():
    rs = np.random.default_rng(3)
    D = 16
    x = rs.standard_normal((3, 2, D))
    pos = np.array([0, 7, 1000])
    y = M.rope(x, pos[:, None], 1e6)
    # complex form: z_i = x_i + j x_{i+D/2} multiplied by e^{j * pos * base^(-2i/D)}
    z = x[..., : D // 2] + 1j * x[..., D // 2:]
    theta = pos[:, None, None] * (1e6 ** (-np.arange(D // 2) * 2.0 / D))
    zr = z * np.exp(1j * theta)
    np.testing.assert_allclose(y, np.concatenate([zr.real, zr.imag], -1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    assert np.array_equal(M.rope(x, np.zeros((3, 1)), 1e6), x)


def test_rope_relative_position():
    rs = np.random.default_rng(4)
    q, k = rs.standard_normal((2, 1, 1, 64))
    def dot(m, n):
        return float((M.rope(q, np.array([[m]]), 1e6) * M.rope(k, np.array([[n]]), 1e6)).sum())
    assert dot(10, 3) == pytest.approx(dot(107, 100), rel=1e-10)
    assert dot(500, 499) == pytest.approx(dot(1, 0), rel=1e-10)


# --------------------------------------------------------------------------- attention

def _sdpa(q, k, v, mask, scale):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=t(mask), scale=scale).numpy()


@pytest.mark.parametrize("n", [0, 1, 37])
def test_draft_attention_matches_sdpa(n):
    rs = np.random.default_rng(10 + n)
    K, Hq, Hkv, D = 8, 4, 2, 16
    q = rs.standard_normal((K, Hq, D))
    kc, vc = rs.standard_normal((2, n, Hkv, D))
    kb, vb = rs.standard_normal((2, K, Hkv, D))
    out = M.draft_attention(q, kc, vc, kb, vb, 0.3)
    kk, vv = np.concatenate([kc, kb]), np.concatenate([vc, vb])
    G = Hq // Hkv
    for h in range(Hq):
        mask = np.ones((K, n + K), bool)
        ref = _sdpa(q[:, h], kk[:, h // G], vv[:, h // G], mask, 0.3)
        np.testing.assert_allclose(out[:, h], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n", [0, 5, 64])
def test_verify_attention_matches_sdpa_causal(n):
    rs = np.random.default_rng(20 + n)
    K, Hq, Hkv, D = 8, 4, 1, 16
    q = rs.standard_normal((K, Hq, D))
    kk, vv = rs.standard_normal((2, n + K, Hkv, D))
    out = M.verify_attention(q, kk, vv, n, 0.25)
    # causal with offset n, built as a lower-triangular mask shifted by n
    mask = torch.ones(K, n + K, dtype=torch.bool).tril(diagonal=n).numpy()
    for h in range(Hq):
        ref = _sdpa(q[:, h], kk[:, 0], vv[:, 0], mask, 0.25)
        np.testing.assert_allclose(out[:, h], ref, rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rs = np.random.default_rng(5)
    q = rs.standard_normal((4, 2, 8))
    k1, v1 = rs.standard_normal((2, 1, 1, 8))
    # one visible key -> output is that key's value
    out = M.verify_attention(q[:1], k1, v1, 0, 1.0)
    np.testing.assert_allclose(out[0, 0], v1[0, 0], rtol=0, atol=1e-15)
    # GQA: kv head h // G; distinct constant values per kv head are reproduced exactly
    Hq, Hkv = 4, 2
    kc = rs.standard_normal((3, Hkv, 8))
    vc = np.stack([np.full((3, 8), 1.0), np.full((3, 8), 2.0)], axis=1)
    kb = rs.standard_normal((4, Hkv, 8))
    vb = np.stack([np.full((4, 8), 1.0), np.full((4, 8), 2.0)], axis=1)
    out = M.draft_attention(rs.standard_normal((4, Hq, 8)), kc, vc, kb, vb, 1.0)
    np.testing.assert_allclose(out[:, [0, 1]], 1.0, atol=1e-14)
    np.testing.assert_allclose(out[:, [2, 3]], 2.0, atol=1e-14)


def test_masked_attention_matches_sdpa_random_mask():
    rs = np.random.default_rng(6)
    q = rs.standard_normal((9, 16))
    k, v = rs.standard_normal((2, 23, 16))
    mask = rs.random((9, 23)) < 0.5
    mask[:, 0] = True
    np.testing.assert_allclose(M.masked_attention(q, k, v, mask, 0.2), _sdpa(q, k, v, mask, 0.2), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n", [0, 40])
def test_grouped_attention_matches_sdpa_and_row_form(n):
    """The matrix-product form gives the draft and verify attention of the row-by-row oracle and
    of torch's SDPA with the explicit masks, with G = 4 query heads per kv head."""
    rs = np.random.default_rng(30 + n)
    K, Hq, Hkv, D = 8, 8, 2, 16
    q = rs.standard_normal((K, Hq, D))
    k, v = rs.standard_normal((2, n + K, Hkv, D))
    kb, vb = rs.standard_normal((2, K, Hkv, D))
    draft = M.grouped_attention(q, np.concatenate([k[:n], kb]), np.concatenate([v[:n], vb]),
                                np.ones((K, n + K), bool), 0.3)
    np.testing.assert_allclose(draft, M.draft_attention(q, k[:n], v[:n], kb, vb, 0.3), rtol=1e-12, atol=1e-12)
    causal = np.ones((K, n + K), bool)
    causal[:, n:] = np.tril(np.ones((K, K), bool))
    ver = M.grouped_attention(q, k, v, causal, 0.3)
    np.testing.assert_allclose(ver, M.verify_attention(q, k, v, n, 0.3), rtol=1e-12, atol=1e-12)
    for h in range(Hq):
        np.testing.assert_allclose(ver[:, h], _sdpa(q[:, h], k[:, h // 4], v[:, h // 4], causal, 0.3),
                                   rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- decoder vs transformers Llama

def _llama(W, shape):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = LlamaConfig(vocab_size=shape.vocab, hidden_size=shape.hidden, intermediate_size=shape.inter,
                      num_hidden_layers=shape.layers, num_attention_heads=shape.q_heads,
                      num_key_value_heads=shape.kv_heads, head_dim=shape.head_dim, rms_norm_eps=shape.eps,
                      rope_theta=shape.rope_base, attention_bias=False, mlp_bias=False,
                      tie_word_embeddings=False, max_position_embeddings=8192)
    cfg._attn_implementation = "eager"
    m = LlamaForCausalLM(cfg).to(torch.float64).eval()
    sd = {"model.embed_tokens.weight": W["embed"], "lm_head.weight": W["lm_head"], "model.norm.weight": W["final_norm"]}
    for l in range(shape.layers):
        p = f"model.layers.{l}."
        sd[p + "self_attn.q_proj.weight"] = W[f"{l}.wq"]
        sd[p + "self_attn.k_proj.weight"] = W[f"{l}.wk"]
        sd[p + "self_attn.v_proj.weight"] = W[f"{l}.wv"]
        sd[p + "self_attn.o_proj.weight"] = W[f"{l}.wo"]
        sd[p + "mlp.gate_proj.weight"] = W[f"{l}.w_gate"]
        sd[p + "mlp.up_proj.weight"] = W[f"{l}.w_up"]
        sd[p + "mlp.down_proj.weight"] = W[f"{l}.w_down"]
        sd[p + "input_layernorm.weight"] = W[f"{l}.attn_norm"]
        sd[p + "post_attention_layernorm.weight"] = W[f"{l}.mlp_norm"]
    m.load_state_dict({k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in sd.items()}, strict=True)
    return m


@pytest.fixture(scope="module")
def tiny():
    shape = synth.TINY
    W = synth.model_weights(shape, cfg=1)
    return shape, W, M.Weights(W, shape)


def test_ar_prefill_matches_transformers_llama(tiny):
    shape, W, Wt = tiny
    ids = synth.prompt_ids(shape, 1, 1, 40)[0]
    cache = Dc.Cache(shape, 64, np.float64)
    z = Dc.ar_pass(Wt, cache, ids)
    with torch.no_grad():
        ref = _llama(W, shape)(torch.from_numpy(ids.astype(np.int64))[None]).logits[0].numpy()
    # transformers takes RoPE angles in float32, hence the 1e-5 band
    np.testing.assert_allclose(z, ref, rtol=0, atol=2e-5 * np.abs(ref).max())
    assert np.array_equal(M.argmax_lowest(z), np.argmax(ref, -1))


def test_chunked_ar_passes_equal_one_pass(tiny):
    shape, W, Wt = tiny
    ids = synth.prompt_ids(shape, 1, 1, 45)[0]
    c1 = Dc.Cache(shape, 64, np.float64)
    z1 = Dc.ar_pass(Wt, c1, ids)
    c2 = Dc.Cache(shape, 64, np.float64)
    za = Dc.ar_pass(Wt, c2, ids[:32])
    c2.n = 32
    zb = Dc.ar_pass(Wt, c2, ids[32:])
    np.testing.assert_array_equal(np.concatenate([za, zb]), z1)
    for l in range(shape.layers):
        np.testing.assert_array_equal(c1.k[l][:45], c2.k[l][:45])


def test_draft_pass_equals_llama_with_block_mask_when_views_share_weights(tiny):
    """With W_diff = W_AR the draft pass is a Llama forward whose block rows see everything
    before the block plus the whole block (bidirectional), and whose context rows are causal."""
    shape, W, _ = tiny
    W2 = dict(W)
    for l in range(shape.layers):
        for ar, df in zip(synth.LAYER_AR, synth.LAYER_DIFF):
            W2[f"{l}.{df}"] = W[f"{l}.{ar}"]
    Wt = M.Weights(W2, shape)
    ids = synth.prompt_ids(shape, 1, 1, 20)[0]
    n, K = 12, 8
    blk = np.concatenate([ids[n:n + 1], np.full(K - 1, shape.mask_id)])
    cache = Dc.Cache(shape, 64, np.float64)
    Dc.ar_pass(Wt, cache, ids[:n])
    cache.n = n
    z = Dc.draft_pass(Wt, cache, blk)
    seq = np.concatenate([ids[:n], blk]).astype(np.int64)
    T = n + K
    allow = np.tril(np.ones((T, T), bool))
    allow[n:, n:] = True
    mask = torch.where(torch.from_numpy(allow), 0.0, -torch.inf).to(torch.float64)[None, None]
    with torch.no_grad():
        ref = _llama(W2, shape)(torch.from_numpy(seq)[None], attention_mask=mask).logits[0, n:].numpy()
    np.testing.assert_allclose(z, ref, rtol=0, atol=2e-5 * np.abs(ref).max())


def test_draft_view_uses_its_own_attention_weights(tiny):
    shape, W, Wt = tiny
    ids = synth.prompt_ids(shape, 1, 1, 10)[0]
    cache = Dc.Cache(shape, 64, np.float64)
    Dc.ar_pass(Wt, cache, ids[:9])
    cache.n = 9
    k_before = [a.copy() for a in cache.k]
    z1 = Dc.draft_pass(Wt, cache, [ids[9]] + [shape.mask_id] * 3)
    for l in range(shape.layers):  # the draft pass never touches the shared cache
        np.testing.assert_array_equal(cache.k[l], k_before[l])
    W2 = dict(W)
    W2["0.dq"] = W["0.dq"] * 1.5
    z2 = Dc.draft_pass(M.Weights(W2, shape), cache, [ids[9]] + [shape.mask_id] * 3)
    assert np.abs(z1 - z2).max() > 1e-3


# --------------------------------------------------------------------------- LM head argmax

def test_argmax_ties_go_to_lowest_id():
    rs = np.random.default_rng(8)
    w = rs.standard_normal((50, 16))
    w[31] = w[7]
    w[44] = w[7]
    h = w[7] * 3.0  # row 7 (and its copies) wins
    z = w @ h
    assert M.argmax_lowest(z[None])[0] == 7


# --------------------------------------------------------------------------- consensus

@pytest.mark.parametrize("K", [1, 4, 32])
def test_consensus_exhaustive_first_mismatch(K):
    rs = np.random.default_rng(K)
    t = rs.integers(0, 100, size=K)
    for j in range(K + 1):
        d = t.copy()
        if j < K:
            d[j] = (t[j] + 1 + rs.integers(0, 50)) % 100
            d[j + 1:] = rs.integers(0, 100, size=K - j - 1)
        k, em = Dc.consensus(d, t)
        assert k == j
        assert em == list(t[: min(j + 1, K)])
        assert 1 <= len(em) == min(k + 1, K)


def test_geometric_drafts_give_closed_form_accepts():
    rs = np.random.default_rng(9)
    t = rs.integers(0, 1000, size=(64, 32)).astype(np.int32)
    d, L = synth.geometric_drafts(4, t, 1000)
    for b in range(64):
        k, em = Dc.consensus(d[b], t[b])
        assert k == L[b] and len(em) == min(L[b] + 1, 32)
    assert 3.0 < L.mean() < 7.0


# --------------------------------------------------------------------------- rejection sampling

def _acc_prob(p, q, d):
    return min(1.0, p[d] / q[d])


def test_rejection_single_slot_distribution_closed_form():
    """P(out=x) = q(x) min(1, p/q) + (1 - sum_y min(q,p)) * r(x) / |r| equals p(x)."""
    rs = np.random.default_rng(10)
    V = 6
    zt, zd = rs.standard_normal((2, 1, V)) * 2
    T = 0.8
    # p and q from scipy, independently of the oracle's own softmax
    p = scipy.special.softmax(zt[0] / T)
    q = scipy.special.softmax(zd[0] / T)
    # exact acceptance probability of the rule u * q(d) < p(d) for u ~ U(0,1)
    for d in range(V):
        assert _acc_prob(p, q, d) == pytest.approx(min(1.0, p[d] / q[d]))
    r = np.maximum(p - q, 0)
    out = q * np.minimum(1, p / q) + (1 - np.minimum(q, p).sum()) * r / r.sum()
    np.testing.assert_allclose(out, p, rtol=1e-12)
    # Monte Carlo through the oracle's rule with seeded uniforms / exponentials
    N = 30000
    counts = np.zeros(V)
    g = np.random.default_rng(11)
    for _ in range(N):
        d = g.choice(V, p=q)
        k, em = Dc.rejection_accept(zd, zt, [d], T, g.random(1), g.exponential(size=V))
        counts[em[-1]] += 1
    chi2 = ((counts - N * p) ** 2 / (N * p)).sum()
    assert chi2 < 25.0  # 5 dof, p ~ 1e-4


def test_rejection_special_cases():
    rs = np.random.default_rng(12)
    V, K = 5, 4
    z = rs.standard_normal((K, V))
    d = [1, 2, 3, 4]
    k, em = Dc.rejection_accept(z, z, d, 0.8, np.full(K, 1 - 2**-24), np.ones(V))
    assert k == K and em == d  # q == p: always accept
    zd = np.full((K, V), -1e9); zd[:, 0] = 0.0
    zt = np.full((K, V), -1e9); zt[:, 1:] = 0.0
    k, em = Dc.rejection_accept(zd, zt, [0] * K, 0.8, np.full(K, 2**-24), rs.exponential(size=V))
    assert k == 0 and em[0] != 0  # disjoint supports: reject, residual = p


def test_race_distribution():
    g = np.random.default_rng(13)
    w = np.array([0.5, 0.0, 0.2, 0.3])
    N = 40000
    wins = np.bincount([Dc.race(w, g.exponential(size=4)) for _ in range(N)], minlength=4)
    assert wins[1] == 0
    exp = N * w / w.sum()
    chi2 = sum((wins[i] - exp[i]) ** 2 / exp[i] for i in (0, 2, 3))
    assert chi2 < 20.0


# --------------------------------------------------------------------------- the round (losslessness)

@pytest.fixture(scope="module")
def tiny_prompt():
    return synth.prompt_ids(synth.TINY, 1, 1, 64)[0]


def test_greedy_orthrus_equals_greedy_ar_fp64(tiny, tiny_prompt):
    shape, W, Wt = tiny
    res = Dc.generate(Wt, tiny_prompt, 48)
    ar = Dc.generate_ar(Wt, tiny_prompt, 48)
    assert res.tokens == ar
    assert all(1 <= len(r.emitted) == min(r.accept + 1, 32) for r in res.rounds)
    assert all(r.n_before == res.rounds[0].n_before + sum(len(x.emitted) for x in res.rounds[:i])
               for i, r in enumerate(res.rounds))
    assert 0.5 <= res.tpf <= 16


def test_greedy_orthrus_equals_greedy_ar_fp32(tiny, tiny_prompt):
    shape, W, _ = tiny
    Wt = M.Weights(W, shape, np.float32)
    assert Dc.generate(Wt, tiny_prompt, 40).tokens == Dc.generate_ar(Wt, tiny_prompt, 40)


def test_forced_full_and_zero_acceptance(tiny, tiny_prompt):
    shape, W, Wt = tiny
    ar = Dc.generate_ar(Wt, tiny_prompt, 96)
    P0 = len(tiny_prompt) - 1
    full = Dc.generate(Wt, tiny_prompt, 96, inject=lambda r, n, a: ar[n - P0: n - P0 + 32])
    assert full.tokens == ar and all(r.accept == 32 for r in full.rounds) and len(full.rounds) == 3
    wrong = Dc.generate(Wt, tiny_prompt, 6,
                        inject=lambda r, n, a: [(t + 1) % (shape.vocab - 1) for t in ar[n - P0: n - P0 + 32]])
    assert wrong.tokens == ar[:6] and all(r.accept == 0 and len(r.emitted) == 1 for r in wrong.rounds)


def test_block_of_one_is_an_ar_step(tiny, tiny_prompt):
    shape, W, Wt = tiny
    res = Dc.generate(Wt, tiny_prompt, 5, block=1)
    assert res.tokens == Dc.generate_ar(Wt, tiny_prompt, 5)
    assert all(len(r.emitted) == 1 for r in res.rounds)


def test_poisoned_dead_slots_do_not_change_trajectory(tiny, tiny_prompt):
    shape, W, Wt = tiny
    a = Dc.generate(Wt, tiny_prompt, 24)
    b = Dc.generate(Wt, tiny_prompt, 24, poison_dead=True)
    assert a.tokens == b.tokens and [r.accept for r in a.rounds] == [r.accept for r in b.rounds]


@pytest.mark.slow
def test_tiny_config_full_256_tokens(tiny, tiny_prompt):
    shape, W, Wt = tiny
    res = Dc.generate(Wt, tiny_prompt, 256)
    assert res.tokens == Dc.generate_ar(Wt, tiny_prompt, 256)
    assert min(len(r.emitted) for r in res.rounds) >= 1


# --------------------------------------------------------------------------- two-step drafting

def test_log_confidence_closed_form_and_normalisation():
    # softmax([0, ln 3]) = (1/4, 3/4)
    z = np.array([[0.0, np.log(3.0)], [5.0, 5.0 + np.log(3.0)]])
    assert np.allclose(Dc.log_confidence(z, [1, 0]), [np.log(0.75), np.log(0.25)], rtol=0, atol=1e-15)
    rs = np.random.default_rng(0)
    z = rs.standard_normal((4, 50)) * 3.0 + 700.0  # large offset: a naive exp would overflow
    for x in range(50):
        assert np.isfinite(Dc.log_confidence(z, [x] * 4)).all()
    total = sum(np.exp(Dc.log_confidence(z, [x] * 4)) for x in range(50))
    assert np.allclose(total, 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_most_confident_is_the_unique_ordered_subset(seed):
    import itertools
    rs = np.random.default_rng(seed)
    c = rs.integers(0, 4, 7).astype(np.float64)  # many ties
    if seed % 2:
        c[rs.integers(0, 7)] = np.nan
    key = np.where(np.isnan(c), -np.inf, c)
    for n_fill in range(8):
        ok = []
        for S in itertools.combinations(range(7), n_fill):
            rest = [j for j in range(7) if j not in S]
            if all(key[i] > key[j] or (key[i] == key[j] and i < j) for i in S for j in rest):
                ok.append(set(S))
        assert len(ok) == 1
        assert set(np.flatnonzero(Dc.most_confident(c, n_fill))) == ok[0]


@pytest.fixture(scope="module")
def tiny_cache(tiny, tiny_prompt):
    shape, W, Wt = tiny
    cache, anchor = Dc.prefill(Wt, tiny_prompt, 160)
    return cache, anchor


def test_two_step_with_no_fill_is_the_one_step_draft(tiny, tiny_cache):
    shape, W, Wt = tiny
    cache, anchor = tiny_cache
    d, d1, d2, filled = Dc.two_step_draft(Wt, cache, anchor, 32, n_fill=0)
    one = M.argmax_lowest(Dc.draft_pass(Wt, cache, [anchor] + [shape.mask_id] * 31))
    assert not filled.any() and np.array_equal(d, one) and np.array_equal(d1, one) and np.array_equal(d2, one)


def test_two_step_fills_half_and_keeps_pass_one_tokens(tiny, tiny_cache):
    shape, W, Wt = tiny
    cache, anchor = tiny_cache
    d, d1, d2, filled = Dc.two_step_draft(Wt, cache, anchor, 32)
    assert filled.sum() == 15 and not filled[31]
    assert np.array_equal(d[filled], d1[filled]) and np.array_equal(d[~filled], d2[~filled])
    # the filled rows are the most confident pass-1 rows
    conf = Dc.log_confidence(Dc.draft_pass(Wt, cache, [anchor] + [shape.mask_id] * 31)[:31], d1[:31])
    assert conf[filled[:31]].min() >= conf[~filled[:31]].max()
    # pass 2 sees the filled tokens: with every mask filled, pass 2's block is the verify block
    # of a one-step round with drafts d1, and only the last row comes from pass 2
    d, d1, d2, filled = Dc.two_step_draft(Wt, cache, anchor, 32, n_fill=31)
    assert filled[:31].all() and np.array_equal(d[:31], d1[:31]) and d[31] == d2[31]
    verify_block = [anchor] + [int(t) for t in d1[:31]]  # slot j holds row j-1's token, as in verify
    assert np.array_equal(d2, M.argmax_lowest(Dc.draft_pass(Wt, cache, verify_block)))


def test_two_step_orthrus_equals_greedy_ar(tiny, tiny_prompt):
    shape, W, Wt = tiny
    res = Dc.generate(Wt, tiny_prompt, 40, two_step=15)
    assert res.tokens == Dc.generate_ar(Wt, tiny_prompt, 40)
    assert res.passes == 3 * len(res.rounds)
    assert all(1 <= len(r.emitted) <= 32 for r in res.rounds)
