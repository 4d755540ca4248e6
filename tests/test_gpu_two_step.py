"""Two-step drafting on the GPU (the Fast-dLLM-v2 style variant that Orthrus paper summary sec. 六
ablates): orthrus_draft_fill / orthrus_draft_merge against the oracle, then whole two-step rounds.

Bars: the fill set, pass-2 block tokens and merged drafts are integer results and must equal the
oracle's, except where the oracle's own confidences (fp64) of two competing rows lie within 1e-5
of each other (the kernel ranks fp32 scores); token trajectories and accept counts bit-exact.
"""
import numpy as np
import pytest
import torch

import orthrus_round_amd as ora
import synth
from orthrus_round_amd.decoder import Decoder
from oracle import decode as Dc
from oracle import model as M

pytestmark = pytest.mark.gpu
DEV = "cuda"
TIE = 1e-5


def fill_case(seed, B, K, hidden, vocab, dtype, dup=False, nan_row=None):
    rs = np.random.default_rng(seed)
    rnd = synth.bf16_round if dtype == ora.BF16 else (lambda a: a.astype(np.float32))
    h = rnd(rs.standard_normal((B * K, hidden)).astype(np.float32))
    w = rnd((rs.standard_normal((vocab, hidden)) * 0.05).astype(np.float32))
    z = h.astype(np.float64) @ w.astype(np.float64).T
    d = M.argmax_lowest(z).astype(np.int32)
    if dup:  # exact score ties: rows 2..5 of every sequence repeat row 1's state and token
        for b in range(B):
            for j in range(2, min(6, K - 1)):
                h[b * K + j] = h[b * K + 1]
                z[b * K + j] = z[b * K + 1]
                d[b * K + j] = d[b * K + 1]
    m = z.max(axis=1)
    lse = (m + np.log(np.exp(z - m[:, None]).sum(axis=1))).astype(np.float32)
    if nan_row is not None:
        lse[nan_row] = np.nan
    return h, w, z, d.reshape(B, K), lse


def gpu_fill(h, w, lse, d, dtype, mask_id, n_fill):
    B, K = d.shape
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    hh = t(h).to(torch.bfloat16) if dtype == ora.BF16 else t(h)
    ww = t(w).to(torch.bfloat16) if dtype == ora.BF16 else t(w)
    tok2 = torch.full((B, K), -7, dtype=torch.int32, device=DEV)
    filled = torch.full((B, K), -7, dtype=torch.int32, device=DEV)
    ora.draft_fill(B, K, h.shape[1], w.shape[0], dtype, hh, ww, t(lse), t(d), mask_id, n_fill, tok2, filled)
    torch.cuda.synchronize()
    return tok2.cpu().numpy(), filled.cpu().numpy()


def check_fill(z, lse, d, tok2, filled, mask_id, n_fill):
    B, K = d.shape
    for b in range(B):
        rows = slice(b * K, b * K + K - 1)
        conf = Dc.log_confidence(z[rows], d[b, : K - 1])
        conf = np.where(np.isnan(lse[rows]), np.nan, conf)
        want = Dc.most_confident(conf, n_fill)
        got = filled[b, : K - 1].astype(bool)
        assert filled[b, K - 1] == 0 and tok2[b, K - 1] == mask_id
        assert got.sum() == n_fill
        diff = np.flatnonzero(got != want)
        if len(diff):
            key = np.where(np.isnan(conf), -np.inf, conf)
            edge = np.sort(key)[::-1][n_fill - 1] if n_fill else np.inf
            assert all(abs(key[i] - edge) <= TIE for i in diff), (b, diff, key[diff], edge)
        assert np.array_equal(tok2[b, : K - 1], np.where(got, d[b, : K - 1], mask_id))


@pytest.mark.parametrize("dtype", [ora.BF16, ora.F32])
@pytest.mark.parametrize("B,K,n_fill", [(4, 32, 15), (3, 32, 0), (2, 32, 31), (5, 5, 2), (2, 1, 0), (1, 64, 20)])
def test_draft_fill_matches_oracle(dtype, B, K, n_fill):
    h, w, z, d, lse = fill_case(B * 100 + K, B, K, 256, 512, dtype)
    tok2, filled = gpu_fill(h, w, lse, d, dtype, 511, n_fill)
    check_fill(z, lse, d, tok2, filled, 511, n_fill)


@pytest.mark.parametrize("dtype", [ora.BF16, ora.F32])
def test_draft_fill_ties_go_to_the_lower_slot_and_nan_last(dtype):
    B, K = 3, 32
    h, w, z, d, lse = fill_case(7, B, K, 512, 300, dtype, dup=True, nan_row=K + 3)
    for n_fill in (1, 3, 15, 31):
        tok2, filled = gpu_fill(h, w, lse, d, dtype, 299, n_fill)
        check_fill(z, lse, d, tok2, filled, 299, n_fill)
    assert filled[1, 3] == 1  # n_fill 31 fills every slot, the NaN one included
    tok2, filled = gpu_fill(h, w, lse, d, dtype, 299, 30)
    assert filled[1, 3] == 0 and filled[1, :31].sum() == 30  # ... and it is the one left out at 30


def test_draft_merge_is_a_select():
    rs = np.random.default_rng(3)
    B, K = 6, 32
    filled = rs.integers(0, 2, (B, K)).astype(np.int32)
    tok2 = rs.integers(0, 1000, (B, K)).astype(np.int32)
    d2 = rs.integers(0, 1000, (B, K)).astype(np.int32)
    t = lambda x: torch.from_numpy(x).to(DEV)
    out = torch.full((B, K), -1, dtype=torch.int32, device=DEV)
    ora.draft_merge(B, K, t(filled), t(tok2), t(d2), out)
    d2g = t(d2)
    ora.draft_merge(B, K, t(filled), t(tok2), d2g, d2g)  # in place
    torch.cuda.synchronize()
    want = np.where(filled != 0, tok2, d2)
    assert np.array_equal(out.cpu().numpy(), want) and np.array_equal(d2g.cpu().numpy(), want)


# ------------------------------------------------------------------- whole rounds, tiny FP32 decoder

SHAPE = synth.TINY


@pytest.fixture(scope="module")
def tiny():
    W = synth.model_weights(SHAPE, cfg=1)
    return W, M.Weights(W, SHAPE)


@pytest.fixture(scope="module")
def prompts():
    return synth.prompt_ids(SHAPE, 1, 4, 64)


def test_first_two_step_round_matches_oracle(tiny, prompts):
    W, Wt = tiny
    dec = Decoder(W, SHAPE, precision="fp32", block=32, max_batch=1, max_ctx=64 + 160)
    dec.prefill(torch.from_numpy(prompts[:1]), max_out=64)
    dec.round_greedy_two_step(15)
    torch.cuda.synchronize()
    cache, anchor = Dc.prefill(Wt, prompts[0], 64 + 160)
    d, d1, d2, filled = Dc.two_step_draft(Wt, cache, anchor, 32, 15)
    assert np.array_equal(dec.filled[0].cpu().numpy().astype(bool), filled)
    assert np.array_equal(dec.draft2[0].cpu().numpy(), d2)
    assert np.array_equal(dec.draft[0].cpu().numpy(), d)
    t = M.argmax_lowest(Dc.ar_pass(Wt, cache, [anchor] + [int(x) for x in d[:31]]))
    k, _ = Dc.consensus(d, t)
    assert int(dec.accept[0]) == k and int(dec.ctx_len[0]) == 63 + min(k + 1, 32)


def test_two_step_trajectory_and_accepts_match_oracle(tiny, prompts):
    W, Wt = tiny
    dec = Decoder(W, SHAPE, precision="fp32", block=32, max_batch=1, max_ctx=64 + 128 + 64)
    toks, st = dec.generate(prompts[:1], 128, poll_every=1, record_accepts=True, two_step=15)
    ref = Dc.generate(Wt, prompts[0], 128, two_step=15)
    assert list(toks[0]) == ref.tokens == Dc.generate_ar(Wt, prompts[0], 128)
    assert [int(h[0]) for h in st.accept_hist[: len(ref.rounds)]] == [r.accept for r in ref.rounds]
    assert st.passes == 3 * st.rounds


@pytest.mark.parametrize("precision", ["fp32", "bf16"])
def test_two_step_batch_equals_ar_with_graphs(tiny, prompts, precision):
    W, _ = tiny
    dec = Decoder(W, SHAPE, precision=precision, block=32, max_batch=4, max_ctx=64 + 96 + 64)
    a, _ = dec.generate(prompts, 96, two_step=15, use_graph=True)
    b, _ = dec.generate_ar(prompts, 96, use_graph=True)
    assert np.array_equal(a, b)
