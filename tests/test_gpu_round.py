"""End-to-end rounds on the GPU: the tiny FP32 decoder against the CPU oracle, losslessness
(GPU Orthrus trajectory == GPU AR trajectory), batch and page-order invariance, graph replay
and temperature > 0 sampling with the oracle's own Philox counters.

Bars: token ids, per-round accept counts and KV lengths bit-exact against the oracle (an
oracle near-tie at a divergence point would be reported, not hidden).
"""
import numpy as np
import pytest
import torch

import synth
from orthrus_round_amd.decoder import Decoder
from oracle import decode as Dc
from oracle import model as M

pytestmark = pytest.mark.gpu
SHAPE = synth.TINY


@pytest.fixture(scope="module")
def tiny():
    W = synth.model_weights(SHAPE, cfg=1)
    return W, M.Weights(W, SHAPE)


@pytest.fixture(scope="module")
def prompts():
    return synth.prompt_ids(SHAPE, 1, 4, 64)


def make(W, precision="fp32", B=1, **kw):
    return Decoder(W, SHAPE, precision=precision, block=32, max_batch=B, max_ctx=64 + 256 + 64, **kw)


def test_tiny_fp32_trajectory_and_accepts_match_oracle(tiny, prompts):
    W, Wt = tiny
    dec = make(W)
    toks, st = dec.generate(prompts[:1], 256, poll_every=1, record_accepts=True)
    ref = Dc.generate(Wt, prompts[0], 256)
    assert list(toks[0]) == ref.tokens
    gpu_acc = [int(h[0]) for h in st.accept_hist[: len(ref.rounds)]]
    assert gpu_acc == [r.accept for r in ref.rounds]
    assert int(dec.ctx_len[0]) == 63 + sum(len(r.emitted) for r in ref.rounds)
    assert st.rounds == len(ref.rounds)
    assert min(gpu_acc) >= 0  # every round commits accept + 1 >= 1 tokens
    print(f"rounds {st.rounds} tpf {st.tpf:.3f}")


def test_other_kv_chunk_matches_oracle_and_accounts_memory(tiny, prompts):
    """Another attention key chunking (another summation order) still reproduces the oracle's
    trajectory and accepts in fp32; the decoder's memory accounting covers the block K/V buffer
    (one layer's block rows, reused by every layer) and the paged cache of every layer."""
    W, Wt = tiny
    dec = make(W)
    dec.set_kv_chunk(64)
    toks, st = dec.generate(prompts[:1], 96, poll_every=1, record_accepts=True)
    ref = Dc.generate(Wt, prompts[0], 96)
    assert list(toks[0]) == ref.tokens
    assert [int(h[0]) for h in st.accept_hist[: len(ref.rounds)]] == [r.accept for r in ref.rounds]
    rb = dec.runtime_bytes()
    s = SHAPE
    assert rb["block_kv"] == 2 * 1 * 32 * s.kv_heads * s.head_dim * 4
    assert rb["kv_cache"] == 2 * s.layers * dec.num_pages * s.kv_heads * dec.page * s.head_dim * 4
    assert rb["weights_diff_view"] == rb["weights_ar_view"] > 0


@pytest.mark.parametrize("block", [8, 1])
def test_smaller_block_matches_oracle(tiny, prompts, block):
    """A decoder built for 32-row rounds, switched to `block` rows: tokens and per-round accepts
    equal the oracle's Orthrus run with the same block (block 1 is plain AR decoding)."""
    W, Wt = tiny
    dec = make(W)
    dec.set_block(block)
    toks, st = dec.generate(prompts[:1], 96, poll_every=1, record_accepts=True)
    ref = Dc.generate(Wt, prompts[0], 96, block=block)
    assert list(toks[0]) == ref.tokens
    assert [int(h[0]) for h in st.accept_hist[: len(ref.rounds)]] == [r.accept for r in ref.rounds]
    assert int(dec.ctx_len[0]) == 63 + sum(len(r.emitted) for r in ref.rounds)


@pytest.mark.parametrize("precision", ["fp32", "bf16"])
def test_orthrus_equals_ar_on_gpu(tiny, prompts, precision):
    W, _ = tiny
    dec = make(W, precision, B=4)
    a, _ = dec.generate(prompts, 200)
    b, _ = dec.generate_ar(prompts, 200)
    match = [bool(np.array_equal(a[i], b[i])) for i in range(4)]
    print(precision, "trajectory match", match)
    assert all(match)


def test_batch_and_page_order_invariance(tiny, prompts):
    W, _ = tiny
    full, _ = make(W, B=4, page_order_seed=5).generate(prompts, 96)
    for i in (0, 3):
        one, _ = make(W, B=1).generate(prompts[i:i + 1], 96)
        assert np.array_equal(one[0], full[i])


def test_graph_replay_matches_eager(tiny, prompts):
    W, _ = tiny
    dec = make(W, "bf16", B=4)
    a, sa = dec.generate(prompts, 128)
    b, sb = dec.generate(prompts, 128, use_graph=True)
    assert np.array_equal(a, b) and sa.rounds == sb.rounds
    c, _ = dec.generate_ar(prompts, 64, use_graph=True)
    d, _ = dec.generate_ar(prompts, 64)
    assert np.array_equal(c, d)


def test_sampled_rounds_match_oracle(tiny, prompts):
    """T = 0.8: drafts (Gumbel), acceptance and residual draws use the same Philox counters."""
    W, Wt = tiny
    T, seed = 0.8, 31
    dec = make(W)
    toks, st = dec.generate(prompts[:1], 64, temperature=T, seed=seed, poll_every=1, record_accepts=True)
    ref = Dc.generate(Wt, prompts[0], 64, temperature=T, seed=seed)
    assert list(toks[0]) == ref.tokens
    assert [int(h[0]) for h in st.accept_hist[: len(ref.rounds)]] == [r.accept for r in ref.rounds]


def test_sampled_ar_matches_oracle(tiny, prompts):
    W, Wt = tiny
    dec = make(W)
    toks, _ = dec.generate_ar(prompts[:1], 48, temperature=0.8, seed=7)
    assert list(toks[0]) == Dc.generate_ar(Wt, prompts[0], 48, temperature=0.8, seed=7)


def test_ar_step_returns_each_sequences_token(tiny, prompts):
    """ar_step's return value holds every sequence's own token of that step."""
    W, _ = tiny
    dec = make(W, B=4)
    dec.prefill(torch.as_tensor(prompts), 6)
    for step in range(6):
        tok = dec.ar_step().cpu().numpy()[:, 0]
        assert np.array_equal(tok, dec.out_tokens[:, step].cpu().numpy()), step
