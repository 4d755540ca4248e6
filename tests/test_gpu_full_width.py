"""GPU parity at the full-size round configuration: 8 decoder layers at Qwen3-8B width (hidden 4096,
32Q/8KV heads x 128, SwiGLU 12288, vocabulary 151936), batch 8, the weights of the timed round.

The prompts are 64 tokens (700 in one case) so that the oracle (float64, BLAS over rows) finishes in
seconds; the kernels and their launch configuration are those of the timed round (256-row GEMMs,
151936-wide LM head, paged attention with the same kv_chunk).

* Sequence 0's first round through the fp32 decoder (the same bf16-valued weights held in fp32)
  against the oracle, after the 64-token prompts and after 700-token ones (two key chunks): the 32
  draft ids and the 32 verify ids, where an id may differ only at an
  oracle near-tie (top two logits within 1e-4 relative); the verify pass is run by the oracle on
  the GPU's own drafts, since an ambiguous draft changes the verify inputs; then the accept count
  and the new KV length, which are integer logic on the GPU's own ids and must be exact.
* The same first round at temperature 0.8: Gumbel-max drafts, logits, and the rejection accept.
* All 8 sequences: GPU Orthrus == GPU AR over 512 tokens, in fp32 and in bf16 (losslessness).
"""
import numpy as np
import pytest
import torch

import synth
from orthrus_round_amd.decoder import Decoder
from oracle import decode as Dc
from oracle import model as M

pytestmark = pytest.mark.gpu
SHAPE = synth.QWEN3_8B_L8
P = 64
KV_CHUNK = 640


@pytest.fixture(scope="module")
def weights():
    return synth.model_weights(SHAPE, cfg=5, diff_std=0.002, bf16=True)


@pytest.fixture(scope="module")
def prompts():
    return synth.prompt_ids(SHAPE, 5, 8, P)


def tie_ok(z, got, ref):
    """Same id, or an oracle near-tie between the two ids."""
    if int(got) == int(ref):
        return True
    return z[ref] - z[got] <= 1e-4 * max(1.0, abs(z[ref]))


@pytest.mark.parametrize("plen", [P, 700])
def test_first_round_matches_oracle(weights, prompts, plen):
    """plen 700: the cache spans two 640-key chunks, so the chunked attention and
    its combine are on the checked path."""
    pr = prompts if plen == P else synth.prompt_ids(SHAPE, 5, 8, plen)
    dec = Decoder(weights, SHAPE, precision="fp32", block=32, max_batch=pr.shape[0], max_ctx=plen + 96,
                  kv_chunk=KV_CHUNK)
    dec.prefill(torch.from_numpy(pr), max_out=64)
    n0 = int(dec.ctx_len[0])
    dec.round_greedy()
    torch.cuda.synchronize()
    d_gpu = dec.draft[0].cpu().numpy().copy()
    t_gpu = dec.target[0].cpu().numpy().copy()
    acc_gpu, n_gpu = int(dec.accept[0]), int(dec.ctx_len[0])
    del dec
    torch.cuda.empty_cache()

    Wt = M.Weights(weights, SHAPE)
    cache, anchor = Dc.prefill(Wt, pr[0], plen + 96, rowwise=False)
    assert cache.n == n0 == plen - 1
    zd = Dc.draft_pass(Wt, cache, [anchor] + [SHAPE.mask_id] * 31, rowwise=False)
    d_ref = M.argmax_lowest(zd)
    bad = [i for i in range(32) if not tie_ok(zd[i], d_gpu[i], d_ref[i])]
    assert not bad, ("drafts", bad, d_gpu[bad], d_ref[bad])
    zt = Dc.ar_pass(Wt, cache, [anchor] + [int(x) for x in d_gpu[:31]], rowwise=False)
    t_ref = M.argmax_lowest(zt)
    bad = [i for i in range(32) if not tie_ok(zt[i], t_gpu[i], t_ref[i])]
    assert not bad, ("targets", bad, t_gpu[bad], t_ref[bad])
    k, emitted = Dc.consensus(d_gpu, t_gpu)
    assert acc_gpu == k
    assert n_gpu == n0 + min(k + 1, 32)
    print(f"drafts equal {int((d_gpu == d_ref).sum())}/32, targets equal {int((t_gpu == t_ref).sum())}/32, "
          f"accept {k}")


def test_first_sampled_round_matches_oracle(weights, prompts):
    """T = 0.8 at full width (fp32 decoder): sequence 0's 32 drafts are the Gumbel-max draws of the
    oracle's draft logits with the oracle's counters (within the eps_tie band of the keys); the
    device's draft and verify logits equal the oracle's within 2e-5 normwise (the verify pass run on
    the device's drafts); the accept count, committed tokens and KV length equal the oracle's
    rejection accept on the device's own logits."""
    T, seed = 0.8, 17
    dec = Decoder(weights, SHAPE, precision="fp32", block=32, max_batch=8, max_ctx=P + 96, kv_chunk=KV_CHUNK)
    dec.prefill(torch.from_numpy(prompts), max_out=64)
    n0 = int(dec.ctx_len[0])
    dec.round_sampled(T, seed)
    torch.cuda.synchronize()
    d_gpu = dec.draft[0].cpu().numpy().copy()
    zd_gpu = dec._logits[0][:32].cpu().numpy().astype(np.float64)
    zt_gpu = dec._logits[1][:32].cpu().numpy().astype(np.float64)
    acc_gpu, n_gpu = int(dec.accept[0]), int(dec.ctx_len[0])
    out_gpu = dec.out_tokens[0].cpu().numpy().copy()
    del dec
    torch.cuda.empty_cache()

    Wt = M.Weights(weights, SHAPE)
    cache, anchor = Dc.prefill(Wt, prompts[0], P + 96, rowwise=False)
    zd = Dc.draft_pass(Wt, cache, [anchor] + [SHAPE.mask_id] * 31, rowwise=False)
    assert np.abs(zd_gpu - zd).max() / np.abs(zd).max() <= 2e-5
    for i in range(32):
        u = Dc.uniforms(seed, Dc.STREAM_DRAFT, i, np.arange(SHAPE.vocab), 0, 0)
        key = zd[i] / T - np.log(-np.log(u))
        assert tie_ok(key, d_gpu[i], int(np.argmax(key))), i
    zt = Dc.ar_pass(Wt, cache, [anchor] + [int(x) for x in d_gpu[:31]], rowwise=False)
    assert np.abs(zt_gpu - zt).max() / np.abs(zt).max() <= 2e-5
    ua = Dc.uniforms(seed, Dc.STREAM_ACCEPT, np.arange(32), 0, 0, 0)
    er = -np.log(Dc.uniforms(seed, Dc.STREAM_RESID, np.arange(SHAPE.vocab), 0, 0, 0))
    k, em = Dc.rejection_accept(zd_gpu, zt_gpu, d_gpu, T, ua, er)
    assert acc_gpu == k
    assert list(out_gpu[:len(em)]) == em
    assert n_gpu == n0 + min(k + 1, 32)
    print(f"sampled round: accept {k}, emitted {em}")


@pytest.mark.parametrize("precision", ["fp32", "bf16"])
def test_orthrus_equals_ar_full_width(weights, prompts, precision):
    """512 generated tokens for all 8 sequences (the full-round workload's length): greedy Orthrus
    and greedy AR through the same kernels give the same trajectories."""
    N = 512
    dec = Decoder(weights, SHAPE, precision=precision, block=32, max_batch=8, max_ctx=P + N + 96,
                  kv_chunk=KV_CHUNK)
    a, st = dec.generate(prompts, N, use_graph=True, poll_every=32)
    b, _ = dec.generate_ar(prompts, N, use_graph=True)
    assert np.array_equal(a, b), [int(np.argmax(a[i] != b[i])) for i in range(8)]
    print(f"{precision}: {st.rounds} rounds for {N} tokens x 8 sequences")


def test_two_step_drafting_equals_ar_full_width(weights, prompts):
    """Two-step drafting (two diffusion passes, 15 masks filled after the first) keeps the round
    lossless at 8B width in bf16."""
    dec = Decoder(weights, SHAPE, precision="bf16", block=32, max_batch=8, max_ctx=P + 96, kv_chunk=KV_CHUNK)
    a, st = dec.generate(prompts, 16, use_graph=True, two_step=15)
    b, _ = dec.generate_ar(prompts, 16, use_graph=True)
    assert np.array_equal(a[:, :16], b[:, :16])
    assert st.passes == 3 * int(dec.round.sum())
