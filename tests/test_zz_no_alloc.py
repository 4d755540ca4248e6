"""orthrus_lmhead_argmax_noalloc (partials in the library's static device array) against
orthrus_lmhead_argmax (partials in a caller workspace), through the C ABI: tokens, logsumexp and
logits bit for bit, on two calls in a row, the second with fewer rows and another mode; a request
above the static array's size is refused before launching."""
import numpy as np
import pytest
import torch

import orthrus_round_amd as ora
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _call(fn, rows, hidden, vocab, h, w, T, sample, seqs, rnds, block):
    d = ora.lmhead_desc(rows, hidden, vocab, ora.BF16, block, ora.STREAM_DRAFT, T, 5, sample)
    tok = torch.full((rows,), -3, dtype=torch.int32, device=DEV)
    lse = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
    logits = torch.full((rows, vocab), float("nan"), dtype=torch.float32, device=DEV)
    if fn == "ws":
        ws = torch.empty(ora.lmhead_workspace_bytes(d), dtype=torch.uint8, device=DEV)
        ora.lmhead_argmax(d, h, w, seqs, rnds, tok, logits, lse, ws)
    else:
        ora.lmhead_argmax_noalloc(d, h, w, seqs, rnds, tok, logits, lse)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), lse.cpu().numpy(), logits.cpu().numpy()


def test_noalloc_lmhead_equals_workspace_call_twice():
    hidden, vocab = 512, 151936
    hs, w = synth.lmhead_inputs(40, 256, hidden, vocab)
    h_t = torch.from_numpy(hs).to(torch.bfloat16).to(DEV)
    w_t = torch.from_numpy(w).to(torch.bfloat16).to(DEV)
    seqs = torch.arange(8, dtype=torch.int32, device=DEV)
    rnds = torch.full((8,), 2, dtype=torch.int32, device=DEV)
    # first call: 256 rows, greedy (256x256 pair tiles plus 128x128 row-halves of the rest)
    a = _call("ws", 256, hidden, vocab, h_t, w_t, 0.0, False, seqs, rnds, 32)
    b = _call("noalloc", 256, hidden, vocab, h_t, w_t, 0.0, False, seqs, rnds, 32)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # second call, smaller: 40 rows sampled at T = 0.8 (another tile shape; the array keeps the
    # first call's partials, which this call must overwrite before reading)
    a = _call("ws", 40, hidden, vocab, h_t[:40], w_t, 0.8, True, seqs, rnds, 8)
    b = _call("noalloc", 40, hidden, vocab, h_t[:40], w_t, 0.8, True, seqs, rnds, 8)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert (b[0] >= 0).all() and np.isfinite(b[1]).all()


def test_noalloc_lmhead_refuses_above_its_array():
    d = ora.lmhead_desc(1024, 4096, 151936, ora.BF16, 32)
    assert ora.lmhead_workspace_bytes(d) > 32 << 20
    tok = torch.full((4,), -3, dtype=torch.int32, device=DEV)
    with pytest.raises(ora.OrthrusError) as e:
        ora.lmhead_argmax_noalloc(d, 1, 1, None, None, tok, None, None)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert (tok.cpu().numpy() == -3).all()
