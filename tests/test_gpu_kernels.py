"""GPU parity of the LM head, consensus/commit, rejection accept, Philox and the support
kernels (C ABI) against the CPU oracle.

Bars: token ids, accept counts, corrections and KV lengths bit-exact, except argmax rows
whose oracle top-2 gap is below eps_tie = 1e-4 * max(1, |z_top|) (either id passes; such
rows are counted and printed); float outputs within 2e-3 normwise (bf16) / 2e-5 (fp32).
"""
import numpy as np
import pytest
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


def gemm_ws(M, N, K, dtype, epi):
    return torch.zeros(max(256, ora.gemm_workspace_bytes(M, N, K, dtype, epi)), dtype=torch.uint8, device=DEV)


def tie_ok(z, gpu_id, ref_id):
    """Same id, or an oracle near-tie between the two ids."""
    if gpu_id == ref_id:
        return True, False
    gap = z[ref_id] - z[gpu_id]
    return gap <= 1e-4 * max(1.0, abs(z[ref_id])), True


def lmhead(h, w, dtype, temperature=0.0, seed=0, block=32, seq=None, rnd=None, want_logits=False, want_lse=True,
           sample=None):
    rows, hidden = h.shape
    vocab = w.shape[0]
    d = ora.lmhead_desc(rows, hidden, vocab, dtype, block, ora.STREAM_DRAFT, temperature, seed, sample)
    ws = torch.empty(ora.lmhead_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    tok = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    lse = torch.empty(rows, dtype=torch.float32, device=DEV) if want_lse else None
    logits = torch.empty((rows, vocab), dtype=torch.float32, device=DEV) if want_logits else None
    nb = rows // block
    seq_t = dev(np.arange(nb, dtype=np.int32) if seq is None else seq)
    rnd_t = dev(np.zeros(nb, np.int32) if rnd is None else rnd)
    ora.lmhead_argmax(d, dev(h, dtype), dev(w, dtype), seq_t, rnd_t, tok, logits, lse, ws)
    torch.cuda.synchronize()
    return (tok.cpu().numpy(), lse.cpu().numpy() if want_lse else None,
            (logits.cpu().numpy() if want_logits else None))


def logits_f64(h, w, chunk=16384):
    """z = h w^T in float64, the vocabulary taken in chunks to bound host memory."""
    h64 = h.astype(np.float64)
    z = np.empty((h.shape[0], w.shape[0]))
    for c in range(0, w.shape[0], chunk):
        z[:, c:c + chunk] = h64 @ w[c:c + chunk].astype(np.float64).T
    return z


def lse_f64(z, T=1.0):
    zt = z / T
    m = zt.max(1)
    return m + np.log(np.exp(zt - m[:, None]).sum(1))


# ------------------------------------------------------------------- LM head

# Above 128 rows: 511*128 + 77 columns are 512 tiles, two whole waves of 256x256 pair workgroups whose
# last pair holds the ragged tile; 515 tiles at 300 rows leave a rest of three tiles, run as 128x128
# row tiles (three of them, the last ragged); hidden 192 (an odd number of k-stages) takes the 256x128
# layout alone.
@pytest.mark.parametrize("rows,hidden,vocab,dtype", [(64, 256, 4096, ora.F32), (37, 256, 4000, ora.BF16),
                                                     (128, 512, 1024 + 64, ora.BF16), (8, 4096, 8192, ora.BF16),
                                                     (256, 256, 511 * 128 + 77, ora.BF16),
                                                     (300, 256, 515 * 128, ora.BF16), (256, 192, 70000, ora.BF16)])
def test_lmhead_argmax_small(rows, hidden, vocab, dtype):
    h, w = synth.lmhead_inputs(8, rows, hidden, vocab, bf16=(dtype == ora.BF16))
    tok, lse, logits = lmhead(h, w, dtype, block=1, want_logits=True)
    z = h.astype(np.float64) @ w.astype(np.float64).T
    ref = M.argmax_lowest(z)
    amb = 0
    for r in range(rows):
        ok, a = tie_ok(z[r], tok[r], ref[r])
        assert ok, (r, tok[r], ref[r])
        amb += a
    tol = 2e-5 if dtype == ora.F32 else 2e-3
    assert np.abs(logits - z).max() / np.abs(z).max() <= tol
    zl = z.max(1) + np.log(np.exp(z - z.max(1, keepdims=True)).sum(1))
    np.testing.assert_allclose(lse, zl, rtol=1e-5, atol=1e-5)
    print("ambiguous rows:", amb)


def test_lmhead_exact_ties_lowest_id():
    rs = np.random.default_rng(3)
    w = synth.bf16_round(rs.standard_normal((2048, 128)).astype(np.float32))
    w[1500] = w[100]
    w[1900] = w[100]
    h = synth.bf16_round((w[100:101] * 2).astype(np.float32))
    tok, _, _ = lmhead(np.repeat(h, 4, 0), w, ora.BF16, block=1)
    assert (tok == 100).all()


@pytest.fixture(scope="module")
def c4():
    h, w = synth.lmhead_inputs(4, 512, 4096, 151936)
    return h, w


def test_lmhead_qwen3_8b_all_rows(c4):
    """Every one of the 512 rows: token (ties per eps_tie), logsumexp and logits."""
    h, w = c4
    tok, lse, logits = lmhead(h, w, ora.BF16, want_logits=True)
    z = logits_f64(h, w)
    ref = M.argmax_lowest(z)
    amb = 0
    for r in range(512):
        ok, a = tie_ok(z[r], tok[r], ref[r])
        assert ok, (r, tok[r], ref[r])
        amb += a
    np.testing.assert_allclose(lse, lse_f64(z), rtol=1e-5)
    assert np.abs(logits - z).max() / np.abs(z).max() <= 2e-3
    print("ambiguous rows:", amb)


def test_lmhead_row_invariance(c4):
    """A row's token and logsumexp have the same bits whatever rows share the launch: 512 and 200
    rows (256x256 pair tiles plus 128x128 row-halves of the rest), 128, 64, 33, 7 and 1 (other tile
    shapes)."""
    h, w = c4
    full = lmhead(h, w, ora.BF16, block=1)
    for m in (200, 128, 64, 33, 7, 1):
        part = lmhead(h[:m], w, ora.BF16, block=1)
        assert np.array_equal(part[0], full[0][:m]), m
        assert np.array_equal(part[1], full[1][:m]), m


def test_lmhead_lse_is_optional_and_temperature_scaled(c4):
    """Without lse_out the token choice is unchanged; an argmax call at T > 0 (the verify pass of a
    sampled round) returns the argmax, the same logits, and logsumexp(z / T)."""
    h, w = c4
    rows = h[:96]
    tok, lse, logits = lmhead(rows, w, ora.BF16, want_logits=True)
    tok2, none, _ = lmhead(rows, w, ora.BF16, want_lse=False)
    assert none is None and np.array_equal(tok, tok2)
    T = 0.8
    tok3, lse3, logits3 = lmhead(rows, w, ora.BF16, temperature=T, block=32, want_logits=True, sample=False)
    assert np.array_equal(tok3, tok) and np.array_equal(logits3, logits)
    np.testing.assert_allclose(lse3, lse_f64(logits.astype(np.float64), T), rtol=1e-5)
    assert np.abs(lse3 - lse).max() > 0.1  # the temperature is applied


@pytest.mark.parametrize("M,block", [(64, 32), (40, 4), (60, 6), (7, 1)])
def test_lmhead_gumbel_sampling_matches_oracle(M, block):
    """Blocks that are a multiple of 4 take one Philox call per four rows of a lane (its four
    words); other blocks one call per element.  Both must draw the oracle's uniforms."""
    T, seed = 0.8, 1234
    h, w = synth.lmhead_inputs(9, M, 256, 4096, bf16=False)
    nseq = M // block
    seqs = (np.arange(nseq, dtype=np.int32) * 4 + 5)
    rnds = (np.arange(nseq, dtype=np.int32) * 3) % 7
    tok, lse, _ = lmhead(h, w, ora.F32, temperature=T, seed=seed, block=block, seq=seqs, rnd=rnds)
    z = h.astype(np.float64) @ w.astype(np.float64).T
    amb = 0
    for r in range(M):
        b, s = divmod(r, block)
        u = P.uniforms(seed, P.STREAM_DRAFT, s, np.arange(4096), rnds[b], seqs[b])
        key = z[r] / T - np.log(-np.log(u))
        ok, a = tie_ok(key, tok[r], int(np.argmax(key)))
        assert ok, r
        amb += a
    zt = z / T
    np.testing.assert_allclose(lse, zt.max(1) + np.log(np.exp(zt - zt.max(1, keepdims=True)).sum(1)), rtol=1e-5)


def test_lmhead_sampling_distribution_tiny_vocab():
    """Gumbel-max on device draws from softmax(z/T): chi-square over many (round) counters."""
    V, T = 64, 0.8
    rs = np.random.default_rng(11)
    w = (rs.standard_normal((V, 64)) * 0.3).astype(np.float32)
    h = np.ones((32, 64), np.float32)
    z = (h[0].astype(np.float64) @ w.T.astype(np.float64))
    p = np.exp(z / T - (z / T).max())
    p /= p.sum()
    counts = np.zeros(V)
    for rnd in range(200):
        tok, _, _ = lmhead(h, w, ora.F32, temperature=T, seed=77, block=32, rnd=np.array([rnd], np.int32))
        counts += np.bincount(tok, minlength=V)
    N = counts.sum()
    mask = p * N >= 5
    chi2 = ((counts[mask] - N * p[mask]) ** 2 / (N * p[mask])).sum()
    assert chi2 < mask.sum() + 6 * np.sqrt(2 * mask.sum())


# ------------------------------------------------------------------- consensus / commit

def test_consensus_commit_geometric_drafts(c4):
    h, w = c4
    t, _, _ = lmhead(h, w, ora.BF16)
    t = t.reshape(16, 32)
    d, L = synth.geometric_drafts(4, t, 151936)
    ctx0 = synth.ragged_lengths(4, 16, 512, 16384)
    max_out, max_ctx = 40, 20000
    st = {k: torch.zeros(16, dtype=torch.int32, device=DEV) for k in ("anchor", "accept", "out_len", "round", "done")}
    ctx = dev(ctx0)
    out = torch.full((16, max_out), -1, dtype=torch.int32, device=DEV)
    st["out_len"][:3] = torch.tensor([0, 20, 39], dtype=torch.int32)
    st["done"][15] = 1
    ora.consensus_commit(16, 32, dev(d), dev(t), ctx, st["anchor"], st["accept"], out, st["out_len"], st["round"],
                         st["done"], max_out, max_ctx)
    torch.cuda.synchronize()
    acc, ol, an, cx = (st["accept"].cpu().numpy(), st["out_len"].cpu().numpy(), st["anchor"].cpu().numpy(),
                       ctx.cpu().numpy())
    outn = out.cpu().numpy()
    ol0 = np.array([0, 20, 39] + [0] * 13)
    for b in range(15):
        k, em = Dc.consensus(d[b], t[b])
        assert acc[b] == k == L[b]
        assert cx[b] == ctx0[b] + min(k + 1, 32)
        assert an[b] == em[-1]
        wr = min(len(em), max_out - ol0[b])
        assert ol[b] == ol0[b] + wr
        assert list(outn[b, ol0[b]:ol0[b] + wr]) == em[:wr]
    assert acc[15] == -1 and cx[15] == ctx0[15] and ol[15] == 0
    dn = st["done"].cpu().numpy()
    assert dn[2] == 1 and dn[15] == 1


def test_consensus_every_mismatch_position():
    K = 32
    B = K + 1
    rs = np.random.default_rng(2)
    t = rs.integers(0, 1000, size=(B, K)).astype(np.int32)
    d = t.copy()
    for b in range(K):
        d[b, b] = (t[b, b] + 1) % 1000
    st = {k: torch.zeros(B, dtype=torch.int32, device=DEV) for k in ("anchor", "accept", "out_len", "round", "done")}
    ctx = torch.full((B,), 100, dtype=torch.int32, device=DEV)
    out = torch.full((B, 64), -1, dtype=torch.int32, device=DEV)
    ora.consensus_commit(B, K, dev(d), dev(t), ctx, st["anchor"], st["accept"], out, st["out_len"], st["round"],
                         st["done"], 64, 100000)
    acc = st["accept"].cpu().numpy()
    assert list(acc) == list(range(K)) + [K]
    assert list(ctx.cpu().numpy()) == [100 + min(k + 1, K) for k in range(K + 1)]
    assert (st["round"].cpu().numpy() == 1).all()


# ------------------------------------------------------------------- rejection accept

@pytest.mark.parametrize("V,mix", [(1000, 0.9), (4096, 0.99), (151936, 0.9)])
def test_rejection_accept_matches_oracle(V, mix):
    B, K, T, seed = 8, 32, 0.8, 4242
    ht, w = synth.lmhead_inputs(12, B * K, 256, V, bf16=False)
    hd = synth.draft_hidden(12, ht, mix=mix, bf16=False)
    seqs = np.arange(B, dtype=np.int32) * 3 + 1
    rnds = np.arange(B, dtype=np.int32)
    # draft logits with their lse, target logits with theirs
    dd = ora.lmhead_desc(B * K, 256, V, ora.F32, K, ora.STREAM_DRAFT, T, seed)
    dt_desc = ora.lmhead_desc(B * K, 256, V, ora.F32, K, ora.STREAM_AR, T, seed, sample=False)
    ws = torch.empty(ora.lmhead_workspace_bytes(dd), dtype=torch.uint8, device=DEV)
    zt_t = torch.empty((B * K, V), dtype=torch.float32, device=DEV)
    zd_t = torch.empty((B * K, V), dtype=torch.float32, device=DEV)
    lt, ld = (torch.empty(B * K, dtype=torch.float32, device=DEV) for _ in range(2))
    tt, dt = (torch.empty(B * K, dtype=torch.int32, device=DEV) for _ in range(2))
    ora.lmhead_argmax(dt_desc, dev(ht), dev(w), dev(seqs), dev(rnds), tt, zt_t, lt, ws)
    ora.lmhead_argmax(dd, dev(hd), dev(w), dev(seqs), dev(rnds), dt, zd_t, ld, ws)
    st = {k: torch.zeros(B, dtype=torch.int32, device=DEV) for k in ("anchor", "accept", "out_len", "done")}
    rnd_t = dev(rnds.copy())
    ctx = torch.full((B,), 500, dtype=torch.int32, device=DEV)
    out = torch.full((B, 64), -1, dtype=torch.int32, device=DEV)
    rws = torch.empty(ora.rejection_workspace_bytes(B, V), dtype=torch.uint8, device=DEV)
    ora.rejection_accept(B, K, V, T, seed, dev(seqs), zd_t, zt_t, ld, lt, dt, ctx, st["anchor"], st["accept"], out,
                         st["out_len"], rnd_t, st["done"], 64, 100000, rws)
    torch.cuda.synchronize()
    acc = st["accept"].cpu().numpy()
    outn = out.cpu().numpy()
    dtn = dt.cpu().numpy().reshape(B, K)
    zdn = zd_t.cpu().numpy().astype(np.float64).reshape(B, K, V)
    ztn = zt_t.cpu().numpy().astype(np.float64).reshape(B, K, V)
    for b in range(B):
        ua = P.uniforms(seed, P.STREAM_ACCEPT, np.arange(K), 0, rnds[b], seqs[b])
        er = -np.log(P.uniforms(seed, P.STREAM_RESID, np.arange(V), 0, rnds[b], seqs[b]))
        k, em = Dc.rejection_accept(zdn[b], ztn[b], dtn[b], T, ua, er)
        assert acc[b] == k, (b, acc[b], k)
        assert list(outn[b, :len(em)]) == em, b
    assert (rnd_t.cpu().numpy() == rnds + 1).all()
    assert (ctx.cpu().numpy() == 500 + np.minimum(acc + 1, K)).all()


# ------------------------------------------------------------------- Philox

def test_philox_words_match_numpy():
    rs = np.random.default_rng(0)
    n = 1000
    ctr = rs.integers(0, 2**63, size=(n, 4), dtype=np.uint64)
    key = rs.integers(0, 2**63, size=2, dtype=np.uint64)
    out = torch.empty((n, 4), dtype=torch.int64, device=DEV)
    ctr_t = torch.from_numpy(ctr.view(np.int64)).to(DEV)
    ora.philox4x64(n, ctr_t, int(key[0]), int(key[1]), out)
    got = out.cpu().numpy().view(np.uint64)
    for i in range(0, n, 97):
        c = [int(x) for x in ctr[i]]
        v = (c[0] | (c[1] << 64) | (c[2] << 128) | (c[3] << 192)) - 1
        v %= 2**256
        bg = np.random.Philox(key=key, counter=np.array([(v >> (64 * j)) & (2**64 - 1) for j in range(4)],
                                                        dtype=np.uint64))
        assert np.array_equal(got[i], bg.random_raw(4))


# ------------------------------------------------------------------- support kernels

@pytest.mark.parametrize("dtype", [ora.BF16, ora.F32])
@pytest.mark.parametrize("M,N,K", [(256, 6144, 4096), (8, 4096, 4096), (45, 1024, 256), (100, 320, 128),
                                   (256, 16384, 256), (40, 16448, 128), (8, 16384, 256), (32, 24576, 192),
                                   (70, 16512, 64)])
@pytest.mark.parametrize("epi", [ora.EPI_STORE, ora.EPI_RESIDUAL, ora.EPI_SWIGLU])
def test_gemm_epilogues(dtype, M, N, K, epi):
    if epi == ora.EPI_SWIGLU and N % 64:
        pytest.skip("SwiGLU needs N % 64 == 0")
    bf = dtype == ora.BF16
    a, w = synth.lmhead_inputs(20, M, K, N, h_std=1.0, w_std=0.02, bf16=bf)
    res = synth.lmhead_inputs(21, M, N, 8, bf16=bf)[0] if epi == ora.EPI_RESIDUAL else None
    z = a.astype(np.float64) @ w.astype(np.float64).T
    if epi == ora.EPI_SWIGLU:
        ncol = N // 2
        g = torch.empty((M, ncol), dtype=torch.bfloat16 if bf else torch.float32, device=DEV)
        packed = torch.empty((N, K), dtype=g.dtype, device=DEV)
        ora.pack_gate_up(ncol, K, dtype, dev(w[:ncol], dtype), dev(w[ncol:], dtype), packed)
        ora.gemm(M, N, K, dtype, dtype, epi, dev(a, dtype), packed, None, g, gemm_ws(M, N, K, dtype, epi))
        gg, uu = z[:, :ncol], z[:, ncol:]
        ref = gg / (1 + np.exp(-gg)) * uu
    else:
        c = torch.empty((M, N), dtype=torch.bfloat16 if bf else torch.float32, device=DEV)
        r_t = dev(res, dtype) if res is not None else None
        if r_t is not None:
            c.copy_(r_t)  # in place: c aliases the residual
        ora.gemm(M, N, K, dtype, dtype, epi, dev(a, dtype), dev(w, dtype), c if r_t is not None else None, c,
                 gemm_ws(M, N, K, dtype, epi))
        g = c
        ref = z + (res.astype(np.float64) if res is not None else 0)
    torch.cuda.synchronize()
    out = g.float().cpu().numpy()
    tol = 1e-5 if not bf else 8e-3  # bf16 output rounding
    assert np.abs(out - ref).max() / np.abs(ref).max() <= tol


@pytest.mark.parametrize("inter", [12288, 8192])
@pytest.mark.parametrize("M", [256, 300, 65, 8, 1000])
def test_gemm_swiglu_fragments_has_the_bits_of_the_row_packed_gemm(M, inter):
    """The register-streamed gate/up + SwiGLU on fragment-packed weights (hidden 4096; 2 x 12288
    gate/up rows take 128x192 tiles of six wavefronts, 2 x 8192 128x256 tiles of four) gives exactly
    the bits of orthrus_gemm(SWIGLU) on the row-interleaved packing, at whole and ragged 128-row
    tiles and at a few rows; both are also checked against float64."""
    H = 4096
    a, w = synth.lmhead_inputs(22, max(M, 1), H, 2 * inter, h_std=1.0, w_std=0.02)
    a = a[:M]
    gate, up = dev(w[:inter], ora.BF16), dev(w[inter:], ora.BF16)
    rows = torch.empty((2 * inter, H), dtype=torch.bfloat16, device=DEV)
    frag = torch.empty_like(rows)
    ora.pack_gate_up(inter, H, ora.BF16, gate, up, rows)
    ora.pack_gate_up_fragments(inter, H, ora.BF16, gate, up, frag)
    a_t = dev(a, ora.BF16)
    ref = torch.full((M, inter), float("nan"), dtype=torch.bfloat16, device=DEV)
    got = torch.full((M, inter), float("nan"), dtype=torch.bfloat16, device=DEV)
    ora.gemm(M, 2 * inter, H, ora.BF16, ora.BF16, ora.EPI_SWIGLU, a_t, rows, None, ref,
             gemm_ws(M, 2 * inter, H, ora.BF16, ora.EPI_SWIGLU))
    ora.gemm_swiglu_fragments(M, inter, H, ora.BF16, a_t, frag, got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    z = a.astype(np.float64) @ w.astype(np.float64).T
    gg, uu = z[:, :inter], z[:, inter:]
    want = gg / (1 + np.exp(-gg)) * uu
    assert np.abs(got.float().cpu().numpy() - want).max() / np.abs(want).max() <= 8e-3
    if M == 8:  # zero rows: nothing is launched or written
        before = got.clone()
        ora.gemm_swiglu_fragments(0, inter, H, ora.BF16, a_t, frag, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), before.view(torch.int16))


@pytest.mark.parametrize("dtype", [ora.BF16, ora.F32])
@pytest.mark.parametrize("N", [1024, 16384])
def test_gemm_row_invariance(dtype, N):
    a, w = synth.lmhead_inputs(22, 256, 4096, N, bf16=(dtype == ora.BF16))
    outs = []
    for m in (256, 64, 32, 1):
        c = torch.empty((m, N), dtype=torch.float32, device=DEV)
        ora.gemm(m, N, 4096, dtype, ora.F32, ora.EPI_STORE, dev(a[:m], dtype), dev(w, dtype), None, c,
                 gemm_ws(m, N, 4096, dtype, ora.EPI_STORE))
        outs.append(c.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o, outs[0][: o.shape[0]])


@pytest.mark.parametrize("dtype", [ora.BF16, ora.F32])
@pytest.mark.parametrize("hidden,offset", [(4096, 0), (256, 0), (1004, 0), (8200, 0), (4096, 1)])
def test_rmsnorm(dtype, hidden, offset):
    """Register-resident 16-byte path (aligned rows up to 1024 chunks per row), and the scalar
    path for ragged widths, very wide rows and tensors not 16-byte aligned (offset)."""
    bf = dtype == ora.BF16
    rows = 33
    x = synth.lmhead_inputs(23, rows, hidden, 8, h_std=3.0, bf16=bf)[0]
    g = (1 + 0.1 * np.random.default_rng(1).standard_normal(hidden)).astype(np.float32)
    tdt = torch.bfloat16 if bf else torch.float32
    xs = torch.zeros(rows * hidden + offset, dtype=tdt, device=DEV)
    xs[offset:] = dev(x, dtype).reshape(-1)
    ys = torch.empty(rows * hidden + offset, dtype=tdt, device=DEV)
    y = ys[offset:]
    ora.rmsnorm(rows, hidden, dtype, xs[offset:], dev(g), 1e-6, y)
    ref = M.rmsnorm(x.astype(np.float64), g.astype(np.float64), 1e-6)
    err = np.abs(y.float().cpu().numpy().reshape(rows, hidden) - ref).max() / np.abs(ref).max()
    assert err <= (4e-3 if bf else 1e-6)


@pytest.mark.parametrize("paged", [True, False])
@pytest.mark.parametrize("dtype", [ora.BF16, ora.F32])
def test_rope_kv_write(paged, dtype):
    B, K, Hq, Hkv, D, page = 3, 32, 8, 2, 128, 16
    bf = dtype == ora.BF16
    ctx = np.array([0, 77, 5000], np.int32)
    qkv = synth.lmhead_inputs(24, B * K, (Hq + 2 * Hkv) * D, 8, bf16=bf)[0]
    maxpos = 8192
    table = torch.empty((maxpos, D // 2, 2), dtype=torch.float32, device=DEV)
    ora.rope_table(maxpos, D, 1e6, table)
    tdt = torch.bfloat16 if bf else torch.float32
    q_out = torch.empty((B * K, Hq * D), dtype=tdt, device=DEV)
    maxp = (5000 + K) // page + 1
    perm = np.random.default_rng(0).permutation(B * maxp).astype(np.int32).reshape(B, maxp)
    if paged:
        kd = torch.full((B * maxp, Hkv, page, D), float("nan"), dtype=tdt, device=DEV)
        vd = torch.full_like(kd, float("nan"))
        pt = dev(perm)
    else:
        kd = torch.empty((B, K, Hkv, D), dtype=tdt, device=DEV)
        vd = torch.empty_like(kd)
        pt = None
    ora.rope_kv_write(B, K, Hq, Hkv, D, page, maxp, dtype, dev(qkv, dtype), table, maxpos, dev(ctx), pt, q_out, kd, vd)
    torch.cuda.synchronize()
    x = qkv.astype(np.float64).reshape(B, K, Hq + 2 * Hkv, D)
    pos = ctx[:, None] + np.arange(K)[None]
    rq = M.rope(x[:, :, :Hq], pos[:, :, None], 1e6)
    rk = M.rope(x[:, :, Hq:Hq + Hkv], pos[:, :, None], 1e6)
    rv = x[:, :, Hq + Hkv:]
    tol = 4e-3 if bf else 1e-6
    assert np.abs(q_out.float().cpu().numpy().reshape(rq.shape) - rq).max() <= tol * np.abs(rq).max()
    kdn, vdn = kd.float().cpu().numpy(), vd.float().cpu().numpy()
    for b in range(B):
        for s in range(K):
            p = pos[b, s]
            if paged:
                gk, gv = kdn[perm[b, p // page], :, p % page], vdn[perm[b, p // page], :, p % page]
            else:
                gk, gv = kdn[b, s], vdn[b, s]
            assert np.abs(gk - rk[b, s]).max() <= tol * np.abs(rk).max()
            assert np.array_equal(gv, rv[b, s].astype(np.float32)) or bf and np.abs(gv - rv[b, s]).max() < 1e-2


def test_embed_block_modes():
    V, H = 4096, 256
    E = synth.lmhead_inputs(25, V, H, 8, bf16=False)[0]
    anchor = np.array([5, 17], np.int32)
    toks = np.array([[1, 2, 3, 4], [9, 8, 7, 6]], np.int32)
    Et = dev(E)
    x = torch.empty((8, H), dtype=torch.float32, device=DEV)
    ora.embed_block(2, 4, H, ora.F32, Et, dev(anchor), None, 0, 0, V - 1, x)       # draft
    ref = np.stack([E[5], E[V - 1], E[V - 1], E[V - 1], E[17], E[V - 1], E[V - 1], E[V - 1]])
    assert np.array_equal(x.cpu().numpy(), ref)
    ora.embed_block(2, 4, H, ora.F32, Et, dev(anchor), dev(toks), 4, 0, V - 1, x)  # verify
    ref = np.stack([E[5], E[1], E[2], E[3], E[17], E[9], E[8], E[7]])
    assert np.array_equal(x.cpu().numpy(), ref)
    ora.embed_block(2, 2, H, ora.F32, Et, None, dev(toks), 4, 1, V - 1, x[:4])    # prefill chunk
    ref = np.stack([E[2], E[3], E[8], E[7]])
    assert np.array_equal(x[:4].cpu().numpy(), ref)


def test_gemm_is_repeatable_and_large_k_accurate():
    """Deterministic: three calls give the same bits (the k-quarter partials are added in a fixed order)."""
    M, N, K = 256, 4096, 12288
    a, w = synth.lmhead_inputs(26, M, K, N)
    outs = []
    for _ in range(3):
        c = torch.empty((M, N), dtype=torch.float32, device=DEV)
        ora.gemm(M, N, K, ora.BF16, ora.F32, ora.EPI_STORE, dev(a, ora.BF16), dev(w, ora.BF16), None, c,
                 gemm_ws(M, N, K, ora.BF16, ora.EPI_STORE))
        outs.append(c.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    ref = a[:16].astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(outs[0][:16] - ref).max() <= 1e-5 * np.abs(ref).max()


def test_zero_sized_calls_launch_nothing():
    """Empty batches and zero-row calls return OK and leave every output untouched."""
    bf = torch.bfloat16
    i32 = lambda v=7: torch.full((4,), v, dtype=torch.int32, device=DEV)
    a = torch.zeros((1, 256), dtype=bf, device=DEV)
    w = torch.zeros((512, 256), dtype=bf, device=DEV)
    c = torch.full((1, 512), 3.0, dtype=bf, device=DEV)
    ora.gemm(0, 512, 256, ora.BF16, ora.BF16, ora.EPI_STORE, a, w, None, c, gemm_ws(0, 512, 256, ora.BF16, ora.EPI_STORE))
    y = torch.full((1, 256), 3.0, dtype=bf, device=DEV)
    ora.rmsnorm(0, 256, ora.BF16, a, torch.ones(256, dtype=torch.float32, device=DEV), 1e-6, y)
    d = ora.lmhead_desc(0, 256, 512, ora.BF16, 1)
    tok = i32()
    ora.lmhead_argmax(d, a, w, i32(0), i32(0), tok, None, None,
                      torch.zeros(max(16, ora.lmhead_workspace_bytes(d)), dtype=torch.uint8, device=DEV))
    desc = ora.attn_desc(0, 8, 2, 128, 32, 16, 4, 64)
    ws = torch.zeros(max(16, ora.attn_workspace_bytes(desc)), dtype=torch.uint8, device=DEV)
    q = torch.zeros((1, 32, 8, 128), dtype=bf, device=DEV)
    pages = torch.zeros((4, 2, 16, 128), dtype=bf, device=DEV)
    blk = torch.zeros((1, 32, 2, 128), dtype=bf, device=DEV)
    out = torch.full((1, 32, 8, 128), 5.0, dtype=torch.float32, device=DEV)
    pt = torch.zeros((1, 4), dtype=torch.int32, device=DEV)
    ora.draft_attn(desc, q, pages, pages, pt, i32(0), blk, blk, out, ws)
    ora.verify_attn(desc, q, pages, pages, pt, i32(0), out, ws)
    st = [i32() for _ in range(7)]
    outs = torch.full((1, 8), 7, dtype=torch.int32, device=DEV)
    ora.consensus_commit(0, 32, st[0], st[1], st[2], st[3], st[4], outs, st[5], st[6], i32(), 8, 64)
    lse = torch.zeros(4, dtype=torch.float32, device=DEV)
    fill = [i32() for _ in range(3)]
    ora.draft_fill(0, 32, 256, 512, ora.BF16, a, w, lse, i32(), 511, 15, fill[0], fill[1])
    ora.draft_merge(0, 32, i32(), i32(), i32(), fill[2])
    torch.cuda.synchronize()
    assert bool((c == 3.0).all()) and bool((y == 3.0).all()) and bool((tok == 7).all())
    assert bool((out == 5.0).all()) and bool((outs == 7).all()) and all(bool((t == 7).all()) for t in st)
    assert all(bool((t == 7).all()) for t in fill)


@pytest.mark.parametrize("dtype", [ora.BF16, ora.F32])
@pytest.mark.parametrize("M,N,K", [(256, 4096, 4096), (8, 4096, 12288), (45, 1024, 256), (17, 320, 128)])
def test_gemm_residual_rmsnorm_has_the_bits_of_the_two_calls(dtype, M, N, K):
    """The fused residual GEMM + RMSNorm (one pass over the rows where the shapes allow, the two calls
    in sequence otherwise) gives exactly the bits of orthrus_gemm(RESIDUAL) then orthrus_rmsnorm."""
    bf = dtype == ora.BF16
    a, w = synth.lmhead_inputs(27, M, K, N, h_std=1.0, w_std=0.02, bf16=bf)
    x0 = synth.lmhead_inputs(28, M, N, 8, bf16=bf)[0]
    gain = dev(np.random.default_rng(29).uniform(0.5, 1.5, N).astype(np.float32))
    ws = gemm_ws(M, N, K, dtype, ora.EPI_RESIDUAL)
    tdt = torch.bfloat16 if bf else torch.float32
    xs, ys = dev(x0, dtype), torch.empty((M, N), dtype=tdt, device=DEV)
    ora.gemm(M, N, K, dtype, dtype, ora.EPI_RESIDUAL, dev(a, dtype), dev(w, dtype), xs, xs, ws)
    ora.rmsnorm(M, N, dtype, xs, gain, 1e-6, ys)
    xf, yf = dev(x0, dtype), torch.empty((M, N), dtype=tdt, device=DEV)
    ora.gemm_residual_rmsnorm(M, N, K, dtype, dev(a, dtype), dev(w, dtype), xf, gain, 1e-6, yf, ws)
    torch.cuda.synchronize()
    assert torch.equal(xs, xf) and torch.equal(ys, yf)
    # and the result is the residual update and the norm
    z = x0.astype(np.float64) + a.astype(np.float64) @ w.astype(np.float64).T
    ref = z / np.sqrt((z ** 2).mean(1, keepdims=True) + 1e-6) * gain.cpu().numpy()
    out = yf.float().cpu().numpy()
    assert np.abs(out - ref).max() / np.abs(ref).max() <= (2e-2 if bf else 1e-5)


@pytest.mark.parametrize("dtype", [ora.BF16, ora.F32])
@pytest.mark.parametrize("paged", [True, False])
@pytest.mark.parametrize("B,H", [(8, 4096), (2, 512), (3, 192)])
def test_gemm_rope_kv_write_has_the_bits_of_the_two_calls(dtype, paged, B, H):
    """The fused QKV projection + RoPE + K/V write (row by row from the k-quarter partials where the
    GEMM splits K, the two calls through qkv otherwise) gives exactly the bits of orthrus_gemm(STORE)
    followed by orthrus_rope_kv_write: q, the written K/V slots, and untouched slots left as they were."""
    K, Hq, Hkv, D, page = 32, 8, 2, 128, 16
    bf = dtype == ora.BF16
    tdt = torch.bfloat16 if bf else torch.float32
    N = (Hq + 2 * Hkv) * D
    a, w = synth.lmhead_inputs(30, B * K, H, N, h_std=1.0, w_std=0.05, bf16=bf)
    ctx = (np.arange(B, dtype=np.int32) * 611) % 3000
    maxpos = 4096
    table = torch.empty((maxpos, D // 2, 2), dtype=torch.float32, device=DEV)
    ora.rope_table(maxpos, D, 1e6, table)
    maxp = (3000 + K) // page + 1
    pt = dev(np.random.default_rng(1).permutation(B * maxp).astype(np.int32).reshape(B, maxp)) if paged else None
    ws = gemm_ws(B * K, N, H, dtype, ora.EPI_STORE)

    def dests():
        shape = (B * maxp, Hkv, page, D) if paged else (B, K, Hkv, D)
        return (torch.empty((B * K, Hq * D), dtype=tdt, device=DEV), torch.full(shape, 7.0, dtype=tdt, device=DEV),
                torch.full(shape, 7.0, dtype=tdt, device=DEV))
    qs, ks, vs = dests()
    qkv = torch.empty((B * K, N), dtype=tdt, device=DEV)
    ora.gemm(B * K, N, H, dtype, dtype, ora.EPI_STORE, dev(a, dtype), dev(w, dtype), None, qkv, ws)
    ora.rope_kv_write(B, K, Hq, Hkv, D, page, maxp, dtype, qkv, table, maxpos, dev(ctx), pt, qs, ks, vs)
    qf, kf, vf = dests()
    ora.gemm_rope_kv_write(B, K, Hq, Hkv, D, page, maxp, H, dtype, dev(a, dtype), dev(w, dtype), table, maxpos,
                           dev(ctx), pt, torch.empty_like(qkv), qf, kf, vf, ws)
    torch.cuda.synchronize()
    assert torch.equal(qs, qf) and torch.equal(ks, kf) and torch.equal(vs, vf)
