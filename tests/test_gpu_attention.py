"""GPU parity: draft/verify attention (C ABI) against the CPU oracle.

Tolerance (attention outputs, bf16 inputs, fp32 accumulate): per (sequence, query head)
max|gpu - oracle| / max|oracle| <= 2e-3.  fp32 path: <= 2e-5.  Invariances that the kernel
design promises are checked bit for bit: page order, and verify slot j at context n == a
one-row verify at context n + j (the AR step).
"""
import numpy as np
import pytest
import torch

import orthrus_round_amd as ora
import synth
from oracle import model as M

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == ora.BF16:
        t = t.to(torch.bfloat16)
    return t.to(DEV)


def run_attn(inp, Hq, Hkv, D, K, draft, dtype=ora.BF16, out_dtype=ora.F32, kv_chunk=0, max_ctx=None,
             page_table=None, pages=None):
    B = len(inp.ctx)
    pt = inp.page_table if page_table is None else page_table
    pk, pv = (inp.pages_k, inp.pages_v) if pages is None else pages
    maxp = pt.shape[1]
    mc = max_ctx or maxp * inp.page_size
    desc = ora.attn_desc(B, Hq, Hkv, D, K, inp.page_size, maxp, mc, kv_chunk, dtype, out_dtype, inp.scale)
    wsb = ora.attn_workspace_bytes(desc)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
    out = torch.full((B, K, Hq, D), float("nan"), dtype=torch.float32 if out_dtype == ora.F32 else torch.bfloat16,
                     device=DEV)
    q = dev(inp.q[:, :K], dtype)
    args = (desc, q, dev(pk, dtype), dev(pv, dtype), dev(pt, None), dev(inp.ctx, None))
    if draft:
        ora.draft_attn(*args, dev(inp.k_blk[:, :K], dtype), dev(inp.v_blk[:, :K], dtype), out, ws)
    else:
        ora.verify_attn(*args, out, ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def oracle_attn(inp, b, K, draft, heads=None):
    n = int(inp.ctx[b])
    k, v = inp.kv[b]
    q = inp.q[b, :K].astype(np.float64)
    if heads is not None:
        G = inp.q.shape[2] // k.shape[1]
        q = q[:, heads]
    if draft:
        kc, vc = k[:n].astype(np.float64), v[:n].astype(np.float64)
        kb, vb = inp.k_blk[b, :K].astype(np.float64), inp.v_blk[b, :K].astype(np.float64)
        if heads is not None:
            hk = sorted({h // G for h in heads})
            assert len(hk) == 1
            kc, vc, kb, vb = kc[:, hk], vc[:, hk], kb[:, hk], vb[:, hk]
        return M.draft_attention(q, kc, vc, kb, vb, inp.scale)
    ka, va = k[: n + K].astype(np.float64), v[: n + K].astype(np.float64)
    if heads is not None:
        hk = sorted({h // G for h in heads})
        ka, va = ka[:, hk], va[:, hk]
    return M.verify_attention(q, ka, va, n, inp.scale)


def normwise(g, o):
    """max |g - o| / max |o| per query head (axis 1 of [K, H, D])."""
    return (np.abs(g - o).max(axis=(0, 2)) / np.abs(o).max(axis=(0, 2))).max()


# ------------------------------------------------------------------- single layer, Qwen3-1.7B shapes

@pytest.mark.parametrize("n", [1024, 4096, 8192])
@pytest.mark.parametrize("draft", [True, False])
def test_qwen3_1p7b_layer(n, draft):
    inp = synth.attn_inputs(2, np.array([n]), 16, 8, 128)
    g = run_attn(inp, 16, 8, 128, 32, draft)
    o = oracle_attn(inp, 0, 32, draft)
    err = normwise(g[0], o)
    print(f"n={n} draft={draft} normwise err {err:.2e}")
    assert err <= 2e-3


@pytest.mark.parametrize("ctx,K,chunk", [([0, 1, 31, 33], 32, 64), ([100, 7, 64, 200], 5, 64),
                                         ([3, 300, 129, 40], 32, 0), ([0, 0, 1, 2], 1, 32)])
@pytest.mark.parametrize("draft", [True, False])
def test_ragged_tails_and_chunks(ctx, K, chunk, draft):
    inp = synth.attn_inputs(3, np.array(ctx), 8, 2, 128, block=32)
    g = run_attn(inp, 8, 2, 128, K, draft, kv_chunk=chunk)
    for b in range(len(ctx)):
        o = oracle_attn(inp, b, K, draft)
        assert normwise(g[b], o) <= 2e-3, (b, ctx[b])


@pytest.mark.parametrize("draft", [True, False])
def test_fp32_path_head64_group2(draft):
    ctx = np.array([63, 0, 95, 170])
    inp = synth.attn_inputs(4, ctx, 4, 2, 64, block=32, bf16=False, q_scale=1.0)
    inp.scale = 1.0 / 8.0
    g = run_attn(inp, 4, 2, 64, 32, draft, dtype=ora.F32, out_dtype=ora.F32, kv_chunk=64)
    for b in range(len(ctx)):
        o = oracle_attn(inp, b, 32, draft)
        assert normwise(g[b], o) <= 2e-5


def test_bf16_output():
    inp = synth.attn_inputs(5, np.array([700, 1500]), 32, 8, 128)
    g = run_attn(inp, 32, 8, 128, 32, False, out_dtype=ora.BF16, kv_chunk=512)
    for b in range(2):
        assert normwise(g[b], oracle_attn(inp, b, 32, False)) <= 4e-3  # + one bf16 rounding of the output


# ------------------------------------------------------------------- batched, paged, ragged at Qwen3-8B shapes

@pytest.fixture(scope="module")
def qwen3_8b_batch():
    ctx = synth.ragged_lengths(3, 16, 512, 16384)
    return synth.attn_inputs(3, ctx, 32, 8, 128)


def oracle_attn_all_heads(inp, b, K, draft):
    """Every query head of sequence b in the oracle's matrix-product form (pinned to the row form
    and to SDPA on the CPU)."""
    n = int(inp.ctx[b])
    k, v = inp.kv[b]
    q = inp.q[b, :K].astype(np.float64)
    if draft:
        kk = np.concatenate([k[:n], inp.k_blk[b, :K]]).astype(np.float64)
        vv = np.concatenate([v[:n], inp.v_blk[b, :K]]).astype(np.float64)
        allowed = np.ones((K, n + K), bool)
    else:
        kk, vv = k[: n + K].astype(np.float64), v[: n + K].astype(np.float64)
        allowed = np.ones((K, n + K), bool)
        allowed[:, n:] = np.tril(np.ones((K, K), bool))
    return M.grouped_attention(q, kk, vv, allowed, inp.scale)


@pytest.mark.parametrize("chunk", [1024, 1280])
@pytest.mark.parametrize("draft", [True, False])
def test_qwen3_8b_batched_paged_ragged(qwen3_8b_batch, draft, chunk):
    """Every sequence, every query head (all 8 kv heads) of the batched paged workload, at 1280-key
    chunks (the launch the benchmark times) and at 1024."""
    inp = qwen3_8b_batch
    g = run_attn(inp, 32, 8, 128, 32, draft, kv_chunk=chunk)
    worst = 0.0
    for b in range(16):
        o = oracle_attn_all_heads(inp, b, 32, draft)
        err = normwise(g[b], o)
        worst = max(worst, err)
        assert err <= 2e-3, (b, err)
    print(f"draft={draft} worst normwise err over 16 x 32 heads {worst:.2e}")


def test_page_order_is_invisible(qwen3_8b_batch):
    inp = qwen3_8b_batch
    a = run_attn(inp, 32, 8, 128, 32, False, kv_chunk=1024)
    pk, pv, pt = synth.page_layout(inp.kv, 8, 128, 16, 99, 7)
    b = run_attn(inp, 32, 8, 128, 32, False, kv_chunk=1024, page_table=pt, pages=(pk, pv))
    assert np.array_equal(a, b)


# ------------------------------------------------------------------- bitwise invariances

@pytest.mark.parametrize("dtype", [ora.BF16, ora.F32])
def test_verify_row_equals_one_row_ar_step(dtype):
    """Slot j of a verify pass at context n gives the same bits as a 1-row pass at n + j."""
    n, K = 1000, 32
    bf = dtype == ora.BF16
    inp = synth.attn_inputs(6, np.array([n]), 32, 8, 128, bf16=bf)
    full = run_attn(inp, 32, 8, 128, K, False, dtype=dtype, kv_chunk=256)
    for j in [0, 5, 23, 31]:
        step = synth.AttnInputs(inp.q[:, j:j + 1], inp.kv, inp.k_blk, inp.v_blk, np.array([n + j], np.int32),
                                inp.scale, inp.page_size, inp.pages_k, inp.pages_v, inp.page_table)
        one = run_attn(step, 32, 8, 128, 1, False, dtype=dtype, kv_chunk=256)
        assert np.array_equal(one[0, 0], full[0, j]), j


@pytest.mark.parametrize("draft", [True, False])
def test_more_than_64_sequences(draft):
    """70 ragged sequences (the grid's slots are matched to the existing chunks 64 sequences at a
    time), several chunks each, one of them past the cache capacity: every sequence against the
    oracle, the overflowing one all NaN."""
    ctx = synth.ragged_lengths(11, 70, 0, 200)
    ctx[66] = 230  # n + K = 262 > max_ctx = 256
    inp = synth.attn_inputs(11, ctx, 8, 2, 128, block=32)
    g = run_attn(inp, 8, 2, 128, 32, draft, kv_chunk=64, max_ctx=256)
    assert np.isnan(g[66]).all()
    for b in range(70):
        if b == 66:
            continue
        o = oracle_attn(inp, b, 32, draft)
        assert normwise(g[b], o) <= 2e-3, (b, int(ctx[b]))


def test_capacity_overflow_marks_rows_nan():
    inp = synth.attn_inputs(7, np.array([40, 10]), 8, 2, 128, block=32)
    g = run_attn(inp, 8, 2, 128, 32, False, max_ctx=64)
    assert np.isnan(g[0]).all() and not np.isnan(g[1]).any()
