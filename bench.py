"""Benchmark: one Orthrus decode round (draft pass + verify pass + consensus/commit) per step
on a random-init Qwen3-8B-width decoder truncated to 8 layers, batch 8, 4096-token prompts,
bf16, greedy -- synthetic seeded inputs, one MI355X.

Prints ONE JSON line: accepted (committed) tokens/s over the timed rounds, round latency,
the roofline record of the round's dominant kernel (timed live with HIP events on the
stream it runs on), the attention roofline at the batched paged Qwen3-8B attention workload,
the AR-step yardstick, and the CPU oracle's throughput on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--batch", type=int, default=8)
    p.add_argument("--prompt", type=int, default=4096)
    p.add_argument("--layers", type=int, default=8)
    p.add_argument("--precision", default="bf16", choices=["bf16", "fp32"])
    p.add_argument("--kv-chunk", type=int, default=640)
    p.add_argument("--attn-chunk", type=int, default=1536,
                   help="kv_chunk of the batched attention measurement (16 ragged sequences up to 16K keys)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-attn", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip the block sweep and trajectory match")
    p.add_argument("--counters", action="store_true",
                   help="hardware-counter mode: prefill, the timed rounds and the calibration copy only")
    p.add_argument("--match-tokens", type=int, default=64)
    p.add_argument("--control-chunk", type=int, default=1024,
                   help="kv_chunk of the divergence control runs (another key summation order)")
    return p.parse_args()


_FLUSH = None


def flush_caches():
    """Evict L2 and the 256 MiB infinity cache by READING 512 MiB (a write would leave dirty
    lines whose write-back would then compete with the next timed kernel)."""
    global _FLUSH
    import torch
    if _FLUSH is None:
        _FLUSH = torch.zeros(128 * 2**20, dtype=torch.float32, device="cuda")
    _FLUSH.sum()


def alternating_ms(fns, replays=5):
    """Average duration of one launch over back-to-back launches of fns[0], fns[1], ... captured
    in a HIP graph and replayed, timed with one pair of HIP events on the current stream."""
    import torch
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    g.replay()
    torch.cuda.synchronize()
    flush_caches()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    del g
    return s.elapsed_time(e) / (replays * len(fns))


def layer_sweep_ms(fn, n_layers, sweeps=4):
    """Average duration of one launch of `fn(layer)` over back-to-back launches that walk every
    layer's weights and caches in turn (as the round does).  The layers' operands together exceed
    the 256 MiB infinity cache, so each launch streams its own from HBM."""
    return alternating_ms([(lambda i=i: fn(i)) for i in range(n_layers)], sweeps)


def kernel_table(dec, ctx_np):
    """Per-launch HIP-event times of each kernel class of the round at its in-round shapes."""
    import orthrus_round_amd._lib as L
    s, B, K = dec.shape, dec.B, dec.K
    M = B * K
    H, D, Hq, Hkv, I, V = s.hidden, s.head_dim, s.q_heads, s.kv_heads, s.inter, s.vocab
    dt = dec.dt
    esz = 2 if dt == L.BF16 else 4
    Ly = dec.layers
    nl = len(Ly)
    desc = dec._attn_desc(B, K)
    ws = dec._ws(desc)
    n_sum = int(ctx_np.sum())
    tab = {}

    def add(name, fn, per_round, bytes_, flops):
        ms = layer_sweep_ms(fn, nl)
        tab[name] = dict(ms=ms, per_round=per_round, bytes=bytes_, flops=flops)

    add("gemm_qkv_rope_kv", lambda i: L.gemm_rope_kv_write(B, K, Hq, Hkv, D, dec.page, dec.max_pages, H, dt, dec.a,
                                                          Ly[i]["qkv_ar"], dec.rope, dec.max_pos, dec.ctx_len, None,
                                                          dec.qkv, dec.q, dec.k_blk, dec.v_blk, dec.gemm_ws),
        2 * s.layers, (dec.nqkv * H + M * H + M * dec.nqkv) * esz, 2 * M * dec.nqkv * H)
    add("gemm_o_residual_rmsnorm", lambda i: L.gemm_residual_rmsnorm(M, H, Hq * D, dt, dec.o, Ly[i]["o_ar"], dec.x,
                                                                     Ly[i]["mlp_norm"], s.eps, dec.a, dec.gemm_ws),
        2 * s.layers, (H * Hq * D + M * Hq * D + 3 * M * H) * esz, 2 * M * H * Hq * D)
    add("gemm_gate_up_swiglu", lambda i: L.gemm(M, 2 * I, H, dt, dt, L.EPI_SWIGLU, dec.a, Ly[i]["gate_up"], None, dec.h, dec.gemm_ws),
        2 * s.layers, (2 * I * H + M * H + M * I) * esz, 2 * M * 2 * I * H)
    add("gemm_down_residual_rmsnorm", lambda i: L.gemm_residual_rmsnorm(M, H, I, dt, dec.h, Ly[i]["down"], dec.x,
                                                                        Ly[i]["attn_norm"], s.eps, dec.a, dec.gemm_ws),
        2 * s.layers, (H * I + M * I + 3 * M * H) * esz, 2 * M * H * I)
    kv_b = Hkv * D * 2 * esz  # K and V bytes per key
    qo_b = 2 * M * Hq * D * esz
    add("attn_draft", lambda i: L.draft_attn(desc, dec.q, dec.k_pages[i], dec.v_pages[i], dec.page_table, dec.ctx_len,
                                           dec.k_blk, dec.v_blk, dec.o, ws),
        s.layers, n_sum * kv_b + M * kv_b + qo_b, 4 * Hq * D * K * (n_sum + B * K))
    add("attn_verify", lambda i: L.verify_attn(desc, dec.q, dec.k_pages[i], dec.v_pages[i], dec.page_table,
                                             dec.ctx_len, dec.o, ws),
        s.layers, (n_sum + M) * kv_b + qo_b, 4 * Hq * D * K * (n_sum + B * K))
    d = L.lmhead_desc(M, H, V, dt, K)
    add("lmhead_argmax", lambda i: L.lmhead_argmax(d, dec.a, dec.lm_head, dec.seq_id, dec.round, dec.target.view(-1),
                                                 None, None, dec.lm_ws),
        2, (V * H + M * H) * esz, 2 * M * V * H)
    add("rmsnorm", lambda i: L.rmsnorm(M, H, dt, dec.x, Ly[i]["attn_norm"], s.eps, dec.a), 2,
        2 * M * H * esz, 0)
    return tab


# The sources each timed kernel is compiled from (orthrus_round_amd/csrc/).
KERNEL_SOURCES = {
    "gemm": ("gemm.hip", "gemm_core.hpp", "common.hpp"),
    "attn": ("attn.hip", "common.hpp"),
    "lmhead": ("lmhead.hip", "gemm_core.hpp", "common.hpp"),
    "rmsnorm": ("elementwise.hip", "common.hpp"),
}


def source_digest(kernel):
    """sha256 over the sources of one timed kernel, in the order KERNEL_SOURCES lists them."""
    import hashlib
    h = hashlib.sha256()
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "orthrus_round_amd", "csrc")
    for name in KERNEL_SOURCES[kernel.split("_")[0]]:
        with open(os.path.join(root, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(name):
    """HBM bytes per launch of a kernel from the committed FETCH_SIZE/WRITE_SIZE profile
    (profiles/traffic.json, counts scaled by a plain 256 MiB copy), or None when the kernel's
    sources changed after the counters were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
    try:
        with open(path) as f:
            prof = json.load(f)
    except OSError:
        return None
    rec = prof.get("bench_kernels", {}).get(name)
    if rec is None or rec.get("source_sha256") != source_digest(name):
        return None
    return rec["bytes"]


def roofline_of(name, rec, bound="hbm"):
    traffic = profiled_traffic(name)
    if bound == "hbm":
        ach = rec["bytes"] / (rec["ms"] * 1e-3) / 1e9
        return {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic, "bytes_per_launch": rec["bytes"],
                "ms_per_launch": round(rec["ms"], 5)}
    ach = rec["flops"] / (rec["ms"] * 1e-3) / 1e12
    return {"kernel": name, "bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": traffic, "flops_per_launch": rec["flops"],
            "ms_per_launch": round(rec["ms"], 5)}


def attention_roofline(kv_chunk):
    """Draft + verify attention at batch 16, 32Q/8KV heads, D 128, ragged contexts 512..16384,
    16-token pages in a seeded random order (bf16 in, fp32 out).  Launches alternate between two
    copies of the paged cache (449 MB each, together 3.5x the 256 MiB infinity cache), so every
    launch streams its keys and values from HBM; the per-launch time includes the chunk combine."""
    import torch
    import orthrus_round_amd as ora
    import synth
    ctx = synth.ragged_lengths(3, 16, 512, 16384)
    inp = synth.attn_inputs(3, ctx, 32, 8, 128)
    dv = lambda x, bf=True: (torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16) if bf
                             else torch.from_numpy(np.ascontiguousarray(x))).cuda()
    maxp = inp.page_table.shape[1]
    desc = ora.attn_desc(16, 32, 8, 128, 32, 16, maxp, maxp * 16, kv_chunk, ora.BF16, ora.F32, 1.0)
    ws = torch.empty(max(16, ora.attn_workspace_bytes(desc)), dtype=torch.uint8, device="cuda")
    q = dv(inp.q)
    pages = [(dv(np.nan_to_num(inp.pages_k)), dv(np.nan_to_num(inp.pages_v)))]
    pages.append((pages[0][0].clone(), pages[0][1].clone()))
    pt, cl = dv(inp.page_table, False), dv(inp.ctx, False)
    kb, vb = dv(inp.k_blk), dv(inp.v_blk)
    out = torch.empty((16, 32, 32, 128), dtype=torch.float32, device="cuda")
    res = {}
    n_sum = int(ctx.sum())
    for name, mk, keys in [
        ("draft", lambda pk, pv: (lambda: ora.draft_attn(desc, q, pk, pv, pt, cl, kb, vb, out, ws)), n_sum + 16 * 32),
        ("verify", lambda pk, pv: (lambda: ora.verify_attn(desc, q, pk, pv, pt, cl, out, ws)), n_sum + 16 * 32),
    ]:
        byts = keys * 8 * 128 * 2 * 2 + q.numel() * 2 + out.numel() * 4
        ms = alternating_ms([mk(pk, pv) for pk, pv in pages])
        res[name] = {"ms": round(ms, 5), "bytes": byts, "GBs": round(byts / ms / 1e6, 1),
                     "frac": round(byts / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del pages
    torch.cuda.empty_cache()
    return {"workload": "batch 16, 32Q/8KV, D128, ctx U[512,16384], 16-token paged random order, bf16->fp32, "
                        "launches alternating between two copies of the cache (each streamed from HBM), "
                        "attention + chunk combine per launch",
            "sum_ctx": n_sum, "kv_chunk": kv_chunk, **res}


def cpu_baseline(W, shape, prompts_np, tokens_per_round_seq, kv_seed=9):
    """The CPU oracle (float64, batched BLAS rows) on a bounded sample: one draft + verify
    round of ONE sequence through layer 0 of the 8 (plus the LM head), over a synthetic
    4095-token AR cache; scaled to the whole model as layers x (layer time) + LM head."""
    import dataclasses
    from oracle import decode as Dc
    from oracle import model as M
    import synth
    one = dataclasses.replace(shape, layers=1)
    keys = ["embed", "lm_head", "final_norm"] + [k for k in W if k.startswith("0.")]
    Wt = M.Weights({k: W[k] for k in keys}, one)
    P = prompts_np.shape[1]
    cache = Dc.Cache(one, P + 64, np.float64)
    rs = np.random.default_rng(kv_seed)
    cache.k[0][: P - 1] = rs.standard_normal((P - 1, one.kv_heads, one.head_dim))
    cache.v[0][: P - 1] = rs.standard_normal((P - 1, one.kv_heads, one.head_dim))
    cache.n = P - 1
    anchor = int(prompts_np[0, -1])
    nthreads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    zd = Dc.draft_pass(Wt, cache, [anchor] + [one.mask_id] * 31, rowwise=False)
    t1 = time.perf_counter()
    zt = Dc.ar_pass(Wt, cache, [anchor] + list(M.argmax_lowest(zd)[:31]), rowwise=False)
    t2 = time.perf_counter()
    # LM head share: time it alone to separate it from the layer
    h = np.ones((32, one.hidden))
    t3 = time.perf_counter()
    M.lm_logits(Wt, h, rowwise=False)
    t4 = time.perf_counter()
    lm = t4 - t3
    layer = (t2 - t0) - 2 * lm
    full_round = shape.layers * layer + 2 * lm
    value = tokens_per_round_seq / full_round
    return {"value": round(value, 4), "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": (f"float64 NumPy oracle, one round (draft+verify) of 1 sequence through layer 0 plus the LM "
                       f"head over a synthetic {P - 1}-token cache; measured {t2 - t0:.2f}s, scaled to "
                       f"{shape.layers} layers = {full_round:.2f}s per round at the GPU's "
                       f"{tokens_per_round_seq:.3f} committed tokens per round per sequence"),
            "round_s": round(full_round, 3)}


def calibration_copy():
    """One plain 256 MiB device-to-device copy: the reference dispatch that scales the HBM
    traffic counters (FETCH_SIZE / WRITE_SIZE) to bytes."""
    import torch
    cal_src = torch.ones(256 * 2**20, dtype=torch.uint8, device="cuda")
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst


def block_sweep(dec, prompts, blocks=(4, 8, 16, 32), rounds=12):
    """Round latency (graph replay, ms) of the same model and context for each block size."""
    import torch
    res = {}
    for K in blocks:
        dec.set_block(K)
        dec.prefill(torch.from_numpy(prompts), max_out=32 * (rounds + 4))
        g = dec.capture(dec.round_greedy)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(rounds):
            g.replay()
        torch.cuda.synchronize()
        res[str(K)] = round((time.perf_counter() - t0) / rounds * 1e3, 4)
        del g
    dec.set_block(dec.block_alloc)
    return res


def two_step_drafting(dec, prompts, n_fill=15, rounds=12, n_tokens=32):
    """Two-step drafting (the variant the pages ablate): round latency by graph replay, committed
    tokens per round and per forward pass (three passes a round), and whether the committed
    trajectory still equals AR decoding.  With random weights the acceptance says nothing about
    the trained model; the latency and the losslessness do."""
    import torch
    B = len(prompts)
    dec.prefill(torch.from_numpy(prompts), max_out=32 * (rounds + 4))
    g = dec.capture(dec.round_greedy_two_step, n_fill)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    out0 = int(dec.out_len.sum())
    t0 = time.perf_counter()
    for _ in range(rounds):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / rounds * 1e3
    per_round = (int(dec.out_len.sum()) - out0) / (rounds * B)
    del g
    a, _ = dec.generate(prompts, n_tokens, two_step=n_fill, use_graph=True)
    b, _ = dec.generate_ar(prompts, n_tokens, use_graph=True)
    return {"n_fill": n_fill, "round_ms": round(ms, 4), "tokens_per_round_per_seq": round(per_round, 4),
            "tpf": round(per_round / 3, 4), "trajectory_equals_ar": bool(np.array_equal(a, b)),
            "match_tokens": n_tokens}


def trajectory_match(dec, W, shape, prompts, n_tokens, kv_chunk):
    """Greedy Orthrus vs greedy AR through the same kernels: fraction of sequences whose first
    n_tokens agree exactly, in bf16 (the timed decoder) and fp32 (the same bf16-valued weights
    held in fp32)."""
    import torch
    from orthrus_round_amd.decoder import Decoder
    B = prompts.shape[0]
    out = {}
    for prec in ("bf16", "fp32"):
        d = dec if prec == "bf16" else Decoder(W, shape, precision="fp32", block=32, max_batch=B,
                                                max_ctx=prompts.shape[1] + n_tokens + 96, kv_chunk=kv_chunk)
        a, st = d.generate(prompts, n_tokens, use_graph=True)
        b, _ = d.generate_ar(prompts, n_tokens, use_graph=True)
        same = [bool(np.array_equal(a[i], b[i])) for i in range(B)]
        out[prec] = {"match_rate": sum(same) / B, "sequences": B, "tokens": n_tokens, "rounds": st.rounds}
        if d is not dec:
            del d
            torch.cuda.empty_cache()
    return out


def first_divergence(a, b):
    """Index of the first differing token of two equal-length rows, or None."""
    d = np.nonzero(np.asarray(a) != np.asarray(b))[0]
    return int(d[0]) if d.size else None


def divergence_control(dec, prompts, n_tokens, kv_chunk, other_chunk):
    """Greedy trajectories when the attention sums keys in another chunking (another summation
    order, as a kernel that is not batch-invariant would): the invariant pairing (Orthrus vs AR at
    one kv_chunk) next to AR vs AR and Orthrus vs AR across two kv_chunks, with the positions at
    which the trajectories part."""
    runs = {}
    for ch in (kv_chunk, other_chunk):
        dec.set_kv_chunk(ch)
        runs[("orthrus", ch)], _ = dec.generate(prompts, n_tokens, use_graph=True)
        runs[("ar", ch)], _ = dec.generate_ar(prompts, n_tokens, use_graph=True)
    dec.set_kv_chunk(kv_chunk)
    B = prompts.shape[0]
    margins = ar_margins(dec, prompts, n_tokens)
    ref = runs[("ar", kv_chunk)]
    assert np.array_equal(margins["tokens"], ref[:, :n_tokens]), "eager AR with logits differs from the graph run"
    gap = margins["top2_gap"]

    def cmp(x, y):
        div = [first_divergence(runs[x][i, :n_tokens], runs[y][i, :n_tokens]) for i in range(B)]
        at = [(d, float(gap[i, d])) for i, d in enumerate(div) if d is not None]
        return {"match_rate": sum(d is None for d in div) / B,
                "first_divergence": sorted(d for d, _ in at),
                "ar_top2_gap_at_divergence": [round(g, 6) for _, g in sorted(at)],
                "gap_percentile_at_divergence": [round(float((gap < g).mean()) * 100, 1) for _, g in sorted(at)]}
    return {f"orthrus_c{kv_chunk}_vs_ar_c{kv_chunk}": cmp(("orthrus", kv_chunk), ("ar", kv_chunk)),
            f"ar_c{kv_chunk}_vs_ar_c{other_chunk}": cmp(("ar", kv_chunk), ("ar", other_chunk)),
            f"orthrus_c{kv_chunk}_vs_ar_c{other_chunk}": cmp(("orthrus", kv_chunk), ("ar", other_chunk)),
            "ar_top2_gap_median": round(float(np.median(gap)), 6),
            "ar_top2_gap_min": round(float(gap.min()), 6),
            "sequences": B, "tokens": n_tokens}


def ar_margins(dec, prompts, n_tokens):
    """Greedy AR steps (eager) that also keep the logits: per sequence and step, the gap between the
    largest and the second-largest logit of the reference AR model (its decisiveness there)."""
    import torch
    B, V = prompts.shape[0], dec.shape.vocab
    dec.prefill(torch.as_tensor(prompts), n_tokens)
    buf = torch.empty((dec.B, V), dtype=torch.float32, device=dec.dev)
    gaps = np.zeros((B, n_tokens))
    for t in range(n_tokens):
        dec.ar_step(0.0, 0, logits=buf)
        top = torch.topk(buf[:B], 2, dim=1).values
        gaps[:, t] = (top[:, 0] - top[:, 1]).cpu().numpy()
    torch.cuda.synchronize()
    return {"tokens": dec.out_tokens.cpu().numpy()[:B, :n_tokens], "top2_gap": gaps}


def memory_overhead(W, shape, batch, kv_chunk, contexts=(1024, 2048, 4096), rounds=4):
    """Device memory of an Orthrus decoder (32-row rounds) against an AR decoder (1-row steps) with
    caches sized for each context.  Every buffer is allocated up front, so holding a cache for a
    context costs the same whatever part of it is filled: a 16-token prompt and a few rounds give
    the peak.  Both decoders load both views' weights, so peak(Orthrus) - peak(AR) is the runtime
    overhead of the round."""
    import torch
    import synth
    from orthrus_round_amd.decoder import Decoder
    prompts = torch.from_numpy(synth.prompt_ids(shape, 7, batch, 16))
    mib = lambda b: round(b / 2**20, 3)
    res = {}
    for ctx in contexts:
        row = {}
        for mode, block in (("orthrus", 32), ("ar", 1)):
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            base = torch.cuda.memory_allocated()
            torch.cuda.reset_peak_memory_stats()
            d = Decoder(W, shape, precision="bf16", block=block, max_batch=batch, max_ctx=ctx, kv_chunk=kv_chunk)
            d.prefill(prompts, max_out=32 * rounds)
            for _ in range(rounds):
                d.round_greedy() if mode == "orthrus" else d.ar_step()
            torch.cuda.synchronize()
            rb = d.runtime_bytes()
            row[mode] = {"peak_MiB": mib(torch.cuda.max_memory_allocated() - base),
                         **{k + "_MiB": mib(v) for k, v in rb.items()}}
            del d
        row["orthrus_minus_ar_peak_MiB"] = round(row["orthrus"]["peak_MiB"] - row["ar"]["peak_MiB"], 3)
        res[str(ctx)] = row
    torch.cuda.empty_cache()
    s = shape
    return {"batch": batch, "contexts": res,
            "block_kv_at_36_layers_batch1_MiB": mib(32 * 36 * s.kv_heads * s.head_dim * 2 * 2),
            "note": "block K/V is one layer's buffer, reused by every layer; the paged KV cache is the AR cache "
                    "and grows with the context"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode round is sharded by "
              "sequence across GPUs with no exchange, so N GPUs = N independent copies of this run.")
        sys.exit(2)
    import torch
    import synth
    from orthrus_round_amd.decoder import Decoder
    import orthrus_round_amd as ora
    ora.lib()
    t_setup = time.perf_counter()
    shape = synth.QWEN3_8B_L8
    if args.layers != shape.layers:
        import dataclasses
        shape = dataclasses.replace(shape, layers=args.layers)
    W = synth.model_weights(shape, cfg=5, diff_std=0.002, bf16=True)
    prompts = synth.prompt_ids(shape, 5, args.batch, args.prompt)
    total_rounds = args.warmup + args.steps + 2
    dec = Decoder(W, shape, precision=args.precision, block=32, max_batch=args.batch,
                  max_ctx=args.prompt + 32 * total_rounds + 64, kv_chunk=args.kv_chunk)
    print(f"[bench] setup {time.perf_counter() - t_setup:.1f}s", file=sys.stderr, flush=True)
    dec.prefill(torch.from_numpy(prompts), max_out=32 * total_rounds)
    torch.cuda.synchronize()
    g = dec.capture(dec.round_greedy)  # its warm-up call is one untimed round
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    out0 = int(dec.out_len.sum())
    r0 = dec.round.cpu().numpy().copy()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    committed = int(dec.out_len.sum()) - out0
    elapsed = t1 - t0
    rounds_done = int((dec.round.cpu().numpy() - r0).min())
    ctx_np = dec.ctx_len.cpu().numpy()
    print(f"[bench] {args.steps} rounds in {elapsed:.3f}s, committed {committed}", file=sys.stderr, flush=True)

    if args.counters:
        calibration_copy()
        print(json.dumps({"mode": "counters", "rounds": args.steps, "ms_per_step": round(elapsed / args.steps * 1e3, 4)}),
              flush=True)
        return
    tab = kernel_table(dec, ctx_np)
    per_round = {k: v["ms"] * v["per_round"] for k, v in tab.items()}
    dominant = max(per_round, key=per_round.get)
    roof = roofline_of(dominant, tab[dominant], "mfma" if dominant == "lmhead_argmax" and args.batch * 32 >= 512
                       else "hbm")

    # AR yardstick on the same kernels (one causal row per sequence per step)
    dec.prefill(torch.from_numpy(prompts), max_out=64)
    ga = dec.capture(dec.ar_step)
    for _ in range(3):
        ga.replay()
    torch.cuda.synchronize()
    ta = time.perf_counter()
    for _ in range(20):
        ga.replay()
    torch.cuda.synchronize()
    ar_ms = (time.perf_counter() - ta) / 20 * 1e3

    sweep = match = control = memory = two = None
    if not args.no_extras:
        sweep = block_sweep(dec, prompts)
        two = two_step_drafting(dec, prompts)
        match = trajectory_match(dec, W, shape, prompts, args.match_tokens, args.kv_chunk)
        control = divergence_control(dec, prompts, args.match_tokens, args.kv_chunk, args.control_chunk)
        memory = memory_overhead(W, shape, args.batch, args.kv_chunk)
    attn = None if args.no_attn else attention_roofline(args.attn_chunk)
    calibration_copy()
    tokens_per_round_seq = committed / (args.steps * args.batch)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(W, shape, prompts, tokens_per_round_seq)

    ms = elapsed / args.steps * 1e3
    rec = {
        "metric": "accepted tokens/s (Orthrus decode rounds, committed tokens)",
        "value": round(committed / elapsed, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.precision,
        "data": "synthetic (seeded random-init weights N(0,0.02), diffusion view = AR + N(0,0.002), uniform prompt ids)",
        "config": {"workload": "Orthrus round, Qwen3-8B width truncated to %d layers, greedy" % shape.layers,
                   "batch": args.batch, "prompt_len": args.prompt, "block": 32, "hidden": shape.hidden,
                   "heads": f"{shape.q_heads}Q/{shape.kv_heads}KV x {shape.head_dim}", "inter": shape.inter,
                   "vocab": shape.vocab, "kv_chunk": args.kv_chunk, "parallelism": "single GPU"},
        "round_latency_ms": round(ms, 4),
        "tokens_per_round_per_seq": round(tokens_per_round_seq, 4),
        "tpf": round(tokens_per_round_seq / 2, 4),
        "rounds_timed_min": rounds_done,
        "ar_step_ms": round(ar_ms, 4),
        "ar_tokens_per_s": round(args.batch / ar_ms * 1e3, 2),
        "projected_tokens_per_s_at_pages_10p78_tokens_per_round": round(args.batch * 10.78 / ms * 1e3, 1),
        "roofline": roof,
        "kernels": {k: {"ms": round(v["ms"], 5), "per_round": v["per_round"],
                        "GBs": round(v["bytes"] / v["ms"] / 1e6, 1)} for k, v in tab.items()},
        "attention_roofline": attn,
        "round_ms_by_block": sweep,
        "two_step_drafting": two,
        "trajectory_match_vs_ar": match,
        "divergence_control_bf16": control,
        "memory_vs_ar": memory,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
