"""Round driver: prefill, Orthrus rounds (draft pass, verify pass, consensus/commit) and the
plain AR reference, all through the C ABI on device-resident state.

Orthrus paper summary (cjcn.com.cn), sec. 二: the frozen AR model owns the only KV cache and
the diffusion view reads it; sec. 四: one round = a parallel draft pass over the anchor and
[MASK] slots, one causal AR pass over the block with the drafts filled in, then left-to-right
consensus (strict rejection sampling at temperature > 0).

Every arithmetic step runs in liborthrus kernels.  PyTorch only allocates device memory and
provides the stream; the host enqueues launches and never reads round state inside a round,
so a whole round can be captured once into a HIP graph and replayed.
"""
from __future__ import annotations

import dataclasses
import time

import numpy as np
import torch

from . import _lib as L


@dataclasses.dataclass
class GenStats:
    rounds: int
    tokens: int
    passes: int
    decode_s: float
    accept_hist: list

    @property
    def tpf(self) -> float:
        return self.tokens / max(1, self.passes)

    @property
    def tokens_per_s(self) -> float:
        return self.tokens / self.decode_s if self.decode_s > 0 else float("nan")


class Decoder:
    """A random-init (or given) decoder with an AR view and a diffusion attention view.

    ``weights``: dict of host float32 arrays in Linear layout (``embed``, ``lm_head``,
    ``final_norm`` and per layer ``l.attn_norm, l.mlp_norm, l.wq, l.wk, l.wv, l.wo, l.w_gate,
    l.w_up, l.w_down`` plus the diffusion view's ``l.dq, l.dk, l.dv, l.do``).
    ``shape``: object with layers, hidden, q_heads, kv_heads, head_dim, inter, vocab,
    rope_base, eps, mask_id.
    ``precision``: 'bf16' (bf16 weights and activations, fp32 inside kernels) or 'fp32'.
    """

    def __init__(self, weights: dict, shape, precision: str = "bf16", block: int = 32, max_batch: int = 1,
                 max_ctx: int = 4096, page_size: int = 16, kv_chunk: int = 1024, device: str = "cuda",
                 page_order_seed: int | None = None):
        L.lib()  # fail loudly if the HIP library is missing
        self.shape = s = shape
        self.K = block            # rows per sequence of a round (set_block may lower it)
        self.block_alloc = block  # rows per sequence the buffers hold; also the prefill chunk
        self.B = max_batch
        self.dev = torch.device(device)
        self.prec = precision
        self.dt = L.BF16 if precision == "bf16" else L.F32
        self.tdt = torch.bfloat16 if precision == "bf16" else torch.float32
        self.page = page_size
        self.kv_chunk = kv_chunk
        self.max_pages = -(-(max_ctx + block) // page_size)
        self.max_ctx = self.max_pages * page_size
        self.max_pos = self.max_ctx + block
        H, D, Hq, Hkv, I, V = s.hidden, s.head_dim, s.q_heads, s.kv_heads, s.inter, s.vocab
        self.nqkv = (Hq + 2 * Hkv) * D

        def up(a, dt=None):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dtype=dt or self.tdt, device=self.dev)

        W = weights
        self.embed = up(W["embed"])
        self.lm_head = up(W["lm_head"])
        self.final_norm = up(W["final_norm"], torch.float32)
        self.layers = []
        # gate/up: the row-interleaved packing for every row count, and where the library builds it,
        # the fragment-packed copy that the register-streamed kernel reads for more than 64 rows
        self.frag_gate_up = True
        for l in range(s.layers):
            gate, upw = up(W[f"{l}.w_gate"]), up(W[f"{l}.w_up"])
            gu = torch.empty((2 * I, H), dtype=self.tdt, device=self.dev)
            L.pack_gate_up(I, H, self.dt, gate, upw, gu)
            gu_frag = None
            if self.frag_gate_up:
                gu_frag = torch.empty((2 * I, H), dtype=self.tdt, device=self.dev)
                try:
                    L.pack_gate_up_fragments(I, H, self.dt, gate, upw, gu_frag)
                except L.OrthrusError as e:
                    if e.status != 2:  # anything but "shape not built" is a real error
                        raise
                    gu_frag, self.frag_gate_up = None, False
            del gate, upw
            self.layers.append(dict(
                attn_norm=up(W[f"{l}.attn_norm"], torch.float32),
                mlp_norm=up(W[f"{l}.mlp_norm"], torch.float32),
                qkv_ar=up(np.concatenate([W[f"{l}.wq"], W[f"{l}.wk"], W[f"{l}.wv"]])),
                o_ar=up(W[f"{l}.wo"]),
                qkv_diff=up(np.concatenate([W[f"{l}.dq"], W[f"{l}.dk"], W[f"{l}.dv"]])),
                o_diff=up(W[f"{l}.do"]),
                gate_up=gu,
                gate_up_frag=gu_frag,
                down=up(W[f"{l}.w_down"]),
            ))
        torch.cuda.synchronize(self.dev)
        # paged AR cache (the only cache), one pool per layer
        self.num_pages = self.B * self.max_pages
        self.k_pages = [torch.zeros((self.num_pages, Hkv, page_size, D), dtype=self.tdt, device=self.dev)
                        for _ in range(s.layers)]
        self.v_pages = [torch.zeros_like(k) for k in self.k_pages]
        order = np.arange(self.num_pages, dtype=np.int32)
        if page_order_seed is not None:
            order = np.random.default_rng(page_order_seed).permutation(self.num_pages).astype(np.int32)
        self.page_table = torch.from_numpy(order.reshape(self.B, self.max_pages)).to(self.dev)
        self.rope = torch.empty((self.max_pos, D // 2, 2), dtype=torch.float32, device=self.dev)
        L.rope_table(self.max_pos, D, float(s.rope_base), self.rope)
        # activations for up to B*K rows
        M = self.B * block
        self.x = torch.empty((M, H), dtype=self.tdt, device=self.dev)
        self.a = torch.empty_like(self.x)
        self.qkv = torch.empty((M, self.nqkv), dtype=self.tdt, device=self.dev)
        self.q = torch.empty((M, Hq * D), dtype=self.tdt, device=self.dev)
        self.o = torch.empty((M, Hq * D), dtype=self.tdt, device=self.dev)
        self.h = torch.empty((M, I), dtype=self.tdt, device=self.dev)
        self.k_blk = torch.empty((self.B, block, Hkv, D), dtype=self.tdt, device=self.dev)
        self.v_blk = torch.empty_like(self.k_blk)
        self.attn_ws = {}
        gw = 0
        for (n, k, e) in ((self.nqkv, H, L.EPI_STORE), (H, Hq * D, L.EPI_RESIDUAL), (2 * I, H, L.EPI_SWIGLU),
                          (H, I, L.EPI_RESIDUAL)):
            gw = max(gw, L.gemm_workspace_bytes(M, n, k, self.dt, e))
        self.gemm_ws = torch.empty(max(gw, 256), dtype=torch.uint8, device=self.dev)  # k-split partials
        self.lm_ws = torch.empty(L.lmhead_workspace_bytes(L.lmhead_desc(M, H, V, self.dt)), dtype=torch.uint8,
                                 device=self.dev)
        # round state
        z = lambda: torch.zeros(self.B, dtype=torch.int32, device=self.dev)
        self.ctx_len, self.anchor, self.accept, self.out_len, self.round, self.done = z(), z(), z(), z(), z(), z()
        self.seq_id = torch.arange(self.B, dtype=torch.int32, device=self.dev)
        self.draft = torch.zeros((self.B, block), dtype=torch.int32, device=self.dev)
        self.target = torch.zeros_like(self.draft)
        # two-step drafting: pass 1's logsumexp, pass 2's block tokens, fill flags, pass 2's choice
        self.lse1 = torch.empty(M, dtype=torch.float32, device=self.dev)
        self.tokens2, self.filled, self.draft2 = (torch.zeros_like(self.draft) for _ in range(3))
        self.out_tokens = None
        self.max_out = 0
        self._logits = None
        self.graph = None

    # ------------------------------------------------------------------ building blocks
    def _attn_desc(self, nb, kb):
        s = self.shape
        return L.attn_desc(nb, s.q_heads, s.kv_heads, s.head_dim, kb, self.page, self.max_pages, self.max_ctx,
                           self.kv_chunk, self.dt, self.dt, 1.0 / float(np.sqrt(s.head_dim)))

    def _ws(self, desc):
        """One attention workspace for every call: its size depends on the batch and the chunk count
        of max_ctx only (not on the block), and is largest at the full batch."""
        need = max(16, L.attn_workspace_bytes(desc))
        ws = self.attn_ws.get("chunk_partials")
        if ws is None or ws.numel() < need:
            full = max(16, L.attn_workspace_bytes(self._attn_desc(self.B, self.block_alloc)))
            ws = torch.empty(max(need, full), dtype=torch.uint8, device=self.dev)
            self.attn_ws["chunk_partials"] = ws
        return ws

    def _layers(self, view: str, nb: int, kb: int, ctx, draft: bool):
        """Decoder layers over nb*kb rows in self.x (in place); K/V to the cache unless draft."""
        s = self.shape
        M = nb * kb
        H, D, Hq, Hkv, I = s.hidden, s.head_dim, s.q_heads, s.kv_heads, s.inter
        dt = self.dt
        desc = self._attn_desc(nb, kb)
        ws = self._ws(desc)
        x, a = self.x[:M], self.a[:M]
        # every residual GEMM also normalises its rows for the next block (the next layer's
        # attention norm, or the final norm before the LM head), so `a` is ready at each step
        L.rmsnorm(M, H, dt, x, self.layers[0]["attn_norm"], s.eps, a)
        for l, Wl in enumerate(self.layers):
            nxt = self.layers[l + 1]["attn_norm"] if l + 1 < len(self.layers) else self.final_norm
            if draft:
                L.gemm_rope_kv_write(nb, kb, Hq, Hkv, D, self.page, self.max_pages, H, dt, a, Wl["qkv_" + view],
                                     self.rope, self.max_pos, ctx, None, self.qkv, self.q, self.k_blk, self.v_blk,
                                     self.gemm_ws)
                L.draft_attn(desc, self.q, self.k_pages[l], self.v_pages[l], self.page_table, ctx, self.k_blk,
                             self.v_blk, self.o, ws)
            else:
                L.gemm_rope_kv_write(nb, kb, Hq, Hkv, D, self.page, self.max_pages, H, dt, a, Wl["qkv_" + view],
                                     self.rope, self.max_pos, ctx, self.page_table, self.qkv, self.q,
                                     self.k_pages[l], self.v_pages[l], self.gemm_ws)
                L.verify_attn(desc, self.q, self.k_pages[l], self.v_pages[l], self.page_table, ctx, self.o, ws)
            L.gemm_residual_rmsnorm(M, H, Hq * D, dt, self.o, Wl["o_" + view], x, Wl["mlp_norm"], s.eps, a,
                                    self.gemm_ws)
            if Wl["gate_up_frag"] is not None and M > 64:
                L.gemm_swiglu_fragments(M, I, H, dt, a, Wl["gate_up_frag"], self.h)
            else:
                L.gemm(M, 2 * I, H, dt, dt, L.EPI_SWIGLU, a, Wl["gate_up"], None, self.h, self.gemm_ws)
            L.gemm_residual_rmsnorm(M, H, I, dt, self.h, Wl["down"], x, nxt, s.eps, a, self.gemm_ws)

    def _lm_head(self, nb, kb, tokens, temperature=0.0, seed=0, stream_id=L.STREAM_DRAFT, logits=None, lse=None,
                 sample=None):
        s = self.shape
        M = nb * kb
        # self.a[:M] already holds final_norm(x): the last layer's down projection wrote it
        d = L.lmhead_desc(M, s.hidden, s.vocab, self.dt, kb, stream_id, temperature, seed, sample)
        L.lmhead_argmax(d, self.a[:M], self.lm_head, self.seq_id, self.round, tokens, logits, lse, self.lm_ws)

    # ------------------------------------------------------------------ prefill / state
    def set_block(self, block: int):
        """Use rounds of `block` rows per sequence (1 <= block <= the block the buffers were built
        for).  Round buffers are used as flat arrays of batch*block rows, so they serve any smaller
        block; graphs captured for another block must be captured again."""
        assert 1 <= block <= self.block_alloc
        self.K = block
        self._logits = None
        self.graph = None

    def set_kv_chunk(self, kv_chunk: int):
        """Use attention key chunks of `kv_chunk` keys.  The chunk fixes the order in which a row's
        keys are summed, so runs compared bit for bit must use the same value; workspaces and graphs
        built for another chunk are dropped."""
        assert kv_chunk > 0 and kv_chunk % 32 == 0
        self.kv_chunk = kv_chunk
        self.attn_ws = {}
        self.graph = None

    def runtime_bytes(self) -> dict:
        """Device bytes held by this decoder, by kind: the two views' weights, the shared weights,
        the paged KV cache, the diffusion view's block K/V buffer, the attention workspaces, and every
        other buffer (activations of a round's rows, LM-head workspace, round state)."""
        def nb(t):
            return t.numel() * t.element_size()
        view = {"ar": 0, "diff": 0}
        shared = nb(self.embed) + nb(self.lm_head) + nb(self.final_norm)
        for ly in self.layers:
            view["ar"] += nb(ly["qkv_ar"]) + nb(ly["o_ar"])
            view["diff"] += nb(ly["qkv_diff"]) + nb(ly["o_diff"])
            shared += nb(ly["attn_norm"]) + nb(ly["mlp_norm"]) + nb(ly["gate_up"]) + nb(ly["down"])
            if ly["gate_up_frag"] is not None:
                shared += nb(ly["gate_up_frag"])
        kv = sum(nb(t) for t in self.k_pages) + sum(nb(t) for t in self.v_pages)
        blk = nb(self.k_blk) + nb(self.v_blk)
        attn_ws = sum(nb(t) for t in self.attn_ws.values())

        def tensors(o):
            if isinstance(o, torch.Tensor):
                yield o
            elif isinstance(o, (list, tuple)):
                for x in o:
                    yield from tensors(x)
            elif isinstance(o, dict):
                for x in o.values():
                    yield from tensors(x)
        seen, total = set(), 0
        for t in tensors(list(vars(self).values())):
            key = (t.untyped_storage().data_ptr(), t.device)
            if t.device.type == self.dev.type and key not in seen:
                seen.add(key)
                total += t.untyped_storage().nbytes()
        named = view["ar"] + view["diff"] + shared + kv + blk + attn_ws
        return {"weights_ar_view": view["ar"], "weights_diff_view": view["diff"], "weights_shared": shared,
                "kv_cache": kv, "block_kv": blk, "attn_workspace": attn_ws, "other_buffers": total - named}

    def prefill(self, prompts: torch.Tensor, max_out: int):
        """AR prefill of prompts[:, :-1] in causal chunks of the allocated block; anchor :=
        prompts[:, -1].  Every kernel's per-row result is independent of the chunking."""
        B, P = prompts.shape
        assert B == self.B and P >= 1 and P - 1 + self.K <= self.max_ctx
        prompts = prompts.to(self.dev, torch.int32).contiguous()
        for c in range(0, P - 1, self.block_alloc):
            kb = min(self.block_alloc, P - 1 - c)
            ctx = torch.full((B,), c, dtype=torch.int32, device=self.dev)
            L.embed_block(B, kb, self.shape.hidden, self.dt, self.embed, None, prompts, P, c, self.shape.mask_id,
                          self.x)
            self._layers("ar", B, kb, ctx, draft=False)
        self.ctx_len.fill_(P - 1)
        self.anchor.copy_(prompts[:, P - 1])
        for t in (self.accept, self.out_len, self.round, self.done):
            t.zero_()
        if self.out_tokens is None or self.max_out != max_out:
            # a new buffer: any graph captured against the old one must be captured again
            self.out_tokens = torch.full((B, max_out), -1, dtype=torch.int32, device=self.dev)
        else:
            self.out_tokens.fill_(-1)
        self.max_out = max_out

    # ------------------------------------------------------------------ one round
    def round_greedy(self):
        B, K, s = self.B, self.K, self.shape
        L.embed_block(B, K, s.hidden, self.dt, self.embed, self.anchor, None, 0, 0, s.mask_id, self.x)
        self._layers("diff", B, K, self.ctx_len, draft=True)
        self._lm_head(B, K, self.draft)
        L.embed_block(B, K, s.hidden, self.dt, self.embed, self.anchor, self.draft, K, 0, s.mask_id, self.x)
        self._layers("ar", B, K, self.ctx_len, draft=False)
        self._lm_head(B, K, self.target)
        L.consensus_commit(B, K, self.draft, self.target, self.ctx_len, self.anchor, self.accept, self.out_tokens,
                           self.out_len, self.round, self.done, self.max_out, self.max_ctx)

    def round_greedy_two_step(self, n_fill: int):
        """A greedy round whose draft takes two diffusion passes (two-step drafting): pass 1 over
        [anchor, MASK...], then its n_fill most confident predictions are written into their slots
        (orthrus_draft_fill), pass 2 runs over that block, and orthrus_draft_merge keeps the filled
        tokens.  Verify and consensus are those of the one-pass round."""
        B, K, s = self.B, self.K, self.shape
        M = B * K
        L.embed_block(B, K, s.hidden, self.dt, self.embed, self.anchor, None, 0, 0, s.mask_id, self.x)
        self._layers("diff", B, K, self.ctx_len, draft=True)
        self._lm_head(B, K, self.draft, lse=self.lse1[:M])
        L.draft_fill(B, K, s.hidden, s.vocab, self.dt, self.a[:M], self.lm_head, self.lse1[:M], self.draft, s.mask_id,
                     n_fill, self.tokens2, self.filled)
        L.embed_block(B, K, s.hidden, self.dt, self.embed, self.anchor, self.tokens2, K, 0, s.mask_id, self.x)
        self._layers("diff", B, K, self.ctx_len, draft=True)
        self._lm_head(B, K, self.draft2)
        L.draft_merge(B, K, self.filled, self.tokens2, self.draft2, self.draft)
        L.embed_block(B, K, s.hidden, self.dt, self.embed, self.anchor, self.draft, K, 0, s.mask_id, self.x)
        self._layers("ar", B, K, self.ctx_len, draft=False)
        self._lm_head(B, K, self.target)
        L.consensus_commit(B, K, self.draft, self.target, self.ctx_len, self.anchor, self.accept, self.out_tokens,
                           self.out_len, self.round, self.done, self.max_out, self.max_ctx)

    def round_sampled(self, temperature: float, seed: int):
        B, K, s = self.B, self.K, self.shape
        if self._logits is None:
            M = B * K
            self._logits = [torch.empty((M, s.vocab), dtype=torch.float32, device=self.dev) for _ in range(2)]
            self._lse = [torch.empty(M, dtype=torch.float32, device=self.dev) for _ in range(2)]
            self._rej_ws = torch.empty(max(16, L.rejection_workspace_bytes(B, s.vocab)),
                                       dtype=torch.uint8, device=self.dev)
        L.embed_block(B, K, s.hidden, self.dt, self.embed, self.anchor, None, 0, 0, s.mask_id, self.x)
        self._layers("diff", B, K, self.ctx_len, draft=True)
        self._lm_head(B, K, self.draft, temperature, seed, L.STREAM_DRAFT, self._logits[0], self._lse[0])
        L.embed_block(B, K, s.hidden, self.dt, self.embed, self.anchor, self.draft, K, 0, s.mask_id, self.x)
        self._layers("ar", B, K, self.ctx_len, draft=False)
        # the verify pass keeps its logits and lse(z/T) for the accept test; it draws no sample
        self._lm_head(B, K, self.target, temperature, seed, L.STREAM_AR, self._logits[1], self._lse[1], sample=False)
        L.rejection_accept(B, K, s.vocab, temperature, seed, self.seq_id, self._logits[0], self._logits[1],
                           self._lse[0], self._lse[1], self.draft, self.ctx_len, self.anchor, self.accept,
                           self.out_tokens, self.out_len, self.round, self.done, self.max_out, self.max_ctx,
                           self._rej_ws)

    def ar_step(self, temperature: float = 0.0, seed: int = 0, logits: torch.Tensor | None = None):
        """One plain AR step for every sequence: a one-row causal pass, argmax/sample, commit.
        With `logits` (fp32 [batch, vocab]) the step also writes the LM head's logits there.
        Returns the step's tokens as a [batch, 1] view of a buffer the next call overwrites."""
        B, s = self.B, self.shape
        L.embed_block(B, 1, s.hidden, self.dt, self.embed, self.anchor, None, 0, 0, s.mask_id, self.x)
        self._layers("ar", B, 1, self.ctx_len, draft=False)
        t_flat = self.target.view(-1)[:B]
        self._lm_head(B, 1, t_flat, temperature, seed, L.STREAM_AR, logits=logits)
        L.consensus_commit(B, 1, t_flat, t_flat, self.ctx_len, self.anchor, self.accept, self.out_tokens,
                           self.out_len, self.round, self.done, self.max_out, self.max_ctx)
        return t_flat.view(B, 1)

    # ------------------------------------------------------------------ graphs
    def capture(self, fn, *args):
        """Capture one call of ``fn`` (a round or AR step) into a HIP graph."""
        st = torch.cuda.Stream(device=self.dev)
        st.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(st):
            fn(*args)  # warm-up: allocates attention workspaces outside the capture
        torch.cuda.current_stream(self.dev).wait_stream(st)
        torch.cuda.synchronize(self.dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(*args)
        return g

    # ------------------------------------------------------------------ drivers
    def generate(self, prompts, max_new: int, temperature: float = 0.0, seed: int = 0, use_graph: bool = False,
                 poll_every: int = 8, record_accepts: bool = False, max_rounds: int | None = None,
                 two_step: int | None = None):
        """Orthrus decoding; returns (tokens [B, max_new] int32 numpy, GenStats).  ``two_step``
        (greedy only) drafts with two diffusion passes, filling that many masks after the first."""
        assert two_step is None or temperature == 0.0
        self.prefill(torch.as_tensor(prompts), max_new)
        torch.cuda.synchronize(self.dev)
        if two_step is not None:
            fn, args = self.round_greedy_two_step, (two_step,)
        elif temperature == 0.0:
            fn, args = self.round_greedy, ()
        else:
            fn, args = self.round_sampled, (temperature, seed)
        hist = []
        t0 = time.perf_counter()
        if use_graph:
            # graph capture runs the round once more during warm-up; redo prefill state after capture
            g = self.capture(fn, *args)
            self.prefill(torch.as_tensor(prompts), max_new)
            torch.cuda.synchronize(self.dev)
            t0 = time.perf_counter()
        rounds = 0
        while True:
            for _ in range(poll_every):
                if use_graph:
                    g.replay()
                else:
                    fn(*args)
                rounds += 1
                if record_accepts:
                    hist.append(self.accept.cpu().numpy().copy())
            if bool((self.done != 0).all()) or (max_rounds is not None and rounds >= max_rounds):
                break
        torch.cuda.synchronize(self.dev)
        dt = time.perf_counter() - t0
        toks = self.out_tokens.cpu().numpy()
        nround = self.round.cpu().numpy()
        passes = (3 if two_step is not None else 2) * int(nround.sum())
        stats = GenStats(int(nround.max()), int(self.out_len.sum().item()), passes, dt, hist)
        return toks, stats

    def generate_ar(self, prompts, max_new: int, temperature: float = 0.0, seed: int = 0, use_graph: bool = False):
        """Plain AR decoding through the same kernels (one causal row per step)."""
        self.prefill(torch.as_tensor(prompts), max_new)
        torch.cuda.synchronize(self.dev)
        if use_graph:
            g = self.capture(self.ar_step, temperature, seed)
            self.prefill(torch.as_tensor(prompts), max_new)
            torch.cuda.synchronize(self.dev)
        t0 = time.perf_counter()
        for _ in range(max_new):
            if use_graph:
                g.replay()
            else:
                self.ar_step(temperature, seed)
        torch.cuda.synchronize(self.dev)
        dt = time.perf_counter() - t0
        return self.out_tokens.cpu().numpy(), GenStats(max_new, self.B * max_new, max_new, dt, [])
