"""Seeded synthetic inputs for the Orthrus decode round.

This module only *draws* data: random weights, prompts, query/key/value
tensors, ragged context lengths, page permutations and draft-token patterns.
It holds none of the method's arithmetic (no attention, no softmax, no
argmax, no acceptance rule) so that the CPU oracle and the HIP path can both
consume the same inputs without sharing any computation.

Seeding rule: tensor ``j`` of workload ``c`` is drawn from
``numpy.random.default_rng([c, j, *extra])``.  Every floating-point input that
the GPU sees in bf16 is rounded to bf16 here (round-to-nearest-even from
FP32) and returned as float32 arrays holding bf16-representable values, so the
oracle and the device see bit-identical operands.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# ---------------------------------------------------------------------------
# bf16 helpers (storage format only)
# ---------------------------------------------------------------------------


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even; NaN kept quiet."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    r = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = r.copy()
        r[nan] = 0x7FC0
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value, returned as float32."""
    return bf16_to_f32(bf16_bits(x))


def rng(c: int, j: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([c, j, *extra])


def _normal(c: int, j: int, shape, std: float, extra=()) -> np.ndarray:
    """N(0, std^2) float32 draw; large tensors are filled in row chunks on threads."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    chunk = 1 << 24
    nchunks = (n + chunk - 1) // chunk

    def fill(i):
        g = rng(c, j, *extra, i)
        lo, hi = i * chunk, min(n, (i + 1) * chunk)
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=8) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


# ---------------------------------------------------------------------------
# Model shapes and weights
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class ModelShape:
    layers: int
    hidden: int
    q_heads: int
    kv_heads: int
    head_dim: int
    inter: int
    vocab: int
    rope_base: float = 1.0e6
    eps: float = 1.0e-6

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def mask_id(self) -> int:
        """Reserved [MASK] token id: the last vocabulary entry."""
        return self.vocab - 1


# Tiny FP32 decoder (runs on CPU in seconds).
TINY = ModelShape(layers=2, hidden=256, q_heads=4, kv_heads=2, head_dim=64, inter=1024, vocab=4096)
# Qwen3-8B width truncated to 8 layers.
QWEN3_8B_L8 = ModelShape(layers=8, hidden=4096, q_heads=32, kv_heads=8, head_dim=128, inter=12288,
                         vocab=151936)

LAYER_AR = ("wq", "wk", "wv", "wo")
LAYER_DIFF = ("dq", "dk", "dv", "do")


def model_weights(shape: ModelShape, cfg: int, w_std: float = 0.02, diff_std: float = 0.005,
                  bf16: bool = False, layers: int | None = None) -> dict:
    """Random-init decoder weights in PyTorch Linear layout ``[out, in]``.

    Keys: ``embed [V,H]``, ``lm_head [V,H]``, ``final_norm [H]`` and per layer ``l``:
    ``l.attn_norm``, ``l.mlp_norm`` ([H], all ones), ``l.wq [Hq*D,H]``, ``l.wk``,
    ``l.wv [Hkv*D,H]``, ``l.wo [H,Hq*D]``, ``l.w_gate``, ``l.w_up [I,H]``,
    ``l.w_down [H,I]`` and the diffusion view's own attention weights
    ``l.dq, l.dk, l.dv, l.do`` = AR weight + N(0, diff_std^2).
    """
    s = shape
    L = s.layers if layers is None else layers
    rnd = bf16_round if bf16 else (lambda a: a)
    H, D, Hq, Hkv, I, V = s.hidden, s.head_dim, s.q_heads, s.kv_heads, s.inter, s.vocab
    W = {}
    W["embed"] = rnd(_normal(cfg, 0, (V, H), w_std))
    W["lm_head"] = rnd(_normal(cfg, 1, (V, H), w_std))
    W["final_norm"] = np.ones(H, np.float32)
    shapes = {"wq": (Hq * D, H), "wk": (Hkv * D, H), "wv": (Hkv * D, H), "wo": (H, Hq * D),
              "w_gate": (I, H), "w_up": (I, H), "w_down": (H, I)}
    for l in range(L):
        W[f"{l}.attn_norm"] = np.ones(H, np.float32)
        W[f"{l}.mlp_norm"] = np.ones(H, np.float32)
        for j, (name, shp) in enumerate(shapes.items()):
            W[f"{l}.{name}"] = rnd(_normal(cfg, 100 + 20 * l + j, shp, w_std))
        for j, (ar, df) in enumerate(zip(LAYER_AR, LAYER_DIFF)):
            base = W[f"{l}.{ar}"]
            noise = _normal(cfg, 100 + 20 * l + 10 + j, base.shape, diff_std)
            W[f"{l}.{df}"] = rnd(base + noise)
    return W


def prompt_ids(shape: ModelShape, cfg: int, batch: int, length: int, j: int = 50) -> np.ndarray:
    """Uniform random prompt ids in [0, V-2] (the [MASK] id V-1 never appears)."""
    return rng(cfg, j).integers(0, shape.vocab - 1, size=(batch, length), dtype=np.int64).astype(np.int32)


# ---------------------------------------------------------------------------
# Attention-layer inputs (dual-view attention at Qwen3 shapes)
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class AttnInputs:
    """Logical (un-paged) attention operands plus their paged layout.

    q       [B, K, Hq, D]     block queries (already scaled; scale passed separately)
    kv      list of (k [n_b+K, Hkv, D], v [n_b+K, Hkv, D]) per sequence; the first n_b
            rows are the prior cache, the last K rows are the block's own AR keys/values
    k_blk   [B, K, Hkv, D]    the diffusion view's block keys (draft mask)
    v_blk   [B, K, Hkv, D]
    ctx     [B] int32         n_b
    pages_k/pages_v [P, Hkv, page, D]; page_table [B, maxp] int32
    """
    q: np.ndarray
    kv: list
    k_blk: np.ndarray
    v_blk: np.ndarray
    ctx: np.ndarray
    scale: float
    page_size: int
    pages_k: np.ndarray
    pages_v: np.ndarray
    page_table: np.ndarray


def page_layout(kv: list, kv_heads: int, head_dim: int, page_size: int, c: int, j: int,
                max_pages: int | None = None, extra_pages: int = 0):
    """Scatter logical per-sequence K/V into a page pool in a seeded random page order.

    Returns (pages_k, pages_v, page_table).  Pool layout ``[P, Hkv, page, D]``; pages not
    covered by a sequence (tail slots, spare pages) are filled with NaN so that any read of
    a dead slot is visible in the output.
    """
    need = [-(-k.shape[0] // page_size) for k, _ in kv]
    P = sum(need) + extra_pages
    maxp = max(need) if max_pages is None else max_pages
    perm = rng(c, j).permutation(P).astype(np.int32)
    pk = np.full((P, kv_heads, page_size, head_dim), np.nan, np.float32)
    pv = np.full_like(pk, np.nan)
    table = np.full((len(kv), maxp), -1, np.int32)
    nxt = 0
    for b, (k, v) in enumerate(kv):
        n = k.shape[0]
        for p in range(need[b]):
            phys = perm[nxt]
            nxt += 1
            table[b, p] = phys
            lo, hi = p * page_size, min(n, (p + 1) * page_size)
            pk[phys, :, : hi - lo, :] = k[lo:hi].transpose(1, 0, 2)
            pv[phys, :, : hi - lo, :] = v[lo:hi].transpose(1, 0, 2)
    table[table < 0] = 0
    return pk, pv, table


def attn_inputs(c: int, ctx: np.ndarray, q_heads: int, kv_heads: int, head_dim: int,
                block: int = 32, page_size: int = 16, bf16: bool = True,
                q_scale: float | None = None) -> AttnInputs:
    """K, V ~ N(0,1); queries ~ N(0,1) * q_scale (default 1/sqrt(D)); scale 1 for the kernel."""
    rnd = bf16_round if bf16 else (lambda a: a)
    B = len(ctx)
    qs = (1.0 / np.sqrt(head_dim)) if q_scale is None else q_scale
    q = rnd(_normal(c, 1, (B, block, q_heads, head_dim), 1.0) * np.float32(qs))
    kv = []
    for b in range(B):
        n = int(ctx[b]) + block
        k = rnd(_normal(c, 2, (n, kv_heads, head_dim), 1.0, extra=(b,)))
        v = rnd(_normal(c, 3, (n, kv_heads, head_dim), 1.0, extra=(b,)))
        kv.append((k, v))
    k_blk = rnd(_normal(c, 4, (B, block, kv_heads, head_dim), 1.0))
    v_blk = rnd(_normal(c, 5, (B, block, kv_heads, head_dim), 1.0))
    pk, pv, table = page_layout(kv, kv_heads, head_dim, page_size, c, 6)
    return AttnInputs(q, kv, k_blk, v_blk, np.asarray(ctx, np.int32), 1.0, page_size, pk, pv, table)


def ragged_lengths(c: int, batch: int, lo: int, hi: int, j: int = 0) -> np.ndarray:
    """Context lengths uniform on the integers [lo, hi]."""
    return rng(c, j).integers(lo, hi + 1, size=batch).astype(np.int32)


# ---------------------------------------------------------------------------
# LM-head + consensus inputs
# ---------------------------------------------------------------------------


def lmhead_inputs(c: int, rows: int, hidden: int, vocab: int, h_std: float = 1.0,
                  w_std: float = 0.02, bf16: bool = True):
    rnd = bf16_round if bf16 else (lambda a: a)
    h = rnd(_normal(c, 10, (rows, hidden), h_std))
    w = rnd(_normal(c, 11, (vocab, hidden), w_std))
    return h, w


def draft_hidden(c: int, h_target: np.ndarray, mix: float = 0.9, bf16: bool = True) -> np.ndarray:
    """Draft-view hidden states correlated with the target's: mix*h + sqrt(1-mix^2)*N(0,1)."""
    rnd = bf16_round if bf16 else (lambda a: a)
    noise = _normal(c, 12, h_target.shape, 1.0)
    return rnd(np.float32(mix) * h_target + np.float32(np.sqrt(1.0 - mix * mix)) * noise)


def geometric_drafts(c: int, target: np.ndarray, vocab: int, mean: float = 5.0, j: int = 13):
    """Drafts that copy the target for a geometric prefix, then differ.

    ``target`` is [B, K] int32 (the target argmax per slot).  For each sequence a prefix
    length L ~ Geometric on {0,1,...} with mean ``mean`` (p = 1/(mean+1)), capped at K, is
    drawn; drafts equal the target on slots < L, slot L (if any) is forced to a different id
    and the remaining slots are uniform ids.  Returns (drafts [B,K] int32, L [B] int32).
    """
    g = rng(c, j)
    B, K = target.shape
    L = np.minimum(g.geometric(1.0 / (mean + 1.0), size=B) - 1, K).astype(np.int32)
    d = g.integers(0, vocab, size=(B, K)).astype(np.int32)
    for b in range(B):
        d[b, : L[b]] = target[b, : L[b]]
        if L[b] < K:
            off = int(g.integers(1, vocab))
            d[b, L[b]] = (int(target[b, L[b]]) + off) % vocab
    return d, L


def seq_ids(batch: int) -> np.ndarray:
    return np.arange(batch, dtype=np.int32)
