"""Plain CPU decoder rows and dual-view attention for the Orthrus decode round.

TEST INFRASTRUCTURE.  This is the oracle: a slow, obviously correct NumPy statement of
what the decode round computes.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark may import it; the HIP library never does, and this
module shares no code with it.

Sources (pages on the Orthrus method):
* Orthrus paper summary (cjcn.com.cn), sec. 二 "two heads, one memory": the frozen AR
  decoder owns the only KV cache; the diffusion view's queries attend to the
  concatenation of the AR keys/values and the parallel block's own keys/values.
* same page, sec. 三 "training": the diffusion view is a set of added attention modules
  (the backbone stays frozen); block = one visible anchor + 31 [MASK] slots; the draft mask
  lets a diffusion query see the AR context before the block's anchor plus every position of
  its own block, and the AR path keeps the standard causal mask.
* Decoder body: the pages only name the Qwen3 family.  The reading used here is the plain
  pre-norm decoder: RMSNorm (eps 1e-6), rotate-half RoPE with inv_freq = base^(-2i/D),
  grouped-query attention with kv head = h // G, SwiGLU MLP, no biases, an untied LM head.

Precision: every function computes in ``dtype`` (float64 by default; float32 mode on
request).  ``rowwise=True`` evaluates every block row on its own with 1-D operations, so a
row's result cannot depend on which other rows share its pass; ``rowwise=False`` uses
batched matrix products for speed on large shapes.
"""
from __future__ import annotations

import numpy as np


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g along the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + x.dtype.type(eps)) * g.astype(x.dtype)


def rope_angles(pos: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    """Angle pos * base^(-2i/D) for i < D/2, computed in float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = np.exp(-(2.0 * i / head_dim) * np.log(base))
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE: pairs (x_i, x_{i+D/2}) rotated by the angle of frequency i.

    ``pos`` broadcasts against ``x.shape[:-1]`` (e.g. x [m, heads, D] with pos [m, 1]).
    The cos/sin values are taken in float64 and then cast to x's dtype.
    """
    D = x.shape[-1]
    half = D // 2
    ang = rope_angles(pos, D, base)                         # [..., D/2]
    cos = np.cos(ang).astype(x.dtype)
    sin = np.sin(ang).astype(x.dtype)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (x.dtype.type(1) + np.exp(-x))


def softmax_attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """One query row against an explicit key set: softmax(scale * k q) weighted sum of v.

    q [D], k [N, D], v [N, D]  ->  [D].  Max-subtracted softmax, every reduction in dtype.
    """
    s = (k * q).sum(axis=1) * q.dtype.type(scale)
    s = s - s.max()
    p = np.exp(s)
    p = p / p.sum()
    return (p[:, None] * v).sum(axis=0)


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray,
                     scale: float) -> np.ndarray:
    """Rows of ``q [R, D]`` each attending to the keys of ``k [N, D]`` marked in ``allowed [R, N]``."""
    out = np.empty((q.shape[0], v.shape[1]), dtype=q.dtype)
    for r in range(q.shape[0]):
        idx = np.nonzero(allowed[r])[0]
        out[r] = softmax_attend(q[r], k[idx], v[idx], scale)
    return out


def draft_attention(q, k_ctx, v_ctx, k_blk, v_blk, scale):
    """Diffusion-view block attention (draft mask).

    q [K, Hq, D] block queries; k_ctx/v_ctx [n, Hkv, D] = the AR cache before the anchor;
    k_blk/v_blk [K, Hkv, D] = the block's own diffusion keys/values.  Every slot sees all of
    ``[K_AR ; K_diff]`` (context before the anchor, bidirectional inside the block).
    Returns [K, Hq, D].
    """
    K, Hq, D = q.shape
    G = Hq // k_ctx.shape[1]
    kk = np.concatenate([k_ctx, k_blk], axis=0)
    vv = np.concatenate([v_ctx, v_blk], axis=0)
    out = np.empty_like(q)
    for h in range(Hq):
        g = h // G
        for i in range(K):
            out[i, h] = softmax_attend(q[i, h], kk[:, g], vv[:, g], scale)
    return out


def verify_attention(q, k_all, v_all, n, scale):
    """AR-view block attention (causal mask): slot j sees keys [0, n + j].

    q [K, Hq, D]; k_all/v_all [>= n + K, Hkv, D] hold the cache with the block's own AR
    keys/values already at [n, n + K).  Returns [K, Hq, D].
    """
    K, Hq, D = q.shape
    G = Hq // k_all.shape[1]
    out = np.empty_like(q)
    for h in range(Hq):
        g = h // G
        for j in range(K):
            out[j, h] = softmax_attend(q[j, h], k_all[: n + j + 1, g], v_all[: n + j + 1, g], scale)
    return out


def grouped_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray,
                      scale: float) -> np.ndarray:
    """The same attention as ``softmax_attend`` row by row, written with matrix products for
    many rows at once: q [R, Hq, D] against k/v [N, Hkv, D] (query head h reads kv head h // G),
    row r seeing the keys marked in ``allowed [R, N]``.  Returns [R, Hq, D]."""
    R, Hq, D = q.shape
    G = Hq // k.shape[1]
    out = np.empty_like(q)
    neg = np.where(allowed, 0.0, -np.inf).astype(q.dtype)
    for h in range(Hq):
        s = (q[:, h] @ k[:, h // G].T) * q.dtype.type(scale) + neg
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h] = p @ v[:, h // G]
    return out


def _linear(x: np.ndarray, w: np.ndarray, rowwise: bool) -> np.ndarray:
    """x [m, in] times w[out, in]^T."""
    if not rowwise:
        return x @ w.T
    return np.stack([w @ x[r] for r in range(x.shape[0])]) if x.shape[0] else np.zeros((0, w.shape[0]), x.dtype)


class Weights:
    """Model weights cast to the oracle's dtype (float64 by default)."""

    def __init__(self, W: dict, shape, dtype=np.float64):
        self.shape = shape
        self.dtype = dtype
        self.W = {k: np.ascontiguousarray(v, dtype=dtype) for k, v in W.items()}

    def __getitem__(self, k):
        return self.W[k]


def layer_rows(Wt: Weights, layer: int, view: str, x: np.ndarray, pos: np.ndarray,
               k_ctx: np.ndarray, v_ctx: np.ndarray, mode: str, rowwise: bool = True):
    """One decoder layer over the ``m`` block rows ``x [m, H]`` at absolute positions ``pos``.

    view  'ar' uses wq/wk/wv/wo, 'diff' uses the diffusion view's dq/dk/dv/do; the norms and
          the MLP are the shared frozen ones.
    mode  'causal': row j sees k_ctx[:n] and the block's rows 0..j (AR path / verify / prefill)
          'draft' : every row sees k_ctx[:n] and all block rows (diffusion view)
    k_ctx/v_ctx [n, Hkv, D] are this layer's AR cache before the block.
    Returns (x_out [m, H], k_blk [m, Hkv, D], v_blk [m, Hkv, D]) where k_blk is post-RoPE.
    """
    s = Wt.shape
    m = x.shape[0]
    D, Hq, Hkv = s.head_dim, s.q_heads, s.kv_heads
    names = ("wq", "wk", "wv", "wo") if view == "ar" else ("dq", "dk", "dv", "do")
    wq, wk, wv, wo = (Wt[f"{layer}.{n}"] for n in names)
    a = rmsnorm(x, Wt[f"{layer}.attn_norm"], s.eps)
    q = _linear(a, wq, rowwise).reshape(m, Hq, D)
    k = _linear(a, wk, rowwise).reshape(m, Hkv, D)
    v = _linear(a, wv, rowwise).reshape(m, Hkv, D)
    q = rope(q, pos[:, None], s.rope_base)
    k = rope(k, pos[:, None], s.rope_base)
    scale = 1.0 / np.sqrt(D)
    n = k_ctx.shape[0]
    kk = np.concatenate([k_ctx, k], axis=0)
    vv = np.concatenate([v_ctx, v], axis=0)
    if mode == "causal":
        o = verify_attention(q, kk, vv, n, scale)
    elif mode == "draft":
        o = draft_attention(q, k_ctx, v_ctx, k, v, scale)
    else:
        raise ValueError(mode)
    x = x + _linear(o.reshape(m, Hq * D), wo, rowwise)
    hm = rmsnorm(x, Wt[f"{layer}.mlp_norm"], s.eps)
    g = _linear(hm, Wt[f"{layer}.w_gate"], rowwise)
    u = _linear(hm, Wt[f"{layer}.w_up"], rowwise)
    x = x + _linear(silu(g) * u, Wt[f"{layer}.w_down"], rowwise)
    return x, k, v


def lm_logits(Wt: Weights, x: np.ndarray, rowwise: bool = True) -> np.ndarray:
    """Final RMSNorm then the LM head: z = rmsnorm(x) W_lm^T, [m, V]."""
    h = rmsnorm(x, Wt["final_norm"], Wt.shape.eps)
    return _linear(h, Wt["lm_head"], rowwise)


def argmax_lowest(z: np.ndarray) -> np.ndarray:
    """Argmax along the last axis; exact ties go to the lowest index (numpy's rule)."""
    return np.argmax(z, axis=-1).astype(np.int32)
