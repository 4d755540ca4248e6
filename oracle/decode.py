"""The Orthrus decode round, step by step, on the CPU (oracle).

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU-baseline leg may
use this module; the HIP library shares no code with it.

Sources:
* Orthrus paper summary (cjcn.com.cn), sec. 四 "inference": (1) the diffusion view turns the
  current text plus [MASK] placeholders into 32 candidate tokens in one parallel forward
  pass; (2) the frozen AR model runs one causal pass over the block with the candidates
  filled in and gives its own choice at every position; (3) candidates are compared left to
  right and accepted while they equal the AR choice; at the first disagreement the AR choice
  is emitted as the correction, the remaining candidates are discarded and the memory (KV
  cache) is updated.  At least one token is committed per round; with a temperature the
  framework uses strict rejection sampling so the output distribution stays the AR one.
* same page, sec. 三: a block is the visible anchor token followed by 31 [MASK] slots.
* Rejection sampling at temperature > 0 follows standard speculative decoding (Leviathan,
  Kalman, Matias, ICML 2023, cited by the PaperDaily review of lossy verification): accept
  a draft d with probability min(1, p(d)/q(d)); on rejection draw from the normalised
  residual max(0, p - q).

Readings where the pages are silent (each listed in the design notes):
* block = anchor + (K-1) [MASK] slots at absolute positions n .. n+K-1, where n is the AR
  context length (the anchor's own K/V are not yet cached);
* shifted prediction: slot i's logits predict position n+i+1, so the draft is
  d_1..d_K and the verify rows are [anchor, d_1 .. d_{K-1}];
* full acceptance commits K tokens (no bonus token); the context grows by min(k+1, K);
* the initial state prefills prompt[:-1] and takes prompt[-1] as the first anchor;
* [MASK] is the reserved id V-1;
* two-step drafting (the sec. 六 ablation): pass 1 fills half of the K-1 masked slots, rounded
  down, choosing its most confident predictions (log-probability of the argmax; equal values to
  the lower slot); pass 2 re-predicts the rest, and a filled slot keeps its pass-1 token.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import model as M
from .philox import STREAM_ACCEPT, STREAM_AR, STREAM_DRAFT, STREAM_RESID, uniforms


class Cache:
    """The AR KV cache: per layer K and V, [capacity, Hkv, D], valid for positions < n."""

    def __init__(self, shape, capacity: int, dtype):
        self.k = [np.zeros((capacity, shape.kv_heads, shape.head_dim), dtype) for _ in range(shape.layers)]
        self.v = [np.zeros_like(a) for a in self.k]
        self.n = 0


def ar_pass(Wt: M.Weights, cache: Cache, tokens, rowwise: bool = True, lm_rows=None):
    """Causal AR pass over ``tokens`` at positions n .. n+m-1; writes their K/V to the cache.

    Used for prefill, for verification and for one-token AR steps.  Does not advance
    ``cache.n`` (the commit step does).  Returns logits [m, V] (or only rows ``lm_rows``).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    m = len(tokens)
    n = cache.n
    pos = np.arange(n, n + m)
    x = Wt["embed"][tokens]
    for l in range(Wt.shape.layers):
        x, k, v = M.layer_rows(Wt, l, "ar", x, pos, cache.k[l][:n], cache.v[l][:n], "causal", rowwise)
        cache.k[l][n:n + m] = k
        cache.v[l][n:n + m] = v
    if lm_rows is not None:
        x = x[lm_rows]
    return M.lm_logits(Wt, x, rowwise)


def draft_pass(Wt: M.Weights, cache: Cache, tokens, rowwise: bool = True):
    """Diffusion-view pass over the block ``tokens`` at positions n .. n+m-1 (draft mask).

    Reads the shared AR cache [0, n); its own block K/V live only inside the pass.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    m = len(tokens)
    n = cache.n
    pos = np.arange(n, n + m)
    x = Wt["embed"][tokens]
    for l in range(Wt.shape.layers):
        x, _, _ = M.layer_rows(Wt, l, "diff", x, pos, cache.k[l][:n], cache.v[l][:n], "draft", rowwise)
    return M.lm_logits(Wt, x, rowwise)


def consensus(draft, target):
    """Greedy intra-model consensus on one sequence.

    ``draft`` = d_1..d_K, ``target`` = t_1..t_K (AR choice at the same positions).
    k = length of the longest prefix with d_i == t_i.  Emitted: d_1..d_k, then the
    correction t_{k+1} if k < K.  Returns (k, emitted list).
    """
    K = len(draft)
    k = 0
    while k < K and int(draft[k]) == int(target[k]):
        k += 1
    emitted = [int(t) for t in draft[:k]]
    if k < K:
        emitted.append(int(target[k]))
    return k, emitted


def softmax_t(z: np.ndarray, temperature: float) -> np.ndarray:
    s = z / z.dtype.type(temperature)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def race(weights: np.ndarray, expo: np.ndarray) -> int:
    """Exponential race: argmax_x w(x) / E_x over w(x) > 0 (E_x i.i.d. Exp(1)).

    The winner is distributed as w / sum(w).  Ties go to the lowest id.
    """
    ratio = np.where(weights > 0, weights / expo, -np.inf)
    return int(np.argmax(ratio))


def rejection_accept(z_draft, z_target, draft, temperature, u_accept, e_resid):
    """Rejection-sampling consensus on one sequence (temperature > 0).

    z_draft, z_target [K, V] logits of the diffusion / AR view at the K block slots;
    draft [K] the sampled drafts; u_accept [K] uniforms; e_resid [V] Exp(1) variates.
    Slot i accepts d_i iff u_i * q_i(d_i) < p_i(d_i) (q = softmax(z_draft/T),
    p = softmax(z_target/T)).  At the first rejection j the emitted token is drawn from the
    residual max(0, p_j - q_j) (from p_j if the residual has no mass) by exponential race.
    Returns (k, emitted).
    """
    K = len(draft)
    for i in range(K):
        p = softmax_t(z_target[i], temperature)
        q = softmax_t(z_draft[i], temperature)
        d = int(draft[i])
        if u_accept[i] * q[d] < p[d]:
            continue
        r = np.maximum(p - q, 0.0)
        if not (r > 0).any():
            r = p
        x = race(r, e_resid)
        return i, [int(t) for t in draft[:i]] + [x]
    return K, [int(t) for t in draft]


def gumbel_sample(z: np.ndarray, temperature: float, u: np.ndarray) -> int:
    """Sample from softmax(z / T) as argmax_x (z_x / T - ln(-ln u_x))."""
    zt = z / z.dtype.type(temperature)
    g = -np.log(-np.log(u))
    return int(np.argmax(zt + g.astype(z.dtype)))


def log_confidence(z: np.ndarray, tok) -> np.ndarray:
    """Per row, the log-probability of the row's chosen token under softmax(z):
    z[i, tok_i] - logsumexp_x z[i, x]."""
    z = np.asarray(z, dtype=np.float64)
    tok = np.asarray(tok, dtype=np.int64)
    m = z.max(axis=1)
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    return z[np.arange(len(tok)), tok] - lse


def most_confident(conf, n_fill: int) -> np.ndarray:
    """Boolean mask of the ``n_fill`` largest entries of ``conf``.  Equal values are taken in
    index order; a NaN counts as -inf."""
    c = np.where(np.isnan(conf), -np.inf, np.asarray(conf, dtype=np.float64))
    order = sorted(range(len(c)), key=lambda i: (-c[i], i))
    sel = np.zeros(len(c), dtype=bool)
    sel[order[:n_fill]] = True
    return sel


def two_step_draft(Wt: M.Weights, cache: Cache, anchor: int, block: int, n_fill: int | None = None,
                   rowwise: bool = True):
    """Two-step drafting, the Fast-dLLM-v2 style variant that Orthrus paper summary sec. 六
    ablates (the diffusion view completes the block in two passes instead of one).

    Pass 1 runs over [anchor, MASK x (K-1)].  Its predictions for the K-1 masked slots (row j
    predicts slot j+1) are ranked by their log-probability; the ``n_fill`` most confident are
    written into their slots (default: half of the masks, rounded down) and pass 2 runs over
    that block.  A filled slot keeps its pass-1 token; every other row takes pass 2's choice.
    Returns (drafts, d1, d2, filled) with filled[j] true when row j's token came from pass 1.
    """
    K = block
    mask = Wt.shape.mask_id
    if n_fill is None:
        n_fill = (K - 1) // 2
    z1 = draft_pass(Wt, cache, [anchor] + [mask] * (K - 1), rowwise)
    d1 = M.argmax_lowest(z1)
    filled = np.zeros(K, dtype=bool)
    filled[: K - 1] = most_confident(log_confidence(z1[: K - 1], d1[: K - 1]), n_fill)
    blk2 = [anchor] + [int(d1[j]) if filled[j] else mask for j in range(K - 1)]
    z2 = draft_pass(Wt, cache, blk2, rowwise)
    d2 = M.argmax_lowest(z2)
    return np.where(filled, d1, d2).astype(np.int32), d1, d2, filled


@dataclasses.dataclass
class RoundLog:
    n_before: int
    accept: int
    emitted: list
    draft: list
    target: list


@dataclasses.dataclass
class GenResult:
    tokens: list
    rounds: list
    passes: int

    @property
    def tpf(self) -> float:
        """Tokens per forward pass, prefill excluded."""
        return len(self.tokens) / max(1, self.passes)


def prefill(Wt: M.Weights, prompt, capacity: int, rowwise: bool = True):
    """Prefill prompt[:-1] on the AR path; the last prompt token becomes the first anchor."""
    cache = Cache(Wt.shape, capacity, Wt.dtype)
    if len(prompt) > 1:
        ar_pass(Wt, cache, prompt[:-1], rowwise, lm_rows=[])
    cache.n = len(prompt) - 1
    return cache, int(prompt[-1])


def generate(Wt: M.Weights, prompt, max_new: int, block: int = 32, temperature: float = 0.0,
             seed: int = 0, seq_id: int = 0, rowwise: bool = True, inject=None,
             poison_dead: bool = False, max_rounds: int | None = None,
             two_step: int | None = None) -> GenResult:
    """Orthrus decoding of one sequence.

    ``inject`` (optional callable round, n, anchor -> drafts[K]) replaces the diffusion
    view's drafts, to force acceptance patterns.  ``poison_dead`` fills cache slots at or
    beyond the committed length with NaN after each round (rollback must make them
    unreachable).  At temperature > 0 drafts are sampled from the diffusion view with the
    DRAFT stream, accepted with the ACCEPT stream and corrected with the RESID stream.
    ``two_step`` (greedy only) drafts with ``two_step_draft`` filling that many masks, which
    costs one more forward pass per round.
    """
    assert two_step is None or temperature == 0.0
    shape = Wt.shape
    K = block
    cache, anchor = prefill(Wt, prompt, len(prompt) + max_new + 2 * K, rowwise)
    out, rounds, passes = [], [], 0
    r = 0
    while len(out) < max_new and (max_rounds is None or r < max_rounds):
        n = cache.n
        blk = [anchor] + [shape.mask_id] * (K - 1)
        if two_step is not None:
            d = two_step_draft(Wt, cache, anchor, K, two_step, rowwise)[0]
            passes += 1
        elif temperature == 0.0:
            zd = draft_pass(Wt, cache, blk, rowwise)
            d = M.argmax_lowest(zd)
        else:
            zd = draft_pass(Wt, cache, blk, rowwise)
            d = np.array([gumbel_sample(zd[i], temperature,
                                        uniforms(seed, STREAM_DRAFT, i, np.arange(shape.vocab), r, seq_id))
                          for i in range(K)], dtype=np.int32)
        if inject is not None:
            d = np.asarray(inject(r, n, anchor), dtype=np.int32)
        zt = ar_pass(Wt, cache, [anchor] + [int(t) for t in d[: K - 1]], rowwise)
        passes += 2
        if temperature == 0.0:
            t = M.argmax_lowest(zt)
            k, emitted = consensus(d, t)
        else:
            t = M.argmax_lowest(zt)
            ua = uniforms(seed, STREAM_ACCEPT, np.arange(K), 0, r, seq_id)
            er = -np.log(uniforms(seed, STREAM_RESID, np.arange(shape.vocab), 0, r, seq_id))
            k, emitted = rejection_accept(zd, zt, d, temperature, ua, er)
        rounds.append(RoundLog(n, k, emitted, [int(x) for x in d], [int(x) for x in t]))
        out.extend(emitted)
        anchor = emitted[-1]
        cache.n = n + len(emitted)
        if poison_dead:
            for l in range(shape.layers):
                cache.k[l][cache.n:] = np.nan
                cache.v[l][cache.n:] = np.nan
        r += 1
    return GenResult(out[:max_new], rounds, passes)


def generate_ar(Wt: M.Weights, prompt, max_new: int, temperature: float = 0.0, seed: int = 0,
                seq_id: int = 0, rowwise: bool = True, with_margin: bool = False):
    """Plain AR decoding: one causal row per step at position n, keys [0, n]."""
    shape = Wt.shape
    cache, anchor = prefill(Wt, prompt, len(prompt) + max_new + 1, rowwise)
    out, margins = [], []
    for step in range(max_new):
        z = ar_pass(Wt, cache, [anchor], rowwise)[0]
        if temperature == 0.0:
            tok = int(M.argmax_lowest(z))
        else:
            tok = gumbel_sample(z, temperature, uniforms(seed, STREAM_AR, 0, np.arange(shape.vocab), step, seq_id))
        if with_margin:
            top2 = np.sort(z)[-2:]
            margins.append(float(top2[1] - top2[0]))
        out.append(tok)
        anchor = tok
        cache.n += 1
    return (out, margins) if with_margin else out
