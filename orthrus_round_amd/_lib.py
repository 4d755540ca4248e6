"""ctypes binding of liborthrus.so: argument marshalling only.

Every function here has the name of the C entry point without the ``orthrus_`` prefix,
takes torch CUDA tensors (or ``None`` for optional pointers) and plain numbers, checks
nothing beyond what marshalling needs, and raises ``OrthrusError`` for a non-zero status.
All work is enqueued on the current torch stream (or ``stream=``).  The library must be
built (``python -m orthrus_round_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liborthrus.so")

BF16, F32 = 0, 1
EPI_STORE, EPI_RESIDUAL, EPI_SWIGLU = 0, 1, 2
STREAM_DRAFT, STREAM_ACCEPT, STREAM_RESID, STREAM_AR = 1, 2, 3, 4

_STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP"}


class OrthrusError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"orthrus {_STATUS.get(status, status)}: {msg}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("kv_chunk", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class LmHeadDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("hidden", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("block", ctypes.c_int32), ("stream_id", ctypes.c_int32),
                ("temperature", ctypes.c_float), ("seed", ctypes.c_uint64), ("sample", ctypes.c_int32)]


_lib = None
_P, _I32, _I64, _U64, _F32, _SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                   ctypes.c_float, ctypes.c_size_t)

_SIGS = {
    "orthrus_abi_version": ([], _I32),
    "orthrus_last_error": ([], ctypes.c_char_p),
    "orthrus_attn_workspace_bytes": ([ctypes.POINTER(AttnDesc)], _SZ),
    "orthrus_draft_attn": ([ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], _I32),
    "orthrus_verify_attn": ([ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P, _SZ, _P], _I32),
    "orthrus_lmhead_workspace_bytes": ([ctypes.POINTER(LmHeadDesc)], _SZ),
    "orthrus_lmhead_argmax": ([ctypes.POINTER(LmHeadDesc), _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], _I32),
    "orthrus_lmhead_argmax_noalloc": ([ctypes.POINTER(LmHeadDesc), _P, _P, _P, _P, _P, _P, _P, _P], _I32),
    "orthrus_consensus_commit": ([_I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _P], _I32),
    "orthrus_draft_fill": ([_I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _I32, _I32, _P, _P, _P], _I32),
    "orthrus_draft_merge": ([_I32, _I32, _P, _P, _P, _P, _P], _I32),
    "orthrus_rejection_workspace_bytes": ([_I32, _I32], _SZ),
    "orthrus_rejection_accept": ([_I32, _I32, _I32, _F32, _U64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  _P, _P, _I32, _I32, _P, _SZ, _P], _I32),
    "orthrus_gemm_workspace_bytes": ([_I32, _I32, _I32, _I32, _I32], _SZ),
    "orthrus_gemm": ([_I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P], _I32),
    "orthrus_gemm_rope_kv_write": ([_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _I32, _P,
                                    _P, _P, _P, _P, _P, _P, _SZ, _P], _I32),
    "orthrus_gemm_residual_rmsnorm": ([_I32, _I32, _I32, _I32, _P, _P, _P, _P, _F32, _P, _P, _SZ, _P], _I32),
    "orthrus_pack_gate_up": ([_I32, _I32, _I32, _P, _P, _P, _P], _I32),
    "orthrus_pack_gate_up_fragments": ([_I32, _I32, _I32, _P, _P, _P, _P], _I32),
    "orthrus_gemm_swiglu_fragments": ([_I32, _I32, _I32, _I32, _P, _P, _P, _P], _I32),
    "orthrus_rmsnorm": ([_I32, _I32, _I32, _P, _P, _F32, _P, _P], _I32),
    "orthrus_rope_table": ([_I32, _I32, ctypes.c_double, _P, _P], _I32),
    "orthrus_rope_kv_write": ([_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _I32, _P, _P, _P, _P,
                               _P, _P], _I32),
    "orthrus_embed_block": ([_I32, _I32, _I32, _I32, _P, _P, _P, _I32, _I32, _I32, _P, _P], _I32),
    "orthrus_philox4x64": ([_I64, _P, _U64, _U64, _P, _P], _I32),
}
EXPORTED = tuple(_SIGS)


def lib():
    """Load liborthrus.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OrthrusError(2, f"{LIB_PATH} is missing: build it with `python -m orthrus_round_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int):
    if status != 0:
        raise OrthrusError(status, lib().orthrus_last_error().decode())


def abi_version() -> int:
    return lib().orthrus_abi_version()


def attn_desc(batch, q_heads, kv_heads, head_dim, block, page_size, max_pages, max_ctx, kv_chunk=0,
              dtype=BF16, out_dtype=F32, scale=1.0) -> AttnDesc:
    return AttnDesc(batch, q_heads, kv_heads, head_dim, block, page_size, max_pages, max_ctx, kv_chunk, dtype,
                    out_dtype, scale)


def attn_workspace_bytes(desc: AttnDesc) -> int:
    return lib().orthrus_attn_workspace_bytes(ctypes.byref(desc))


def draft_attn(desc, q, k_pages, v_pages, page_table, ctx_len, k_blk, v_blk, out, ws, stream=None):
    _check(lib().orthrus_draft_attn(ctypes.byref(desc), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table),
                                    _ptr(ctx_len), _ptr(k_blk), _ptr(v_blk), _ptr(out), _ptr(ws),
                                    0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def verify_attn(desc, q, k_pages, v_pages, page_table, ctx_len, out, ws, stream=None):
    _check(lib().orthrus_verify_attn(ctypes.byref(desc), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table),
                                     _ptr(ctx_len), _ptr(out), _ptr(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def lmhead_desc(rows, hidden, vocab, dtype=BF16, block=32, stream_id=STREAM_DRAFT, temperature=0.0, seed=0,
                sample=None):
    """``sample`` defaults to sampling exactly when ``temperature`` > 0."""
    if sample is None:
        sample = temperature > 0.0
    return LmHeadDesc(rows, hidden, vocab, dtype, block, stream_id, temperature, seed, int(bool(sample)))


def lmhead_workspace_bytes(desc: LmHeadDesc) -> int:
    return lib().orthrus_lmhead_workspace_bytes(ctypes.byref(desc))


def lmhead_argmax(desc, h, w, seq_id, round_, token_out, logits_out, lse_out, ws, stream=None):
    _check(lib().orthrus_lmhead_argmax(ctypes.byref(desc), _ptr(h), _ptr(w), _ptr(seq_id), _ptr(round_),
                                       _ptr(token_out), _ptr(logits_out), _ptr(lse_out), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)))


def lmhead_argmax_noalloc(desc, h, w, seq_id, round_, token_out, logits_out, lse_out, stream=None):
    _check(lib().orthrus_lmhead_argmax_noalloc(ctypes.byref(desc), _ptr(h), _ptr(w), _ptr(seq_id), _ptr(round_),
                                               _ptr(token_out), _ptr(logits_out), _ptr(lse_out), _stream(stream)))


def consensus_commit(batch, block, draft, target, ctx_len, anchor, accept, out_tokens, out_len, round_, done,
                     max_out, max_ctx, stream=None):
    _check(lib().orthrus_consensus_commit(batch, block, _ptr(draft), _ptr(target), _ptr(ctx_len), _ptr(anchor),
                                          _ptr(accept), _ptr(out_tokens), _ptr(out_len), _ptr(round_), _ptr(done),
                                          max_out, max_ctx, _stream(stream)))


def draft_fill(batch, block, hidden, vocab, dtype, h, w, lse, draft, mask_id, n_fill, tokens2, filled, stream=None):
    _check(lib().orthrus_draft_fill(batch, block, hidden, vocab, dtype, _ptr(h), _ptr(w), _ptr(lse), _ptr(draft),
                                    mask_id, n_fill, _ptr(tokens2), _ptr(filled), _stream(stream)))


def draft_merge(batch, block, filled, tokens2, draft2, draft_out, stream=None):
    _check(lib().orthrus_draft_merge(batch, block, _ptr(filled), _ptr(tokens2), _ptr(draft2), _ptr(draft_out),
                                     _stream(stream)))


def rejection_workspace_bytes(batch, vocab) -> int:
    return lib().orthrus_rejection_workspace_bytes(batch, vocab)


def rejection_accept(batch, block, vocab, temperature, seed, seq_id, draft_logits, target_logits, draft_lse,
                     target_lse, draft, ctx_len, anchor, accept, out_tokens, out_len, round_, done, max_out,
                     max_ctx, ws, stream=None):
    _check(lib().orthrus_rejection_accept(batch, block, vocab, temperature, seed, _ptr(seq_id), _ptr(draft_logits),
                                          _ptr(target_logits), _ptr(draft_lse), _ptr(target_lse), _ptr(draft),
                                          _ptr(ctx_len), _ptr(anchor), _ptr(accept), _ptr(out_tokens),
                                          _ptr(out_len), _ptr(round_), _ptr(done), max_out, max_ctx, _ptr(ws),
                                          0 if ws is None or isinstance(ws, int) else ws.numel() * ws.element_size(),
                                          _stream(stream)))


def gemm_workspace_bytes(M, N, K, dtype, epilogue) -> int:
    return lib().orthrus_gemm_workspace_bytes(M, N, K, dtype, epilogue)


def gemm(M, N, K, dtype, out_dtype, epilogue, a, w, residual, c, ws=None, stream=None):
    _check(lib().orthrus_gemm(M, N, K, dtype, out_dtype, epilogue, _ptr(a), _ptr(w), _ptr(residual), _ptr(c),
                              _ptr(ws), 0 if ws is None or isinstance(ws, int) else ws.numel() * ws.element_size(),
                              _stream(stream)))


def gemm_residual_rmsnorm(M, N, K, dtype, a, w, x, gain, eps, y, ws=None, stream=None):
    _check(lib().orthrus_gemm_residual_rmsnorm(M, N, K, dtype, _ptr(a), _ptr(w), _ptr(x), _ptr(gain), eps, _ptr(y),
                                               _ptr(ws), 0 if ws is None or isinstance(ws, int)
                                               else ws.numel() * ws.element_size(), _stream(stream)))


def gemm_rope_kv_write(batch, block, q_heads, kv_heads, head_dim, page_size, max_pages, hidden, dtype, a, w, table,
                       max_pos, ctx_len, page_table, qkv, q_out, k_dst, v_dst, ws=None, stream=None):
    _check(lib().orthrus_gemm_rope_kv_write(batch, block, q_heads, kv_heads, head_dim, page_size, max_pages, hidden,
                                            dtype, _ptr(a), _ptr(w), _ptr(table), max_pos, _ptr(ctx_len),
                                            _ptr(page_table), _ptr(qkv), _ptr(q_out), _ptr(k_dst), _ptr(v_dst),
                                            _ptr(ws), 0 if ws is None or isinstance(ws, int)
                                            else ws.numel() * ws.element_size(), _stream(stream)))


def pack_gate_up(inter, hidden, dtype, gate, up, packed, stream=None):
    _check(lib().orthrus_pack_gate_up(inter, hidden, dtype, _ptr(gate), _ptr(up), _ptr(packed), _stream(stream)))


def pack_gate_up_fragments(inter, hidden, dtype, gate, up, packed, stream=None):
    _check(lib().orthrus_pack_gate_up_fragments(inter, hidden, dtype, _ptr(gate), _ptr(up), _ptr(packed),
                                                _stream(stream)))


def gemm_swiglu_fragments(M, inter, hidden, dtype, a, w_fragments, c, stream=None):
    _check(lib().orthrus_gemm_swiglu_fragments(M, inter, hidden, dtype, _ptr(a), _ptr(w_fragments), _ptr(c),
                                               _stream(stream)))


def rmsnorm(rows, hidden, dtype, x, gain, eps, y, stream=None):
    _check(lib().orthrus_rmsnorm(rows, hidden, dtype, _ptr(x), _ptr(gain), eps, _ptr(y), _stream(stream)))


def rope_table(max_pos, head_dim, base, table, stream=None):
    _check(lib().orthrus_rope_table(max_pos, head_dim, base, _ptr(table), _stream(stream)))


def rope_kv_write(batch, block, q_heads, kv_heads, head_dim, page_size, max_pages, dtype, qkv, table, max_pos,
                  ctx_len, page_table, q_out, k_dst, v_dst, stream=None):
    _check(lib().orthrus_rope_kv_write(batch, block, q_heads, kv_heads, head_dim, page_size, max_pages, dtype,
                                       _ptr(qkv), _ptr(table), max_pos, _ptr(ctx_len), _ptr(page_table),
                                       _ptr(q_out), _ptr(k_dst), _ptr(v_dst), _stream(stream)))


def embed_block(batch, block, hidden, dtype, embed, anchor, tokens, tok_stride, tok_offset, mask_id, x,
                stream=None):
    _check(lib().orthrus_embed_block(batch, block, hidden, dtype, _ptr(embed), _ptr(anchor), _ptr(tokens),
                                     tok_stride, tok_offset, mask_id, _ptr(x), _stream(stream)))


def philox4x64(n, ctr, k0, k1, out, stream=None):
    _check(lib().orthrus_philox4x64(n, _ptr(ctr), k0, k1, _ptr(out), _stream(stream)))
