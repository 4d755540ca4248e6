"""Orthrus decode round on AMD Instinct MI355X (gfx950).

``orthrus_round_amd._lib`` is the thin ctypes binding of ``liborthrus.so`` (the HIP kernels
behind the C ABI in ``include/orthrus.h``); ``orthrus_round_amd.decoder`` drives whole
rounds (draft pass, verify pass, consensus/commit) on device-resident state through those
calls only.  PyTorch provides device memory and streams.
"""
from ._lib import (BF16, F32, EPI_RESIDUAL, EPI_STORE, EPI_SWIGLU, STREAM_ACCEPT, STREAM_AR, STREAM_DRAFT,
                   STREAM_RESID, OrthrusError, abi_version, attn_desc, attn_workspace_bytes, consensus_commit,
                   draft_attn, draft_fill, draft_merge, embed_block, gemm, gemm_residual_rmsnorm,
                   gemm_rope_kv_write, gemm_swiglu_fragments, gemm_workspace_bytes, lib, lmhead_argmax,
                   lmhead_argmax_noalloc, lmhead_desc, lmhead_workspace_bytes, pack_gate_up, pack_gate_up_fragments,
                   philox4x64, rejection_accept, rejection_workspace_bytes, rmsnorm, rope_kv_write, rope_table,
                   verify_attn)

__all__ = [n for n in dir() if not n.startswith("_")]
