"""The C-ABI library loads on the CPU and exports every symbol the header declares.

No compute call is made here (no GPU in this process): only entry points that answer from
host-side validation before touching the device.
"""
import ctypes
import os
import re

import pytest

import orthrus_round_amd as ora
from orthrus_round_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "orthrus.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int32_t|size_t|const char\*)\s+(orthrus_[a-z0-9_]+)\(", text, re.M)))


def test_header_symbols_exported_and_bound():
    L = ora.lib()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTED)


def test_abi_version_matches_header():
    m = re.search(r"#define ORTHRUS_ABI_VERSION (\d+)", open(HEADER).read())
    assert ora.abi_version() == int(m.group(1))


def test_struct_layouts_match_header():
    # orthrus_attn_desc_t: 11 int32 + float; orthrus_lmhead_desc_t: 6 int32 + float + pad + uint64
    # + int32 + pad
    assert ctypes.sizeof(_lib.AttnDesc) == 48
    assert ctypes.sizeof(_lib.LmHeadDesc) == 48 and _lib.LmHeadDesc.seed.offset == 32
    assert _lib.LmHeadDesc.sample.offset == 40


@pytest.mark.parametrize("call,status", [
    (lambda: ora.gemm(4, 64, 63, ora.BF16, ora.BF16, 0, 1, 1, None, 1, stream=0), 2),
    (lambda: ora.gemm(4, 64, 64, ora.BF16, ora.BF16, 1, 1, 1, None, 1, stream=0), 1),
    (lambda: ora.gemm(4, 64, 64, ora.F32, ora.BF16, 0, 1, 1, None, 1, stream=0), 2),
    (lambda: ora.gemm(4, 64, 256, ora.BF16, ora.BF16, 0, 1, 1, None, 1, stream=0), 3),  # no workspace
    (lambda: ora.gemm(4, 64, 256, ora.BF16, ora.BF16, 0, 1, 1, None, 1, ws=17, stream=0), 3),  # 0 bytes given
    (lambda: ora.gemm_residual_rmsnorm(4, 64, 256, ora.BF16, 1, 1, 1, 1, 1e-6, 1, stream=0), 3),
    (lambda: ora.gemm_residual_rmsnorm(4, 64, 96, ora.BF16, 1, 1, 1, 1, 1e-6, 1, stream=0), 2),  # K % 64
    (lambda: ora.gemm_residual_rmsnorm(4, 64, 64, ora.BF16, 1, 1, 1, None, 1e-6, 1, stream=0), 1),  # no gain
    (lambda: ora.gemm_rope_kv_write(1, 32, 8, 2, 128, 16, 4, 4096, ora.BF16, 1, 1, 1, 64, 1, None, 1, 1, 1, 1,
                                    stream=0), 3),  # no workspace
    (lambda: ora.gemm_rope_kv_write(1, 32, 8, 2, 127, 16, 4, 4096, ora.BF16, 1, 1, 1, 64, 1, None, 1, 1, 1, 1,
                                    stream=0), 1),  # odd head_dim
    (lambda: ora.gemm_rope_kv_write(1, 0, 8, 2, 128, 16, 4, 4096, ora.BF16, 1, 1, 1, 64, 1, None, 1, 1, 1, 1,
                                    stream=0), 1),  # empty block
    (lambda: ora.consensus_commit(2, 33, 1, 1, 1, 1, 1, 1, 1, 1, 1, 8, 64, stream=0), 1),
    (lambda: ora.draft_fill(2, 65, 64, 100, ora.BF16, 1, 1, 1, 1, 99, 3, 1, 1, stream=0), 1),  # block > 64
    (lambda: ora.draft_fill(2, 32, 64, 100, ora.BF16, 1, 1, 1, 1, 99, 32, 1, 1, stream=0), 1),  # n_fill > 31
    (lambda: ora.draft_fill(2, 32, 60, 100, ora.BF16, 1, 1, 1, 1, 99, 3, 1, 1, stream=0), 2),  # hidden % 8
    (lambda: ora.draft_fill(2, 32, 64, 100, 7, 1, 1, 1, 1, 99, 3, 1, 1, stream=0), 2),  # dtype
    (lambda: ora.draft_fill(2, 32, 64, 100, ora.F32, None, 1, 1, 1, 99, 3, 1, 1, stream=0), 1),
    (lambda: ora.draft_merge(2, 32, 1, 1, None, 1, stream=0), 1),
    (lambda: ora.draft_merge(-1, 32, 1, 1, 1, 1, stream=0), 1),
    (lambda: ora.rmsnorm(2, 64, 7, 1, 1, 1e-6, 1, stream=0), 1),
    (lambda: ora.pack_gate_up_fragments(1024, 256, ora.BF16, 16, 16, 16, stream=0), 2),  # width not built
    (lambda: ora.pack_gate_up_fragments(8192, 4096, ora.F32, 16, 16, 16, stream=0), 2),  # fp32 not built
    (lambda: ora.pack_gate_up_fragments(8192, 4096, ora.BF16, 16, None, 16, stream=0), 1),
    (lambda: ora.pack_gate_up_fragments(8192, 4096, ora.BF16, 16, 24, 16, stream=0), 1),  # misaligned
    (lambda: ora.gemm_swiglu_fragments(8, 4096, 4096, ora.BF16, 16, 16, 16, stream=0), 2),  # 2I < 16384
    (lambda: ora.gemm_swiglu_fragments(8, 8224, 4096, ora.BF16, 16, 16, 16, stream=0), 2),  # no whole tiles
    (lambda: ora.gemm_swiglu_fragments(8, 8192, 4096, ora.BF16, 16, None, 16, stream=0), 1),
    (lambda: ora.rejection_accept(2, 32, 1000, 0.8, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 8, 64, None,
                                  stream=0), 3),  # no workspace
    (lambda: ora.rejection_accept(2, 32, 1000, 0.0, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 8, 64, 1,
                                  stream=0), 1),  # temperature 0
    (lambda: ora.rope_table(0, 64, 1e6, 1, stream=0), 1),
])
def test_validation_errors_before_launch(call, status):
    with pytest.raises(ora.OrthrusError) as e:
        call()
    assert e.value.status == status
    assert ora.lib().orthrus_last_error()


def test_attention_descriptor_validation():
    d = ora.attn_desc(1, 16, 8, 128, 32, 16, 4, 64, kv_chunk=0)
    assert ora.attn_workspace_bytes(d) == 0  # one chunk at max_ctx 64
    d2 = ora.attn_desc(2, 32, 8, 128, 32, 16, 1100, 17600, kv_chunk=1024)
    assert ora.attn_workspace_bytes(d2) == 2 * 8 * 18 * 4 * 32 * 130 * 4
    bad = [ora.attn_desc(1, 12, 8, 128, 32, 16, 4, 64), ora.attn_desc(1, 16, 8, 96, 32, 16, 4, 64),
           ora.attn_desc(1, 16, 8, 128, 33, 16, 4, 64), ora.attn_desc(1, 16, 8, 128, 32, 16, 4, 65),
           ora.attn_desc(1, 16, 8, 128, 32, 16, 4, 64, kv_chunk=48), ora.attn_desc(1, 24, 8, 128, 32, 16, 4, 64)]
    for d in bad:
        with pytest.raises(ora.OrthrusError):
            ora.verify_attn(d, 1, 1, 1, 1, 1, 1, None, stream=0)


def test_gemm_workspace_holds_the_k_quarter_partials():
    # N < 16384 with whole-stage quarters of K: four fp32 partial tiles of [M, N]
    assert ora.gemm_workspace_bytes(256, 4096, 4096, ora.BF16, ora.EPI_STORE) == 4 * 256 * 4096 * 4
    assert ora.gemm_workspace_bytes(8, 6144, 4096, ora.F32, ora.EPI_RESIDUAL) == 4 * 8 * 6144 * 4
    assert ora.gemm_workspace_bytes(8, 6144, 128, ora.F32, ora.EPI_STORE) == 4 * 8 * 6144 * 4
    # deep K (the down projection) splits eight ways
    assert ora.gemm_workspace_bytes(256, 4096, 12288, ora.BF16, ora.EPI_RESIDUAL) == 8 * 256 * 4096 * 4
    assert ora.gemm_workspace_bytes(8, 4096, 8192 + 256, ora.BF16, ora.EPI_RESIDUAL) == 4 * 8 * 4096 * 4
    # the wide (gate/up) family and K that does not split into whole 128-byte stages need none
    assert ora.gemm_workspace_bytes(8, 24576, 4096, ora.BF16, ora.EPI_SWIGLU) == 0
    assert ora.gemm_workspace_bytes(8, 4096, 192, ora.BF16, ora.EPI_STORE) == 0
    assert ora.gemm_workspace_bytes(0, 4096, 4096, ora.BF16, ora.EPI_STORE) == 0


def test_rejection_refuses_a_misaligned_workspace():
    L = ora.lib()
    args = [2, 32, 1000, 0.8, 1] + [16] * 13 + [8, 64]
    st = L.orthrus_rejection_accept(*args, 24, 1 << 20, None)  # 24 is not a multiple of 16
    assert st == 1 and b"aligned" in L.orthrus_last_error()


def test_rejection_workspace_holds_one_pair_per_vocabulary_chunk():
    # two packed race maxima (16 bytes) per 2048-entry chunk of the vocabulary, per sequence
    assert ora.rejection_workspace_bytes(16, 151936) == 16 * 75 * 16
    assert ora.rejection_workspace_bytes(1, 2048) == 16 and ora.rejection_workspace_bytes(1, 2049) == 32
    assert ora.rejection_workspace_bytes(0, 151936) == 0
