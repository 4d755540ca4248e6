"""The HBM-traffic summary that bench.py builds from two rocprofv3 counter passes, on synthetic
counter files: only dispatches after the marker count, each bench kernel is the sum of its
dispatches (k-slice GEMM + its reduce, attention + combine, LM-head launches + finalize), and the
counts are scaled by what the same counter read for the 256 MiB calibration copy."""
import csv
import json
import os

import bench

NAMES = {
    "qkv": "_ZN7orthrus12_GLOBAL__N_119gemm_quarter_kernelIDF16bNS_7GemmCfgIDF16bLi128ELi192E",
    "qkv_red": "_ZN7orthrus12_GLOBAL__N_126gemm_reduce_rope_kv_kernelIDF16bLi4EEEv",
    "attn_d": "_ZN7orthrus12_GLOBAL__N_111attn_kernelIDF16bDF16bLi128ELi4ELb1EEEvNS0_8AttnArgsE",
    "attn_v": "_ZN7orthrus12_GLOBAL__N_111attn_kernelIDF16bDF16bLi128ELi4ELb0EEEvNS0_8AttnArgsE",
    "comb_d": "_ZN7orthrus12_GLOBAL__N_119attn_combine_kernelIDF16bLi128ELi4ELb1EEEvNS0_8AttnArgsE",
    "comb_v": "_ZN7orthrus12_GLOBAL__N_119attn_combine_kernelIDF16bLi128ELi4ELb0EEEvNS0_8AttnArgsE",
    "o": "_ZN7orthrus12_GLOBAL__N_119gemm_quarter_kernelIDF16bNS_7GemmCfgIDF16bLi128ELi128ELi4ELi2E",
    "o_red": "_ZN7orthrus12_GLOBAL__N_126gemm_reduce_rmsnorm_kernelIDF16bLi4EEEv",
    "gu": "_ZN7orthrus12_GLOBAL__N_116rs_swiglu_kernelINS_5RsCfgILi4ELi2ELi4ELi2ELi4EEEEEv",
    "down": "_ZN7orthrus12_GLOBAL__N_119gemm_quarter_kernelIDF16bNS_7GemmCfgIDF16bLi128ELi128ELi2ELi2E",
    "down_red": "_ZN7orthrus12_GLOBAL__N_126gemm_reduce_rmsnorm_kernelIDF16bLi8EEEv",
    "lm1": "_ZN7orthrus12_GLOBAL__N_113lmhead_kernelIDF16bNS_7GemmCfgIDF16bLi256ELi256E",
    "lm2": "_ZN7orthrus12_GLOBAL__N_113lmhead_kernelIDF16bNS_7GemmCfgIDF16bLi256ELi128E",
    "fin": "orthrus::(anonymous namespace)::lmhead_finalize(unsigned long const*)",
    "embed": "_ZN7orthrus12_GLOBAL__N_112embed_kernelIDF16bEEvPKT_",
    "norm": "_ZN7orthrus12_GLOBAL__N_114rmsnorm_kernelIDF16bEEvPKT_",
    "cons": "orthrus::(anonymous namespace)::consensus_kernel(int)",
    "marker": "orthrus::(anonymous namespace)::philox_kernel(long)",
    "copy": "__amd_rocclr_copyBuffer",
}


def round_dispatches(layers=2):
    """One round as the decoder enqueues it (draft pass, LM head, verify pass, LM head, commit)."""
    seq = []
    for attn, comb in (("attn_d", "comb_d"), ("attn_v", "comb_v")):
        seq += ["embed", "norm"]
        for _ in range(layers):
            seq += ["qkv", "qkv_red", attn, comb, "o", "o_red", "gu", "down", "down_red"]
        seq += ["lm1", "lm2", "fin"]
    return seq + ["cons"]


def write_pass(path, counter, values, prefill_junk=True):
    """A counter_collection.csv: some prefill dispatches, the marker, two rounds, the copy."""
    os.makedirs(path, exist_ok=True)
    seq = (["qkv", "gu", "lm1"] if prefill_junk else []) + ["marker"] + round_dispatches() * 2 + ["copy"]
    with open(os.path.join(path, "bench_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, k in enumerate(seq):
            w.writerow([i + 1, NAMES[k], counter, values(k, i)])


def test_summary_groups_scales_and_skips_the_prefill(tmp_path):
    # fetch: every kernel reads 100 KiB except the parts we check; the copy reads half its bytes
    def fetch(k, i):
        return {"copy": 131072.0, "qkv": 1000.0, "qkv_red": 10.0, "attn_d": 500.0, "comb_d": 5.0, "gu": 7000.0,
                "lm1": 3000.0, "lm2": 600.0, "fin": 1.0, "down": 2000.0, "down_red": 20.0, "o": 300.0,
                "o_red": 3.0}.get(k, 99999.0 if i < 3 else 100.0)

    def write(k, i):
        return {"copy": 262144.0, "qkv": 200.0, "qkv_red": 20.0, "gu": 60.0}.get(k, 1.0)
    write_pass(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    write_pass(str(tmp_path / "w"), "WRITE_SIZE", write)
    out_json = str(tmp_path / "traffic.json")
    out = bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"), out_json)
    assert out["fetch_scale"] == 2.0 and out["write_scale"] == 1.0
    bk = out["bench_kernels"]
    assert bk["gemm_qkv_rope_kv"]["fetch_kib"] == 1010.0 and bk["gemm_qkv_rope_kv"]["write_kib"] == 220.0
    assert bk["gemm_gate_up_swiglu"]["fetch_kib"] == 7000.0
    assert bk["gemm_gate_up_swiglu"]["bytes"] == int((7000.0 * 2 + 60.0) * 1024)
    assert bk["gemm_down_residual_rmsnorm"]["fetch_kib"] == 2020.0
    assert bk["gemm_o_residual_rmsnorm"]["fetch_kib"] == 303.0
    assert bk["attn_draft"]["fetch_kib"] == 505.0
    assert bk["lmhead_argmax"]["fetch_kib"] == 3601.0
    # 2 rounds x 2 passes x 2 layers of each layer GEMM, 2 x 2 LM heads, 2 x 2 of each attention mask
    assert bk["gemm_gate_up_swiglu"]["dispatch_groups"] == 8 and bk["lmhead_argmax"]["dispatch_groups"] == 4
    assert bk["attn_draft"]["dispatch_groups"] == 4 and bk["attn_verify"]["dispatch_groups"] == 4
    assert json.load(open(out_json)) == out
