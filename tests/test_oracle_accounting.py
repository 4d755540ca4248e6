"""The oracle's round accounting against numbers printed on the pages (tests/golden)."""
import json
import os

import pytest

from oracle import decode as Dc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_accounting.json")))


def _result(accepts, K=32):
    rounds = [Dc.RoundLog(0, k, [0] * min(k + 1, K), [], []) for k in accepts]
    toks = [t for r in rounds for t in r.emitted]
    return Dc.GenResult(toks, rounds, 2 * len(rounds))


def test_tpf_is_half_the_tokens_per_round():
    g = GOLD["tpf_8b_mean"]
    assert g["tokens_per_round"] == pytest.approx(2 * g["tpf"])
    # a round accepting k drafts commits k + 1 tokens over two passes
    assert _result([9, 10]).tpf == pytest.approx((10 + 11) / 4)


def test_tpf_from_mean_accept_length():
    g = GOLD["tpf_from_mean_accept"]
    res = _result([11, 12, 12, 12, 11, 12, 12, 12, 11, 12])  # mean 11.7
    assert res.tpf == pytest.approx(g["tpf"], abs=1e-9)


def test_tpf_bounds():
    g = GOLD["tpf_bounds"]
    assert _result([0] * 7).tpf == pytest.approx(g["orthrus_min"])
    assert _result([32] * 3).tpf == 16.0


def test_block_state_constant():
    g = GOLD["block_state_bytes"]
    b = g["slots"] * g["layers"] * g["kv_heads"] * g["head_dim"] * g["tensors"] * g["bytes_per_elem"]
    assert b / 2**20 == pytest.approx(g["mib"])
