"""The oracle against the hand-worked cases in tests/golden/.

Each fixture names the passage of the pages it follows and the readings it
relies on; its expected values were worked out by hand (the derivation is
stored beside each case), so these pins do not depend on the oracle itself.
CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        doc = json.load(f)
    assert doc["source"] and doc["cases"]
    return doc["cases"]


def _e4m3_exact(vals):
    """E4M3 bytes of values that E4M3 holds exactly (checked against torch's own conversion)."""
    v = np.asarray(vals, dtype=np.float32)
    back = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(back, v.astype(np.float64)), "fixture value not exact in E4M3"
    return gen.f32_to_e4m3_bits(v)


def _bf16_exact(vals):
    v = np.asarray(vals, dtype=np.float32)
    back = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(back, v), "fixture value not exact in bf16"
    return gen.f32_to_bf16_bits(v)


@pytest.mark.parametrize("case", _load("indexer_scores.json"), ids=lambda c: c["name"])
def test_golden_indexer_scores(case):
    got = oracle.indexer_row(_e4m3_exact(case["q"]), np.asarray(case["w"], np.float32), _e4m3_exact(case["k"]))
    assert np.array_equal(got, np.asarray(case["expect"], np.float64))


@pytest.mark.parametrize("case", _load("topk.json"), ids=lambda c: c["name"])
def test_golden_topk(case):
    got = oracle.topk_row(np.asarray(case["scores"], np.float64), int(case["k"]))
    assert np.array_equal(got, np.asarray(case["expect"], np.int32))


@pytest.mark.parametrize("case", _load("attention.json"), ids=lambda c: c["name"])
def test_golden_attention(case):
    out, lse = oracle.sparse_mla_row(_bf16_exact(case["q"]), _bf16_exact(case["kv"]), float(case["scale"]),
                                     int(case["D_v"]))
    np.testing.assert_allclose(out, np.asarray(case["expect_out"]), rtol=1e-14, atol=0)
    np.testing.assert_allclose(lse, np.asarray(case["expect_lse"]), rtol=1e-14, atol=0)


@pytest.mark.parametrize("case", _load("indexer_kl.json"), ids=lambda c: c["name"])
def test_golden_indexer_kl(case):
    got = oracle.indexer_kl_row(_bf16_exact(case["q"]), _bf16_exact(case["kv"]), float(case["scale"]),
                                np.asarray(case["iscore"], np.float64))
    want = float(case["expect"])
    if want == 0.0:
        assert abs(got) < 1e-15
    else:
        assert got == pytest.approx(want, rel=1e-13)
