"""Stored expected values and the seeded input generators (CPU only)."""

import hashlib
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_seed0.json")


def _sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_tiny_golden_regenerates():
    g = json.load(open(GOLDEN))
    w = W.WORKLOADS["tiny"]
    inp = W.make_all(w, seed=0, device="cpu")
    assert inp["topk_ids"].numpy().tolist() == g["inputs"]["topk_ids"]
    wts = np.array([[float.fromhex(v) for v in row] for row in g["inputs"]["topk_weights_f32_hex"]], np.float32)
    np.testing.assert_array_equal(inp["topk_weights"].numpy(), wts)
    assert _sha(inp["hidden_states"].numpy()) == g["inputs"]["hidden_states_sha256"]
    assert _sha(inp["expert_output"].numpy()) == g["inputs"]["expert_output_sha256"]
    p = oracle.permute(inp["hidden_states"].numpy(), inp["topk_ids"].numpy(), w.num_experts)
    assert p["expert_first_token_offset"].tolist() == g["expected"]["expert_first_token_offset"]
    assert p["permuted_idx"].tolist() == g["expected"]["permuted_idx"]
    assert p["inv_permuted_idx"].tolist() == g["expected"]["inv_permuted_idx"]
    assert _sha(p["permuted_hidden_states"]) == g["expected"]["permuted_hidden_states_sha256"]
    out = oracle.unpermute(inp["expert_output"].numpy(), wts, p["inv_permuted_idx"], "f32")
    assert _sha(out) == g["expected"]["output_sha256"]


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_routing_shapes_and_ranges(name):
    w = W.WORKLOADS[name]
    ids, wts = W.make_routing(w)
    assert ids.shape == (w.num_tokens, w.topk) and ids.dtype == np.int32
    assert wts.shape == (w.num_tokens, w.topk) and wts.dtype == np.float32
    assert ids.min() >= 0 and ids.max() < w.num_experts
    # every workload draws distinct experts per token
    s = np.sort(ids, axis=1)
    assert np.all(np.diff(s, axis=1) > 0)
    assert np.all(wts > 0)
    np.testing.assert_allclose(wts.sum(axis=1), 1.0, rtol=0, atol=w.topk * 2.0**-23)
    ids2, wts2 = W.make_routing(w)
    assert np.array_equal(ids, ids2) and np.array_equal(wts, wts2)  # seeded


def test_softmax_topk_picks_largest_in_descending_order():
    w = W.WORKLOADS["qwen3"].with_tokens(64)
    ids, wts = W.make_routing(w)
    assert np.all(np.diff(wts, axis=1) <= 0)  # descending probability


def test_zipf_routing_is_skewed_with_empty_experts():
    w = W.WORKLOADS["dsv3"]
    ids, _ = W.make_routing(w)
    counts = np.bincount(ids.ravel(), minlength=w.num_experts)
    assert counts[0] == 0 and counts[-1] == 0
    assert (counts == 0).sum() == w.zipf_empty
    assert counts.max() > 0.9 * w.num_tokens  # the top expert takes most tokens


def test_fp8_quantisation_properties():
    torch = pytest.importorskip("torch")
    w = W.WORKLOADS["decode"].with_tokens(8)
    q, scale = W.make_hidden(w)
    assert q.dtype == torch.uint8 and q.shape == (8, w.hidden_size)
    assert scale.dtype == torch.float32 and scale.shape == (8,)
    deq = q.view(torch.float8_e4m3fn).to(torch.float32) * scale[:, None]
    x = W._randn((8, w.hidden_size), W._streams(0)["hidden_seed"], "cpu")
    # e4m3 keeps 3 fraction bits: relative error <= 2^-4 above the subnormal range
    big = x.abs() > scale[:, None] * 2.0**-6
    assert torch.all((deq - x).abs()[big] <= 2.0**-4 * x.abs()[big])
    # the row maximum maps to +-448
    assert torch.all(q.view(torch.float8_e4m3fn).to(torch.float32).abs().amax(dim=1) == 448.0)
