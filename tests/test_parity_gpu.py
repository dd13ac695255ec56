"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: expert_first_token_offset, permuted_idx, inv_permuted_idx, permuted rows
and permuted scales bit-exact; unpermute within 2^-7 * max(1, |ref|) for
bf16 and 1e-5 * max(1, |ref|) for fp32.  Every output buffer and the
workspace are filled with 0xFF before each call, so a result that leans on
earlier memory contents fails.
"""

import hashlib
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _parity import (POISON, assert_permute_equal, assert_permute_local_equal, assert_unpermute_close, gpu_permute,
                     gpu_permute_local, gpu_unpermute, oracle_permute, oracle_permute_local, poisoned, to_np)
from mixture_experts_token_amd import binding

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _say(msg):
    print("[case] " + msg, flush=True)


def _inputs(name, dev, seed=0, n=None):
    w = W.WORKLOADS[name]
    if n is not None:
        w = w.with_tokens(n)
    gen_dev = "cpu" if w.num_rows * w.hidden_size <= (1 << 22) else dev
    inp = W.make_all(w, seed=seed, device=gen_dev)
    for key in ("topk_ids", "topk_weights", "hidden_states", "token_scale", "expert_output"):
        if inp[key] is not None:
            inp[key] = inp[key].to(dev)
    return w, inp


def _run_and_check(w, inp):
    _say("%s N=%d H=%d E=%d topk=%d %s" % (w.name, w.num_tokens, w.hidden_size, w.num_experts, w.topk,
                                           w.hidden_dtype))
    outs = gpu_permute(inp["hidden_states"], inp["topk_ids"], w.num_experts, token_scale=inp["token_scale"])
    out = gpu_unpermute(inp["expert_output"], inp["topk_weights"], outs["inv_permuted_idx"])
    torch.cuda.synchronize()
    ref = oracle_permute(inp["hidden_states"], inp["topk_ids"], w.num_experts, inp["token_scale"])
    assert_permute_equal(outs, ref)
    y = to_np(inp["expert_output"])
    wts = to_np(inp["topk_weights"])
    inv = ref["inv_permuted_idx"]
    ref_out = oracle.unpermute(y, wts, inv, w.output_dtype)
    return assert_unpermute_close(to_np(out), ref_out, w.output_dtype)


@pytest.mark.parametrize("name", ["tiny", "mixtral", "qwen3"])
def test_workload_parity(name, hip_device):
    w, inp = _inputs(name, hip_device)
    _run_and_check(w, inp)


def test_dsv3_parity_full(hip_device):
    """Every output of the DSv3-shaped call against the oracle: indices, all
    131072 permuted rows, and the unpermute of all 16384 tokens."""
    w, inp = _inputs("dsv3", hip_device)
    _run_and_check(w, inp)


def test_tiny_matches_stored_golden(hip_device):
    g = json.load(open(os.path.join(HERE, "golden", "tiny_seed0.json")))
    w, inp = _inputs("tiny", hip_device)
    _say("tiny golden")
    outs = gpu_permute(inp["hidden_states"], inp["topk_ids"], w.num_experts)
    torch.cuda.synchronize()
    assert to_np(outs["expert_first_token_offset"]).tolist() == g["expected"]["expert_first_token_offset"]
    assert to_np(outs["permuted_idx"]).tolist() == g["expected"]["permuted_idx"]
    assert to_np(outs["inv_permuted_idx"]).tolist() == g["expected"]["inv_permuted_idx"]
    sha = hashlib.sha256(to_np(outs["permuted_hidden_states"]).tobytes()).hexdigest()
    assert sha == g["expected"]["permuted_hidden_states_sha256"]


def test_decode_sweep_with_one_reused_scratch(hip_device):
    """Scratch sized once for N=256 and reused for N = 1, 4, 16, 64, 256 in that order."""
    w, inp = _inputs("decode", hip_device)
    dev = hip_device
    scratch = binding.MoEPermuteScratch(256, w.topk, w.num_experts, dev, hidden_size=w.hidden_size,
                                        hidden_dtype=torch.uint8, with_scale=True)
    scratch.workspace.fill_(POISON)
    scratch.permuted_hidden_states.fill_(POISON)
    for n in W.DECODE_SWEEP:
        _say("decode sweep N=%d (reused scratch)" % n)
        x = inp["hidden_states"][:n]
        s = inp["token_scale"][:n]
        ids = inp["topk_ids"][:n]
        res = scratch.permute(x, ids, token_scale=s)
        out = gpu_unpermute(inp["expert_output"][: n * w.topk], inp["topk_weights"][:n], res["inv_permuted_idx"])
        fresh = gpu_permute(x, ids, w.num_experts, token_scale=s)
        torch.cuda.synchronize()
        ref = oracle_permute(x, ids, w.num_experts, s)
        assert_permute_equal(res, ref)
        assert_permute_equal(fresh, ref)
        ref_out = oracle.unpermute(to_np(inp["expert_output"][: n * w.topk]), to_np(inp["topk_weights"][:n]),
                                   ref["inv_permuted_idx"], "bf16")
        assert_unpermute_close(to_np(out), ref_out, "bf16")


# ----------------------------------------------------------------------------
# Edge cases: several tiles with ragged tails, both permute schedules.
# ----------------------------------------------------------------------------
def _edge_ids(rng, n, k, e, mode):
    if mode == "distinct":
        return np.stack([rng.permutation(e)[:k] for _ in range(n)]) if n else np.zeros((0, k))
    if mode == "one_expert":
        return np.full((n, k), e - 1)
    if mode == "first_expert":
        return np.zeros((n, k))
    if mode == "dups":
        return rng.integers(0, e, size=(n, k))
    if mode == "empties":  # experts 0, E-1 and every third one never chosen
        allowed = np.array([x for x in range(1, e - 1) if x % 3])
        return np.stack([rng.choice(allowed, k, replace=False) for _ in range(n)])
    raise ValueError(mode)


EDGE = [
    # (N, topk, E, H, dtype, ids mode)
    (1, 1, 1, 8, "f32", "distinct"),
    (5, 4, 4, 64, "bf16", "distinct"),
    (3000, 2, 64, 136, "bf16", "one_expert"),
    (5000, 4, 16, 72, "bf16", "first_expert"),
    (1000, 3, 3, 4, "f32", "dups"),
    (9000, 3, 5, 40, "bf16", "dups"),
    (4099, 8, 1024, 64, "bf16", "distinct"),
    (100, 16, 1024, 128, "f32", "distinct"),
    (2500, 8, 1000, 96, "bf16", "empties"),
    (2048, 8, 256, 264, "bf16", "distinct"),   # exactly the largest fused row count
    (2049, 8, 256, 264, "bf16", "distinct"),   # one token past the fused bound: the first coarse row count
    (777, 3, 37, 328, "f32", "distinct"),
    (300, 64, 512, 16, "bf16", "distinct"),
    (40, 512, 1024, 8, "f32", "distinct"),
    (20, 600, 1000, 24, "bf16", "distinct"),
    (3001, 8, 160, 7168, "bf16", "empties"),
    (513, 8, 256, 16, "fp8_e4m3", "distinct"),
    (2600, 8, 256, 7168, "fp8_e4m3", "distinct"),
    (140000, 2, 16, 8, "bf16", "dups"),        # > 2048 tiles: the tile scan takes several passes
    # the wave schedule (at most 128 rows, one wave per workgroup) holds 1 or 2 ids per lane
    (64, 1, 5, 32, "fp8_e4m3", "dups"),        # 64 rows: one batch, fp8 codes with scales
    (65, 1, 5, 32, "fp8_e4m3", "dups"),        # 65 rows: two
    (32, 4, 9, 1040, "bf16", "dups"),          # 128 rows, the largest wave call; 130-vector rows, ragged
    (4, 32, 1024, 96, "bf16", "distinct"),     # 128 rows over 1024 experts (16 per lane in the scan)
    # the fused kernel holds 1, 4, 16 or 32 id batches of 512 per thread: each side of each switch
    (43, 3, 7, 200, "f32", "distinct"),        # 129 rows: the first fused call, one batch
    (32, 8, 64, 32, "bf16", "one_expert"),     # 256 rows, every row one expert
    (64, 8, 256, 7168, "fp8_e4m3", "empties"),  # 512 rows: one batch (decode N = 64)
    (65, 8, 256, 16, "bf16", "distinct"),      # 520 rows: four
    (1024, 2, 8, 16, "bf16", "dups"),          # 2048 rows: four
    (1025, 2, 8, 16, "bf16", "dups"),          # 2050 rows: sixteen
    (4096, 2, 8, 16, "f32", "distinct"),       # 8192 rows: sixteen
    (4097, 2, 8, 16, "f32", "distinct"),       # 8194 rows: thirty-two
]


@pytest.mark.parametrize("n,k,e,h,dtype,mode", EDGE, ids=["-".join(map(str, c)) for c in EDGE])
def test_edge_case_parity(hip_device, n, k, e, h, dtype, mode):
    dev = hip_device
    rng = np.random.default_rng(n * 31 + k * 7 + e)
    ids = torch.from_numpy(_edge_ids(rng, n, k, e, mode).astype(np.int32)).to(dev)
    g = torch.Generator(device="cpu").manual_seed(n + k + e)
    xf = torch.randn((n, h), generator=g)
    scale = None
    if dtype == "f32":
        x = xf
    elif dtype == "bf16":
        x = xf.to(torch.bfloat16)
    else:
        x, scale = W.quantize_fp8_per_token(xf)
        scale = scale.to(dev)
    x = x.to(dev)
    out_dtype = "f32" if dtype == "f32" else "bf16"
    y = torch.randn((n * k, h), generator=g)
    y = (y if out_dtype == "f32" else y.to(torch.bfloat16)).to(dev)
    wts = torch.softmax(torch.randn((n, k), generator=g, dtype=torch.float64), dim=1).to(torch.float32).to(dev)
    _say("edge N=%d topk=%d E=%d H=%d %s %s" % (n, k, e, h, dtype, mode))
    outs = gpu_permute(x, ids, e, token_scale=scale)
    out = gpu_unpermute(y, wts, outs["inv_permuted_idx"])
    torch.cuda.synchronize()
    ref = oracle_permute(x, ids, e, scale)
    assert_permute_equal(outs, ref)
    ref_out = oracle.unpermute(to_np(y), to_np(wts), ref["inv_permuted_idx"], out_dtype)
    assert_unpermute_close(to_np(out), ref_out, out_dtype)


def test_sizes_that_loop_inside_kernels(hip_device):
    """4.3M tokens with topk 1: the tile scan runs many passes and unpermute waves
    loop over items (more items than the capped grid has waves)."""
    n, k, e, h = 4_300_000, 1, 4, 8
    rng = np.random.default_rng(17)
    ids = torch.from_numpy(rng.integers(0, e, size=(n, k)).astype(np.int32)).to(hip_device)
    x = torch.randn((n, h), device=hip_device).to(torch.bfloat16)
    y = torch.randn((n * k, h), device=hip_device).to(torch.bfloat16)
    wts = torch.rand((n, k), device=hip_device) + 0.5
    _say("looping sizes N=%d topk=%d E=%d H=%d" % (n, k, e, h))
    outs = gpu_permute(x, ids, e)
    out = gpu_unpermute(y, wts, outs["inv_permuted_idx"])
    torch.cuda.synchronize()
    ref = oracle_permute(x, ids, e)
    assert_permute_equal(outs, ref)
    ref_out = oracle.unpermute(to_np(y), to_np(wts), ref["inv_permuted_idx"], "bf16")
    assert_unpermute_close(to_np(out), ref_out, "bf16")


@pytest.mark.parametrize("n,k,e", [(700, 4, 32), (6000, 4, 32)])
def test_index_only_permute(hip_device, n, k, e):
    rng = np.random.default_rng(5)
    ids = torch.from_numpy(_edge_ids(rng, n, k, e, "distinct").astype(np.int32)).to(hip_device)
    _say("index-only N=%d topk=%d E=%d" % (n, k, e))
    outs = gpu_permute(None, ids, e)
    torch.cuda.synchronize()
    assert_permute_equal(outs, oracle_permute(None, ids, e), check_rows=False)


@pytest.mark.parametrize("n,k,e", [(5, 8, 256), (700, 4, 32)])
def test_index_only_permute_moves_scales(hip_device, n, k, e):
    """hidden_size 0 with per-token scales: no rows, the scales still move."""
    rng = np.random.default_rng(6)
    ids = torch.from_numpy(_edge_ids(rng, n, k, e, "distinct").astype(np.int32)).to(hip_device)
    scale = torch.rand(n, device=hip_device) + 0.25
    _say("index-only with scales N=%d topk=%d E=%d" % (n, k, e))
    outs = gpu_permute(None, ids, e, token_scale=scale)
    torch.cuda.synchronize()
    assert_permute_equal(outs, oracle_permute(None, ids, e, scale), check_rows=False)


def test_zero_tokens(hip_device):
    ids = torch.zeros((0, 2), dtype=torch.int32, device=hip_device)
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=hip_device)
    _say("zero tokens")
    outs = gpu_permute(x, ids, 8)
    out = gpu_unpermute(torch.zeros((0, 64), dtype=torch.bfloat16, device=hip_device),
                        torch.zeros((0, 2), dtype=torch.float32, device=hip_device), outs["inv_permuted_idx"])
    torch.cuda.synchronize()
    assert to_np(outs["expert_first_token_offset"]).tolist() == [0] * 9
    assert out.shape == (0, 64)


# ----------------------------------------------------------------------------
# Split schedule: from 2^30 bytes of expanded rows (no expert map) the index is
# written by the index-only schedule and a separate kernel copies the rows.
# The DSv3-shaped call (topk 8) is compared in full above; these cover the
# other copy kernels (topk 4 and 2, and a runtime topk), a ragged last chunk,
# the threshold itself, moved scales and the rejected-id path.  Indices are
# compared with the oracle in full; rows and scales against a gather of the
# inputs by the (already verified) permuted_idx, on the device.
# ----------------------------------------------------------------------------
SPLIT_CASES = [
    # (N, topk, E, H bf16): N*topk*H*2 bytes >= 2^30
    (65536, 3, 64, 2816),    # runtime-topk kernel; rows of 352 vectors: a ragged second chunk
    (65536, 4, 128, 2048),   # exactly 2^30 bytes: the first size that splits
    (131072, 2, 8, 4096),    # topk 2 (non-temporal row stores)
]


def _distinct_ids(rng, n, k, e):
    return np.argsort(rng.random((n, e)), axis=1)[:, :k].astype(np.int32)


@pytest.mark.parametrize("n,k,e,h", SPLIT_CASES, ids=["-".join(map(str, c)) for c in SPLIT_CASES])
def test_split_schedule_parity(hip_device, n, k, e, h):
    assert n * k * h * 2 >= 1 << 30
    rng = np.random.default_rng(n + k)
    ids_np = _distinct_ids(rng, n, k, e)
    ids = torch.from_numpy(ids_np).to(hip_device)
    g = torch.Generator(device=hip_device).manual_seed(k)
    x = torch.randn((n, h), device=hip_device, generator=g).to(torch.bfloat16)
    scale = torch.rand(n, device=hip_device, generator=g) + 0.5
    _say("split schedule N=%d topk=%d E=%d H=%d" % (n, k, e, h))
    outs = gpu_permute(x, ids, e, token_scale=scale)
    torch.cuda.synchronize()
    ref = oracle_permute(None, ids, e)
    for key in ("expert_first_token_offset", "permuted_idx", "inv_permuted_idx"):
        np.testing.assert_array_equal(to_np(outs[key]), ref[key], err_msg=key)
    src = outs["permuted_idx"].long() // k
    assert torch.equal(outs["permuted_hidden_states"].view(torch.int16), x.view(torch.int16)[src])
    assert torch.equal(outs["permuted_scale"], scale[src])


def test_split_schedule_rejected_id_writes_nothing(hip_device):
    """DSv3 shape (split schedule) with one expert id out of range: offsets -1,
    and the index and all 1.88 GB of row buffer keep their poison."""
    w = W.WORKLOADS["dsv3"]
    rng = np.random.default_rng(11)
    ids_np = _distinct_ids(rng, w.num_tokens, w.topk, w.num_experts)
    ids_np[w.num_tokens - 5, 3] = w.num_experts
    ids = torch.from_numpy(ids_np).to(hip_device)
    x = torch.randn((w.num_tokens, w.hidden_size), device=hip_device).to(torch.bfloat16)
    _say("split schedule, bad id")
    outs = gpu_permute(x, ids, w.num_experts)
    torch.cuda.synchronize()
    assert to_np(outs["expert_first_token_offset"]).tolist() == [-1] * (w.num_experts + 1)
    for key in ("permuted_idx", "inv_permuted_idx", "permuted_hidden_states"):
        assert bool((outs[key].view(torch.uint8) == POISON).all()), key


@pytest.mark.parametrize("n,k,e,bad", [(50, 2, 8, 8), (50, 2, 8, -1), (4000, 8, 64, 64), (4000, 8, 64, -7)])
def test_out_of_range_expert_id_is_reported(hip_device, n, k, e, bad):
    """The kernels' own check: offsets become -1 and nothing else is written."""
    rng = np.random.default_rng(3)
    ids_np = _edge_ids(rng, n, k, e, "distinct").astype(np.int32)
    ids_np[n // 2, k - 1] = bad
    ids = torch.from_numpy(ids_np).to(hip_device)
    x = torch.randn((n, 32), device=hip_device).to(torch.bfloat16)
    _say("bad id %d N=%d topk=%d E=%d" % (bad, n, k, e))
    outs = gpu_permute(x, ids, e)
    torch.cuda.synchronize()
    assert to_np(outs["expert_first_token_offset"]).tolist() == [-1] * (e + 1)
    for key in ("permuted_idx", "inv_permuted_idx", "permuted_hidden_states"):
        assert np.all(to_np(outs[key]).view(np.uint8) == POISON), key


@pytest.mark.parametrize("k", [1, 2, 3, 4, 8])
def test_out_of_range_inverse_index_gives_nan_row(hip_device, k):
    n, h = 64, 128
    inv = torch.randperm(n * k, dtype=torch.int32).to(hip_device)
    inv[10 * k + (k - 1)] = n * k  # token 10 points past the end
    y = torch.randn((n * k, h), device=hip_device).to(torch.bfloat16)
    wts = torch.full((n, k), 1.0 / k, device=hip_device)
    _say("bad inverse index topk=%d" % k)
    out = gpu_unpermute(y, wts, inv)
    torch.cuda.synchronize()
    o = out.float().cpu()
    assert torch.isnan(o[10]).all()
    keep = [t for t in range(n) if t != 10]
    inv_np = to_np(inv).reshape(n, k)
    y_np = to_np(y)
    rows = inv_np[keep].reshape(-1)
    ref = oracle.unpermute(y_np[rows], to_np(wts)[keep], np.arange(rows.size, dtype=np.int32), "bf16")
    assert_unpermute_close(to_np(out)[keep], ref, "bf16")


# ----------------------------------------------------------------------------
# Reuse, determinism, streams, round trip.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["mixtral", "qwen3"])
def test_scratch_reuse_same_pointers_identical_results(hip_device, name):
    """Two calls with one scratch: same output pointers, identical bits (as the
    pages' reuse test asserts), also after the scratch is poisoned in between."""
    w, inp = _inputs(name, hip_device, n=W.WORKLOADS[name].num_tokens // 2)
    scratch = binding.MoEPermuteScratch(w.num_tokens, w.topk, w.num_experts, hip_device,
                                        hidden_size=w.hidden_size, hidden_dtype=torch.bfloat16)
    _say("reuse %s" % name)
    r1 = scratch.permute(inp["hidden_states"], inp["topk_ids"])
    snap1 = {k: v.clone() for k, v in r1.items() if v is not None}
    ptrs1 = {k: v.data_ptr() for k, v in r1.items() if v is not None}
    scratch.workspace.fill_(POISON)
    scratch.permuted_hidden_states.fill_(POISON)
    scratch.permuted_idx.fill_(-1)
    r2 = scratch.permute(inp["hidden_states"], inp["topk_ids"])
    torch.cuda.synchronize()
    for k, v in r2.items():
        if v is None:
            continue
        assert v.data_ptr() == ptrs1[k], k
        assert torch.equal(v.view(torch.uint8) if v.dtype == torch.bfloat16 else v,
                           snap1[k].view(torch.uint8) if v.dtype == torch.bfloat16 else snap1[k]), k


def test_smaller_call_after_larger_one(hip_device):
    """Leftovers of a larger call in the scratch must not leak into a smaller one."""
    w, inp = _inputs("qwen3", hip_device)
    scratch = binding.MoEPermuteScratch(w.num_tokens, w.topk, w.num_experts, hip_device,
                                        hidden_size=w.hidden_size, hidden_dtype=torch.bfloat16)
    scratch.permute(inp["hidden_states"], inp["topk_ids"])
    for n in (3000, 2049, 2048, 100, 1):
        _say("qwen3 prefix N=%d after full call" % n)
        res = scratch.permute(inp["hidden_states"][:n], inp["topk_ids"][:n])
        torch.cuda.synchronize()
        assert_permute_equal(res, oracle_permute(inp["hidden_states"][:n], inp["topk_ids"][:n], w.num_experts))


@pytest.mark.parametrize("name", ["tiny", "qwen3", "dsv3"])
def test_repeat_is_bit_identical(hip_device, name):
    w, inp = _inputs(name, hip_device, n=min(W.WORKLOADS[name].num_tokens, 4096))
    _say("repeat %s" % name)
    a = gpu_permute(inp["hidden_states"], inp["topk_ids"], w.num_experts)
    oa = gpu_unpermute(inp["expert_output"], inp["topk_weights"], a["inv_permuted_idx"])
    b = gpu_permute(inp["hidden_states"], inp["topk_ids"], w.num_experts)
    ob = gpu_unpermute(inp["expert_output"], inp["topk_weights"], b["inv_permuted_idx"])
    torch.cuda.synchronize()
    for k in a:
        if a[k] is not None:
            assert np.array_equal(to_np(a[k]).view(np.uint8), to_np(b[k]).view(np.uint8)), k
    assert np.array_equal(to_np(oa).view(np.uint8), to_np(ob).view(np.uint8))


def test_non_default_stream_with_queued_work(hip_device):
    w, inp = _inputs("qwen3", hip_device)
    s = torch.cuda.Stream(device=hip_device)
    big = torch.randn((4096, 4096), device=hip_device)
    ref = oracle_permute(inp["hidden_states"], inp["topk_ids"], w.num_experts)
    _say("side stream")
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(4):
            big = big * 1.0001  # queue work ahead of the permute on the same stream
        outs = gpu_permute(inp["hidden_states"], inp["topk_ids"], w.num_experts, stream=s)
        out = gpu_unpermute(inp["expert_output"], inp["topk_weights"], outs["inv_permuted_idx"], stream=s)
    s.synchronize()
    assert_permute_equal(outs, ref)
    ref_out = oracle.unpermute(to_np(inp["expert_output"]), to_np(inp["topk_weights"]), ref["inv_permuted_idx"],
                               "bf16")
    assert_unpermute_close(to_np(out), ref_out, "bf16")


@pytest.mark.parametrize("k,e", [(1, 8), (2, 8), (4, 64), (8, 256)])
def test_round_trip_identity_experts_bf16_exact(hip_device, k, e):
    """unpermute(permute(x)) with Y = permuted x and weights 1/topk gives x back bit for bit."""
    n, h = 3000, 256
    rng = np.random.default_rng(k)
    ids = torch.from_numpy(_edge_ids(rng, n, k, e, "distinct").astype(np.int32)).to(hip_device)
    x = torch.randn((n, h), device=hip_device).to(torch.bfloat16)
    _say("round trip topk=%d" % k)
    outs = gpu_permute(x, ids, e)
    wts = torch.full((n, k), 1.0 / k, device=hip_device)
    out = gpu_unpermute(outs["permuted_hidden_states"], wts, outs["inv_permuted_idx"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), x.view(torch.int16))


@pytest.mark.parametrize("name,n", [("decode", 64), ("qwen3", 3000)])
def test_graph_replay_matches_eager(hip_device, name, n):
    """permute + unpermute captured in a HIP graph: every replay equals the eager result,
    with eager work and a poisoning of the outputs between replays."""
    w, inp = _inputs(name, hip_device, n=n)
    _say("graph replay %s N=%d" % (name, n))
    eager = gpu_permute(inp["hidden_states"], inp["topk_ids"], w.num_experts, token_scale=inp["token_scale"])
    eager_out = gpu_unpermute(inp["expert_output"], inp["topk_weights"], eager["inv_permuted_idx"])
    torch.cuda.synchronize()
    ref_bytes = {k: to_np(v).view(np.uint8).copy() for k, v in eager.items() if v is not None}
    ref_out = to_np(eager_out).view(np.uint8).copy()

    outs = {k: (None if v is None else torch.empty_like(v)) for k, v in eager.items()}
    ws = poisoned((max(16, binding.moe_permute_workspace_size(w.num_tokens, w.topk, w.num_experts)),),
                  torch.uint8, hip_device)
    out = torch.empty_like(eager_out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.moe_permute(inp["hidden_states"], inp["topk_ids"], w.num_experts, outs["permuted_hidden_states"],
                            outs["expert_first_token_offset"], outs["permuted_idx"], outs["inv_permuted_idx"], ws,
                            token_scale=inp["token_scale"], permuted_scale=outs["permuted_scale"])
        binding.moe_unpermute(inp["expert_output"], inp["topk_weights"], outs["inv_permuted_idx"], out)
    scratch = torch.randn((2048, 2048), device=hip_device)
    for rep in range(3):
        for v in list(outs.values()) + [out, ws]:
            if v is not None:
                v.view(torch.uint8).fill_(POISON)
        scratch = scratch @ scratch.T * 1e-3  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            if v is not None:
                assert np.array_equal(to_np(v).view(np.uint8), ref_bytes[k]), (rep, k)
        assert np.array_equal(to_np(out).view(np.uint8), ref_out), rep


# ----------------------------------------------------------------------------
# int64 expert ids, read directly (no cast pass).
# ----------------------------------------------------------------------------
I64_CASES = [("tiny", None), ("mixtral", None), ("qwen3", None), ("dsv3", 3000), ("decode", 256)]


@pytest.mark.parametrize("name,n", I64_CASES, ids=["%s-%s" % c for c in I64_CASES])
def test_int64_ids_match_oracle_and_int32_path(hip_device, name, n):
    w, inp = _inputs(name, hip_device, n=n)
    ids64 = inp["topk_ids"].to(torch.int64)
    _say("int64 ids %s N=%d" % (name, w.num_tokens))
    o64 = gpu_permute(inp["hidden_states"], ids64, w.num_experts, token_scale=inp["token_scale"])
    o32 = gpu_permute(inp["hidden_states"], inp["topk_ids"], w.num_experts, token_scale=inp["token_scale"])
    torch.cuda.synchronize()
    ref = oracle_permute(inp["hidden_states"], ids64, w.num_experts, inp["token_scale"])
    assert_permute_equal(o64, ref)
    for key, v in o64.items():
        if v is not None:
            assert torch.equal(v.view(torch.uint8), o32[key].view(torch.uint8)), key


@pytest.mark.parametrize("n,k,e", [(3000, 2, 16), (30000, 8, 256), (140000, 2, 16)])
def test_int64_ids_all_schedules_and_local(hip_device, n, k, e):
    rng = np.random.default_rng(n + k)
    ids64 = torch.from_numpy(rng.integers(0, e, size=(n, k)).astype(np.int64)).to(hip_device)
    x = torch.randn((n, 64), device=hip_device).to(torch.bfloat16)
    _say("int64 ids N=%d topk=%d E=%d" % (n, k, e))
    outs = gpu_permute(x, ids64, e)
    emap, nl = W.expert_map_for(e, 4, 1, "shuffled")
    louts = gpu_permute_local(x, ids64, e, emap, nl)
    torch.cuda.synchronize()
    assert_permute_equal(outs, oracle_permute(x, ids64, e))
    assert_permute_local_equal(louts, oracle_permute_local(x, ids64, e, emap, nl))


@pytest.mark.parametrize("bad", [2**32 + 3, -1, 2**31, -(2**32)])
@pytest.mark.parametrize("n,k,e", [(50, 2, 8), (4000, 8, 64), (30000, 8, 256), (140000, 2, 16)])
def test_int64_ids_outside_range_detected_not_truncated(hip_device, n, k, e, bad):
    """Values whose low 32 bits would be a valid id must still be rejected."""
    rng = np.random.default_rng(7)
    ids_np = rng.integers(0, e, size=(n, k)).astype(np.int64)
    ids_np[n // 3, k - 1] = bad
    ids64 = torch.from_numpy(ids_np).to(hip_device)
    _say("int64 bad id %d N=%d E=%d" % (bad, n, e))
    outs = gpu_permute(None, ids64, e)
    emap, nl = W.expert_map_for(e, 2, 0)
    louts = gpu_permute_local(None, ids64, e, emap, nl)
    torch.cuda.synchronize()
    assert to_np(outs["expert_first_token_offset"]).tolist() == [-1] * (e + 1)
    assert np.all(to_np(outs["inv_permuted_idx"]).view(np.uint32) == 0xFFFFFFFF)
    assert to_np(louts["expert_first_token_offset"]).tolist() == [-1] * (nl + 1)
