"""GPU parity of the local-expert permute (expert parallelism) against the oracle.

The reading pinned in the oracle: the expert map sends a global expert to its
local id or -1; local rows are counted, stably ordered by local id and copied;
other rows get inverse index -1, are not copied, and add nothing when
unpermuted.  Bar as for the plain permute: offsets, indices, rows and scales
bit-exact (the permuted buffers past the local rows must keep their poison);
unpermute within 2^-7 * max(1, |ref|) for bf16, 1e-5 * max(1, |ref|) for fp32.
Both reductions of a local inverse index, moe_unpermute_local and
moe_unpermute (different occupancy, same kernel arithmetic), must agree bit
for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _parity import (POISON, assert_permute_equal, assert_permute_local_equal, assert_unpermute_close, gpu_permute,
                     gpu_permute_local, gpu_unpermute, oracle_permute_local, poisoned, to_np)
from mixture_experts_token_amd import binding

pytestmark = pytest.mark.gpu


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


def _assert_same_bits(a, b):
    assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.uint8) if b.dtype == torch.bfloat16 else b.view(torch.int32)), \
        "moe_unpermute_local and moe_unpermute differ"


def _unpermute_ref(y, wts, inv, k, dtype):
    """Oracle unpermute of every token (a -1 slot adds nothing)."""
    return oracle.unpermute(y, wts, inv, dtype)


CASES = [
    # (workload, ep_size, rank, layout, tokens or None); every token is compared
    ("tiny", 2, 1, "contiguous", None),
    ("mixtral", 2, 0, "contiguous", None),
    ("mixtral", 4, 3, "shuffled", None),
    ("qwen3", 4, 1, "round_robin", None),
    ("qwen3", 8, 7, "shuffled", None),
    ("dsv3", 8, 0, "contiguous", None),     # the most popular experts sit in some rank's share
    ("dsv3", 8, 5, "round_robin", 6000),
    ("decode", 8, 5, "contiguous", None),   # fp8 codes + per-token scales
    ("decode", 8, 2, "shuffled", 1),
]


@pytest.mark.parametrize("name,ep,rank,layout,n", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_local_workload_parity(hip_device, name, ep, rank, layout, n):
    w, inp = _inputs(name, hip_device, n=n)
    emap, nl = W.expert_map_for(w.num_experts, ep, rank, layout)
    _say("local %s N=%d E=%d topk=%d ep=%d rank=%d %s" % (name, w.num_tokens, w.num_experts, w.topk, ep, rank, layout))
    outs = gpu_permute_local(inp["hidden_states"], inp["topk_ids"], w.num_experts, emap, nl,
                             token_scale=inp["token_scale"])
    out = gpu_unpermute(inp["expert_output"], inp["topk_weights"], outs["inv_permuted_idx"], local=True)
    out_plain = gpu_unpermute(inp["expert_output"], inp["topk_weights"], outs["inv_permuted_idx"])
    torch.cuda.synchronize()
    ref = oracle_permute_local(inp["hidden_states"], inp["topk_ids"], w.num_experts, emap, nl, inp["token_scale"])
    assert_permute_local_equal(outs, ref)
    y, wts, inv = to_np(inp["expert_output"]), to_np(inp["topk_weights"]), ref["inv_permuted_idx"]
    assert_unpermute_close(to_np(out), _unpermute_ref(y, wts, inv, w.topk, w.output_dtype), w.output_dtype)
    _assert_same_bits(out, out_plain)


def _ids(rng, n, k, e, mode):
    if mode == "distinct":
        return np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    return rng.integers(0, e, size=(n, k)).astype(np.int32)


EDGE = [
    # (N, topk, E, H, dtype, ids mode, map kind) -- the schedules: fused up to 16384 rows, then coarse, staged
    (1, 1, 4, 8, "f32", "distinct", "half"),
    (3, 2, 8, 64, "bf16", "distinct", "none_local"),
    (1000, 4, 16, 64, "f32", "dups", "identity"),
    (1000, 4, 16, 64, "bf16", "dups", "shared_local"),
    (4097, 3, 12, 136, "bf16", "distinct", "odd"),
    (16384, 2, 64, 72, "f32", "dups", "half"),          # 32768 rows: coarse
    (30000, 8, 256, 8, "bf16", "distinct", "odd"),      # coarse, many tiles
    (140000, 2, 16, 8, "bf16", "dups", "half"),         # staged
    (140000, 2, 16, 8, "bf16", "dups", "none_local"),   # staged, nothing local
]


def _edge_map(kind, e, rng):
    if kind == "identity":
        return np.arange(e, dtype=np.int32), e
    if kind == "none_local":
        return np.full(e, -1, dtype=np.int32), 1
    if kind == "half":
        m = np.full(e, -1, dtype=np.int32)
        m[e // 2:] = np.arange(e - e // 2)
        return m, e - e // 2
    if kind == "shared_local":  # global experts g and g + e/2 share local id g
        m = np.full(e, -1, dtype=np.int32)
        m[: e // 4] = np.arange(e // 4)
        m[e // 2: e // 2 + e // 4] = np.arange(e // 4)
        return m, e // 4
    if kind == "odd":  # odd experts, numbered in a random order
        odd = np.arange(1, e, 2)
        m = np.full(e, -1, dtype=np.int32)
        m[odd] = rng.permutation(odd.size)
        return m, odd.size
    raise ValueError(kind)


@pytest.mark.parametrize("n,k,e,h,dtype,mode,kind", EDGE, ids=["-".join(map(str, c)) for c in EDGE])
def test_local_edge_parity(hip_device, n, k, e, h, dtype, mode, kind):
    dev = hip_device
    rng = np.random.default_rng(n * 17 + k * 5 + e)
    ids = torch.from_numpy(_ids(rng, n, k, e, mode)).to(dev)
    emap, nl = _edge_map(kind, e, rng)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    x = torch.randn((n, h), generator=torch.Generator().manual_seed(n + h)).to(tdt).to(dev)
    y = torch.randn((n * k, h), generator=torch.Generator().manual_seed(n + h + 1)).to(tdt).to(dev)
    wts = torch.rand((n, k), generator=torch.Generator().manual_seed(n + 2)).to(dev)
    _say("local edge N=%d topk=%d E=%d H=%d %s %s %s" % (n, k, e, h, dtype, mode, kind))
    outs = gpu_permute_local(x, ids, e, emap, nl)
    out = gpu_unpermute(y, wts, outs["inv_permuted_idx"], local=True)
    out_plain = gpu_unpermute(y, wts, outs["inv_permuted_idx"])
    torch.cuda.synchronize()
    ref = oracle_permute_local(x, ids, e, emap, nl)
    assert_permute_local_equal(outs, ref)
    assert_unpermute_close(to_np(out), oracle.unpermute(to_np(y), to_np(wts), ref["inv_permuted_idx"], dtype), dtype)
    _assert_same_bits(out, out_plain)
    if kind == "identity":  # every expert local: exactly the plain permute
        plain = gpu_permute(x, ids, e)
        torch.cuda.synchronize()
        for key in ("expert_first_token_offset", "permuted_idx", "inv_permuted_idx"):
            assert torch.equal(plain[key], outs[key]), key
        assert torch.equal(plain["permuted_hidden_states"].view(torch.uint8),
                           outs["permuted_hidden_states"].view(torch.uint8))


def test_local_zero_tokens_writes_zero_offsets(hip_device):
    ids = torch.zeros((0, 2), dtype=torch.int32, device=hip_device)
    emap, nl = W.expert_map_for(8, 2, 1)
    _say("local zero tokens")
    outs = gpu_permute_local(None, ids, 8, emap, nl)
    torch.cuda.synchronize()
    assert to_np(outs["expert_first_token_offset"]).tolist() == [0] * (nl + 1)


@pytest.mark.parametrize("n,k,e,bad", [(50, 2, 8, "past_local"), (50, 2, 8, "below_minus_one"),
                                       (30000, 8, 256, "past_local"), (140000, 2, 16, "below_minus_one")])
def test_local_bad_map_entry_detected(hip_device, n, k, e, bad):
    """A used expert whose map entry is outside [-1, L): offsets -1, nothing else written."""
    rng = np.random.default_rng(3)
    ids_np = rng.integers(0, e, size=(n, k)).astype(np.int32)
    emap, nl = W.expert_map_for(e, 2, 0)
    used = int(ids_np[n // 2, 0])
    emap[used] = nl if bad == "past_local" else -5
    ids = torch.from_numpy(ids_np).to(hip_device)
    _say("local bad map N=%d E=%d %s" % (n, e, bad))
    outs = gpu_permute_local(None, ids, e, emap, nl)
    torch.cuda.synchronize()
    assert to_np(outs["expert_first_token_offset"]).tolist() == [-1] * (nl + 1)
    assert np.all(to_np(outs["inv_permuted_idx"]).view(np.uint32) == 0xFFFFFFFF)
    assert np.all(to_np(outs["permuted_idx"]).view(np.uint32) == 0xFFFFFFFF)


def test_local_bad_entry_of_unused_expert_is_ignored(hip_device):
    n, k, e = 64, 2, 8
    ids_np = np.random.default_rng(4).integers(0, 4, size=(n, k)).astype(np.int32)  # experts 0..3 only
    emap = np.array([0, -1, 1, -1, 7, 9, -3, 2], dtype=np.int32)  # bad entries only for experts 4..6
    ids = torch.from_numpy(ids_np).to(hip_device)
    _say("local bad entry of an unused expert")
    outs = gpu_permute_local(None, ids, e, emap, 3)
    torch.cuda.synchronize()
    assert_permute_local_equal(outs, oracle_permute_local(None, ids, e, emap, 3))


def test_local_scratch_reuse_and_ranks_cover_every_slot(hip_device):
    """Scratch built with an expert map, reused across ranks' maps of one
    problem: every expanded row is local on exactly one rank, each rank's
    offsets count its rows, and a second call repeats the first bit for bit."""
    w, inp = _inputs("qwen3", hip_device, n=3000)
    ep = 4
    covered = np.zeros(w.num_rows, dtype=np.int64)
    for rank in range(ep):
        emap, nl = W.expert_map_for(w.num_experts, ep, rank, "round_robin")
        emap_t = torch.from_numpy(emap).to(hip_device)
        scratch = binding.MoEPermuteScratch(w.num_tokens, w.topk, w.num_experts, hip_device,
                                            hidden_size=w.hidden_size, hidden_dtype=torch.bfloat16,
                                            expert_map=emap_t, num_local_experts=nl)
        assert scratch.expert_first_token_offset.numel() == nl + 1
        _say("local scratch rank %d" % rank)
        r1 = scratch.permute(inp["hidden_states"], inp["topk_ids"])
        snap = {k: v.clone() for k, v in r1.items() if v is not None}
        scratch.workspace.fill_(POISON)
        r2 = scratch.permute(inp["hidden_states"], inp["topk_ids"])
        torch.cuda.synchronize()
        for key, v in r2.items():
            if v is not None:
                assert torch.equal(v.view(torch.uint8) if v.dtype == torch.bfloat16 else v,
                                   snap[key].view(torch.uint8) if v.dtype == torch.bfloat16 else snap[key]), key
        inv = to_np(r2["inv_permuted_idx"])
        covered += inv >= 0
        assert int(to_np(r2["expert_first_token_offset"])[-1]) == int((inv >= 0).sum())
    assert covered.tolist() == [1] * w.num_rows


@pytest.mark.parametrize("local", [False, True], ids=["unpermute", "unpermute_local"])
@pytest.mark.parametrize("k", [1, 2, 3, 4, 8])
def test_unpermute_minus_one_slots_skip_and_others_nan(hip_device, k, local):
    """-1 slots add nothing (their rows are not read); any other out-of-range
    index still turns its token into NaN."""
    n, h = 64, 128
    rng = np.random.default_rng(k)
    inv_np = rng.permutation(n * k).astype(np.int32)
    inv_np[rng.random(n * k) < 0.3] = -1
    inv_np[0:k] = -1                     # token 0: nothing local, zero row
    inv_np[7 * k] = -2                   # token 7: invalid
    inv = torch.from_numpy(inv_np).to(hip_device)
    y = torch.randn((n * k, h), device=hip_device).to(torch.bfloat16)
    wts = torch.rand((n, k), device=hip_device)
    wts[3, 0] = float("inf")             # weight of a -1 slot is never used
    inv[3 * k] = -1
    inv_np[3 * k] = -1
    _say("unpermute -1 slots topk=%d local=%s" % (k, local))
    out = gpu_unpermute(y, wts, inv, local=local)
    torch.cuda.synchronize()
    o = to_np(out)
    of = out.float().cpu()
    assert torch.isnan(of[7]).all()
    keep = [t for t in range(n) if t != 7]
    valid = inv_np.copy()
    valid[7 * k] = -1  # the oracle rejects the invalid entry; token 7 is not compared
    ref = oracle.unpermute(to_np(y), to_np(wts), valid, "bf16")
    assert_unpermute_close(o[keep], ref[keep], "bf16")
    assert np.all(o[0] == 0)


# (topk, hidden, dtype): rows of several 64-vector chunks with a ragged last one;
# topk 3 and 6 take the runtime-topk kernel, the others the compile-time ones.
# From topk 4 a whole-remote token's row is stored by one wave; below it, chunk
# by chunk -- both must leave no element unwritten.
REMOTE_ROWS = [(2, 1560, "bf16"), (8, 1000, "f32"), (3, 1560, "bf16"), (1, 4096, "bf16"), (4, 7168, "bf16"),
               (6, 1560, "bf16")]


@pytest.mark.parametrize("local", [False, True], ids=["unpermute", "unpermute_local"])
@pytest.mark.parametrize("k,h,dtype", REMOTE_ROWS, ids=["-".join(map(str, c)) for c in REMOTE_ROWS])
def test_unpermute_tokens_with_no_local_slot_get_whole_zero_rows(hip_device, k, h, dtype, local):
    """Tokens whose every slot is -1 get rows of +0.0 over the whole row (the
    output is poisoned first, so an unwritten chunk shows); tokens with some
    local slots are summed as usual; a token with one bad index among -1 slots
    is not taken for remote and becomes NaN."""
    n = 300
    rng = np.random.default_rng(k * 1000 + h)
    inv_np = rng.permutation(n * k).astype(np.int32)
    remote = rng.random(n) < 0.4
    remote[0] = remote[n - 1] = True
    for t in np.nonzero(remote)[0]:
        inv_np[t * k:(t + 1) * k] = -1
    part = (~remote) & (rng.random(n) < 0.3)
    for t in np.nonzero(part)[0]:
        inv_np[t * k + rng.integers(0, k)] = -1
    bad_t = 5
    inv_np[bad_t * k:(bad_t + 1) * k] = -1
    inv_np[bad_t * k + k - 1] = -3
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    y = torch.randn((n * k, h), generator=torch.Generator().manual_seed(h)).to(tdt).to(hip_device)
    wts = torch.rand((n, k), generator=torch.Generator().manual_seed(k)).to(hip_device)
    inv = torch.from_numpy(inv_np).to(hip_device)
    _say("unpermute zero rows topk=%d H=%d %s remote=%d local=%s" % (k, h, dtype, int(remote.sum()), local))
    out = gpu_unpermute(y, wts, inv, local=local)
    torch.cuda.synchronize()
    o = to_np(out)
    assert torch.isnan(out[bad_t].float().cpu()).all()
    zero_rows = np.nonzero(remote)[0]
    zero_rows = zero_rows[zero_rows != bad_t]
    assert np.all(o[zero_rows].view(np.uint8) == 0)
    valid = inv_np.copy()
    valid[bad_t * k + k - 1] = -1  # the oracle rejects the bad entry; that token is checked above
    ref = oracle.unpermute(to_np(y), to_np(wts), valid, dtype)
    keep = [t for t in range(n) if t != bad_t]
    assert_unpermute_close(o[keep], ref[keep], dtype)


# (N, H, dtype): the span schedule of moe_unpermute_local (topk 8, at least
# 32768 spans of 4 chunks): rows of 17 chunks, the last one a single vector.
SPAN_CASES = [(8192, 8200, "bf16"), (8192, 4100, "f32")]


@pytest.mark.parametrize("n,h,dtype", SPAN_CASES, ids=["-".join(map(str, c)) for c in SPAN_CASES])
def test_unpermute_local_span_schedule(hip_device, n, h, dtype):
    """moe_unpermute_local at a size that takes its span schedule, on an
    expert-split inverse index (each slot live with probability 1/6, some
    tokens with every slot remote, one token with a bad index): bit-equal to
    moe_unpermute, and equal to the oracle on a sample of tokens of every
    live-slot count."""
    k = 8
    rng = np.random.default_rng(n + h)
    rows = n * k
    inv_np = np.full(rows, -1, dtype=np.int32)
    live = rng.random(rows) < 1.0 / 6
    live[np.arange(0, 40) * k] = False        # tokens 0..39: every slot remote
    for t in range(40):
        live[t * k:(t + 1) * k] = False
    live[(40 * k):(41 * k)] = True             # token 40: all eight live
    inv_np[live] = rng.permutation(rows)[:int(live.sum())].astype(np.int32)
    bad_t = 77
    inv_np[bad_t * k + 5] = rows + 3
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    g = torch.Generator(device=hip_device).manual_seed(h)
    y = torch.randn((rows, h), device=hip_device, generator=g).to(tdt)
    wts = torch.rand((n, k), device=hip_device, generator=g)
    inv = torch.from_numpy(inv_np).to(hip_device)
    _say("unpermute_local span schedule N=%d H=%d %s" % (n, h, dtype))
    out = gpu_unpermute(y, wts, inv, local=True)
    out_plain = gpu_unpermute(y, wts, inv)
    torch.cuda.synchronize()
    _assert_same_bits(out, out_plain)
    o = to_np(out)
    assert torch.isnan(out[bad_t].float().cpu()).all()
    assert np.all(o[:40].view(np.uint8) == 0)
    # oracle on sampled tokens: their referenced rows gathered into a compact problem
    counts = live.reshape(n, k).sum(axis=1)
    sample = [t for c in range(0, k + 1) for t in np.nonzero(counts == c)[0][:6] if t != bad_t]
    sample = np.array(sorted(set(sample + list(rng.choice(n, 40, replace=False)))) , dtype=np.int64)
    sample = sample[sample != bad_t]
    sub_inv = inv_np.reshape(n, k)[sample].reshape(-1)
    used = sub_inv[sub_inv >= 0]
    remap = np.full(sub_inv.shape, -1, dtype=np.int32)
    remap[sub_inv >= 0] = np.arange(used.size, dtype=np.int32)
    y_sub = np.zeros((sample.size * k, h), dtype=to_np(y[:1]).dtype)
    y_sub[:used.size] = to_np(y[torch.from_numpy(used.astype(np.int64)).to(hip_device)])
    ref = oracle.unpermute(y_sub, to_np(wts)[sample], remap, dtype)
    assert_unpermute_close(o[sample], ref, dtype)


def test_local_split_schedule_with_scales_and_bad_id(hip_device):
    """A local permute large enough for the split schedule (16384 tokens of
    14 KiB, topk 8): with per-token scales against the oracle in full (the
    buffers past the local rows keep their poison), then with one expert id
    out of range (offsets -1, nothing else written)."""
    w = W.WORKLOADS["dsv3"]
    n, k, e, h = w.num_tokens, w.topk, w.num_experts, w.hidden_size
    assert n * h * 2 >= 128 << 20
    ids_np, _ = W.make_routing(w, seed=5)
    ids = torch.from_numpy(ids_np).to(hip_device)
    g = torch.Generator(device=hip_device).manual_seed(3)
    x = torch.randn((n, h), device=hip_device, generator=g).to(torch.bfloat16)
    scale = torch.rand(n, device=hip_device, generator=g) + 0.25
    emap, nl = W.expert_map_for(e, 8, 3, "shuffled")
    _say("local split schedule dsv3 ep8 rank 3 shuffled, scales")
    outs = gpu_permute_local(x, ids, e, emap, nl, token_scale=scale)
    torch.cuda.synchronize()
    assert_permute_local_equal(outs, oracle_permute_local(x, ids, e, emap, nl, scale))
    bad = ids_np.copy()
    bad[n // 3, 2] = e + 7
    _say("local split schedule, bad id")
    outs = gpu_permute_local(x, torch.from_numpy(bad).to(hip_device), e, emap, nl, token_scale=scale)
    torch.cuda.synchronize()
    assert to_np(outs["expert_first_token_offset"]).tolist() == [-1] * (nl + 1)
    for key in ("permuted_idx", "inv_permuted_idx", "permuted_hidden_states", "permuted_scale"):
        assert bool((outs[key].view(torch.uint8) == POISON).all()), key
