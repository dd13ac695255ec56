"""GPU parity of quantise-while-permuting (moe_permute_quant_fp8) against the oracle.

The oracle quantises every token row (per token or per group: scale = amax /
448 in float, code = E4M3FN of the float quotient, nearest-even, saturating)
and permutes the codes with their scales.  Bar: offsets, indices, codes and
scales bit-exact; with an expert map, nothing past the local rows written.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _parity import POISON, poisoned, to_np
from mixture_experts_token_amd import binding

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[case] " + msg, flush=True)


def gpu_quant(x, ids, e, group=0, emap=None, nl=0):
    dev = ids.device
    n, k = ids.shape
    rows, h = n * k, x.shape[1]
    groups = 1 if group == 0 else h // group
    nb = nl if emap is not None else e
    outs = {
        "permuted_hidden_states": poisoned((rows, h), torch.uint8, dev),
        "permuted_scale": poisoned((rows, groups), torch.float32, dev),
        "expert_first_token_offset": poisoned((nb + 1,), torch.int64, dev),
        "permuted_idx": poisoned((rows,), torch.int32, dev),
        "inv_permuted_idx": poisoned((rows,), torch.int32, dev),
    }
    if emap is None:
        ws = binding.moe_permute_workspace_size(n, k, e)
        emap_t = None
    else:
        ws = binding.moe_permute_local_workspace_size(n, k, e, nl)
        emap_t = torch.from_numpy(np.asarray(emap, np.int32)).to(dev)
    workspace = poisoned((max(ws, 16),), torch.uint8, dev)
    binding.moe_permute_quant_fp8(x, ids, e, outs["permuted_hidden_states"], outs["permuted_scale"],
                                  outs["expert_first_token_offset"], outs["permuted_idx"], outs["inv_permuted_idx"],
                                  workspace, group_size=group, expert_map=emap_t, num_local_experts=nl)
    return outs


def oracle_quant(x, ids, e, group=0, emap=None, nl=None):
    dtype = "bf16" if x.dtype == torch.bfloat16 else "f32"
    return oracle.permute_quant_fp8(to_np(x), dtype, to_np(ids), e, None if group == 0 else group, emap, nl)


def assert_quant_equal(outs, ref):
    np.testing.assert_array_equal(to_np(outs["expert_first_token_offset"]), ref["expert_first_token_offset"])
    np.testing.assert_array_equal(to_np(outs["inv_permuted_idx"]), ref["inv_permuted_idx"])
    m = int(ref["expert_first_token_offset"][-1])
    perm = to_np(outs["permuted_idx"])
    np.testing.assert_array_equal(perm[:m], ref["permuted_idx"])
    codes = to_np(outs["permuted_hidden_states"])
    if not np.array_equal(codes[:m], ref["permuted_hidden_states"]):
        bad = np.argwhere(codes[:m] != ref["permuted_hidden_states"])
        r, c = bad[0]
        raise AssertionError("codes differ at %d places, first row %d col %d: got %#x want %#x" % (
            len(bad), r, c, codes[r, c], ref["permuted_hidden_states"][r, c]))
    sc = to_np(outs["permuted_scale"]).view(np.uint32)
    np.testing.assert_array_equal(sc[:m], ref["permuted_scale"].view(np.uint32))
    assert np.all(codes[m:] == POISON) and np.all(sc[m:] == 0xFFFFFFFF) and np.all(perm[m:].view(np.uint32) == 0xFFFFFFFF)


def _inputs(name, dev, n=None, dtype=torch.bfloat16, hidden=None):
    w = W.WORKLOADS[name]
    if n is not None:
        w = w.with_tokens(n)
    if hidden is not None:
        w = dataclasses.replace(w, hidden_size=hidden)
    ids_np, _ = W.make_routing(w, seed=0)
    g = torch.Generator(device="cpu").manual_seed(w.num_tokens * 7 + w.hidden_size)
    # a spread of row magnitudes so scales differ by orders of magnitude
    mag = torch.exp(torch.randn((w.num_tokens, 1), generator=g) * 3)
    x = (torch.randn((w.num_tokens, w.hidden_size), generator=g) * mag).to(dtype).to(dev)
    return w, torch.from_numpy(ids_np).to(dev), x


CASES = [
    # (workload, tokens, group, input dtype, expert split (ep, rank, layout) or None)
    ("tiny", None, 0, torch.float32, None),
    ("tiny", None, 4, torch.float32, None),
    ("tiny", None, 32, torch.float32, None),
    ("mixtral", None, 0, torch.bfloat16, None),
    ("mixtral", None, 128, torch.bfloat16, None),
    ("mixtral", 1000, 0, torch.float32, None),
    ("qwen3", None, 0, torch.bfloat16, None),
    ("qwen3", None, 64, torch.bfloat16, (4, 1, "round_robin")),
    ("dsv3", 4000, 0, torch.bfloat16, None),
    ("dsv3", 4000, 128, torch.bfloat16, (8, 3, "contiguous")),
    ("decode", 1, 0, torch.bfloat16, None),
    ("decode", 256, 128, torch.bfloat16, None),
    ("decode", 64, 0, torch.bfloat16, (8, 0, "contiguous")),
]


@pytest.mark.parametrize("name,n,group,dtype,ep", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_quant_parity(hip_device, name, n, group, dtype, ep):
    w, ids, x = _inputs(name, hip_device, n, dtype)
    emap, nl = (None, None) if ep is None else W.expert_map_for(w.num_experts, *ep)
    _say("quant %s N=%d H=%d group=%d %s ep=%s" % (name, w.num_tokens, w.hidden_size, group, dtype, ep))
    outs = gpu_quant(x, ids, w.num_experts, group, emap, nl or 0)
    torch.cuda.synchronize()
    assert_quant_equal(outs, oracle_quant(x, ids, w.num_experts, group, emap, nl))


# The quantise-scatter holds adjacent vector pairs per thread with several
# waves per token (one 16-byte code store per pair) for bf16 rows of an even
# vector count, an even number of vectors per thread and scale groups of at
# least two vectors; single vectors otherwise.  (tokens, hidden, group), topk
# 2: pairs with one pair per 16-element group; single vectors for 8-element
# groups; an odd vector count; an even count that leaves pair slots idle, per
# token and per 16 elements; four vectors per thread with a ragged tail; one
# wave per token.
PAIR_CASES = [
    (9000, 4096, 16),
    (9000, 4096, 8),
    (9000, 2056, 0),
    (9000, 2064, 0),
    (9000, 2064, 16),
    (100, 6160, 0),
    (9000, 1024, 0),
]


@pytest.mark.parametrize("n,hidden,group", PAIR_CASES, ids=["-".join(map(str, c)) for c in PAIR_CASES])
def test_quant_pair_layout_edges(hip_device, n, hidden, group):
    w, ids, x = _inputs("mixtral", hip_device, n, torch.bfloat16, hidden)
    _say("quant pairs N=%d H=%d group=%d" % (w.num_tokens, w.hidden_size, group))
    outs = gpu_quant(x, ids, w.num_experts, group)
    torch.cuda.synchronize()
    assert_quant_equal(outs, oracle_quant(x, ids, w.num_experts, group))


# Row counts of the fused index plan (above the one-kernel decode plan, at
# most 16384 rows): the index permute, then the quantise-scatter.  (tokens,
# topk, experts, hidden, dtype, group, expert split (ep, rank, layout) or
# None, ids dtype): the largest fused row count; f32 rows of 128 and 512
# vectors; a ragged row of 257 vectors; groups of 16 elements (two vectors);
# an expert split (tokens with no local row are not read); int64 ids.
FUSED_CASES = [
    (8192, 2, 8, 1024, torch.bfloat16, 0, None, torch.int32),
    (1000, 2, 8, 512, torch.float32, 0, None, torch.int32),
    (1000, 2, 8, 2048, torch.float32, 64, None, torch.int32),
    (700, 4, 16, 2056, torch.bfloat16, 0, None, torch.int32),
    (700, 4, 16, 2064, torch.bfloat16, 16, None, torch.int32),
    (4096, 2, 8, 4096, torch.bfloat16, 0, (2, 0, "contiguous"), torch.int32),
    (3000, 4, 64, 2048, torch.bfloat16, 128, (4, 1, "round_robin"), torch.int64),
]


@pytest.mark.parametrize("n,k,e,h,dtype,group,ep,idt", FUSED_CASES,
                         ids=["-".join(map(str, c[:6])) + ("-ep" if c[6] else "") for c in FUSED_CASES])
def test_quant_fused_plan(hip_device, n, k, e, h, dtype, group, ep, idt):
    w = dataclasses.replace(W.WORKLOADS["mixtral"], num_tokens=n, topk=k, num_experts=e, hidden_size=h)
    ids_np, _ = W.make_routing(w, seed=1)
    ids = torch.from_numpy(ids_np).to(idt).to(hip_device)
    g = torch.Generator(device="cpu").manual_seed(n + h)
    mag = torch.exp(torch.randn((n, 1), generator=g) * 3)
    x = (torch.randn((n, h), generator=g) * mag).to(dtype).to(hip_device)
    emap, nl = (None, None) if ep is None else W.expert_map_for(e, *ep)
    _say("quant fused plan N=%d K=%d E=%d H=%d %s group=%d ep=%s" % (n, k, e, h, dtype, group, ep))
    outs = gpu_quant(x, ids, e, group, emap, nl or 0)
    torch.cuda.synchronize()
    assert_quant_equal(outs, oracle_quant(x, ids, e, group, emap, nl))


def test_quant_fused_plan_non_finite_and_boundaries(hip_device):
    """Non-finite, zero and E4M3 rounding-boundary rows at a fused-plan row
    count (400 rows: above the one-kernel decode plan)."""
    row = _e4m3_boundary_row()
    h = row.size
    rng = np.random.default_rng(5)
    x = rng.standard_normal((200, h)).astype(np.float32) * 10
    x[0] = row
    x[1] = -row
    x[2] = 0.0
    x[3] = -0.0
    x[4, 3] = np.nan
    x[5, 7] = np.inf
    x[6, ::2] = np.nan
    x[7, 9] = -np.inf
    xt = torch.from_numpy(x).to(hip_device)
    ids = torch.from_numpy(np.stack([np.arange(200) % 5, (np.arange(200) + 2) % 5], 1).astype(np.int32)).to(hip_device)
    _say("quant fused plan non-finite H=%d" % h)
    for group in (0, 4):
        outs = gpu_quant(xt, ids, 5, group)
        torch.cuda.synchronize()
        assert_quant_equal(outs, oracle_quant(xt, ids, 5, group))


def _bf16_from_bits(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)


def test_quant_bf16_scale_ranges(hip_device):
    """Bf16 rows whose scales fall on both sides of the bound of the kernels'
    reciprocal-and-FMA quotient (scales in [2^-100, 2^126]; below it the
    division per element stays): tiny rows, rows around the bound, subnormal
    values beside normal ones, signed zeros, values near the bf16 maximum,
    NaN beside finite values, and rows of log-uniform magnitudes; one scale per
    token and 8-element groups (one 16-byte vector each, so scales change
    within a wave).  400 rows
    (above the one-kernel decode plan) and 8 rows (the decode plan)."""
    h = 512
    rng = np.random.default_rng(11)
    rows = []
    rows.append(rng.standard_normal(h) * 1e-30)                    # amax ~1e-30: below the bound
    rows.append(rng.standard_normal(h) * 2.0**-91)                 # amax around 448 * 2^-100
    r = rng.standard_normal(h) * 2.0**-128; r[5] = 2.0**-120; rows.append(r)   # subnormals, tiny scale
    r = rng.standard_normal(h) * 2.0**-128; r[5] = 1.0; rows.append(r)         # subnormals, scale 1/448
    rows.append(rng.uniform(-3.3e38, 3.3e38, h))                   # near the bf16 maximum
    r = np.zeros(h); r[1::2] = -0.0; r[7] = 1.0; rows.append(r)   # signed zeros beside 1
    r = rng.standard_normal(h); r[3] = np.nan; r[10] = 2.5; rows.append(r)    # NaN beside finite values
    while len(rows) < 200:                                          # log-uniform magnitudes per element
        rows.append(rng.choice([-1.0, 1.0], h) * np.exp2(rng.uniform(-140, 120, h)))
    xb = torch.from_numpy(np.stack(rows).astype(np.float32)).to(torch.bfloat16)
    signed_zeros = _bf16_from_bits(np.where(np.arange(h) % 2 == 1, 0x8000, 0)).to(torch.bfloat16)
    signed_zeros[7] = 1.0
    xb[5] = signed_zeros
    x = xb.to(hip_device)
    for n in (200, 8):
        ids = torch.from_numpy(np.stack([np.arange(n) % 5, (np.arange(n) + 2) % 5], 1).astype(np.int32)).to(hip_device)
        for group in (0, 8):
            _say("quant bf16 scale ranges N=%d group=%d" % (n, group))
            outs = gpu_quant(x[:n].contiguous(), ids, 5, group)
            torch.cuda.synchronize()
            assert_quant_equal(outs, oracle_quant(x[:n].contiguous(), ids, 5, group))


@pytest.mark.parametrize("group", [0, 128])
def test_quant_dsv3_full_size(hip_device, group):
    """DSv3 shape at full size: offsets, indices, and the codes and scales of
    every one of the 131072 permuted rows against the oracle."""
    w, ids, x = _inputs("dsv3", hip_device)
    _say("quant dsv3 full N=%d group=%d" % (w.num_tokens, group))
    outs = gpu_quant(x, ids, w.num_experts, group)
    torch.cuda.synchronize()
    assert_quant_equal(outs, oracle_quant(x, ids, w.num_experts, group))


def _e4m3_boundary_row():
    """448 (so the scale is exactly 1) followed by every finite E4M3FN value,
    every midpoint between neighbours and the floats next to each midpoint."""
    vals = sorted({oracle.e4m3_to_double(c) for c in range(0x7F) if not np.isnan(oracle.e4m3_to_double(c))})
    probes = [448.0]
    for lo, hi in zip(vals, vals[1:]):
        mid = np.float32((lo + hi) / 2)
        probes += [lo, mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    probes += [-p for p in probes[1:]]
    probes += [0.0, -0.0, 2.0**-12, -(2.0**-12), 447.99, 448.0]
    row = np.array(probes, np.float32)
    pad = (-row.size) % 4
    return np.concatenate([row, np.zeros(pad, np.float32)])


def test_quant_e4m3_rounding_boundaries(hip_device):
    row = _e4m3_boundary_row()
    h = row.size
    x = torch.from_numpy(np.stack([row, -row, row * 0.5])).to(hip_device)  # 0.5 * row: scale 0.5, same quotients
    ids = torch.tensor([[0], [1], [0]], dtype=torch.int32, device=hip_device)
    _say("quant e4m3 boundaries H=%d" % h)
    outs = gpu_quant(x, ids, 2)
    torch.cuda.synchronize()
    assert_quant_equal(outs, oracle_quant(x, ids, 2))


def test_quant_non_finite_and_zero_rows(hip_device):
    h = 64
    x = np.random.default_rng(4).standard_normal((6, h)).astype(np.float32)
    x[0] = 0.0
    x[1, 3] = np.nan
    x[2, 7] = np.inf
    x[3, 9] = -np.inf
    x[3, 10] = np.inf
    x[4] = -0.0
    x[5, ::2] = np.nan
    xt = torch.from_numpy(x).to(hip_device)
    ids = torch.arange(6, dtype=torch.int32, device=hip_device).reshape(6, 1) % 3
    _say("quant non-finite rows")
    for group in (0, 16):
        outs = gpu_quant(xt, ids, 3, group)
        torch.cuda.synchronize()
        assert_quant_equal(outs, oracle_quant(xt, ids, 3, group))


def test_quant_int64_ids_and_bad_id(hip_device):
    w, ids, x = _inputs("qwen3", hip_device, 2000)
    ids64 = ids.to(torch.int64)
    _say("quant int64 ids")
    outs = gpu_quant(x, ids64, w.num_experts, 128)
    torch.cuda.synchronize()
    assert_quant_equal(outs, oracle_quant(x, ids64, w.num_experts, 128))
    bad = ids64.clone()
    bad[77, 3] = 2**32 + 5
    outs = gpu_quant(x, bad, w.num_experts, 0)
    torch.cuda.synchronize()
    assert to_np(outs["expert_first_token_offset"]).tolist() == [-1] * (w.num_experts + 1)
    assert np.all(to_np(outs["permuted_hidden_states"]) == POISON)
    assert np.all(to_np(outs["permuted_scale"]).view(np.uint32) == 0xFFFFFFFF)


def test_quant_zero_tokens(hip_device):
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=hip_device)
    ids = torch.zeros((0, 2), dtype=torch.int32, device=hip_device)
    _say("quant zero tokens")
    outs = gpu_quant(x, ids, 4)
    torch.cuda.synchronize()
    assert to_np(outs["expert_first_token_offset"]).tolist() == [0] * 5


# Decode sizes (N*topk <= 128, no expert map) take the one-kernel quantising
# permute: one or two ids per lane, rows read whole for a per-token scale
# (4 or 16 vectors per lane) or groups within a 64-vector chunk.
WAVE_CASES = [
    # (N, topk, E, H, dtype, group, ids dtype)
    (16, 8, 256, 7168, torch.bfloat16, 0, torch.int32),     # 128 rows: two ids per lane
    (16, 8, 256, 7168, torch.bfloat16, 128, torch.int32),
    (9, 8, 64, 2048, torch.float32, 0, torch.int32),         # f32 rows of 512 vectors
    (5, 4, 16, 256, torch.bfloat16, 32, torch.int32),        # a single, partly filled chunk
    (3, 8, 256, 4096, torch.bfloat16, 0, torch.int64),
    (2, 8, 256, 8192, torch.bfloat16, 0, torch.int32),       # the largest row: 1024 vectors
    (1, 8, 256, 7168, torch.bfloat16, 64, torch.int64),
]


@pytest.mark.parametrize("n,k,e,h,dtype,group,idt", WAVE_CASES, ids=["-".join(map(str, c[:4])) + "-%s-g%d-%s" % (
    str(c[4]).split(".")[-1], c[5], str(c[6]).split(".")[-1]) for c in WAVE_CASES])
def test_quant_decode_sizes_one_kernel(hip_device, n, k, e, h, dtype, group, idt):
    rng = np.random.default_rng(n * 31 + h)
    ids = torch.from_numpy(np.argsort(rng.random((n, e)), axis=1)[:, :k]).to(idt).to(hip_device)
    g = torch.Generator(device="cpu").manual_seed(n + h)
    mag = torch.exp(torch.randn((n, 1), generator=g) * 3)
    x = (torch.randn((n, h), generator=g) * mag).to(dtype).to(hip_device)
    _say("quant decode size N=%d topk=%d H=%d group=%d" % (n, k, h, group))
    outs = gpu_quant(x, ids, e, group)
    torch.cuda.synchronize()
    assert_quant_equal(outs, oracle_quant(x, ids, e, group))
    bad = ids.clone()
    bad[n - 1, k - 1] = e if idt == torch.int32 else 2**32 + 1
    outs = gpu_quant(x, bad, e, group)
    torch.cuda.synchronize()
    assert to_np(outs["expert_first_token_offset"]).tolist() == [-1] * (e + 1)
    assert np.all(to_np(outs["permuted_hidden_states"]) == POISON)
    assert np.all(to_np(outs["permuted_scale"]).view(np.uint32) == 0xFFFFFFFF)
    assert np.all(to_np(outs["permuted_idx"]).view(np.uint32) == 0xFFFFFFFF)
