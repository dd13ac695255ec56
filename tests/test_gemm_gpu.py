"""GPU parity of the grouped GEMM over permuted rows (moe_grouped_gemm_bf16).

Reference: the oracle's per-expert double-precision sum of products rounded
once to bf16.  The kernel accumulates in fp32 on the matrix cores, in an order
of its own, then rounds once, so the bar is
    |gpu - ref| <= 2^-7 |ref| + k * 2^-22 * sum_i |x_i w_i|
(two bf16 roundings of half an ulp each, plus four times the worst-case fp32
accumulation error k * 2^-24 of a k-term sum).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _parity import POISON, gpu_permute, gpu_unpermute, oracle_permute, poisoned, to_np
from mixture_experts_token_amd import binding

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[case] " + msg, flush=True)


def _bf16(t):
    return t.to(torch.bfloat16)


def _f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_gemm_close(got_bits, ref_bits, x_bits, w_bits, off):
    got, ref = _f64(got_bits), _f64(ref_bits)
    xa, wa = np.abs(_f64(x_bits)), np.abs(_f64(w_bits))
    k = x_bits.shape[1]
    for e in range(w_bits.shape[0]):
        seg = slice(int(off[e]), int(off[e + 1]))
        if off[e + 1] == off[e]:
            continue
        mag = xa[seg] @ wa[e].T
        tol = 2.0**-7 * np.abs(ref[seg]) + k * 2.0**-22 * mag + 1e-30
        err = np.abs(got[seg] - ref[seg])
        if not np.all(err <= tol):
            i = np.unravel_index(np.argmax(err - tol), err.shape)
            raise AssertionError("expert %d row %d col %d: got %g want %g (tol %g)" % (
                e, seg.start + i[0], i[1], got[seg][i], ref[seg][i], tol[i]))


def _offsets(rng, e, rows, mode):
    if mode == "even":
        counts = np.full(e, rows // e)
        counts[: rows % e] += 1
    elif mode == "skewed":
        p = 1.0 / np.arange(1, e + 1) ** 1.2
        counts = rng.multinomial(rows, p / p.sum())
        counts[1] += counts[e // 2]  # one empty expert in the middle
        counts[e // 2] = 0
    else:  # one expert only
        counts = np.zeros(e, int)
        counts[e - 1] = rows
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


CASES = [
    # (experts, rows, n, k, offsets mode)
    (1, 1, 128, 64, "even"),
    (4, 130, 128, 64, "even"),          # ragged last row tile
    (8, 1000, 256, 512, "skewed"),      # empty expert, several row / column tiles and k steps
    (16, 700, 384, 192, "skewed"),
    (5, 300, 128, 1024, "one"),
    (3, 2, 640, 128, "even"),           # fewer rows than experts
    # n a multiple of 256: 128 x 256 tiles with three LDS stages
    (2, 300, 256, 64, "even"),          # a single k-step
    (4, 257, 512, 128, "skewed"),       # two k-steps
    (4, 129, 256, 320, "even"),         # a round of three k-steps, then two
    (6, 700, 768, 192, "one"),          # exactly one round
]


@pytest.mark.parametrize("e,rows,n,k,mode", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_grouped_gemm_parity(hip_device, e, rows, n, k, mode):
    rng = np.random.default_rng(rows + n + k)
    off = _offsets(rng, e, rows, mode)
    g = torch.Generator().manual_seed(rows * 3 + k)
    x = _bf16(torch.randn((rows, k), generator=g))
    w = _bf16(torch.randn((e, n, k), generator=g) * k**-0.5)
    spare = 37  # rows past off[E] must stay untouched
    xs = torch.cat([x, _bf16(torch.randn((spare, k), generator=g))]).to(hip_device)
    y = poisoned((rows + spare, n), torch.bfloat16, hip_device)
    _say("grouped gemm E=%d rows=%d n=%d k=%d %s" % (e, rows, n, k, mode))
    binding.moe_grouped_gemm_bf16(xs, w.to(hip_device), torch.from_numpy(off).to(hip_device), y)
    torch.cuda.synchronize()
    got = to_np(y)
    ref = oracle.grouped_gemm_bf16(to_np(x), to_np(w), off)
    assert_gemm_close(got[:rows], ref, to_np(x), to_np(w), off)
    assert np.all(got[rows:].view(np.uint8) == POISON)


def test_grouped_gemm_rejected_offsets_write_nothing(hip_device):
    x = _bf16(torch.randn((64, 128))).to(hip_device)
    w = _bf16(torch.randn((2, 128, 128))).to(hip_device)
    for bad in ([-1, -1, -1], [0, 40, 30], [0, 10, 65], [3, 10, 20]):
        y = poisoned((64, 128), torch.bfloat16, hip_device)
        _say("grouped gemm bad offsets %s" % bad)
        binding.moe_grouped_gemm_bf16(x, w, torch.tensor(bad, dtype=torch.int64, device=hip_device), y)
        torch.cuda.synchronize()
        assert np.all(to_np(y).view(np.uint8) == POISON)


def test_moe_layer_permute_gemm_unpermute(hip_device):
    """The three steps chained on the device (permute -> grouped GEMM -> unpermute)
    against the oracle chain: permuted rows and offsets bit-exact, expert output
    within the GEMM bar, final output within the unpermute bar."""
    w8 = W.WORKLOADS["mixtral"].with_tokens(512)
    inp = W.make_all(w8, seed=3, device="cpu")
    e, k, n = w8.num_experts, w8.hidden_size, 256
    g = torch.Generator().manual_seed(5)
    wts = _bf16(torch.randn((e, n, k), generator=g) * k**-0.5)
    ids, x = inp["topk_ids"].to(hip_device), inp["hidden_states"].to(hip_device)
    _say("moe layer N=%d k=%d n=%d" % (w8.num_tokens, k, n))
    outs = gpu_permute(x, ids, e)
    y = poisoned((w8.num_rows, n), torch.bfloat16, hip_device)
    binding.moe_grouped_gemm_bf16(outs["permuted_hidden_states"], wts.to(hip_device),
                                  outs["expert_first_token_offset"], y)
    out = gpu_unpermute(y, inp["topk_weights"].to(hip_device), outs["inv_permuted_idx"])
    torch.cuda.synchronize()
    ref_p = oracle_permute(x, ids, e)
    np.testing.assert_array_equal(to_np(outs["permuted_hidden_states"]), ref_p["permuted_hidden_states"])
    ref_y = oracle.grouped_gemm_bf16(ref_p["permuted_hidden_states"], to_np(wts), ref_p["expert_first_token_offset"])
    assert_gemm_close(to_np(y), ref_y, ref_p["permuted_hidden_states"], to_np(wts), ref_p["expert_first_token_offset"])
    # unpermute of the GPU's own expert output against the oracle's unpermute of it
    ref_out = oracle.unpermute(to_np(y), to_np(inp["topk_weights"]), ref_p["inv_permuted_idx"], "bf16")
    got = _f64(to_np(out))
    want = _f64(ref_out)
    assert np.all(np.abs(got - want) <= 2.0**-7 * np.maximum(1.0, np.abs(want)))


@pytest.mark.parametrize("name,n", [("qwen3", 1536), ("dsv3", 4096)])
def test_grouped_gemm_full_size_sampled_rows(hip_device, name, n):
    """Model-shaped routing at full size: every row computed on the GPU, a
    sample of rows (one expert each) recomputed by the oracle."""
    w8 = W.WORKLOADS[name]
    ids_np, _ = W.make_routing(w8, seed=0)
    e, k = w8.num_experts, w8.hidden_size
    counts = np.bincount(ids_np.reshape(-1), minlength=e)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rows = int(off[-1])
    gen = torch.Generator(device=hip_device).manual_seed(9)
    x = torch.randn((rows, k), device=hip_device, generator=gen).to(torch.bfloat16)
    wts = (torch.randn((e, n, k), device=hip_device, generator=gen) * k**-0.5).to(torch.bfloat16)
    y = poisoned((rows, n), torch.bfloat16, hip_device)
    _say("grouped gemm full %s rows=%d n=%d k=%d" % (name, rows, n, k))
    binding.moe_grouped_gemm_bf16(x, wts, torch.from_numpy(off).to(hip_device), y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    sample = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, 120, replace=False),
                                       off[1:-1][counts[1:] > 0][:20]]))
    expert_of = np.searchsorted(off, sample, side="right") - 1
    for j, ex in zip(sample, expert_of):
        xr = to_np(x[int(j):int(j) + 1])
        wr = to_np(wts[int(ex):int(ex) + 1])
        ref = oracle.grouped_gemm_bf16(xr, wr, np.array([0, 1], np.int64))
        assert_gemm_close(to_np(y[int(j):int(j) + 1]), ref, xr, wr, np.array([0, 1], np.int64))


# ----------------------------------------------------------------------------
# Decode-size kernels, chosen from the host's sizes (M rows, E experts):
#  * row-streaming: M <= E and k a multiple of 512 up to 8192 (two x rows per
#    item), or E < M <= 2E and k a multiple of 512 up to 4096 (four x rows per
#    item); one wave per 8 weight rows of an expert, each weight row read
#    whole into bf16 dot products, a cross-lane sum per row;
#  * LDS-staged: M <= 4E, or M <= 16E with fewer tiled-kernel tiles,
#    min(M, E + M // 128) x ceil(n / 256), than CUs; one wave per 32 output
#    columns of an expert and 16 of its rows, weights staged through LDS in
#    512-byte runs of the 32 rows;
#  * otherwise the tiled kernel.
# ----------------------------------------------------------------------------
def _kernel_for(max_rows, e, n, k):
    if max_rows <= e and k % 512 == 0 and k <= 8192:
        return "rowstream"
    if max_rows <= 2 * e and k % 512 == 0 and k <= 4096:
        return "rowstream4"
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = min(max_rows, e + max_rows // 128) * ((n + 255) // 256)
    if max_rows <= 4 * e or (max_rows <= 16 * e and tiles < cus):
        return "skinny"
    return "tiled"


SKINNY_CASES = [
    # (experts, per-expert row counts or a mode with a total, n, k, spare rows)
    (8, [0, 1, 33, 40, 0, 20, 2, 0], 256, 832, 16),   # 13 k chunks: 3 whole stages and one chunk; 2 row groups
    (8, [8] * 8, 128, 512, 0),                         # exactly two stages
    (16, ("skewed", 200), 384, 256, 16),               # one stage
    (4, [0, 0, 0, 1], 128, 64, 3),                     # one row, one chunk (a partial stage)
    (200, ("even", 1600), 128, 320, 0),                # 200 experts, 5 chunks: a whole stage and one chunk
    (8, [3] * 8, 128, 640, 0),                         # 10 chunks: an odd stage count, the last stage partial
    (4, [1, 0, 2, 1], 128, 8704, 0),                   # k past the row-streaming kernel's 8192: 34 stages
    (8, [4] * 8, 8192, 512, 0),                        # M = 4E with as many tiles as CUs
    (4, [5, 1, 0, 2], 128, 4608, 0),                   # M = 2E, k past the four-row kernel's 4096
]

ROWSTREAM_CASES = [
    # (experts, per-expert row counts or a mode with a total, n, k, spare rows)
    (8, [0, 2, 1, 0, 0, 3, 0, 1], 128, 512, 1),        # a 3-row expert: a 2-row and a 1-row item; 16 rows in flight
    (16, [1] * 10 + [0] * 6, 256, 1024, 6),            # one row each; 2 loads per row
    (64, ("even", 60), 384, 4608, 4),                  # 9 loads per row: one row in flight
    (4, [1, 0, 2, 1], 128, 8192, 0),                   # the largest k: 16 loads per row
    (3, [0, 0, 3], 4096, 2560, 0),                     # one expert with all rows, 128 column blocks
]

ROWSTREAM4_CASES = [
    # four x rows per item (E < M <= 2E)
    (8, [3, 0, 4, 1, 0, 2, 3, 1], 256, 1024, 2),       # 14 rows; a 4-row and a 3-row expert
    (4, [5, 1, 0, 2], 128, 512, 0),                    # a 5-row expert: a 4-row and a 1-row item
    (16, ("even", 30), 384, 4096, 0),                  # the largest k with four x rows
]


def _skinny_offsets(rng, e, spec):
    if isinstance(spec, tuple):
        return _offsets(rng, e, spec[1], spec[0])
    return np.concatenate([[0], np.cumsum(spec)]).astype(np.int64)


def _decode_kernel_parity(hip_device, e, spec, n, k, spare, kernel):
    rng = np.random.default_rng(n + k + e)
    off = _skinny_offsets(rng, e, spec)
    rows = int(off[-1])
    assert _kernel_for(rows + spare, e, n, k) == kernel
    g = torch.Generator().manual_seed(rows * 7 + k)
    x = _bf16(torch.randn((rows, k), generator=g))
    w = _bf16(torch.randn((e, n, k), generator=g) * k**-0.5)
    xs = torch.cat([x, _bf16(torch.randn((spare, k), generator=g))]).to(hip_device)
    y = poisoned((rows + spare, n), torch.bfloat16, hip_device)
    _say("%s grouped gemm E=%d rows=%d n=%d k=%d" % (kernel, e, rows, n, k))
    binding.moe_grouped_gemm_bf16(xs, w.to(hip_device), torch.from_numpy(off).to(hip_device), y)
    torch.cuda.synchronize()
    got = to_np(y)
    ref = oracle.grouped_gemm_bf16(to_np(x), to_np(w), off)
    assert_gemm_close(got[:rows], ref, to_np(x), to_np(w), off)
    assert np.all(got[rows:].view(np.uint8) == POISON)


@pytest.mark.parametrize("e,spec,n,k,spare", SKINNY_CASES, ids=["skinny-%d-%d-%d" % (c[0], c[2], c[3]) for c in SKINNY_CASES])
def test_grouped_gemm_skinny_parity(hip_device, e, spec, n, k, spare):
    _decode_kernel_parity(hip_device, e, spec, n, k, spare, "skinny")


@pytest.mark.parametrize("e,spec,n,k,spare", ROWSTREAM_CASES,
                         ids=["rowstream-%d-%d-%d" % (c[0], c[2], c[3]) for c in ROWSTREAM_CASES])
def test_grouped_gemm_rowstream_parity(hip_device, e, spec, n, k, spare):
    _decode_kernel_parity(hip_device, e, spec, n, k, spare, "rowstream")


@pytest.mark.parametrize("e,spec,n,k,spare", ROWSTREAM4_CASES,
                         ids=["rowstream4-%d-%d-%d" % (c[0], c[2], c[3]) for c in ROWSTREAM4_CASES])
def test_grouped_gemm_rowstream4_parity(hip_device, e, spec, n, k, spare):
    _decode_kernel_parity(hip_device, e, spec, n, k, spare, "rowstream4")


@pytest.mark.parametrize("kernel,n,k", [("skinny", 128, 128), ("rowstream", 128, 512)])
def test_grouped_gemm_decode_kernels_rejected_offsets_write_nothing(hip_device, kernel, n, k):
    x = _bf16(torch.randn((8, k))).to(hip_device)
    w = _bf16(torch.randn((8, n, k))).to(hip_device)
    assert _kernel_for(8, 8, n, k) == kernel
    for bad in ([-1] * 9, [0, 1, 0, 2, 3, 4, 5, 6, 7], [0, 1, 2, 3, 4, 5, 6, 7, 9], [1] * 9):
        y = poisoned((8, n), torch.bfloat16, hip_device)
        _say("%s grouped gemm bad offsets %s" % (kernel, bad))
        binding.moe_grouped_gemm_bf16(x, w, torch.tensor(bad, dtype=torch.int64, device=hip_device), y)
        torch.cuda.synchronize()
        assert np.all(to_np(y).view(np.uint8) == POISON)


def test_grouped_gemm_skinny_rejected_offsets_write_nothing(hip_device):
    x = _bf16(torch.randn((64, 128))).to(hip_device)
    w = _bf16(torch.randn((8, 128, 128))).to(hip_device)
    for bad in ([-1] * 9, [0, 4, 3, 5, 6, 7, 8, 9, 10], [0, 1, 2, 3, 4, 5, 6, 7, 65], [2] * 9):
        y = poisoned((64, 128), torch.bfloat16, hip_device)
        _say("skinny grouped gemm bad offsets %s" % bad)
        binding.moe_grouped_gemm_bf16(x, w, torch.tensor(bad, dtype=torch.int64, device=hip_device), y)
        torch.cuda.synchronize()
        assert np.all(to_np(y).view(np.uint8) == POISON)


@pytest.mark.parametrize("tokens", [1, 4, 256])
def test_grouped_gemm_decode_shape_sampled(hip_device, tokens):
    """The decode shape (topk 8, 256 experts, n=4096, k=7168) at N=1 and 4
    (row-streaming kernel) and 256 tokens (tiled): every expert's rows on the
    device; the oracle checks a sample of experts (the ones with the most and
    the fewest rows, and up to four others)."""
    w8 = W.WORKLOADS["decode"].with_tokens(tokens)
    ids_np, _ = W.make_routing(w8, 0)
    e, n, k = w8.num_experts, 4096, w8.hidden_size
    counts = np.bincount(ids_np.reshape(-1), minlength=e)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rows = int(off[-1])
    g = torch.Generator(device=hip_device).manual_seed(9)
    x = _bf16(torch.randn((rows, k), device=hip_device, generator=g))
    w = _bf16(torch.randn((e, n, k), device=hip_device, generator=g) * k**-0.5)
    y = poisoned((rows, n), torch.bfloat16, hip_device)
    kernel = _kernel_for(rows, e, n, k)
    _say("grouped gemm decode shape N=%d rows=%d kernel=%s" % (tokens, rows, kernel))
    assert kernel == ("tiled" if tokens == 256 else "rowstream")
    binding.moe_grouped_gemm_bf16(x, w, torch.from_numpy(off).to(hip_device), y)
    torch.cuda.synchronize()
    used = np.nonzero(counts)[0]
    pick = sorted(set([int(used[np.argmax(counts[used])]), int(used[np.argmin(counts[used])])] +
                      [int(v) for v in np.random.default_rng(1).choice(used, min(4, used.size), replace=False)]))
    sub_rows = np.concatenate([np.arange(off[p], off[p + 1]) for p in pick])
    sub_off = np.concatenate([[0], np.cumsum(counts[pick])]).astype(np.int64)
    xs = to_np(x[torch.from_numpy(sub_rows).to(hip_device)])
    ws = to_np(w[torch.tensor(pick, device=hip_device)])
    ref = oracle.grouped_gemm_bf16(xs, ws, sub_off)
    got = to_np(y)[sub_rows]
    assert_gemm_close(got, ref, xs, ws, sub_off)
