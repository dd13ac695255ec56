"""Pins for the CPU oracle: checks against things other than the oracle itself.

What pins what:
* a pure-Python brute force written from the definition on exhaustive tiny
  grids (ids, counts, offsets, order, gathered rows);
* numpy library routines: ``bincount``/``cumsum`` for the offsets,
  ``argsort(kind="stable")`` for the order, fancy indexing for the gather,
  ``einsum`` in float64 for the unpermute sum;
* invariants that hold at any size (offsets, bijection, inverse, sortedness);
* a hand-worked example whose every number is derived in the comments;
* exact special cases of unpermute (topk=1 with weight 1; the round trip with
  identity experts and equal power-of-two weights);
* bfloat16 decoding against torch on all 65536 patterns, and bfloat16
  rounding against an exact brute-force nearest-value search.

The definition being pinned: vLLM PR #14568 "permute/unpermute kernel for moe
optimization" (PR description) and the buffer contract in the prhub summary
of vLLM PR #43014, section "key code snippets" (MoEPermuteScratch).
"""

import bisect
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402


# --------------------------------------------------------------------------
# Brute force, written independently from the definition.
# --------------------------------------------------------------------------
def brute_permute(ids2d, num_experts, hidden_rows):
    flat = [int(v) for row in ids2d for v in row]  # expanded row r = t*topk + k
    topk = len(ids2d[0]) if len(ids2d) else 1
    rows = len(flat)
    perm = [r for e in range(num_experts) for r in range(rows) if flat[r] == e]
    inv = [0] * rows
    for j, r in enumerate(perm):
        inv[r] = j
    off = [0]
    for e in range(num_experts):
        off.append(off[-1] + sum(1 for v in flat if v == e))
    gathered = [hidden_rows[r // topk] for r in perm]
    return off, perm, inv, gathered


def _grid_ids(rng, n, k, e, mode):
    if mode == "random":
        return rng.integers(0, e, size=(n, k))
    if mode == "one_expert":
        return np.full((n, k), e - 1)
    if mode == "distinct" and k <= e:
        return np.stack([rng.permutation(e)[:k] for _ in range(n)]) if n else np.zeros((0, k), int)
    if mode == "skip_first_last" and e >= 3:
        return rng.integers(1, e - 1, size=(n, k))
    return rng.integers(0, e, size=(n, k))


@pytest.mark.parametrize("n,k,e", list(itertools.product([0, 1, 2, 3, 5, 16], [1, 2, 3, 8], [1, 2, 3, 8])))
def test_oracle_permute_matches_brute_force(n, k, e):
    rng = np.random.default_rng(1000 + 97 * n + 13 * k + e)
    for mode in ("random", "one_expert", "distinct", "skip_first_last"):
        ids = _grid_ids(rng, n, k, e, mode).astype(np.int32).reshape(n, k)
        hidden = rng.standard_normal((n, 3)).astype(np.float32)
        got = oracle.permute(hidden, ids, e)
        off, perm, inv, gathered = brute_permute(ids.tolist(), e, [row.tobytes() for row in hidden])
        assert got["expert_first_token_offset"].tolist() == off
        assert got["permuted_idx"].tolist() == perm
        assert got["inv_permuted_idx"].tolist() == inv
        assert [row.tobytes() for row in got["permuted_hidden_states"]] == gathered


def test_hand_worked_example():
    # N=3 tokens, topk=2, E=3 experts; token 2 picks expert 2 twice (allowed).
    ids = np.array([[2, 0], [0, 1], [2, 2]], dtype=np.int32)
    # expanded rows r = t*2+k carry experts [2, 0, 0, 1, 2, 2]
    # counts: e0 <- rows 1,2 (2); e1 <- row 3 (1); e2 <- rows 0,4,5 (3)
    # offsets: [0, 2, 3, 6]
    # stable order: slots 0,1 <- rows 1,2; slot 2 <- row 3; slots 3,4,5 <- rows 0,4,5
    # inverse: r0->3, r1->0, r2->1, r3->2, r4->4, r5->5
    # source tokens of the slots: perm // 2 = [0, 1, 1, 0, 2, 2]
    x = np.array([[10, 11], [20, 21], [30, 31]], dtype=np.float32)
    got = oracle.permute(x, ids, 3)
    assert got["expert_first_token_offset"].tolist() == [0, 2, 3, 6]
    assert got["permuted_idx"].tolist() == [1, 2, 3, 0, 4, 5]
    assert got["inv_permuted_idx"].tolist() == [3, 0, 1, 2, 4, 5]
    assert got["permuted_hidden_states"].tolist() == [[10, 11], [20, 21], [20, 21], [10, 11], [30, 31], [30, 31]]
    # Unpermute with Y[j] = (j+1) * [1, -1] and weights [[.5,.25],[1,2],[.75,-1]]:
    # out[0] = .5*Y[inv[0]=3] + .25*Y[inv[1]=0] = .5*4 + .25*1 = 2.25
    # out[1] = 1*Y[inv[2]=1] + 2*Y[inv[3]=2] = 1*2 + 2*3 = 8
    # out[2] = .75*Y[inv[4]=4] + (-1)*Y[inv[5]=5] = .75*5 - 6 = -2.25
    y = np.array([[j + 1, -(j + 1)] for j in range(6)], dtype=np.float32)
    w = np.array([[0.5, 0.25], [1.0, 2.0], [0.75, -1.0]], dtype=np.float32)
    out = oracle.unpermute(y, w, got["inv_permuted_idx"], "f32")
    assert out.tolist() == [[2.25, -2.25], [8.0, -8.0], [-2.25, 2.25]]
    yb = (y.view(np.uint32) >> 16).astype(np.uint16)  # these values are exact in bf16
    outb = oracle.unpermute(yb, w, got["inv_permuted_idx"], "bf16")
    assert ((outb.astype(np.uint32) << 16).view(np.float32)).tolist() == [[2.25, -2.25], [8.0, -8.0], [-2.25, 2.25]]


def test_bad_ids_rejected():
    with pytest.raises(oracle.OracleError):
        oracle.permute(np.zeros((2, 4), np.float32), np.array([[0, 3]], np.int32).repeat(2, 0), 3)
    with pytest.raises(oracle.OracleError):
        oracle.permute(np.zeros((1, 4), np.float32), np.array([[-1, 0]], np.int32), 3)
    with pytest.raises(oracle.OracleError):
        oracle.unpermute(np.zeros((2, 4), np.float32), np.ones((1, 2), np.float32), np.array([0, 2], np.int32), "f32")


# --------------------------------------------------------------------------
# Invariants at any size, and library cross-checks on every workload.
# --------------------------------------------------------------------------
def check_permute_invariants(ids2d, num_experts, res):
    flat = np.asarray(ids2d, dtype=np.int64).reshape(-1)
    rows = flat.shape[0]
    off = res["expert_first_token_offset"]
    perm = res["permuted_idx"].astype(np.int64)
    inv = res["inv_permuted_idx"].astype(np.int64)
    assert off.dtype == np.int64 and off.shape == (num_experts + 1,)
    assert off[0] == 0 and off[-1] == rows and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.sort(perm), np.arange(rows))  # bijection on [0, R)
    assert np.array_equal(inv[perm], np.arange(rows))  # inv o perm = identity
    assert np.array_equal(perm[inv], np.arange(rows))  # perm o inv = identity
    keys = flat[perm]
    assert np.all(np.diff(keys) >= 0)
    for e in range(num_experts):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(keys[off[e]:off[e + 1]] == e)
        assert np.all(np.diff(seg) > 0)  # ties keep ascending expanded row


@settings(max_examples=150, deadline=None)
@given(
    n=st.integers(0, 40),
    k=st.integers(1, 6),
    e=st.integers(1, 12),
    seed=st.integers(0, 2**31 - 1),
)
def test_oracle_invariants_property(n, k, e, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, e, size=(n, k)).astype(np.int32)
    res = oracle.permute(rng.standard_normal((n, 2)).astype(np.float32), ids, e)
    check_permute_invariants(ids, e, res)
    np.testing.assert_array_equal(res["expert_first_token_offset"],
                                  np.concatenate([[0], np.cumsum(np.bincount(ids.ravel(), minlength=e))]))


@pytest.mark.parametrize("name", ["tiny", "mixtral", "qwen3", "dsv3", "decode"])
def test_oracle_order_matches_numpy_at_workload_sizes(name):
    w = W.WORKLOADS[name]
    ids, _ = W.make_routing(w)
    counts = oracle.expert_counts(ids, w.num_experts)
    np.testing.assert_array_equal(counts, np.bincount(ids.ravel(), minlength=w.num_experts))
    off = oracle.expert_first_token_offset(counts)
    np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(counts)]))
    perm, inv = oracle.stable_expert_order(ids, w.num_experts, off)
    np.testing.assert_array_equal(perm, np.argsort(ids.ravel(), kind="stable"))
    check_permute_invariants(ids, w.num_experts, {"expert_first_token_offset": off,
                                                  "permuted_idx": perm, "inv_permuted_idx": inv})


@pytest.mark.parametrize("dtype", [np.float32, np.uint16, np.uint8])
def test_oracle_gather_matches_fancy_indexing(dtype):
    rng = np.random.default_rng(7)
    n, k, e, h = 37, 3, 5, 48
    ids = rng.integers(0, e, size=(n, k)).astype(np.int32)
    x = rng.integers(0, 255, size=(n, h)).astype(dtype)
    scale = rng.random(n).astype(np.float32)
    res = oracle.permute(x, ids, e, token_scale=scale)
    src = res["permuted_idx"] // k
    np.testing.assert_array_equal(res["permuted_hidden_states"], x[src])
    np.testing.assert_array_equal(res["permuted_scale"], scale[src])


# --------------------------------------------------------------------------
# bfloat16 decoding and rounding.
# --------------------------------------------------------------------------
def test_bf16_decode_all_patterns_against_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _finite_bf16_table():
    vals = []
    for b in range(0x0000, 0x7F80):  # +0 .. largest finite
        vals.append(oracle.bf16_to_double(b))
    return vals  # ascending, patterns 0..0x7F7F


_TABLE = None


def brute_nearest_bf16(x: float) -> int:
    """Nearest bf16 by exhaustive search with exact rational arithmetic (ties -> even pattern)."""
    global _TABLE
    if _TABLE is None:
        _TABLE = _finite_bf16_table()
    sign = 0x8000 if np.signbit(x) else 0
    a = abs(x)
    fa = Fraction(a)
    max_finite = Fraction(_TABLE[-1])
    overflow_at = max_finite + (Fraction(2) ** 128 - max_finite) / 2
    if fa >= overflow_at:
        return sign | 0x7F80
    i = bisect.bisect_left(_TABLE, a)
    if i < len(_TABLE) and _TABLE[i] == a:
        return sign | i
    lo, hi = i - 1, i
    dlo = fa - Fraction(_TABLE[lo])
    dhi = Fraction(_TABLE[hi]) - fa
    if dlo < dhi:
        return sign | lo
    if dhi < dlo:
        return sign | hi
    return sign | (lo if lo % 2 == 0 else hi)


def test_bf16_rounding_against_exhaustive_nearest():
    rng = np.random.default_rng(3)
    tests = [0.0, -0.0, 1.0, -1.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, 1.0 + 2.0**-8 + 2.0**-40,
             1.0 + 2.0**-8 - 2.0**-40, 2.0**-126, 2.0**-133, 2.0**-134, 3 * 2.0**-134, 2.0**-135,
             2.0**-126 - 2.0**-134, 65504.0, 3.0e38, 3.4e38, 3.3895313892515355e38, 2.0**128, 1e300, -1e-300]
    # exact midpoints between neighbours, and points just beside them
    table = _finite_bf16_table()
    for i in rng.integers(0, len(table) - 1, size=200):
        mid = (table[i] + table[i + 1]) / 2.0
        tests += [mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf), -mid]
    tests += list(rng.standard_normal(300) * 10.0 ** rng.integers(-40, 38, size=300))
    for x in tests:
        assert oracle.double_to_bf16(float(x)) == brute_nearest_bf16(float(x)), x


def test_bf16_rounding_of_floats_against_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    xs = np.concatenate([rng.standard_normal(4000).astype(np.float32),
                         (rng.standard_normal(1000) * 1e-38).astype(np.float32),
                         np.array([1 + 2**-8, 1 + 3 * 2**-8, 3.3895e38, -3.39e38], dtype=np.float32)])
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.double_to_bf16(float(x)) for x in xs], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)


# --------------------------------------------------------------------------
# Unpermute.
# --------------------------------------------------------------------------
def _bf16_bits_from_f32(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f32_from_bf16_bits(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unpermute_topk1_weight1_is_a_gather(dtype):
    rng = np.random.default_rng(5)
    n, h = 29, 40
    inv = rng.permutation(n).astype(np.int32)
    y = rng.standard_normal((n, h)).astype(np.float32)
    if dtype == "bf16":
        y = _bf16_bits_from_f32(y)
    out = oracle.unpermute(y, np.ones((n, 1), np.float32), inv, dtype)
    np.testing.assert_array_equal(out, y[inv])


@pytest.mark.parametrize("dtype,topk", [("f32", 1), ("f32", 2), ("bf16", 1), ("bf16", 2), ("bf16", 4), ("bf16", 8)])
def test_round_trip_identity_experts_is_exact(dtype, topk):
    # With identity experts (Y = permuted X) and all weights 1/topk, every partial sum
    # j*x/topk is exact in fp32 for bf16 x (8 significant bits + log2(topk) <= 24), and
    # for fp32 x when topk <= 2; the double sum is exact as well, so out == x bit for bit.
    rng = np.random.default_rng(6)
    n, e, h = 50, 9, 24
    ids = np.stack([rng.permutation(e)[:topk] for _ in range(n)]).astype(np.int32)
    x = rng.standard_normal((n, h)).astype(np.float32)
    if dtype == "bf16":
        x = _bf16_bits_from_f32(x)
    p = oracle.permute(x, ids, e)
    w = np.full((n, topk), 1.0 / topk, np.float32)
    out = oracle.unpermute(p["permuted_hidden_states"], w, p["inv_permuted_idx"], dtype)
    np.testing.assert_array_equal(out, x)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_round_trip_weights_sum_to_one(dtype):
    rng = np.random.default_rng(8)
    n, e, k, h = 64, 16, 6, 32
    ids = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    x = rng.standard_normal((n, h)).astype(np.float32)
    wt = rng.random((n, k))
    wt = (wt / wt.sum(1, keepdims=True)).astype(np.float32)
    if dtype == "bf16":
        x = _bf16_bits_from_f32(x)
    p = oracle.permute(x, ids, e)
    out = oracle.unpermute(p["permuted_hidden_states"], wt, p["inv_permuted_idx"], dtype)
    xf = _f32_from_bf16_bits(x) if dtype == "bf16" else x
    of = _f32_from_bf16_bits(out) if dtype == "bf16" else out
    # weights sum to 1 up to float32 rounding of each weight (k * 2^-24) plus one output rounding
    tol = (2.0**-8 if dtype == "bf16" else 2.0**-23) * np.abs(xf) + k * 2.0**-23 * np.abs(xf) + 1e-30
    assert np.all(np.abs(of - xf) <= tol)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unpermute_against_float64_einsum(dtype):
    rng = np.random.default_rng(9)
    n, e, k, h = 41, 7, 3, 35
    ids = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    p = oracle.permute(np.zeros((n, 1), np.float32), ids, e)
    inv = p["inv_permuted_idx"]
    y32 = rng.standard_normal((n * k, h)).astype(np.float32)
    w = rng.standard_normal((n, k)).astype(np.float32)
    y = _bf16_bits_from_f32(y32) if dtype == "bf16" else y32
    yv = _f32_from_bf16_bits(y) if dtype == "bf16" else y
    ref = np.einsum("tk,tkh->th", w.astype(np.float64), yv.astype(np.float64)[inv.reshape(n, k)])
    out = oracle.unpermute(y, w, inv, dtype)
    if dtype == "f32":
        np.testing.assert_array_equal(out, ref.astype(np.float32))
    else:
        # every output is the nearest bf16 of the exact sum
        flat_ref = ref.reshape(-1)
        flat_out = out.reshape(-1)
        for i in range(0, flat_ref.shape[0], 7):
            assert flat_out[i] == brute_nearest_bf16(float(flat_ref[i]))
        of = _f32_from_bf16_bits(out).astype(np.float64)
        assert np.all(np.abs(of - ref) <= 2.0**-8 * np.abs(ref) + 2.0**-133)


def test_unpermute_weight_index_is_token_major():
    # w[t, k] multiplies the row of expanded row r = t*topk + k (not w[k, t]).
    n, k, h = 3, 2, 1
    inv = np.arange(n * k, dtype=np.int32)
    y = np.arange(1, n * k + 1, dtype=np.float32).reshape(n * k, h)
    w = np.array([[1, 10], [100, 1000], [10000, 100000]], np.float32)
    out = oracle.unpermute(y, w, inv, "f32")
    assert out.reshape(-1).tolist() == [1 * 1 + 10 * 2, 100 * 3 + 1000 * 4, 10000 * 5 + 100000 * 6]


# --------------------------------------------------------------------------
# Local-expert filter (expert parallelism).  The reading pinned here: the
# expert map sends a global expert id to its local id, or to -1 when the expert
# lives on another rank; local rows are ordered by local id, then ascending
# expanded row; other rows get inverse index -1 and add nothing when unpermuted.
# --------------------------------------------------------------------------
def brute_permute_local(ids2d, emap, num_local, hidden_rows):
    flat = [int(v) for row in ids2d for v in row]
    topk = len(ids2d[0]) if len(ids2d) else 1
    keyed = sorted((emap[g], r) for r, g in enumerate(flat) if emap[g] >= 0)  # tuple sort, not a counting pass
    perm = [r for _, r in keyed]
    inv = [-1] * len(flat)
    for j, r in enumerate(perm):
        inv[r] = j
    off = [0]
    for l in range(num_local):
        off.append(off[-1] + sum(1 for g in flat if emap[g] == l))
    return off, perm, inv, [hidden_rows[r // topk] for r in perm]


def _maps(rng, e):
    """(name, expert_map, num_local) cases of several shapes for e global experts."""
    out = [("identity", list(range(e)), e), ("none_local", [-1] * e, 1)]
    if e >= 2:
        half = e // 2
        out.append(("upper_half", [-1] * half + list(range(e - half)), e - half))
        out.append(("lower_half", list(range(half)) + [-1] * (e - half), half))
        out.append(("even", [g // 2 if g % 2 == 0 else -1 for g in range(e)], (e + 1) // 2))
    if e >= 3:  # local ids not monotone in the global id
        chosen = rng.permutation(e)[: e - 1]
        m = [-1] * e
        for l, g in enumerate(chosen):
            m[int(g)] = l
        out.append(("shuffled", m, e - 1))
        out.append(("one_local_unused_slot", [0 if g == e - 1 else -1 for g in range(e)], 2))
    return out


@pytest.mark.parametrize("n,k,e", list(itertools.product([0, 1, 3, 7, 16], [1, 2, 3, 8], [1, 2, 3, 8])))
def test_oracle_permute_local_matches_brute_force(n, k, e):
    rng = np.random.default_rng(2000 + 97 * n + 13 * k + e)
    for mode in ("random", "one_expert", "distinct", "skip_first_last"):
        ids = _grid_ids(rng, n, k, e, mode).astype(np.int32).reshape(n, k)
        hidden = rng.standard_normal((n, 3)).astype(np.float32)
        scale = rng.random(n).astype(np.float32)
        for name, emap, nl in _maps(rng, e):
            got = oracle.permute_local(hidden, ids, e, emap, nl, token_scale=scale)
            off, perm, inv, gathered = brute_permute_local(ids.tolist(), emap, nl, [row.tobytes() for row in hidden])
            assert got["expert_first_token_offset"].tolist() == off, name
            assert got["permuted_idx"].tolist() == perm, name
            assert got["inv_permuted_idx"].tolist() == inv, name
            assert [row.tobytes() for row in got["permuted_hidden_states"]] == gathered, name
            assert got["permuted_scale"].tolist() == [float(scale[r // k]) for r in perm], name


def test_local_hand_worked_example():
    # 3 tokens, topk 2, 4 global experts; this rank holds experts 3 and 1 as
    # local 0 and 1 (map [-1, 1, -1, 0]).
    # ids: t0 -> (1, 2), t1 -> (3, 1), t2 -> (0, 3); expanded rows r = 2t + k:
    #   r0:1  r1:2  r2:3  r3:1  r4:0  r5:3
    # local ids: r0:1  r1:-  r2:0  r3:1  r4:-  r5:0
    # local 0 (expert 3) gets rows 2, 5; local 1 (expert 1) gets rows 0, 3.
    # offsets [0, 2, 4]; permuted_idx [2, 5, 0, 3];
    # inv: r0->2, r1->-1, r2->0, r3->3, r4->-1, r5->1.
    # Gathered tokens r // 2: [1, 2, 0, 1].
    ids = np.array([[1, 2], [3, 1], [0, 3]], np.int32)
    hidden = np.array([[10.0], [20.0], [30.0]], np.float32)
    got = oracle.permute_local(hidden, ids, 4, [-1, 1, -1, 0], 2)
    assert got["expert_first_token_offset"].tolist() == [0, 2, 4]
    assert got["permuted_idx"].tolist() == [2, 5, 0, 3]
    assert got["inv_permuted_idx"].tolist() == [2, -1, 0, 3, -1, 1]
    assert got["permuted_hidden_states"].reshape(-1).tolist() == [20.0, 30.0, 10.0, 20.0]
    # unpermute with Y = the gathered rows times (slot + 1): token 0 gets
    # w00 * Y[2] + (nothing for r1) = 0.5 * 30; token 1 gets w10*Y[0] + w11*Y[3]
    # = 0.25*20 + 2*80; token 2 gets (nothing for r4) + w21*Y[1] = 4 * 60.
    y = (got["permuted_hidden_states"].reshape(-1) * np.arange(1, 5, dtype=np.float32)).reshape(4, 1)
    w = np.array([[0.5, 9.0], [0.25, 2.0], [9.0, 4.0]], np.float32)
    out = oracle.unpermute(y, w, got["inv_permuted_idx"], "f32")
    assert out.reshape(-1).tolist() == [15.0, 165.0, 240.0]


@pytest.mark.parametrize("bad_map", [[0, 2, -1], [0, -2, 1], [3, 0, 1]])
def test_local_bad_map_rejected(bad_map):
    ids = np.array([[0, 1], [2, 1]], np.int32)
    with pytest.raises(oracle.OracleError):
        oracle.permute_local(np.zeros((2, 4), np.float32), ids, 3, bad_map, 2)


def test_local_bad_id_rejected():
    ids = np.array([[0, 3]], np.int32)
    with pytest.raises(oracle.OracleError):
        oracle.permute_local(np.zeros((1, 4), np.float32), ids, 3, [0, -1, 1], 2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ranks,layout", [(2, "contiguous"), (4, "contiguous"), (4, "round_robin"), (3, "contiguous")])
def test_expert_parallel_ranks_sum_to_the_full_unpermute(dtype, ranks, layout):
    # Split the experts over ranks; each rank permutes only its experts, runs
    # its "experts" on its rows and unpermutes with -1 for remote slots.  The
    # partial outputs summed over ranks must equal the single-rank result.  The
    # values are small integers and the weights powers of two, so every sum is
    # exact and the comparison is bit for bit.  For bfloat16 (8 significant
    # bits) x is in {-1, 0, 1} and w in {1/2, 1}: every term is a multiple of
    # 1/2 of size <= 12 and every sum of 4 terms at most 192 halves < 2^8.
    rng = np.random.default_rng(11 + ranks)
    n, e, k, h = 57, 12, 4, 6
    ids = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    if dtype == "bf16":
        x = _bf16_bits_from_f32(rng.integers(-1, 2, size=(n, h)).astype(np.float32))
        w = (2.0 ** rng.integers(-1, 1, size=(n, k))).astype(np.float32)
    else:
        x = rng.integers(-8, 9, size=(n, h)).astype(np.float32)
        w = (2.0 ** rng.integers(-3, 3, size=(n, k))).astype(np.float32)

    def expert_fn(rows, expert_ids):  # a per-expert map of the row: x * (expert + 1)
        xf = _f32_from_bf16_bits(rows) if dtype == "bf16" else rows
        yf = xf * (expert_ids[:, None] + 1).astype(np.float32)
        return _bf16_bits_from_f32(yf) if dtype == "bf16" else yf

    full = oracle.permute(x, ids, e)
    full_experts = ids.reshape(-1)[full["permuted_idx"]]
    want = oracle.unpermute(expert_fn(full["permuted_hidden_states"], full_experts), w,
                            full["inv_permuted_idx"], dtype)
    total = np.zeros((n, h), np.float64)
    covered = np.zeros(n * k, np.int64)
    for rank in range(ranks):
        if layout == "contiguous":
            owned = [g for g in range(e) if g * ranks // e == rank]
        else:
            owned = [g for g in range(e) if g % ranks == rank]
        emap = [-1] * e
        for l, g in enumerate(owned):
            emap[g] = l
        part = oracle.permute_local(x, ids, e, emap, len(owned))
        covered += part["inv_permuted_idx"] >= 0
        experts = ids.reshape(-1)[part["permuted_idx"]]
        y = expert_fn(part["permuted_hidden_states"], experts)
        out = oracle.unpermute(y, w, part["inv_permuted_idx"], dtype)
        total += (_f32_from_bf16_bits(out) if dtype == "bf16" else out).astype(np.float64)
    assert covered.tolist() == [1] * (n * k)  # every slot is local on exactly one rank
    wantf = (_f32_from_bf16_bits(want) if dtype == "bf16" else want).astype(np.float64)
    np.testing.assert_array_equal(total, wantf)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unpermute_minus_one_slots_match_masked_einsum(dtype):
    rng = np.random.default_rng(12)
    n, k, h = 37, 3, 20
    inv = rng.permutation(n * k).astype(np.int32)
    drop = rng.random(n * k) < 0.4
    inv[drop] = -1
    inv[0:k] = -1  # token 0 has no local slot: its output is exactly zero
    y32 = rng.standard_normal((n * k, h)).astype(np.float32)
    w = rng.standard_normal((n, k)).astype(np.float32)
    y = _bf16_bits_from_f32(y32) if dtype == "bf16" else y32
    yv = (_f32_from_bf16_bits(y) if dtype == "bf16" else y).astype(np.float64)
    mask = (inv >= 0).reshape(n, k).astype(np.float64)
    gathered = yv[np.where(inv >= 0, inv, 0)].reshape(n, k, h)
    ref = np.einsum("tk,tkh->th", w.astype(np.float64) * mask, gathered)
    out = oracle.unpermute(y, w, inv, dtype)
    of = (_f32_from_bf16_bits(out) if dtype == "bf16" else out).astype(np.float64)
    if dtype == "f32":
        np.testing.assert_array_equal(out, ref.astype(np.float32))
    else:
        assert np.all(np.abs(of - ref) <= 2.0**-8 * np.abs(ref) + 2.0**-133)
    assert np.all(of[0] == 0.0)


# --------------------------------------------------------------------------
# int64 expert ids.  The permute depends only on the id values; an int64 value
# outside [0, E) is an error even when its low 32 bits are a valid id.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n,k,e", [(0, 2, 4), (1, 1, 1), (7, 3, 8), (16, 8, 8), (50, 4, 300)])
def test_int64_ids_permute_like_their_values(n, k, e):
    rng = np.random.default_rng(300 + n + k + e)
    ids64 = rng.integers(0, e, size=(n, k)).astype(np.int64)
    hidden = rng.standard_normal((n, 4)).astype(np.float32)
    got = oracle.permute(hidden, ids64, e)
    off, perm, inv, gathered = brute_permute([[int(v) for v in row] for row in ids64.tolist()], e,
                                             [row.tobytes() for row in hidden])
    assert got["expert_first_token_offset"].tolist() == off
    assert got["permuted_idx"].tolist() == perm
    assert got["inv_permuted_idx"].tolist() == inv
    assert [row.tobytes() for row in got["permuted_hidden_states"]] == gathered


@pytest.mark.parametrize("bad", [8, -1, 2**31, 2**32 + 3, -(2**32), -(2**32) + 5, 2**63 - 1, -(2**63)])
def test_int64_ids_outside_range_rejected_not_truncated(bad):
    ids = np.array([[0, 1], [2, 3]], dtype=np.int64)
    ids[1, 0] = bad
    with pytest.raises(oracle.OracleError):
        oracle.permute(np.zeros((2, 4), np.float32), ids, 8)
    with pytest.raises(oracle.OracleError):
        oracle.permute_local(np.zeros((2, 4), np.float32), ids, 8, list(range(8)), 8)


# --------------------------------------------------------------------------
# fp8 E4M3FN and the dynamic fp8 quantiser (quantise while permuting).
# --------------------------------------------------------------------------
def _e4m3_finite_table():
    """(value, code) for every finite E4M3FN code, decoded by torch."""
    import torch

    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return [(float(vals[c]), c) for c in range(256) if not np.isnan(vals[c])]


def test_e4m3_decode_all_codes_against_torch():
    import torch

    vals = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = oracle.e4m3_to_double(c)
        if np.isnan(vals[c]):
            assert np.isnan(got), c
        else:
            assert got == vals[c], (c, got, vals[c])
    assert oracle.e4m3_to_double(0x7E) == 448.0 and np.isnan(oracle.e4m3_to_double(0x7F))


def brute_nearest_e4m3(x: float) -> int:
    """Exhaustive search over the finite codes of the clamped value; ties go to the
    code with an even fraction; zero keeps the sign of x."""
    if np.isnan(x):
        return 0xFF if np.signbit(x) else 0x7F
    a = min(abs(x), 448.0)
    best = None
    for v, c in _E4M3:
        if v < 0 or (v == 0 and c != 0):
            continue
        d = abs(Fraction(v) - Fraction(a))
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c)
    code = best[1]
    return code | 0x80 if np.signbit(x) else code


_E4M3 = None


def test_e4m3_encode_against_exhaustive_nearest():
    global _E4M3
    _E4M3 = _e4m3_finite_table()
    pos = sorted(v for v, c in _E4M3 if v >= 0 and not (v == 0 and c != 0))
    probes = [0.0, -0.0, 448.0, 449.0, 464.0, 465.0, 1e9, -1e9, 2.0**-12, 2.0**-10, 2.0**-9, 2.0**-6 - 2.0**-10]
    for lo, hi in zip(pos, pos[1:]):
        mid = (lo + hi) / 2
        probes += [lo, mid, np.nextafter(mid, 0.0), np.nextafter(mid, 1e9), -mid]
    rng = np.random.default_rng(13)
    probes += list(rng.uniform(-460, 460, 3000)) + list(rng.uniform(-2.0**-5, 2.0**-5, 1000))
    for x in probes:
        assert oracle.double_to_e4m3(float(x)) == brute_nearest_e4m3(float(x)), x
    assert oracle.double_to_e4m3(float("nan")) == 0x7F


def test_e4m3_encode_against_torch_in_range():
    import torch

    rng = np.random.default_rng(14)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-1, 1, 20000),
                        rng.uniform(-2.0**-6, 2.0**-6, 5000)]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.double_to_e4m3(float(v)) for v in x], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def _rows(rng, n, h, dtype):
    x = (rng.standard_normal((n, h)) * rng.choice([1e-3, 1.0, 50.0], size=(n, 1))).astype(np.float32)
    return _bf16_bits_from_f32(x) if dtype == "bf16" else x


def _as_f32(x, dtype):
    return _f32_from_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("group", [None, 8, 32, 128])
def test_quantizer_properties(dtype, group):
    rng = np.random.default_rng(15)
    n, h = 40, 256
    x = _rows(rng, n, h, dtype)
    xf = _as_f32(x, dtype).astype(np.float64)
    codes, scales = oracle.quantize_fp8_rows(x, dtype, group)
    g = h if group is None else group
    assert scales.shape == (n, h // g)
    dq = np.vectorize(oracle.e4m3_to_double)(codes)
    for r in range(n):
        for q in range(h // g):
            seg = slice(q * g, (q + 1) * g)
            amax = np.max(np.abs(xf[r, seg]))
            s = float(scales[r, q])
            # scale is amax / 448 to float precision
            assert abs(s - amax / 448.0) <= 2.0**-24 * amax / 448.0
            # the element of largest magnitude lands on +-448
            i = q * g + int(np.argmax(np.abs(xf[r, seg])))
            assert codes[r, i] & 0x7F == 0x7E
            # every element is within half an fp8 step (relative 2^-4) plus one float rounding
            y = xf[r, seg] / s
            err = np.abs(dq[r, seg] - y)
            step = np.maximum(np.abs(y), 2.0**-6) * 2.0**-3
            assert np.all(err <= step / 2 * (1 + 2.0**-20) + 1e-30)
            # signs are kept
            nz = xf[r, seg] != 0
            assert np.all((codes[r, seg][nz] >= 0x80) == (xf[r, seg][nz] < 0) | (codes[r, seg][nz] == 0x80) |
                          (codes[r, seg][nz] == 0))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantizer_special_cases(dtype):
    h = 64
    x = np.zeros((3, h), np.float32)
    x[1, 5] = -3.0
    x[2] = np.linspace(-1, 1, h, dtype=np.float32)
    if dtype == "bf16":
        x = _bf16_bits_from_f32(x)
    codes, scales = oracle.quantize_fp8_rows(x, dtype)
    assert scales[0, 0] == 1.0 and np.all(codes[0] == 0)          # all-zero row
    assert scales[1, 0] == np.float32(3.0) / np.float32(448.0)
    assert codes[1, 5] == 0xFE and np.all(np.delete(codes[1], 5) == 0)
    # sign symmetry (every code's sign bit flips, zeros to -0) and power-of-two scaling
    xf = _as_f32(x, dtype)
    neg, dbl = -xf, xf * 2
    if dtype == "bf16":
        neg, dbl = _bf16_bits_from_f32(neg), _bf16_bits_from_f32(dbl)
    c_neg, s_neg = oracle.quantize_fp8_rows(neg, dtype)
    np.testing.assert_array_equal(c_neg, codes ^ 0x80)
    np.testing.assert_array_equal(s_neg, scales)
    c_dbl, s_dbl = oracle.quantize_fp8_rows(dbl, dtype)
    np.testing.assert_array_equal(c_dbl, codes)
    np.testing.assert_array_equal(s_dbl[1:], scales[1:] * 2)
    assert s_dbl[0, 0] == 1.0


def test_quantizer_group_is_not_the_whole_row():
    # two groups with very different magnitudes get different scales
    x = np.concatenate([np.full((1, 8), 1000.0), np.full((1, 8), 0.001)], axis=1).astype(np.float32)
    codes, scales = oracle.quantize_fp8_rows(x, "f32", 8)
    assert scales.shape == (1, 2) and scales[0, 0] > 1.0 and scales[0, 1] < 1e-5
    assert np.all(codes == 0x7E)


@pytest.mark.parametrize("local", [False, True])
def test_permute_quant_moves_scales_with_rows(local):
    rng = np.random.default_rng(16)
    n, k, e, h = 33, 3, 8, 64
    ids = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    x = _bf16_bits_from_f32(rng.standard_normal((n, h)).astype(np.float32))
    emap, nl = (W.expert_map_for(e, 2, 1, "shuffled") if local else (None, None))
    res = oracle.permute_quant_fp8(x, "bf16", ids, e, 16, emap, nl)
    codes, scales = oracle.quantize_fp8_rows(x, "bf16", 16)
    perm = res["permuted_idx"]
    np.testing.assert_array_equal(res["permuted_hidden_states"], codes[perm // k])
    np.testing.assert_array_equal(res["permuted_scale"], scales[perm // k])


def test_quantizer_non_finite_inputs():
    x = np.array([[1.0, np.nan, -2.0, 0.5], [np.inf, 1.0, -1.0, 0.0], [-np.inf, np.inf, 3.0, -0.0]], np.float32)
    codes, scales = oracle.quantize_fp8_rows(x, "f32")
    # NaN is ignored by amax and coded 0x7F; the rest quantise against amax 2
    assert scales[0, 0] == np.float32(2.0) / np.float32(448.0)
    assert codes[0, 1] == 0x7F and codes[0, 2] == 0xFE
    # an infinite amax gives an infinite scale: finite values go to (signed) zero, inf / inf is NaN
    assert np.isinf(scales[1, 0]) and codes[1].tolist() == [0x7F, 0x00, 0x80, 0x00]
    assert codes[2].tolist() == [0x7F, 0x7F, 0x00, 0x80]


# --------------------------------------------------------------------------
# Grouped GEMM over the permuted rows: y[j] = x[j] w[e]^T for the rows of expert e.
# --------------------------------------------------------------------------
def _random_offsets(rng, e, rows, empties=()):
    counts = rng.multinomial(rows, np.ones(e) / e)
    for x in empties:
        rows_moved = counts[x]
        counts[x] = 0
        counts[(x + 1) % e] += rows_moved
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def test_grouped_gemm_against_float64_matmul():
    rng = np.random.default_rng(21)
    e, n, k, rows = 5, 24, 40, 70
    off = _random_offsets(rng, e, rows, empties=(2,))
    x = _bf16_bits_from_f32(rng.standard_normal((rows, k)).astype(np.float32))
    w = _bf16_bits_from_f32(rng.standard_normal((e, n, k)).astype(np.float32) * 0.1)
    y = oracle.grouped_gemm_bf16(x, w, off)
    xf = _f32_from_bf16_bits(x).astype(np.float64)
    wf = _f32_from_bf16_bits(w).astype(np.float64)
    for ex in range(e):
        seg = slice(off[ex], off[ex + 1])
        ref = xf[seg] @ wf[ex].T
        got = _f32_from_bf16_bits(y[seg]).astype(np.float64)
        # every output is the nearest bf16 of the float64 product sum
        assert np.all(np.abs(got - ref) <= 2.0**-8 * np.abs(ref) + 2.0**-133)
        for v_got, v_ref in list(zip(y[seg].reshape(-1), ref.reshape(-1)))[::17]:
            assert int(v_got) == brute_nearest_bf16(float(v_ref))


def test_grouped_gemm_exact_small_integers():
    # small integers: every product and sum is exact, so y is the integer result
    rng = np.random.default_rng(22)
    e, n, k, rows = 3, 8, 16, 11
    off = np.array([0, 4, 4, 11], np.int64)
    xi = rng.integers(-4, 5, size=(rows, k))
    wi = rng.integers(-3, 4, size=(e, n, k))
    y = oracle.grouped_gemm_bf16(_bf16_bits_from_f32(xi.astype(np.float32)),
                                 _bf16_bits_from_f32(wi.astype(np.float32)), off)
    for ex in range(e):
        for j in range(off[ex], off[ex + 1]):
            for c in range(n):
                want = sum(int(xi[j, q]) * int(wi[ex, c, q]) for q in range(k))
                assert _f32_from_bf16_bits(y[j:j + 1, c:c + 1])[0, 0] == want


def test_grouped_gemm_routes_rows_to_their_expert():
    # w[e] = (e + 1) * I: each row comes back scaled by its expert's number
    e, k, rows = 4, 16, 13
    off = np.array([0, 3, 3, 9, 13], np.int64)
    x = _bf16_bits_from_f32(np.arange(rows * k, dtype=np.float32).reshape(rows, k) % 7 - 3)
    w = _bf16_bits_from_f32(np.stack([np.eye(k, dtype=np.float32) * (ex + 1) for ex in range(e)]))
    y = _f32_from_bf16_bits(oracle.grouped_gemm_bf16(x, w, off))
    xf = _f32_from_bf16_bits(x)
    for ex in range(e):
        np.testing.assert_array_equal(y[off[ex]:off[ex + 1]], xf[off[ex]:off[ex + 1]] * (ex + 1))


def test_grouped_gemm_rejects_bad_offsets():
    x = np.zeros((4, 8), np.uint16)
    w = np.zeros((2, 8, 8), np.uint16)
    with pytest.raises(oracle.OracleError):
        oracle.grouped_gemm_bf16(x, w, np.array([0, 3, 2], np.int64))
    with pytest.raises(oracle.OracleError):
        oracle.grouped_gemm_bf16(x, w, np.array([1, 2, 3], np.int64))


@pytest.mark.parametrize("local", [False, True])
def test_scales_move_on_an_indices_only_call(local):
    """Rows zero bytes wide: the indices are the usual ones and each token's
    scale still reaches every destination of its rows (slot j gets the scale of
    token perm[j] // topk), with and without an expert map."""
    rng = np.random.default_rng(12)
    n, k, e = 9, 3, 5
    ids = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    scale = (rng.random(n) + 0.5).astype(np.float32)
    empty = np.zeros((n, 0), np.float32)
    if local:
        emap = np.array([0, -1, 1, -1, 0], np.int32)
        got = oracle.permute_local(empty, ids, e, emap, 2, token_scale=scale)
        full = oracle.permute_local(np.zeros((n, 4), np.float32), ids, e, emap, 2, token_scale=scale)
    else:
        got = oracle.permute(empty, ids, e, token_scale=scale)
        full = oracle.permute(np.zeros((n, 4), np.float32), ids, e, token_scale=scale)
    m = int(got["expert_first_token_offset"][-1])
    perm = got["permuted_idx"][:m]
    assert got["permuted_scale"][:m].tolist() == [float(scale[r // k]) for r in perm]
    np.testing.assert_array_equal(got["permuted_idx"], full["permuted_idx"])
    np.testing.assert_array_equal(got["permuted_scale"], full["permuted_scale"])
