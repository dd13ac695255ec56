"""Host-side checks of the benchmark's measurement logic (no GPU).

Every GB/s figure and roofline fraction the benchmark prints divides the
algorithmic bytes of an operation -- each input read once, each output written
once -- by a measured time.  These tests pin those byte counts to values
worked out by hand for each workload shape (N tokens, hidden H, E experts,
topk K, R = N*K expanded rows, b bytes per element):

  permute   = N*H*b (read the rows) + R*H*b (write the permuted rows)
              + 4R (int32 ids) + 8R (permuted_idx and inv_permuted_idx)
              + 8(E+1) (int64 offsets) [+ 4N + 4R fp8 token scales]
  unpermute = R*H*b (read the expert rows) + 4R (inverse index) + 4R (weights)
              + N*H*b (write the output)

and check the local-expert and quantising variants against the plain one.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402

# (workload, tokens or None, permute bytes, unpermute bytes)
EXPECTED = [
    ("tiny", None, 25_032, 24_832),
    ("mixtral", None, 100_761_672, 100_728_832),
    ("qwen3", None, 302_777_352, 302_514_176),
    ("dsv3", None, 2_115_504_136, 2_114_977_792),
    ("decode", 1, 66_700, 129_088),
    ("decode", 4, 260_632, 516_352),
    ("decode", 16, 1_036_360, 2_065_408),
    ("decode", 64, 4_139_272, 8_261_632),
    ("decode", 256, 16_550_920, 33_046_528),
]


def _workload(name, tokens):
    w = W.WORKLOADS[name]
    return w if tokens is None else w.with_tokens(tokens)


@pytest.mark.parametrize("name,tokens,permute,unpermute", EXPECTED,
                         ids=["%s-%s" % (c[0], c[1]) for c in EXPECTED])
def test_algorithmic_bytes_match_hand_counts(name, tokens, permute, unpermute):
    got = bench.algorithmic_bytes(_workload(name, tokens))
    assert got["permute"] == permute
    assert got["unpermute"] == unpermute
    assert got["total"] == permute + unpermute


@pytest.mark.parametrize("name,tokens", [("mixtral", None), ("qwen3", None), ("decode", 16)])
def test_local_permute_with_every_expert_local_costs_the_map_read_more(name, tokens):
    """All tokens read, all rows local: the local permute moves the plain
    permute's bytes plus the E-entry expert map; the unpermute is unchanged."""
    w = _workload(name, tokens)
    plain = bench.algorithmic_bytes(w)
    local = bench.algorithmic_bytes(w, local=(w.num_tokens, w.num_rows, w.num_experts))
    assert local["permute"] == plain["permute"] + 4 * w.num_experts
    assert local["unpermute"] == plain["unpermute"]


def test_local_permute_with_nothing_local_moves_only_indices_and_zero_rows():
    w = W.WORKLOADS["mixtral"]
    n, h, r, e = w.num_tokens, w.hidden_size, w.num_rows, w.num_experts
    got = bench.algorithmic_bytes(w, local=(0, 0, 1))
    # ids, the map, the inverse index and the offsets of one local expert
    assert got["permute"] == 4 * r + 4 * e + 4 * r + 8 * 2
    # every token still gets a (zero) output row; the inverse index is read
    assert got["unpermute"] == 4 * r + n * h * 2


@pytest.mark.parametrize("name,groups,permute", [("mixtral", 1, 67_240_008), ("dsv3", 56, 1_205_340_168)])
def test_quantising_permute_bytes(name, groups, permute):
    """bf16 rows in (2 bytes per element), one fp8 code per element and
    `groups` float scales per permuted row out, plus the index outputs."""
    w = W.WORKLOADS[name]
    got = bench.algorithmic_bytes(w, quant_groups=groups)
    assert got["permute"] == permute
    assert got["unpermute"] == bench.algorithmic_bytes(w)["unpermute"]


def test_int64_ids_count_eight_bytes_each():
    w = W.WORKLOADS["mixtral"]
    assert (bench.algorithmic_bytes(w, id_bytes=8)["permute"] - bench.algorithmic_bytes(w)["permute"]
            == 4 * w.num_rows)


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""
