"""The Python binding rejects buffers the kernels would overrun, before any library call (no GPU).

Every entry point derives its sizes from a few tensors (topk_ids or
topk_weights for N and topk, hidden_states for H, num_experts for the offsets)
and hands raw pointers to the C library, which cannot see a tensor's type or
length.  A wrong type or length here would be an out-of-bounds access on the
device, so the binding checks each buffer's dtype, element count, layout and
device first.  The checks run on CPU tensors: every check but the last (GPU
memory) fires the same way; a second device for the mismatch cases is torch's
"meta" device.
"""

import pytest
import torch

from mixture_experts_token_amd import binding as B

N, K, E, H = 6, 2, 4, 16


def _permute_bufs(dtype=torch.bfloat16):
    return dict(
        hidden_states=torch.zeros((N, H), dtype=dtype),
        topk_ids=torch.zeros((N, K), dtype=torch.int32),
        num_experts=E,
        permuted_hidden_states=torch.zeros((N * K, H), dtype=dtype),
        expert_first_token_offset=torch.zeros(E + 1, dtype=torch.int64),
        permuted_idx=torch.zeros(N * K, dtype=torch.int32),
        inv_permuted_idx=torch.zeros(N * K, dtype=torch.int32),
        workspace=torch.zeros(16, dtype=torch.uint8),
    )


def _unpermute_bufs(dtype=torch.bfloat16):
    return dict(
        expanded_output=torch.zeros((N * K, H), dtype=dtype),
        topk_weights=torch.zeros((N, K), dtype=torch.float32),
        inv_permuted_idx=torch.zeros(N * K, dtype=torch.int32),
        output=torch.zeros((N, H), dtype=dtype),
    )


def test_valid_permute_on_cpu_is_rejected_only_for_the_device():
    with pytest.raises(TypeError, match="GPU tensors"):
        B.moe_permute(**_permute_bufs())


UNPERMUTES = [B.moe_unpermute, B.moe_unpermute_local]


@pytest.mark.parametrize("fn", UNPERMUTES, ids=lambda f: f.__name__)
def test_valid_unpermute_on_cpu_is_rejected_only_for_the_device(fn):
    with pytest.raises(TypeError, match="GPU tensors"):
        fn(**_unpermute_bufs())


@pytest.mark.parametrize("key,bad,exc", [
    # int32 offsets: 8 (E + 1) bytes would be written into 4 (E + 1)
    ("expert_first_token_offset", torch.zeros(E + 1, dtype=torch.int32), TypeError),
    ("expert_first_token_offset", torch.zeros(E, dtype=torch.int64), ValueError),
    ("permuted_idx", torch.zeros(N * K - 1, dtype=torch.int32), ValueError),
    ("permuted_idx", torch.zeros(N * K, dtype=torch.int64), TypeError),
    ("inv_permuted_idx", torch.zeros(N * K + 1, dtype=torch.int32), ValueError),
    # rows of another type: a bf16 output for f32 rows would be written twice its size
    ("permuted_hidden_states", torch.zeros((N * K, H), dtype=torch.float32), TypeError),
    ("permuted_hidden_states", torch.zeros((N * K - 1, H), dtype=torch.bfloat16), ValueError),
    ("hidden_states", torch.zeros((N + 1, H), dtype=torch.bfloat16), ValueError),
    ("topk_ids", torch.zeros((N, K), dtype=torch.float32), TypeError),
    ("workspace", torch.zeros(64, dtype=torch.uint8)[::2], ValueError),
])
def test_permute_rejects_wrong_buffers(key, bad, exc):
    bufs = _permute_bufs()
    bufs[key] = bad
    with pytest.raises(exc):
        B.moe_permute(**bufs)


def test_permute_rejects_scales_that_do_not_fit():
    bufs = _permute_bufs(torch.uint8)
    with pytest.raises(ValueError, match="go together"):
        B.moe_permute(**bufs, token_scale=torch.zeros(N, dtype=torch.float32))
    with pytest.raises(ValueError, match="permuted_scale"):
        B.moe_permute(**bufs, token_scale=torch.zeros(N, dtype=torch.float32),
                      permuted_scale=torch.zeros(N, dtype=torch.float32))
    with pytest.raises(TypeError, match="token_scale"):
        B.moe_permute(**bufs, token_scale=torch.zeros(N, dtype=torch.bfloat16),
                      permuted_scale=torch.zeros(N * K, dtype=torch.float32))


def test_permute_rejects_a_buffer_on_another_device():
    bufs = _permute_bufs()
    bufs["inv_permuted_idx"] = torch.empty(N * K, dtype=torch.int32, device="meta")
    with pytest.raises(TypeError, match="meta"):
        B.moe_permute(**bufs)


@pytest.mark.parametrize("key,bad,exc", [
    # bf16 weights would be read as 4-byte floats past their end
    ("topk_weights", torch.zeros((N, K), dtype=torch.bfloat16), TypeError),
    ("inv_permuted_idx", torch.zeros(N * K, dtype=torch.int64), TypeError),
    ("inv_permuted_idx", torch.zeros(N * K - 2, dtype=torch.int32), ValueError),
    # a bf16 output for f32 rows is written with 4-byte elements
    ("output", torch.zeros((N, H), dtype=torch.float32), TypeError),
    ("output", torch.zeros((N - 1, H), dtype=torch.bfloat16), ValueError),
    ("expanded_output", torch.zeros((N * K - 1, H), dtype=torch.bfloat16), ValueError),
    ("output", torch.zeros((N, 2 * H), dtype=torch.bfloat16)[:, ::2], ValueError),
])
@pytest.mark.parametrize("fn", UNPERMUTES, ids=lambda f: f.__name__)
def test_unpermute_rejects_wrong_buffers(fn, key, bad, exc):
    bufs = _unpermute_bufs()
    bufs[key] = bad
    with pytest.raises(exc):
        fn(**bufs)


@pytest.mark.parametrize("fn", UNPERMUTES, ids=lambda f: f.__name__)
def test_unpermute_rejects_a_buffer_on_another_device(fn):
    bufs = _unpermute_bufs()
    bufs["output"] = torch.empty((N, H), dtype=torch.bfloat16, device="meta")
    with pytest.raises(TypeError, match="meta"):
        fn(**bufs)


def _local_bufs():
    bufs = _permute_bufs()
    L = 2
    bufs["expert_first_token_offset"] = torch.zeros(L + 1, dtype=torch.int64)
    return dict(bufs, expert_map=torch.tensor([0, 1, -1, -1], dtype=torch.int32), num_local_experts=L)


def test_local_permute_sizes_the_offsets_by_local_experts():
    bufs = _local_bufs()
    with pytest.raises(TypeError, match="GPU tensors"):
        B.moe_permute_local(**bufs)
    bufs["expert_first_token_offset"] = torch.zeros(E + 1, dtype=torch.int64)
    with pytest.raises(ValueError, match="expert_first_token_offset"):
        B.moe_permute_local(**bufs)


def _quant_bufs(group_size=0):
    groups = 1 if group_size == 0 else H // group_size
    return dict(
        hidden_states=torch.zeros((N, H), dtype=torch.bfloat16),
        topk_ids=torch.zeros((N, K), dtype=torch.int32),
        num_experts=E,
        permuted_codes=torch.zeros((N * K, H), dtype=torch.uint8),
        permuted_scale=torch.zeros((N * K, groups), dtype=torch.float32),
        expert_first_token_offset=torch.zeros(E + 1, dtype=torch.int64),
        permuted_idx=torch.zeros(N * K, dtype=torch.int32),
        inv_permuted_idx=torch.zeros(N * K, dtype=torch.int32),
        workspace=torch.zeros(16, dtype=torch.uint8),
        group_size=group_size,
    )


def test_quant_permute_checks_codes_and_scales():
    with pytest.raises(TypeError, match="GPU tensors"):
        B.moe_permute_quant_fp8(**_quant_bufs(8))
    bufs = _quant_bufs(8)
    bufs["permuted_scale"] = torch.zeros((N * K, 1), dtype=torch.float32)  # per-group scales need H / 8 columns
    with pytest.raises(ValueError, match="permuted_scale"):
        B.moe_permute_quant_fp8(**bufs)
    bufs = _quant_bufs()
    bufs["permuted_codes"] = torch.zeros((N * K, H), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="permuted_codes"):
        B.moe_permute_quant_fp8(**bufs)
    bufs = _quant_bufs()
    bufs["group_size"] = 3
    with pytest.raises(ValueError, match="group_size"):
        B.moe_permute_quant_fp8(**bufs)


def test_grouped_gemm_checks_its_buffers():
    rows, n, k = 8, 128, 64
    x = torch.zeros((rows, k), dtype=torch.bfloat16)
    w = torch.zeros((E, n, k), dtype=torch.bfloat16)
    y = torch.zeros((rows, n), dtype=torch.bfloat16)
    off = torch.zeros(E + 1, dtype=torch.int64)
    with pytest.raises(TypeError, match="GPU tensors"):
        B.moe_grouped_gemm_bf16(x, w, off, y)
    with pytest.raises(ValueError, match="expert_first_token_offset"):
        B.moe_grouped_gemm_bf16(x, w, torch.zeros(E, dtype=torch.int64), y)
    with pytest.raises(ValueError, match="y"):
        B.moe_grouped_gemm_bf16(x, w, off, torch.zeros((rows - 1, n), dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        B.moe_grouped_gemm_bf16(x, w, off, torch.zeros((rows, n), dtype=torch.float32))
