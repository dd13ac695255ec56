"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
(via the binding) and the CPU oracle on the same inputs, and compare."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from mixture_experts_token_amd import binding

POISON = 0xFF  # fill byte for outputs and workspace before a call


def to_np(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy; bfloat16 comes back as uint16 bit patterns, fp8 as uint8."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def poisoned(shape, dtype, device):
    t = torch.empty(shape, dtype=dtype, device=device)
    t.view(torch.uint8).fill_(POISON)
    return t


def gpu_permute(hidden, ids, num_experts, token_scale=None, workspace=None, stream=None, outs=None):
    """Run moe_permute into poisoned (or given) outputs; returns the output tensors."""
    dev = ids.device
    n, k = ids.shape
    rows = n * k
    if outs is None:
        outs = {
            "permuted_hidden_states": None if hidden is None else poisoned((rows, hidden.shape[1]), hidden.dtype, dev),
            "permuted_scale": None if token_scale is None else poisoned((rows,), torch.float32, dev),
            "expert_first_token_offset": poisoned((num_experts + 1,), torch.int64, dev),
            "permuted_idx": poisoned((rows,), torch.int32, dev),
            "inv_permuted_idx": poisoned((rows,), torch.int32, dev),
        }
    if workspace is None:
        ws = binding.moe_permute_workspace_size(n, k, num_experts)
        workspace = poisoned((max(ws, 16),), torch.uint8, dev)
    binding.moe_permute(hidden, ids, num_experts, outs["permuted_hidden_states"], outs["expert_first_token_offset"],
                        outs["permuted_idx"], outs["inv_permuted_idx"], workspace, token_scale=token_scale,
                        permuted_scale=outs["permuted_scale"], stream=stream)
    return outs


def gpu_unpermute(y, weights, inv, stream=None, local=False):
    """moe_unpermute, or moe_unpermute_local (local=True), into a poisoned output."""
    n = weights.shape[0]
    out = poisoned((n, y.shape[1]), y.dtype, y.device)
    (binding.moe_unpermute_local if local else binding.moe_unpermute)(y, weights, inv, out, stream=stream)
    return out


def oracle_permute(hidden, ids, num_experts, token_scale=None):
    h = to_np(hidden) if hidden is not None else np.zeros((ids.shape[0], 0), np.float32)
    return oracle.permute(h, to_np(ids), num_experts, None if token_scale is None else to_np(token_scale))


def assert_permute_equal(outs, ref, check_rows=True):
    np.testing.assert_array_equal(to_np(outs["expert_first_token_offset"]), ref["expert_first_token_offset"])
    np.testing.assert_array_equal(to_np(outs["permuted_idx"]), ref["permuted_idx"])
    np.testing.assert_array_equal(to_np(outs["inv_permuted_idx"]), ref["inv_permuted_idx"])
    if check_rows and outs["permuted_hidden_states"] is not None:
        got = to_np(outs["permuted_hidden_states"])
        exp = ref["permuted_hidden_states"]
        assert got.shape == exp.shape
        if not np.array_equal(got.view(np.uint8), exp.view(np.uint8)):
            bad = np.nonzero(np.any(got.view(np.uint8).reshape(got.shape[0], -1)
                                    != exp.view(np.uint8).reshape(exp.shape[0], -1), axis=1))[0]
            raise AssertionError("permuted rows differ at %d rows, first %s" % (bad.size, bad[:8].tolist()))
    if outs.get("permuted_scale") is not None:
        np.testing.assert_array_equal(to_np(outs["permuted_scale"]).view(np.uint32),
                                      ref["permuted_scale"].view(np.uint32))


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def tolerance(dtype: str) -> float:
    # |gpu - oracle| <= tol * max(1, |oracle|): bf16 2^-7, fp32 1e-5
    return 2.0**-7 if dtype == "bf16" else 1e-5


def assert_unpermute_close(got: np.ndarray, ref: np.ndarray, dtype: str):
    g = as_f64(got, dtype)
    r = as_f64(ref, dtype)
    assert g.shape == r.shape
    assert not np.isnan(g).any(), "NaN in unpermute output"
    err = np.abs(g - r) / np.maximum(1.0, np.abs(r))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tolerance(dtype), "max scaled error %.3g > %.3g" % (worst, tolerance(dtype))
    return worst


def gpu_permute_local(hidden, ids, num_experts, expert_map, num_local, token_scale=None, workspace=None, stream=None,
                      outs=None):
    """Run moe_permute_local into poisoned (or given) outputs; returns the output tensors."""
    dev = ids.device
    n, k = ids.shape
    rows = n * k
    if outs is None:
        outs = {
            "permuted_hidden_states": None if hidden is None else poisoned((rows, hidden.shape[1]), hidden.dtype, dev),
            "permuted_scale": None if token_scale is None else poisoned((rows,), torch.float32, dev),
            "expert_first_token_offset": poisoned((num_local + 1,), torch.int64, dev),
            "permuted_idx": poisoned((rows,), torch.int32, dev),
            "inv_permuted_idx": poisoned((rows,), torch.int32, dev),
        }
    if workspace is None:
        ws = binding.moe_permute_local_workspace_size(n, k, num_experts, num_local)
        workspace = poisoned((max(ws, 16),), torch.uint8, dev)
    emap = torch.as_tensor(np.asarray(expert_map, dtype=np.int32)).to(dev)
    binding.moe_permute_local(hidden, ids, num_experts, emap, num_local, outs["permuted_hidden_states"],
                              outs["expert_first_token_offset"], outs["permuted_idx"], outs["inv_permuted_idx"],
                              workspace, token_scale=token_scale, permuted_scale=outs["permuted_scale"],
                              stream=stream)
    return outs


def oracle_permute_local(hidden, ids, num_experts, expert_map, num_local, token_scale=None):
    h = to_np(hidden) if hidden is not None else np.zeros((ids.shape[0], 0), np.float32)
    return oracle.permute_local(h, to_np(ids), num_experts, np.asarray(expert_map, dtype=np.int32), num_local,
                                None if token_scale is None else to_np(token_scale))


def assert_permute_local_equal(outs, ref):
    """Offsets and inverse indices whole; the first M permuted entries equal the
    oracle's and the rest of each permuted buffer still holds the poison."""
    np.testing.assert_array_equal(to_np(outs["expert_first_token_offset"]), ref["expert_first_token_offset"])
    np.testing.assert_array_equal(to_np(outs["inv_permuted_idx"]), ref["inv_permuted_idx"])
    m = int(ref["expert_first_token_offset"][-1])
    perm = to_np(outs["permuted_idx"])
    np.testing.assert_array_equal(perm[:m], ref["permuted_idx"])
    assert np.all(perm[m:].view(np.uint32) == 0xFFFFFFFF), "permuted_idx written past the local rows"
    if outs["permuted_hidden_states"] is not None:
        got = to_np(outs["permuted_hidden_states"])
        gb = got.view(np.uint8).reshape(got.shape[0], -1)
        eb = ref["permuted_hidden_states"].view(np.uint8).reshape(m, gb.shape[1])
        if not np.array_equal(gb[:m], eb):
            bad = np.nonzero(np.any(gb[:m] != eb, axis=1))[0]
            raise AssertionError("local permuted rows differ at %d rows, first %s" % (bad.size, bad[:8].tolist()))
        assert np.all(gb[m:] == POISON), "permuted rows written past the local rows"
    if outs.get("permuted_scale") is not None:
        sc = to_np(outs["permuted_scale"]).view(np.uint32)
        np.testing.assert_array_equal(sc[:m], ref["permuted_scale"].view(np.uint32))
        assert np.all(sc[m:] == 0xFFFFFFFF), "permuted_scale written past the local rows"
