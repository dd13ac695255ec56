"""moe_permute_static_scratch, the permute that allocates nothing, against moe_permute.

The static entry point takes no workspace: the library's static per-GPU array
stands in for it.  Through the C ABI it must produce exactly what moe_permute
produces with a caller workspace (offsets, both index arrays, permuted rows and
scales, bit for bit) on consecutive calls that share the array -- the staged
schedule (the largest workspace), then smaller coarse and fused calls after it
-- and reject a call that needs more than the array holds before writing
anything.  Every output is poisoned (0xFF) before each call.
"""

import numpy as np
import pytest
import torch

from _parity import POISON, gpu_permute, poisoned, to_np
from mixture_experts_token_amd import binding

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[case] " + msg, flush=True)


def _static_permute(hidden, ids, e, token_scale=None):
    dev = ids.device
    n, k = ids.shape
    rows = n * k
    outs = {
        "permuted_hidden_states": None if hidden is None else poisoned((rows, hidden.shape[1]), hidden.dtype, dev),
        "permuted_scale": None if token_scale is None else poisoned((rows,), torch.float32, dev),
        "expert_first_token_offset": poisoned((e + 1,), torch.int64, dev),
        "permuted_idx": poisoned((rows,), torch.int32, dev),
        "inv_permuted_idx": poisoned((rows,), torch.int32, dev),
    }
    binding.moe_permute_static_scratch(hidden, ids, e, outs["permuted_hidden_states"],
                                       outs["expert_first_token_offset"], outs["permuted_idx"],
                                       outs["inv_permuted_idx"], token_scale=token_scale,
                                       permuted_scale=outs["permuted_scale"])
    return outs


def _case(dev, n, k, e, h, dtype, seed, with_scale=False):
    g = torch.Generator(device="cpu").manual_seed(seed)
    rng = np.random.default_rng(seed)
    ids = torch.from_numpy(rng.integers(0, e, size=(n, k)).astype(np.int32)).to(dev)
    hidden = None
    if h:
        if dtype == torch.uint8:
            hidden = torch.randint(0, 256, (n, h), generator=g, dtype=torch.uint8).to(dev)
        else:
            hidden = torch.randn((n, h), generator=g).to(dtype).to(dev)
    scale = torch.rand((n,), generator=g).to(dev) if with_scale else None
    return hidden, ids, scale


def _assert_same(got, want):
    for key, t in want.items():
        if t is None:
            assert got[key] is None
            continue
        a, b = to_np(got[key]), to_np(t)
        assert a.shape == b.shape, key
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), "%s differs from moe_permute" % key


# (N, topk, E, hidden, dtype, per-token scale): staged first (its workspace is
# the largest), then smaller coarse and fused calls reusing the same array
SEQUENCE = [
    (140000, 2, 16, 64, torch.bfloat16, False),   # staged: 280000 rows, about 1.3 MB of workspace
    (3000, 8, 256, 512, torch.bfloat16, False),   # coarse: one histogram row per coarse tile
    (700, 8, 256, 1024, torch.uint8, True),       # coarse, fp8 codes with their scales
    (100, 2, 8, 128, torch.float32, False),       # fused: no workspace at all
    (140000, 2, 16, 64, torch.bfloat16, False),   # staged again after the smaller calls
]


def test_static_scratch_matches_moe_permute_on_consecutive_calls(hip_device):
    for i, (n, k, e, h, dtype, with_scale) in enumerate(SEQUENCE):
        _say("static scratch call %d: N=%d topk=%d E=%d H=%d %s" % (i, n, k, e, h, dtype))
        hidden, ids, scale = _case(hip_device, n, k, e, h, dtype, seed=i, with_scale=with_scale)
        want = gpu_permute(hidden, ids, e, token_scale=scale)
        got = _static_permute(hidden, ids, e, token_scale=scale)
        torch.cuda.synchronize()
        _assert_same(got, want)


def test_static_scratch_index_only_then_smaller(hip_device):
    for i, (n, k, e) in enumerate([(70000, 4, 64), (5000, 8, 128)]):
        _say("static scratch index-only call %d: N=%d topk=%d E=%d" % (i, n, k, e))
        _, ids, _ = _case(hip_device, n, k, e, 0, None, seed=10 + i)
        want = gpu_permute(None, ids, e)
        got = _static_permute(None, ids, e)
        torch.cuda.synchronize()
        _assert_same(got, want)


def test_static_scratch_rejects_a_call_beyond_its_size(hip_device):
    n, k, e = 600000, 2, 16  # staged: 1.2 M rows need about 4.8 MB of workspace
    _say("static scratch over-size call N=%d topk=%d" % (n, k))
    assert binding.moe_permute_workspace_size(n, k, e) > binding.MOE_STATIC_SCRATCH_BYTES
    _, ids, _ = _case(hip_device, n, k, e, 0, None, seed=20)
    off = poisoned((e + 1,), torch.int64, hip_device)
    perm = poisoned((n * k,), torch.int32, hip_device)
    inv = poisoned((n * k,), torch.int32, hip_device)
    with pytest.raises(binding.MoEError) as err:
        binding.moe_permute_static_scratch(None, ids, e, None, off, perm, inv)
    assert err.value.status == binding.MOE_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    for t in (off, perm, inv):
        assert bool((t.view(torch.uint8) == POISON).all())
