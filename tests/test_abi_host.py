"""The C ABI on a host without a GPU: the library loads, exports every entry
point the header declares, and rejects bad arguments before touching HIP.

No call here launches a kernel: every case fails a host-side check, which
returns before any HIP call.  Pointers are fake addresses that are never
dereferenced.
"""

import ctypes
import os
import re
import subprocess

import pytest

from mixture_experts_token_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_permute.h")

OK, INVALID, TOO_SMALL, MISALIGNED, UNSUPPORTED = 0, 1, 2, 3, 4
BF16, F32, FP8 = binding.MOE_DTYPE_BF16, binding.MOE_DTYPE_F32, binding.MOE_DTYPE_FP8_E4M3
I32, I64 = binding.MOE_DTYPE_INT32, binding.MOE_DTYPE_INT64


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def _no_gpu():
    import torch

    return not torch.cuda.is_available()


# Cases below pass fake addresses; each must fail a host check before any
# launch.  Where a GPU is visible they are skipped, so that a check that
# wrongly passes can never launch a kernel on fake pointers.
host_only = pytest.mark.skipif(not _no_gpu(), reason="fake-pointer checks run only on a host without a GPU")


def test_header_declares_the_boundary():
    assert declared_functions() == ["moe_grouped_gemm_bf16", "moe_permute", "moe_permute_local",
                                    "moe_permute_local_workspace_size", "moe_permute_quant_fp8",
                                    "moe_permute_static_scratch", "moe_permute_supported",
                                    "moe_permute_workspace_size", "moe_status_string", "moe_unpermute",
                                    "moe_unpermute_local"]


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (moe_[a-z0-9_]+)\b", out))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_header_compiles_as_c():
    src = '#include "moe_permute.h"\nint main(void) { return (int)moe_permute_workspace_size(1, 1, 1); }\n'
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I", os.path.dirname(HEADER),
                          "-x", "c", "-"], input=src, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_supported_is_safe_without_gpu(lib):
    import torch

    expected = None if torch.cuda.is_available() else 0
    for dev in (0, 1, -1, 1000):
        v = lib.moe_permute_supported(dev)
        assert v in (0, 1)
        if expected is not None:
            assert v == expected
    assert lib.moe_permute_supported(-1) == 0


def test_workspace_size_pure_and_monotone(lib):
    for k, e in [(1, 1), (2, 8), (8, 128), (8, 256), (16, 1024), (600, 1000)]:
        prev = 0
        for n in [0, 1, 7, 100, 2048, 2049, 4096, 16384, 100000, 1 << 20]:
            if n * k >= 2**31:
                continue
            s = lib.moe_permute_workspace_size(n, k, e)
            assert s == lib.moe_permute_workspace_size(n, k, e)
            assert s >= prev
            prev = s
    assert lib.moe_permute_workspace_size(-1, 2, 8) == 0
    assert lib.moe_permute_workspace_size(10, 0, 8) == 0
    assert lib.moe_permute_workspace_size(10, 9, 8) == 0  # topk > experts
    assert lib.moe_permute_workspace_size(10, 2, 1025) == 0
    assert lib.moe_permute_workspace_size(2**31 // 8, 8, 256) == 0  # N*topk reaches 2^31


def test_small_calls_need_no_workspace(lib):
    assert lib.moe_permute_workspace_size(2048, 8, 256) == 0
    assert lib.moe_permute_workspace_size(4096, 2, 8) == 0
    assert lib.moe_permute_workspace_size(16384, 8, 256) > 0


A = 0x10000  # fake, 256-aligned device addresses spaced far apart


def addr(i, extra=0):
    return ctypes.c_void_p(A * (1 << 20) * (i + 1) + extra)


def permute_call(lib, **kw):
    args = dict(hidden=addr(0), dtype=BF16, scale=None, ids=addr(1), ids_dtype=I32, n=4096, h=4096, k=2, e=8,
                out=addr(2), pscale=None, off=addr(3), perm=addr(4), inv=addr(5), ws=addr(6), ws_bytes=1 << 30,
                stream=None)
    args.update(kw)
    return lib.moe_permute(args["hidden"], args["dtype"], args["scale"], args["ids"], args["ids_dtype"], args["n"],
                           args["h"],
                           args["k"], args["e"], args["out"], args["pscale"], args["off"], args["perm"], args["inv"],
                           args["ws"], args["ws_bytes"], args["stream"])


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), INVALID),
    (dict(dtype=-1), INVALID),
    (dict(n=-1), INVALID),
    (dict(k=0), INVALID),
    (dict(k=9), INVALID),               # topk > num_experts
    (dict(e=0), INVALID),
    (dict(e=1025), INVALID),
    (dict(n=2**31 // 2), INVALID),      # N*topk reaches 2^31
    (dict(h=-4), INVALID),
    (dict(off=None), INVALID),
    (dict(ids=None), INVALID),
    (dict(perm=None), INVALID),
    (dict(inv=None), INVALID),
    (dict(hidden=None), INVALID),
    (dict(out=None), INVALID),
    (dict(scale=addr(7)), INVALID),     # scale without permuted_scale
    (dict(pscale=addr(7)), INVALID),    # permuted_scale without scale
    (dict(h=4095), MISALIGNED),         # 8190-byte rows
    (dict(dtype=FP8, h=4100), MISALIGNED),
    (dict(hidden=addr(0, 8)), MISALIGNED),
    (dict(out=addr(2, 4)), MISALIGNED),
    (dict(ids=addr(1, 2)), MISALIGNED),
    (dict(off=addr(3, 4)), MISALIGNED),
    (dict(perm=addr(4, 1)), MISALIGNED),
    (dict(out=addr(0)), INVALID),                          # output aliases the input rows
    (dict(perm=addr(5)), INVALID),                         # two outputs alias
    (dict(inv=addr(1)), INVALID),                          # output aliases topk_ids
    (dict(n=20000, k=8, e=256, ws_bytes=0), TOO_SMALL),    # staged schedule needs a workspace
    (dict(n=20000, k=8, e=256, ws=None), INVALID),
    (dict(n=20000, k=8, e=256, ws=addr(6, 8)), MISALIGNED),
    (dict(ids_dtype=BF16), INVALID),                       # ids must be int32 or int64
    (dict(ids_dtype=7), INVALID),
    (dict(ids_dtype=I64, ids=addr(1, 4)), MISALIGNED),     # int64 ids: 8-byte alignment
    (dict(dtype=I32), INVALID),                            # an id type is not a hidden type
    (dict(ids_dtype=I64, inv=addr(1, 1 << 15)), INVALID),  # output inside the (longer) int64 id buffer
])
def test_permute_rejects(lib, kw, status):
    assert permute_call(lib, **kw) == status


@host_only
def test_permute_workspace_boundary(lib):
    # rows of 2 KiB: 0.33 GB of expanded rows, below the split schedule's
    # threshold, so the call takes the copying plan the size is tight for
    need = lib.moe_permute_workspace_size(20000, 8, 256)
    assert permute_call(lib, n=20000, k=8, e=256, h=1024, ws_bytes=need - 1) == TOO_SMALL


def test_local_workspace_size_pure_and_monotone(lib):
    for k, e, nl in [(1, 1, 1), (2, 8, 4), (8, 128, 16), (8, 256, 32), (8, 256, 256), (16, 1024, 1024), (2, 8, 1024)]:
        prev = 0
        for n in [0, 1, 7, 100, 2048, 2049, 4096, 16384, 100000, 1 << 20]:
            s = lib.moe_permute_local_workspace_size(n, k, e, nl)
            assert s == lib.moe_permute_local_workspace_size(n, k, e, nl)
            assert s >= prev
            prev = s
    assert lib.moe_permute_local_workspace_size(10, 2, 8, 0) == 0
    assert lib.moe_permute_local_workspace_size(10, 2, 8, 1025) == 0
    assert lib.moe_permute_local_workspace_size(10, 9, 8, 4) == 0
    assert lib.moe_permute_local_workspace_size(16384, 8, 256, 32) > 0


def local_call(lib, **kw):
    args = dict(hidden=addr(0), dtype=BF16, scale=None, ids=addr(1), ids_dtype=I32, n=4096, h=4096, k=2, e=8,
                emap=addr(8), nl=4, out=addr(2), pscale=None, off=addr(3), perm=addr(4), inv=addr(5), ws=addr(6),
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return lib.moe_permute_local(args["hidden"], args["dtype"], args["scale"], args["ids"], args["ids_dtype"],
                                 args["n"], args["h"],
                                 args["k"], args["e"], args["emap"], args["nl"], args["out"], args["pscale"],
                                 args["off"], args["perm"], args["inv"], args["ws"], args["ws_bytes"], args["stream"])


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(emap=None), INVALID),
    (dict(nl=0), INVALID),
    (dict(nl=1025), INVALID),
    (dict(emap=addr(8, 2)), MISALIGNED),
    (dict(off=addr(8)), INVALID),                           # offsets alias the map
    (dict(k=9), INVALID),
    (dict(dtype=5), INVALID),
    (dict(n=20000, k=8, e=256, nl=32, ws_bytes=0), TOO_SMALL),
    (dict(ids_dtype=FP8), INVALID),
    (dict(ids_dtype=I64, ids=addr(1, 4)), MISALIGNED),
])
def test_permute_local_rejects(lib, kw, status):
    assert local_call(lib, **kw) == status


@host_only
def test_permute_local_workspace_boundary(lib):
    need = lib.moe_permute_local_workspace_size(20000, 8, 256, 32)
    assert need > 0
    assert local_call(lib, n=20000, k=8, e=256, nl=32, ws_bytes=need - 1) == TOO_SMALL


def quant_call(lib, **kw):
    args = dict(hidden=addr(0), dtype=BF16, ids=addr(1), ids_dtype=I32, n=4096, h=4096, k=2, e=8, emap=None, nl=0,
                group=0, codes=addr(2), scales=addr(9), off=addr(3), perm=addr(4), inv=addr(5), ws=addr(6),
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return lib.moe_permute_quant_fp8(args["hidden"], args["dtype"], args["ids"], args["ids_dtype"], args["n"],
                                     args["h"], args["k"], args["e"], args["emap"], args["nl"], args["group"],
                                     args["codes"], args["scales"], args["off"], args["perm"], args["inv"], args["ws"],
                                     args["ws_bytes"], args["stream"])


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(dtype=FP8), UNSUPPORTED),      # input must be bf16 or f32
    (dict(dtype=9), UNSUPPORTED),
    (dict(h=8200), INVALID),             # bf16 rows above 16 KiB
    (dict(dtype=F32, h=4100), INVALID),  # f32 rows above 16 KiB
    (dict(h=4092), MISALIGNED),          # not whole 16-byte vectors
    (dict(group=100), INVALID),          # not a power of two
    (dict(group=4), INVALID),            # below one vector of bf16
    (dict(group=1024), INVALID),         # above 64 vectors
    (dict(group=8192), INVALID),         # does not divide h
    (dict(nl=4), INVALID),               # local count without a map
    (dict(codes=None), INVALID),
    (dict(scales=None), INVALID),
    (dict(codes=addr(2, 8)), MISALIGNED),
    (dict(scales=addr(9, 2)), MISALIGNED),
    (dict(codes=addr(0)), INVALID),      # codes alias the input
    (dict(scales=addr(5)), INVALID),     # scales alias inv_permuted_idx
    (dict(ids_dtype=BF16), INVALID),
    (dict(k=9), INVALID),
    (dict(n=20000, k=8, e=256, ws_bytes=0), TOO_SMALL),
])
def test_permute_quant_rejects(lib, kw, status):
    assert quant_call(lib, **kw) == status


def gemm_call(lib, **kw):
    args = dict(x=addr(0), w=addr(1), off=addr(2), e=8, rows=8192, n=1024, k=4096, y=addr(3), stream=None)
    args.update(kw)
    return lib.moe_grouped_gemm_bf16(args["x"], args["w"], args["off"], args["e"], args["rows"], args["n"],
                                     args["k"], args["y"], args["stream"])


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(e=0), INVALID),
    (dict(e=1025), INVALID),
    (dict(rows=-1), INVALID),
    (dict(n=100), INVALID),           # n must be a multiple of 128
    (dict(n=0), INVALID),
    (dict(k=96), INVALID),            # k must be a multiple of 64
    (dict(k=(1 << 20) + 64), INVALID),  # and at most 2^20
    (dict(off=None), INVALID),
    (dict(w=None), INVALID),
    (dict(x=None), INVALID),
    (dict(y=None), INVALID),
    (dict(x=addr(0, 8)), MISALIGNED),
    (dict(y=addr(3, 2)), MISALIGNED),
    (dict(off=addr(2, 4)), MISALIGNED),
    (dict(y=addr(0)), INVALID),       # output aliases the rows
    (dict(y=addr(2)), INVALID),       # output aliases the offsets
])
def test_grouped_gemm_rejects(lib, kw, status):
    assert gemm_call(lib, **kw) == status


def test_grouped_gemm_zero_rows_is_a_no_op(lib):
    assert gemm_call(lib, rows=0, x=None, y=None) == OK


def unpermute_call(lib, fn="moe_unpermute", **kw):
    args = dict(y=addr(0), dtype=BF16, w=addr(1), inv=addr(2), n=4096, h=4096, k=2, out=addr(3), stream=None)
    args.update(kw)
    return getattr(lib, fn)(args["y"], args["dtype"], args["w"], args["inv"], args["n"], args["h"], args["k"],
                            args["out"], args["stream"])


UNPERMUTE_FNS = ["moe_unpermute", "moe_unpermute_local"]


@host_only
@pytest.mark.parametrize("kw,status", [
    (dict(dtype=FP8), UNSUPPORTED),
    (dict(dtype=9), INVALID),
    (dict(n=-1), INVALID),
    (dict(k=0), INVALID),
    (dict(k=1025), INVALID),
    (dict(h=0), INVALID),
    (dict(y=None), INVALID),
    (dict(w=None), INVALID),
    (dict(inv=None), INVALID),
    (dict(out=None), INVALID),
    (dict(h=4), MISALIGNED),            # 8-byte bf16 rows
    (dict(y=addr(0, 4)), MISALIGNED),
    (dict(out=addr(3, 8)), MISALIGNED),
    (dict(w=addr(1, 2)), MISALIGNED),
    (dict(out=addr(0)), INVALID),       # output aliases the input
])
@pytest.mark.parametrize("fn", UNPERMUTE_FNS)
def test_unpermute_rejects(lib, fn, kw, status):
    assert unpermute_call(lib, fn, **kw) == status


@pytest.mark.parametrize("fn", UNPERMUTE_FNS)
def test_unpermute_zero_tokens_is_a_no_op(lib, fn):
    assert unpermute_call(lib, fn, n=0, y=None, w=None, inv=None, out=None) == OK


def test_status_strings(lib):
    for code, name in [(0, b"MOE_OK"), (1, b"MOE_ERR_INVALID_ARG"), (2, b"MOE_ERR_WORKSPACE_TOO_SMALL"),
                       (3, b"MOE_ERR_MISALIGNED"), (4, b"MOE_ERR_UNSUPPORTED"), (5, b"MOE_ERR_HIP")]:
        assert lib.moe_status_string(code) == name


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(FileNotFoundError):
        binding.load_library()


def test_streaming_probe_library_checks_arguments():
    """The bench's ceiling probe (libhbm_probe.so) loads and rejects bad sizes before any launch."""
    import os

    path = os.path.join(os.path.dirname(os.path.abspath(binding.__file__)), "libhbm_probe.so")
    probe = ctypes.CDLL(path)
    for fn in (probe.hbm_probe_fanout, probe.hbm_probe_reduce):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                       ctypes.c_void_p]
        fn.restype = ctypes.c_int
        assert fn(None, addr(1), 10, 64, 2, 1, None) == 1
        assert fn(addr(0), addr(1), 0, 64, 2, 1, None) == 1
        assert fn(addr(0), addr(1), 10, 24, 2, 1, None) == 1
        assert fn(addr(0), addr(1), 10, 64, 0, 1, None) == 1
        assert fn(addr(0), addr(1), 10, 64, 2, 8, None) == 1  # variant out of range


@host_only
def test_static_scratch_rejects_calls_beyond_its_array(lib):
    """moe_permute_static_scratch: a call whose workspace would exceed the
    static array is refused on the host; other checks are moe_permute's."""
    fake = ctypes.c_void_p(1 << 20)
    n, k, e = 600000, 2, 16
    assert lib.moe_permute_workspace_size(n, k, e) > binding.MOE_STATIC_SCRATCH_BYTES
    st = lib.moe_permute_static_scratch(None, BF16, None, fake, I32, n, 0, k, e, None, None, fake,
                                        ctypes.c_void_p((1 << 20) + (1 << 24)), ctypes.c_void_p((1 << 20) + (2 << 24)),
                                        None)
    assert st == TOO_SMALL
    # moe_permute's own checks still apply (here: topk > num_experts)
    assert lib.moe_permute_static_scratch(None, BF16, None, fake, I32, 8, 0, 9, 8, None, None, fake, fake, fake,
                                          None) == INVALID
