"""CPU oracle for the MoE token permute / unpermute path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  The product path
(the HIP library and its Python binding) never imports, links or runs it, and
the two share no code.

The arithmetic lives in ``moe_oracle.c`` (plain C, scalar loops, built with
``-O2 -ffp-contract=off``); this module only marshals numpy arrays into it.
bfloat16 arrays travel as their ``uint16`` bit patterns because numpy has no
bfloat16 type.

Definitions followed (see the comments in ``moe_oracle.c`` for the passage
behind each step):

* vLLM PR #14568, "permute/unpermute kernel for moe optimization", PR
  description -- what permute and unpermute compute.
* prhub summary of vLLM PR #43014, section "key code snippets"
  (MoEPermuteScratch) -- names, dtypes and lengths of every buffer, and the
  numbering of expanded rows as an arange viewed ``[n_token, topk]``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
# A test that plants mistakes in a copy of the oracle points this at the copy.
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB")

OK = 0
BAD_ID = -1
BAD_ARG = -2
BAD_INV = -3


class OracleError(RuntimeError):
    pass


def build(force: bool = False) -> str:
    """Compile ``moe_oracle.c`` with gcc into ``libmoe_oracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int32
        lib.oracle_expert_counts.argtypes = [p, i64, i32, i32, p]
        lib.oracle_expert_counts.restype = ctypes.c_int
        lib.oracle_expert_first_token_offset.argtypes = [p, i32, p]
        lib.oracle_expert_first_token_offset.restype = None
        lib.oracle_stable_expert_order.argtypes = [p, i64, i32, p, p, p]
        lib.oracle_stable_expert_order.restype = ctypes.c_int
        lib.oracle_gather_rows.argtypes = [p, i64, p, p, i64, i32, p, p]
        lib.oracle_gather_rows.restype = None
        lib.oracle_moe_permute.argtypes = [p, i64, p, p, i64, i32, i32, p, p, p, p, p]
        lib.oracle_moe_permute.restype = ctypes.c_int
        lib.oracle_moe_permute_local.argtypes = [p, i64, p, p, i64, i32, i32, p, i32, p, p, p, p, p]
        lib.oracle_moe_permute_local.restype = ctypes.c_int
        lib.oracle_ids_from_int64.argtypes = [p, i64, i32, p]
        lib.oracle_ids_from_int64.restype = ctypes.c_int
        lib.oracle_unpermute_f32.argtypes = [p, p, p, i64, i32, i64, p]
        lib.oracle_unpermute_f32.restype = ctypes.c_int
        lib.oracle_unpermute_bf16.argtypes = [p, p, p, i64, i32, i64, p]
        lib.oracle_unpermute_bf16.restype = ctypes.c_int
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_double_to_bf16.restype = ctypes.c_uint16
        lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_to_double.restype = ctypes.c_double
        lib.oracle_double_to_e4m3.argtypes = [ctypes.c_double]
        lib.oracle_double_to_e4m3.restype = ctypes.c_uint8
        lib.oracle_quantize_fp8_rows.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p]
        lib.oracle_quantize_fp8_rows.restype = ctypes.c_int
        lib.oracle_grouped_gemm_bf16.argtypes = [p, p, p, i32, i64, i64, p]
        lib.oracle_grouped_gemm_bf16.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(status: int):
    if status != OK:
        raise OracleError({BAD_ID: "expert id out of range", BAD_ARG: "bad argument",
                           BAD_INV: "inv_permuted_idx out of range"}.get(status, str(status)))


def _ids2d(topk_ids, num_experts: int | None = None) -> np.ndarray:
    """int32 [N, topk] ids.  int64 ids go through oracle_ids_from_int64, which
    rejects every value outside [0, num_experts) instead of truncating it."""
    arr = np.asarray(topk_ids)
    if arr.dtype == np.int64:
        if num_experts is None:
            raise ValueError("int64 ids need num_experts to be checked")
        src = np.ascontiguousarray(arr)
        ids = np.zeros(src.shape, dtype=np.int32)
        _check(_load().oracle_ids_from_int64(_ptr(src), src.size, num_experts, _ptr(ids)))
    else:
        ids = np.ascontiguousarray(arr, dtype=np.int32)
    if ids.ndim != 2:
        raise ValueError("topk_ids must be [num_tokens, topk]")
    return ids


# --------------------------------------------------------------------------
# Permute, step by step
# --------------------------------------------------------------------------
def expert_counts(topk_ids, num_experts: int) -> np.ndarray:
    """Step 1: expanded rows routed to each expert (int64 [E])."""
    ids = _ids2d(topk_ids, num_experts)
    counts = np.zeros(num_experts, dtype=np.int64)
    _check(_load().oracle_expert_counts(_ptr(ids), ids.shape[0], ids.shape[1], num_experts, _ptr(counts)))
    return counts


def expert_first_token_offset(counts) -> np.ndarray:
    """Step 2: exclusive prefix sum of the counts (int64 [E+1])."""
    counts = np.ascontiguousarray(counts, dtype=np.int64)
    off = np.zeros(counts.shape[0] + 1, dtype=np.int64)
    _load().oracle_expert_first_token_offset(_ptr(counts), counts.shape[0], _ptr(off))
    return off


def stable_expert_order(topk_ids, num_experts: int, offsets) -> tuple[np.ndarray, np.ndarray]:
    """Step 3: (permuted_idx, inv_permuted_idx), both int32 [N*topk]."""
    ids = _ids2d(topk_ids, num_experts)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    rows = ids.size
    perm = np.zeros(rows, dtype=np.int32)
    inv = np.zeros(rows, dtype=np.int32)
    _check(_load().oracle_stable_expert_order(_ptr(ids), rows, num_experts, _ptr(offsets),
                                              _ptr(perm), _ptr(inv)))
    return perm, inv


def gather_rows(hidden_bytes: np.ndarray, permuted_idx, topk: int, token_scale=None):
    """Step 4: permuted rows (raw bytes) and, if given, permuted per-token scales."""
    hb = np.ascontiguousarray(hidden_bytes, dtype=np.uint8)
    perm = np.ascontiguousarray(permuted_idx, dtype=np.int32)
    rows = perm.shape[0]
    out = np.zeros((rows, hb.shape[1]), dtype=np.uint8)
    scale = None if token_scale is None else np.ascontiguousarray(token_scale, dtype=np.float32)
    out_scale = None if scale is None else np.zeros(rows, dtype=np.float32)
    _load().oracle_gather_rows(_ptr(hb), hb.shape[1], _ptr(scale), _ptr(perm), rows, topk,
                               _ptr(out), _ptr(out_scale))
    return out, out_scale


def as_row_bytes(hidden: np.ndarray) -> np.ndarray:
    """View a C-contiguous [N, H] array of any element type as [N, H*itemsize] bytes."""
    h = np.ascontiguousarray(hidden)
    return h.view(np.uint8).reshape(h.shape[0], -1)


def permute(hidden: np.ndarray, topk_ids, num_experts: int, token_scale=None) -> dict:
    """The whole permute (steps 1-4).

    ``hidden`` is [N, H] of any element type (float32, bf16 bits as uint16, or
    fp8 codes as uint8); the permuted rows come back with the same element
    type.  Returns a dict with ``expert_first_token_offset``, ``permuted_idx``,
    ``inv_permuted_idx``, ``permuted_hidden_states`` and ``permuted_scale``.
    ``topk_ids`` may be int32 or int64 (checked, never truncated).
    """
    ids = _ids2d(topk_ids, num_experts)
    n, topk = ids.shape
    h = np.ascontiguousarray(hidden)
    if h.shape[0] != n:
        raise ValueError("hidden and topk_ids disagree on num_tokens")
    hb = as_row_bytes(h) if h.size else np.zeros((n, 0), dtype=np.uint8)
    rows = n * topk
    off = np.zeros(num_experts + 1, dtype=np.int64)
    perm = np.zeros(rows, dtype=np.int32)
    inv = np.zeros(rows, dtype=np.int32)
    out = np.zeros((rows, hb.shape[1]), dtype=np.uint8)
    scale = None if token_scale is None else np.ascontiguousarray(token_scale, dtype=np.float32)
    out_scale = None if scale is None else np.zeros(rows, dtype=np.float32)
    _check(_load().oracle_moe_permute(_ptr(hb), hb.shape[1], _ptr(scale), _ptr(ids), n, topk,
                                      num_experts, _ptr(out), _ptr(out_scale), _ptr(off),
                                      _ptr(perm), _ptr(inv)))
    return {
        "expert_first_token_offset": off,
        "permuted_idx": perm,
        "inv_permuted_idx": inv,
        "permuted_hidden_states": out.view(h.dtype).reshape((rows,) + h.shape[1:]) if h.ndim == 2 else out,
        "permuted_scale": out_scale,
    }


def permute_local(hidden: np.ndarray, topk_ids, num_experts: int, expert_map, num_local_experts: int,
                  token_scale=None) -> dict:
    """Permute with a local-expert filter: expert_map[g] = local id of global expert g, or -1.

    Returns the same keys as ``permute``; ``expert_first_token_offset`` has
    num_local_experts + 1 entries, ``permuted_idx`` / ``permuted_hidden_states``
    / ``permuted_scale`` hold only the local rows, and ``inv_permuted_idx`` is
    -1 for rows of experts on other ranks.  ``topk_ids`` may be int32 or int64.
    """
    ids = _ids2d(topk_ids, num_experts)
    n, topk = ids.shape
    emap = np.ascontiguousarray(expert_map, dtype=np.int32)
    if emap.shape != (num_experts,):
        raise ValueError("expert_map must have num_experts entries")
    h = np.ascontiguousarray(hidden)
    hb = as_row_bytes(h) if h.size else np.zeros((n, 0), dtype=np.uint8)
    rows = n * topk
    off = np.zeros(num_local_experts + 1, dtype=np.int64)
    perm = np.zeros(rows, dtype=np.int32)
    inv = np.zeros(rows, dtype=np.int32)
    out = np.zeros((rows, hb.shape[1]), dtype=np.uint8)
    scale = None if token_scale is None else np.ascontiguousarray(token_scale, dtype=np.float32)
    out_scale = None if scale is None else np.zeros(rows, dtype=np.float32)
    _check(_load().oracle_moe_permute_local(_ptr(hb), hb.shape[1], _ptr(scale), _ptr(ids), n, topk, num_experts,
                                            _ptr(emap), num_local_experts, _ptr(out), _ptr(out_scale), _ptr(off),
                                            _ptr(perm), _ptr(inv)))
    local_rows = int(off[-1])
    return {
        "expert_first_token_offset": off,
        "permuted_idx": perm[:local_rows],
        "inv_permuted_idx": inv,
        "permuted_hidden_states": (out[:local_rows].view(h.dtype).reshape((local_rows,) + h.shape[1:])
                                   if h.ndim == 2 else out[:local_rows]),
        "permuted_scale": None if out_scale is None else out_scale[:local_rows],
    }


# --------------------------------------------------------------------------
# Unpermute
# --------------------------------------------------------------------------
def unpermute(expanded_output: np.ndarray, topk_weights, inv_permuted_idx, dtype: str) -> np.ndarray:
    """out[t] = sum_k w[t,k] * Y[inv[t*topk+k]], double-precision sum rounded once.

    Slots whose index is -1 (experts on another rank) contribute nothing.

    ``dtype`` is ``"f32"`` (Y float32) or ``"bf16"`` (Y as uint16 bit patterns);
    the output has the same representation as Y.
    """
    w = np.ascontiguousarray(topk_weights, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("topk_weights must be [num_tokens, topk]")
    n, topk = w.shape
    inv = np.ascontiguousarray(inv_permuted_idx, dtype=np.int32).reshape(-1)
    lib = _load()
    if dtype == "f32":
        y = np.ascontiguousarray(expanded_output, dtype=np.float32)
        out = np.zeros((n, y.shape[1]), dtype=np.float32)
        _check(lib.oracle_unpermute_f32(_ptr(y), _ptr(w), _ptr(inv), n, topk, y.shape[1], _ptr(out)))
    elif dtype == "bf16":
        y = np.ascontiguousarray(expanded_output, dtype=np.uint16)
        out = np.zeros((n, y.shape[1]), dtype=np.uint16)
        _check(lib.oracle_unpermute_bf16(_ptr(y), _ptr(w), _ptr(inv), n, topk, y.shape[1], _ptr(out)))
    else:
        raise ValueError("unpermute dtype must be 'f32' or 'bf16'")
    return out


def bf16_to_double(bits: int) -> float:
    return float(_load().oracle_bf16_to_double(int(bits) & 0xFFFF))


def double_to_bf16(x: float) -> int:
    return int(_load().oracle_double_to_bf16(float(x)))


def e4m3_to_double(code: int) -> float:
    return float(_load().oracle_e4m3_to_double(int(code) & 0xFF))


def double_to_e4m3(x: float) -> int:
    return int(_load().oracle_double_to_e4m3(float(x)))


def quantize_fp8_rows(x: np.ndarray, dtype: str, group: int | None = None):
    """(codes uint8 [rows, h], scales float32 [rows, h / group]) of the dynamic
    fp8 quantiser; ``x`` is float32 ("f32") or bf16 bit patterns ("bf16");
    group None means one scale per row."""
    src = np.ascontiguousarray(x, dtype=np.float32 if dtype == "f32" else np.uint16)
    rows, h = src.shape
    g = h if group is None else int(group)
    codes = np.zeros((rows, h), dtype=np.uint8)
    scales = np.zeros((rows, h // g if g else 0), dtype=np.float32)
    _check(_load().oracle_quantize_fp8_rows(_ptr(src), 1 if dtype == "bf16" else 0, rows, h, g, _ptr(codes),
                                            _ptr(scales)))
    return codes, scales


def grouped_gemm_bf16(x: np.ndarray, w: np.ndarray, offsets) -> np.ndarray:
    """y[j] = x[j] @ w[e]^T for the rows j of expert e ([off[e], off[e+1])), double
    accumulation rounded once to bf16.  x: bf16 bits [rows, k]; w: bf16 bits
    [E, n, k]; returns bf16 bits [off[E], n]."""
    xs = np.ascontiguousarray(x, dtype=np.uint16)
    ws = np.ascontiguousarray(w, dtype=np.uint16)
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    e, n, k = ws.shape
    if off.shape != (e + 1,) or xs.ndim != 2 or xs.shape[1] != k or xs.shape[0] < off[-1]:
        raise ValueError("shapes of x, w and offsets disagree")
    y = np.zeros((int(off[-1]), n), dtype=np.uint16)
    _check(_load().oracle_grouped_gemm_bf16(_ptr(xs), _ptr(ws), _ptr(off), e, n, k, _ptr(y)))
    return y


def permute_quant_fp8(hidden: np.ndarray, dtype: str, topk_ids, num_experts: int, group: int | None = None,
                      expert_map=None, num_local_experts: int | None = None) -> dict:
    """Quantise every token row to fp8 (see quantize_fp8_rows), then permute the
    codes and move each row's scales with it: the plain permute, or the
    local-expert permute when ``expert_map`` is given.  ``permuted_scale`` is
    [rows out, h / group].  Quantisation acts on each row alone, so quantising
    before or after the permute gives the same rows."""
    codes, scales = quantize_fp8_rows(hidden, dtype, group)
    if expert_map is None:
        res = permute(codes, topk_ids, num_experts)
    else:
        res = permute_local(codes, topk_ids, num_experts, expert_map, num_local_experts)
    topk = np.asarray(topk_ids).shape[1]
    sb, _ = gather_rows(as_row_bytes(scales), res["permuted_idx"], topk)
    res["permuted_scale"] = sb.view(np.float32).reshape(res["permuted_idx"].shape[0], scales.shape[1])
    return res
