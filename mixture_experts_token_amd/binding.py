"""Python binding of libmoe_permute.so (argument marshalling only).

Every step of the path runs in the HIP library; this module turns torch
tensors into raw device pointers and sizes, passes the caller's current HIP
stream, and raises on a non-OK status.  There is no fallback: if the library
is missing the first call raises.

The entry points carry the C names: ``moe_permute_supported``,
``moe_permute_workspace_size``, ``moe_permute``, ``moe_unpermute``, ``moe_unpermute_local``,
``moe_permute_local_workspace_size``, ``moe_permute_local``,
``moe_permute_quant_fp8``, ``moe_grouped_gemm_bf16``, ``moe_permute_static_scratch``.
``MoEPermuteScratch`` follows the preallocated-buffer design of the prhub
summary of vLLM PR #43014 (section "key code snippets", MoEPermuteScratch):
every buffer is allocated once for ``max_num_tokens`` and reused by each call.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_permute.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_WORKSPACE_TOO_SMALL = 2
MOE_ERR_MISALIGNED = 3
MOE_ERR_UNSUPPORTED = 4
MOE_ERR_HIP = 5

MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_DTYPE_FP8_E4M3 = 2
MOE_DTYPE_INT32 = 3
MOE_DTYPE_INT64 = 4
MOE_MAX_EXPERTS = 1024


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s" % (what, _status_name(status)))


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libmoe_permute.so; raises FileNotFoundError if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                "libmoe_permute.so is not built (%s); run "
                "`python -m mixture_experts_token_amd.build_lib`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.moe_permute_supported.argtypes = [ctypes.c_int]
        lib.moe_permute_supported.restype = ctypes.c_int
        lib.moe_permute_workspace_size.argtypes = [i64, i32, i32]
        lib.moe_permute_workspace_size.restype = sz
        lib.moe_permute.argtypes = [p, i32, p, p, i32, i64, i64, i32, i32, p, p, p, p, p, p, sz, p]
        lib.moe_permute.restype = ctypes.c_int
        lib.moe_permute_static_scratch.argtypes = [p, i32, p, p, i32, i64, i64, i32, i32, p, p, p, p, p, p]
        lib.moe_permute_static_scratch.restype = ctypes.c_int
        lib.moe_permute_local_workspace_size.argtypes = [i64, i32, i32, i32]
        lib.moe_permute_local_workspace_size.restype = sz
        lib.moe_permute_local.argtypes = [p, i32, p, p, i32, i64, i64, i32, i32, p, i32, p, p, p, p, p, p, sz, p]
        lib.moe_permute_local.restype = ctypes.c_int
        lib.moe_permute_quant_fp8.argtypes = [p, i32, p, i32, i64, i64, i32, i32, p, i32, i64, p, p, p, p, p, p,
                                              sz, p]
        lib.moe_permute_quant_fp8.restype = ctypes.c_int
        lib.moe_grouped_gemm_bf16.argtypes = [p, p, p, i32, i64, i64, i64, p, p]
        lib.moe_grouped_gemm_bf16.restype = ctypes.c_int
        for fn in (lib.moe_unpermute, lib.moe_unpermute_local):
            fn.argtypes = [p, i32, p, p, i64, i64, i32, p, p]
            fn.restype = ctypes.c_int
        lib.moe_status_string.argtypes = [ctypes.c_int]
        lib.moe_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _status_name(status: int) -> str:
    try:
        return load_library().moe_status_string(status).decode()
    except Exception:
        return str(status)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return MOE_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return MOE_DTYPE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MOE_DTYPE_FP8_E4M3
    raise TypeError("unsupported element type %s" % t.dtype)


def _check(t, name: str, dtypes, numel: int, device, optional: bool = False) -> None:
    """Reject a buffer the kernels would read or write out of bounds.

    ``dtypes``: allowed torch dtypes; ``numel``: the element count the C entry
    point derives from its sizes; ``device``: the device every buffer of the
    call must be on (a GPU device).  Raises TypeError (type, device) or
    ValueError (size, layout) before anything reaches the library.
    """
    if t is None:
        if optional:
            return
        raise ValueError("%s is required" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s must be %s, got %s" % (name, " or ".join(str(d) for d in dtypes), t.dtype))
    if t.numel() != numel:
        raise ValueError("%s must have %d elements, got %d (shape %s)" % (name, numel, t.numel(), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise TypeError("%s is on %s, expected %s (every buffer of the call on one GPU)" % (name, t.device, device))


def _require_gpu(device) -> None:
    """The last check of a call: its buffers (all on `device`) must be GPU memory."""
    if device.type != "cuda":
        raise TypeError("the MoE library takes GPU tensors; got tensors on %s" % device)


def _ptr(t):
    """Raw device address of a contiguous tensor (None stays None)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _stream(stream, t):
    """hipStream_t handle: the given torch stream, else torch's current stream on t's device."""
    if stream is not None:
        return stream.cuda_stream
    import torch

    return torch._C._cuda_getCurrentRawStream(t.get_device())


def moe_permute_supported(device: int = 0) -> bool:
    return bool(load_library().moe_permute_supported(int(device)))


def moe_permute_workspace_size(max_num_tokens: int, topk: int, num_experts: int) -> int:
    return int(load_library().moe_permute_workspace_size(int(max_num_tokens), int(topk), int(num_experts)))


def moe_permute_local_workspace_size(max_num_tokens: int, topk: int, num_experts: int,
                                     num_local_experts: int) -> int:
    return int(load_library().moe_permute_local_workspace_size(int(max_num_tokens), int(topk), int(num_experts),
                                                               int(num_local_experts)))


_ROW_TYPES = None


def _row_types():
    """Element types of hidden rows: float32, bfloat16, fp8 E4M3 codes (uint8 or float8_e4m3fn)."""
    global _ROW_TYPES
    if _ROW_TYPES is None:
        import torch

        _ROW_TYPES = (torch.float32, torch.bfloat16, torch.uint8, torch.float8_e4m3fn)
    return _ROW_TYPES


def _same_row_type(a, b) -> bool:
    import torch

    fp8 = (torch.uint8, torch.float8_e4m3fn)
    return a.dtype == b.dtype or (a.dtype in fp8 and b.dtype in fp8)


def _permute_args(hidden_states, topk_ids, workspace, offsets, permuted_idx, inv_permuted_idx, num_offsets: int,
                  permuted_hidden_states=None, token_scale=None, permuted_scale=None, check_rows: bool = True):
    """Checks shared by the permute entry points; returns (hidden, dtype code, H, workspace bytes, id code)."""
    import torch

    if topk_ids is None or topk_ids.dtype not in (torch.int32, torch.int64) or topk_ids.dim() != 2:
        raise TypeError("topk_ids must be an int32 or int64 [num_tokens, topk] tensor")
    dev = topk_ids.device
    n, topk = topk_ids.shape
    rows = n * topk
    _check(topk_ids, "topk_ids", (torch.int32, torch.int64), rows, dev)
    ids_code = MOE_DTYPE_INT64 if topk_ids.dtype == torch.int64 else MOE_DTYPE_INT32
    if hidden_states is None:
        hidden, code, hsize = None, MOE_DTYPE_BF16, 0
    else:
        if hidden_states.dim() != 2 or hidden_states.shape[0] != n:
            raise ValueError("hidden_states must be [num_tokens=%d, hidden_size], got shape %s"
                             % (n, tuple(hidden_states.shape)))
        hidden, code, hsize = hidden_states, _dtype_code(hidden_states), hidden_states.shape[-1]
        _check(hidden_states, "hidden_states", _row_types(), n * hsize, dev)
        if check_rows:
            _check(permuted_hidden_states, "permuted_hidden_states", _row_types(), rows * hsize, dev)
            if not _same_row_type(permuted_hidden_states, hidden_states):
                raise TypeError("permuted_hidden_states (%s) must have the type of hidden_states (%s)"
                                % (permuted_hidden_states.dtype, hidden_states.dtype))
    _check(offsets, "expert_first_token_offset", (torch.int64,), num_offsets, dev)
    _check(permuted_idx, "permuted_idx", (torch.int32,), rows, dev)
    _check(inv_permuted_idx, "inv_permuted_idx", (torch.int32,), rows, dev)
    if (token_scale is None) != (permuted_scale is None):
        raise ValueError("token_scale and permuted_scale go together")
    _check(token_scale, "token_scale", (torch.float32,), n, dev, optional=True)
    _check(permuted_scale, "permuted_scale", (torch.float32,), rows, dev, optional=True)
    if workspace is not None:
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        if workspace.device != dev:
            raise TypeError("workspace is on %s, expected %s" % (workspace.device, dev))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return hidden, code, hsize, ws_bytes, ids_code


def _permute_done(topk_ids) -> None:
    _require_gpu(topk_ids.device)


def moe_permute(hidden_states, topk_ids, num_experts: int, permuted_hidden_states,
                expert_first_token_offset, permuted_idx, inv_permuted_idx, workspace=None,
                token_scale=None, permuted_scale=None, stream=None) -> None:
    """Enqueue the permute on ``stream`` (default: torch's current stream).

    ``hidden_states`` [N, H] (float32, bfloat16, or fp8 codes as uint8 /
    float8_e4m3fn) or None for an index-only permute; ``topk_ids`` int32 or
    int64 [N, topk] (int64 is read directly, no cast pass).  Outputs are
    written in place.
    """
    hidden, code, hsize, ws_bytes, ids_code = _permute_args(
        hidden_states, topk_ids, workspace, expert_first_token_offset, permuted_idx, inv_permuted_idx,
        int(num_experts) + 1, permuted_hidden_states, token_scale, permuted_scale)
    _permute_done(topk_ids)
    n, topk = topk_ids.shape
    status = load_library().moe_permute(
        _ptr(hidden), code, _ptr(token_scale), _ptr(topk_ids), ids_code, n, hsize, topk, int(num_experts),
        _ptr(permuted_hidden_states) if hsize else None, _ptr(permuted_scale),
        _ptr(expert_first_token_offset), _ptr(permuted_idx), _ptr(inv_permuted_idx),
        _ptr(workspace), ws_bytes, _stream(stream, topk_ids))
    if status != MOE_OK:
        raise MoEError(status, "moe_permute")


MOE_STATIC_SCRATCH_BYTES = 4 << 20  # the library's static workspace per GPU (moe_permute_static_scratch)


def moe_permute_static_scratch(hidden_states, topk_ids, num_experts: int, permuted_hidden_states,
                               expert_first_token_offset, permuted_idx, inv_permuted_idx, token_scale=None,
                               permuted_scale=None, stream=None) -> None:
    """moe_permute without a workspace argument, for callers that cannot allocate.

    The library's static per-GPU array (MOE_STATIC_SCRATCH_BYTES) is the
    workspace; calls that overlap on one GPU race.  A call that needs more
    workspace than that raises MoEError (MOE_ERR_WORKSPACE_TOO_SMALL).
    """
    hidden, code, hsize, _, ids_code = _permute_args(
        hidden_states, topk_ids, None, expert_first_token_offset, permuted_idx, inv_permuted_idx,
        int(num_experts) + 1, permuted_hidden_states, token_scale, permuted_scale)
    _permute_done(topk_ids)
    n, topk = topk_ids.shape
    status = load_library().moe_permute_static_scratch(
        _ptr(hidden), code, _ptr(token_scale), _ptr(topk_ids), ids_code, n, hsize, topk, int(num_experts),
        _ptr(permuted_hidden_states) if hsize else None, _ptr(permuted_scale),
        _ptr(expert_first_token_offset), _ptr(permuted_idx), _ptr(inv_permuted_idx), _stream(stream, topk_ids))
    if status != MOE_OK:
        raise MoEError(status, "moe_permute_static_scratch")


def moe_permute_local(hidden_states, topk_ids, num_experts: int, expert_map, num_local_experts: int,
                      permuted_hidden_states, expert_first_token_offset, permuted_idx, inv_permuted_idx,
                      workspace=None, token_scale=None, permuted_scale=None, stream=None) -> None:
    """Permute restricted to this rank's experts (see moe_permute_local in the C header).

    ``expert_map`` int32 [num_experts] on the device: local id or -1.  The
    offsets have num_local_experts + 1 entries; inv_permuted_idx is -1 for
    rows of remote experts; only the first offsets[-1] rows are written.
    """
    import torch

    if expert_map is None or expert_map.dtype != torch.int32 or expert_map.shape != (int(num_experts),):
        raise TypeError("expert_map must be an int32 [num_experts] tensor")
    hidden, code, hsize, ws_bytes, ids_code = _permute_args(
        hidden_states, topk_ids, workspace, expert_first_token_offset, permuted_idx, inv_permuted_idx,
        int(num_local_experts) + 1, permuted_hidden_states, token_scale, permuted_scale)
    _check(expert_map, "expert_map", (torch.int32,), int(num_experts), topk_ids.device)
    _permute_done(topk_ids)
    n, topk = topk_ids.shape
    status = load_library().moe_permute_local(
        _ptr(hidden), code, _ptr(token_scale), _ptr(topk_ids), ids_code, n, hsize, topk, int(num_experts),
        _ptr(expert_map), int(num_local_experts),
        _ptr(permuted_hidden_states) if hsize else None, _ptr(permuted_scale),
        _ptr(expert_first_token_offset), _ptr(permuted_idx), _ptr(inv_permuted_idx),
        _ptr(workspace), ws_bytes, _stream(stream, topk_ids))
    if status != MOE_OK:
        raise MoEError(status, "moe_permute_local")


def moe_permute_quant_fp8(hidden_states, topk_ids, num_experts: int, permuted_codes, permuted_scale,
                          expert_first_token_offset, permuted_idx, inv_permuted_idx, workspace=None,
                          group_size: int = 0, expert_map=None, num_local_experts: int = 0, stream=None) -> None:
    """Quantise while permuting (see moe_permute_quant_fp8 in the C header).

    ``hidden_states`` bfloat16 or float32 [N, H]; ``permuted_codes`` uint8 (or
    float8_e4m3fn) [N*topk, H]; ``permuted_scale`` float32 [N*topk, H / group]
    (one column for group_size 0); with ``expert_map`` the local-expert
    permute over ``num_local_experts``.
    """
    import torch

    if hidden_states is None or hidden_states.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("hidden_states must be bfloat16 or float32")
    if expert_map is not None and (expert_map.dtype != torch.int32 or expert_map.shape != (int(num_experts),)):
        raise TypeError("expert_map must be an int32 [num_experts] tensor")
    num_offsets = (int(num_local_experts) if expert_map is not None else int(num_experts)) + 1
    _, code, hsize, ws_bytes, ids_code = _permute_args(
        hidden_states, topk_ids, workspace, expert_first_token_offset, permuted_idx, inv_permuted_idx, num_offsets,
        check_rows=False)
    n, topk = topk_ids.shape
    if group_size < 0 or (group_size and hsize % group_size):
        raise ValueError("group_size must be 0 (one scale per token) or divide the hidden size %d" % hsize)
    groups = 1 if group_size == 0 else hsize // group_size
    _check(permuted_codes, "permuted_codes", (torch.uint8, torch.float8_e4m3fn), n * topk * hsize, topk_ids.device)
    _check(permuted_scale, "permuted_scale", (torch.float32,), n * topk * groups, topk_ids.device)
    _check(expert_map, "expert_map", (torch.int32,), int(num_experts), topk_ids.device, optional=True)
    _permute_done(topk_ids)
    status = load_library().moe_permute_quant_fp8(
        _ptr(hidden_states), code, _ptr(topk_ids), ids_code, n, hsize, topk, int(num_experts), _ptr(expert_map),
        int(num_local_experts) if expert_map is not None else 0, int(group_size), _ptr(permuted_codes),
        _ptr(permuted_scale), _ptr(expert_first_token_offset), _ptr(permuted_idx), _ptr(inv_permuted_idx),
        _ptr(workspace), ws_bytes, _stream(stream, topk_ids))
    if status != MOE_OK:
        raise MoEError(status, "moe_permute_quant_fp8")


def moe_grouped_gemm_bf16(x, w, expert_first_token_offset, y, stream=None) -> None:
    """y[j] = x[j] @ w[e]^T for the permuted rows j of expert e (see the C header).

    ``x`` bfloat16 [max_rows, k]; ``w`` bfloat16 [E, n, k]; offsets int64
    [E + 1] on the device; ``y`` bfloat16 [max_rows, n].
    """
    import torch

    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16 or y.dtype != torch.bfloat16:
        raise TypeError("x, w and y must be bfloat16")
    if w.dim() != 3 or x.dim() != 2 or y.dim() != 2:
        raise ValueError("w must be [E, n, k], x [max_rows, k] and y [max_rows, n]")
    e, n, k = w.shape
    dev = y.device
    _check(x, "x", (torch.bfloat16,), x.shape[0] * k, dev)
    _check(w, "w", (torch.bfloat16,), e * n * k, dev)
    _check(y, "y", (torch.bfloat16,), x.shape[0] * n, dev)
    _check(expert_first_token_offset, "expert_first_token_offset", (torch.int64,), e + 1, dev)
    _require_gpu(dev)
    status = load_library().moe_grouped_gemm_bf16(_ptr(x), _ptr(w), _ptr(expert_first_token_offset), e,
                                                   x.shape[0], n, k, _ptr(y), _stream(stream, y))
    if status != MOE_OK:
        raise MoEError(status, "moe_grouped_gemm_bf16")


def moe_unpermute(expanded_output, topk_weights, inv_permuted_idx, output, stream=None) -> None:
    """Enqueue the unpermute on ``stream`` (default: torch's current stream).

    ``expanded_output`` [N*topk, H] float32 or bfloat16 in permuted order,
    ``topk_weights`` float32 [N, topk], ``inv_permuted_idx`` int32 [N*topk],
    ``output`` [N, H] of the same type as ``expanded_output``.
    """
    _unpermute("moe_unpermute", expanded_output, topk_weights, inv_permuted_idx, output, stream)


def moe_unpermute_local(expanded_output, topk_weights, inv_permuted_idx, output, stream=None) -> None:
    """moe_unpermute scheduled for the inverse index of ``moe_permute_local``
    (most entries -1); same arguments and result."""
    _unpermute("moe_unpermute_local", expanded_output, topk_weights, inv_permuted_idx, output, stream)


def _unpermute(name, expanded_output, topk_weights, inv_permuted_idx, output, stream) -> None:
    import torch

    if topk_weights is None or topk_weights.dim() != 2:
        raise ValueError("topk_weights must be a float32 [num_tokens, topk] tensor")
    n, topk = topk_weights.shape
    if expanded_output is None or expanded_output.dim() != 2 or expanded_output.shape[0] != n * topk:
        raise ValueError("expanded_output must be [num_tokens * topk = %d, hidden_size]" % (n * topk))
    h = expanded_output.shape[-1]
    dev = expanded_output.device
    _check(expanded_output, "expanded_output", (torch.float32, torch.bfloat16), n * topk * h, dev)
    _check(topk_weights, "topk_weights", (torch.float32,), n * topk, dev)
    _check(inv_permuted_idx, "inv_permuted_idx", (torch.int32,), n * topk, dev)
    _check(output, "output", (expanded_output.dtype,), n * h, dev)
    _require_gpu(dev)
    status = getattr(load_library(), name)(
        _ptr(expanded_output), _dtype_code(expanded_output), _ptr(topk_weights), _ptr(inv_permuted_idx),
        n, expanded_output.shape[-1], topk, _ptr(output), _stream(stream, output))
    if status != MOE_OK:
        raise MoEError(status, name)


class MoEPermuteScratch:
    """Every permute buffer, allocated once for ``max_num_tokens`` and reused.

    Mirrors MoEPermuteScratch in the prhub summary of vLLM PR #43014 (section
    "key code snippets"): offsets int64 [num_local_experts + 1]; permuted_idx
    and inv_permuted_idx int32 [max_num_tokens * topk]; permuted_hidden_states
    only when ``hidden_size`` is given; an opaque workspace sized by the
    library's size query.  ``validate`` performs the same checks the summary
    lists (device, token count, topk, hidden size and type).  With
    ``expert_map`` (int32 [num_experts], local id or -1) every call runs the
    local-expert permute over ``num_local_experts`` experts.
    """

    def __init__(self, max_num_tokens: int, topk: int, num_experts: int, device, hidden_size: int | None = None,
                 hidden_dtype=None, with_scale: bool = False, expert_map=None, num_local_experts: int | None = None):
        import torch

        self.max_num_tokens = int(max_num_tokens)
        self.topk = int(topk)
        self.num_experts = int(num_experts)
        if (expert_map is None) != (num_local_experts is None):
            raise ValueError("expert_map and num_local_experts go together")
        self.expert_map = expert_map
        self.num_local_experts = self.num_experts if expert_map is None else int(num_local_experts)
        self.device = torch.device(device)
        self.hidden_size = hidden_size
        self.hidden_dtype = hidden_dtype
        self.max_expanded_rows = self.max_num_tokens * self.topk
        rows = self.max_expanded_rows
        self.expert_first_token_offset = torch.empty(self.num_local_experts + 1, dtype=torch.int64,
                                                     device=self.device)
        self.permuted_idx = torch.empty(rows, dtype=torch.int32, device=self.device)
        self.inv_permuted_idx = torch.empty(rows, dtype=torch.int32, device=self.device)
        self.permuted_hidden_states = None
        if hidden_size is not None:
            self.permuted_hidden_states = torch.empty(rows * hidden_size, dtype=hidden_dtype, device=self.device)
        self.permuted_scale = torch.empty(rows, dtype=torch.float32, device=self.device) if with_scale else None
        if expert_map is None:
            ws = moe_permute_workspace_size(self.max_num_tokens, self.topk, self.num_experts)
        else:
            ws = moe_permute_local_workspace_size(self.max_num_tokens, self.topk, self.num_experts,
                                                  self.num_local_experts)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=self.device)

    def validate(self, hidden_states, topk_ids) -> None:
        n = topk_ids.shape[0]
        if topk_ids.device != self.device or (hidden_states is not None and hidden_states.device != self.device):
            raise ValueError("inputs are not on the scratch device")
        if n > self.max_num_tokens:
            raise ValueError("num_tokens %d exceeds max_num_tokens %d" % (n, self.max_num_tokens))
        if topk_ids.dim() != 2 or topk_ids.shape[1] != self.topk:
            raise ValueError("topk_ids must be [num_tokens, %d]" % self.topk)
        if hidden_states is not None:
            if hidden_states.shape[0] != n:
                raise ValueError("hidden_states and topk_ids disagree on num_tokens")
            if self.hidden_size is not None and (hidden_states.shape[-1] != self.hidden_size
                                                 or hidden_states.dtype != self.hidden_dtype):
                raise ValueError("hidden_states does not match the scratch hidden size / type")

    def permute(self, hidden_states, topk_ids, token_scale=None, stream=None) -> dict:
        """Run moe_permute into the scratch buffers; returns views sized for this call."""
        self.validate(hidden_states, topk_ids)
        n = topk_ids.shape[0]
        rows = n * self.topk
        out_hidden = None
        if hidden_states is not None:
            if self.permuted_hidden_states is None:
                raise ValueError("scratch was created without hidden_size")
            out_hidden = self.permuted_hidden_states[: rows * self.hidden_size].view(rows, self.hidden_size)
        out_scale = None
        if token_scale is not None:
            if self.permuted_scale is None:
                raise ValueError("scratch was created without with_scale=True")
            out_scale = self.permuted_scale[:rows]
        if self.expert_map is None:
            moe_permute(hidden_states, topk_ids, self.num_experts, out_hidden, self.expert_first_token_offset,
                        self.permuted_idx[:rows], self.inv_permuted_idx[:rows], self.workspace,
                        token_scale=token_scale, permuted_scale=out_scale, stream=stream)
        else:
            moe_permute_local(hidden_states, topk_ids, self.num_experts, self.expert_map, self.num_local_experts,
                              out_hidden, self.expert_first_token_offset, self.permuted_idx[:rows],
                              self.inv_permuted_idx[:rows], self.workspace, token_scale=token_scale,
                              permuted_scale=out_scale, stream=stream)
        return {
            "permuted_hidden_states": out_hidden,
            "permuted_scale": out_scale,
            "expert_first_token_offset": self.expert_first_token_offset,
            "permuted_idx": self.permuted_idx[:rows],
            "inv_permuted_idx": self.inv_permuted_idx[:rows],
        }
