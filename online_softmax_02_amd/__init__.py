"""Online-softmax attention and row softmax on MI355X (gfx950).

A thin ``ctypes`` binding over ``libosx.so`` (the C ABI in ``include/osx.h``).
It only marshals arguments: every step of the computation runs in the
library's HIP kernels.  PyTorch supplies device memory and the current stream.

The library must be built first (``python -m online_softmax_02_amd.build``);
importing this package without it raises ``ImportError``.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libosx.so")
# The same sources built with extra waits and barriers at every LDS stage
# (see build.py); used by the tests through using_library().
DEBUG_SYNC_LIB_PATH = os.path.join(_HERE, "libosx_debug_sync.so")

OSX_OK, OSX_EINVAL, OSX_EUNSUPPORTED, OSX_EHIP, OSX_EWORKSPACE = 0, -1, -2, -3, -4
OSX_F32, OSX_BF16 = 0, 1
OSX_3PASS_ATOMIC, OSX_3PASS_STASH = 1, 2
KERNELS = {0: "none", 1: "prefill_f32", 2: "prefill_bf16", 3: "decode_bf16", 4: "softmax_row", 5: "softmax_split",
           6: "softmax_wave"}

_i, _i64, _sz, _vp, _f = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float


class Plan(ctypes.Structure):
    _fields_ = [("kernel", _i), ("threads", _i), ("block_m", _i), ("block_n", _i), ("splits", _i),
                ("heads_per_wg", _i), ("grid", _i64), ("workspace_bytes", _sz)]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["kernel_name"] = KERNELS.get(self.kernel, "?")
        return d


class OsxError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)}: {detail}")
        self.status = status


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    # libosx.so links libamdhip64.so.7.  PyTorch ships its own copy of that
    # runtime; loading torch first makes the library bind to the same runtime
    # instead of pulling a second one into the process (two HIP runtimes in one
    # process do not share devices, streams or allocations).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m online_softmax_02_amd.build` "
                          "(hipcc for gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    attn_shape = [_i, _i, _i, _i, _i, _i, _i, _i]  # dtype, B, Hq, Hkv, Sq, Sk, D, causal
    lib.osx_attn_plan.argtypes = attn_shape + [ctypes.POINTER(Plan)]
    lib.osx_attn_fwd_workspace.argtypes = attn_shape + [ctypes.POINTER(_sz)]
    lib.osx_attn_fwd_workspace_bytes.argtypes = attn_shape
    lib.osx_attn_fwd_workspace_bytes.restype = _sz
    lib.osx_attn_fwd.argtypes = [_vp, _vp, _vp, _vp] + attn_shape + [_f, _vp, _sz, _vp]
    lib.osx_attn_fwd_lse.argtypes = [_vp, _vp, _vp, _vp, _vp] + attn_shape + [_f, _vp, _sz, _vp]
    lib.osx_attn_fwd_normalised.argtypes = [_vp, _vp, _vp, _vp, _vp] + attn_shape + [_f, _vp, _sz, _vp]
    lib.osx_attn_fwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp] + attn_shape + [_f, _vp]
    lib.osx_softmax_rows_plan.argtypes = [_i64, _i64, ctypes.POINTER(Plan)]
    lib.osx_softmax_rows_workspace.argtypes = [_i64, _i64, ctypes.POINTER(_sz)]
    lib.osx_softmax_rows_workspace_bytes.argtypes = [_i64, _i64]
    lib.osx_softmax_rows_workspace_bytes.restype = _sz
    lib.osx_softmax_rows.argtypes = [_vp, _vp, _i64, _i64, _vp, _sz, _vp]
    lib.osx_softmax_rows_ex.argtypes = [_vp, _vp, _i, _i64, _i64, _i64, _f, _vp, _sz, _vp]
    lib.osx_attn_fwd_unfused_workspace.argtypes = attn_shape + [ctypes.POINTER(_sz)]
    lib.osx_attn_fwd_unfused.argtypes = [_vp, _vp, _vp, _vp] + attn_shape + [_f, _vp, _sz, _vp]
    lib.osx_softmax_rows_3pass_workspace.argtypes = [_i64, _i64, _i, ctypes.POINTER(_sz)]
    lib.osx_softmax_rows_3pass.argtypes = [_vp, _vp, _i64, _i64, _i, _vp, _sz, _vp]
    lib.osx_read_probe_sink_bytes.argtypes = []
    lib.osx_read_probe_sink_bytes.restype = _sz
    lib.osx_read_probe.argtypes = [_vp, _sz, _vp, _sz, _vp]
    lib.osx_read_probe.restype = _i
    lib.osx_status_string.argtypes = [_i]
    lib.osx_status_string.restype = ctypes.c_char_p
    lib.osx_last_error.argtypes = []
    lib.osx_last_error.restype = ctypes.c_char_p
    lib.osx_version.argtypes = []
    for name in ("osx_attn_plan", "osx_attn_fwd_workspace", "osx_attn_fwd", "osx_attn_fwd_lse",
                 "osx_attn_fwd_normalised", "osx_attn_fwd_noalloc", "osx_softmax_rows_plan",
                 "osx_softmax_rows_workspace", "osx_softmax_rows", "osx_softmax_rows_ex",
                 "osx_softmax_rows_3pass_workspace", "osx_softmax_rows_3pass", "osx_attn_fwd_unfused_workspace",
                 "osx_attn_fwd_unfused", "osx_version"):
        getattr(lib, name).restype = _i
    return lib


lib = _load()


@contextlib.contextmanager
def using_library(path: str):
    """Route this module's calls through another build of the library (same C
    ABI, e.g. DEBUG_SYNC_LIB_PATH) until the block ends."""
    global lib
    saved = lib
    lib = _load(path)
    try:
        yield lib
    finally:
        lib = saved


def status_string(status: int) -> str:
    return lib.osx_status_string(status).decode()


def last_error() -> str:
    return lib.osx_last_error().decode()


def version() -> int:
    return lib.osx_version()


def _check(status: int) -> None:
    if status != OSX_OK:
        raise OsxError(status, last_error())


def attn_plan(dtype: int, batch: int, heads_q: int, heads_kv: int, seq_q: int, seq_k: int, head_dim: int,
              causal: bool = False) -> dict:
    """Kernel choice for an attention problem (no GPU needed); raises OsxError on bad arguments."""
    p = Plan()
    _check(lib.osx_attn_plan(dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, int(causal), ctypes.byref(p)))
    return p.as_dict()


def attn_fwd_workspace(dtype: int, batch: int, heads_q: int, heads_kv: int, seq_q: int, seq_k: int, head_dim: int,
                       causal: bool = False) -> int:
    n = _sz(0)
    _check(lib.osx_attn_fwd_workspace(dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, int(causal),
                                      ctypes.byref(n)))
    return n.value


def softmax_rows_plan(rows: int, cols: int) -> dict:
    p = Plan()
    _check(lib.osx_softmax_rows_plan(rows, cols, ctypes.byref(p)))
    return p.as_dict()


def softmax_rows_workspace(rows: int, cols: int) -> int:
    n = _sz(0)
    _check(lib.osx_softmax_rows_workspace(rows, cols, ctypes.byref(n)))
    return n.value


def _torch():
    import torch
    return torch


def _common_device(*tensors, stream=None):
    """The one device of the tensors (None entries skipped); ValueError when they, or a torch stream given for
    them, are on different devices."""
    torch = _torch()
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError("the tensors of one call must be on one CUDA device, got " + ", ".join(sorted(map(str, devs))))
    dev = devs.pop()
    if isinstance(stream, torch.cuda.Stream) and stream.device != dev:
        raise ValueError(f"the stream belongs to {stream.device}, the tensors to {dev}")
    return dev


def _device_of(*tensors, stream=None):
    """Context in which the tensors' common device is current: the C ABI launches on the current device."""
    return _torch().cuda.device(_common_device(*tensors, stream=stream))


def _stream(t, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return _vp(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _workspace(need: int, workspace, device):
    """The workspace tensor to pass (the caller's, or a new one when `need` > 0 and none was given), its pointer and
    its length in bytes.  The caller of this helper keeps the returned tensor referenced until the launch is
    enqueued, and hands it to _hold() afterwards."""
    torch = _torch()
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace is None:
        return None, None, 0
    if not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor")
    return workspace, workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _hold(ws, stream) -> None:
    """Keep a workspace the binding allocated from being reused before the kernels on `stream` are done with it.

    torch's caching allocator hands freed memory to later allocations in the order of the current stream; work
    launched on another stream is ordered only once the tensor is recorded on that stream."""
    if ws is None or stream is None:
        return
    torch = _torch()
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(
        stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream), device=ws.device)
    if s.cuda_stream != torch.cuda.current_stream(ws.device).cuda_stream:
        ws.record_stream(s)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return OSX_F32
    if t.dtype == torch.bfloat16:
        return OSX_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _attn_prepare(q, k, v, causal, out, workspace, stream=None):
    """Checks q, k, v and out, allocates what is missing (on q's device); returns the 4-D views and the call
    arguments."""
    torch = _torch()
    squeeze = q.dim() == 2
    if squeeze:
        q, k, v = q[None, None], k[None, None], v[None, None]
        if out is not None and out.dim() == 2:
            out = out[None, None]
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, S, D] (or 2-D [S, D])")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CUDA tensor")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError("batch and head_dim of q and k must match")
    code = _dtype_code(q)
    if out is not None and (out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor like q")
    with _device_of(q, k, v, out, workspace, stream=stream):
        if out is None:
            out = torch.empty_like(q)
        need = attn_fwd_workspace(code, B, Hq, Hkv, Sq, Sk, D, causal)
        ws = _workspace(need, workspace, q.device)
    return squeeze, q, k, v, out, code, (B, Hq, Hkv, Sq, Sk, D), ws


def _lse_tensor(q, shape, lse):
    torch = _torch()
    B, Hq, Sq = shape[0], shape[1], shape[3]
    if lse is None:
        return torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if lse.numel() != B * Hq * Sq or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of B * Hq * Sq elements")
    return lse


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, workspace=None, stream=None,
             return_lse: bool = False, lse=None):
    """O = softmax(mask(q k^T * scale)) v on the GPU.

    q: [B, Hq, Sq, D] (or [M, D] for one head), k, v: [B, Hkv, Sk, D] (or
    [N, D]); contiguous CUDA tensors of one dtype (float32 or bfloat16).
    Query head h reads KV head h // (Hq // Hkv).  Returns a tensor like q; with
    ``return_lse`` also the float32 [B, Hq, Sq] (or [M]) log-sum-exp of each
    row's scaled, masked scores (``lse`` may supply that tensor).
    """
    squeeze, q, k, v, out, code, shape, (ws, ws_ptr, ws_len) = _attn_prepare(q, k, v, causal, out, workspace, stream)
    sc = float(scale) if scale else 0.0
    if not (return_lse or lse is not None):
        with _device_of(q, k, v, out, ws, stream=stream):
            _check(lib.osx_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), code, *shape,
                                    int(causal), sc, ws_ptr, ws_len, _stream(q, stream)))
        _hold(ws if workspace is None else None, stream)
        return out[0, 0] if squeeze else out
    lse = _lse_tensor(q, shape, lse)
    with _device_of(q, k, v, out, ws, lse, stream=stream):
        _check(lib.osx_attn_fwd_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), code,
                                    *shape, int(causal), sc, ws_ptr, ws_len, _stream(q, stream)))
    _hold(ws if workspace is None else None, stream)
    if squeeze:
        return out[0, 0], lse.reshape(-1)
    return out, lse


def attn_fwd_normalised(q, k, v, causal: bool = False, scale: float | None = None, out=None, workspace=None,
                        stream=None, return_lse: bool = False, lse=None):
    """attn_fwd computed with the normalised-output recurrence (osx_attn_fwd_normalised): float32 only."""
    squeeze, q, k, v, out, code, shape, (ws, ws_ptr, ws_len) = _attn_prepare(q, k, v, causal, out, workspace, stream)
    sc = float(scale) if scale else 0.0
    want = return_lse or lse is not None
    if want:
        lse = _lse_tensor(q, shape, lse)
    with _device_of(q, k, v, out, ws, lse if want else None, stream=stream):
        _check(lib.osx_attn_fwd_normalised(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                           lse.data_ptr() if want else None, code, *shape, int(causal), sc, ws_ptr,
                                           ws_len, _stream(q, stream)))
    _hold(ws if workspace is None else None, stream)
    o = out[0, 0] if squeeze else out
    if not want:
        return o
    return o, (lse.reshape(-1) if squeeze else lse)


NOALLOC_SCRATCH_BYTES = 64 << 20  # OSX_NOALLOC_SCRATCH_BYTES


def attn_fwd_noalloc(q, k, v, out, causal: bool = False, scale: float | None = None, lse=None, stream=None):
    """:func:`attn_fwd` through osx_attn_fwd_noalloc: the library's static scratch instead of a workspace.

    ``out`` (and ``lse``, if given) must be supplied: nothing is allocated here.  Calls that overlap in time on one
    GPU share the scratch and must be ordered by the caller."""
    squeeze = q.dim() == 2
    if squeeze:
        q, k, v, out = q[None, None], k[None, None], v[None, None], out[None, None]
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D (or 2-D) CUDA tensor")
    if not (q.dtype == k.dtype == v.dtype == out.dtype) or k.shape != v.shape or out.shape != q.shape:
        raise ValueError("q, k, v, out must share one dtype; k and v one shape; out q's shape")
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    if lse is not None and (lse.numel() != B * Hq * Sq or not lse.is_contiguous()
                            or lse.dtype != _torch().float32):
        raise ValueError("lse must be a contiguous float32 tensor of B * Hq * Sq elements")
    with _device_of(q, k, v, out, lse, stream=stream):
        _check(lib.osx_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        lse.data_ptr() if lse is not None else None, _dtype_code(q), B, Hq, Hkv, Sq,
                                        Sk, D, int(causal), float(scale) if scale else 0.0, _stream(q, stream)))
    return out[0, 0] if squeeze else out


def softmax_rows(x, out=None, workspace=None, stream=None, causal_period: int = 0, scale: float = 1.0):
    """y = softmax(scale * x) along the last dimension of a contiguous float32 or bfloat16 CUDA tensor.

    ``causal_period`` P > 0 masks, in row r (of the rows flattened to 2-D),
    the columns c > r mod P (y = 0 there).  ``out`` may be ``x`` itself (in
    place); y has x's dtype.
    """
    torch = _torch()
    if x.dtype not in (torch.float32, torch.bfloat16) or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 or bfloat16 CUDA tensor")
    cols = x.shape[-1] if x.dim() else 1
    rows = x.numel() // cols if cols else 0
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x")
    with _device_of(x, out, workspace, stream=stream):
        ws, ws_ptr, ws_len = _workspace(softmax_rows_workspace(rows, cols), workspace, x.device)
        if x.dtype == torch.float32 and not causal_period and scale == 1.0:
            _check(lib.osx_softmax_rows(x.data_ptr(), out.data_ptr(), rows, cols, ws_ptr, ws_len,
                                        _stream(x, stream)))
        else:
            _check(lib.osx_softmax_rows_ex(x.data_ptr(), out.data_ptr(), _dtype_code(x), rows, cols,
                                           int(causal_period), float(scale), ws_ptr, ws_len, _stream(x, stream)))
    _hold(ws if workspace is None else None, stream)
    return out


def attn_fwd_unfused_workspace(dtype: int, batch: int, heads_q: int, heads_kv: int, seq_q: int, seq_k: int,
                               head_dim: int, causal: bool = False) -> int:
    n = _sz(0)
    _check(lib.osx_attn_fwd_unfused_workspace(dtype, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, int(causal),
                                              ctypes.byref(n)))
    return n.value


def attn_fwd_unfused(q, k, v, causal: bool = False, scale: float | None = None, out=None, workspace=None,
                     stream=None):
    """The same O as :func:`attn_fwd` (bf16 only), computed by the unfused comparator: the score matrix
    S = scale * q k^T is written to the workspace (fp32, 4 bytes per score), softmaxed in place, then
    multiplied by v.  Shapes as :func:`attn_fwd`."""
    torch = _torch()
    squeeze = q.dim() == 2
    if squeeze:
        q, k, v = q[None, None], k[None, None], v[None, None]
        if out is not None and out.dim() == 2:
            out = out[None, None]
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D (or 2-D) CUDA tensor")
    if k.shape != v.shape or q.dtype != k.dtype or k.dtype != v.dtype:
        raise ValueError("k and v must match, and q, k, v share one dtype")
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    code = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    with _device_of(q, k, v, out, workspace, stream=stream):
        ws, ws_ptr, ws_len = _workspace(attn_fwd_unfused_workspace(code, B, Hq, Hkv, Sq, Sk, D, causal), workspace,
                                        q.device)
        _check(lib.osx_attn_fwd_unfused(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), code, B, Hq, Hkv,
                                        Sq, Sk, D, int(causal), float(scale) if scale else 0.0, ws_ptr, ws_len,
                                        _stream(q, stream)))
    _hold(ws if workspace is None else None, stream)
    return out[0, 0] if squeeze else out


def softmax_rows_3pass_workspace(rows: int, cols: int, method: int) -> int:
    n = _sz(0)
    _check(lib.osx_softmax_rows_3pass_workspace(rows, cols, method, ctypes.byref(n)))
    return n.value


def softmax_rows_3pass(x, method: int, out=None, workspace=None, stream=None):
    """Row softmax of a contiguous float32 CUDA tensor by a three-pass comparator design.

    ``method``: OSX_3PASS_ATOMIC (max, sum of exp and normalise launches, each
    reading x, merged by atomics) or OSX_3PASS_STASH (max; exp stashed in y and
    summed; y rescaled).  Same result as :func:`softmax_rows`.
    """
    torch = _torch()
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 CUDA tensor")
    cols = x.shape[-1] if x.dim() else 1
    rows = x.numel() // cols if cols else 0
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x")
    with _device_of(x, out, workspace, stream=stream):
        ws, ws_ptr, ws_len = _workspace(softmax_rows_3pass_workspace(rows, cols, method), workspace, x.device)
        _check(lib.osx_softmax_rows_3pass(x.data_ptr(), out.data_ptr(), rows, cols, method, ws_ptr, ws_len,
                                          _stream(x, stream)))
    _hold(ws if workspace is None else None, stream)
    return out


def read_probe(x, sink=None, stream=None):
    """Plain streaming read of the contiguous CUDA tensor x (osx_read_probe: a measurement aid).

    Returns the int32 sink tensor: the XOR of its words is the XOR of x's 32-bit words."""
    torch = _torch()
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous CUDA tensor")
    nbytes = x.numel() * x.element_size()
    if sink is None:
        sink = torch.empty(lib.osx_read_probe_sink_bytes() // 4, dtype=torch.int32, device=x.device)
    with _device_of(x, sink, stream=stream):
        _check(lib.osx_read_probe(x.data_ptr(), nbytes, sink.data_ptr(), sink.numel() * sink.element_size(),
                                  _stream(x, stream)))
    return sink


__all__ = ["attn_fwd", "softmax_rows", "attn_plan", "attn_fwd_workspace", "softmax_rows_plan",
           "softmax_rows_workspace", "status_string", "last_error", "version", "OsxError", "lib", "LIB_PATH",
           "OSX_F32", "OSX_BF16", "softmax_rows_3pass", "softmax_rows_3pass_workspace", "OSX_3PASS_ATOMIC",
           "OSX_3PASS_STASH", "attn_fwd_unfused", "attn_fwd_unfused_workspace", "attn_fwd_normalised",
           "read_probe", "attn_fwd_noalloc", "NOALLOC_SCRATCH_BYTES"]
