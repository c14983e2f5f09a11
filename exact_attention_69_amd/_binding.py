"""ctypes binding of libexattn.so: argument marshalling only.

Every step of the attention path runs in the library's HIP kernels; this
module checks tensor shapes/dtypes, allocates outputs with PyTorch (device
memory only) and passes raw device pointers and the current HIP stream to the
C entry points declared in include/exattn.h.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""

import ctypes
import functools
import inspect
import math
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# The library built in the package directory; EXATTN_LIBRARY names another
# build of it (the host-sanitizer build of exact_attention_69_amd.build).
LIB_PATH = os.environ.get("EXATTN_LIBRARY") or os.path.join(PKG_DIR, "libexattn.so")

EXATTN_F32 = 0
EXATTN_BF16 = 1
EXATTN_FP8_ROWS = 0
EXATTN_FP8_V_TRANSPOSED = 1
STATUS = {0: "EXATTN_OK", -1: "EXATTN_EINVAL", -2: "EXATTN_EUNSUPPORTED", -3: "EXATTN_EWORKSPACE", -4: "EXATTN_EHIP",
          -5: "EXATTN_ESCRATCH"}
# Size of attn_bwd_noalloc's fixed per-GPU scratch buffer (the header's
# EXATTN_NOALLOC_SCRATCH_BYTES).
EXATTN_NOALLOC_SCRATCH_BYTES = 16 << 20

_lib = None


class ExattnPatternC(ctypes.Structure):
    """The C ABI's exattn_pattern descriptor (device pointers inside)."""
    _fields_ = [("window", ctypes.c_int), ("n_global", ctypes.c_int), ("global_idx", ctypes.c_void_p),
                ("layout_block", ctypes.c_int), ("layout", ctypes.c_void_p)]


class AttnPattern:
    """Sparse pattern on the GPU: window (-1: none), global token positions
    (int32 tensor or None) and a 64-token block layout (uint8 [nb, nb] tensor
    or None).  Holds references to the tensors while in use."""

    def __init__(self, window=-1, global_idx=None, layout=None):
        self.window = int(window)
        self.global_idx = global_idx
        self.layout = layout

    def as_c(self, n, device):
        torch = _torch()
        g, lay = self.global_idx, self.layout
        if g is not None:
            if g.dtype != torch.int32 or g.dim() != 1 or not g.is_contiguous() or g.device != device:
                raise ValueError("global_idx must be a contiguous int32 1-D tensor on the inputs' device")
        if lay is not None:
            nb = -(-n // 64)
            if lay.dtype != torch.uint8 or tuple(lay.shape) != (nb, nb) or not lay.is_contiguous() \
                    or lay.device != device:
                raise ValueError(f"layout must be a contiguous uint8 [{nb}, {nb}] tensor on the inputs' device")
        return ExattnPatternC(self.window, 0 if g is None else g.numel(), None if g is None else g.data_ptr(),
                              0 if lay is None else 64, None if lay is None else lay.data_ptr())


class ExattnError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")
        self.status = status


def load_library(path=None):
    """Load (once) and return the ctypes handle of libexattn.so."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m exact_attention_69_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    vp, ci, cf, cs = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [ci, ci, ci, ci, ci, vp, vp, vp, cf, ci, vp, vp, vp]
    lib.attn_fwd.restype = ci
    lib.attn_bwd_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.attn_bwd_workspace_bytes.restype = cs
    lib.attn_bwd.argtypes = [ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, cf, ci, vp, vp, vp, vp, cs, vp]
    lib.attn_bwd.restype = ci
    lib.attn_bwd_noalloc.argtypes = [ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, cf, ci, vp, vp, vp, vp]
    lib.attn_bwd_noalloc.restype = ci
    lib.attn_bwd_rowdot.argtypes = [ci, ci, ci, ci, ci, vp, vp, vp, vp, cs, vp]
    lib.attn_bwd_rowdot.restype = ci
    lib.attn_bwd_dkdv.argtypes = [ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, cf, ci, vp, vp, vp, cs, vp]
    lib.attn_bwd_dkdv.restype = ci
    lib.attn_bwd_dq.argtypes = [ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, cf, ci, vp, vp, cs, vp]
    lib.attn_bwd_dq.restype = ci
    lib.attn_fwd_gqa.argtypes = [ci, ci, ci, ci, ci, ci, vp, vp, vp, cf, ci, vp, vp, vp]
    lib.attn_fwd_gqa.restype = ci
    lib.attn_bwd_gqa.argtypes = [ci, ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, cf, ci, vp, vp, vp, vp, cs, vp]
    lib.attn_bwd_gqa.restype = ci
    lib.attn_bwd_dkdv_gqa.argtypes = [ci, ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, cf, ci, vp, vp, vp, cs, vp]
    lib.attn_bwd_dkdv_gqa.restype = ci
    lib.attn_bwd_dq_gqa.argtypes = [ci, ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, cf, ci, vp, vp, cs, vp]
    lib.attn_bwd_dq_gqa.restype = ci
    lib.attn_pattern_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.attn_pattern_workspace_bytes.restype = cs
    pp = ctypes.POINTER(ExattnPatternC)
    lib.attn_fwd_pattern.argtypes = [ci, ci, ci, ci, ci, vp, vp, vp, cf, pp, vp, vp, vp, cs, vp]
    lib.attn_fwd_pattern.restype = ci
    lib.attn_bwd_pattern.argtypes = [ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, cf, pp, vp, vp, vp, vp, cs, vp]
    lib.attn_bwd_pattern.restype = ci
    lib.attn_fp8_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.attn_fp8_bytes.restype = cs
    fp = ctypes.POINTER(ctypes.c_float)
    lib.attn_quant_fp8.argtypes = [ci, ci, ci, ci, vp, vp, ci, vp, vp, vp]
    lib.attn_quant_fp8.restype = ci
    lib.attn_fwd_fp8.argtypes = [ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, cf, ci, vp, vp, vp]
    lib.attn_fwd_fp8.restype = ci
    lib.exattn_status_string.argtypes = [ci]
    lib.exattn_status_string.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def exattn_status_string(status):
    return load_library().exattn_status_string(int(status)).decode()


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return EXATTN_BF16
    if t.dtype == torch.float32:
        return EXATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check_inputs(*ts):
    t0 = ts[0]
    if t0.dim() != 4:
        raise ValueError(f"expected [B, H, n, d] tensors, got shape {tuple(t0.shape)}")
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if t.shape != t0.shape or t.dtype != t0.dtype:
            raise ValueError("Q, K, V (and O, dO) must share shape and dtype")
        if t.device != t0.device:
            raise ValueError("all tensors of a call must be on one GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, n, d]")


def _check_gqa(q, k, v, *qlike):
    """Q (and O, dO) [B, H, n, d]; K, V [B, Hkv, n, d] with H % Hkv == 0.
    Returns Hkv."""
    _check_inputs(q, *qlike)
    _check_inputs(k, v)
    B, H, n, d = q.shape
    Bk, Hkv, nk, dk = k.shape
    if k.dtype != q.dtype or (Bk, nk, dk) != (B, n, d) or Hkv < 1 or H % Hkv:
        raise ValueError(f"K/V shape {tuple(k.shape)} does not fit Q {tuple(q.shape)} "
                         "(need [B, Hkv, n, d] with H a multiple of Hkv, same dtype)")
    return Hkv


def _out(t, shape, dtype, device):
    """An output tensor: allocated when t is None; otherwise it must be a
    contiguous GPU tensor of exactly this shape and dtype on this device,
    since the kernels write every element of the shape they are given."""
    torch = _torch()
    shape = tuple(int(x) for x in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if (not t.is_cuda or t.device != torch.device(device) or tuple(t.shape) != shape or t.dtype != dtype
            or not t.is_contiguous()):
        raise ValueError(f"output must be a contiguous {dtype} GPU tensor of shape {shape} on {device}; got "
                         f"shape {tuple(t.shape)}, {t.dtype}, on {t.device}"
                         + ("" if t.is_contiguous() else ", not contiguous"))
    return t


def _call(fn, *args):
    with _torch().cuda.device(args[-1][0]):
        st = getattr(load_library(), fn)(*args[:-1], args[-1][1])
    if st != 0:
        raise ExattnError(fn, st, exattn_status_string(st))


def _stream_ptr(t, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _on_call_stream(fn):
    """Run an entry point's wrapper with its `stream` argument (when one is
    given) as the current stream, so that every tensor the wrapper allocates
    (outputs, workspaces, scratch) belongs to the stream its kernels run on.
    The caching allocator then hands that memory to another allocation only
    in that stream's order: a workspace freed when the wrapper returns cannot
    be reused by work on some other stream while the queued kernels still
    read it."""
    pos = list(inspect.signature(fn).parameters).index("stream")

    @functools.wraps(fn)
    def wrapped(*args, **kw):
        stream = kw.get("stream") if "stream" in kw else (args[pos] if len(args) > pos else None)
        if stream is None:
            return fn(*args, **kw)
        with _torch().cuda.stream(stream):
            return fn(*args, **kw)
    return wrapped


@_on_call_stream
def attn_fwd(q, k, v, scale=None, window=-1, out=None, lse=None, stream=None):
    """Forward pass.  Returns (O, LSE): O like q, LSE float32 [B, H, n]."""
    torch = _torch()
    _check_inputs(q, k, v)
    B, H, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = _out(out, q.shape, q.dtype, q.device)
    lse = _out(lse, (B, H, n), torch.float32, q.device)
    with torch.cuda.device(q.device):
        st = load_library().attn_fwd(_dtype_code(q), B, H, n, d, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     scale, int(window), out.data_ptr(), lse.data_ptr(), _stream_ptr(q, stream))
    if st != 0:
        raise ExattnError("attn_fwd", st, exattn_status_string(st))
    return out, lse


def attn_bwd_workspace_bytes(dtype_code, B, H, n, d):
    return int(load_library().attn_bwd_workspace_bytes(dtype_code, B, H, n, d))


def _check_lse(lse, q):
    torch = _torch()
    B, H, n, _ = q.shape
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, n) or not lse.is_contiguous() or not lse.is_cuda
            or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 tensor [B, H, n] on the inputs' GPU")


@_on_call_stream
def attn_bwd(q, k, v, o, do, lse, scale=None, window=-1, workspace=None, dq=None, dk=None, dv=None, stream=None):
    """Backward pass.  Returns (dQ, dK, dV), each like q."""
    torch = _torch()
    _check_inputs(q, k, v, o, do)
    _check_lse(lse, q)
    B, H, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    need = attn_bwd_workspace_bytes(code, B, H, n, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dq = _out(dq, q.shape, q.dtype, q.device)
    dk = _out(dk, q.shape, q.dtype, q.device)
    dv = _out(dv, q.shape, q.dtype, q.device)
    with torch.cuda.device(q.device):
        st = load_library().attn_bwd(code, B, H, n, d, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     do.data_ptr(), lse.data_ptr(), scale, int(window), dq.data_ptr(),
                                     dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                                     _ws_bytes(workspace, q.device), _stream_ptr(q, stream))
    if st != 0:
        raise ExattnError("attn_bwd", st, exattn_status_string(st))
    return dq, dk, dv


@_on_call_stream
def attn_bwd_noalloc(q, k, v, o, do, lse, scale=None, window=-1, dq=None, dk=None, dv=None, stream=None):
    """Backward pass through the entry point that allocates nothing (its
    row arrays live in the library's fixed per-GPU scratch buffer).  Returns
    (dQ, dK, dV); pass dq, dk, dv to keep this wrapper from allocating them."""
    torch = _torch()
    _check_inputs(q, k, v, o, do)
    _check_lse(lse, q)
    B, H, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = _out(dq, q.shape, q.dtype, q.device)
    dk = _out(dk, q.shape, q.dtype, q.device)
    dv = _out(dv, q.shape, q.dtype, q.device)
    _call("attn_bwd_noalloc", _dtype_code(q), B, H, n, d, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
          do.data_ptr(), lse.data_ptr(), scale, int(window), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
          (q.device, _stream_ptr(q, stream)))
    return dq, dk, dv


def _ws_bytes(workspace, device):
    """Size in bytes of a caller's workspace, which must be a contiguous GPU
    tensor on the problem's device (the library checks the size)."""
    torch = _torch()
    if not workspace.is_cuda or workspace.device != torch.device(device) or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous GPU tensor on {device}; got one on {workspace.device}"
                         + ("" if workspace.is_contiguous() else ", not contiguous"))
    return workspace.numel() * workspace.element_size()


def _workspace(q, code, workspace):
    torch = _torch()
    B, H, n, d = q.shape
    need = attn_bwd_workspace_bytes(code, B, H, n, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    return workspace, _ws_bytes(workspace, q.device)


@_on_call_stream
def attn_bwd_rowdot(o, do, lse, workspace=None, stream=None):
    """Backward stage 1: D = rowsum(dO * O) and LSE*log2(e) into the workspace
    (returned)."""
    torch = _torch()
    _check_inputs(o, do)
    _check_lse(lse, o)
    B, H, n, d = o.shape
    code = _dtype_code(o)
    workspace, wsb = _workspace(o, code, workspace)
    with torch.cuda.device(o.device):
        st = load_library().attn_bwd_rowdot(code, B, H, n, d, o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                                            workspace.data_ptr(), wsb, _stream_ptr(o, stream))
    if st != 0:
        raise ExattnError("attn_bwd_rowdot", st, exattn_status_string(st))
    return workspace


@_on_call_stream
def attn_bwd_dkdv(q, k, v, do, lse, workspace, scale=None, window=-1, dk=None, dv=None, stream=None):
    """Backward stage 2: dK, dV (needs the workspace from attn_bwd_rowdot)."""
    torch = _torch()
    _check_inputs(q, k, v, do)
    _check_lse(lse, q)
    B, H, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dk = _out(dk, q.shape, q.dtype, q.device)
    dv = _out(dv, q.shape, q.dtype, q.device)
    with torch.cuda.device(q.device):
        st = load_library().attn_bwd_dkdv(_dtype_code(q), B, H, n, d, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          do.data_ptr(), lse.data_ptr(), scale, int(window), dk.data_ptr(),
                                          dv.data_ptr(), workspace.data_ptr(),
                                          _ws_bytes(workspace, q.device), _stream_ptr(q, stream))
    if st != 0:
        raise ExattnError("attn_bwd_dkdv", st, exattn_status_string(st))
    return dk, dv


@_on_call_stream
def attn_bwd_dq(q, k, v, do, lse, workspace, scale=None, window=-1, dq=None, stream=None):
    """Backward stage 3: dQ (needs the workspace from attn_bwd_rowdot)."""
    torch = _torch()
    _check_inputs(q, k, v, do)
    _check_lse(lse, q)
    B, H, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = _out(dq, q.shape, q.dtype, q.device)
    with torch.cuda.device(q.device):
        st = load_library().attn_bwd_dq(_dtype_code(q), B, H, n, d, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        do.data_ptr(), lse.data_ptr(), scale, int(window), dq.data_ptr(),
                                        workspace.data_ptr(), _ws_bytes(workspace, q.device),
                                        _stream_ptr(q, stream))
    if st != 0:
        raise ExattnError("attn_bwd_dq", st, exattn_status_string(st))
    return dq


# ---------------------------------------------------------------------------
# Grouped-query attention: K, V (and dK, dV) have Hkv heads, Hkv dividing H.
# ---------------------------------------------------------------------------

@_on_call_stream
def attn_fwd_gqa(q, k, v, scale=None, window=-1, out=None, lse=None, stream=None):
    """Forward with Hkv = k.shape[1] key/value heads shared by groups of
    H / Hkv consecutive query heads.  Returns (O like q, LSE float32 [B, H, n])."""
    torch = _torch()
    Hkv = _check_gqa(q, k, v)
    B, H, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = _out(out, q.shape, q.dtype, q.device)
    lse = _out(lse, (B, H, n), torch.float32, q.device)
    _call("attn_fwd_gqa", _dtype_code(q), B, H, Hkv, n, d, q.data_ptr(), k.data_ptr(), v.data_ptr(), scale,
          int(window), out.data_ptr(), lse.data_ptr(), (q.device, _stream_ptr(q, stream)))
    return out, lse


@_on_call_stream
def attn_bwd_gqa(q, k, v, o, do, lse, scale=None, window=-1, workspace=None, dq=None, dk=None, dv=None,
                 stream=None):
    """Backward of attn_fwd_gqa.  Returns (dQ like q, dK like k, dV like v);
    dK and dV sum over each group's query heads."""
    torch = _torch()
    Hkv = _check_gqa(q, k, v, o, do)
    _check_lse(lse, q)
    B, H, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    workspace, wsb = _workspace(q, code, workspace)
    dq = _out(dq, q.shape, q.dtype, q.device)
    dk = _out(dk, k.shape, k.dtype, k.device)
    dv = _out(dv, v.shape, v.dtype, v.device)
    _call("attn_bwd_gqa", code, B, H, Hkv, n, d, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
          do.data_ptr(), lse.data_ptr(), scale, int(window), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
          workspace.data_ptr(), wsb, (q.device, _stream_ptr(q, stream)))
    return dq, dk, dv


@_on_call_stream
def attn_bwd_dkdv_gqa(q, k, v, do, lse, workspace, scale=None, window=-1, dk=None, dv=None, stream=None):
    """Backward stage 2 with shared key/value heads: dK, dV like k, v."""
    torch = _torch()
    Hkv = _check_gqa(q, k, v, do)
    _check_lse(lse, q)
    B, H, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dk = _out(dk, k.shape, k.dtype, k.device)
    dv = _out(dv, v.shape, v.dtype, v.device)
    _call("attn_bwd_dkdv_gqa", _dtype_code(q), B, H, Hkv, n, d, q.data_ptr(), k.data_ptr(), v.data_ptr(),
          do.data_ptr(), lse.data_ptr(), scale, int(window), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
          _ws_bytes(workspace, q.device), (q.device, _stream_ptr(q, stream)))
    return dk, dv


@_on_call_stream
def attn_bwd_dq_gqa(q, k, v, do, lse, workspace, scale=None, window=-1, dq=None, stream=None):
    """Backward stage 3 with shared key/value heads: dQ like q."""
    torch = _torch()
    Hkv = _check_gqa(q, k, v, do)
    _check_lse(lse, q)
    B, H, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = _out(dq, q.shape, q.dtype, q.device)
    _call("attn_bwd_dq_gqa", _dtype_code(q), B, H, Hkv, n, d, q.data_ptr(), k.data_ptr(), v.data_ptr(),
          do.data_ptr(), lse.data_ptr(), scale, int(window), dq.data_ptr(), workspace.data_ptr(),
          _ws_bytes(workspace, q.device), (q.device, _stream_ptr(q, stream)))
    return dq


# ---------------------------------------------------------------------------
# Sparse patterns: window + global tokens + block layout
# ---------------------------------------------------------------------------

def attn_pattern_workspace_bytes(dtype_code, B, H, n, d):
    return int(load_library().attn_pattern_workspace_bytes(dtype_code, B, H, n, d))


def _pattern_workspace(q, workspace):
    torch = _torch()
    B, H, n, d = q.shape
    need = attn_pattern_workspace_bytes(_dtype_code(q), B, H, n, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    return workspace, _ws_bytes(workspace, q.device)


@_on_call_stream
def attn_fwd_pattern(q, k, v, pattern, scale=None, out=None, lse=None, workspace=None, stream=None):
    """Forward over a sparse pattern (AttnPattern).  Returns (O, LSE)."""
    torch = _torch()
    _check_inputs(q, k, v)
    B, H, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = _out(out, q.shape, q.dtype, q.device)
    lse = _out(lse, (B, H, n), torch.float32, q.device)
    workspace, wsb = _pattern_workspace(q, workspace)
    pc = pattern.as_c(n, q.device)
    _call("attn_fwd_pattern", _dtype_code(q), B, H, n, d, q.data_ptr(), k.data_ptr(), v.data_ptr(), scale,
          ctypes.byref(pc), out.data_ptr(), lse.data_ptr(), workspace.data_ptr(), wsb,
          (q.device, _stream_ptr(q, stream)))
    return out, lse


@_on_call_stream
def attn_bwd_pattern(q, k, v, o, do, lse, pattern, scale=None, workspace=None, dq=None, dk=None, dv=None,
                     stream=None):
    """Backward over a sparse pattern (AttnPattern).  Returns (dQ, dK, dV)."""
    torch = _torch()
    _check_inputs(q, k, v, o, do)
    _check_lse(lse, q)
    B, H, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    workspace, wsb = _pattern_workspace(q, workspace)
    dq = _out(dq, q.shape, q.dtype, q.device)
    dk = _out(dk, k.shape, k.dtype, k.device)
    dv = _out(dv, v.shape, v.dtype, v.device)
    pc = pattern.as_c(n, q.device)
    _call("attn_bwd_pattern", _dtype_code(q), B, H, n, d, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
          do.data_ptr(), lse.data_ptr(), scale, ctypes.byref(pc), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
          workspace.data_ptr(), wsb, (q.device, _stream_ptr(q, stream)))
    return dq, dk, dv


# ---------------------------------------------------------------------------
# FP8 (E4M3) forward and its quantiser
# ---------------------------------------------------------------------------

def attn_fp8_bytes(B, H, n, d, layout):
    return int(load_library().attn_fp8_bytes(B, H, n, d, layout))


@_on_call_stream
def attn_quant_fp8(x, signs=None, layout=EXATTN_FP8_ROWS, stream=None):
    """Quantise a bf16 [B, H, n, d] tensor to E4M3 codes (uint8 tensor in
    the requested layout) and per-head scales (float32 [B, H])."""
    torch = _torch()
    _check_inputs(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("attn_quant_fp8 takes bfloat16 input")
    B, H, n, d = x.shape
    if signs is not None and (signs.dtype != torch.float32 or signs.numel() != d or not signs.is_cuda
                              or signs.device != x.device or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous float32 tensor of d entries (+1 or -1) on x's GPU")
    x8 = torch.empty(max(attn_fp8_bytes(B, H, n, d, layout), 1), dtype=torch.uint8, device=x.device)
    scale = torch.empty((B, H), dtype=torch.float32, device=x.device)
    _call("attn_quant_fp8", B, H, n, d, x.data_ptr(), None if signs is None else signs.data_ptr(), int(layout),
          x8.data_ptr(), scale.data_ptr(), (x.device, _stream_ptr(x, stream)))
    return x8, scale


@_on_call_stream
def attn_fwd_fp8(q8, k8, v8t, q_scale, k_scale, v_scale, shape, scale=None, rotated=False, out=None, lse=None,
                 stream=None):
    """FP8 forward on quantised inputs (from attn_quant_fp8; V in the
    transposed layout).  `shape` = (B, H, n, d).  Returns (O bf16, LSE)."""
    torch = _torch()
    B, H, n, d = shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = _out(out, (B, H, n, d), torch.bfloat16, q8.device)
    lse = _out(lse, (B, H, n), torch.float32, q8.device)
    for t, lay in ((q8, EXATTN_FP8_ROWS), (k8, EXATTN_FP8_ROWS), (v8t, EXATTN_FP8_V_TRANSPOSED)):
        if (t.dtype != torch.uint8 or not t.is_cuda or t.device != q8.device or not t.is_contiguous()
                or t.numel() < attn_fp8_bytes(B, H, n, d, lay)):
            raise ValueError("FP8 inputs must be contiguous uint8 tensors of attn_fp8_bytes() bytes on one GPU")
    for t in (q_scale, k_scale, v_scale):
        if (t.dtype != torch.float32 or t.numel() != B * H or not t.is_cuda or t.device != q8.device
                or not t.is_contiguous()):
            raise ValueError("scales must be contiguous float32 tensors of B*H entries on the inputs' GPU")
    _call("attn_fwd_fp8", B, H, n, d, q8.data_ptr(), k8.data_ptr(), v8t.data_ptr(), q_scale.data_ptr(),
          k_scale.data_ptr(), v_scale.data_ptr(), scale, int(bool(rotated)), out.data_ptr(), lse.data_ptr(),
          (q8.device, _stream_ptr(q8, stream)))
    return out, lse
