"""Exact scaled-dot-product attention on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of libfa.so (include/fa.h). Every step of
the computation runs in the library's HIP kernels; this module only checks
tensors, allocates outputs with torch on the GPU and passes raw pointers and
the current HIP stream. There is no CPU fallback: without the built library
or without a GPU the calls raise.

The C functions are re-exported under their own names (fa_fwd, fa_fwd_ws,
fa_fwd_workspace_bytes, fa_bwd, fa_bwd_timed, fa_bwd_noalloc,
fa_bwd_workspace_bytes, fa_row_softmax, fa_status_str, fa_abi_version),
taking plain ints for pointers. The tensor-level helpers
are forward(), backward(), row_softmax() and the autograd wrapper
FlashAttention / attention().
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # imported before libfa.so so the process shares torch's HIP runtime

__all__ = [
    "FA_BF16", "FA_F32", "FA_NO_MASK", "FA_CAUSAL_TOP_LEFT", "FA_CAUSAL_BOTTOM_RIGHT",
    "FAError", "library_path", "load_library",
    "fa_fwd", "fa_fwd_ws", "fa_fwd_workspace_bytes",
    "fa_bwd", "fa_bwd_timed", "fa_bwd_noalloc", "fa_bwd_workspace_bytes", "fa_row_softmax",
    "fa_status_str", "fa_abi_version",
    "forward", "backward", "row_softmax", "FlashAttention", "attention",
]

FA_BF16 = 0
FA_F32 = 1

# values of the `causal` argument
FA_NO_MASK = 0
FA_CAUSAL_TOP_LEFT = 1       # key j visible to query i iff j <= i
FA_CAUSAL_BOTTOM_RIGHT = 2   # key j visible to query i iff j <= i + n_k - n_q

_STATUS = {0: "FA_OK", 1: "FA_E_NULLPTR", 2: "FA_E_SHAPE", 3: "FA_E_DTYPE", 4: "FA_E_HEADDIM",
           5: "FA_E_SCALE", 6: "FA_E_WORKSPACE", 7: "FA_E_HIP", 8: "FA_E_CAUSAL", 9: "FA_E_SCRATCH",
           10: "FA_E_ALIGN"}
_ABI_VERSION = 5
# bytes of the library's static per-GPU scratch behind fa_bwd_noalloc
FA_BWD_NOALLOC_SCRATCH_BYTES = 16 << 20
_SIZE_MAX = (1 << 64) - 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({fa_status_str(status)})")


def library_path() -> str:
    return os.environ.get("FA_LIBRARY", os.path.join(_HERE, "libfa.so"))


def load_library():
    """Load libfa.so (built in-tree by exact_tiled_attention_29_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_tiled_attention_29_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp]
    lib.fa_fwd.restype = i32
    lib.fa_fwd_ws.argtypes = lib.fa_fwd.argtypes[:-1] + [vp, sz, vp]
    lib.fa_fwd_ws.restype = i32
    lib.fa_fwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.fa_fwd_workspace_bytes.restype = sz
    lib.fa_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                           i32, i32, i32, i32, i32, i32, i32, f32, vp, sz, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_timed.argtypes = lib.fa_bwd.argtypes + [vp]
    lib.fa_bwd_timed.restype = i32
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                   i32, i32, i32, i32, i32, i32, i32, f32, vp]
    lib.fa_bwd_noalloc.restype = i32
    lib.fa_row_softmax.argtypes = [vp, i32, ctypes.c_longlong, i32, f32, vp, vp, i32, vp]
    lib.fa_row_softmax.restype = i32
    lib.fa_status_str.argtypes = [i32]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i32
    if lib.fa_abi_version() != _ABI_VERSION:
        raise RuntimeError("libfa.so ABI version mismatch")
    _lib = lib
    return lib


# ---- C functions under their own names (pointers as ints) ----

def _i32(**values):
    """Sizes and codes cross the C ABI as 32-bit ints, which ctypes would
    wrap without a word (2**32 + 100 arrives as 100): refuse what does not
    fit."""
    for name, v in values.items():
        if not -(1 << 31) <= int(v) < (1 << 31):
            raise ValueError(f"{name}={v} does not fit the C ABI's 32-bit int")


def fa_fwd(q, k, v, o, o_dtype, lse, batch, heads, n_q, n_k, d, dtype, causal, scale, stream):
    _i32(o_dtype=o_dtype, batch=batch, heads=heads, n_q=n_q, n_k=n_k, d=d, dtype=dtype, causal=causal)
    return load_library().fa_fwd(q, k, v, o, o_dtype, lse, batch, heads, n_q, n_k, d, dtype,
                                 int(causal), float(scale), stream)


def fa_fwd_ws(q, k, v, o, o_dtype, lse, batch, heads, n_q, n_k, d, dtype, causal, scale,
              workspace, workspace_bytes, stream):
    _i32(o_dtype=o_dtype, batch=batch, heads=heads, n_q=n_q, n_k=n_k, d=d, dtype=dtype, causal=causal)
    return load_library().fa_fwd_ws(q, k, v, o, o_dtype, lse, batch, heads, n_q, n_k, d, dtype,
                                    int(causal), float(scale), workspace, workspace_bytes, stream)


def fa_fwd_workspace_bytes(batch, heads, n_q, n_k, d, dtype, causal):
    _i32(batch=batch, heads=heads, n_q=n_q, n_k=n_k, d=d, dtype=dtype, causal=causal)
    return load_library().fa_fwd_workspace_bytes(batch, heads, n_q, n_k, d, dtype, int(causal))


def fa_bwd(q, k, v, o, o_dtype, lse, d_o, dq, dk, dv, batch, heads, n_q, n_k, d, dtype, causal,
           scale, workspace, workspace_bytes, stream):
    _i32(o_dtype=o_dtype, batch=batch, heads=heads, n_q=n_q, n_k=n_k, d=d, dtype=dtype, causal=causal)
    return load_library().fa_bwd(q, k, v, o, o_dtype, lse, d_o, dq, dk, dv, batch, heads, n_q,
                                 n_k, d, dtype, int(causal), float(scale), workspace,
                                 workspace_bytes, stream)


def fa_bwd_timed(q, k, v, o, o_dtype, lse, d_o, dq, dk, dv, batch, heads, n_q, n_k, d, dtype,
                 causal, scale, workspace, workspace_bytes, stream, events):
    _i32(o_dtype=o_dtype, batch=batch, heads=heads, n_q=n_q, n_k=n_k, d=d, dtype=dtype, causal=causal)
    return load_library().fa_bwd_timed(q, k, v, o, o_dtype, lse, d_o, dq, dk, dv, batch, heads,
                                       n_q, n_k, d, dtype, int(causal), float(scale), workspace,
                                       workspace_bytes, stream, events)


def fa_bwd_noalloc(q, k, v, o, o_dtype, lse, d_o, dq, dk, dv, batch, heads, n_q, n_k, d, dtype,
                   causal, scale, stream):
    _i32(o_dtype=o_dtype, batch=batch, heads=heads, n_q=n_q, n_k=n_k, d=d, dtype=dtype, causal=causal)
    return load_library().fa_bwd_noalloc(q, k, v, o, o_dtype, lse, d_o, dq, dk, dv, batch, heads,
                                         n_q, n_k, d, dtype, int(causal), float(scale), stream)


def fa_row_softmax(x, dtype, rows, cols, scale, lse, y, y_dtype, stream):
    _i32(dtype=dtype, cols=cols, y_dtype=y_dtype)
    return load_library().fa_row_softmax(x, dtype, rows, cols, float(scale), lse, y, y_dtype, stream)


def fa_bwd_workspace_bytes(batch, heads, n_q, n_k, d, dtype, causal):
    _i32(batch=batch, heads=heads, n_q=n_q, n_k=n_k, d=d, dtype=dtype, causal=causal)
    return load_library().fa_bwd_workspace_bytes(batch, heads, n_q, n_k, d, dtype, int(causal))


def fa_status_str(status: int) -> str:
    try:
        return load_library().fa_status_str(status).decode()
    except RuntimeError:
        return _STATUS.get(status, "unknown")


def fa_abi_version() -> int:
    return load_library().fa_abi_version()


# ---- tensor-level helpers ----

def _code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return FA_BF16
    if dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {dtype}; expected bfloat16 or float32")


def _mask_code(causal) -> int:
    """The C `causal` value of False / True / "top_left" / "bottom_right"
    (or the ints 0, 1, 2 themselves)."""
    if isinstance(causal, str):
        codes = {"none": FA_NO_MASK, "top_left": FA_CAUSAL_TOP_LEFT,
                 "bottom_right": FA_CAUSAL_BOTTOM_RIGHT}
        if causal not in codes:
            raise ValueError(f"causal must be one of {sorted(codes)}, got {causal!r}")
        return codes[causal]
    return int(causal)


def _check(t: torch.Tensor, name: str, shape, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (the HIP kernels are the only implementation)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other tensors on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _event_handle(e) -> int:
    """hipEvent_t of a torch.cuda.Event (torch creates it on first record)."""
    if not e.cuda_event:
        e.record()
    return e.cuda_event


def forward(q, k, v, causal=False, scale=None, o_dtype=None, out=None, lse=None, split=True,
            workspace=None):
    """O, L = attention(q, k, v). q: [B,H,n_q,d]; k, v: [B,H,n_k,d].

    causal: False, True (= "top_left": key j visible to query i iff j <= i)
    or "bottom_right" (j <= i + n_k - n_q; a query that sees no key gets
    O = 0, L = -inf).

    o_dtype defaults to the input dtype; torch.float32 gives the unrounded
    fp32 O for bf16 inputs. Returns (O, L) with L fp32 [B,H,n_q].

    split: when the library asks for a workspace (grids with few query
    tiles, see fa_fwd_ws), let it split the keys over several workgroups,
    in `workspace` (a uint8 CUDA tensor of at least
    fa_fwd_workspace_bytes(...) bytes) or in one allocated here; False
    always calls fa_fwd.
    """
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    dt = _code(q.dtype)
    _check(q, "q", (B, H, n_q, d))
    dev = q.device
    _check(k, "k", (B, H, n_k, d), q.dtype, dev)
    _check(v, "v", (B, H, n_k, d), q.dtype, dev)
    o_dtype = q.dtype if o_dtype is None else o_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, n_q, d), dtype=o_dtype, device=q.device)
    _check(out, "out", (B, H, n_q, d), o_dtype, dev)
    if lse is None:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device)
    _check(lse, "lse", (B, H, n_q), torch.float32, dev)
    with torch.cuda.device(dev):   # kernels launch on the current device
        need = fa_fwd_workspace_bytes(B, H, n_q, n_k, d, dt, _mask_code(causal)) if split else 0
        if need == _SIZE_MAX:
            need = 0   # rejected arguments: fa_fwd reports why
        if need:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
            _check(workspace, "workspace", tuple(workspace.shape), None, dev)
            st = fa_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _code(o_dtype),
                           lse.data_ptr(), B, H, n_q, n_k, d, dt, _mask_code(causal), scale,
                           workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                           _stream(dev))
            where = "fa_fwd_ws"
        else:
            st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _code(o_dtype),
                        lse.data_ptr(), B, H, n_q, n_k, d, dt, _mask_code(causal), scale, _stream(dev))
            where = "fa_fwd"
    if st != 0:
        raise FAError(st, where)
    return out, lse


def backward(q, k, v, o, lse, do, causal=False, scale=None, workspace=None, grads=None,
             events=None):
    """dQ, dK, dV from the forward's O and L and the upstream gradient dO.

    events: optional 4 torch.cuda.Event(enable_timing=True), recorded on the
    current stream around the backward's three kernels (see fa_bwd_timed)."""
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    dt = _code(q.dtype)
    _check(q, "q", (B, H, n_q, d))
    dev = q.device
    _check(k, "k", (B, H, n_k, d), q.dtype, dev)
    _check(v, "v", (B, H, n_k, d), q.dtype, dev)
    _check(o, "o", (B, H, n_q, d), None, dev)
    _check(lse, "lse", (B, H, n_q), torch.float32, dev)
    _check(do, "do", (B, H, n_q, d), q.dtype, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mask = _mask_code(causal)
    with torch.cuda.device(dev):   # the split plan depends on this device's CU count
        need = fa_bwd_workspace_bytes(B, H, n_q, n_k, d, dt, mask)
    if need == _SIZE_MAX:    # arguments fa_bwd rejects: let it name the error
        need = 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    _check(dq, "dq", (B, H, n_q, d), q.dtype, dev)
    _check(dk, "dk", (B, H, n_k, d), q.dtype, dev)
    _check(dv, "dv", (B, H, n_k, d), q.dtype, dev)
    _check(workspace, "workspace", tuple(workspace.shape), None, dev)
    ev = None
    if events is not None:
        if len(events) != 4:
            raise ValueError("events must hold 4 torch.cuda.Event")
        ev = (ctypes.c_void_p * 4)(*[_event_handle(e) for e in events])
    with torch.cuda.device(dev):   # kernels launch on the current device
        st = fa_bwd_timed(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _code(o.dtype),
                          lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                          B, H, n_q, n_k, d, dt, mask, scale, workspace.data_ptr(),
                          workspace.numel() * workspace.element_size(), _stream(dev), ev)
    if st != 0:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv


def row_softmax(x, scale=1.0, softmax=True, y_dtype=None, lse=None, out=None):
    """Row logsumexp (and softmax) of scale * x over its last dimension.

    x: contiguous bf16 or fp32 GPU tensor of shape [..., cols]. Returns
    (y, lse): y the softmax rows in y_dtype (default x.dtype), or None when
    softmax=False; lse fp32 of shape x.shape[:-1] (natural log)."""
    if not isinstance(x, torch.Tensor) or x.dim() < 1:
        raise TypeError("x must be a tensor with at least one dimension")
    dt = _code(x.dtype)
    _check(x, "x", tuple(x.shape))
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    if lse is None:
        lse = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _check(lse, "lse", tuple(x.shape[:-1]), torch.float32, x.device)
    y = None
    ydt = FA_BF16
    if softmax:
        y_dtype = x.dtype if y_dtype is None else y_dtype
        ydt = _code(y_dtype)
        y = torch.empty(x.shape, dtype=y_dtype, device=x.device) if out is None else out
        _check(y, "out", tuple(x.shape), y_dtype, x.device)
    with torch.cuda.device(x.device):   # the kernel launches on the current device
        st = fa_row_softmax(x.data_ptr(), dt, rows, cols, scale, lse.data_ptr(),
                            y.data_ptr() if y is not None else None, ydt, _stream(x.device))
    if st != 0:
        raise FAError(st, "fa_row_softmax")
    return y, lse


class FlashAttention(torch.autograd.Function):
    """autograd wrapper: the forward saves only Q, K, V, O and L; the
    backward rebuilds P from L inside the kernels."""

    @staticmethod
    def forward(ctx, q, k, v, causal=False, scale=None):
        o, lse = forward(q, k, v, causal, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal = causal
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), ctx.causal, ctx.scale)
        return dq, dk, dv, None, None


def attention(q, k, v, causal=False, scale=None):
    return FlashAttention.apply(q, k, v, causal, scale)
