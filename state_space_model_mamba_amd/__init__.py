"""Python binding of libssd, the MI355X (gfx950) Mamba-2 SSD prefill scan and
O(1) cached decode step.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libssd.so`` (C ABI in ``include/ssd.h``).  PyTorch provides device
memory and the stream.  There is no fallback: if the library is missing, or a
call fails, an exception is raised.

Functions keep the C names (each call also takes dt_softplus=True, dt_bias=[H]
to pass u instead of dt; the step size is then softplus(u + dt_bias) in the kernels):
    ssd_state_init(state, src=None)
    ssd_chunk_scan_workspace_size(...)
    ssd_chunk_scan(x, dt, A, B, C, D, chunk, initial_state=None, ...) -> (y, final_state)
    ssd_decode_step(x, dt, A, B, C, D, state, y=None) -> y
    ssd_decode_steps(x, dt, A, B, C, D, state, y=None) -> y   (S steps in one launch)
    ssd_chunk_scan_timed(...) -> (y, final_state, [(kernel, ms), ...])
    ssd_chunk_scan_noalloc(x, dt, A, B, C, D, chunk, ...) -> (y, final_state)  (no workspace)
    ssd_chunk_scan_varlen(x, dt, A, B, C, D, cu_seqlens, chunk, ...) -> (y, final_states)
    ssd_gdn_decode_step(q, k, v, g, beta, state, o=None) -> o   (Gated DeltaNet step)
    ssd_gdn_decode_steps(q, k, v, g, beta, state, o=None) -> o  (S steps in one launch)
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libssd.so")

SSD_F32, SSD_BF16 = 0, 1
SSD_DT_SOFTPLUS = 1            # ssd_dims.flags: dt holds u, the step size is softplus(u + dt_bias)
STATUS = {0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_UNSUPPORTED",
          4: "SSD_ERR_ALIAS", 5: "SSD_ERR_WORKSPACE", 6: "SSD_ERR_DEVICE", 7: "SSD_ERR_ALIGNMENT"}
EXPORTS = ("ssd_status_string", "ssd_version", "ssd_state_init", "ssd_chunk_scan_workspace_size",
           "ssd_chunk_scan", "ssd_decode_step", "ssd_decode_steps", "ssd_chunk_scan_timed",
           "ssd_chunk_scan_varlen_workspace_size", "ssd_chunk_scan_varlen",
           "ssd_gdn_decode_step", "ssd_gdn_decode_steps", "ssd_chunk_scan_noalloc")
NOALLOC_SCRATCH_BYTES = 96 << 20   # SSD_NOALLOC_SCRATCH_BYTES of include/ssd.h


class SsdError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {msg}")
        self.code = code


class SsdDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("dt_bias", ctypes.c_void_p)]


class SsdGdnDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("qk_heads", ctypes.c_int64),
                ("v_heads", ctypes.c_int64), ("dk", ctypes.c_int64), ("dv", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None


def load(path: str | None = None):
    """Load libssd.so (built in-tree by ``state_space_model_mamba_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIBRARY
    if not os.path.exists(p):
        raise RuntimeError(f"libssd not built: {p} is missing "
                           "(run `python -m state_space_model_mamba_amd.build`)")
    lib = ctypes.CDLL(p)
    vp, fp, i64p = ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)
    dims = ctypes.POINTER(SsdDims)
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_version.argtypes = []
    lib.ssd_version.restype = ctypes.c_int
    lib.ssd_state_init.argtypes = [dims, fp, fp, vp]
    lib.ssd_state_init.restype = ctypes.c_int
    lib.ssd_chunk_scan_workspace_size.argtypes = [dims, i64p]
    lib.ssd_chunk_scan_workspace_size.restype = ctypes.c_int
    lib.ssd_chunk_scan.argtypes = [dims] + [vp] * 10 + [ctypes.c_size_t, vp]
    lib.ssd_chunk_scan.restype = ctypes.c_int
    lib.ssd_chunk_scan_timed.argtypes = ([dims] + [vp] * 10 + [ctypes.c_size_t, vp] +
                                         [ctypes.POINTER(ctypes.c_float),
                                          ctypes.POINTER(ctypes.c_char_p),
                                          ctypes.POINTER(ctypes.c_int)])
    lib.ssd_chunk_scan_timed.restype = ctypes.c_int
    lib.ssd_chunk_scan_noalloc.argtypes = [dims] + [vp] * 10
    lib.ssd_chunk_scan_noalloc.restype = ctypes.c_int
    lib.ssd_decode_step.argtypes = [dims] + [vp] * 9
    lib.ssd_decode_step.restype = ctypes.c_int
    lib.ssd_decode_steps.argtypes = [dims, ctypes.c_int64] + [vp] * 9
    lib.ssd_decode_steps.restype = ctypes.c_int
    cu = ctypes.POINTER(ctypes.c_int64)
    lib.ssd_chunk_scan_varlen_workspace_size.argtypes = [dims, cu, i64p]
    lib.ssd_chunk_scan_varlen_workspace_size.restype = ctypes.c_int
    lib.ssd_chunk_scan_varlen.argtypes = [dims, cu] + [vp] * 10 + [ctypes.c_size_t, vp]
    lib.ssd_chunk_scan_varlen.restype = ctypes.c_int
    lib.ssd_gdn_decode_step.argtypes = [ctypes.POINTER(SsdGdnDims)] + [vp] * 8
    lib.ssd_gdn_decode_step.restype = ctypes.c_int
    lib.ssd_gdn_decode_steps.argtypes = [ctypes.POINTER(SsdGdnDims), ctypes.c_int64] + [vp] * 8
    lib.ssd_gdn_decode_steps.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _check(fn: str, rc: int):
    if rc != 0:
        msg = load().ssd_status_string(rc).decode()
        raise SsdError(fn, rc, msg)


def _ptr(t):
    """A tensor's device address as an int (ctypes passes it as void*), or NULL."""
    return None if t is None else t.data_ptr()


def _current_raw_stream(di):
    """The current stream's handle on device `di`, without building a Stream object."""
    get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    return get(di) if get is not None else torch.cuda.current_stream(di).cuda_stream


def _stream(stream, di):
    """hipStream_t of `stream`, or of device `di`'s current stream."""
    return _current_raw_stream(di) if stream is None else stream.cuda_stream


def _on(stream):
    """Allocation context of a call: the caller's stream when one is given (the
    current stream is the allocator's default otherwise), so that blocks
    allocated for the call are not handed to other work while its kernels run."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _io_dtype(t):
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    raise TypeError(f"x/B/C must be bfloat16 or float32, got {t.dtype}")


def _need(name, t, di, dtype=None, shape=None, optional=False):
    """Checks that a tensor argument can be handed to the kernels as a plain
    device pointer: a contiguous tensor on GPU `di` of the stated dtype and
    shape.  A host tensor would hand a host address to a kernel, and a strided
    view or a wrong dtype would be read as something else, so each raises here
    instead.  (One combined test on the common path: small decode calls are
    bound by host time.)"""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    try:
        ok = (t.get_device() == di and (dtype is None or t.dtype == dtype) and t.is_contiguous()
              and (shape is None or t.shape == shape))
    except AttributeError:
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}") from None
    if not ok:
        if t.get_device() != di:
            raise ValueError(f"{name} is on {t.device}, expected cuda:{di}")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _device_of(t):
    """The device index of the first tensor argument, which must be a GPU tensor."""
    di = t.get_device()
    if di < 0:
        raise ValueError(f"arguments must be device (HIP) tensors, got one on {t.device}")
    return di


def _bias_check(di, H, dt_softplus, dt_bias):
    if dt_softplus:
        _need("dt_bias", dt_bias, di, torch.float32, (H,), optional=True)


def make_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, io_dtype,
              dt_softplus=False, dt_bias=None) -> SsdDims:
    """ssd_dims; with dt_softplus the dt arguments hold u and the step size is
    softplus(u + dt_bias[h]) (dt_bias: a [H] fp32 device tensor or None)."""
    flags = SSD_DT_SOFTPLUS if dt_softplus else 0
    bias = dt_bias.data_ptr() if (dt_softplus and dt_bias is not None) else None
    return SsdDims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, io_dtype, flags, bias)


def ssd_chunk_scan_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                                  io_dtype=SSD_BF16) -> int:
    d = make_dims(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, io_dtype)
    n = ctypes.c_size_t(0)
    _check("ssd_chunk_scan_workspace_size",
           load().ssd_chunk_scan_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return int(n.value)


def ssd_state_init(state, src=None, stream=None):
    """state [B, H, P, N] fp32 <- src (or zeros)."""
    dev = _device_of(state)
    _need("state", state, dev, torch.float32)
    if state.dim() != 4:
        raise ValueError(f"state must be [B, H, P, N], got shape {tuple(state.shape)}")
    b, h, p, n = state.shape
    _need("src", src, dev, torch.float32, state.shape, optional=True)
    d = make_dims(b, 0, h, p, n, 1, 1, SSD_F32)
    _check("ssd_state_init", load().ssd_state_init(ctypes.byref(d), _ptr(state), _ptr(src),
                                                   _stream(stream, dev)))
    return state


def _scan_args(x, dt, A, B, C, D, chunk, initial_state, y, final_state, workspace,
               dt_softplus=False, dt_bias=None, stream=None, need_workspace=True):
    dev = _device_of(x)
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [B, L, H, P] and B, C [B, L, G, N]")
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = _io_dtype(x)
    f32 = torch.float32
    _need("x", x, dev, x.dtype)
    _need("dt", dt, dev, f32, (bsz, L, H))
    _need("A", A, dev, f32, (H,))
    _need("B", B, dev, x.dtype, (bsz, L, G, N))
    _need("C", C, dev, x.dtype, (bsz, L, G, N))
    _need("D", D, dev, f32, (H,))
    _need("initial_state", initial_state, dev, f32, (bsz, H, P, N), optional=True)
    _need("y", y, dev, x.dtype, x.shape, optional=True)
    _need("final_state", final_state, dev, f32, (bsz, H, P, N), optional=True)
    _need("workspace", workspace, dev, optional=True)
    _bias_check(dev, H, dt_softplus, dt_bias)
    d = make_dims(bsz, L, H, P, N, G, chunk, io, dt_softplus, dt_bias)
    need = ssd_chunk_scan_workspace_size(bsz, L, H, P, N, G, chunk, io) if need_workspace else 0
    # outputs and workspace come from the allocator on the call's own stream, so
    # that their blocks are not handed to other work while the kernels run
    with _on(stream):
        if y is None:
            y = torch.empty_like(x)
        if final_state is None:
            final_state = torch.empty((bsz, H, P, N), dtype=f32, device=dev)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(initial_state), _ptr(y), _ptr(final_state), _ptr(workspace), ws_bytes]
    return args, y, final_state, workspace


def ssd_chunk_scan(x, dt, A, B, C, D, chunk, initial_state=None, y=None, final_state=None,
                   workspace=None, stream=None, dt_softplus=False, dt_bias=None):
    """Prefill over x[B, L, H, P]; returns (y, final_state)."""
    args, y, fs, ws = _scan_args(x, dt, A, B, C, D, chunk, initial_state, y, final_state,
                                 workspace, dt_softplus, dt_bias, stream)
    _check("ssd_chunk_scan", load().ssd_chunk_scan(*args, _stream(stream, x.get_device())))
    return y, fs


def ssd_chunk_scan_noalloc(x, dt, A, B, C, D, chunk, initial_state=None, y=None,
                           final_state=None, stream=None, dt_softplus=False, dt_bias=None):
    """ssd_chunk_scan with the library's own per-device scratch array as its
    workspace (nothing is allocated by the library; pass y and final_state to
    allocate nothing here either).  Calls that overlap in time on one device
    race on the scratch array.  Returns (y, final_state)."""
    args, y, fs, _ = _scan_args(x, dt, A, B, C, D, chunk, initial_state, y, final_state, None,
                                dt_softplus, dt_bias, stream, need_workspace=False)
    _check("ssd_chunk_scan_noalloc",
           load().ssd_chunk_scan_noalloc(*args[:10], _stream(stream, x.get_device())))
    return y, fs


def ssd_chunk_scan_timed(x, dt, A, B, C, D, chunk, initial_state=None, y=None, final_state=None,
                         workspace=None, stream=None, dt_softplus=False, dt_bias=None):
    """As ssd_chunk_scan, synchronously, also returning [(kernel name, ms), ...]."""
    args, y, fs, ws = _scan_args(x, dt, A, B, C, D, chunk, initial_state, y, final_state,
                                 workspace, dt_softplus, dt_bias, stream)
    cap = 8
    ms = (ctypes.c_float * cap)()
    names = (ctypes.c_char_p * cap)()
    n = ctypes.c_int(cap)
    _check("ssd_chunk_scan_timed", load().ssd_chunk_scan_timed(
        *args, _stream(stream, x.get_device()), ms, names, ctypes.byref(n)))
    return y, fs, [(names[i].decode(), float(ms[i])) for i in range(n.value)]


def ssd_decode_step(x, dt, A, B, C, D, state, y=None, stream=None, dt_softplus=False,
                    dt_bias=None):
    """One decode step: x[B, H, P], B/C[B, G, N], state[B, H, P, N] updated in place; returns y."""
    dev = _device_of(x)
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError("x must be [B, H, P] and B, C [B, G, N]")
    bsz, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    f32 = torch.float32
    _need("x", x, dev, x.dtype)
    _need("dt", dt, dev, f32, (bsz, H))
    _need("A", A, dev, f32, (H,))
    _need("B", B, dev, x.dtype, (bsz, G, N))
    _need("C", C, dev, x.dtype, (bsz, G, N))
    _need("D", D, dev, f32, (H,))
    _need("state", state, dev, f32, (bsz, H, P, N))
    _need("y", y, dev, x.dtype, x.shape, optional=True)
    _bias_check(dev, H, dt_softplus, dt_bias)
    d = make_dims(bsz, 1, H, P, N, G, 1, _io_dtype(x), dt_softplus, dt_bias)
    if y is None:
        with _on(stream):
            y = torch.empty_like(x)
    _check("ssd_decode_step", load().ssd_decode_step(
        ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(state),
        _ptr(y), _stream(stream, dev)))
    return y


def ssd_decode_steps(x, dt, A, B, C, D, state, y=None, stream=None, dt_softplus=False,
                     dt_bias=None):
    """S decode steps in one launch: x[S, B, H, P], dt[S, B, H], B/C[S, B, G, N];
    state[B, H, P, N] updated in place (read and written once); returns y[S, B, H, P]."""
    dev = _device_of(x)
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [S, B, H, P] and B, C [S, B, G, N]")
    nsteps, bsz, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    f32 = torch.float32
    _need("x", x, dev, x.dtype)
    _need("dt", dt, dev, f32, (nsteps, bsz, H))
    _need("A", A, dev, f32, (H,))
    _need("B", B, dev, x.dtype, (nsteps, bsz, G, N))
    _need("C", C, dev, x.dtype, (nsteps, bsz, G, N))
    _need("D", D, dev, f32, (H,))
    _need("state", state, dev, f32, (bsz, H, P, N))
    _need("y", y, dev, x.dtype, x.shape, optional=True)
    _bias_check(dev, H, dt_softplus, dt_bias)
    d = make_dims(bsz, 1, H, P, N, G, 1, _io_dtype(x), dt_softplus, dt_bias)
    if y is None:
        with _on(stream):
            y = torch.empty_like(x)
    _check("ssd_decode_steps", load().ssd_decode_steps(
        ctypes.byref(d), ctypes.c_int64(nsteps), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
        _ptr(D), _ptr(state), _ptr(y), _stream(stream, dev)))
    return y


def _cu_array(cu_seqlens):
    import numpy as np
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    return cu, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def ssd_chunk_scan_varlen_workspace_size(cu_seqlens, nheads, headdim, dstate, ngroups, chunk,
                                         io_dtype=SSD_BF16) -> int:
    cu, cup = _cu_array(cu_seqlens)
    d = make_dims(len(cu) - 1, int(cu[-1]), nheads, headdim, dstate, ngroups, chunk, io_dtype)
    n = ctypes.c_size_t(0)
    _check("ssd_chunk_scan_varlen_workspace_size",
           load().ssd_chunk_scan_varlen_workspace_size(ctypes.byref(d), cup, ctypes.byref(n)))
    return int(n.value)


def ssd_chunk_scan_varlen(x, dt, A, B, C, D, cu_seqlens, chunk, initial_states=None, y=None,
                          final_states=None, workspace=None, stream=None, dt_softplus=False,
                          dt_bias=None):
    """Prefill of a packed batch: x[T, H, P], dt[T, H], B/C[T, G, N]; sequence i is
    tokens cu_seqlens[i] .. cu_seqlens[i+1]-1 (a host sequence of S + 1 offsets).
    Returns (y[T, H, P], final_states[S, H, P, N])."""
    dev = _device_of(x)
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError("x must be [T, H, P] and B, C [T, G, N]")
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    cu, cup = _cu_array(cu_seqlens)
    nseq = len(cu) - 1
    io = _io_dtype(x)
    f32 = torch.float32
    _need("x", x, dev, x.dtype)
    _need("dt", dt, dev, f32, (T, H))
    _need("A", A, dev, f32, (H,))
    _need("B", B, dev, x.dtype, (T, G, N))
    _need("C", C, dev, x.dtype, (T, G, N))
    _need("D", D, dev, f32, (H,))
    _need("initial_states", initial_states, dev, f32, (nseq, H, P, N), optional=True)
    _need("y", y, dev, x.dtype, x.shape, optional=True)
    _need("final_states", final_states, dev, f32, (nseq, H, P, N), optional=True)
    _need("workspace", workspace, dev, optional=True)
    _bias_check(dev, H, dt_softplus, dt_bias)
    d = make_dims(nseq, T, H, P, N, G, chunk, io, dt_softplus, dt_bias)
    need = ssd_chunk_scan_varlen_workspace_size(cu, H, P, N, G, chunk, io)
    with _on(stream):
        if y is None:
            y = torch.empty_like(x)
        if final_states is None:
            final_states = torch.empty((nseq, H, P, N), dtype=f32, device=dev)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("ssd_chunk_scan_varlen", load().ssd_chunk_scan_varlen(
        ctypes.byref(d), cup, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(initial_states), _ptr(y), _ptr(final_states), _ptr(workspace), ws_bytes,
        _stream(stream, dev)))
    return y, final_states


def ssd_gdn_decode_step(q, k, v, g, beta, state, o=None, stream=None):
    """One Gated DeltaNet decode step: q, k [B, Hk, dk], v [B, Hv, dv], g, beta [B, Hv]
    fp32, state [B, Hv, dk, dv] fp32 updated in place; returns o [B, Hv, dv]."""
    dev = _device_of(q)
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k must be [B, Hk, dk] and v [B, Hv, dv]")
    bsz, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    f32 = torch.float32
    _need("q", q, dev, q.dtype)
    _need("k", k, dev, q.dtype, q.shape)
    _need("v", v, dev, q.dtype)
    _need("g", g, dev, f32, (bsz, Hv))
    _need("beta", beta, dev, f32, (bsz, Hv))
    _need("state", state, dev, f32, (bsz, Hv, dk, dv))
    _need("o", o, dev, q.dtype, v.shape, optional=True)
    d = SsdGdnDims(bsz, Hk, Hv, dk, dv, _io_dtype(q), 0)
    if o is None:
        with _on(stream):
            o = torch.empty_like(v)
    _check("ssd_gdn_decode_step", load().ssd_gdn_decode_step(
        ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
        _stream(stream, dev)))
    return o


def ssd_gdn_decode_steps(q, k, v, g, beta, state, o=None, stream=None):
    """S Gated DeltaNet steps in one launch: q, k [S, B, Hk, dk], v [S, B, Hv, dv],
    g, beta [S, B, Hv]; state [B, Hv, dk, dv] read and written once; returns o [S, B, Hv, dv]."""
    dev = _device_of(q)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k must be [S, B, Hk, dk] and v [S, B, Hv, dv]")
    nsteps, bsz, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    f32 = torch.float32
    _need("q", q, dev, q.dtype)
    _need("k", k, dev, q.dtype, q.shape)
    _need("v", v, dev, q.dtype)
    _need("g", g, dev, f32, (nsteps, bsz, Hv))
    _need("beta", beta, dev, f32, (nsteps, bsz, Hv))
    _need("state", state, dev, f32, (bsz, Hv, dk, dv))
    _need("o", o, dev, q.dtype, v.shape, optional=True)
    d = SsdGdnDims(bsz, Hk, Hv, dk, dv, _io_dtype(q), 0)
    if o is None:
        with _on(stream):
            o = torch.empty_like(v)
    _check("ssd_gdn_decode_steps", load().ssd_gdn_decode_steps(
        ctypes.byref(d), ctypes.c_int64(nsteps), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(state), _ptr(o), _stream(stream, dev)))
    return o
