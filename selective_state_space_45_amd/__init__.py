"""Python binding of libselscan: the selective state-space scan on MI355X (gfx950).

Argument marshalling only: every step of the scan runs in the HIP kernels of
``libselscan.so`` (see ``include/selscan.h`` for the operation and its sources on
the reference pages).  PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libselscan.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libselscan.so not found at {LIB_PATH}; build it with "
        "`python -m selective_state_space_45_amd.build` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_lib.sscan_version.argtypes = []
_lib.sscan_version.restype = ctypes.c_int
_lib.sscan_last_error.argtypes = []
_lib.sscan_last_error.restype = ctypes.c_char_p
_lib.sscan_fwd_workspace_size.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_int]
_lib.sscan_fwd_workspace_size.restype = _SZ
_lib.sscan_fwd_segmented_workspace_size.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_int, _I64]
_lib.sscan_fwd_segmented_workspace_size.restype = _SZ
_U32 = ctypes.c_uint
_lib.sscan_fwd.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_int, _U32] + [_P] * 11 + [_P, _SZ, _P]
_lib.sscan_fwd.restype = ctypes.c_int
_lib.sscan_fwd_segmented.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_int, _U32] + [_P] * 11 + [_P, _SZ, _I64, _P]
_lib.sscan_fwd_segmented.restype = ctypes.c_int
_lib.sscan_fwd_noalloc.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_int, _U32] + [_P] * 11 + [_P]
_lib.sscan_fwd_noalloc.restype = ctypes.c_int
_lib.sscan_step.argtypes = [_I64, _I64, _I64, ctypes.c_int, _U32] + [_P] * 11
_lib.sscan_step.restype = ctypes.c_int
_lib.sscan_fwd_conv.argtypes = [_I64, _I64, _I64, _I64, _I64, ctypes.c_int, _U32] + [_P] * 15 + [_P, _SZ, _P]
_lib.sscan_fwd_conv.restype = ctypes.c_int
_lib.sscan_step_conv.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_int, _U32] + [_P] * 14
_lib.sscan_step_conv.restype = ctypes.c_int
_lib.sscan_bwd_workspace_size.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_int]
_lib.sscan_bwd_workspace_size.restype = _SZ
_lib.sscan_bwd.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_int, _U32] + [_P] * 21 + [_SZ, _P]
_lib.sscan_bwd.restype = ctypes.c_int
_lib.sscan_checkpoint_bytes.argtypes = [_I64, _I64, _I64, _I64]
_lib.sscan_checkpoint_bytes.restype = _SZ
_lib.sscan_fwd_checkpointed.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_int, _U32] + [_P] * 11 + [_P, _SZ, _P, _SZ, _P]
_lib.sscan_fwd_checkpointed.restype = ctypes.c_int
_lib.sscan_bwd_checkpointed_workspace_size.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_int]
_lib.sscan_bwd_checkpointed_workspace_size.restype = _SZ
_lib.sscan_bwd_checkpointed.argtypes = ([_I64, _I64, _I64, _I64, ctypes.c_int, _U32] + [_P] * 8 + [_P, _SZ] + [_P] * 11
                                        + [_P, _SZ, _P])
_lib.sscan_bwd_checkpointed.restype = ctypes.c_int

SSCAN_F32, SSCAN_BF16 = 0, 1
SSCAN_FLAG_EULER = 1
SSCAN_FLAG_STRUCTURED_A = 2
_DTYPES = {torch.float32: SSCAN_F32, torch.bfloat16: SSCAN_BF16}
STATUS = {0: "SSCAN_OK", 1: "SSCAN_ERR_INVALID_ARG", 2: "SSCAN_ERR_UNSUPPORTED", 3: "SSCAN_ERR_HIP"}


class SelScanError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def version() -> int:
    return int(_lib.sscan_version())


def last_error() -> str:
    return _lib.sscan_last_error().decode()


def library():
    """The loaded ctypes library (for callers that marshal pointers themselves)."""
    return _lib


def _check(rc: int):
    if rc != 0:
        raise SelScanError(rc, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def fwd_workspace_size(batch: int, seqlen: int, dim: int, dstate: int, dtype=torch.bfloat16,
                       num_segments: Optional[int] = None) -> int:
    """Workspace bytes for the automatic split, or for num_segments segments."""
    if num_segments is not None:
        return int(_lib.sscan_fwd_segmented_workspace_size(batch, seqlen, dim, dstate, _DTYPES[dtype], num_segments))
    return int(_lib.sscan_fwd_workspace_size(batch, seqlen, dim, dstate, _DTYPES[dtype]))


def sscan_fwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
              D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
              delta_bias: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
              return_last_state: bool = False, out: Optional[torch.Tensor] = None,
              last_state: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
              num_segments: Optional[int] = None, euler: bool = False,
              conv_w: Optional[torch.Tensor] = None, conv_b: Optional[torch.Tensor] = None,
              conv_state_in: Optional[torch.Tensor] = None, conv_state_out: Optional[torch.Tensor] = None,
              checkpoints: Optional[torch.Tensor] = None, structured_a: bool = False):
    """Forward selective scan.  x, delta, z: [batch, seqlen, dim]; B, C: [batch, seqlen, dstate]
    (all float32 or all bfloat16); A: [dim, dstate], D, delta_bias: [dim], initial_state:
    [batch, dim, dstate] (float32).  euler: Bbar = Delta B instead of the zero-order hold.
    conv_w [dim, dconv] (float32): x is the raw input of the fused causal depthwise
    convolution + SiLU prologue (conv_b [dim], conv_state_in / conv_state_out
    [batch, dim, dconv - 1], float32, optional).  checkpoints (a device buffer of at least
    ``checkpoint_bytes(...)`` bytes): also save the states that ``sscan_bwd(...,
    checkpoints=...)`` starts from.  structured_a: the caller states A[d, n] = c_d a_n
    (SSCAN_FLAG_STRUCTURED_A, a hint the library verifies).  Returns y, or (y, last_state)."""
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, dim]")
    batch, seqlen, dim = x.shape
    if x.dtype not in _DTYPES:
        raise ValueError("x must be float32 or bfloat16")
    dt = _DTYPES[x.dtype]
    dstate = A.shape[1] if A.dim() == 2 else -1
    _dev(x, "x")
    _dev(delta, "delta", x.dtype, x.shape)
    _dev(A, "A", torch.float32, (dim, dstate))
    _dev(B, "B", x.dtype, (batch, seqlen, dstate))
    _dev(C, "C", x.dtype, (batch, seqlen, dstate))
    if D is not None:
        _dev(D, "D", torch.float32, (dim,))
    if z is not None:
        _dev(z, "z", x.dtype, x.shape)
    if delta_bias is not None:
        _dev(delta_bias, "delta_bias", torch.float32, (dim,))
    if initial_state is not None:
        _dev(initial_state, "initial_state", torch.float32, (batch, dim, dstate))
    y = out if out is not None else torch.empty_like(x)
    _dev(y, "out", x.dtype, x.shape)
    ls = last_state
    if ls is None and return_last_state:
        ls = torch.empty((batch, dim, dstate), dtype=torch.float32, device=x.device)
    if ls is not None:
        _dev(ls, "last_state", torch.float32, (batch, dim, dstate))
    if workspace is None:
        need = fwd_workspace_size(batch, seqlen, dim, dstate, x.dtype, num_segments)
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device) if need > 0 else None
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    flags = (SSCAN_FLAG_EULER if euler else 0) | (SSCAN_FLAG_STRUCTURED_A if structured_a else 0)
    args = [batch, seqlen, dim, dstate, dt, flags, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), _ptr(initial_state), _ptr(y), _ptr(ls), _ptr(workspace), wbytes]
    if conv_w is not None:
        if num_segments is not None:
            raise ValueError("num_segments is not available with the convolution prologue")
        if checkpoints is not None:
            raise ValueError("checkpoints are not available with the convolution prologue")
        dconv = conv_w.shape[1] if conv_w.dim() == 2 else -1
        _dev(conv_w, "conv_w", torch.float32, (dim, dconv))
        if conv_b is not None:
            _dev(conv_b, "conv_b", torch.float32, (dim,))
        for t, name in ((conv_state_in, "conv_state_in"), (conv_state_out, "conv_state_out")):
            if t is not None:
                _dev(t, name, torch.float32, (batch, dim, dconv - 1))
        cargs = [batch, seqlen, dim, dstate, dconv, dt, flags, _ptr(x), _ptr(conv_w), _ptr(conv_b),
                 _ptr(conv_state_in), _ptr(conv_state_out)] + args[7:]
        _check(_lib.sscan_fwd_conv(*cargs, _stream(x.device)))
    elif checkpoints is not None:
        if num_segments is not None:
            raise ValueError("num_segments is not available with checkpoints")
        _dev(checkpoints, "checkpoints")
        _check(_lib.sscan_fwd_checkpointed(*args, _ptr(checkpoints),
                                           checkpoints.numel() * checkpoints.element_size(), _stream(x.device)))
    elif num_segments is None:
        _check(_lib.sscan_fwd(*args, _stream(x.device)))
    else:
        _check(_lib.sscan_fwd_segmented(*args, int(num_segments), _stream(x.device)))
    if return_last_state:
        return y, ls
    return y


def sscan_fwd_noalloc(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                      D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                      delta_bias: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, last_state: Optional[torch.Tensor] = None,
                      euler: bool = False) -> torch.Tensor:
    """``sscan_fwd`` for callers that cannot allocate: the library's static device
    scratch replaces the workspace.  ``out`` (and ``last_state`` if wanted) must be
    given, so this call allocates nothing either.  Returns ``out``."""
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, dim]")
    if out is None:
        raise ValueError("out is required (the no-allocation path allocates nothing)")
    batch, seqlen, dim = x.shape
    if x.dtype not in _DTYPES:
        raise ValueError("x must be float32 or bfloat16")
    dstate = A.shape[1] if A.dim() == 2 else -1
    _dev(x, "x")
    _dev(delta, "delta", x.dtype, x.shape)
    _dev(A, "A", torch.float32, (dim, dstate))
    _dev(B, "B", x.dtype, (batch, seqlen, dstate))
    _dev(C, "C", x.dtype, (batch, seqlen, dstate))
    for t, name, shape in ((D, "D", (dim,)), (delta_bias, "delta_bias", (dim,)),
                           (initial_state, "initial_state", (batch, dim, dstate)),
                           (last_state, "last_state", (batch, dim, dstate))):
        if t is not None:
            _dev(t, name, torch.float32, shape)
    if z is not None:
        _dev(z, "z", x.dtype, x.shape)
    _dev(out, "out", x.dtype, x.shape)
    flags = SSCAN_FLAG_EULER if euler else 0
    _check(_lib.sscan_fwd_noalloc(batch, seqlen, dim, dstate, _DTYPES[x.dtype], flags, _ptr(x), _ptr(delta),
                                  _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                  _ptr(initial_state), _ptr(out), _ptr(last_state), _stream(x.device)))
    return out


def sscan_step(state: torch.Tensor, x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
               C: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
               delta_bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               euler: bool = False, conv_w: Optional[torch.Tensor] = None, conv_b: Optional[torch.Tensor] = None,
               conv_state: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step.  state: [batch, dim, dstate] float32, updated in place; x, delta, z:
    [batch, dim]; B, C: [batch, dstate] (float32 or bfloat16); A: [dim, dstate].  euler: Bbar =
    Delta B instead of the zero-order hold.  conv_w [dim, dconv]: x is a raw input of the
    convolution prologue whose cache conv_state [batch, dim, dconv - 1] (float32) is
    updated in place.  Returns y [batch, dim]."""
    if x.dim() != 2:
        raise ValueError("x must be [batch, dim]")
    batch, dim = x.shape
    if x.dtype not in _DTYPES:
        raise ValueError("x must be float32 or bfloat16")
    dstate = A.shape[1] if A.dim() == 2 else -1
    _dev(state, "state", torch.float32, (batch, dim, dstate))
    _dev(x, "x")
    _dev(delta, "delta", x.dtype, x.shape)
    _dev(A, "A", torch.float32, (dim, dstate))
    _dev(B, "B", x.dtype, (batch, dstate))
    _dev(C, "C", x.dtype, (batch, dstate))
    if D is not None:
        _dev(D, "D", torch.float32, (dim,))
    if z is not None:
        _dev(z, "z", x.dtype, x.shape)
    if delta_bias is not None:
        _dev(delta_bias, "delta_bias", torch.float32, (dim,))
    y = out if out is not None else torch.empty_like(x)
    _dev(y, "out", x.dtype, x.shape)
    flags = SSCAN_FLAG_EULER if euler else 0
    if conv_w is not None:
        dconv = conv_w.shape[1] if conv_w.dim() == 2 else -1
        _dev(conv_w, "conv_w", torch.float32, (dim, dconv))
        if conv_b is not None:
            _dev(conv_b, "conv_b", torch.float32, (dim,))
        if conv_state is not None:
            _dev(conv_state, "conv_state", torch.float32, (batch, dim, dconv - 1))
        _check(_lib.sscan_step_conv(batch, dim, dstate, dconv, _DTYPES[x.dtype], flags, _ptr(state),
                                    _ptr(conv_state), _ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(delta), _ptr(A),
                                    _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(y),
                                    _stream(x.device)))
        return y
    _check(_lib.sscan_step(batch, dim, dstate, _DTYPES[x.dtype], flags, _ptr(state), _ptr(x), _ptr(delta),
                           _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(y),
                           _stream(x.device)))
    return y


def bwd_workspace_size(batch: int, seqlen: int, dim: int, dstate: int, dtype=torch.bfloat16,
                       checkpointed: bool = False) -> int:
    fn = _lib.sscan_bwd_checkpointed_workspace_size if checkpointed else _lib.sscan_bwd_workspace_size
    return int(fn(batch, seqlen, dim, dstate, _DTYPES[dtype]))


def checkpoint_bytes(batch: int, seqlen: int, dim: int, dstate: int) -> int:
    """Bytes of the checkpoint buffer for ``sscan_fwd(..., checkpoints=...)`` and
    ``sscan_bwd(..., checkpoints=...)``: the state entering every 8 timesteps,
    [batch, ceil(seqlen / 8), dstate, dim] float32."""
    return int(_lib.sscan_checkpoint_bytes(batch, seqlen, dim, dstate))


def sscan_bwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
              dy: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
              delta_bias: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
              dlast_state: Optional[torch.Tensor] = None, euler: bool = False,
              want_ddelta_bias: bool = True, want_dinitial_state: bool = True,
              workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
              checkpoints: Optional[torch.Tensor] = None) -> dict:
    """Backward pass of ``sscan_fwd``: gradients of a scalar loss given dy = dLoss/dy
    (same shape and dtype as x) and optionally dlast_state = dLoss/d(last state).
    Returns a dict with dx, ddelta, dA, dB, dC and, as applicable, dD, dz,
    ddelta_bias, dinitial_state (``out`` may supply preallocated tensors by name).
    checkpoints: the buffer ``sscan_fwd(..., checkpoints=...)`` filled for the same
    inputs; the forward recurrence is then not run again (initial_state then enters
    through the checkpoints and is not needed)."""
    if x.dim() != 3:
        raise ValueError("x must be [batch, seqlen, dim]")
    batch, seqlen, dim = x.shape
    if x.dtype not in _DTYPES:
        raise ValueError("x must be float32 or bfloat16")
    dstate = A.shape[1] if A.dim() == 2 else -1
    _dev(x, "x")
    _dev(delta, "delta", x.dtype, x.shape)
    _dev(dy, "dy", x.dtype, x.shape)
    _dev(A, "A", torch.float32, (dim, dstate))
    _dev(B, "B", x.dtype, (batch, seqlen, dstate))
    _dev(C, "C", x.dtype, (batch, seqlen, dstate))
    for t, name, shape in ((D, "D", (dim,)), (delta_bias, "delta_bias", (dim,)),
                           (initial_state, "initial_state", (batch, dim, dstate)),
                           (dlast_state, "dlast_state", (batch, dim, dstate))):
        if t is not None:
            _dev(t, name, torch.float32, shape)
    if z is not None:
        _dev(z, "z", x.dtype, x.shape)
    out = dict(out or {})
    dev = x.device

    def get(name, shape, dtype):
        t = out.get(name)
        if t is None:
            t = torch.empty(shape, dtype=dtype, device=dev)
            out[name] = t
        return _dev(t, name, dtype, shape)

    dx = get("dx", x.shape, x.dtype)
    ddelta = get("ddelta", x.shape, x.dtype)
    dA = get("dA", (dim, dstate), torch.float32)
    dB = get("dB", (batch, seqlen, dstate), x.dtype)
    dC = get("dC", (batch, seqlen, dstate), x.dtype)
    dD = get("dD", (dim,), torch.float32) if D is not None else None
    dz = get("dz", x.shape, x.dtype) if z is not None else None
    dbias = get("ddelta_bias", (dim,), torch.float32) if want_ddelta_bias else None
    dh0 = get("dinitial_state", (batch, dim, dstate), torch.float32) if want_dinitial_state else None
    need = bwd_workspace_size(batch, seqlen, dim, dstate, x.dtype, checkpointed=checkpoints is not None)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    wbytes = workspace.numel() * workspace.element_size()
    flags = SSCAN_FLAG_EULER if euler else 0
    if checkpoints is not None:
        _dev(checkpoints, "checkpoints")
        _check(_lib.sscan_bwd_checkpointed(
            batch, seqlen, dim, dstate, _DTYPES[x.dtype], flags, _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
            _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(checkpoints), checkpoints.numel() * checkpoints.element_size(),
            _ptr(dy), _ptr(dlast_state), _ptr(dx), _ptr(ddelta), _ptr(dA), _ptr(dB), _ptr(dC), _ptr(dD), _ptr(dz),
            _ptr(dbias), _ptr(dh0), _ptr(workspace), wbytes, _stream(dev)))
        return out
    _check(_lib.sscan_bwd(batch, seqlen, dim, dstate, _DTYPES[x.dtype], flags, _ptr(x), _ptr(delta), _ptr(A),
                          _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(initial_state), _ptr(dy),
                          _ptr(dlast_state), _ptr(dx), _ptr(ddelta), _ptr(dA), _ptr(dB), _ptr(dC), _ptr(dD),
                          _ptr(dz), _ptr(dbias), _ptr(dh0), _ptr(workspace), wbytes, _stream(dev)))
    return out
