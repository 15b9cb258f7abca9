"""Python binding of the C-ABI library libssm_hip.so (argument marshalling only).

Every function here checks tensor devices, dtypes, shapes and contiguity,
allocates the outputs it is not given, and passes raw device pointers plus
torch's current HIP stream to the library.  All arithmetic runs in the HIP
kernels; if the library is missing this module raises instead of computing
anything itself.

Names and semantics mirror include/ssm.h.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssm_hip.so")

SSM_OK = 0
SSM_ERR_NULL_ARG = 1
SSM_ERR_BAD_SHAPE = 2
SSM_ERR_BAD_DTYPE = 3
SSM_ERR_UNSUPPORTED = 4
SSM_ERR_ALIAS = 5
SSM_ERR_WORKSPACE = 6
SSM_ERR_HIP = 7
SSM_ERR_ALIGN = 8
SSM_F32 = 0
SSM_BF16 = 1
MAX_DSTATE = 16
MAX_CONV_K = 4

EXPORTED_SYMBOLS = ("ssm_selective_scan_workspace_size", "ssm_selective_scan_fwd",
                    "ssm_causal_conv1d_silu", "ssm_state_update", "ssm_status_string",
                    "ssm_last_error_message", "ssm_abi_version",
                    "ssm_selective_scan_bwd_workspace_size", "ssm_selective_scan_bwd",
                    "ssm_block_plan_create", "ssm_block_workspace_size", "ssm_block_fwd",
                    "ssm_block_plan_destroy", "ssm_ssd_fwd", "ssm_ssd_workspace_size",
                    "ssm_ssd_step", "ssm_selective_scan_fwd_noalloc")
NOALLOC_SCRATCH_BYTES = 32 << 20

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


class ScanArgs(ctypes.Structure):
    """Mirror of ssm_scan_args_t."""
    _fields_ = [("batch", _I64), ("seqlen", _I64), ("dim", _I64), ("dstate", _I64),
                ("io_dtype", _I32), ("delta_softplus", _I32), ("conv_k", _I64),
                ("x", _P), ("delta", _P), ("Bm", _P), ("Cm", _P), ("z", _P),
                ("A", _P), ("Dskip", _P), ("delta_bias", _P), ("conv_w", _P), ("conv_b", _P),
                ("h0", _P), ("y", _P), ("h_final", _P),
                ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
                ("conv_state_in", _P), ("conv_state_out", _P), ("checkpoints", _P)]


class StateUpdateArgs(ctypes.Structure):
    """Mirror of ssm_state_update_args_t."""
    _fields_ = [("batch", _I64), ("dim", _I64), ("dstate", _I64),
                ("io_dtype", _I32), ("delta_softplus", _I32),
                ("state", _P), ("x", _P), ("delta", _P), ("z", _P), ("Bm", _P), ("Cm", _P),
                ("A", _P), ("Dskip", _P), ("delta_bias", _P), ("y", _P),
                ("conv_k", _I64), ("conv_w", _P), ("conv_b", _P), ("conv_state", _P)]


class ScanBwdArgs(ctypes.Structure):
    """Mirror of ssm_scan_bwd_args_t."""
    _fields_ = [("batch", _I64), ("seqlen", _I64), ("dim", _I64), ("dstate", _I64),
                ("io_dtype", _I32), ("delta_softplus", _I32), ("conv_k", _I64),
                ("x", _P), ("delta", _P), ("Bm", _P), ("Cm", _P), ("z", _P),
                ("A", _P), ("Dskip", _P), ("delta_bias", _P), ("conv_w", _P), ("conv_b", _P),
                ("h0", _P), ("dy", _P), ("dh_final", _P),
                ("dx", _P), ("ddelta", _P), ("dz", _P), ("dA", _P), ("dBm", _P), ("dCm", _P),
                ("dDskip", _P), ("ddelta_bias", _P), ("dconv_w", _P), ("dconv_b", _P),
                ("dh0", _P), ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
                ("conv_state_in", _P), ("dconv_state_in", _P), ("checkpoints", _P)]


class BlockDims(ctypes.Structure):
    """Mirror of ssm_block_dims_t."""
    _fields_ = [("batch", _I64), ("seqlen", _I64), ("d_model", _I64), ("d_inner", _I64),
                ("dstate", _I64), ("dt_rank", _I64), ("conv_k", _I64)]


class BlockWeights(ctypes.Structure):
    """Mirror of ssm_block_weights_t."""
    _fields_ = [("norm_w", _P), ("w_in", _P), ("conv_w", _P), ("conv_b", _P), ("w_x", _P),
                ("w_dt", _P), ("dt_bias", _P), ("A", _P), ("Dskip", _P), ("w_out", _P),
                ("norm_eps", ctypes.c_float)]


class SsdArgs(ctypes.Structure):
    """Mirror of ssm_ssd_args_t."""
    _fields_ = [("batch", _I64), ("seqlen", _I64), ("nheads", _I64), ("headdim", _I64),
                ("ngroups", _I64), ("dstate", _I64), ("io_dtype", _I32), ("delta_softplus", _I32),
                ("x", _P), ("delta", _P), ("A", _P), ("Bm", _P), ("Cm", _P), ("Dskip", _P),
                ("z", _P), ("delta_bias", _P), ("h0", _P), ("y", _P), ("h_final", _P),
                ("workspace", _P), ("workspace_bytes", ctypes.c_size_t)]


class SsdStepArgs(ctypes.Structure):
    """Mirror of ssm_ssd_step_args_t."""
    _fields_ = [("batch", _I64), ("nheads", _I64), ("headdim", _I64), ("ngroups", _I64),
                ("dstate", _I64), ("io_dtype", _I32), ("delta_softplus", _I32), ("state", _P),
                ("x", _P), ("delta", _P), ("A", _P), ("Bm", _P), ("Cm", _P), ("Dskip", _P),
                ("z", _P), ("delta_bias", _P), ("y", _P)]


class SSMError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libssm_hip.so (built by selective_state_space_59_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libssm_hip.so is not built; run "
                               "`python -m selective_state_space_59_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        L.ssm_selective_scan_workspace_size.argtypes = [ctypes.POINTER(ScanArgs)]
        L.ssm_selective_scan_workspace_size.restype = ctypes.c_size_t
        L.ssm_selective_scan_fwd.argtypes = [ctypes.POINTER(ScanArgs), _P]
        L.ssm_selective_scan_fwd.restype = ctypes.c_int
        L.ssm_selective_scan_fwd_noalloc.argtypes = [ctypes.POINTER(ScanArgs), _P]
        L.ssm_selective_scan_fwd_noalloc.restype = ctypes.c_int
        L.ssm_causal_conv1d_silu.argtypes = [_I64, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P]
        L.ssm_causal_conv1d_silu.restype = ctypes.c_int
        L.ssm_state_update.argtypes = [ctypes.POINTER(StateUpdateArgs), _P]
        L.ssm_state_update.restype = ctypes.c_int
        L.ssm_status_string.argtypes = [ctypes.c_int]
        L.ssm_status_string.restype = ctypes.c_char_p
        L.ssm_last_error_message.argtypes = []
        L.ssm_last_error_message.restype = ctypes.c_char_p
        L.ssm_abi_version.argtypes = []
        L.ssm_abi_version.restype = ctypes.c_int
        L.ssm_selective_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(ScanBwdArgs)]
        L.ssm_selective_scan_bwd_workspace_size.restype = ctypes.c_size_t
        L.ssm_selective_scan_bwd.argtypes = [ctypes.POINTER(ScanBwdArgs), _P]
        L.ssm_selective_scan_bwd.restype = ctypes.c_int
        L.ssm_block_plan_create.argtypes = [ctypes.POINTER(BlockDims), ctypes.POINTER(_P)]
        L.ssm_block_plan_create.restype = ctypes.c_int
        L.ssm_block_workspace_size.argtypes = [_P]
        L.ssm_block_workspace_size.restype = ctypes.c_size_t
        L.ssm_block_fwd.argtypes = [_P, ctypes.POINTER(BlockWeights), _P, _P, _P, ctypes.c_size_t, _P]
        L.ssm_block_fwd.restype = ctypes.c_int
        L.ssm_block_plan_destroy.argtypes = [_P]
        L.ssm_block_plan_destroy.restype = None
        L.ssm_ssd_fwd.argtypes = [ctypes.POINTER(SsdArgs), _P]
        L.ssm_ssd_fwd.restype = ctypes.c_int
        L.ssm_ssd_workspace_size.argtypes = [ctypes.POINTER(SsdArgs)]
        L.ssm_ssd_step.argtypes = [ctypes.POINTER(SsdStepArgs), _P]
        L.ssm_ssd_step.restype = ctypes.c_int
        L.ssm_ssd_workspace_size.restype = ctypes.c_size_t
        _lib = L
    return _lib


def abi_version() -> int:
    return lib().ssm_abi_version()


def status_string(status: int) -> str:
    return lib().ssm_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != SSM_OK:
        msg = lib().ssm_last_error_message().decode()
        raise SSMError(status, "%s failed: %s (%s)" % (what, status_string(status), msg))


def _io_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return SSM_BF16
    if dtype == torch.float32:
        return SSM_F32
    raise TypeError("I/O tensors must be bfloat16 or float32, got %s" % dtype)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _req(t, name, shape, dtype, device):
    if t is None:
        raise ValueError("%s is required" % name)
    return _opt(t, name, shape, dtype, device)


def _opt(t, name, shape, dtype, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _scan_args(x, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, conv_w, conv_b, h0,
               y, h_final, conv_state_in=None, conv_state_out=None, checkpoints=None):
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a (B, L, D) tensor")
    if x.device.type != "cuda":
        raise ValueError("x must be on a GPU")
    dev = x.device
    Bsz, L, D = x.shape
    if not isinstance(A, torch.Tensor) or A.dim() != 2:
        raise ValueError("A must be a (D, N) float32 tensor")
    N = A.shape[1]
    io = x.dtype
    _req(x, "x", (Bsz, L, D), io, dev)
    _req(delta, "delta", (Bsz, L, D), io, dev)
    _req(A, "A", (D, N), torch.float32, dev)
    _req(Bm, "Bm", (Bsz, L, N), io, dev)
    _req(Cm, "Cm", (Bsz, L, N), io, dev)
    _opt(z, "z", (Bsz, L, D), io, dev)
    _opt(Dskip, "Dskip", (D,), torch.float32, dev)
    _opt(delta_bias, "delta_bias", (D,), torch.float32, dev)
    K = 0
    if conv_w is not None:
        if conv_w.dim() != 2:
            raise ValueError("conv_w must be (D, K)")
        K = conv_w.shape[1]
        _req(conv_w, "conv_w", (D, K), torch.float32, dev)
    _opt(conv_b, "conv_b", (D,), torch.float32, dev)
    _opt(h0, "h0", (Bsz, D, N), torch.float32, dev)
    _req(y, "y", (Bsz, L, D), io, dev)
    _opt(h_final, "h_final", (Bsz, D, N), torch.float32, dev)
    if (conv_state_in is not None or conv_state_out is not None) and K == 0:
        raise ValueError("a conv state needs conv_w")
    _opt(conv_state_in, "conv_state_in", (Bsz, max(K - 1, 0), D), io, dev)
    _opt(conv_state_out, "conv_state_out", (Bsz, max(K - 1, 0), D), io, dev)
    _opt(checkpoints, "checkpoints", checkpoint_shape(Bsz, L, D), torch.float32, dev)
    a = ScanArgs(batch=Bsz, seqlen=L, dim=D, dstate=N, io_dtype=_io_code(io),
                 delta_softplus=int(bool(delta_softplus)), conv_k=K,
                 x=_ptr(x), delta=_ptr(delta), Bm=_ptr(Bm), Cm=_ptr(Cm), z=_ptr(z), A=_ptr(A),
                 Dskip=_ptr(Dskip), delta_bias=_ptr(delta_bias), conv_w=_ptr(conv_w),
                 conv_b=_ptr(conv_b), h0=_ptr(h0), y=_ptr(y), h_final=_ptr(h_final),
                 workspace=None, workspace_bytes=0, conv_state_in=_ptr(conv_state_in),
                 conv_state_out=_ptr(conv_state_out), checkpoints=_ptr(checkpoints))
    return a, dev


SCAN_BLOCK = 16  # SSM_SCAN_BLOCK
MAX_DSTATE = 16  # SSM_MAX_DSTATE


def checkpoint_shape(batch: int, seqlen: int, dim: int) -> tuple:
    """Shape of the fp32 checkpoint tensor a forward writes for the backward: the state
    entering every SCAN_BLOCK-step block, (ceil(L / SCAN_BLOCK), B, D, MAX_DSTATE)."""
    return ((seqlen + SCAN_BLOCK - 1) // SCAN_BLOCK, batch, dim, MAX_DSTATE)


_ws_cache = {}


def _workspace(dev: torch.device, nbytes: int) -> torch.Tensor:
    """Cached scratch tensor per device and stream (grown on demand).  Calls on one stream
    run in order and share it; calls on different streams get different ones.

    A call made while the current stream is being captured into a HIP graph gets a fresh
    tensor of its own instead: every capture without an explicit stream runs on the same
    side stream, and two graphs that recorded one cached buffer would race on it when
    replayed at the same time.  The graph's memory pool keeps that tensor alive."""
    if torch.cuda.is_current_stream_capturing():
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    key = (dev.type, dev.index, torch.cuda.current_stream(dev).cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf


def selective_scan_workspace_size(x, delta, A, Bm, Cm, Dskip=None, z=None, delta_bias=None,
                                  delta_softplus=False, conv_w=None, conv_b=None, h0=None,
                                  return_final_state=False) -> int:
    y = torch.empty_like(x)
    hf = (torch.empty(x.shape[0], x.shape[2], A.shape[1], device=x.device, dtype=torch.float32)
          if return_final_state else None)
    a, _ = _scan_args(x, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, conv_w, conv_b,
                      h0, y, hf)
    n = lib().ssm_selective_scan_workspace_size(ctypes.byref(a))
    if n == ctypes.c_size_t(-1).value:
        raise SSMError(SSM_ERR_BAD_SHAPE, "invalid sizes")
    return int(n)


def selective_scan_fwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                       Cm: torch.Tensor, Dskip: Optional[torch.Tensor] = None,
                       z: Optional[torch.Tensor] = None,
                       delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
                       conv_w: Optional[torch.Tensor] = None,
                       conv_b: Optional[torch.Tensor] = None,
                       h0: Optional[torch.Tensor] = None, return_final_state: bool = False,
                       y: Optional[torch.Tensor] = None,
                       h_final: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       conv_state_in: Optional[torch.Tensor] = None,
                       conv_state_out: Optional[torch.Tensor] = None,
                       return_conv_state: bool = False,
                       checkpoints: Optional[torch.Tensor] = None):
    """ssm_selective_scan_fwd.  Returns (y, h_final or None), or with
    return_conv_state (or a conv_state_out given) (y, h_final or None,
    conv_state_out); conv states are (B, K-1, D) in x's dtype.  A float32 tensor
    `checkpoints` of checkpoint_shape(B, L, D) also receives the state entering every
    SCAN_BLOCK-step block, for selective_scan_bwd(checkpoints=...)."""
    if y is None:
        y = torch.empty_like(x)
    if return_final_state and h_final is None:
        h_final = torch.empty(x.shape[0], x.shape[2], A.shape[1], device=x.device,
                              dtype=torch.float32)
    want_cs = return_conv_state or conv_state_out is not None
    if return_conv_state and conv_state_out is None:
        if conv_w is None:
            raise ValueError("a conv state needs conv_w")
        conv_state_out = torch.empty(x.shape[0], max(conv_w.shape[1] - 1, 0), x.shape[2],
                                     device=x.device, dtype=x.dtype)
    a, dev = _scan_args(x, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, conv_w,
                        conv_b, h0, y, h_final, conv_state_in, conv_state_out, checkpoints)
    need = lib().ssm_selective_scan_workspace_size(ctypes.byref(a))
    if need == ctypes.c_size_t(-1).value:
        _check(lib().ssm_selective_scan_fwd(ctypes.byref(a), None), "ssm_selective_scan_fwd")
    if need > 0:
        ws = workspace if workspace is not None else _workspace(dev, need)
        if ws.device != dev or ws.numel() * ws.element_size() < need:
            raise ValueError("workspace must be a device tensor of >= %d bytes" % need)
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel() * ws.element_size()
    _check(lib().ssm_selective_scan_fwd(ctypes.byref(a), _stream(dev)), "ssm_selective_scan_fwd")
    return (y, h_final, conv_state_out) if want_cs else (y, h_final)


def selective_scan_fwd_noalloc(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor,
                               Bm: torch.Tensor, Cm: torch.Tensor,
                               Dskip: Optional[torch.Tensor] = None,
                               z: Optional[torch.Tensor] = None,
                               delta_bias: Optional[torch.Tensor] = None,
                               delta_softplus: bool = False,
                               conv_w: Optional[torch.Tensor] = None,
                               conv_b: Optional[torch.Tensor] = None,
                               h0: Optional[torch.Tensor] = None,
                               y: Optional[torch.Tensor] = None,
                               h_final: Optional[torch.Tensor] = None,
                               conv_state_in: Optional[torch.Tensor] = None,
                               conv_state_out: Optional[torch.Tensor] = None,
                               checkpoints: Optional[torch.Tensor] = None):
    """ssm_selective_scan_fwd_noalloc: the scan with its workspace in the library's
    scratch array on the device (no workspace tensor).  The outputs y, h_final,
    conv_state_out and checkpoints must be given when wanted (nothing is allocated here
    either).  Returns (y, h_final)."""
    if y is None:
        raise ValueError("y is required (the no-allocation scan allocates nothing)")
    a, dev = _scan_args(x, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, conv_w,
                        conv_b, h0, y, h_final, conv_state_in, conv_state_out, checkpoints)
    _check(lib().ssm_selective_scan_fwd_noalloc(ctypes.byref(a), _stream(dev)),
           "ssm_selective_scan_fwd_noalloc")
    return y, h_final


def selective_scan_args(x, delta, A, Bm, Cm, Dskip=None, z=None, delta_bias=None,
                        delta_softplus=False, conv_w=None, conv_b=None, h0=None, y=None,
                        h_final=None, conv_state_in=None, conv_state_out=None, checkpoints=None):
    """The checked ssm_scan_args_t of a selective_scan_fwd call with a workspace of its own,
    for callers that launch the same scan repeatedly through lib().ssm_selective_scan_fwd.
    Returns (args, y, workspace or None); y is allocated when not given.  The tensors must
    outlive the struct."""
    if y is None:
        y = torch.empty_like(x)
    a, dev = _scan_args(x, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, conv_w,
                        conv_b, h0, y, h_final, conv_state_in, conv_state_out, checkpoints)
    need = lib().ssm_selective_scan_workspace_size(ctypes.byref(a))
    if need == ctypes.c_size_t(-1).value:
        _check(lib().ssm_selective_scan_fwd(ctypes.byref(a), None), "ssm_selective_scan_fwd")
    ws = None
    if need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        a.workspace = ws.data_ptr()
        a.workspace_bytes = need
    return a, y, ws


def causal_conv1d_silu(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ssm_causal_conv1d_silu on x (B, L, D) with weights w (D, K)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 3 or x.device.type != "cuda":
        raise ValueError("x must be a (B, L, D) GPU tensor")
    dev = x.device
    Bsz, L, D = x.shape
    if w.dim() != 2:
        raise ValueError("w must be (D, K)")
    K = w.shape[1]
    _req(x, "x", (Bsz, L, D), x.dtype, dev)
    _req(w, "w", (D, K), torch.float32, dev)
    _opt(bias, "bias", (D,), torch.float32, dev)
    if out is None:
        out = torch.empty_like(x)
    _req(out, "out", (Bsz, L, D), x.dtype, dev)
    _check(lib().ssm_causal_conv1d_silu(Bsz, L, D, K, _io_code(x.dtype), _ptr(x), _ptr(w),
                                        _ptr(bias), _ptr(out), _stream(dev)),
           "ssm_causal_conv1d_silu")
    return out


def state_update(state: torch.Tensor, x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor,
                 Bm: torch.Tensor, Cm: torch.Tensor, Dskip: Optional[torch.Tensor] = None,
                 z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                 delta_softplus: bool = False, y: Optional[torch.Tensor] = None,
                 conv_w: Optional[torch.Tensor] = None, conv_b: Optional[torch.Tensor] = None,
                 conv_state: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ssm_state_update: advances `state` (B, D, N) -- and with conv_w the conv
    window `conv_state` (B, K-1, D) -- in place and returns y (B, D)."""
    a, y = state_update_args(state, x, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, y,
                             conv_w, conv_b, conv_state)
    _check(lib().ssm_state_update(ctypes.byref(a), _stream(state.device)), "ssm_state_update")
    return y


def state_update_args(state, x, delta, A, Bm, Cm, Dskip=None, z=None, delta_bias=None,
                      delta_softplus=False, y=None, conv_w=None, conv_b=None, conv_state=None):
    """The checked ssm_state_update_args_t of a state_update call, and its y (allocated
    when not given), for callers that launch the same step repeatedly through
    lib().ssm_state_update.  The tensors must outlive the struct."""
    if not isinstance(state, torch.Tensor) or state.dim() != 3 or state.device.type != "cuda":
        raise ValueError("state must be a (B, D, N) float32 GPU tensor")
    dev = state.device
    Bsz, D, N = state.shape
    io = x.dtype
    _req(state, "state", (Bsz, D, N), torch.float32, dev)
    _req(x, "x", (Bsz, D), io, dev)
    _req(delta, "delta", (Bsz, D), io, dev)
    _opt(z, "z", (Bsz, D), io, dev)
    _req(Bm, "Bm", (Bsz, N), io, dev)
    _req(Cm, "Cm", (Bsz, N), io, dev)
    _req(A, "A", (D, N), torch.float32, dev)
    _opt(Dskip, "Dskip", (D,), torch.float32, dev)
    _opt(delta_bias, "delta_bias", (D,), torch.float32, dev)
    if y is None:
        y = torch.empty_like(x)
    _req(y, "y", (Bsz, D), io, dev)
    K = 0
    if conv_w is not None:
        if conv_w.dim() != 2:
            raise ValueError("conv_w must be (D, K)")
        K = conv_w.shape[1]
        _req(conv_w, "conv_w", (D, K), torch.float32, dev)
        if K > 1:
            _req(conv_state, "conv_state", (Bsz, K - 1, D), io, dev)
    elif conv_b is not None or conv_state is not None:
        raise ValueError("conv_b/conv_state need conv_w")
    _opt(conv_b, "conv_b", (D,), torch.float32, dev)
    a = StateUpdateArgs(batch=Bsz, dim=D, dstate=N, io_dtype=_io_code(io),
                        delta_softplus=int(bool(delta_softplus)), state=_ptr(state), x=_ptr(x),
                        delta=_ptr(delta), z=_ptr(z), Bm=_ptr(Bm), Cm=_ptr(Cm), A=_ptr(A),
                        Dskip=_ptr(Dskip), delta_bias=_ptr(delta_bias), y=_ptr(y), conv_k=K,
                        conv_w=_ptr(conv_w), conv_b=_ptr(conv_b),
                        conv_state=_ptr(conv_state) if K > 1 else None)
    return a, y


def selective_scan_bwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                       Cm: torch.Tensor, dy: torch.Tensor, Dskip: Optional[torch.Tensor] = None,
                       z: Optional[torch.Tensor] = None,
                       delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
                       h0: Optional[torch.Tensor] = None,
                       dh_final: Optional[torch.Tensor] = None,
                       conv_w: Optional[torch.Tensor] = None,
                       conv_b: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       conv_state_in: Optional[torch.Tensor] = None,
                       checkpoints: Optional[torch.Tensor] = None) -> dict:
    """ssm_selective_scan_bwd: gradients of the scan (1 <= N <= 16).  `checkpoints` are
    the ones a selective_scan_fwd call with the same inputs wrote (else the backward
    recomputes them).

    Returns a dict with dx, ddelta (x's dtype), dA, dBm, dCm (float32) and, for the
    optional inputs given, dz, dDskip, ddelta_bias, dh0, dconv_w, dconv_b and
    dconv_state_in (x's dtype, the gradient of the conv state entering the sequence)."""
    a, dev = _scan_args(x, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, conv_w, conv_b,
                        h0, torch.empty_like(x), None, conv_state_in=conv_state_in,
                        checkpoints=checkpoints)
    Bsz, L, D = x.shape
    N = A.shape[1]
    io = x.dtype
    _req(dy, "dy", (Bsz, L, D), io, dev)
    _opt(dh_final, "dh_final", (Bsz, D, N), torch.float32, dev)
    f32 = dict(device=dev, dtype=torch.float32)
    out = dict(dx=torch.empty_like(x), ddelta=torch.empty_like(x), dA=torch.empty(D, N, **f32),
               dBm=torch.empty(Bsz, L, N, **f32), dCm=torch.empty(Bsz, L, N, **f32))
    if z is not None:
        out["dz"] = torch.empty_like(x)
    if Dskip is not None:
        out["dDskip"] = torch.empty(D, **f32)
    if delta_softplus:
        out["ddelta_bias"] = torch.empty(D, **f32)
    if h0 is not None:
        out["dh0"] = torch.empty(Bsz, D, N, **f32)
    if conv_w is not None:
        out["dconv_w"] = torch.empty(D, a.conv_k, **f32)
        out["dconv_b"] = torch.empty(D, **f32)
    if conv_state_in is not None:
        out["dconv_state_in"] = torch.empty_like(conv_state_in)
    g = lambda k: _ptr(out.get(k))
    b = ScanBwdArgs(batch=Bsz, seqlen=L, dim=D, dstate=N, io_dtype=a.io_dtype,
                    delta_softplus=a.delta_softplus, conv_k=a.conv_k, x=a.x, delta=a.delta, Bm=a.Bm,
                    Cm=a.Cm, z=a.z, A=a.A, Dskip=a.Dskip, delta_bias=a.delta_bias, h0=a.h0,
                    conv_w=a.conv_w, conv_b=a.conv_b, dconv_w=g("dconv_w"), dconv_b=g("dconv_b"),
                    dy=_ptr(dy), dh_final=_ptr(dh_final), dx=g("dx"), ddelta=g("ddelta"),
                    dz=g("dz"), dA=g("dA"), dBm=g("dBm"), dCm=g("dCm"), dDskip=g("dDskip"),
                    ddelta_bias=g("ddelta_bias"), dh0=g("dh0"), conv_state_in=a.conv_state_in,
                    dconv_state_in=g("dconv_state_in"), checkpoints=_ptr(checkpoints))
    need = lib().ssm_selective_scan_bwd_workspace_size(ctypes.byref(b))
    if need == ctypes.c_size_t(-1).value:
        _check(lib().ssm_selective_scan_bwd(ctypes.byref(b), None), "ssm_selective_scan_bwd")
    if need > 0:
        ws = workspace if workspace is not None else _workspace(dev, need)
        if ws.device != dev or ws.numel() * ws.element_size() < need:
            raise ValueError("workspace must be a device tensor of >= %d bytes" % need)
        b.workspace = ws.data_ptr()
        b.workspace_bytes = ws.numel() * ws.element_size()
    _check(lib().ssm_selective_scan_bwd(ctypes.byref(b), _stream(dev)), "ssm_selective_scan_bwd")
    return out


class _SelectiveScanFn(torch.autograd.Function):
    """selective_scan as a torch autograd function: the forward writes the block
    checkpoints, the backward reads them (ssm_selective_scan_fwd / _bwd)."""

    @staticmethod
    def forward(ctx, x, delta, A, Bm, Cm, Dskip, z, delta_bias, h0, conv_w, conv_b, delta_softplus):
        ck = torch.empty(checkpoint_shape(x.shape[0], x.shape[1], x.shape[2]), device=x.device,
                         dtype=torch.float32)
        y, hf = selective_scan_fwd(x, delta, A, Bm, Cm, Dskip=Dskip, z=z, delta_bias=delta_bias,
                                   delta_softplus=delta_softplus, conv_w=conv_w, conv_b=conv_b, h0=h0,
                                   return_final_state=True, checkpoints=ck)
        ctx.save_for_backward(x, delta, A, Bm, Cm, Dskip, z, delta_bias, h0, conv_w, conv_b, ck)
        ctx.delta_softplus = delta_softplus
        return y, hf

    @staticmethod
    def backward(ctx, dy, dh_final):
        x, delta, A, Bm, Cm, Dskip, z, delta_bias, h0, conv_w, conv_b, ck = ctx.saved_tensors
        if dy is None:
            dy = torch.zeros_like(x)
        g = selective_scan_bwd(x, delta, A, Bm, Cm, dy.contiguous(), Dskip=Dskip, z=z,
                               delta_bias=delta_bias, delta_softplus=ctx.delta_softplus, h0=h0,
                               dh_final=None if dh_final is None else dh_final.contiguous(),
                               conv_w=conv_w, conv_b=conv_b, checkpoints=ck)
        given = lambda t, k: g.get(k) if t is not None else None
        return (g["dx"], g["ddelta"], g["dA"], g["dBm"], g["dCm"], given(Dskip, "dDskip"), given(z, "dz"),
                given(delta_bias, "ddelta_bias"), given(h0, "dh0"), given(conv_w, "dconv_w"),
                given(conv_b, "dconv_b"), None)


def selective_scan(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                   Cm: torch.Tensor, Dskip: Optional[torch.Tensor] = None,
                   z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                   delta_softplus: bool = False, h0: Optional[torch.Tensor] = None,
                   conv_w: Optional[torch.Tensor] = None, conv_b: Optional[torch.Tensor] = None):
    """The scan as a differentiable torch op (1 <= N <= 16): returns (y, h_final), and
    backward() runs ssm_selective_scan_bwd from the checkpoints the forward kept.  The
    gradients of B and C are computed in fp32 and cast to their dtype by autograd."""
    return _SelectiveScanFn.apply(x, delta, A, Bm, Cm, Dskip, z, delta_bias, h0, conv_w, conv_b,
                                  bool(delta_softplus))


class BlockPlan:
    """A plan of ssm_block_fwd for fixed sizes (owns the library's plan handle)."""

    def __init__(self, batch: int, seqlen: int, d_model: int, d_inner: int, dstate: int,
                 dt_rank: int, conv_k: int):
        self.dims = BlockDims(batch=batch, seqlen=seqlen, d_model=d_model, d_inner=d_inner,
                              dstate=dstate, dt_rank=dt_rank, conv_k=conv_k)
        self._h = _P()
        self._lib = lib()
        _check(self._lib.ssm_block_plan_create(ctypes.byref(self.dims), ctypes.byref(self._h)),
               "ssm_block_plan_create")
        self.workspace_bytes = int(self._lib.ssm_block_workspace_size(self._h))

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h:
            self._lib.ssm_block_plan_destroy(self._h)
            self._h = _P()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_plan_cache = {}


def mamba_block_fwd(h: torch.Tensor, norm_w: torch.Tensor, w_in: torch.Tensor, conv_w: torch.Tensor,
                    conv_b: Optional[torch.Tensor], w_x: torch.Tensor, w_dt: torch.Tensor,
                    dt_bias: torch.Tensor, A: torch.Tensor, Dskip: Optional[torch.Tensor],
                    w_out: torch.Tensor, eps: float = 1e-5, out: Optional[torch.Tensor] = None,
                    plan: Optional[BlockPlan] = None, workspace: Optional[torch.Tensor] = None):
    """One Mamba block with its pre-norm residual (ssm_block_fwd): h (B, L, d_model) bf16 ->
    h + out_proj(S6(...) * silu(z)).  Weight shapes as in ssm_block_weights_t; `out` may be h."""
    if not isinstance(h, torch.Tensor) or h.dim() != 3 or h.device.type != "cuda":
        raise ValueError("h must be a (B, L, d_model) GPU tensor")
    dev = h.device
    Bsz, L, dm = h.shape
    if A.dim() != 2 or w_dt.dim() != 2 or conv_w.dim() != 2:
        raise ValueError("A, w_dt and conv_w must be 2-D")
    D, N = A.shape
    R = w_dt.shape[1]
    K = conv_w.shape[1]
    bf, f32 = torch.bfloat16, torch.float32
    _req(h, "h", (Bsz, L, dm), bf, dev)
    _req(norm_w, "norm_w", (dm,), f32, dev)
    _req(w_in, "w_in", (2 * D, dm), bf, dev)
    _req(conv_w, "conv_w", (D, K), f32, dev)
    _opt(conv_b, "conv_b", (D,), f32, dev)
    _req(w_x, "w_x", (R + 2 * N, D), bf, dev)
    _req(w_dt, "w_dt", (D, R), bf, dev)
    _req(dt_bias, "dt_bias", (D,), f32, dev)
    _req(A, "A", (D, N), f32, dev)
    _opt(Dskip, "Dskip", (D,), f32, dev)
    _req(w_out, "w_out", (dm, D), bf, dev)
    if out is None:
        out = torch.empty_like(h)
    _req(out, "out", (Bsz, L, dm), bf, dev)
    if plan is None:
        key = (dev.index, Bsz, L, dm, D, N, R, K)
        plan = _plan_cache.get(key)
        if plan is None:
            with torch.cuda.device(dev):
                plan = BlockPlan(Bsz, L, dm, D, N, R, K)
            _plan_cache[key] = plan
    d = plan.dims
    if (d.batch, d.seqlen, d.d_model, d.d_inner, d.dstate, d.dt_rank, d.conv_k) != (Bsz, L, dm, D, N, R, K):
        raise ValueError("the plan was made for other sizes")
    if workspace is None:
        workspace = _workspace(dev, plan.workspace_bytes)
    wts = BlockWeights(norm_w=_ptr(norm_w), w_in=_ptr(w_in), conv_w=_ptr(conv_w), conv_b=_ptr(conv_b),
                       w_x=_ptr(w_x), w_dt=_ptr(w_dt), dt_bias=_ptr(dt_bias), A=_ptr(A),
                       Dskip=_ptr(Dskip), w_out=_ptr(w_out), norm_eps=float(eps))
    _check(lib().ssm_block_fwd(plan.handle, ctypes.byref(wts), _ptr(h), _ptr(out), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(dev)),
           "ssm_block_fwd")
    return out


def ssd_fwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor, Cm: torch.Tensor,
            Dskip: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
            delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
            h0: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
            h_final: Optional[torch.Tensor] = None, return_final_state: bool = False):
    """ssm_ssd_fwd: the SSD (Mamba-2) layer.  x, z: (B, L, H, P) and delta: (B, L, H), bf16
    (chunked on the matrix cores) or fp32 (the recurrent form); A, Dskip, delta_bias: (H,)
    fp32; Bm, Cm: (B, L, G, N) in x's dtype; h0, h_final: (B, H, P, N) fp32.
    Returns y, or (y, h_final) with return_final_state or h_final given."""
    if not isinstance(x, torch.Tensor) or x.dim() != 4 or x.device.type != "cuda":
        raise ValueError("x must be a (B, L, H, P) GPU tensor")
    if not isinstance(Bm, torch.Tensor) or Bm.dim() != 4:
        raise ValueError("Bm must be (B, L, G, N)")
    dev = x.device
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    bf, f32 = x.dtype, torch.float32
    _io_code(bf)
    _req(x, "x", (Bsz, L, H, P), bf, dev)
    _req(delta, "delta", (Bsz, L, H), bf, dev)
    _req(A, "A", (H,), f32, dev)
    _req(Bm, "Bm", (Bsz, L, G, N), bf, dev)
    _req(Cm, "Cm", (Bsz, L, G, N), bf, dev)
    _opt(Dskip, "Dskip", (H,), f32, dev)
    _opt(z, "z", (Bsz, L, H, P), bf, dev)
    _opt(delta_bias, "delta_bias", (H,), f32, dev)
    _opt(h0, "h0", (Bsz, H, P, N), f32, dev)
    if y is None:
        y = torch.empty_like(x)
    _req(y, "y", (Bsz, L, H, P), bf, dev)
    if h_final is None and return_final_state:
        h_final = torch.empty(Bsz, H, P, N, device=dev, dtype=f32)
    _opt(h_final, "h_final", (Bsz, H, P, N), f32, dev)
    a = SsdArgs(batch=Bsz, seqlen=L, nheads=H, headdim=P, ngroups=G, dstate=N, io_dtype=_io_code(bf),
                delta_softplus=int(bool(delta_softplus)), x=_ptr(x), delta=_ptr(delta), A=_ptr(A),
                Bm=_ptr(Bm), Cm=_ptr(Cm), Dskip=_ptr(Dskip), z=_ptr(z), delta_bias=_ptr(delta_bias),
                h0=_ptr(h0), y=_ptr(y), h_final=_ptr(h_final), workspace=None, workspace_bytes=0)
    need = lib().ssm_ssd_workspace_size(ctypes.byref(a))
    if need == ctypes.c_size_t(-1).value:
        _check(lib().ssm_ssd_fwd(ctypes.byref(a), _stream(dev)), "ssm_ssd_fwd")  # reports the error
    if need:
        ws = _workspace(dev, need)
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel()
    _check(lib().ssm_ssd_fwd(ctypes.byref(a), _stream(dev)), "ssm_ssd_fwd")
    return (y, h_final) if h_final is not None else y


def ssd_step(state: torch.Tensor, x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor,
             Bm: torch.Tensor, Cm: torch.Tensor, Dskip: Optional[torch.Tensor] = None,
             z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
             delta_softplus: bool = False, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ssm_ssd_step: one decode step of the SSD layer; advances `state` (B, H, P, N) fp32 in
    place.  x, z: (B, H, P) bf16; delta: (B, H) bf16; A, Dskip, delta_bias: (H,) fp32;
    Bm, Cm: (B, G, N) bf16.  Returns y (B, H, P) bf16."""
    a, y = ssd_step_args(state, x, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, y)
    _check(lib().ssm_ssd_step(ctypes.byref(a), _stream(state.device)), "ssm_ssd_step")
    return y


def ssd_step_args(state, x, delta, A, Bm, Cm, Dskip=None, z=None, delta_bias=None,
                  delta_softplus=False, y=None):
    """The checked ssm_ssd_step_args_t of an ssd_step call, and its y (allocated when not
    given), for callers that launch the same step repeatedly through lib().ssm_ssd_step.
    The tensors must outlive the struct."""
    if not isinstance(state, torch.Tensor) or state.dim() != 4 or state.device.type != "cuda":
        raise ValueError("state must be a (B, H, P, N) GPU tensor")
    if not isinstance(Bm, torch.Tensor) or Bm.dim() != 3:
        raise ValueError("Bm must be (B, G, N)")
    dev = state.device
    Bsz, H, P, N = state.shape
    G = Bm.shape[1]
    bf, f32 = torch.bfloat16, torch.float32
    _req(state, "state", (Bsz, H, P, N), f32, dev)
    _req(x, "x", (Bsz, H, P), bf, dev)
    _req(delta, "delta", (Bsz, H), bf, dev)
    _req(A, "A", (H,), f32, dev)
    _req(Bm, "Bm", (Bsz, G, N), bf, dev)
    _req(Cm, "Cm", (Bsz, G, N), bf, dev)
    _opt(Dskip, "Dskip", (H,), f32, dev)
    _opt(z, "z", (Bsz, H, P), bf, dev)
    _opt(delta_bias, "delta_bias", (H,), f32, dev)
    if y is None:
        y = torch.empty_like(x)
    _req(y, "y", (Bsz, H, P), bf, dev)
    a = SsdStepArgs(batch=Bsz, nheads=H, headdim=P, ngroups=G, dstate=N, io_dtype=SSM_BF16,
                    delta_softplus=int(bool(delta_softplus)), state=_ptr(state), x=_ptr(x),
                    delta=_ptr(delta), A=_ptr(A), Bm=_ptr(Bm), Cm=_ptr(Cm), Dskip=_ptr(Dskip),
                    z=_ptr(z), delta_bias=_ptr(delta_bias), y=_ptr(y))
    return a, y
