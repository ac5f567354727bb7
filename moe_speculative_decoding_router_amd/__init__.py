"""Python binding of libmoeverify (the union-expert MoE verify layer and
EcoSpec cost-aware draft selection for MI355X).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch provides device memory and the current stream.  If the library is
not built, the first call raises; there is no fallback.

Entry points (same names as the C ABI in include/moe_verify.h):
  pack_weights(src, wdtype, gate_up)  -> packed weights (one-time preparation)
  verify_layer(x, layer, bias=None)   -> (y, aux)
  verify_layer_noalloc(x, layer, bias=None, out=None, aux=None) -> (y, aux)
  union_stats(topk_idx, E)            -> (counts, reuse)
  select_drafts(parent, P, Epred, gamma, eps=1e-6, static=False) -> S
  expand_drafts(parent, P, Epred, t_ar, t_exp, c_draft=None) -> (S, count)
  union_stats_segments(topk_idx, E, offsets) -> (per, total)
  gate_depths(c, Epred, t_base, t_exp) -> d
  workspace_bytes(layer, T, bias=None)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoeverify.so")

MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}
NUM_STAGES = 5
MAX_SEGMENTS = 64
STAGE_NAMES = ("router", "route", "gate_up", "down", "combine")
EXPORTED = ("moe_pack_weights", "moe_verify_workspace_bytes", "moe_verify_layer", "union_stats",
            "select_drafts", "select_drafts_static", "expand_drafts", "union_stats_segments", "gate_depths",
            "moe_stream_read", "moe_last_error", "moe_verify_layer_noalloc")

_vp, _i32, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float


class _Layer(ctypes.Structure):
    _fields_ = [("H", _i32), ("I", _i32), ("E", _i32), ("k", _i32), ("wdtype", _i32),
                ("Wr", _vp), ("W_gu", _vp), ("W_d", _vp), ("s_gu", _vp), ("s_d", _vp),
                ("Wsh_gu", _vp), ("Wsh_d", _vp), ("ssh_gu", _vp), ("ssh_d", _vp)]


class _Bias(ctypes.Structure):
    _fields_ = [("cap", _i32), ("alpha", _f32), ("w_conf", _vp), ("nseg", _i32), ("seg_off", _vp)]


class _Aux(ctypes.Structure):
    _fields_ = [("logits", _vp), ("topk_idx", _vp), ("topk_w", _vp), ("union_size", _vp),
                ("union_experts", _vp), ("csr_ptr", _vp), ("csr_tok", _vp), ("csr_w", _vp),
                ("pstar", _vp), ("pstar_size", _vp), ("events", _vp)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoeverify.so from this package directory (raises if missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build()); "
                              "there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_verify_workspace_bytes.argtypes = [ctypes.POINTER(_Layer), _i32, ctypes.POINTER(_Bias)]
        L.moe_verify_workspace_bytes.restype = ctypes.c_size_t
        L.moe_verify_layer.argtypes = [ctypes.POINTER(_Layer), _vp, _i32, ctypes.POINTER(_Bias), _vp,
                                       ctypes.POINTER(_Aux), _vp, ctypes.c_size_t, _vp]
        L.moe_verify_layer.restype = ctypes.c_int
        L.moe_verify_layer_noalloc.argtypes = [ctypes.POINTER(_Layer), _vp, _i32, ctypes.POINTER(_Bias), _vp,
                                               ctypes.POINTER(_Aux), _vp]
        L.moe_verify_layer_noalloc.restype = ctypes.c_int
        L.union_stats.argtypes = [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]
        L.union_stats.restype = ctypes.c_int
        L.select_drafts.argtypes = [_vp, _i32, _vp, _vp, _i32, _i32, _f32, _i32, _vp, _vp]
        L.select_drafts.restype = ctypes.c_int
        L.select_drafts_static.argtypes = L.select_drafts.argtypes
        L.select_drafts_static.restype = ctypes.c_int
        L.expand_drafts.argtypes = [_vp, _i32, _vp, _vp, _i32, _f32, _f32, _vp, _i32, _vp, _vp, _vp]
        L.expand_drafts.restype = ctypes.c_int
        L.union_stats_segments.argtypes = [_vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _vp]
        L.union_stats_segments.restype = ctypes.c_int
        L.gate_depths.argtypes = [_vp, _vp, _i32, _i32, _i32, _f32, _f32, _vp, _vp]
        L.gate_depths.restype = ctypes.c_int
        L.moe_pack_weights.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp]
        L.moe_pack_weights.restype = ctypes.c_int
        L.moe_stream_read.argtypes = [_vp, ctypes.c_size_t, _vp, _vp]
        L.moe_stream_read.restype = ctypes.c_int
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libmoeverify error {code}: {msg}")
        self.code = code


def _check(rc: int) -> None:
    if rc != 0:
        raise MoeError(rc, lib().moe_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# torch dtype names accepted for each weight format (bf16 weights may be given
# as bf16 or as their 16-bit patterns; fp8 as float8_e4m3fn or as uint8 codes)
_WDT = {"f32": ("float32",), "bf16": ("bfloat16", "int16", "uint16"), "fp8": ("uint8", "float8_e4m3fn")}


def _dtname(t) -> str:
    return str(t.dtype).replace("torch.", "")


def _check_tensor(t, name: str, dtypes, numel: Optional[int] = None, shape=None, device=None,
                  at_least: bool = False) -> None:
    """Raise ValueError unless t is a contiguous tensor with one of `dtypes`,
    the given shape (or element count; `at_least`: no fewer elements) and on
    `device`.  The C ABI sees only pointers, so these checks are what keeps
    the kernels inside the caller's buffers."""
    if t is None:
        raise ValueError(f"{name} is missing")
    if not hasattr(t, "data_ptr") or not hasattr(t, "is_contiguous"):
        raise ValueError(f"{name} must be a tensor")
    if _dtname(t) not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(dtypes)}, got {_dtname(t)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None:
        n = t.numel()
        if (n < numel) if at_least else (n != numel):
            raise ValueError(f"{name} must have {'at least ' if at_least else ''}{numel} elements, got {n}")


@dataclass
class LayerWeights:
    """Device tensors of one MoE layer (layouts in include/moe_verify.h).

    wdtype 'f32' uses float32 W_gu/W_d; 'bf16' uses bf16 or uint16 bit
    tensors; 'fp8' uses uint8 (or float8_e4m3fn) codes with float32 block
    scales s_gu [E, 2I/128, H/128] and s_d [E, H/128, I/128]."""
    H: int
    I: int
    E: int
    k: int
    wdtype: str
    Wr: object
    W_gu: object
    W_d: object
    s_gu: object = None
    s_d: object = None
    Wsh_gu: object = None
    Wsh_d: object = None
    ssh_gu: object = None
    ssh_d: object = None

    def __setattr__(self, name, value):
        # any reassignment invalidates the result of the last validate()
        object.__setattr__(self, "_valid_on", None)
        object.__setattr__(self, name, value)

    def validate(self, device) -> None:
        """Check every tensor against the layout of include/moe_verify.h
        (dtype, element count, contiguity, device); raises ValueError.  The
        result is remembered until a field is reassigned (tensors resized in
        place are not noticed)."""
        if getattr(self, "_valid_on", None) == device:
            return
        self._check_fields(device)
        object.__setattr__(self, "_valid_on", device)

    def _check_fields(self, device) -> None:
        H, I, E, k, wd = self.H, self.I, self.E, self.k, self.wdtype
        if wd not in DTYPES:
            raise ValueError(f"unknown wdtype {wd!r}")
        if min(H, I, E, k) < 1:
            raise ValueError("H, I, E and k must be positive")
        _check_tensor(self.Wr, "Wr", ("float32",), numel=E * H, device=device)
        _check_tensor(self.W_gu, "W_gu", _WDT[wd], numel=E * 2 * I * H, device=device)
        _check_tensor(self.W_d, "W_d", _WDT[wd], numel=E * H * I, device=device)
        if (self.Wsh_gu is None) != (self.Wsh_d is None):
            raise ValueError("the shared expert needs both Wsh_gu and Wsh_d")
        if self.Wsh_gu is not None:
            _check_tensor(self.Wsh_gu, "Wsh_gu", _WDT[wd], numel=2 * I * H, device=device)
            _check_tensor(self.Wsh_d, "Wsh_d", _WDT[wd], numel=H * I, device=device)
        if wd == "fp8":
            if H % 128 or I % 128:
                raise ValueError("fp8 weights need H and I multiples of 128")
            gs, ds = (2 * I // 128) * (H // 128), (H // 128) * (I // 128)
            _check_tensor(self.s_gu, "s_gu", ("float32",), numel=E * gs, device=device)
            _check_tensor(self.s_d, "s_d", ("float32",), numel=E * ds, device=device)
            if self.Wsh_gu is not None:
                _check_tensor(self.ssh_gu, "ssh_gu", ("float32",), numel=gs, device=device)
                _check_tensor(self.ssh_d, "ssh_d", ("float32",), numel=ds, device=device)
        else:
            for name in ("s_gu", "s_d", "ssh_gu", "ssh_d"):
                if getattr(self, name) is not None:
                    raise ValueError(f"{name} is only used with fp8 weights")

    def _c(self) -> _Layer:
        return _Layer(self.H, self.I, self.E, self.k, DTYPES[self.wdtype], _ptr(self.Wr), _ptr(self.W_gu),
                      _ptr(self.W_d), _ptr(self.s_gu), _ptr(self.s_d), _ptr(self.Wsh_gu), _ptr(self.Wsh_d),
                      _ptr(self.ssh_gu), _ptr(self.ssh_d))


@dataclass
class Bias:
    """Reuse-aware soft bias parameters (w_conf: [T] float32 device tensor).
    offsets: None (the importance and the preferred set are pooled over the
    call) or the [S + 1] token offsets of the call's sequences, each with its
    own preferred set (host sequence of ints, 0 .. T)."""
    cap: int
    alpha: float
    w_conf: object
    offsets: Optional[Sequence[int]] = None

    @property
    def nseq(self) -> int:
        """Sequences with a preferred set of their own (1 when pooled)."""
        return 1 if self.offsets is None else len(self.offsets) - 1

    def check(self, T: int, device) -> None:
        _check_tensor(self.w_conf, "bias.w_conf", ("float32",), numel=T, device=device)
        if self.offsets is not None:
            off = np.asarray(self.offsets)
            if (off.ndim != 1 or len(off) < 2 or len(off) - 1 > MAX_SEGMENTS or off[0] != 0 or off[-1] != T
                    or np.any(np.diff(off) < 0)):
                raise ValueError(f"bias.offsets must be 2 .. {MAX_SEGMENTS + 1} non-decreasing offsets from 0 to T={T}")

    def _c(self) -> _Bias:
        if self.offsets is None:
            return _Bias(self.cap, self.alpha, _ptr(self.w_conf), 0, None)
        off = np.ascontiguousarray(np.asarray(self.offsets, dtype=np.int32))
        c = _Bias(self.cap, self.alpha, _ptr(self.w_conf), len(off) - 1, off.ctypes.data)
        c._keep = off   # the C side reads the host offsets during the call
        return c


def _launch_stream(stream, device, owned=()) -> int:
    """Raw handle of the launch stream: torch's current stream when `stream`
    is None, else a torch.cuda.Stream or a raw hipStream_t handle.  Tensors in
    `owned` were allocated by the caller from the current stream's pool; on
    another stream the launch first waits for the current stream (the memory
    may still have pending uses there), and the tensors are marked as used
    by the launch stream."""
    import torch
    cur = torch.cuda.current_stream(device)
    if stream is None:
        return cur.cuda_stream
    sobj = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream), device=device)
    owned = [t for t in owned if t is not None]
    if owned and sobj.cuda_stream != cur.cuda_stream:
        sobj.wait_stream(cur)
        for t in owned:
            t.record_stream(sobj)
    return sobj.cuda_stream


def pack_weights(src, wdtype: str, gate_up: bool, out=None, stream=None):
    """Pack row-major expert weights src [E, rows, K] (bf16 bits or fp8 codes,
    device) into the tile layout moe_verify_layer streams.  Returns the packed
    tensor (same shape and dtype; only the byte order differs)."""
    import torch
    if src.dim() == 2:
        src = src.unsqueeze(0)
    if src.dim() != 3 or not src.is_contiguous():
        raise ValueError("src must be a contiguous [E, rows, K] tensor")
    E, rows, K = (int(v) for v in src.shape)
    dst = out if out is not None else torch.empty_like(src)
    s = _launch_stream(stream, src.device, [dst] if out is None else [])
    _check(lib().moe_pack_weights(src.data_ptr(), dst.data_ptr(), E, rows, K, DTYPES[wdtype], int(bool(gate_up)), s))
    return dst


def stream_read(src, checksum, stream=None) -> None:
    """moe_stream_read: stream `src` (a contiguous device tensor, byte size a
    multiple of 16) with the FFN kernels' load pattern, XOR-folding its
    32-bit words into `checksum` (a zeroed int32 device tensor of 1)."""
    import torch
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    nbytes = src.numel() * src.element_size()
    s = _launch_stream(stream, src.device)
    _check(lib().moe_stream_read(src.data_ptr(), nbytes, checksum.data_ptr(), s))


def pack_layer_tensors(W: dict, wdtype: str) -> dict:
    """Pack the row-major weight tensors of a layer dict (keys W_gu, W_d and
    optionally Wsh_gu, Wsh_d); scales and other entries pass through."""
    out = dict(W)
    for key, gu in (("W_gu", True), ("W_d", False), ("Wsh_gu", True), ("Wsh_d", False)):
        if W.get(key) is not None:
            packed = pack_weights(W[key].contiguous(), wdtype, gu)
            out[key] = packed if W[key].dim() == 3 else packed[0]
    return out


def workspace_bytes(layer: LayerWeights, T: int, bias: Optional[Bias] = None) -> int:
    L = layer._c()
    b = bias._c() if bias is not None else None
    n = lib().moe_verify_workspace_bytes(ctypes.byref(L), T, ctypes.byref(b) if b else None)
    if n == 0:
        raise MoeError(-1, lib().moe_last_error().decode())
    return int(n)


def expert_bytes(H: int, I: int, wdtype: str) -> int:
    """Bytes of one expert's weights (gate, up and down) plus fp8 block scales."""
    if wdtype == "f32":
        return 3 * H * I * 4
    if wdtype == "bf16":
        return 3 * H * I * 2
    if wdtype == "fp8":
        return 3 * H * I + (2 * I // 128) * (H // 128) * 4 + (H // 128) * (I // 128) * 4
    raise ValueError(wdtype)


@dataclass
class Aux:
    def __setattr__(self, name, value):
        object.__setattr__(self, "_valid", False)
        object.__setattr__(self, name, value)

    logits: object
    topk_idx: object
    topk_w: object
    union_size: object
    union_experts: object
    csr_ptr: object
    csr_tok: object
    csr_w: object
    pstar: object
    pstar_size: object


@dataclass
class Workspace:
    """Reusable device workspace plus output buffers for one (layer shape, T)."""
    ws: object
    nbytes: int
    aux: Optional[Aux] = None
    extra: dict = field(default_factory=dict)

    def __setattr__(self, name, value):
        object.__setattr__(self, "_valid_for", None)
        object.__setattr__(self, name, value)


def alloc_aux(layer: LayerWeights, T: int, device, bias: Optional[Bias] = None) -> Aux:
    import torch
    E, k = layer.E, layer.k
    nseq = 1 if bias is None else bias.nseq
    i32, f32 = torch.int32, torch.float32
    return Aux(logits=torch.empty((T, E), dtype=f32, device=device),
               topk_idx=torch.empty((T, k), dtype=i32, device=device),
               topk_w=torch.empty((T, k), dtype=f32, device=device),
               union_size=torch.empty(1, dtype=i32, device=device),
               union_experts=torch.empty(E, dtype=i32, device=device),
               csr_ptr=torch.empty(E + 1, dtype=i32, device=device),
               csr_tok=torch.empty(T * k, dtype=i32, device=device),
               csr_w=torch.empty(T * k, dtype=f32, device=device),
               pstar=torch.empty(max(E, nseq * (bias.cap if bias else 0)), dtype=i32, device=device),
               pstar_size=torch.empty(nseq, dtype=i32, device=device))


def alloc_workspace(layer: LayerWeights, T: int, bias: Optional[Bias] = None, device=None,
                    with_aux: bool = True) -> Workspace:
    import torch
    device = device or layer.Wr.device
    n = workspace_bytes(layer, T, bias)
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + n]
    return Workspace(ws=ws, nbytes=n, aux=alloc_aux(layer, T, device, bias) if with_aux else None)


def _aux_sizes(layer: LayerWeights, T: int, bias: Optional[Bias] = None):
    """Element count and dtype of each Aux field (include/moe_verify.h)."""
    E, k = layer.E, layer.k
    nseq = 1 if bias is None else bias.nseq
    i32, f32 = ("int32",), ("float32",)
    return {"logits": (T * E, f32), "topk_idx": (T * k, i32), "topk_w": (T * k, f32), "union_size": (1, i32),
            "union_experts": (E, i32), "csr_ptr": (E + 1, i32), "csr_tok": (T * k, i32), "csr_w": (T * k, f32),
            "pstar": (max(E, nseq * (bias.cap if bias else 0)), i32), "pstar_size": (nseq, i32)}


def _check_workspace(wsp: Workspace, layer: LayerWeights, T: int, bias: Optional[Bias], dev) -> None:
    """A caller-supplied workspace must hold at least what this call needs:
    the C side trusts the byte count it is given.  The last passing
    (layer shape, T, bias cap, device) is remembered until a field of the
    workspace or of its aux is reassigned."""
    key = (layer.H, layer.I, layer.E, layer.k, layer.wdtype, T, None if bias is None else (bias.cap, bias.nseq), dev)
    if getattr(wsp, "_valid_for", None) == key and (wsp.aux is None or getattr(wsp.aux, "_valid", False)):
        return
    need = workspace_bytes(layer, T, bias)
    if wsp.nbytes < need:
        raise ValueError(f"workspace holds {wsp.nbytes} bytes, this call needs {need}")
    _check_tensor(wsp.ws, "workspace.ws", ("uint8", "int8"), numel=wsp.nbytes, device=dev, at_least=True)
    if wsp.aux is not None:
        for f, (n, dt) in _aux_sizes(layer, T, bias).items():
            t = getattr(wsp.aux, f)
            if t is not None:
                _check_tensor(t, f"workspace.aux.{f}", dt, numel=n, device=dev, at_least=True)
        object.__setattr__(wsp.aux, "_valid", True)
    object.__setattr__(wsp, "_valid_for", key)


def verify_layer(x, layer: LayerWeights, bias: Optional[Bias] = None, *, out=None,
                 workspace: Optional[Workspace] = None, events: Optional[Sequence] = None, stream=None):
    """One MoE-layer verify step for x [T, H] float32 (device).  Returns
    (y [T, H] float32, Aux or None).  `stream`: a torch.cuda.Stream or a raw
    hipStream_t handle (default: torch's current stream).  Buffers this call
    allocates itself (workspace, y) come from the current stream's pool; on
    another stream the launch first waits for the current stream, and the
    buffers are marked as used by the launch stream."""
    import torch
    if not hasattr(x, "dim") or x.dim() != 2:
        raise ValueError("x must be a contiguous float32 [T, H] tensor")
    T = int(x.shape[0])
    dev = x.device
    _check_tensor(x, "x", ("float32",), shape=(T, layer.H))
    if dev.type != "cuda":
        raise ValueError(f"x must be a device tensor, got {dev}")
    layer.validate(dev)
    if bias is not None:
        bias.check(T, dev)
    owned = []
    if workspace is None:
        workspace = alloc_workspace(layer, T, bias, device=dev)
        owned.append(workspace.ws)
        if workspace.aux is not None:
            owned += [getattr(workspace.aux, f) for f in Aux.__dataclass_fields__]
    else:
        _check_workspace(workspace, layer, T, bias, dev)
    if out is not None:
        _check_tensor(out, "out", ("float32",), shape=(T, layer.H), device=dev)
    y = out if out is not None else torch.empty_like(x)
    if out is None:
        owned.append(y)
    L = layer._c()
    b = bias._c() if bias is not None else None
    a = workspace.aux
    ev_arr = None
    if events is not None:
        if len(events) != 2 * NUM_STAGES:
            raise ValueError(f"events: need {2 * NUM_STAGES} events (start, end of each stage)")
        ev_arr = (ctypes.c_void_p * (2 * NUM_STAGES))(*[int(e.cuda_event) if hasattr(e, "cuda_event") else int(e)
                                                        for e in events])
    caux = _Aux(*([_ptr(getattr(a, f)) for f in Aux.__dataclass_fields__] if a else [None] * 10),
                ctypes.cast(ev_arr, ctypes.c_void_p) if ev_arr is not None else None)
    s = _launch_stream(stream, x.device, owned)
    rc = lib().moe_verify_layer(ctypes.byref(L), x.data_ptr(), T, ctypes.byref(b) if b else None, y.data_ptr(),
                                ctypes.byref(caux), workspace.ws.data_ptr(), workspace.nbytes, s)
    _check(rc)
    return y, a


def verify_layer_noalloc(x, layer: LayerWeights, bias: Optional[Bias] = None, *, out=None,
                         aux: Optional[Aux] = None, stream=None):
    """moe_verify_layer_noalloc: the verify call on the library's own per-GPU
    workspace array, for callers that cannot allocate (`out` and `aux` given,
    this call allocates nothing either).  Calls that overlap on one GPU race
    on the shared array.  Returns (y, aux)."""
    import torch
    if not hasattr(x, "dim") or x.dim() != 2:
        raise ValueError("x must be a contiguous float32 [T, H] tensor")
    T = int(x.shape[0])
    dev = x.device
    _check_tensor(x, "x", ("float32",), shape=(T, layer.H))
    if dev.type != "cuda":
        raise ValueError(f"x must be a device tensor, got {dev}")
    layer.validate(dev)
    if bias is not None:
        bias.check(T, dev)
    if out is not None:
        _check_tensor(out, "out", ("float32",), shape=(T, layer.H), device=dev)
    if aux is not None:
        for f, (n, dt) in _aux_sizes(layer, T, bias).items():
            t = getattr(aux, f)
            if t is not None:
                _check_tensor(t, f"aux.{f}", dt, numel=n, device=dev, at_least=True)
    y = out if out is not None else torch.empty_like(x)
    L = layer._c()
    b = bias._c() if bias is not None else None
    caux = _Aux(*([_ptr(getattr(aux, f)) for f in Aux.__dataclass_fields__] if aux else [None] * 10), None)
    s = _launch_stream(stream, dev, [y] if out is None else [])
    _check(lib().moe_verify_layer_noalloc(ctypes.byref(L), x.data_ptr(), T, ctypes.byref(b) if b else None,
                                          y.data_ptr(), ctypes.byref(caux), s))
    return y, aux


def union_stats(topk_idx, E: int, counts=None, reuse=None, stream=None):
    """counts [nL] int32 and reuse [nL] float32 for topk_idx [nL, T, k] int32."""
    import torch
    if topk_idx.dtype != torch.int32 or topk_idx.dim() != 3 or not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be a contiguous int32 [nL, T, k] tensor")
    nL, T, k = (int(v) for v in topk_idx.shape)
    owned = []
    if counts is None:
        counts = torch.empty(nL, dtype=torch.int32, device=topk_idx.device)
        owned.append(counts)
    else:
        _check_tensor(counts, "counts", ("int32",), shape=(nL,), device=topk_idx.device)
    if reuse is None:
        reuse = torch.empty(nL, dtype=torch.float32, device=topk_idx.device)
        owned.append(reuse)
    else:
        _check_tensor(reuse, "reuse", ("float32",), shape=(nL,), device=topk_idx.device)
    s = _launch_stream(stream, topk_idx.device, owned)
    _check(lib().union_stats(topk_idx.data_ptr(), nL, T, k, E, counts.data_ptr(), reuse.data_ptr(), s))
    return counts, reuse


def select_drafts(parent, P, Epred, gamma: int, eps: float = 1e-6, out=None, stream=None, static: bool = False):
    """EcoSpec greedy selection for nt trees: parent (host) [N], P [nt, N]
    float32 and Epred [nt, N, W] uint32/int32 (device).  Returns S [nt, gamma]
    int32 (device).  static=True runs the static-cost ablation
    (select_drafts_static)."""
    import torch
    par = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
    if P.dtype != torch.float32 or P.dim() != 2 or not P.is_contiguous():
        raise ValueError("P must be a contiguous float32 [nt, N] tensor")
    if Epred.dim() != 3 or Epred.element_size() != 4 or not Epred.is_contiguous():
        raise ValueError("Epred must be a contiguous 32-bit [nt, N, W] tensor")
    nt, N = (int(v) for v in P.shape)
    if tuple(Epred.shape[:2]) != (nt, N) or par.shape != (N,):
        raise ValueError("shape mismatch between parent, P and Epred")
    W = int(Epred.shape[2])
    if Epred.device != P.device:
        raise ValueError("P and Epred must be on the same device")
    if out is not None:
        _check_tensor(out, "out", ("int32",), shape=(nt, gamma), device=P.device)
    S = out if out is not None else torch.empty((nt, gamma), dtype=torch.int32, device=P.device)
    s = _launch_stream(stream, P.device, [S] if out is None else [])
    fn = lib().select_drafts_static if static else lib().select_drafts
    _check(fn(par.ctypes.data, N, P.data_ptr(), Epred.data_ptr(), W, gamma, eps, nt, S.data_ptr(), s))
    return S


def expand_drafts(parent, P, Epred, t_ar: float, t_exp: float, c_draft=None, stream=None):
    """S2-MoE utility-driven expansion for nt trees: parent (host) [N], P [nt, N]
    float32, Epred [nt, N, W] 32-bit and c_draft [nt, N] float32 or None
    (device).  Returns (S [nt, N] int32 join order padded with -1, count [nt]
    int32), both on the device."""
    import torch
    par = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
    if P.dtype != torch.float32 or P.dim() != 2 or not P.is_contiguous():
        raise ValueError("P must be a contiguous float32 [nt, N] tensor")
    if Epred.dim() != 3 or Epred.element_size() != 4 or not Epred.is_contiguous():
        raise ValueError("Epred must be a contiguous 32-bit [nt, N, W] tensor")
    nt, N = (int(v) for v in P.shape)
    if tuple(Epred.shape[:2]) != (nt, N) or par.shape != (N,):
        raise ValueError("shape mismatch between parent, P and Epred")
    if c_draft is not None and (c_draft.dtype != torch.float32 or tuple(c_draft.shape) != (nt, N)
                                or not c_draft.is_contiguous()):
        raise ValueError("c_draft must be a contiguous float32 [nt, N] tensor")
    if Epred.device != P.device or (c_draft is not None and c_draft.device != P.device):
        raise ValueError("P, Epred and c_draft must be on the same device")
    W = int(Epred.shape[2])
    S = torch.empty((nt, N), dtype=torch.int32, device=P.device)
    count = torch.empty((nt,), dtype=torch.int32, device=P.device)
    s = _launch_stream(stream, P.device, [S, count])
    _check(lib().expand_drafts(par.ctypes.data, N, P.data_ptr(), Epred.data_ptr(), W, t_ar, t_exp,
                               c_draft.data_ptr() if c_draft is not None else None, nt, S.data_ptr(),
                               count.data_ptr(), s))
    return S, count


def union_stats_segments(topk_idx, E: int, offsets, stream=None):
    """Per-sequence unique experts of a call grouped by sequence:
    topk_idx [nL, T, k] int32 (device), offsets (host) [S + 1].  Returns
    (per [nL, S] int32, total [nL] int32) on the device."""
    import torch
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int32))
    if topk_idx.dtype != torch.int32 or topk_idx.dim() != 3 or not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be a contiguous int32 [nL, T, k] tensor")
    nL, T, k = (int(v) for v in topk_idx.shape)
    S = int(off.shape[0]) - 1
    per = torch.empty((nL, S), dtype=torch.int32, device=topk_idx.device)
    total = torch.empty((nL,), dtype=torch.int32, device=topk_idx.device)
    s = _launch_stream(stream, topk_idx.device, [per, total])
    _check(lib().union_stats_segments(topk_idx.data_ptr(), nL, T, k, E, off.ctypes.data, S, per.data_ptr(),
                                      total.data_ptr(), s))
    return per, total


def gate_depths(c, Epred, t_base: float, t_exp: float, stream=None):
    """Confidence-gated depths: c [S, Dmax + 1] float32 cumulative confidences
    and Epred [S, Dmax + 1, W] 32-bit expert bitsets (device).  Returns d [S]
    int32 (device)."""
    import torch
    if c.dtype != torch.float32 or c.dim() != 2 or not c.is_contiguous():
        raise ValueError("c must be a contiguous float32 [S, Dmax + 1] tensor")
    if Epred.dim() != 3 or Epred.element_size() != 4 or not Epred.is_contiguous():
        raise ValueError("Epred must be a contiguous 32-bit [S, Dmax + 1, W] tensor")
    S, D1 = (int(v) for v in c.shape)
    if tuple(Epred.shape[:2]) != (S, D1):
        raise ValueError("shape mismatch between c and Epred")
    if Epred.device != c.device:
        raise ValueError("c and Epred must be on the same device")
    d = torch.empty((S,), dtype=torch.int32, device=c.device)
    s = _launch_stream(stream, c.device, [d])
    _check(lib().gate_depths(c.data_ptr(), Epred.data_ptr(), S, D1 - 1, int(Epred.shape[2]), t_base, t_exp,
                             d.data_ptr(), s))
    return d
