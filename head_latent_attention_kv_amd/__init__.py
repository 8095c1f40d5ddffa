"""Python binding of libmla_laga.so, the MI355X latent-attention block.

The names follow the C ABI in include/mla_laga.h. This layer only marshals
arguments: it reads shapes off torch tensors, allocates outputs and the
workspace with torch (device memory and the current stream are all torch is
used for) and calls the library. Every step of the computation runs in the
library's HIP kernels; if the library is not built, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = [
    "MLAError", "MLADesc", "load_library", "library_path", "mla_laga_fwd", "mla_laga_bwd",
    "mla_laga_fwd_workspace_size", "mla_laga_bwd_workspace_size", "mla_laga_count",
    "mla_laga_uses_fast_path", "MLACall", "MLA_F32", "MLA_BF16", "MLA_FLAG_GENERIC", "MLA_FLAG_STORED_DS",
    "MLA_MAX_RANGES", "MLADecodeDesc", "MLADecodeCall", "mla_laga_decode",
    "mla_laga_decode_workspace_size", "mla_laga_decode_noalloc", "MLA_DECODE_NOALLOC_MAX_BYTES",
    "mla_laga_row_window", "MLA_ERR_DEBUG_CHECK",
]

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = 0, -1, -2, -3, -4
MLA_ERR_DEBUG_CHECK = -5
MLA_F32, MLA_BF16 = 0, 1
MLA_FLAG_GENERIC = 1
MLA_FLAG_STORED_DS = 4
MLA_MAX_RANGES = 16
MLA_DECODE_NOALLOC_MAX_BYTES = 256 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    """The in-tree build, unless MLA_LAGA_LIBRARY names another build of it."""
    return os.environ.get("MLA_LAGA_LIBRARY") or os.path.join(_HERE, "libmla_laga.so")


class MLAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


class MLADesc(ctypes.Structure):
    _fields_ = [
        ("n_h", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_rope", ctypes.c_int32),
        ("d_nope", ctypes.c_int32), ("d_v", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
        ("S", ctypes.c_int64), ("S_loc", ctypes.c_int64), ("q_offset", ctypes.c_int64),
        ("in_dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("n_ranges", ctypes.c_int32), ("q_ranges", ctypes.POINTER(ctypes.c_int64)),
    ]


class MLADecodeDesc(ctypes.Structure):
    _fields_ = [
        ("n_h", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_rope", ctypes.c_int32),
        ("d_nope", ctypes.c_int32), ("d_v", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("S", ctypes.c_int64), ("in_dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
    ]


_lib = None
_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)
_DESCP = ctypes.POINTER(MLADesc)
_DDESCP = ctypes.POINTER(MLADecodeDesc)

EXPORTED = {
    "mla_laga_fwd_workspace_size": (ctypes.c_int, [_DESCP, _I32P, ctypes.POINTER(ctypes.c_size_t)]),
    "mla_laga_bwd_workspace_size": (ctypes.c_int, [_DESCP, _I32P, ctypes.POINTER(ctypes.c_size_t)]),
    "mla_laga_fwd": (ctypes.c_int, [_DESCP, _P, _P, _P, _P, _P, _I32P, _P, _P, _P, _P,
                                    ctypes.c_size_t, _P]),
    "mla_laga_bwd": (ctypes.c_int, [_DESCP, _P, _P, _P, _P, _P, _P, _I32P, _P, _P, _P,
                                    _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "mla_laga_count": (ctypes.c_int, [_DESCP, _I32P, _I64P, _I64P, _I64P]),
    "mla_laga_decode_workspace_size": (ctypes.c_int, [_DDESCP, _I32P, ctypes.POINTER(ctypes.c_size_t)]),
    "mla_laga_decode": (ctypes.c_int, [_DDESCP, _P, _P, _P, _P, _P, _I32P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]),
    "mla_laga_decode_noalloc": (ctypes.c_int, [_DDESCP, _P, _P, _P, _P, _P, _I32P, _P, _P, _P, _P]),
    "mla_laga_uses_fast_path": (ctypes.c_int, [_DESCP]),
    "mla_laga_row_window": (ctypes.c_int, [_DESCP, _I32P, _P, _P, _P]),
    "mla_laga_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "mla_laga_timing_select": (ctypes.c_int, [ctypes.c_char_p]),
    "mla_laga_timing_read": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), _I64P]),
    "mla_laga_timing_names": (ctypes.c_char_p, []),
    "mla_laga_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_laga_last_error": (ctypes.c_char_p, []),
}


def load_library():
    """Load libmla_laga.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m head_latent_attention_kv_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTED.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _status_name(s: int) -> str:
    try:
        return load_library().mla_laga_status_string(s).decode()
    except ImportError:
        return str(s)


def _check(status: int):
    if status != MLA_OK:
        raise MLAError(status, load_library().mla_laga_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _in_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    if t.dtype == torch.float32:
        return MLA_F32
    raise TypeError(f"inputs must be bfloat16 or float32, got {t.dtype}")


def _host_cu(cu_seqlens) -> Optional[np.ndarray]:
    if cu_seqlens is None:
        return None
    if isinstance(cu_seqlens, torch.Tensor):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))


def _cu_ptr(cu: Optional[np.ndarray]):
    return None if cu is None else cu.ctypes.data_as(_I32P)


def _host_ranges(q_ranges) -> Optional[np.ndarray]:
    if q_ranges is None:
        return None
    r = np.ascontiguousarray(np.asarray(q_ranges, dtype=np.int64).reshape(-1, 2))
    return r


def make_desc(q: torch.Tensor, c_kv: torch.Tensor, k_rope: torch.Tensor, W_UV: torch.Tensor,
              q_offset: int = 0, cu_seqlens=None, softmax_scale: Optional[float] = None,
              generic: bool = False, q_ranges=None, stored_ds: bool = False
              ) -> Tuple[MLADesc, Optional[np.ndarray], Optional[np.ndarray]]:
    """Descriptor plus the host arrays it points at (cu_seqlens, ranges):
    keep those alive as long as the descriptor is used. stored_ds sets
    MLA_FLAG_STORED_DS (the backward keeps dS, all heads at once up to 16 GiB,
    else in head groups of 8 or more heads and at most 1 GiB through two
    buffers, and dQ reads it instead of recomputing the scores)."""
    S_loc, n_h, d_qk = q.shape
    S, d_c = c_kv.shape
    d_rope = k_rope.shape[1]
    cu = _host_cu(cu_seqlens)
    d = MLADesc()
    d.n_h, d.d_c, d.d_rope = n_h, d_c, d_rope
    d.d_nope, d.d_v = d_qk - d_rope, W_UV.shape[1] // n_h
    d.n_seqs = 0 if cu is None else len(cu) - 1
    d.S, d.S_loc, d.q_offset = S, S_loc, int(q_offset)
    d.in_dtype = _in_dtype(q)
    d.flags = (MLA_FLAG_GENERIC if generic else 0) | (MLA_FLAG_STORED_DS if stored_ds else 0)
    d.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
    rng = _host_ranges(q_ranges)
    d.n_ranges = 0 if rng is None else len(rng)
    d.q_ranges = None if rng is None else rng.ctypes.data_as(_I64P)
    return d, cu, rng


def _check_inputs(d: MLADesc, tensors, dtype=None):
    """Every tensor must exist on the device, be contiguous, have its shape
    and share one dtype (`dtype` when given). The library reads and writes
    raw pointers, so a wrong shape or dtype here would run off a buffer."""
    dt = dtype
    for name, t, shape in tensors:
        if t is None:
            raise ValueError(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        dt = t.dtype if dt is None else dt
        if t.dtype != dt:
            raise ValueError(f"{name} is {t.dtype}, expected {dt}")


def _in_torch_dtype(d: MLADesc):
    return torch.bfloat16 if d.in_dtype == MLA_BF16 else torch.float32


def _output_specs(d: MLADesc, out, lse):
    return [("out", out, (d.S_loc, d.n_h, d.d_v)), ("lse", lse, (d.S_loc, d.n_h))]


def _grad_specs(d: MLADesc, grads):
    if len(grads) != 5:
        raise ValueError("grads must be (dq, dc_kv, dk_rope, dW_UK, dW_UV)")
    shapes = [(d.S_loc, d.n_h, d.d_nope + d.d_rope), (d.S, d.d_c), (d.S, d.d_rope),
              (d.d_c, d.n_h * d.d_nope), (d.d_c, d.n_h * d.d_v)]
    return list(zip(("dq", "dc_kv", "dk_rope", "dW_UK", "dW_UV"), grads, shapes))


def _input_specs(d: MLADesc, q, c_kv, k_rope, W_UK, W_UV):
    d_qk = d.d_nope + d.d_rope
    return [("q", q, (d.S_loc, d.n_h, d_qk)), ("c_kv", c_kv, (d.S, d.d_c)),
            ("k_rope", k_rope, (d.S, d.d_rope)), ("W_UK", W_UK, (d.d_c, d.n_h * d.d_nope)),
            ("W_UV", W_UV, (d.d_c, d.n_h * d.d_v))]


def mla_laga_fwd_workspace_size(desc: MLADesc, cu: Optional[np.ndarray] = None) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().mla_laga_fwd_workspace_size(ctypes.byref(desc), _cu_ptr(cu), ctypes.byref(n)))
    return n.value


def mla_laga_bwd_workspace_size(desc: MLADesc, cu: Optional[np.ndarray] = None) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().mla_laga_bwd_workspace_size(ctypes.byref(desc), _cu_ptr(cu), ctypes.byref(n)))
    return n.value


def mla_laga_count(desc: MLADesc, cu: Optional[np.ndarray] = None) -> Tuple[int, int, int]:
    """(visible pairs per head, key_lo, key_hi) from the library's host plan."""
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().mla_laga_count(ctypes.byref(desc), _cu_ptr(cu), ctypes.byref(a),
                                         ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def mla_laga_uses_fast_path(desc: MLADesc) -> bool:
    return bool(load_library().mla_laga_uses_fast_path(ctypes.byref(desc)))


def mla_laga_row_window(desc: MLADesc, cu: Optional[np.ndarray] = None,
                        cu_dev: Optional[torch.Tensor] = None, device="cuda") -> torch.Tensor:
    """int64 [S_loc, 2]: the first and last global key position each local
    row of `desc` sees, as the library's kernels compute them. `cu` and
    `cu_dev` hold the same cu_seqlens on the host and the device."""
    if (cu is None) != (cu_dev is None):
        raise ValueError("cu and cu_dev go together")
    if cu_dev is not None:
        _check_inputs(desc, [("cu_dev", cu_dev, (len(cu),))], torch.int32)
    w = torch.empty((desc.S_loc, 2), dtype=torch.int64, device=device)
    stream = torch.cuda.current_stream(w.device).cuda_stream
    _check(load_library().mla_laga_row_window(ctypes.byref(desc), _cu_ptr(cu), _ptr(cu_dev),
                                              _ptr(w) if desc.S_loc > 0 else None,
                                              ctypes.c_void_p(stream)))
    return w


def timing_enable(on: bool = True):
    """Bracket every library kernel with HIP events on its stream (and forget
    earlier records)."""
    _check(load_library().mla_laga_timing_enable(1 if on else 0))


def timing_select(names=None):
    """Bracket only the kernels named in `names` (a list; None: every kernel)."""
    arg = None if not names else ";".join(names).encode()
    _check(load_library().mla_laga_timing_select(arg))


def timing_read(kernel: str) -> Tuple[float, int]:
    """(summed ms, launches) of the recorded kernels named `kernel`; waits for them."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(load_library().mla_laga_timing_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def timing_names():
    return [n for n in load_library().mla_laga_timing_names().decode().split(";") if n]


def _workspace(nbytes: int, device) -> torch.Tensor:
    # the caching allocator returns 512-byte aligned blocks
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


class MLACall:
    """One shard's shapes, prepared once: descriptor, host and device
    cu_seqlens and workspaces, for repeated forward/backward calls."""

    def __init__(self, q, c_kv, k_rope, W_UK, W_UV, q_offset: int = 0, cu_seqlens=None,
                 softmax_scale: Optional[float] = None, generic: bool = False,
                 backward: bool = False, q_ranges=None, stored_ds: bool = False):
        self.desc, self.cu, self.ranges = make_desc(q, c_kv, k_rope, W_UV, q_offset, cu_seqlens,
                                                    softmax_scale, generic, q_ranges, stored_ds)
        _check_inputs(self.desc, _input_specs(self.desc, q, c_kv, k_rope, W_UK, W_UV))
        self.device = q.device
        self.cu_dev = None if self.cu is None else torch.from_numpy(self.cu).to(self.device)
        self.ws_fwd = _workspace(mla_laga_fwd_workspace_size(self.desc, self.cu), self.device)
        self.ws_bwd = (_workspace(mla_laga_bwd_workspace_size(self.desc, self.cu), self.device)
                       if backward else None)

    @property
    def fast(self) -> bool:
        return mla_laga_uses_fast_path(self.desc)

    def _check_call(self, q, c_kv, k_rope, W_UK, W_UV):
        d = self.desc
        _check_inputs(d, _input_specs(d, q, c_kv, k_rope, W_UK, W_UV), _in_torch_dtype(d))
        for name, t in (("q", q), ("c_kv", c_kv), ("k_rope", k_rope), ("W_UK", W_UK), ("W_UV", W_UV)):
            if t.device != self.device:
                raise ValueError(f"{name} is on {t.device}, the call was prepared on {self.device}")

    def fwd(self, q, c_kv, k_rope, W_UK, W_UV, out=None, lse=None):
        d = self.desc
        self._check_call(q, c_kv, k_rope, W_UK, W_UV)
        if out is None:
            out = torch.empty((d.S_loc, d.n_h, d.d_v), dtype=torch.float32, device=self.device)
        if lse is None:
            lse = torch.empty((d.S_loc, d.n_h), dtype=torch.float32, device=self.device)
        _check_inputs(d, _output_specs(d, out, lse), torch.float32)
        stream = torch.cuda.current_stream(self.device).cuda_stream
        _check(load_library().mla_laga_fwd(
            ctypes.byref(d), _ptr(q), _ptr(c_kv), _ptr(k_rope), _ptr(W_UK), _ptr(W_UV),
            _cu_ptr(self.cu), _ptr(self.cu_dev), _ptr(out), _ptr(lse), _ptr(self.ws_fwd),
            self.ws_fwd.numel(), ctypes.c_void_p(stream)))
        return out, lse

    def bwd(self, dout, q, c_kv, k_rope, W_UK, W_UV, out, lse, grads=None):
        d = self.desc
        self._check_call(q, c_kv, k_rope, W_UK, W_UV)
        _check_inputs(d, [("dout", dout, (d.S_loc, d.n_h, d.d_v))], _in_torch_dtype(d))
        _check_inputs(d, _output_specs(d, out, lse), torch.float32)
        if grads is not None:
            _check_inputs(d, _grad_specs(d, grads), torch.float32)
        if self.ws_bwd is None:
            self.ws_bwd = _workspace(mla_laga_bwd_workspace_size(d, self.cu), self.device)
        f32 = dict(dtype=torch.float32, device=self.device)
        if grads is None:
            grads = (torch.empty((d.S_loc, d.n_h, d.d_nope + d.d_rope), **f32),
                     torch.empty((d.S, d.d_c), **f32), torch.empty((d.S, d.d_rope), **f32),
                     torch.empty((d.d_c, d.n_h * d.d_nope), **f32),
                     torch.empty((d.d_c, d.n_h * d.d_v), **f32))
        dq, dc_kv, dk_rope, dW_UK, dW_UV = grads
        stream = torch.cuda.current_stream(self.device).cuda_stream
        _check(load_library().mla_laga_bwd(
            ctypes.byref(d), _ptr(dout), _ptr(q), _ptr(c_kv), _ptr(k_rope), _ptr(W_UK),
            _ptr(W_UV), _cu_ptr(self.cu), _ptr(self.cu_dev), _ptr(out), _ptr(lse), _ptr(dq),
            _ptr(dc_kv), _ptr(dk_rope), _ptr(dW_UK), _ptr(dW_UV), _ptr(self.ws_bwd),
            self.ws_bwd.numel(), ctypes.c_void_p(stream)))
        return grads


def mla_laga_fwd(q, c_kv, k_rope, W_UK, W_UV, q_offset: int = 0, cu_seqlens=None,
                 softmax_scale: Optional[float] = None, generic: bool = False, q_ranges=None):
    """out [S_loc,n_h,d_v] fp32 and lse [S_loc,n_h] fp32 for one query shard.
    q_ranges: optional (start, length) position blocks of the rows (q_offset 0)."""
    call = MLACall(q, c_kv, k_rope, W_UK, W_UV, q_offset, cu_seqlens, softmax_scale, generic,
                   q_ranges=q_ranges)
    return call.fwd(q, c_kv, k_rope, W_UK, W_UV)


def mla_laga_bwd(dout, q, c_kv, k_rope, W_UK, W_UV, out, lse, q_offset: int = 0,
                 cu_seqlens=None, softmax_scale: Optional[float] = None, generic: bool = False,
                 q_ranges=None, stored_ds: bool = False):
    """(dq, dc_kv, dk_rope, dW_UK, dW_UV), all fp32, gradients of sum(out*dout).
    stored_ds: keep dS in the workspace for dQ (faster; memory grows with
    rows x keys)."""
    call = MLACall(q, c_kv, k_rope, W_UK, W_UV, q_offset, cu_seqlens, softmax_scale, generic,
                   backward=True, q_ranges=q_ranges, stored_ds=stored_ds)
    return call.bwd(dout, q, c_kv, k_rope, W_UK, W_UV, out, lse)


# ------------------------------------------------------------------ decode
def make_decode_desc(q: torch.Tensor, c_kv: torch.Tensor, k_rope: torch.Tensor,
                     W_UV: torch.Tensor, cu_seqlens,
                     softmax_scale: Optional[float] = None) -> Tuple[MLADecodeDesc, np.ndarray]:
    batch, n_h, d_qk = q.shape
    S, d_c = c_kv.shape
    d_rope = k_rope.shape[1]
    cu = _host_cu(cu_seqlens)
    d = MLADecodeDesc()
    d.n_h, d.d_c, d.d_rope = n_h, d_c, d_rope
    d.d_nope, d.d_v = d_qk - d_rope, W_UV.shape[1] // n_h
    d.batch, d.S = batch, S
    d.in_dtype = _in_dtype(q)
    d.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
    return d, cu


def mla_laga_decode_workspace_size(desc: MLADecodeDesc, cu: np.ndarray) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().mla_laga_decode_workspace_size(ctypes.byref(desc), _cu_ptr(cu),
                                                          ctypes.byref(n)))
    return n.value


class MLADecodeCall:
    """One decode batch's shapes, prepared once: one query per sequence over
    the latent cache (c_kv, k_rope) packed by cu_seqlens."""

    def __init__(self, q, c_kv, k_rope, W_UK, W_UV, cu_seqlens,
                 softmax_scale: Optional[float] = None):
        self.desc, self.cu = make_decode_desc(q, c_kv, k_rope, W_UV, cu_seqlens, softmax_scale)
        d = self.desc
        _check_inputs(d, self._specs(q, c_kv, k_rope, W_UK, W_UV))
        self.device = q.device
        self.cu_dev = torch.from_numpy(self.cu).to(self.device)
        self.ws = _workspace(mla_laga_decode_workspace_size(d, self.cu), self.device)

    def _specs(self, q, c_kv, k_rope, W_UK, W_UV):
        d = self.desc
        return [("q", q, (d.batch, d.n_h, d.d_nope + d.d_rope)),
                ("c_kv", c_kv, (d.S, d.d_c)), ("k_rope", k_rope, (d.S, d.d_rope)),
                ("W_UK", W_UK, (d.d_c, d.n_h * d.d_nope)), ("W_UV", W_UV, (d.d_c, d.n_h * d.d_v))]

    def __call__(self, q, c_kv, k_rope, W_UK, W_UV, out=None, lse=None):
        d = self.desc
        _check_inputs(d, self._specs(q, c_kv, k_rope, W_UK, W_UV), _in_torch_dtype(d))
        if out is None:
            out = torch.empty((d.batch, d.n_h, d.d_v), dtype=torch.float32, device=self.device)
        if lse is None:
            lse = torch.empty((d.batch, d.n_h), dtype=torch.float32, device=self.device)
        _check_inputs(d, [("out", out, (d.batch, d.n_h, d.d_v)), ("lse", lse, (d.batch, d.n_h))],
                      torch.float32)
        stream = torch.cuda.current_stream(self.device).cuda_stream
        _check(load_library().mla_laga_decode(
            ctypes.byref(d), _ptr(q), _ptr(c_kv), _ptr(k_rope), _ptr(W_UK), _ptr(W_UV),
            _cu_ptr(self.cu), _ptr(self.cu_dev), _ptr(out), _ptr(lse), _ptr(self.ws),
            self.ws.numel(), ctypes.c_void_p(stream)))
        return out, lse


def mla_laga_decode_noalloc(q, c_kv, k_rope, W_UK, W_UV, cu_seqlens, cu_seqlens_dev, out, lse,
                            softmax_scale: Optional[float] = None):
    """The decode into the caller's out [batch,n_h,d_v] and lse [batch,n_h]
    (fp32) with the library's static scratch instead of a workspace: the
    library allocates nothing. cu_seqlens (host) and cu_seqlens_dev (an int32
    device tensor) hold the same batch+1 values."""
    d, cu = make_decode_desc(q, c_kv, k_rope, W_UV, cu_seqlens, softmax_scale)
    _check_inputs(d, [("q", q, (d.batch, d.n_h, d.d_nope + d.d_rope)),
                      ("c_kv", c_kv, (d.S, d.d_c)), ("k_rope", k_rope, (d.S, d.d_rope)),
                      ("W_UK", W_UK, (d.d_c, d.n_h * d.d_nope)),
                      ("W_UV", W_UV, (d.d_c, d.n_h * d.d_v))], _in_torch_dtype(d))
    _check_inputs(d, [("out", out, (d.batch, d.n_h, d.d_v)), ("lse", lse, (d.batch, d.n_h))],
                  torch.float32)
    _check_inputs(d, [("cu_seqlens_dev", cu_seqlens_dev, (d.batch + 1,))], torch.int32)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(load_library().mla_laga_decode_noalloc(
        ctypes.byref(d), _ptr(q), _ptr(c_kv), _ptr(k_rope), _ptr(W_UK), _ptr(W_UV), _cu_ptr(cu),
        _ptr(cu_seqlens_dev), _ptr(out), _ptr(lse), ctypes.c_void_p(stream)))
    return out, lse


def mla_laga_decode(q, c_kv, k_rope, W_UK, W_UV, cu_seqlens,
                    softmax_scale: Optional[float] = None):
    """out [batch,n_h,d_v] fp32 and lse [batch,n_h] fp32: one query per
    sequence (at its last cached position) over the latent cache."""
    return MLADecodeCall(q, c_kv, k_rope, W_UK, W_UV, cu_seqlens, softmax_scale)(
        q, c_kv, k_rope, W_UK, W_UV)
