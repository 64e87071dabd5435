"""Compressed-key attention scoring on MI355X (gfx950): Python binding.

Thin ctypes layer over the C ABI in ``include/tq.h`` (library ``libtq.so``,
built in-tree by ``python compressed_attention_scoring_amd/build.py``). The
functions keep the C names:

    tq_query_transform(q, Pi, S_mat)           -> (A, T)
    tq_score(A, T, keys, codebook)             -> scores
    tq_score_with_kernel(A, T, keys, codebook, kernel)
    tq_decode_debug(keys, D)                   -> (idx, sign, gamma)
    tq_compress_keys(keys, Pi, S_mat, codebook, layout, bits) -> Keys (with .norm)
    tq_attend(scores, values, codebook, Pi_v, scale) -> out
    tq_attend_workspace_bytes(P, B, S, D)
    tq_score_attend(A, T, keys, codebook, values, codebook_v, Pi_v, scale) -> out   (fused decode step)
    tq_query_transform_hadamard(q, signs)      -> A
    tq_score_mse(A, keys, codebook)            -> scores   (MSE-only keys: Values format)
    tq_query_transform_split(q, perm, Pi_hi, Pi_lo, D_hi) -> (A_hi, A_lo)
    tq_score_split(A_hi, A_lo, SplitKeys, codebook_hi, codebook_lo) -> scores
    tq_score_kernel_name(layout, bits, C, P, B, S, D, kernel)

Only argument marshalling happens here: shapes, dtypes, contiguity and device
are checked, output tensors are allocated with torch, and pointers plus the
current HIP stream are handed to the library. Every step of the computation
runs in the library's HIP kernels. There is no CPU fallback: importing this
package raises if ``libtq.so`` is missing, and tensors not on a GPU are refused.
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

__all__ = [
    "Keys", "Values", "TqError", "tq_attend", "tq_attend_workspace_bytes", "tq_query_transform_hadamard",
    "tq_score_mse", "tq_score_attend", "tq_attend_no_alloc", "tq_score_attend_workspace_bytes", "SplitKeys", "tq_query_transform_split", "tq_score_split", "tq_query_transform", "tq_score", "tq_score_with_kernel",
    "tq_decode_debug", "tq_compress_keys", "tq_score_kernel_name", "tq_status_string", "library_path",
    "TQ_UNPACKED", "TQ_PACKED", "KERNELS", "TQ_OK", "TQ_ERR_ARG", "TQ_ERR_UNSUPPORTED", "TQ_ERR_ALIGN", "TQ_NO_ALLOC_SCRATCH_BYTES",
    "TQ_ERR_LAUNCH",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libtq.so")
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "tq.h")

TQ_OK = 0
TQ_ERR_ARG = -1
TQ_ERR_UNSUPPORTED = -2
TQ_ERR_ALIGN = -3
TQ_ERR_LAUNCH = -4
#: bytes of the per-GPU scratch tq_attend_no_alloc uses as its workspace (tq.h)
TQ_NO_ALLOC_SCRATCH_BYTES = 48 * 1024 * 1024
TQ_UNPACKED = 0
TQ_PACKED = 1
KERNELS = {"auto": 0, "valu": 1, "mfma": 2, "mfma_lds": 3, "mfma_reg": 4, "mfma16": 5, "mfma_shared": 6,
           "mfma_f16": 7}   # mfma_f16: single-pass f16, 2e-2 accuracy (tq.h)


class _CKeys(ctypes.Structure):
    _fields_ = [
        ("layout", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("idx", ctypes.c_void_p),
        ("sign", ctypes.c_void_p),
        ("gamma", ctypes.c_void_p),
    ]


class _CKeysOut(ctypes.Structure):
    _fields_ = [
        ("layout", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("idx", ctypes.c_void_p),
        ("sign", ctypes.c_void_p),
        ("gamma", ctypes.c_void_p),
        ("norm", ctypes.c_void_p),
    ]


class _CValues(ctypes.Structure):
    _fields_ = [
        ("layout", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("idx", ctypes.c_void_p),
        ("norm", ctypes.c_void_p),
    ]


class _CSplit(ctypes.Structure):
    _fields_ = [("hi", _CValues), ("lo", _CValues)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python compressed_attention_scoring_amd/build.py` "
            "(needs hipcc) before using the library")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.tq_query_transform.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
    lib.tq_query_transform.restype = i32
    lib.tq_score.argtypes = [vp, vp, ctypes.POINTER(_CKeys), vp, i32, vp, i32, i32, i32, i32, vp]
    lib.tq_score.restype = i32
    lib.tq_score_with_kernel.argtypes = [vp, vp, ctypes.POINTER(_CKeys), vp, i32, vp,
                                         i32, i32, i32, i32, i32, vp]
    lib.tq_score_with_kernel.restype = i32
    lib.tq_score_kernel_name.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    lib.tq_score_kernel_name.restype = ctypes.c_char_p
    lib.tq_decode_debug.argtypes = [ctypes.POINTER(_CKeys), vp, vp, vp, i32, i32, i32, vp]
    lib.tq_decode_debug.restype = i32
    lib.tq_compress_keys.argtypes = [vp, vp, vp, vp, i32, ctypes.POINTER(_CKeysOut), i32, i32, i32, i32, vp]
    lib.tq_compress_keys.restype = i32
    lib.tq_attend_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.tq_attend_workspace_bytes.restype = ctypes.c_size_t
    lib.tq_attend.argtypes = [vp, ctypes.POINTER(_CValues), vp, i32, vp, ctypes.c_float, vp, vp, ctypes.c_size_t,
                              i32, i32, i32, i32, i32, vp]
    lib.tq_attend.restype = i32
    lib.tq_attend_no_alloc.argtypes = [vp, ctypes.POINTER(_CValues), vp, i32, vp, ctypes.c_float, vp,
                                       i32, i32, i32, i32, i32, vp]
    lib.tq_attend_no_alloc.restype = i32
    sz = ctypes.c_size_t
    lib.tq_probe_read.argtypes = [vp, sz, vp, vp]
    lib.tq_probe_read.restype = i32
    lib.tq_probe_write.argtypes = [vp, sz, vp]
    lib.tq_probe_write.restype = i32
    lib.tq_probe_read_write.argtypes = [vp, sz, vp, sz, vp]
    lib.tq_probe_read_write.restype = i32
    lib.tq_score_attend_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.tq_score_attend_workspace_bytes.restype = ctypes.c_size_t
    lib.tq_score_attend.argtypes = [vp, vp, ctypes.POINTER(_CKeys), vp, i32, ctypes.POINTER(_CValues), vp, i32, vp,
                                    ctypes.c_float, vp, vp, ctypes.c_size_t, i32, i32, i32, i32, i32, vp]
    lib.tq_score_attend.restype = i32
    lib.tq_score_attend_with_mode.argtypes = [vp, vp, ctypes.POINTER(_CKeys), vp, i32, ctypes.POINTER(_CValues), vp,
                                              i32, vp, ctypes.c_float, vp, vp, ctypes.c_size_t, i32, i32, i32, i32,
                                              i32, i32, vp]
    lib.tq_score_attend_with_mode.restype = i32
    lib.tq_query_transform_hadamard.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
    lib.tq_query_transform_hadamard.restype = i32
    lib.tq_score_mse.argtypes = [vp, ctypes.POINTER(_CValues), vp, i32, vp, i32, i32, i32, i32, vp]
    lib.tq_score_mse.restype = i32
    lib.tq_query_transform_split.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.tq_query_transform_split.restype = i32
    lib.tq_score_split.argtypes = [vp, vp, ctypes.POINTER(_CSplit), vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, vp]
    lib.tq_score_split.restype = i32
    lib.tq_status_string.argtypes = [i32]
    lib.tq_status_string.restype = ctypes.c_char_p
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def header_functions() -> list[str]:
    """Names of the functions ``include/tq.h`` declares."""
    with open(_HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(tq_\w+)\s*\(", text, re.M)))


class TqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {tq_status_string(status)} (status {status})")


def tq_status_string(status: int) -> str:
    return _lib.tq_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != TQ_OK:
        raise TqError(status, where)


def _gpu(t: torch.Tensor, name: str, dtype) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a GPU (got {t.device}); there is no CPU path")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(device: torch.device, stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


@dataclass
class Keys:
    """Compressed keys of P problems with S keys of D coordinates each.

    layout "unpacked": idx uint8 [P,S,D], sign int8 [P,S,D] (+-1), gamma float32 [P,S].
    layout "packed":   idx uint8 [P,S,D*bits/8] (LSB-first bitstream), sign uint8 [P,S,D/8]
                       (bit 1 = +1), gamma float16 [P,S]; bits 2 or 3.
    A leading problem axis may be omitted (P = 1).
    """
    layout: str
    idx: torch.Tensor
    sign: torch.Tensor
    gamma: torch.Tensor
    bits: int = 0
    #: the keys' lengths ||k|| (gamma's dtype) when produced by tq_compress_keys, else None;
    #: scores are against the unit keys, norm * score is the score against k as given
    norm: torch.Tensor | None = None

    def _c(self, D: int):
        if self.layout == "unpacked":
            lay, bits = TQ_UNPACKED, 0
            _gpu(self.idx, "keys.idx", torch.uint8)
            _gpu(self.sign, "keys.sign", torch.int8)
            _gpu(self.gamma, "keys.gamma", torch.float32)
            row_i, row_s = D, D
        elif self.layout == "packed":
            lay, bits = TQ_PACKED, int(self.bits)
            _gpu(self.idx, "keys.idx", torch.uint8)
            _gpu(self.sign, "keys.sign", torch.uint8)
            _gpu(self.gamma, "keys.gamma", torch.float16)
            if bits not in (2, 3) or D % 8:
                raise ValueError("packed keys need bits in (2, 3) and D % 8 == 0")
            row_i, row_s = D * bits // 8, D // 8
        else:
            raise ValueError(f"unknown layout {self.layout!r}")
        g = self.gamma if self.gamma.dim() == 2 else self.gamma.unsqueeze(0)
        P, S = g.shape
        if self.idx.numel() != P * S * row_i or self.sign.numel() != P * S * row_s:
            raise ValueError(f"key streams do not match gamma's [P={P}, S={S}] with D={D}")
        return _CKeys(lay, bits, self.idx.data_ptr(), self.sign.data_ptr(), self.gamma.data_ptr()), P, S

    @property
    def device(self) -> torch.device:
        return self.gamma.device


def _as3(t: torch.Tensor) -> torch.Tensor:
    return t if t.dim() == 3 else t.unsqueeze(0)


def tq_query_transform(q: torch.Tensor, Pi: torch.Tensor, S_mat: torch.Tensor,
                       A: torch.Tensor | None = None, T: torch.Tensor | None = None,
                       stream=None):
    """A = Pi q and T = S_mat q. q [P,B,D] or [B,D]; Pi, S_mat [H,D,D] or [D,D]."""
    squeeze = q.dim() == 2
    q3 = _as3(_gpu(q, "q", torch.float32))
    Pi3 = _as3(_gpu(Pi, "Pi", torch.float32))
    S3 = _as3(_gpu(S_mat, "S_mat", torch.float32))
    P, B, D = q3.shape
    H = Pi3.shape[0]
    if Pi3.shape != (H, D, D) or S3.shape != (H, D, D):
        raise ValueError(f"Pi and S_mat must be [H, {D}, {D}]")
    if A is None:
        A = torch.empty_like(q3)
    if T is None:
        T = torch.empty_like(q3)
    _gpu(A, "A", torch.float32)
    _gpu(T, "T", torch.float32)
    if A.numel() != q3.numel() or T.numel() != q3.numel():
        raise ValueError("A and T must have q's shape")
    st = _stream(q.device, stream)
    _check(_lib.tq_query_transform(_ptr(q3), _ptr(Pi3), _ptr(S3), _ptr(A), _ptr(T),
                                   P, H, B, D, st), "tq_query_transform")
    if squeeze:
        return A.view(B, D), T.view(B, D)
    return A.view(P, B, D), T.view(P, B, D)


def tq_score_with_kernel(A: torch.Tensor, T: torch.Tensor, keys: Keys, codebook: torch.Tensor,
                         kernel: str = "auto", scores: torch.Tensor | None = None, stream=None):
    """Raw scores [P,B,S] (or [B,S] for 2-D A) with an explicit kernel family."""
    squeeze = A.dim() == 2
    A3 = _as3(_gpu(A, "A", torch.float32))
    T3 = _as3(_gpu(T, "T", torch.float32))
    _gpu(codebook, "codebook", torch.float32)
    if A3.shape != T3.shape:
        raise ValueError("A and T must have the same shape")
    P, B, D = A3.shape
    ck, Pk, S = keys._c(D)
    if Pk != P:
        raise ValueError(f"keys hold {Pk} problems, A holds {P}")
    if scores is None:
        scores = torch.empty((P, B, S), dtype=torch.float32, device=A.device)
    _gpu(scores, "scores", torch.float32)
    if scores.numel() != P * B * S:
        raise ValueError("scores must hold P*B*S floats")
    st = _stream(A.device, stream)
    _check(_lib.tq_score_with_kernel(_ptr(A3), _ptr(T3), ctypes.byref(ck), _ptr(codebook),
                                     codebook.numel(), _ptr(scores), P, B, S, D,
                                     KERNELS[kernel], st), "tq_score")
    return scores.view(B, S) if squeeze else scores.view(P, B, S)


def tq_score(A, T, keys: Keys, codebook, scores=None, stream=None):
    """Raw scores [P,B,S] of transformed queries A, T against compressed keys."""
    return tq_score_with_kernel(A, T, keys, codebook, "auto", scores, stream)


def tq_score_kernel_name(layout: str, bits: int, C: int, P: int, B: int, S: int, D: int,
                         kernel: str = "auto"):
    """Name of the kernel tq_score would launch for this shape, or None if unsupported."""
    lay = TQ_UNPACKED if layout == "unpacked" else TQ_PACKED
    name = _lib.tq_score_kernel_name(lay, int(bits), int(C), int(P), int(B), int(S), int(D), KERNELS[kernel])
    return None if name is None else name.decode()


def tq_decode_debug(keys: Keys, D: int, stream=None):
    """Expand keys to (idx uint8 [P,S,D], sign int8 [P,S,D], gamma float32 [P,S])."""
    ck, P, S = keys._c(D)
    dev = keys.device
    idx = torch.empty((P, S, D), dtype=torch.uint8, device=dev)
    sign = torch.empty((P, S, D), dtype=torch.int8, device=dev)
    gamma = torch.empty((P, S), dtype=torch.float32, device=dev)
    st = _stream(dev, stream)
    _check(_lib.tq_decode_debug(ctypes.byref(ck), _ptr(idx), _ptr(sign), _ptr(gamma),
                                P, S, D, st), "tq_decode_debug")
    return idx, sign, gamma


def tq_compress_keys(keys: torch.Tensor, Pi: torch.Tensor, S_mat: torch.Tensor, codebook: torch.Tensor,
                     layout: str = "packed", bits: int = 3, stream=None) -> Keys:
    """Normalise and compress float32 keys [P,S,D] (or [S,D]) with head p % H's Pi and
    S_mat into a new Keys; its ``norm`` holds the keys' lengths."""
    k3 = _as3(_gpu(keys, "keys", torch.float32))
    Pi3 = _as3(_gpu(Pi, "Pi", torch.float32))
    S3 = _as3(_gpu(S_mat, "S_mat", torch.float32))
    _gpu(codebook, "codebook", torch.float32)
    P, S, D = k3.shape
    H = Pi3.shape[0]
    if Pi3.shape != (H, D, D) or S3.shape != (H, D, D):
        raise ValueError(f"Pi and S_mat must be [H, {D}, {D}]")
    dev = keys.device
    if layout == "unpacked":
        lay, b = TQ_UNPACKED, 0
        idx = torch.empty((P, S, D), dtype=torch.uint8, device=dev)
        sign = torch.empty((P, S, D), dtype=torch.int8, device=dev)
        gamma = torch.empty((P, S), dtype=torch.float32, device=dev)
    elif layout == "packed":
        lay, b = TQ_PACKED, int(bits)
        if b not in (2, 3) or D % 8:
            raise ValueError("packed keys need bits in (2, 3) and D % 8 == 0")
        idx = torch.empty((P, S, D * b // 8), dtype=torch.uint8, device=dev)
        sign = torch.empty((P, S, D // 8), dtype=torch.uint8, device=dev)
        gamma = torch.empty((P, S), dtype=torch.float16, device=dev)
    else:
        raise ValueError(f"unknown layout {layout!r}")
    norm = torch.empty_like(gamma)
    out = _CKeysOut(lay, b, idx.data_ptr(), sign.data_ptr(), gamma.data_ptr(), norm.data_ptr())
    st = _stream(dev, stream)
    _check(_lib.tq_compress_keys(_ptr(k3), _ptr(Pi3), _ptr(S3), _ptr(codebook), codebook.numel(),
                                 ctypes.byref(out), P, H, S, D, st), "tq_compress_keys")
    squeeze = keys.dim() == 2
    if squeeze:
        idx, sign, gamma, norm = idx[0], sign[0], gamma[0], norm[0]
    return Keys(layout, idx, sign, gamma, bits=b, norm=norm)


@dataclass
class Values:
    """MSE-only codes of P problems with S vectors of D coordinates each
    (x_s = norm_s * Pi^T codebook[idx_s]): compressed values for tq_attend, and
    keys for tq_score_mse.

    layout "unpacked": idx uint8 [P,S,D], norm float32 [P,S].
    layout "packed":   idx uint8 [P,S,D*bits/8] (LSB-first bitstream), norm float16 [P,S]; bits 2 or 3.
    A leading problem axis may be omitted (P = 1).
    """
    layout: str
    idx: torch.Tensor
    norm: torch.Tensor
    bits: int = 0

    def _c(self, D: int):
        if self.layout == "unpacked":
            lay, bits, row, ndt = TQ_UNPACKED, 0, D, torch.float32
        elif self.layout == "packed":
            lay, bits, ndt = TQ_PACKED, int(self.bits), torch.float16
            if bits not in (2, 3) or D % 8:
                raise ValueError("packed values need bits in (2, 3) and D % 8 == 0")
            row = D * bits // 8
        else:
            raise ValueError(f"unknown layout {self.layout!r}")
        _gpu(self.idx, "values.idx", torch.uint8)
        _gpu(self.norm, "values.norm", ndt)
        n = self.norm if self.norm.dim() == 2 else self.norm.unsqueeze(0)
        P, S = n.shape
        if self.idx.numel() != P * S * row:
            raise ValueError(f"value indices do not match norm's [P={P}, S={S}] with D={D}")
        return _CValues(lay, bits, self.idx.data_ptr(), self.norm.data_ptr()), P, S


def tq_attend_workspace_bytes(P: int, B: int, S: int, D: int) -> int:
    """Workspace bytes tq_attend needs for this shape."""
    return int(_lib.tq_attend_workspace_bytes(int(P), int(B), int(S), int(D)))


def tq_attend(scores: torch.Tensor, values: Values, codebook: torch.Tensor, Pi_v: torch.Tensor,
              scale: float | None = None, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """softmax(scale * scores) times the dequantized values: out [P,B,D] (or [B,D]).

    scores [P,B,S] or [B,S]; Pi_v [H,D,D] or [D,D]; scale defaults to 1/sqrt(D).
    workspace: a uint8 GPU tensor of at least tq_attend_workspace_bytes bytes
    (allocated here when omitted).
    """
    squeeze = scores.dim() == 2
    s3 = _as3(_gpu(scores, "scores", torch.float32))
    Pv = _as3(_gpu(Pi_v, "Pi_v", torch.float32))
    _gpu(codebook, "codebook", torch.float32)
    P, B, S = s3.shape
    H, D = Pv.shape[0], Pv.shape[-1]
    if Pv.shape != (H, D, D):
        raise ValueError("Pi_v must be [H, D, D]")
    cv, Pk, Sk = values._c(D)
    if (Pk, Sk) != (P, S):
        raise ValueError(f"values hold [P={Pk}, S={Sk}], scores [P={P}, S={S}]")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    dev = scores.device
    if out is None:
        out = torch.empty((P, B, D), dtype=torch.float32, device=dev)
    _gpu(out, "out", torch.float32)
    if out.numel() != P * B * D:
        raise ValueError("out must hold P*B*D floats")
    need = tq_attend_workspace_bytes(P, B, S, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _gpu(workspace, "workspace", torch.uint8)
    st = _stream(dev, stream)
    _check(_lib.tq_attend(_ptr(s3), ctypes.byref(cv), _ptr(codebook), codebook.numel(), _ptr(Pv),
                          float(scale), _ptr(out), _ptr(workspace), workspace.numel(), P, H, B, S, D, st),
           "tq_attend")
    return out.view(B, D) if squeeze else out.view(P, B, D)


def tq_attend_no_alloc(scores: torch.Tensor, values: Values, codebook: torch.Tensor, Pi_v: torch.Tensor,
                       scale: float | None = None, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """tq_attend with the library's fixed per-GPU scratch as workspace (no allocation
    inside the call; pass ``out`` to allocate nothing at all). Calls that may overlap
    on one GPU race on the scratch."""
    squeeze = scores.dim() == 2
    s3 = _as3(_gpu(scores, "scores", torch.float32))
    Pv = _as3(_gpu(Pi_v, "Pi_v", torch.float32))
    _gpu(codebook, "codebook", torch.float32)
    P, B, S = s3.shape
    H, D = Pv.shape[0], Pv.shape[-1]
    if Pv.shape != (H, D, D):
        raise ValueError("Pi_v must be [H, D, D]")
    cv, Pk, Sk = values._c(D)
    if (Pk, Sk) != (P, S):
        raise ValueError(f"values hold [P={Pk}, S={Sk}], scores [P={P}, S={S}]")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    dev = scores.device
    if out is None:
        out = torch.empty((P, B, D), dtype=torch.float32, device=dev)
    _gpu(out, "out", torch.float32)
    if out.numel() != P * B * D:
        raise ValueError("out must hold P*B*D floats")
    st = _stream(dev, stream)
    _check(_lib.tq_attend_no_alloc(_ptr(s3), ctypes.byref(cv), _ptr(codebook), codebook.numel(), _ptr(Pv),
                                   float(scale), _ptr(out), P, H, B, S, D, st), "tq_attend_no_alloc")
    return out.view(B, D) if squeeze else out.view(P, B, D)


def tq_query_transform_hadamard(q: torch.Tensor, signs: torch.Tensor, A: torch.Tensor | None = None,
                                stream=None) -> torch.Tensor:
    """A = H (signs * q) / sqrt(D): q [P,B,D] or [B,D]; signs [H,D] or [D] of +-1."""
    squeeze = q.dim() == 2
    q3 = _as3(_gpu(q, "q", torch.float32))
    sg = _gpu(signs, "signs", torch.float32)
    sg2 = sg if sg.dim() == 2 else sg.unsqueeze(0)
    P, B, D = q3.shape
    H = sg2.shape[0]
    if sg2.shape != (H, D):
        raise ValueError(f"signs must be [H, {D}]")
    if A is None:
        A = torch.empty_like(q3)
    _gpu(A, "A", torch.float32)
    if A.numel() != q3.numel():
        raise ValueError("A must have q's shape")
    _check(_lib.tq_query_transform_hadamard(_ptr(q3), _ptr(sg2), _ptr(A), P, H, B, D, _stream(q.device, stream)),
           "tq_query_transform_hadamard")
    return A.view(B, D) if squeeze else A.view(P, B, D)


def tq_score_mse(A: torch.Tensor, keys: Values, codebook: torch.Tensor, scores: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """Scores [P,B,S] (or [B,S]) of transformed queries against MSE-only keys:
    norm_s * sum_d A[b,d] codebook[idx[s,d]]."""
    squeeze = A.dim() == 2
    A3 = _as3(_gpu(A, "A", torch.float32))
    _gpu(codebook, "codebook", torch.float32)
    P, B, D = A3.shape
    ck, Pk, S = keys._c(D)
    if Pk != P:
        raise ValueError(f"keys hold {Pk} problems, A holds {P}")
    if scores is None:
        scores = torch.empty((P, B, S), dtype=torch.float32, device=A.device)
    _gpu(scores, "scores", torch.float32)
    if scores.numel() != P * B * S:
        raise ValueError("scores must hold P*B*S floats")
    _check(_lib.tq_score_mse(_ptr(A3), ctypes.byref(ck), _ptr(codebook), codebook.numel(), _ptr(scores),
                             P, B, S, D, _stream(A.device, stream)), "tq_score_mse")
    return scores.view(B, S) if squeeze else scores.view(P, B, S)


@dataclass
class SplitKeys:
    """Outlier-split keys: one set of MSE-only codes per instance (hot channels, the rest)."""
    hi: Values
    lo: Values


def tq_query_transform_split(q: torch.Tensor, perm: torch.Tensor, Pi_hi: torch.Tensor, Pi_lo: torch.Tensor,
                             A_hi: torch.Tensor | None = None, A_lo: torch.Tensor | None = None, stream=None):
    """(A_hi, A_lo) = (Pi_hi q[perm[:D_hi]], Pi_lo q[perm[D_hi:]]). q [P,B,D]; perm int32 [D];
    Pi_hi [H,D_hi,D_hi]; Pi_lo [H,D-D_hi,D-D_hi]."""
    q3 = _as3(_gpu(q, "q", torch.float32))
    _gpu(perm, "perm", torch.int32)
    Ph = _as3(_gpu(Pi_hi, "Pi_hi", torch.float32))
    Pl = _as3(_gpu(Pi_lo, "Pi_lo", torch.float32))
    P, B, D = q3.shape
    H, D_hi = Ph.shape[0], Ph.shape[-1]
    if perm.numel() != D or Ph.shape != (H, D_hi, D_hi) or Pl.shape != (H, D - D_hi, D - D_hi):
        raise ValueError("perm must be [D], Pi_hi [H,D_hi,D_hi], Pi_lo [H,D-D_hi,D-D_hi]")
    if A_hi is None:
        A_hi = torch.empty((P, B, D_hi), dtype=torch.float32, device=q.device)
    if A_lo is None:
        A_lo = torch.empty((P, B, D - D_hi), dtype=torch.float32, device=q.device)
    _gpu(A_hi, "A_hi", torch.float32)
    _gpu(A_lo, "A_lo", torch.float32)
    if A_hi.numel() != P * B * D_hi or A_lo.numel() != P * B * (D - D_hi):
        raise ValueError("A_hi must hold P*B*D_hi floats and A_lo P*B*(D-D_hi)")
    _check(_lib.tq_query_transform_split(_ptr(q3), _ptr(perm), _ptr(Ph), _ptr(Pl), _ptr(A_hi), _ptr(A_lo),
                                         P, H, B, D, D_hi, _stream(q.device, stream)), "tq_query_transform_split")
    return A_hi, A_lo


def tq_score_split(A_hi: torch.Tensor, A_lo: torch.Tensor, keys: SplitKeys, codebook_hi: torch.Tensor,
                   codebook_lo: torch.Tensor, scores: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Scores [P,B,S]: the two instances' MSE scores added."""
    Ah = _as3(_gpu(A_hi, "A_hi", torch.float32))
    Al = _as3(_gpu(A_lo, "A_lo", torch.float32))
    _gpu(codebook_hi, "codebook_hi", torch.float32)
    _gpu(codebook_lo, "codebook_lo", torch.float32)
    P, B, D_hi = Ah.shape
    D_lo = Al.shape[-1]
    if Al.shape[:2] != (P, B):
        raise ValueError("A_hi and A_lo must share [P, B]")
    ch, Ph, S = keys.hi._c(D_hi)
    cl, Pl, Sl = keys.lo._c(D_lo)
    if (Ph, Pl, Sl) != (P, P, S):
        raise ValueError("both instances must hold [P, S] keys matching A")
    if scores is None:
        scores = torch.empty((P, B, S), dtype=torch.float32, device=A_hi.device)
    _gpu(scores, "scores", torch.float32)
    if scores.numel() != P * B * S:
        raise ValueError("scores must hold P*B*S floats")
    c = _CSplit(ch, cl)
    _check(_lib.tq_score_split(_ptr(Ah), _ptr(Al), ctypes.byref(c), _ptr(codebook_hi), codebook_hi.numel(),
                               _ptr(codebook_lo), codebook_lo.numel(), _ptr(scores), P, B, S, D_hi, D_lo,
                               _stream(A_hi.device, stream)), "tq_score_split")
    return scores.view(P, B, S)


ATTEND_MODES = {"auto": 0, "fused": 1, "two_pass": 2}


def tq_score_attend_workspace_bytes(P: int, B: int, S: int, D: int, mode: str = "auto") -> int:
    """Workspace bytes tq_score_attend needs for this shape and form."""
    return int(_lib.tq_score_attend_workspace_bytes(int(P), int(B), int(S), int(D), ATTEND_MODES[mode]))


def tq_score_attend(A: torch.Tensor, T: torch.Tensor, keys: Keys, codebook: torch.Tensor, values: Values,
                    codebook_v: torch.Tensor, Pi_v: torch.Tensor, scale: float | None = None,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    stream=None, mode: str = "auto") -> torch.Tensor:
    """The fused decode step: softmax(scale * scores) times the dequantized values.
    out [P,B,D]. mode: "auto", "fused" (scores never written) or "two_pass"."""
    A3 = _as3(_gpu(A, "A", torch.float32))
    T3 = _as3(_gpu(T, "T", torch.float32))
    _gpu(codebook, "codebook", torch.float32)
    _gpu(codebook_v, "codebook_v", torch.float32)
    Pv = _as3(_gpu(Pi_v, "Pi_v", torch.float32))
    P, B, D = A3.shape
    H = Pv.shape[0]
    if T3.shape != A3.shape or Pv.shape != (H, D, D):
        raise ValueError("T must match A and Pi_v must be [H, D, D]")
    ck, Pk, S = keys._c(D)
    cv, Pv_, Sv = values._c(D)
    if (Pk, Pv_, Sv) != (P, P, S):
        raise ValueError("keys and values must hold [P, S] vectors matching A")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    dev = A.device
    if out is None:
        out = torch.empty((P, B, D), dtype=torch.float32, device=dev)
    _gpu(out, "out", torch.float32)
    if out.numel() != P * B * D:
        raise ValueError("out must hold P*B*D floats")
    need = tq_score_attend_workspace_bytes(P, B, S, D, mode)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _gpu(workspace, "workspace", torch.uint8)
    _check(_lib.tq_score_attend_with_mode(_ptr(A3), _ptr(T3), ctypes.byref(ck), _ptr(codebook), codebook.numel(),
                                          ctypes.byref(cv), _ptr(codebook_v), codebook_v.numel(), _ptr(Pv),
                                          float(scale), _ptr(out), _ptr(workspace), workspace.numel(), P, H, B, S, D,
                                          ATTEND_MODES[mode], _stream(dev, stream)), "tq_score_attend")
    return out.view(P, B, D)
