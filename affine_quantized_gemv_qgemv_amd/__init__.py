"""Python binding of libqdecode (affine-quantized decode kernels for MI355X).

Argument marshalling only: every step of every call runs in the HIP kernels
of ``libqdecode.so``; PyTorch supplies device memory and the current
stream. There is no fallback path: if the library is missing or the call
fails, a ``QDecodeError`` is raised.

Tensor conventions (see include/qdecode.h for the full contract):
  * packed codes: int32 (or uint32) tensor [N][K*bits/32], LSB-first codes;
  * scales / biases: float16 tensors [N][K/64] (bfloat16 scales and packed
    int32 zero points [N][ceil(K/512)] for the Mirai-M format; bfloat16
    scales and signed byte codes for Mirai-L);
  * activations: float16 (decode) or bfloat16 (prefill) [batch][K];
  * outputs: float32.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqdecode.so")

QD_OK, QD_ERR_INVALID_ARGUMENT, QD_ERR_MISALIGNED, QD_ERR_UNSUPPORTED, QD_ERR_WORKSPACE, QD_ERR_HIP = range(6)
QD_F16, QD_BF16 = 0, 1
QD_GELU_ERF, QD_GELU_TANH = 0, 1

EXPORTS = ("qgemv_affine4", "qgemv_affine8", "qgemv_mirai_m", "qgemv_mirai_l", "qgemv_mirai_m_rht",
           "qgemv_mirai_l_rht", "qmoe_route_topk",
           "qmoe_expert_workspace_bytes", "qmoe_expert_gemv", "qgemm_affine4_chunk_workspace_bytes",
           "qgemm_affine4_chunk",
           "qgemm_affine4_verify_workspace_bytes", "qgemm_affine4_verify",
           "qgemm_affine4_verify_i8_workspace_bytes", "qgemm_affine4_verify_i8",
           "qattn_decode_workspace_bytes", "qattn_decode",
           "qmoe_layer_decode", "qmoe_layer_decode_noalloc", "qmoe_layer_prefill_workspace_bytes",
           "qmoe_layer_prefill", "qd_stream_read",
           "qd_status_string", "qd_last_error")


class QDecodeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


_P = ctypes.c_void_p
_I32 = ctypes.c_int32


class MoeWeightsC(ctypes.Structure):
    """Mirror of qd_moe_weights."""
    _fields_ = [("E", _I32), ("H", _I32), ("I", _I32), ("I_shared", _I32), ("group_size", _I32),
                ("act", ctypes.c_int)] + \
        [(n, _P) for n in ("gu_q", "dn_q", "sgu_q", "sdn_q", "gu_s", "gu_b", "dn_s", "dn_b",
                           "sgu_s", "sgu_b", "sdn_s", "sdn_b")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library with argument types declared. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python affine_quantized_gemv_qgemv_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    gemv_args = [_P, _P, _P, _P, ctypes.c_int, _P, _I32, _I32, _I32, _I32, _P]
    L.qgemv_affine4.argtypes = gemv_args
    L.qgemv_affine8.argtypes = gemv_args
    L.qgemv_mirai_m.argtypes = gemv_args
    L.qgemv_mirai_l.argtypes = [_P, _P, _P, ctypes.c_int, _P, _I32, _I32, _I32, _I32, _P]
    L.qgemv_mirai_m_rht.argtypes = [_P, _P, _P, _P, _P, ctypes.c_float, _P, ctypes.c_int, _P,
                                    _I32, _I32, _I32, _I32, _P]
    L.qgemv_mirai_l_rht.argtypes = [_P, _P, _P, _P, ctypes.c_float, _P, ctypes.c_int, _P,
                                    _I32, _I32, _I32, _I32, _P]
    L.qmoe_route_topk.argtypes = [_P, _I32, _I32, _I32, _P, _P, _P]
    L.qmoe_expert_workspace_bytes.argtypes = [ctypes.POINTER(MoeWeightsC), _I32, _I32]
    L.qmoe_expert_workspace_bytes.restype = ctypes.c_size_t
    L.qmoe_expert_gemv.argtypes = [ctypes.POINTER(MoeWeightsC), _P, _P, _I32, _I32, _P, ctypes.c_int,
                                   _P, _P, ctypes.c_size_t, _P]
    L.qgemm_affine4_chunk_workspace_bytes.argtypes = [_I32, _I32, _I32]
    L.qgemm_affine4_chunk_workspace_bytes.restype = ctypes.c_size_t
    L.qgemm_affine4_chunk.argtypes = [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, ctypes.c_size_t, _P]
    L.qgemm_affine4_verify_workspace_bytes.argtypes = [_I32, _I32, _I32]
    L.qgemm_affine4_verify_workspace_bytes.restype = ctypes.c_size_t
    L.qgemm_affine4_verify.argtypes = [_P, _P, _P, _P, ctypes.c_int, _P, _I32, _I32, _I32, _I32, _P,
                                       ctypes.c_size_t, _P]
    L.qgemm_affine4_verify_i8_workspace_bytes.argtypes = [_I32, _I32]
    L.qgemm_affine4_verify_i8_workspace_bytes.restype = ctypes.c_size_t
    L.qgemm_affine4_verify_i8.argtypes = [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, ctypes.c_size_t,
                                          _P]
    L.qmoe_layer_decode.argtypes = [ctypes.POINTER(MoeWeightsC), _P, _P, _P, _I32, _P, ctypes.c_int, _P,
                                    _P, _P, _P, _P, ctypes.c_size_t, _P]
    L.qmoe_layer_prefill_workspace_bytes.argtypes = [ctypes.POINTER(MoeWeightsC), _I32, _I32]
    L.qmoe_layer_prefill_workspace_bytes.restype = ctypes.c_size_t
    L.qmoe_layer_prefill.argtypes = [ctypes.POINTER(MoeWeightsC), _P, _P, _P, _I32, _I32, _P, ctypes.c_int,
                                     _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    L.qmoe_layer_decode_noalloc.argtypes = [ctypes.POINTER(MoeWeightsC), _P, _P, _P, _I32, _P,
                                            ctypes.c_int, _P, _P, _P, _P, _P]
    L.qattn_decode_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32]
    L.qattn_decode_workspace_bytes.restype = ctypes.c_size_t
    L.qattn_decode.argtypes = [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, ctypes.c_float,
                               _P, _P, ctypes.c_size_t, _P]
    L.qd_stream_read.argtypes = [_P, ctypes.c_size_t, _P, _P]
    L.qd_stream_read.restype = ctypes.c_int
    L.qd_status_string.argtypes = [ctypes.c_int]
    L.qd_status_string.restype = ctypes.c_char_p
    L.qd_last_error.argtypes = []
    L.qd_last_error.restype = ctypes.c_char_p
    for fn in ("qgemv_affine4", "qgemv_affine8", "qgemv_mirai_m", "qgemv_mirai_l",
               "qgemv_mirai_m_rht", "qgemv_mirai_l_rht",
               "qmoe_route_topk", "qmoe_expert_gemv", "qgemm_affine4_chunk", "qgemm_affine4_verify",
               "qgemm_affine4_verify_i8", "qattn_decode", "qmoe_layer_decode", "qmoe_layer_decode_noalloc"):
        getattr(L, fn).restype = ctypes.c_int
    _lib = L
    return L


def status_name(status: int) -> str:
    return lib().qd_status_string(status).decode()


def last_error() -> str:
    return lib().qd_last_error().decode()


def _check(status: int) -> None:
    if status != QD_OK:
        raise QDecodeError(status, last_error())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _x_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.float16:
        return QD_F16
    if x.dtype == torch.bfloat16:
        return QD_BF16
    raise TypeError(f"activations must be float16 or bfloat16, got {x.dtype}")


def _need(t: torch.Tensor, name: str, dtypes, ndim: int) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor, got shape {tuple(t.shape)}")


_CODES = (torch.int32, torch.uint32)
_HALF = (torch.float16,)


def _qgemv(bits: int, wq, scales, biases, x, out):
    squeeze = x.dim() == 1
    x2 = x.unsqueeze(0) if squeeze else x
    _need(wq, "wq", _CODES, 2)
    _need(scales, "scales", _HALF, 2)
    _need(biases, "biases", _HALF, 2)
    _need(x2, "x", (torch.float16, torch.bfloat16), 2)
    N = wq.shape[0]
    K = wq.shape[1] * (32 // bits)
    batch = x2.shape[0]
    if x2.shape[1] != K:
        raise ValueError(f"x has {x2.shape[1]} columns, the codes imply K = {K}")
    if tuple(scales.shape) != (N, K // 64) or tuple(biases.shape) != (N, K // 64):
        raise ValueError("scales/biases must be [N][K/64]")
    if out is None:
        out = torch.empty((batch, N), dtype=torch.float32, device=x2.device)
    _need(out, "out", (torch.float32,), 2)
    if tuple(out.shape) != (batch, N):
        raise ValueError("out must be [batch][N]")
    fn = lib().qgemv_affine4 if bits == 4 else lib().qgemv_affine8
    _check(fn(_ptr(wq), _ptr(scales), _ptr(biases), _ptr(x2), _x_dtype(x2), _ptr(out), N, K, batch,
              64, _stream()))
    return out[0] if squeeze else out


def qgemv_affine4(wq, scales, biases, x, out=None):
    """y[b][n] = sum_k (s*q + b)[n][k] x[b][k] with 4-bit codes; batch <= 8."""
    return _qgemv(4, wq, scales, biases, x, out)


def qgemv_affine8(wq, scales, biases, x, out=None):
    """Same with 8-bit codes (router); batch <= 128."""
    return _qgemv(8, wq, scales, biases, x, out)


def _mirai(fmt: str, wq, scales, zeros, x, out, rot=None):
    bits = 4 if fmt == "M" else 8
    squeeze = x.dim() == 1
    x2 = x.unsqueeze(0) if squeeze else x
    _need(wq, "wq", _CODES, 2)
    _need(scales, "scales", (torch.bfloat16,), 2)
    _need(x2, "x", (torch.float16, torch.bfloat16), 2)
    N = wq.shape[0]
    K = wq.shape[1] * (32 // bits)
    batch = x2.shape[0]
    if x2.shape[1] != K:
        raise ValueError(f"x has {x2.shape[1]} columns, the codes imply K = {K}")
    if tuple(scales.shape) != (N, K // 64):
        raise ValueError("scales must be [N][K/64]")
    if fmt == "M":
        _need(zeros, "zeros", _CODES, 2)
        if tuple(zeros.shape) != (N, (K // 64 + 7) // 8):
            raise ValueError("zeros must be [N][ceil(K/512)]")
    if out is None:
        out = torch.empty((batch, N), dtype=torch.float32, device=x2.device)
    _need(out, "out", (torch.float32,), 2)
    if tuple(out.shape) != (batch, N):
        raise ValueError("out must be [batch][N]")
    if rot is not None:
        signs, gamma, eps = rot
        if signs is not None:
            _need(signs, "signs", _CODES, 1)
            if signs.numel() != K // 32:
                raise ValueError("signs must hold K/32 words")
        if gamma is not None:
            _need(gamma, "gamma", (x2.dtype,), 1)
            if gamma.numel() != K:
                raise ValueError("gamma must hold K values")
        if fmt == "M":
            _check(lib().qgemv_mirai_m_rht(_ptr(wq), _ptr(scales), _ptr(zeros), _ptr(signs),
                                           _ptr(gamma), float(eps), _ptr(x2), _x_dtype(x2), _ptr(out),
                                           N, K, batch, 64, _stream()))
        else:
            _check(lib().qgemv_mirai_l_rht(_ptr(wq), _ptr(scales), _ptr(signs), _ptr(gamma),
                                           float(eps), _ptr(x2), _x_dtype(x2), _ptr(out), N, K,
                                           batch, 64, _stream()))
    elif fmt == "M":
        _check(lib().qgemv_mirai_m(_ptr(wq), _ptr(scales), _ptr(zeros), _ptr(x2), _x_dtype(x2),
                                   _ptr(out), N, K, batch, 64, _stream()))
    else:
        _check(lib().qgemv_mirai_l(_ptr(wq), _ptr(scales), _ptr(x2), _x_dtype(x2), _ptr(out), N, K,
                                   batch, 64, _stream()))
    return out[0] if squeeze else out


def qgemv_mirai_m(wq, scales, zeros, x, out=None):
    """y[b][n] = sum_k s*(q - z) x[b][k]: 4-bit codes, bf16 scales, packed 4-bit zero points."""
    return _mirai("M", wq, scales, zeros, x, out)


def qgemv_mirai_l(wq, scales, x, out=None):
    """y[b][n] = sum_k s*q x[b][k]: signed 8-bit codes, bf16 scales; batch <= 8."""
    return _mirai("L", wq, scales, None, x, out)


def qgemv_mirai_m_rht(wq, scales, zeros, x, signs=None, gamma=None, eps: float = 1e-6, out=None):
    """Mirai-M GEMV on the rotated activations H D (RMSNorm(x) * gamma), block 32.

    signs: int32 [K/32] sign bits (None = no flips); gamma: [K] in x's dtype
    (None = no RMSNorm)."""
    return _mirai("M", wq, scales, zeros, x, out, (signs, gamma, eps))


def qgemv_mirai_l_rht(wq, scales, x, signs=None, gamma=None, eps: float = 1e-6, out=None):
    """Mirai-L GEMV on the rotated activations H D (RMSNorm(x) * gamma), block 32."""
    return _mirai("L", wq, scales, None, x, out, (signs, gamma, eps))


def qmoe_route_topk(logits, k: int, idx=None, weights=None):
    """Top-k experts of each row of logits [T][E] and their renormalized softmax weights."""
    _need(logits, "logits", (torch.float32,), 2)
    T, E = logits.shape
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _need(idx, "idx", (torch.int32,), 2)
    _need(weights, "weights", (torch.float32,), 2)
    if tuple(idx.shape) != (T, k) or tuple(weights.shape) != (T, k):
        raise ValueError("idx/weights must be [T][k]")
    _check(lib().qmoe_route_topk(_ptr(logits), T, E, k, _ptr(idx), _ptr(weights), _stream()))
    return idx, weights


@dataclass
class MoeWeights:
    """Device tensors of one MoE layer (see qd_moe_weights in include/qdecode.h)."""
    E: int
    H: int
    I: int
    Is: int
    router_q: torch.Tensor
    router_s: torch.Tensor
    router_b: torch.Tensor
    gu_q: torch.Tensor
    gu_s: torch.Tensor
    gu_b: torch.Tensor
    dn_q: torch.Tensor
    dn_s: torch.Tensor
    dn_b: torch.Tensor
    sgu_q: torch.Tensor
    sgu_s: torch.Tensor
    sgu_b: torch.Tensor
    sdn_q: torch.Tensor
    sdn_s: torch.Tensor
    sdn_b: torch.Tensor
    act: int = QD_GELU_ERF

    def cstruct(self) -> MoeWeightsC:
        return MoeWeightsC(self.E, self.H, self.I, self.Is, 64, self.act,
                           *(t.data_ptr() for t in (self.gu_q, self.dn_q, self.sgu_q, self.sdn_q,
                                                    self.gu_s, self.gu_b, self.dn_s, self.dn_b,
                                                    self.sgu_s, self.sgu_b, self.sdn_s, self.sdn_b)))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (
            self.router_q, self.router_s, self.router_b, self.gu_q, self.gu_s, self.gu_b,
            self.dn_q, self.dn_s, self.dn_b, self.sgu_q, self.sgu_s, self.sgu_b,
            self.sdn_q, self.sdn_s, self.sdn_b))


def qmoe_workspace_bytes(w: MoeWeights, T: int, k: int) -> int:
    """Workspace bytes of qmoe_layer (and of qmoe_expert_gemv) for T tokens."""
    st = w.cstruct()
    e = int(lib().qmoe_expert_workspace_bytes(ctypes.byref(st), T, k))
    return max(e, int(lib().qmoe_layer_prefill_workspace_bytes(ctypes.byref(st), T, k)))


def qmoe_expert_gemv(w: MoeWeights, idx, weights, x, out=None, workspace=None):
    """Routed + shared experts of one MoE layer for tokens x [T][H] (fp16 or bf16)."""
    _need(x, "x", (torch.float16, torch.bfloat16), 2)
    _need(idx, "idx", (torch.int32,), 2)
    _need(weights, "weights", (torch.float32,), 2)
    T, k = idx.shape
    if x.shape[0] != T or x.shape[1] != w.H:
        raise ValueError("x must be [T][H]")
    if out is None:
        out = torch.empty((T, w.H), dtype=torch.float32, device=x.device)
    _need(out, "out", (torch.float32,), 2)
    st = w.cstruct()
    need = int(lib().qmoe_expert_workspace_bytes(ctypes.byref(st), T, k))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(lib().qmoe_expert_gemv(ctypes.byref(st), _ptr(idx), _ptr(weights), T, k, _ptr(x),
                                  _x_dtype(x), _ptr(out), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream()))
    return out


def qmoe_layer(w: MoeWeights, x, k: int = 8, workspace=None, logits=None, idx=None, weights=None,
               out=None):
    """One MoE FFN layer: int8 router GEMV -> top-k routing -> expert block.

    One token (decode) takes qmoe_layer_decode (the ranking inside the gate+up
    kernel, identical results); several take qmoe_layer_prefill (the router split
    over the hidden size, its partial logits added by the routing)."""
    T = x.shape[0]
    if logits is None:
        logits = torch.empty((T, w.E), dtype=torch.float32, device=x.device)
    if T == 1 and w.E <= 256:
        _need(x, "x", (torch.float16, torch.bfloat16), 2)
        if idx is None:
            idx = torch.empty((1, k), dtype=torch.int32, device=x.device)
        if weights is None:
            weights = torch.empty((1, k), dtype=torch.float32, device=x.device)
        if out is None:
            out = torch.empty((1, w.H), dtype=torch.float32, device=x.device)
        st = w.cstruct()
        need = int(lib().qmoe_expert_workspace_bytes(ctypes.byref(st), 1, k))
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
        _check(lib().qmoe_layer_decode(ctypes.byref(st), _ptr(w.router_q), _ptr(w.router_s),
                                       _ptr(w.router_b), k, _ptr(x), _x_dtype(x), _ptr(logits),
                                       _ptr(idx), _ptr(weights), _ptr(out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream()))
        return out
    _need(x, "x", (torch.float16, torch.bfloat16), 2)
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if out is None:
        out = torch.empty((T, w.H), dtype=torch.float32, device=x.device)
    st = w.cstruct()
    need = int(lib().qmoe_layer_prefill_workspace_bytes(ctypes.byref(st), T, k))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(lib().qmoe_layer_prefill(ctypes.byref(st), _ptr(w.router_q), _ptr(w.router_s),
                                    _ptr(w.router_b), k, T, _ptr(x), _x_dtype(x), _ptr(logits),
                                    _ptr(idx), _ptr(weights), _ptr(out), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream()))
    return out


def qmoe_layer_decode_noalloc(w: MoeWeights, x, k: int = 8, logits=None, idx=None, weights=None,
                              out=None):
    """One decode token through a MoE layer (as qmoe_layer with T = 1) with the
    intermediate activations in the library's per-device scratch: no workspace
    is allocated for the call. Calls on one device must not overlap."""
    _need(x, "x", (torch.float16, torch.bfloat16), 2)
    if x.shape[0] != 1 or x.shape[1] != w.H:
        raise ValueError("x must be [1][H]")
    if logits is None:
        logits = torch.empty((1, w.E), dtype=torch.float32, device=x.device)
    if idx is None:
        idx = torch.empty((1, k), dtype=torch.int32, device=x.device)
    if weights is None:
        weights = torch.empty((1, k), dtype=torch.float32, device=x.device)
    if out is None:
        out = torch.empty((1, w.H), dtype=torch.float32, device=x.device)
    st = w.cstruct()
    _check(lib().qmoe_layer_decode_noalloc(ctypes.byref(st), _ptr(w.router_q), _ptr(w.router_s),
                                           _ptr(w.router_b), k, _ptr(x), _x_dtype(x), _ptr(logits),
                                           _ptr(idx), _ptr(weights), _ptr(out), _stream()))
    return out


def stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Reads every byte of the device tensor buf once (the HBM read ceiling;
    see qd_stream_read). sink: a device tensor of at least 4 bytes."""
    if not buf.is_cuda or not sink.is_cuda or not buf.is_contiguous():
        raise ValueError("buf and sink must be contiguous device tensors")
    _check(lib().qd_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream()))


def chunk_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().qgemm_affine4_chunk_workspace_bytes(M, N, K))


def qgemm_affine4_chunk(wq, scales, biases, x, out=None, workspace=None):
    """Prefill chunk Y[m][n] = sum_k w[n][k] X[m][k] for bf16 X [M][K], M <= 128. Shapes
    with few column tiles split K and need `workspace` (uint8, device) of
    chunk_workspace_bytes(M, N, K) bytes; by default a fresh one is allocated when the
    shape needs it."""
    _need(wq, "wq", _CODES, 2)
    _need(scales, "scales", _HALF, 2)
    _need(biases, "biases", _HALF, 2)
    _need(x, "x", (torch.bfloat16,), 2)
    N, K = wq.shape[0], wq.shape[1] * 8
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must be [M][K]")
    if tuple(scales.shape) != (N, K // 64) or tuple(biases.shape) != (N, K // 64):
        raise ValueError("scales/biases must be [N][K/64]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _need(out, "out", (torch.float32,), 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M][N]")
    if workspace is None:
        need = chunk_workspace_bytes(M, N, K)
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qgemm_affine4_chunk(_ptr(wq), _ptr(scales), _ptr(biases), _ptr(x), _ptr(out), M, N,
                                     K, 64, _ptr(workspace), wsb, _stream()))
    return out


def verify_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().qgemm_affine4_verify_workspace_bytes(M, N, K))


def qgemm_affine4_verify(wq, scales, biases, x, out=None, workspace=None):
    """Verification GEMM Y[m][n] = sum_k w[n][k] X[m][k] over drafted tokens, fp16 or bf16
    X [M][K], M <= 128 (built for 9..64 tokens). Shapes with few column tiles split K and
    need `workspace` (uint8, device) of verify_workspace_bytes(M, N, K) bytes; by default a
    fresh one is allocated when the shape needs it."""
    _need(wq, "wq", _CODES, 2)
    _need(scales, "scales", _HALF, 2)
    _need(biases, "biases", _HALF, 2)
    _need(x, "x", (torch.float16, torch.bfloat16), 2)
    N, K = wq.shape[0], wq.shape[1] * 8
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must be [M][K]")
    if tuple(scales.shape) != (N, K // 64) or tuple(biases.shape) != (N, K // 64):
        raise ValueError("scales/biases must be [N][K/64]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _need(out, "out", (torch.float32,), 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M][N]")
    if workspace is None:
        need = verify_workspace_bytes(M, N, K)
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qgemm_affine4_verify(_ptr(wq), _ptr(scales), _ptr(biases), _ptr(x), _x_dtype(x),
                                      _ptr(out), M, N, K, 64, _ptr(workspace), wsb, _stream()))
    return out


def verify_i8_workspace_bytes(M: int, K: int) -> int:
    return int(lib().qgemm_affine4_verify_i8_workspace_bytes(M, K))


def qgemm_affine4_verify_i8(wq, scales, biases, x, out=None, workspace=None):
    """Verification GEMM on per-token int8 activations: sx[m] = max|X[m]| / 127,
    xq = round-half-even(X / sx) in fp32, Y[m][n] = sx[m] sum_k w[n][k] xq[m][k];
    fp16 X [M][K], M <= 32. `workspace` (uint8, device) defaults to a fresh one."""
    _need(wq, "wq", _CODES, 2)
    _need(scales, "scales", _HALF, 2)
    _need(biases, "biases", _HALF, 2)
    _need(x, "x", (torch.float16,), 2)
    N, K = wq.shape[0], wq.shape[1] * 8
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must be [M][K]")
    if tuple(scales.shape) != (N, K // 64) or tuple(biases.shape) != (N, K // 64):
        raise ValueError("scales/biases must be [N][K/64]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _need(out, "out", (torch.float32,), 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M][N]")
    if workspace is None:
        need = verify_i8_workspace_bytes(M, K)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(lib().qgemm_affine4_verify_i8(_ptr(wq), _ptr(scales), _ptr(biases), _ptr(x), _ptr(out), M, N,
                                         K, 64, _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream()))
    return out


def qattn_workspace_bytes(Hq: int, Hkv: int, D: int, cap: int) -> int:
    return int(lib().qattn_decode_workspace_bytes(Hq, Hkv, D, cap))


def qattn_decode(q, k_new, v_new, k_cache, v_cache, pos: int, window: int = 0, scale=None,
                 out=None, workspace=None):
    """Decode attention of one token: stores k_new / v_new at the token's slot of the
    fp16 caches [Hkv][cap][D] (circular when window > 0), then attends over the
    occupied slots. q [Hq][D], k_new / v_new [Hkv][D] fp16; returns out [Hq][D] fp32."""
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new")):
        _need(t, nm, (torch.float16,), 2)
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm, (torch.float16,), 3)
    Hq, D = q.shape
    Hkv, cap, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(k_new.shape) != (Hkv, D) \
            or tuple(v_new.shape) != (Hkv, D):
        raise ValueError("attention shapes do not match")
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((Hq, D), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), 2)
    need = qattn_workspace_bytes(Hq, Hkv, D, cap)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib().qattn_decode(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                              Hq, Hkv, D, cap, window, pos, float(scale), _ptr(out),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream()))
    return out
