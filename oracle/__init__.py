"""numpy front end of the fp64 CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library and its
Python binding never do. It shares no code with the HIP path: inputs come
from ``synth`` as raw packed words and fp16/bf16 bit patterns, and every
conversion and every sum happens in ``oracle.c``.

Definitions followed (jeff.news/article/5193, TurboFieldfare; sections
"성능과 제약" (performance and constraints) and "내부 구조가 진짜 흥미로운
부분" (internals)): affine 4-bit group-64 weights with an 8-bit router,
w = s*q + b; top-8 routing with renormalized weights; shared and routed
expert outputs combined; prefill in chunks of at most 128 tokens.
Decode attention follows the same article's internals section (circular KV
for sliding-window layers, linear KV for full attention, exact attention).
Mirai-M and Mirai-L weights follow the uzu page on discuss.pytorch.kr
(section on model conversion and the Mirai quantization formats): 4-bit
asymmetric codes with a 4-bit zero point and a bf16 scale per group of 64,
w = s*(q - z); 8-bit symmetric codes, w = s*q.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.qo_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.qo_f16_to_f64.restype = ctypes.c_double
    lib.qo_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.qo_bf16_to_f64.restype = ctypes.c_double
    lib.qo_f16_array.argtypes = [_P, _I64, _P]
    lib.qo_bf16_array.argtypes = [_P, _I64, _P]
    lib.qo_code.argtypes = [ctypes.c_int, _P, _I64]
    lib.qo_code.restype = ctypes.c_int
    lib.qo_dequant.argtypes = [ctypes.c_int, _P, _P, _P, _I64, _I64, _P]
    lib.qo_gemv.argtypes = [ctypes.c_int, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P]
    lib.qo_gemv_rows.argtypes = [ctypes.c_int, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _P]
    lib.qo_route_topk.argtypes = [_P, _I64, _I64, _I64, _P, _P]
    lib.qo_route_topk.restype = ctypes.c_int
    lib.qo_gelu.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.qo_gelu.restype = ctypes.c_double
    lib.qo_moe_experts.argtypes = [_P, _P, _I64, _I64, _P, _P, ctypes.c_int, _P, _P, _P, _P]
    lib.qo_mirai_dequant.argtypes = [ctypes.c_int, _P, _P, _P, _I64, _I64, _P]
    lib.qo_mirai_gemv.argtypes = [ctypes.c_int, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _P]
    lib.qo_rht.argtypes = [_P, _I64, _P, _P]
    lib.qo_rmsnorm.argtypes = [_P, _I64, _P, ctypes.c_double, _P]
    lib.qo_attn_slot.argtypes = [_I64, _I64]
    lib.qo_attn_slot.restype = _I64
    lib.qo_attn_decode.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64,
                                   ctypes.c_double, _P, _P]
    lib.qo_quant_i8_rows.argtypes = [_P, _I64, _I64, _P, _P]
    lib.qo_set_threads.argtypes = [ctypes.c_int]
    lib.qo_get_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(_P)


def set_threads(n: int) -> None:
    _load().qo_set_threads(int(n))


def get_threads() -> int:
    return int(_load().qo_get_threads())


def f16_to_f64(bits) -> np.ndarray:
    a, p = _c(bits, np.uint16)
    out = np.empty(a.shape, dtype=np.float64)
    _load().qo_f16_array(p, a.size, out.ctypes.data_as(_P))
    return out


def bf16_to_f64(bits) -> np.ndarray:
    a, p = _c(bits, np.uint16)
    out = np.empty(a.shape, dtype=np.float64)
    _load().qo_bf16_array(p, a.size, out.ctypes.data_as(_P))
    return out


def code(bits: int, row, k: int) -> int:
    a, p = _c(row, np.uint32)
    return int(_load().qo_code(bits, p, k))


def dequant(w) -> np.ndarray:
    """Dequantized fp64 matrix [N][K] of a ``synth.AffineWeights``."""
    out = np.empty((w.N, w.K), dtype=np.float64)
    q, pq = _c(w.wq, np.uint32)
    s, ps = _c(w.scales, np.uint16)
    b, pb = _c(w.biases, np.uint16)
    _load().qo_dequant(w.bits, pq, ps, pb, w.N, w.K, out.ctypes.data_as(_P))
    return out


def gemv(w, x, rows=None):
    """y[T][N] = W x and A[T][N] = sum_k |w x| for fp64 activations x[T][K].

    With ``rows``, only those output rows are computed: y[T][len(rows)].
    """
    x2, px = _c(np.atleast_2d(x), np.float64)
    T = x2.shape[0]
    if x2.shape[1] != w.K:
        raise ValueError("x has the wrong length")
    q, pq = _c(w.wq, np.uint32)
    s, ps = _c(w.scales, np.uint16)
    b, pb = _c(w.biases, np.uint16)
    if rows is None:
        y = np.empty((T, w.N), dtype=np.float64)
        a = np.empty((T, w.N), dtype=np.float64)
        _load().qo_gemv(w.bits, pq, ps, pb, px, T, w.N, w.K, y.ctypes.data_as(_P),
                        a.ctypes.data_as(_P))
    else:
        r, pr = _c(rows, np.int64)
        if r.size and (r.min() < 0 or r.max() >= w.N):
            raise ValueError("row out of range")
        y = np.empty((T, r.size), dtype=np.float64)
        a = np.empty((T, r.size), dtype=np.float64)
        _load().qo_gemv_rows(w.bits, pq, ps, pb, px, T, w.N, w.K, pr, r.size,
                             y.ctypes.data_as(_P), a.ctypes.data_as(_P))
    return y, a


def gemv_f16(w, x_bits, rows=None):
    """GEMV on fp16 activations given as raw bits [T][K]."""
    return gemv(w, f16_to_f64(np.atleast_2d(x_bits)), rows)


def gemm_chunk(w, x_bits_bf16, rows=None):
    """Prefill chunk: Y[M][N] = X W^T with bf16 activations X[M][K] (raw bits)."""
    return gemv(w, bf16_to_f64(np.atleast_2d(x_bits_bf16)), rows)


def quant_i8(x_bits):
    """Per-token symmetric int8 quantization of fp16 activations (raw bits
    [M][K]): codes int8 [M][K] and fp32 scales [M], scale = max|x| / 127 and
    codes round(x / scale) with ties to even, in fp32 (uzu page, section on
    speculative decoding: activations quantized to 8 bits on the fly for the
    int8 verification GEMM; the scheme is this oracle's reading)."""
    x, px = _c(np.atleast_2d(x_bits), np.uint16)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    sc = np.empty(M, dtype=np.float32)
    _load().qo_quant_i8_rows(px, M, K, q.ctypes.data_as(_P), sc.ctypes.data_as(_P))
    return q, sc


def verify_i8(w, x_bits, rows=None):
    """Verification GEMM on dynamically quantized int8 activations:
    Y = X^ W^T with X^[m] = scale[m] * q[m] from quant_i8 (exact in fp64).
    Returns (y, A) as gemv does, A = sum_k |w x^|."""
    q, sc = quant_i8(x_bits)
    xh = sc.astype(np.float64)[:, None] * q.astype(np.float64)
    return gemv(w, xh, rows)


MIRAI_FMT = {"M": 1, "L": 2}


def _mirai_ptrs(w):
    q, pq = _c(w.wq, np.uint32)
    s, ps = _c(w.scales, np.uint16)
    if w.zeros is None:
        return (q, s), pq, ps, None
    z, pz = _c(w.zeros, np.uint32)
    return (q, s, z), pq, ps, pz


def mirai_dequant(w) -> np.ndarray:
    """Dequantized fp64 matrix [N][K] of a ``synth.MiraiWeights``."""
    out = np.empty((w.N, w.K), dtype=np.float64)
    keep, pq, ps, pz = _mirai_ptrs(w)
    _load().qo_mirai_dequant(MIRAI_FMT[w.fmt], pq, ps, pz, w.N, w.K, out.ctypes.data_as(_P))
    return out


def mirai_gemv(w, x, rows=None):
    """y[T][N] = W x and A = sum_k |w x| for a Mirai-M / Mirai-L matrix and fp64 x[T][K]."""
    x2, px = _c(np.atleast_2d(x), np.float64)
    T = x2.shape[0]
    if x2.shape[1] != w.K:
        raise ValueError("x has the wrong length")
    keep, pq, ps, pz = _mirai_ptrs(w)
    if rows is None:
        m, pr = w.N, None
    else:
        r, pr = _c(rows, np.int64)
        keep = keep + (r,)
        if r.size and (r.min() < 0 or r.max() >= w.N):
            raise ValueError("row out of range")
        m = r.size
    y = np.empty((T, m), dtype=np.float64)
    a = np.empty((T, m), dtype=np.float64)
    _load().qo_mirai_gemv(MIRAI_FMT[w.fmt], pq, ps, pz, px, T, w.N, w.K, pr, m,
                          y.ctypes.data_as(_P), a.ctypes.data_as(_P))
    return y, a


def mirai_gemv_x(w, x_bits, x_dtype: str = "f16", rows=None):
    """Mirai GEMV on fp16 or bf16 activations given as raw bits [T][K]."""
    xd = f16_to_f64(np.atleast_2d(x_bits)) if x_dtype == "f16" else bf16_to_f64(np.atleast_2d(x_bits))
    return mirai_gemv(w, xd, rows)


def rht(x, signs=None) -> np.ndarray:
    """Block-32 random Hadamard transform of each row of x[T][K] (fp64)."""
    x2, px = _c(np.atleast_2d(x), np.float64)
    T, K = x2.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    sg, ps = (None, None) if signs is None else _c(signs, np.uint32)
    if sg is not None and sg.size != K // 32:
        raise ValueError("signs must hold K/32 words")
    out = np.empty_like(x2)
    for t in range(T):
        _load().qo_rht(x2[t].ctypes.data_as(_P), K, ps, out[t].ctypes.data_as(_P))
    return out


def rmsnorm(x, gamma=None, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm of each row of x[T][K] with weight gamma[K] (fp64; None = 1)."""
    x2, px = _c(np.atleast_2d(x), np.float64)
    T, K = x2.shape
    g, pg = (None, None) if gamma is None else _c(gamma, np.float64)
    out = np.empty_like(x2)
    for t in range(T):
        _load().qo_rmsnorm(x2[t].ctypes.data_as(_P), K, pg, float(eps), out[t].ctypes.data_as(_P))
    return out


def mirai_gemv_rht(w, x_bits, x_dtype="f16", signs=None, gamma_bits=None, eps: float = 1e-6,
                   rows=None):
    """GEMV with the rotation prologue: y = W' (H D rmsnorm(x)).

    gamma_bits None skips the RMSNorm (a projection whose input does not come
    from a norm); gamma is given in the activations' dtype. Returns
    (y, A, x') with A = sum_k |w'_k x'_k| and x' the rotated activations.
    """
    dec = f16_to_f64 if x_dtype == "f16" else bf16_to_f64
    xd = dec(np.atleast_2d(x_bits))
    if gamma_bits is not None:
        xd = rmsnorm(xd, dec(gamma_bits), eps)
    xr = rht(xd, signs)
    y, a = mirai_gemv(w, xr, rows)
    return y, a, xr


def attn_slot(pos: int, window: int) -> int:
    return int(_load().qo_attn_slot(pos, window))


def attn_decode(q, k_new, v_new, kc, vc, window: int, pos: int, scale: float):
    """Decode attention of one token (fp64 inputs): q [Hq][D], k_new/v_new
    [Hkv][D], caches [Hkv][cap][D]. Returns (out [Hq][D], A [Hq][D])."""
    q2, pq = _c(q, np.float64)
    kn, pkn = _c(k_new, np.float64)
    vn, pvn = _c(v_new, np.float64)
    k3, pk = _c(kc, np.float64)
    v3, pv = _c(vc, np.float64)
    Hq, D = q2.shape
    Hkv, cap, D2 = k3.shape
    if D2 != D or kn.shape != (Hkv, D) or vn.shape != (Hkv, D) or v3.shape != k3.shape:
        raise ValueError("attention shapes")
    if Hq % Hkv or pos < 0 or (window > 0 and cap != window) or (window == 0 and pos >= cap):
        raise ValueError("attention sizes")
    out = np.empty((Hq, D))
    a = np.empty((Hq, D))
    _load().qo_attn_decode(pq, pkn, pvn, pk, pv, Hq, Hkv, D, cap, window, pos, float(scale),
                           out.ctypes.data_as(_P), a.ctypes.data_as(_P))
    return out, a


def route_topk(logits, k: int):
    l, pl = _c(np.atleast_2d(logits), np.float64)
    T, E = l.shape
    idx = np.empty((T, k), dtype=np.int32)
    p = np.empty((T, k), dtype=np.float64)
    rc = _load().qo_route_topk(pl, T, E, k, idx.ctypes.data_as(_P), p.ctypes.data_as(_P))
    if rc != 0:
        raise ValueError("bad routing sizes")
    return idx, p


def gelu(u: float, variant: int = 0) -> float:
    return float(_load().qo_gelu(float(u), int(variant)))


class _Moe(ctypes.Structure):
    _fields_ = [("E", _I64), ("H", _I64), ("I", _I64), ("Is", _I64)] + \
        [(n, _P) for n in ("gu_q", "dn_q", "sgu_q", "sdn_q", "gu_s", "gu_b", "dn_s", "dn_b",
                           "sgu_s", "sgu_b", "sdn_s", "sdn_b")]


def moe_experts(mw, x, idx, p, act: int = 0, want_h: bool = False):
    """Expert block on fp64 activations x[T][H] with routing idx/p [T][k].

    Returns (y, A) or (y, A, h, hs) with ``want_h``.
    """
    x2, px = _c(np.atleast_2d(x), np.float64)
    T = x2.shape[0]
    idx2, pidx = _c(np.atleast_2d(idx), np.int32)
    p2, pp = _c(np.atleast_2d(p), np.float64)
    k = idx2.shape[1]
    keep = []

    def ptr(a, dt):
        arr, pa = _c(a, dt)
        keep.append(arr)
        return pa

    st = _Moe(mw.E, mw.H, mw.I, mw.Is,
              ptr(mw.gu_wq, np.uint32), ptr(mw.dn_wq, np.uint32),
              ptr(mw.sgu.wq, np.uint32), ptr(mw.sdn.wq, np.uint32),
              ptr(mw.gu_s, np.uint16), ptr(mw.gu_b, np.uint16),
              ptr(mw.dn_s, np.uint16), ptr(mw.dn_b, np.uint16),
              ptr(mw.sgu.scales, np.uint16), ptr(mw.sgu.biases, np.uint16),
              ptr(mw.sdn.scales, np.uint16), ptr(mw.sdn.biases, np.uint16))
    y = np.empty((T, mw.H), dtype=np.float64)
    a = np.empty((T, mw.H), dtype=np.float64)
    h = np.empty((T, k, mw.I), dtype=np.float64) if want_h else None
    hs = np.empty((T, mw.Is), dtype=np.float64) if want_h else None
    _load().qo_moe_experts(ctypes.byref(st), px, T, k, pidx, pp, act,
                           y.ctypes.data_as(_P), a.ctypes.data_as(_P),
                           h.ctypes.data_as(_P) if want_h else None,
                           hs.ctypes.data_as(_P) if want_h else None)
    if want_h:
        return y, a, h, hs
    return y, a


def moe_layer(mw, x_bits, k: int = 8, act: int = 0, x_dtype: str = "f16"):
    """Whole MoE layer: int8 router GEMV -> top-k -> expert block.

    Returns dict with logits, logits_abs, idx, p, y, A.
    """
    xd = f16_to_f64(x_bits) if x_dtype == "f16" else bf16_to_f64(x_bits)
    xd = np.atleast_2d(xd)
    logits, la = gemv(mw.router, xd)
    idx, p = route_topk(logits, k)
    y, a = moe_experts(mw, xd, idx, p, act)
    return dict(logits=logits, logits_abs=la, idx=idx, p=p, y=y, A=a)


def tolerance(a) -> np.ndarray:
    """Per-output bound on |y_gpu - y_ref|: 1e-4 * sum|w x| + 1e-6."""
    return 1e-4 * np.asarray(a) + 1e-6
