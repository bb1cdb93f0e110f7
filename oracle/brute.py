"""Second, independent CPU implementation for tiny inputs (numpy + Python).

TEST INFRASTRUCTURE ONLY. It pins the C oracle: every step is written a
different way from ``oracle.c`` so that a slip in one (a wrong shift, a
dropped term, a transposed operand) shows up as a disagreement:

  * codes come from integer division and modulo of the packed word
    (``word // base**i % base``), not from shifts and masks;
  * fp16/bf16 values come from numpy's own float16 / float32 decoding;
  * the contraction is numpy's float64 matrix product of the dequantized
    matrix (a library routine);
  * top-k is Python's stable ``sorted`` over (-logit, index);
  * GELU uses ``math.erf`` / ``math.tanh``.
"""
from __future__ import annotations

import math

import numpy as np


def f16(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16(bits) -> np.ndarray:
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) * np.uint32(65536)
    with np.errstate(invalid="ignore"):
        return u32.view(np.float32).astype(np.float64)


def codes(bits: int, wq: np.ndarray, K: int) -> np.ndarray:
    """Integer codes [N][K] by division/modulo of each packed word."""
    base = 1 << bits
    per = 32 // bits
    words = np.asarray(wq, dtype=np.uint32).astype(np.int64)
    N = words.shape[0]
    out = np.empty((N, K), dtype=np.int64)
    for k in range(K):
        out[:, k] = (words[:, k // per] // (base ** (k % per))) % base
    return out


def dense(w) -> np.ndarray:
    """fp64 matrix [N][K] of a synth.AffineWeights: s*q + b per group of 64."""
    q = codes(w.bits, w.wq, w.K)
    s = np.repeat(f16(w.scales), 64, axis=1)
    b = np.repeat(f16(w.biases), 64, axis=1)
    return s * q + b


def mirai_dense(w) -> np.ndarray:
    """fp64 matrix [N][K] of a synth.MiraiWeights.

    Mirai-M: s * (q - z) with the zero points decoded by the same division
    route as the codes; Mirai-L: s * q with q the byte read as numpy int8.
    """
    G = w.K // 64
    s = np.repeat(bf16(w.scales), 64, axis=1)
    if w.fmt == "M":
        q = codes(4, w.wq, w.K)
        z = codes(4, w.zeros, G)
        return s * (q - np.repeat(z, 64, axis=1))
    q = np.ascontiguousarray(w.wq, dtype=np.uint32).view(np.int8).astype(np.float64)
    return s * q


def mirai_gemv(w, x: np.ndarray) -> np.ndarray:
    return np.atleast_2d(x) @ mirai_dense(w).T


def rotation(K: int, signs) -> np.ndarray:
    """The block-diagonal rotation R [K][K] = diag over blocks of H_32 D_b / sqrt(32),
    from scipy's Hadamard matrix and the sign bits read with divmod."""
    from scipy.linalg import hadamard
    H = hadamard(32).astype(np.float64) / math.sqrt(32.0)
    R = np.zeros((K, K))
    for b in range(K // 32):
        word = int(signs[b]) if signs is not None else 0
        d = np.array([-1.0 if (word // 2 ** j) % 2 else 1.0 for j in range(32)])
        R[32 * b:32 * b + 32, 32 * b:32 * b + 32] = H * d[None, :]
    return R


def rmsnorm(x, gamma=None, eps: float = 1e-6) -> np.ndarray:
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    g = np.ones(x.shape[1]) if gamma is None else np.asarray(gamma, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps) * g[None, :]


def gemv(w, x: np.ndarray) -> np.ndarray:
    return np.atleast_2d(x) @ dense(w).T


def route_topk(logits, k: int):
    L = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    T, E = L.shape
    idx = np.zeros((T, k), dtype=np.int32)
    p = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-L[t, e], e))[:k]
        ex = [math.exp(L[t, e] - L[t].max()) for e in range(E)]
        tot = math.fsum(ex)
        probs = [ex[e] / tot for e in order]
        kept = math.fsum(probs)
        idx[t] = order
        p[t] = [v / kept for v in probs]
    return idx, p


def gelu(u: float, variant: int = 0) -> float:
    if variant == 1:
        return 0.5 * u * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3)))
    return 0.5 * u * (1.0 + math.erf(u / math.sqrt(2.0)))


def moe_experts(mw, x, idx, p, act: int = 0):
    x = np.atleast_2d(x)
    T = x.shape[0]
    y = np.zeros((T, mw.H))
    ge = np.vectorize(lambda u: gelu(u, act))
    for t in range(T):
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            z = dense(mw.expert_gu(e)) @ x[t]
            h = ge(z[:mw.I]) * z[mw.I:]
            y[t] += p[t, j] * (dense(mw.expert_dn(e)) @ h)
        z = dense(mw.sgu) @ x[t]
        hs = ge(z[:mw.Is]) * z[mw.Is:]
        y[t] += dense(mw.sdn) @ hs
    return y


def attn_decode(q, k_new, v_new, kc, vc, window: int, pos: int, scale: float):
    """Decode attention by a second route: copy the caches, store the new
    token at its slot, keep the occupied slots, and use scipy's softmax and
    numpy matrix products per query head."""
    from scipy.special import softmax
    q = np.asarray(q, np.float64)
    kc = np.array(kc, np.float64)
    vc = np.array(vc, np.float64)
    Hq, D = q.shape
    Hkv, cap, _ = kc.shape
    slot = pos - (pos // window) * window if window else pos
    kc[:, slot] = k_new
    vc[:, slot] = v_new
    n = min(pos + 1, window) if window else pos + 1
    out = np.zeros((Hq, D))
    for h in range(Hq):
        hk = h // (Hq // Hkv)
        p = softmax(scale * (kc[hk, :n] @ q[h]))
        out[h] = p @ vc[hk, :n]
    return out


def quant_i8(x_bits):
    """Per-token int8 quantization by a second route: numpy float32 array
    arithmetic (maximum of |x|, the scale max/127, x/scale rounded half to
    even by np.rint), zero rows kept at zero."""
    x = np.atleast_2d(np.asarray(x_bits, np.uint16)).view(np.float16).astype(np.float32)
    amax = np.max(np.abs(x), axis=1)
    sc = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(sc > 0, sc, np.float32(1.0)).astype(np.float32)
    q = np.rint(x / safe[:, None]).astype(np.float32)
    q = np.where(sc[:, None] > 0, q, np.float32(0.0)).astype(np.int8)
    return q, sc
