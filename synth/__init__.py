"""Seeded synthetic inputs for the affine-quantized decode path.

This module only draws random inputs. It holds none of the method's
arithmetic (no unpacking, no dequantization, no contraction), so that the
CPU oracle under ``oracle/`` and the HIP path can both be fed from it
without sharing any of the computation they are compared on.

Weight format (TurboFieldfare article, "성능과 제약" section: MLX affine
4-bit weights with group 64, router at 8 bits): per output row n and group
g of 64 inputs there is one fp16 scale s and one fp16 bias b, and a code q
per input, with w = s*q + b. Codes are drawn as uniform random uint32
words: every nibble (4-bit) or byte (8-bit) of a uniform word is an
independent uniform code, so no packing step is needed here.

Distributions (the workload description the build targets):
  * int4 scales fp16(U[0.002, 0.02]); bias fp16(-8*s + N(0, sigma=1e-3)),
    with s the fp16-rounded scale;
  * int8 router scales fp16(U[0.002, 0.02] * 15/255); bias
    fp16(-128*s + N(0, 1e-3)), so that int8 weights span the same range
    as int4 ones;
  * decode activations fp16(N(0, 1)); prefill activations bf16(N(0, 1)).

Mirai formats (uzu page on discuss.pytorch.kr, section on model conversion
and the Mirai quantization formats): Mirai-M has 4-bit codes, a bf16 scale
and a 4-bit zero point per group of 64; Mirai-L has signed 8-bit codes and
a bf16 scale per group of 64. Drawn as:
  * Mirai-M scales bf16(U[0.002, 0.02]); zero points uniform in [0, 15],
    packed eight per uint32 along the groups of a row, rows padded to whole
    words (the padding nibbles are random too);
  * Mirai-L scales bf16(U[0.002, 0.02] / 16); codes uniform bytes, so
    every signed value in [-128, 127] occurs.

Every stream is numpy Generator(PCG64(SeedSequence([cfg, set, tensor]))).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 64

# tensor ids inside one weight set
T_CODES, T_SCALE, T_BIAS, T_X, T_SIGNS, T_GAMMA = 0, 1, 2, 3, 4, 5


def rng(cfg: int, set_id: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, set_id, tensor])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); return the raw uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


@dataclass
class AffineWeights:
    """Packed affine-quantized matrix [N][K]: codes wq (uint32), scales and biases as fp16 bits."""
    bits: int
    N: int
    K: int
    wq: np.ndarray      # uint32 [N][K*bits/32]
    scales: np.ndarray  # uint16 (fp16 bits) [N][K/64]
    biases: np.ndarray  # uint16 (fp16 bits) [N][K/64]

    @property
    def nbytes(self) -> int:
        return self.wq.nbytes + self.scales.nbytes + self.biases.nbytes


def _pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes [N][K] LSB-first into uint32 words (code i of a word at
    bits [bits*i, bits*(i+1)))."""
    per_word = 32 // bits
    N, K = q.shape
    qq = q.astype(np.uint64).reshape(N, K // per_word, per_word)
    shifts = (np.arange(per_word, dtype=np.uint64) * np.uint64(bits))
    return (qq << shifts).sum(axis=2).astype(np.uint32)


def affine_weights(bits: int, N: int, K: int, cfg: int, set_id: int, tensor_base: int = 0,
                   codes: str = "uniform", const_code: int = 0, code_set=None,
                   bias_code: float | None = None) -> AffineWeights:
    """Draw one packed weight matrix.

    codes: "uniform" (random words), "zero" (all codes 0), "const" (every
    code equal to ``const_code``) or "set" (each code drawn uniformly from
    ``code_set``). bias_code: the code c in b = fp16(-c*s + N(0, 1e-3));
    default the middle code (8 or 128), so that a weight w = s*q + b sits near
    zero when q = c.
    """
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    if K % GROUP:
        raise ValueError("K must be a multiple of 64")
    per_word = 32 // bits
    G = K // GROUP
    if codes == "uniform":
        wq = rng(cfg, set_id, tensor_base + T_CODES).integers(
            0, 2**32, size=(N, K // per_word), dtype=np.uint32)
    elif codes == "zero":
        wq = np.zeros((N, K // per_word), dtype=np.uint32)
    elif codes == "const":
        c = int(const_code)
        if not 0 <= c < (1 << bits):
            raise ValueError("const_code out of range")
        word = 0
        for i in range(per_word):
            word |= c << (bits * i)
        wq = np.full((N, K // per_word), word, dtype=np.uint32)
    elif codes == "set":
        vals = np.asarray(list(code_set), dtype=np.int64)
        if vals.size == 0 or vals.min() < 0 or vals.max() >= (1 << bits):
            raise ValueError("code_set out of range")
        q = vals[rng(cfg, set_id, tensor_base + T_CODES).integers(0, vals.size, size=(N, K))]
        wq = _pack_codes(q, bits)
    else:
        raise ValueError(codes)
    su = rng(cfg, set_id, tensor_base + T_SCALE).uniform(0.002, 0.02, size=(N, G))
    if bits == 8:
        su = su * (15.0 / 255.0)
    s16 = su.astype(np.float16)
    mid = (8.0 if bits == 4 else 128.0) if bias_code is None else float(bias_code)
    noise = rng(cfg, set_id, tensor_base + T_BIAS).normal(0.0, 1e-3, size=(N, G))
    b16 = (-mid * s16.astype(np.float64) + noise).astype(np.float16)
    return AffineWeights(bits, N, K, wq, s16.view(np.uint16), b16.view(np.uint16))


@dataclass
class MiraiWeights:
    """Packed Mirai-M ("M") or Mirai-L ("L") matrix [N][K].

    wq: uint32 [N][K/8] (M) or [N][K/4] (L, signed bytes); scales: bf16 bits
    [N][K/64]; zeros: uint32 [N][ceil(K/512)] (M) or None (L).
    """
    fmt: str
    N: int
    K: int
    wq: np.ndarray
    scales: np.ndarray
    zeros: np.ndarray | None

    @property
    def bits(self) -> int:
        return 4 if self.fmt == "M" else 8

    @property
    def nbytes(self) -> int:
        return self.wq.nbytes + self.scales.nbytes + (0 if self.zeros is None else self.zeros.nbytes)


def _const_words(N: int, words: int, bits: int, value: int) -> np.ndarray:
    word = 0
    for i in range(32 // bits):
        word |= (value & ((1 << bits) - 1)) << (bits * i)
    return np.full((N, words), word, dtype=np.uint32)


def mirai_weights(fmt: str, N: int, K: int, cfg: int, set_id: int, tensor_base: int = 0,
                  codes: str = "uniform", const_code: int = 0,
                  zeros: str = "uniform", const_zero: int = 0,
                  code_set=None) -> MiraiWeights:
    """Draw one packed Mirai-M / Mirai-L matrix.

    codes: "uniform", "const" (every code ``const_code``: 0..15 for M,
    -128..127 for L) or "set" (each code drawn uniformly from ``code_set``,
    same ranges); zeros (M only): "uniform" or "const" (``const_zero``).
    """
    if fmt not in ("M", "L"):
        raise ValueError("fmt must be 'M' or 'L'")
    if K % GROUP:
        raise ValueError("K must be a multiple of 64")
    bits = 4 if fmt == "M" else 8
    G = K // GROUP
    words = K * bits // 32
    if codes == "uniform":
        wq = rng(cfg, set_id, tensor_base + T_CODES).integers(0, 2**32, size=(N, words), dtype=np.uint32)
    elif codes == "const":
        lo, hi = (0, 15) if fmt == "M" else (-128, 127)
        if not lo <= const_code <= hi:
            raise ValueError("const_code out of range")
        wq = _const_words(N, words, bits, int(const_code))
    elif codes == "set":
        lo, hi = (0, 15) if fmt == "M" else (-128, 127)
        vals = np.asarray(list(code_set), dtype=np.int64)
        if vals.size == 0 or vals.min() < lo or vals.max() > hi:
            raise ValueError("code_set out of range")
        q = vals[rng(cfg, set_id, tensor_base + T_CODES).integers(0, vals.size, size=(N, K))]
        wq = _pack_codes(q & ((1 << bits) - 1), bits)
    else:
        raise ValueError(codes)
    su = rng(cfg, set_id, tensor_base + T_SCALE).uniform(0.002, 0.02, size=(N, G))
    if fmt == "L":
        su = su / 16.0
    sb = f32_to_bf16_bits(su.astype(np.float32))
    zq = None
    if fmt == "M":
        zw = (G + 7) // 8
        if zeros == "uniform":
            zq = rng(cfg, set_id, tensor_base + T_BIAS).integers(0, 2**32, size=(N, zw), dtype=np.uint32)
        elif zeros == "const":
            if not 0 <= const_zero <= 15:
                raise ValueError("const_zero out of range")
            zq = _const_words(N, zw, 4, int(const_zero))
        else:
            raise ValueError(zeros)
    return MiraiWeights(fmt, N, K, wq, sb, zq)


def rht_signs(K: int, cfg: int, set_id: int) -> np.ndarray:
    """Random signs of a block-32 Hadamard rotation: uint32 [K/32], bit j of word b
    set = input 32b + j negated (each bit an independent fair coin)."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    return rng(cfg, set_id, T_SIGNS).integers(0, 2**32, size=K // 32, dtype=np.uint32)


def rmsnorm_gamma(K: int, cfg: int, set_id: int, dtype: str = "f16") -> np.ndarray:
    """RMSNorm weights U[0.5, 1.5] as fp16 or bf16 bits [K]."""
    g = rng(cfg, set_id, T_GAMMA).uniform(0.5, 1.5, size=K)
    if dtype == "f16":
        return g.astype(np.float16).view(np.uint16)
    return f32_to_bf16_bits(g.astype(np.float32))


def attn_inputs(Hq: int, Hkv: int, D: int, cap: int, cfg: int, set_id: int,
                scale_q: float = 1.0) -> dict:
    """Decode-attention inputs as fp16 bits, all N(0, 1) (queries times scale_q):
    q [Hq][D], k_new / v_new [Hkv][D], k_cache / v_cache [Hkv][cap][D]."""
    r = rng(cfg, set_id, T_X)
    f = lambda shape, sc=1.0: (r.standard_normal(shape) * sc).astype(np.float16).view(np.uint16)
    return dict(q=f((Hq, D), scale_q), k_new=f((Hkv, D)), v_new=f((Hkv, D)),
                k_cache=f((Hkv, cap, D)), v_cache=f((Hkv, cap, D)))


def x_f16(T: int, K: int, cfg: int, set_id: int, tensor: int = T_X) -> np.ndarray:
    """Decode activations: fp16 N(0,1), returned as uint16 bits [T][K]."""
    return rng(cfg, set_id, tensor).standard_normal((T, K)).astype(np.float16).view(np.uint16)


def x_bf16(T: int, K: int, cfg: int, set_id: int, tensor: int = T_X) -> np.ndarray:
    """Prefill activations: bf16 N(0,1), returned as uint16 bits [T][K]."""
    v = rng(cfg, set_id, tensor).standard_normal((T, K)).astype(np.float32)
    return f32_to_bf16_bits(v)


@dataclass
class MoEWeights:
    """One MoE FFN layer: int8 router, E routed experts and one shared expert (int4).

    gate/up are fused per expert: rows [0, I) are gate, rows [I, 2I) are up.
    """
    E: int
    H: int
    I: int
    Is: int
    router: AffineWeights        # [E][H], 8-bit
    gu_wq: np.ndarray            # [E][2I][H/8]
    gu_s: np.ndarray             # [E][2I][H/64]
    gu_b: np.ndarray
    dn_wq: np.ndarray            # [E][H][I/8]
    dn_s: np.ndarray             # [E][H][I/64]
    dn_b: np.ndarray
    sgu: AffineWeights           # [2Is][H]
    sdn: AffineWeights           # [H][Is]

    @property
    def nbytes(self) -> int:
        return (self.router.nbytes + self.gu_wq.nbytes + self.gu_s.nbytes + self.gu_b.nbytes
                + self.dn_wq.nbytes + self.dn_s.nbytes + self.dn_b.nbytes
                + self.sgu.nbytes + self.sdn.nbytes)

    def expert_gu(self, e: int) -> AffineWeights:
        return AffineWeights(4, 2 * self.I, self.H, self.gu_wq[e], self.gu_s[e], self.gu_b[e])

    def expert_dn(self, e: int) -> AffineWeights:
        return AffineWeights(4, self.H, self.I, self.dn_wq[e], self.dn_s[e], self.dn_b[e])


def moe_weights(E: int, H: int, I: int, Is: int, cfg: int, layer: int,
                identical_experts: bool = False, flat_router: bool = False,
                expert_codes: dict | None = None) -> MoEWeights:
    """Draw one MoE layer. Tensor ids are spaced by 8 per matrix.

    identical_experts: every routed expert gets expert 0's tensors.
    flat_router: router codes all zero, and scales and biases all equal, so every
    router row holds the same stored values and all logits tie exactly.
    expert_codes: keyword arguments of ``affine_weights`` (codes, const_code,
    code_set, bias_code) for every expert matrix, routed and shared.
    """
    ek = dict(expert_codes or {})
    router = affine_weights(8, E, H, cfg, layer, 0)
    if flat_router:
        router = AffineWeights(8, E, H, np.zeros_like(router.wq),
                               np.full_like(router.scales, router.scales.flat[0]),
                               np.full_like(router.biases, router.biases.flat[0]))
    gus, dns = [], []
    for e in range(E):
        src = 0 if identical_experts else e
        gus.append(affine_weights(4, 2 * I, H, cfg, layer, 16 + 16 * src, **ek))
        dns.append(affine_weights(4, H, I, cfg, layer, 24 + 16 * src, **ek))
    sgu = affine_weights(4, 2 * Is, H, cfg, layer, 8, **ek)
    sdn = affine_weights(4, H, Is, cfg, layer, 12, **ek)
    return MoEWeights(
        E, H, I, Is, router,
        np.stack([a.wq for a in gus]), np.stack([a.scales for a in gus]),
        np.stack([a.biases for a in gus]),
        np.stack([a.wq for a in dns]), np.stack([a.scales for a in dns]),
        np.stack([a.biases for a in dns]),
        sgu, sdn)


# ---------------------------------------------------------------------------
# Workload shapes. These are the synthetic stand-ins for the pages' decode
# and prefill workloads (dense 7B/70B-class projections, and the Gemma-4
# 26B-A4B MoE layer with an 8-bit router, top-8 of 128 experts, a shared
# expert, 30 layers and prefill chunks of at most 128 tokens).
# ---------------------------------------------------------------------------
# "gemv" entries are (K inputs, N outputs).
CONFIGS = {
    "c1_dense_4096": dict(cfg=1, gemv=[(4096, 4096)], batch=[1], sets=64),
    "c2_7b_ffn": dict(cfg=2, gemv=[(4096, 2 * 14336), (14336, 4096)], batch=[1], sets=16),
    "c3_moe_decode": dict(cfg=3, E=128, H=2816, I=704, Is=2112, top_k=8, layers=30, T=1),
    "c4_chunk": dict(cfg=4, M=128, K=4096, N=14336, sets=16),
    "c4_moe_prefill": dict(cfg=4, E=128, H=2816, I=704, Is=2112, top_k=8, layers=30, T=128),
    "c5_70b_sweep": dict(cfg=5, gemv=[(8192, 28672), (28672, 8192)], batch=[1, 2, 4, 8], sets=80),
}
