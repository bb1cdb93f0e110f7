"""Pins of the fp64 CPU oracle against things other than itself.

Each check compares the oracle with an independent route to the same
number: exhaustive format decoding by numpy, a brute force that unpacks
with integer division, exact rational arithmetic, the grouped closed form
of the affine contraction, special inputs with known answers, Python's
stable sort, and textbook values of the normal CDF.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import brute


# ---------------------------------------------------------------- formats

def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.f16_to_f64(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    # signed zero
    assert math.copysign(1.0, oracle.f16_to_f64(np.array([0x8000], np.uint16))[0]) == -1.0


def test_bf16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = brute.bf16(bits)
    got = oracle.bf16_to_f64(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


@pytest.mark.parametrize("bits", [4, 8])
def test_code_unpack_matches_divmod(bits):
    w = synth.affine_weights(bits, 3, 256, cfg=90, set_id=bits)
    q = brute.codes(bits, w.wq, 256)
    for n in range(3):
        got = [oracle.code(bits, w.wq[n], k) for k in range(256)]
        assert got == list(q[n])
    assert q.min() == 0 and q.max() == (1 << bits) - 1


def test_code_order_lsb_first():
    # word 0x76543210: code k of the row is k (LSB-first nibble order)
    row = np.array([0x76543210, 0xFEDCBA98], dtype=np.uint32)
    assert [oracle.code(4, row, k) for k in range(16)] == list(range(16))
    row8 = np.array([0x03020100], dtype=np.uint32)
    assert [oracle.code(8, row8, k) for k in range(4)] == [0, 1, 2, 3]


# ---------------------------------------------------------------- GEMV

SHAPES = [(1, 64, 1), (3, 128, 2), (17, 256, 3), (5, 192, 8), (2, 64, 5)]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("N,K,T", SHAPES)
def test_gemv_matches_bruteforce(bits, N, K, T):
    w = synth.affine_weights(bits, N, K, cfg=91, set_id=N * 1000 + K + T)
    xb = synth.x_f16(T, K, cfg=91, set_id=N * 1000 + K + T)
    y, a = oracle.gemv_f16(w, xb)
    yb = brute.gemv(w, brute.f16(xb))
    assert y.shape == (T, N)
    assert np.all(np.abs(y - yb) <= 1e-12 * a + 1e-300)
    # A really is sum |w x|
    ab = np.abs(brute.f16(xb)) @ np.abs(brute.dense(w)).T
    assert np.allclose(a, ab, rtol=1e-13, atol=0)


def test_dequant_matches_bruteforce():
    w = synth.affine_weights(4, 5, 192, cfg=92, set_id=0)
    assert np.array_equal(oracle.dequant(w), brute.dense(w))


@pytest.mark.parametrize("bits", [4, 8])
def test_gemv_against_exact_rationals(bits):
    N, K, T = 3, 128, 2
    w = synth.affine_weights(bits, N, K, cfg=93, set_id=bits)
    xb = synth.x_f16(T, K, cfg=93, set_id=bits)
    y, a = oracle.gemv_f16(w, xb)
    q = brute.codes(bits, w.wq, K)
    s = [[Fraction(float(v)) for v in row] for row in w.scales.view(np.float16)]
    b = [[Fraction(float(v)) for v in row] for row in w.biases.view(np.float16)]
    x = [[Fraction(float(v)) for v in row] for row in xb.view(np.float16)]
    for t in range(T):
        for n in range(N):
            exact = sum((s[n][k // 64] * int(q[n, k]) + b[n][k // 64]) * x[t][k] for k in range(K))
            assert abs(float(exact) - y[t, n]) <= 4 * K * 2.0 ** -53 * a[t, n]


@pytest.mark.parametrize("bits", [4, 8])
def test_gemv_grouped_closed_form(bits):
    # y_n = sum_g s_g * (q . x)_g + b_g * (sum x)_g
    N, K, T = 7, 320, 2
    w = synth.affine_weights(bits, N, K, cfg=94, set_id=bits)
    xb = synth.x_f16(T, K, cfg=94, set_id=bits)
    x = brute.f16(xb)
    q = brute.codes(bits, w.wq, K).astype(np.float64)
    s, b = brute.f16(w.scales), brute.f16(w.biases)
    G = K // 64
    qx = np.einsum("nk,tk->tnk", q, x).reshape(T, N, G, 64).sum(-1)      # (q.x)_g
    xs = x.reshape(T, G, 64).sum(-1)                                      # (sum x)_g
    yc = (s[None] * qx).sum(-1) + (b[None] * xs[:, None, :]).sum(-1)
    y, a = oracle.gemv_f16(w, xb)
    assert np.all(np.abs(y - yc) <= 1e-12 * a)


@pytest.mark.parametrize("bits", [4, 8])
def test_zero_codes_give_bias_term(bits):
    N, K = 4, 256
    w = synth.affine_weights(bits, N, K, cfg=95, set_id=0, codes="zero")
    xb = synth.x_f16(1, K, cfg=95, set_id=0)
    x = brute.f16(xb)[0]
    y, a = oracle.gemv_f16(w, xb)
    xs = x.reshape(-1, 64).sum(-1)
    exp = (brute.f16(w.biases) * xs[None]).sum(-1)
    assert np.allclose(y[0], exp, rtol=0, atol=1e-13 * a.max())


@pytest.mark.parametrize("bits,c", [(4, 0), (4, 7), (4, 15), (8, 200)])
def test_constant_codes(bits, c):
    N, K = 3, 192
    w = synth.affine_weights(bits, N, K, cfg=96, set_id=c, codes="const", const_code=c)
    xb = synth.x_f16(1, K, cfg=96, set_id=c)
    x = brute.f16(xb)[0]
    y, a = oracle.gemv_f16(w, xb)
    xs = x.reshape(-1, 64).sum(-1)
    exp = ((c * brute.f16(w.scales) + brute.f16(w.biases)) * xs[None]).sum(-1)
    assert np.allclose(y[0], exp, rtol=0, atol=1e-13 * a.max())


def test_zero_activation_gives_exact_zero():
    w = synth.affine_weights(4, 5, 128, cfg=97, set_id=0)
    y, a = oracle.gemv_f16(w, np.zeros((2, 128), np.uint16))
    assert np.all(y == 0.0) and np.all(a == 0.0)


@pytest.mark.parametrize("bits", [4, 8])
def test_one_hot_activation_is_exact_weight(bits):
    N, K = 4, 256
    w = synth.affine_weights(bits, N, K, cfg=98, set_id=bits)
    q = brute.codes(bits, w.wq, K)
    one = np.float16(1.0).view(np.uint16)
    for k in (0, 5, 63, 64, 200, 255):
        xb = np.zeros((1, K), np.uint16)
        xb[0, k] = one
        y, _ = oracle.gemv_f16(w, xb)
        sv = w.scales.view(np.float16)[:, k // 64].astype(np.float64)
        bv = w.biases.view(np.float16)[:, k // 64].astype(np.float64)
        assert np.array_equal(y[0], sv * q[:, k] + bv)


def test_rows_variant_matches_full():
    w = synth.affine_weights(4, 33, 256, cfg=99, set_id=0)
    xb = synth.x_f16(2, 256, cfg=99, set_id=0)
    y, a = oracle.gemv_f16(w, xb)
    rows = np.array([0, 7, 32, 13])
    yr, ar = oracle.gemv_f16(w, xb, rows=rows)
    assert np.array_equal(yr, y[:, rows]) and np.array_equal(ar, a[:, rows])


def test_chunk_is_rowwise_gemv_on_bf16():
    w = synth.affine_weights(4, 9, 192, cfg=100, set_id=0)
    X = synth.x_bf16(5, 192, cfg=100, set_id=0)
    Y, A = oracle.gemm_chunk(w, X)
    Yb = brute.gemv(w, brute.bf16(X))
    assert np.all(np.abs(Y - Yb) <= 1e-12 * A)
    for m in range(5):
        ym, _ = oracle.gemv(w, brute.bf16(X[m:m + 1]))
        assert np.array_equal(ym[0], Y[m])


# ---------------------------------------------------------------- routing

def test_topk_matches_stable_sort():
    r = np.random.default_rng(5)
    L = r.standard_normal((20, 128)) * 3
    L[3, 10] = L[3, 20] = L[3, 5] = L[3].max() + 1.0      # three-way tie at the top
    L[4, :] = 0.5                                           # all tied
    idx, p = oracle.route_topk(L, 8)
    ib, pb = brute.route_topk(L, 8)
    assert np.array_equal(idx, ib)
    assert np.allclose(p, pb, rtol=1e-14, atol=1e-15)
    assert list(idx[3, :3]) == [5, 10, 20]
    assert list(idx[4]) == list(range(8))
    assert np.allclose(p[4], 1.0 / 8, rtol=0, atol=1e-15)
    assert np.allclose(p.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(p, axis=1) <= 0)


def test_topk_renormalized_softmax_identity():
    # softmax over all experts then renormalizing over the kept ones equals a
    # softmax over the kept logits alone
    r = np.random.default_rng(6)
    L = r.standard_normal((10, 64)) * 2
    idx, p = oracle.route_topk(L, 8)
    for t in range(10):
        kl = L[t, idx[t]]
        direct = np.exp(kl - kl.max()) / np.exp(kl - kl.max()).sum()
        assert np.allclose(p[t], direct, rtol=1e-13, atol=0)


def test_topk_k_equals_e_and_bad_sizes():
    L = np.array([[1.0, 3.0, 2.0]])
    idx, p = oracle.route_topk(L, 3)
    assert list(idx[0]) == [1, 2, 0]
    with pytest.raises(ValueError):
        oracle.route_topk(L, 4)


# ---------------------------------------------------------------- GELU

def test_gelu_textbook_values_and_identities():
    # GELU(u) = u * Phi(u); Phi(1) = 0.8413447460685429, Phi(2) = 0.9772498680518208
    assert abs(oracle.gelu(1.0) - 0.8413447460685429) < 1e-15
    assert abs(oracle.gelu(2.0) - 2 * 0.9772498680518208) < 2e-15
    assert abs(oracle.gelu(-1.0) + (1 - 0.8413447460685429)) < 1e-15
    for v in (0, 1):
        assert oracle.gelu(0.0, v) == 0.0
        for u in (0.1, 0.7, 1.3, 3.0, 6.5):
            assert abs(oracle.gelu(u, v) - oracle.gelu(-u, v) - u) < 1e-14
        assert abs(oracle.gelu(40.0, v) - 40.0) < 1e-12
        assert abs(oracle.gelu(-40.0, v)) < 1e-12


def test_gelu_against_torch():
    import torch
    u = torch.linspace(-6, 6, 241, dtype=torch.float64)
    ex = torch.nn.functional.gelu(u)
    th = torch.nn.functional.gelu(u, approximate="tanh")
    for i in range(u.numel()):
        assert abs(oracle.gelu(float(u[i]), 0) - float(ex[i])) < 1e-14
        assert abs(oracle.gelu(float(u[i]), 1) - float(th[i])) < 1e-14


# ---------------------------------------------------------------- MoE block

def _tiny_moe(**kw):
    return synth.moe_weights(E=6, H=128, I=64, Is=128, cfg=101, layer=0, **kw)


@pytest.mark.parametrize("act", [0, 1])
def test_moe_block_matches_bruteforce(act):
    mw = _tiny_moe()
    xb = synth.x_f16(3, 128, cfg=101, set_id=1)
    x = brute.f16(xb)
    logits, _ = oracle.gemv(mw.router, x)
    idx, p = oracle.route_topk(logits, 3)
    y, a = oracle.moe_experts(mw, x, idx, p, act)
    yb = brute.moe_experts(mw, x, idx, p, act)
    assert np.all(np.abs(y - yb) <= 1e-12 * a + 1e-300)


def test_moe_identical_experts_do_not_depend_on_routing():
    mw = _tiny_moe(identical_experts=True)
    xb = synth.x_f16(1, 128, cfg=101, set_id=2)
    x = brute.f16(xb)
    ya, aa = oracle.moe_experts(mw, x, np.array([[0, 1, 2]]), np.array([[0.5, 0.3, 0.2]]))
    yb, _ = oracle.moe_experts(mw, x, np.array([[5, 3, 4]]), np.array([[0.6, 0.25, 0.15]]))
    assert np.all(np.abs(ya - yb) <= 1e-12 * aa)
    # equals one expert with weight one plus the shared expert
    y1, _ = oracle.moe_experts(mw, x, np.array([[2]]), np.array([[1.0]]))
    assert np.all(np.abs(ya - y1) <= 1e-12 * aa)


def test_flat_router_routes_first_k_evenly():
    mw = _tiny_moe(flat_router=True)
    xb = synth.x_f16(2, 128, cfg=101, set_id=3)
    out = oracle.moe_layer(mw, xb, k=4)
    assert np.all(out["idx"] == np.arange(4))
    assert np.allclose(out["p"], 0.25, rtol=0, atol=1e-15)


def test_moe_layer_composes_steps():
    mw = _tiny_moe()
    xb = synth.x_f16(2, 128, cfg=101, set_id=4)
    out = oracle.moe_layer(mw, xb, k=2)
    x = brute.f16(xb)
    assert np.allclose(out["logits"], brute.gemv(mw.router, x), rtol=0, atol=1e-12 * out["logits_abs"].max())
    ib, _ = brute.route_topk(out["logits"], 2)
    assert np.array_equal(out["idx"], ib)


# ---------------------------------------------------------------- inputs

def test_generator_is_deterministic_and_in_range():
    a = synth.affine_weights(4, 16, 256, cfg=1, set_id=3)
    b = synth.affine_weights(4, 16, 256, cfg=1, set_id=3)
    c = synth.affine_weights(4, 16, 256, cfg=1, set_id=4)
    assert a.wq.tobytes() == b.wq.tobytes() and a.scales.tobytes() == b.scales.tobytes()
    assert a.wq.tobytes() != c.wq.tobytes()
    s = a.scales.view(np.float16).astype(np.float64)
    assert s.min() >= np.float16(0.002) and s.max() <= np.float16(0.02)
    bias = a.biases.view(np.float16).astype(np.float64)
    assert np.all(np.abs(bias + 8 * s) < 0.01)
    x = synth.x_bf16(4, 256, cfg=1, set_id=0)
    xd = brute.bf16(x)
    assert abs(xd.mean()) < 0.2 and 0.8 < xd.std() < 1.2


# ---------------------------------------------------------------- Mirai formats
# uzu page (discuss.pytorch.kr), section on model conversion and the Mirai
# quantization formats: Mirai-M = 4-bit asymmetric codes, 4-bit zero point,
# bf16 scale, group 64; Mirai-L = 8-bit symmetric.

MIRAI_SHAPES = [(1, 64, 1), (3, 128, 2), (5, 704, 3), (4, 1024, 8), (2, 576, 5)]


@pytest.mark.parametrize("fmt", ["M", "L"])
@pytest.mark.parametrize("N,K,T", MIRAI_SHAPES)
def test_mirai_gemv_matches_bruteforce(fmt, N, K, T):
    w = synth.mirai_weights(fmt, N, K, cfg=120, set_id=N * 1000 + K + T)
    xb = synth.x_f16(T, K, cfg=120, set_id=N * 1000 + K + T)
    y, a = oracle.mirai_gemv_x(w, xb)
    d = brute.mirai_dense(w)
    assert np.array_equal(oracle.mirai_dequant(w), d)
    yb = brute.f16(xb) @ d.T
    assert np.all(np.abs(y - yb) <= 1e-12 * a + 1e-300)
    assert np.allclose(a, np.abs(brute.f16(xb)) @ np.abs(d).T, rtol=1e-13, atol=0)


@pytest.mark.parametrize("fmt", ["M", "L"])
def test_mirai_gemv_against_exact_rationals(fmt):
    N, K, T = 3, 192, 2
    w = synth.mirai_weights(fmt, N, K, cfg=121, set_id=0)
    xb = synth.x_f16(T, K, cfg=121, set_id=0)
    y, a = oracle.mirai_gemv_x(w, xb)
    G = K // 64
    s = [[Fraction(float(v)) for v in row] for row in brute.bf16(w.scales)]
    x = [[Fraction(float(v)) for v in row] for row in xb.view(np.float16)]
    for n in range(N):
        raw = [int(v) for v in np.ascontiguousarray(w.wq[n]).view(np.uint8)]
        if fmt == "M":
            # code k is nibble k of the row's little-endian byte stream
            q = [(raw[k // 2] >> (4 * (k % 2))) & 15 for k in range(K)]
            zb = [int(v) for v in np.ascontiguousarray(w.zeros[n]).view(np.uint8)]
            z = [(zb[g // 2] >> (4 * (g % 2))) & 15 for g in range(G)]
            wk = [s[n][k // 64] * (q[k] - z[k // 64]) for k in range(K)]
        else:
            q = [v - 256 if v >= 128 else v for v in raw]
            wk = [s[n][k // 64] * q[k] for k in range(K)]
        for t in range(T):
            exact = sum(wk[k] * x[t][k] for k in range(K))
            assert abs(float(exact) - y[t, n]) <= 4 * K * 2.0 ** -53 * a[t, n]


def test_mirai_m_explicit_decode():
    # one row, K = 512 (8 groups): codes all 15, zero point of group g is g
    K = 512
    w = synth.MiraiWeights("M", 1, K, np.full((1, K // 8), 0xFFFFFFFF, np.uint32),
                           np.full((1, 8), 0x3F80, np.uint16),           # bf16 1.0
                           np.array([[0x76543210]], np.uint32))
    d = oracle.mirai_dequant(w)
    assert np.array_equal(d[0], np.repeat(15.0 - np.arange(8), 64))
    # scale 0.5 (bf16 0x3F00), zero point 8 everywhere, codes k mod 16
    row = np.array([[0x76543210, 0xFEDCBA98] * (K // 16)], np.uint32)
    w2 = synth.MiraiWeights("M", 1, K, row, np.full((1, 8), 0x3F00, np.uint16),
                            np.array([[0x88888888]], np.uint32))
    assert np.array_equal(oracle.mirai_dequant(w2)[0], 0.5 * (np.arange(K) % 16 - 8))


def test_mirai_l_explicit_decode():
    # bytes FF 01 7F 80 -> -1, 1, 127, -128 (two's complement), scale 2.0 (bf16 0x4000)
    K = 64
    w = synth.MiraiWeights("L", 1, K, np.full((1, K // 4), 0x807F01FF, np.uint32),
                           np.array([[0x4000]], np.uint16), None)
    assert np.array_equal(oracle.mirai_dequant(w)[0], np.tile([-2.0, 2.0, 254.0, -256.0], 16))


def test_mirai_m_zero_point_padding_is_ignored():
    # K = 704: 11 groups, so nibbles 11..15 of the second zero-point word are padding
    w = synth.mirai_weights("M", 6, 704, cfg=122, set_id=0)
    xb = synth.x_f16(2, 704, cfg=122, set_id=0)
    y1, _ = oracle.mirai_gemv_x(w, xb)
    z2 = w.zeros.copy()
    z2[:, 1] ^= np.uint32(0xFFFFF000)
    y2, _ = oracle.mirai_gemv_x(synth.MiraiWeights("M", 6, 704, w.wq, w.scales, z2), xb)
    assert np.array_equal(y1, y2)
    z3 = w.zeros.copy()
    z3[:, 1] ^= np.uint32(0x00000F00)      # group 10's zero point does matter
    y3, _ = oracle.mirai_gemv_x(synth.MiraiWeights("M", 6, 704, w.wq, w.scales, z3), xb)
    assert not np.array_equal(y1, y3)


def test_mirai_m_equals_affine_with_bias_minus_s_z():
    # With scales of at most 7 significant bits, s and -s*z are exact in fp16,
    # so Mirai-M (s, z) is the affine format (s, b = -s*z) weight for weight:
    # both oracle routes must agree bit for bit.
    N, K = 9, 1024
    w = synth.mirai_weights("M", N, K, cfg=123, set_id=0)
    sb = (w.scales & np.uint16(0xFFFE)).astype(np.uint16)
    w = synth.MiraiWeights("M", N, K, w.wq, sb, w.zeros)
    s = brute.bf16(sb)
    z = brute.codes(4, w.zeros, K // 64).astype(np.float64)
    s16, b16 = s.astype(np.float16), (-s * z).astype(np.float16)
    assert np.array_equal(s16.astype(np.float64), s) and np.array_equal(b16.astype(np.float64), -s * z)
    aw = synth.AffineWeights(4, N, K, w.wq, s16.view(np.uint16), b16.view(np.uint16))
    xb = synth.x_f16(3, K, cfg=123, set_id=0)
    ym, am = oracle.mirai_gemv_x(w, xb)
    ya, aa = oracle.gemv_f16(aw, xb)
    assert np.array_equal(ym, ya) and np.array_equal(am, aa)


def test_mirai_l_equals_affine8_with_offset_codes():
    # signed byte q = (q XOR 0x80) - 128, so Mirai-L (s) is the affine 8-bit
    # format with codes XOR 0x80 and bias -128*s (exact in fp16 for bf16 s)
    N, K = 7, 832
    w = synth.mirai_weights("L", N, K, cfg=124, set_id=0)
    s = brute.bf16(w.scales)
    s16, b16 = s.astype(np.float16), (-128.0 * s).astype(np.float16)
    assert np.array_equal(s16.astype(np.float64), s) and np.array_equal(b16.astype(np.float64), -128 * s)
    aw = synth.AffineWeights(8, N, K, w.wq ^ np.uint32(0x80808080), s16.view(np.uint16),
                             b16.view(np.uint16))
    xb = synth.x_f16(2, K, cfg=124, set_id=0)
    ym, _ = oracle.mirai_gemv_x(w, xb)
    ya, _ = oracle.gemv_f16(aw, xb)
    assert np.array_equal(ym, ya)


def test_mirai_l_is_symmetric():
    # negating every code (none is -128) negates every output exactly
    N, K = 5, 512
    w = synth.mirai_weights("L", N, K, cfg=125, set_id=0)
    b = np.ascontiguousarray(w.wq).view(np.int8).copy()
    b[b == -128] = 127
    wpos = synth.MiraiWeights("L", N, K, b.view(np.uint32), w.scales, None)
    wneg = synth.MiraiWeights("L", N, K, (-b).view(np.uint32), w.scales, None)
    xb = synth.x_f16(2, K, cfg=125, set_id=0)
    yp, _ = oracle.mirai_gemv_x(wpos, xb)
    yn, _ = oracle.mirai_gemv_x(wneg, xb)
    assert np.array_equal(yp, -yn)


def test_mirai_code_equal_to_zero_point_gives_zero():
    w = synth.mirai_weights("M", 4, 512, cfg=126, set_id=0, codes="const", const_code=9,
                            zeros="const", const_zero=9)
    xb = synth.x_f16(2, 512, cfg=126, set_id=0)
    y, a = oracle.mirai_gemv_x(w, xb)
    assert np.all(y == 0.0) and np.all(a == 0.0)


def test_mirai_rows_variant_matches_full():
    w = synth.mirai_weights("M", 40, 704, cfg=127, set_id=0)
    xb = synth.x_bf16(3, 704, cfg=127, set_id=0)
    y, a = oracle.mirai_gemv_x(w, xb, "bf16")
    rows = np.array([0, 7, 39, 13])
    yr, ar = oracle.mirai_gemv_x(w, xb, "bf16", rows=rows)
    assert np.array_equal(yr, y[:, rows]) and np.array_equal(ar, a[:, rows])


def test_mirai_generator_ranges():
    m = synth.mirai_weights("M", 8, 1024, cfg=2, set_id=0)
    s = brute.bf16(m.scales)
    assert s.min() >= 0.00199 and s.max() <= 0.0201
    z = brute.codes(4, m.zeros, 16)
    assert z.min() == 0 and z.max() == 15
    el = synth.mirai_weights("L", 8, 1024, cfg=2, set_id=0)
    q = np.ascontiguousarray(el.wq).view(np.int8)
    assert q.min() == -128 and q.max() == 127
    assert brute.bf16(el.scales).max() <= 0.0201 / 16
    assert m.nbytes == 8 * (512 + 32 + 8)


# ---------------------------------------------------------------- rotation prologue
# uzu page (discuss.pytorch.kr), quantization-format section: a block-32
# random Hadamard transform applied before quantization, fused with RMSNorm
# and the matmul.

def test_rht_columns_are_scipy_hadamard():
    from scipy.linalg import hadamard
    K = 64
    eye = np.eye(K)
    cols = oracle.rht(eye)                      # row j = transform of unit vector j
    R = cols.T
    H = hadamard(32) / math.sqrt(32.0)
    assert np.allclose(R[:32, :32], H, rtol=0, atol=1e-15)
    assert np.allclose(R[32:, 32:], H, rtol=0, atol=1e-15)
    assert np.all(R[:32, 32:] == 0) and np.all(R[32:, :32] == 0)


def test_rht_with_signs_matches_explicit_rotation():
    K = 256
    sg = synth.rht_signs(K, cfg=130, set_id=0)
    x = np.random.default_rng(0).standard_normal((3, K))
    R = brute.rotation(K, sg)
    assert np.allclose(oracle.rht(x, sg), x @ R.T, rtol=0, atol=1e-13)
    # signs act on the inputs: rotate(x, d) = rotate(d * x, none)
    d = np.concatenate([[-1.0 if (int(w) >> j) & 1 else 1.0 for j in range(32)] for w in sg])
    assert np.allclose(oracle.rht(x, sg), oracle.rht(x * d[None, :]), rtol=0, atol=1e-13)


def test_rht_is_orthogonal_and_self_inverse_without_signs():
    K = 512
    x = np.random.default_rng(1).standard_normal((2, K))
    y = oracle.rht(x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    assert np.allclose(oracle.rht(y), x, rtol=0, atol=1e-13)
    sg = synth.rht_signs(K, cfg=131, set_id=0)
    assert np.allclose(np.linalg.norm(oracle.rht(x, sg), axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)


def test_rotated_weights_preserve_the_product():
    # W' = W R^T gives W' (R x) = W x: the reason the rotation can be fused
    K, N = 128, 5
    sg = synth.rht_signs(K, cfg=132, set_id=0)
    rng = np.random.default_rng(2)
    W, x = rng.standard_normal((N, K)), rng.standard_normal((1, K))
    R = brute.rotation(K, sg)
    assert np.allclose((W @ R.T) @ oracle.rht(x, sg)[0], W @ x[0], rtol=0, atol=1e-12)


def test_rmsnorm_closed_forms():
    K = 192
    c, eps = 3.0, 1e-6
    out = oracle.rmsnorm(np.full((1, K), c), None, eps)
    assert np.allclose(out, c / math.sqrt(c * c + eps), rtol=1e-15)
    x = np.random.default_rng(3).standard_normal((2, K))
    g = np.random.default_rng(4).uniform(0.5, 1.5, K)
    assert np.allclose(oracle.rmsnorm(x, g, 1e-5), brute.rmsnorm(x, g, 1e-5), rtol=1e-14)
    assert np.array_equal(oracle.rmsnorm(np.zeros((1, K)), g, eps), np.zeros((1, K)))
    # scale invariance when eps = 0
    assert np.allclose(oracle.rmsnorm(5 * x, g, 0.0), oracle.rmsnorm(x, g, 0.0), rtol=1e-14)


@pytest.mark.parametrize("fmt", ["M", "L"])
def test_mirai_gemv_with_rotation_prologue_matches_bruteforce(fmt):
    N, K, T = 7, 704, 2
    w = synth.mirai_weights(fmt, N, K, cfg=133, set_id=0)
    xb = synth.x_bf16(T, K, cfg=133, set_id=0)
    sg = synth.rht_signs(K, cfg=133, set_id=0)
    gb = synth.rmsnorm_gamma(K, cfg=133, set_id=0, dtype="bf16")
    y, a, xr = oracle.mirai_gemv_rht(w, xb, "bf16", sg, gb, 1e-5)
    xn = brute.rmsnorm(brute.bf16(xb), brute.bf16(gb), 1e-5)
    R = brute.rotation(K, sg)
    d = brute.mirai_dense(w)
    assert np.allclose(xr, xn @ R.T, rtol=0, atol=1e-13)
    yb = (xn @ R.T) @ d.T
    assert np.all(np.abs(y - yb) <= 1e-12 * a)
    # without the norm, only the rotation
    y2, _, _ = oracle.mirai_gemv_rht(w, xb, "bf16", sg, None)
    assert np.allclose(y2, (brute.bf16(xb) @ R.T) @ d.T, rtol=1e-12, atol=1e-12)


def test_rht_generators():
    sg = synth.rht_signs(1024, cfg=3, set_id=0)
    assert sg.shape == (32,) and sg.dtype == np.uint32
    bits = np.unpackbits(sg.view(np.uint8))
    assert 0.4 < bits.mean() < 0.6
    g = brute.f16(synth.rmsnorm_gamma(1024, cfg=3, set_id=0))
    assert g.min() >= 0.5 and g.max() <= 1.5


# ---------------------------------------------------------------- decode attention
# jeff.news/article/5193 (TurboFieldfare), internals section: circular KV for
# sliding-window layers, linear KV for full attention, exact decode attention.

def _attn_case(Hq, Hkv, D, cap, seed, scale_q=1.0):
    t = synth.attn_inputs(Hq, Hkv, D, cap, cfg=140, set_id=seed, scale_q=scale_q)
    return {k: brute.f16(v) for k, v in t.items()}


@pytest.mark.parametrize("Hq,Hkv,D,cap,window,pos", [
    (4, 2, 64, 40, 0, 0), (4, 2, 64, 40, 0, 17), (4, 2, 64, 40, 0, 39),
    (6, 3, 32, 16, 16, 5), (6, 3, 32, 16, 16, 15), (6, 3, 32, 16, 16, 16), (6, 3, 32, 16, 16, 37),
    (2, 2, 128, 8, 0, 7), (8, 1, 64, 24, 24, 100)])
def test_attn_matches_bruteforce(Hq, Hkv, D, cap, window, pos):
    t = _attn_case(Hq, Hkv, D, cap, seed=Hq * 100 + pos)
    sc = 1.0 / math.sqrt(D)
    out, a = oracle.attn_decode(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], window, pos, sc)
    ob = brute.attn_decode(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], window, pos, sc)
    assert np.allclose(out, ob, rtol=0, atol=1e-13)
    assert np.all(a >= np.abs(out) - 1e-15)


def test_attn_first_token_returns_its_value():
    t = _attn_case(4, 2, 64, 10, seed=1)
    out, _ = oracle.attn_decode(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], 0, 0, 0.125)
    assert np.array_equal(out, np.repeat(t["v_new"], 2, axis=0))


def test_attn_equal_keys_give_the_mean_value():
    Hq, Hkv, D, cap, pos = 4, 2, 32, 12, 9
    t = _attn_case(Hq, Hkv, D, cap, seed=2)
    kc = np.repeat(t["k_new"][:, None, :], cap, axis=1)
    out, _ = oracle.attn_decode(t["q"], t["k_new"], t["v_new"], kc, t["v_cache"], 0, pos, 0.2)
    vals = t["v_cache"].copy()
    vals[:, pos] = t["v_new"]
    expect = np.repeat(vals[:, :pos + 1].mean(axis=1), 2, axis=0)
    assert np.allclose(out, expect, rtol=0, atol=1e-14)


def test_attn_circular_equals_linear_over_the_window():
    # a window of W: the circular store after position pos holds positions
    # pos-W+1 .. pos at slots p mod W; laid out in order they form a linear
    # store, and attention over either gives the same result
    Hq, Hkv, D, W, pos = 4, 2, 32, 8, 21
    t = _attn_case(Hq, Hkv, D, W, seed=3)
    circ, _ = oracle.attn_decode(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], W, pos, 0.3)
    kc, vc = t["k_cache"].copy(), t["v_cache"].copy()
    kc[:, pos % W], vc[:, pos % W] = t["k_new"], t["v_new"]
    order = [p % W for p in range(pos - W + 1, pos + 1)]
    kl, vl = kc[:, order], vc[:, order]          # positions in order; the last is the new token
    lin, _ = oracle.attn_decode(t["q"], kl[:, -1], vl[:, -1], kl, vl, 0, W - 1, 0.3)
    assert np.allclose(circ, lin, rtol=0, atol=1e-14)


def test_attn_overwritten_position_has_no_effect():
    Hq, Hkv, D, W, pos = 2, 1, 16, 6, 14       # slot 2 held position 8, now position 14
    t = _attn_case(Hq, Hkv, D, W, seed=4)
    o1, _ = oracle.attn_decode(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], W, pos, 0.25)
    kc, vc = t["k_cache"].copy(), t["v_cache"].copy()
    kc[:, pos % W] += 100.0
    vc[:, pos % W] -= 50.0
    o2, _ = oracle.attn_decode(t["q"], t["k_new"], t["v_new"], kc, vc, W, pos, 0.25)
    assert np.array_equal(o1, o2)
    # and a slot still inside the window does matter
    kc2 = t["k_cache"].copy()
    kc2[:, (pos + 1) % W] += 3.0
    o3, _ = oracle.attn_decode(t["q"], t["k_new"], t["v_new"], kc2, t["v_cache"], W, pos, 0.25)
    assert not np.array_equal(o1, o3)


def test_attn_large_scores_are_stable():
    t = _attn_case(2, 1, 64, 20, seed=5, scale_q=400.0)
    out, _ = oracle.attn_decode(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], 0, 19, 1.0)
    ob = brute.attn_decode(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], 0, 19, 1.0)
    assert np.all(np.isfinite(out)) and np.allclose(out, ob, rtol=0, atol=1e-12)


def test_attn_slot_rule():
    assert [oracle.attn_slot(p, 4) for p in range(9)] == [0, 1, 2, 3, 0, 1, 2, 3, 0]
    assert [oracle.attn_slot(p, 0) for p in (0, 5, 4095)] == [0, 5, 4095]


# ------------------------------------------------ int8 activations (verify)
# uzu page on discuss.pytorch.kr, section on speculative decoding: the
# verification GEMM runs on an int8 matrix path with the activations
# quantized to 8 bits on the fly. Reading: per token, symmetric,
# scale = max|x| / 127, codes rounded half to even, in fp32.

def _grid_rows(M, K, seed):
    """fp16 activations on the grid k * 2^-4 (|k| <= 127, each row holding
    +-127), where scale = 2^-4 exactly and quantization changes nothing."""
    rng = np.random.default_rng(seed)
    k = rng.integers(-127, 128, size=(M, K))
    k[:, rng.integers(0, K, size=M)] = 0
    for m in range(M):
        k[m, rng.integers(0, K)] = 127 if m % 2 else -127
    return (k.astype(np.float64) * 2.0 ** -4).astype(np.float16).view(np.uint16)


def test_int8_activations_on_the_exact_grid_reduce_to_the_gemm():
    w = synth.affine_weights(4, 37, 704, cfg=901, set_id=0)
    xb = _grid_rows(5, 704, 1)
    q, sc = oracle.quant_i8(xb)
    assert np.all(sc == np.float32(2.0 ** -4))
    assert np.array_equal(q.astype(np.float64) * 2.0 ** -4, xb.view(np.float16).astype(np.float64))
    y8, a8 = oracle.verify_i8(w, xb)
    y, a = oracle.gemv_f16(w, xb)
    assert np.array_equal(y8, y) and np.array_equal(a8, a)


def test_int8_activation_ties_go_to_even():
    # max |x| = 127 gives scale 1 exactly, so x / scale = x and the halves
    # are exact ties; Python's round() rounds ties to even
    vals = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, -1.5, 126.5, -126.5, 0.0]
    xb = np.array([vals], np.float16).view(np.uint16)
    q, sc = oracle.quant_i8(xb)
    assert sc[0] == np.float32(1.0)
    assert q[0].tolist() == [round(v) for v in vals]


def test_int8_activation_bounds_and_extremes():
    for scale in (1e-4, 1.0, 300.0):
        x = (synth.x_f16(6, 1024, cfg=902, set_id=int(scale * 7)).view(np.float16).astype(np.float32)
             * np.float32(scale)).astype(np.float16)
        q, sc = oracle.quant_i8(x.view(np.uint16))
        xf = x.astype(np.float64)
        xh = sc.astype(np.float64)[:, None] * q
        assert np.all(np.abs(q.astype(np.int32)) <= 127)
        assert np.all(np.max(np.abs(q.astype(np.int32)), axis=1) == 127)
        # round to nearest: within half a step (plus the fp32 quotient's rounding)
        assert np.all(np.abs(xh - xf) <= sc.astype(np.float64)[:, None] * (0.5 + 1e-6))


def test_int8_activation_zero_row_and_row_independence():
    w = synth.affine_weights(4, 20, 256, cfg=903, set_id=0)
    xb = synth.x_f16(3, 256, cfg=903, set_id=1).copy()
    q1, s1 = oracle.quant_i8(xb)
    xb2 = xb.copy()
    xb2[1] = 0
    q2, s2 = oracle.quant_i8(xb2)
    assert s2[1] == 0 and np.all(q2[1] == 0)
    assert np.array_equal(q1[[0, 2]], q2[[0, 2]]) and np.array_equal(s1[[0, 2]], s2[[0, 2]])
    y, _ = oracle.verify_i8(w, xb2)
    assert np.all(y[1] == 0.0)


def test_int8_activations_match_the_second_route():
    w = synth.affine_weights(4, 33, 2112, cfg=904, set_id=0)
    xb = synth.x_f16(17, 2112, cfg=904, set_id=1)
    q, sc = oracle.quant_i8(xb)
    qb, sb = brute.quant_i8(xb)
    assert np.array_equal(q, qb) and np.array_equal(sc, sb)
    y, _ = oracle.verify_i8(w, xb)
    xh = sb.astype(np.float64)[:, None] * qb.astype(np.float64)
    yb = xh @ brute.dense(w).T
    assert np.allclose(y, yb, rtol=1e-12, atol=1e-12)
