"""GPU parity of qgemv_mirai_m_rht / qgemv_mirai_l_rht (RMSNorm + block-32
random Hadamard rotation fused ahead of the Mirai GEMV) against the oracle.

Source: uzu page on discuss.pytorch.kr, section on model conversion and the
Mirai quantization formats (both formats rotate with a block-32 random
Hadamard transform; the transform is fused with RMSNorm and the matmul).

Bar: |y_gpu - y_ref| <= 1e-4 * sum_k |w'_k x'_k| + 1e-6 per output, x' the
oracle's fp64 rotated activations.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within, dev_bf16, dev_codes, dev_half

qd = pytest.importorskip("affine_quantized_gemv_qgemv_amd")

pytestmark = pytest.mark.gpu


def run(w, xb, xdt, signs, gamma_bits, eps=1e-6, out=None):
    dx = dev_half if xdt == "f16" else dev_bf16
    wq, s = dev_codes(w.wq), dev_bf16(w.scales)
    sg = None if signs is None else dev_codes(signs)
    g = None if gamma_bits is None else dx(gamma_bits)
    x = dx(xb)
    if w.fmt == "M":
        y = qd.qgemv_mirai_m_rht(wq, s, dev_codes(w.zeros), x, sg, g, eps, out=out)
    else:
        y = qd.qgemv_mirai_l_rht(wq, s, x, sg, g, eps, out=out)
    torch.cuda.synchronize()
    return y


def draw_x(T, K, xdt, seed, scale=1.0):
    v = np.random.default_rng(seed).standard_normal((T, K)) * scale
    if xdt == "f16":
        return v.astype(np.float16).view(np.uint16)
    return synth.f32_to_bf16_bits(v.astype(np.float32))


def check(w, xb, xdt, signs, gb, eps=1e-6, what=""):
    y = run(w, xb, xdt, signs, gb, eps).cpu().numpy()
    yr, a, _ = oracle.mirai_gemv_rht(w, xb, xdt, signs, gb, eps)
    return assert_within(y, yr, a, what)


SMALL = [(1, 64), (3, 128), (17, 704), (5, 2112), (129, 2816), (33, 4096), (9, 14336)]


@pytest.mark.parametrize("fmt", ["M", "L"])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("N,K", SMALL)
def test_small_shapes(fmt, xdt, N, K):
    for batch, norm in ((1, True), (3, False), (8, True)):
        seed = N * 7 + K + batch
        w = synth.mirai_weights(fmt, N, K, cfg=230, set_id=seed)
        xb = draw_x(batch, K, xdt, seed)
        sg = synth.rht_signs(K, cfg=230, set_id=seed)
        gb = synth.rmsnorm_gamma(K, cfg=230, set_id=seed, dtype=xdt) if norm else None
        print(f"rht mirai-{fmt} {xdt} N={N} K={K} batch={batch} norm={norm}", flush=True)
        check(w, xb, xdt, sg, gb, 1e-5, f"mirai-{fmt} {xdt} N={N} K={K} b={batch} norm={norm}")


@pytest.mark.parametrize("fmt", ["M", "L"])
def test_every_batch_size_and_no_signs(fmt):
    K = 1024
    w = synth.mirai_weights(fmt, 100, K, cfg=231, set_id=0)
    gb = synth.rmsnorm_gamma(K, cfg=231, set_id=0)
    for batch in range(1, 9):
        xb = draw_x(batch, K, "f16", batch)
        check(w, xb, "f16", None, gb, 1e-6, f"mirai-{fmt} batch={batch} no signs")
    # absent signs and all-zero sign words are the same rotation, bit for bit
    xb = draw_x(2, K, "f16", 99)
    y0 = run(w, xb, "f16", None, gb).cpu()
    y1 = run(w, xb, "f16", np.zeros(K // 32, np.uint32), gb).cpu()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("fmt", ["M", "L"])
@pytest.mark.parametrize("xdt,scale,norm", [("bf16", 2.0 ** 40, False), ("bf16", 2.0 ** -40, False),
                                            ("bf16", 2.0 ** 30, True), ("f16", 2.0 ** 12, False),
                                            ("f16", 2.0 ** -10, True)])
def test_activation_range_is_covered_by_the_prescale(fmt, xdt, scale, norm):
    # values far outside fp16's range (bf16 inputs, no norm) must not overflow
    # or lose precision in the two fp16 planes
    K = 2816
    w = synth.mirai_weights(fmt, 64, K, cfg=232, set_id=0)
    xb = draw_x(2, K, xdt, 5, scale)
    sg = synth.rht_signs(K, cfg=232, set_id=0)
    gb = synth.rmsnorm_gamma(K, cfg=232, set_id=0, dtype=xdt) if norm else None
    check(w, xb, xdt, sg, gb, 0.0 if norm else 1e-6, f"scale {scale} norm {norm}")


@pytest.mark.parametrize("fmt", ["M", "L"])
def test_norm_is_invariant_to_power_of_two_scaling(fmt):
    # with eps = 0, RMSNorm(2^j x) = RMSNorm(x) exactly, and so is every fp32
    # step of the prologue: the outputs agree bit for bit
    K = 4096
    w = synth.mirai_weights(fmt, 300, K, cfg=233, set_id=0)
    sg = synth.rht_signs(K, cfg=233, set_id=0)
    gb = synth.rmsnorm_gamma(K, cfg=233, set_id=0, dtype="bf16")
    xb = draw_x(3, K, "bf16", 7)
    y0 = run(w, xb, "bf16", sg, gb, 0.0).cpu()
    for j in (-20, -3, 5, 30):
        xs = synth.f32_to_bf16_bits(oracle.bf16_to_f64(xb).astype(np.float32) * np.float32(2.0 ** j))
        assert torch.equal(run(w, xs, "bf16", sg, gb, 0.0).cpu(), y0), f"2^{j}"


def test_zero_activation_gives_zero():
    K = 1024
    for fmt in ("M", "L"):
        w = synth.mirai_weights(fmt, 40, K, cfg=234, set_id=0)
        gb = synth.rmsnorm_gamma(K, cfg=234, set_id=0)
        sg = synth.rht_signs(K, cfg=234, set_id=0)
        for g in (gb, None):
            y = run(w, np.zeros((2, K), np.uint16), "f16", sg, g, 1e-6).cpu().numpy()
            assert np.all(y == 0.0)


@pytest.mark.parametrize("fmt", ["M", "L"])
def test_split_k_path(fmt):
    # 8 vectors of K = 14336 do not fit one workgroup's LDS as two fp16
    # planes: the chunk range is split across workgroups and summed atomically
    K, N, batch = 14336, 200, 8
    w = synth.mirai_weights(fmt, N, K, cfg=235, set_id=0)
    xb = draw_x(batch, K, "bf16", 11, 3.0)
    sg = synth.rht_signs(K, cfg=235, set_id=0)
    gb = synth.rmsnorm_gamma(K, cfg=235, set_id=0, dtype="bf16")
    check(w, xb, "bf16", sg, gb, 1e-6, f"split-K mirai-{fmt}")


def test_deterministic_and_no_out_of_bounds_writes():
    for fmt in ("M", "L"):
        N, K, batch = 1000, 4096, 3
        w = synth.mirai_weights(fmt, N, K, cfg=236, set_id=0)
        xb = draw_x(batch, K, "f16", 1)
        sg = synth.rht_signs(K, cfg=236, set_id=0)
        gb = synth.rmsnorm_gamma(K, cfg=236, set_id=0)
        guard = 4096
        buf = torch.full((guard + batch * N + guard,), float("nan"), device="cuda")
        out = buf[guard:guard + batch * N].view(batch, N)
        y1 = run(w, xb, "f16", sg, gb, 1e-6, out=out).clone()
        y2 = run(w, xb, "f16", sg, gb, 1e-6).clone()
        assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + batch * N:]).all()
        assert torch.equal(y1, y2)


FULL = [
    ("c2 gate+up 4096->28672", 4096, 28672, 1, 512),
    ("c2 down 14336->4096", 14336, 4096, 1, 256),
    ("c5 8192->28672 b4", 8192, 28672, 4, 256),
]


@pytest.mark.parametrize("fmt", ["M", "L"])
@pytest.mark.parametrize("name,K,N,batch,nsample", FULL, ids=[f[0] for f in FULL])
def test_full_size(fmt, name, K, N, batch, nsample):
    print(f"rht mirai-{fmt} {name}", flush=True)
    w = synth.mirai_weights(fmt, N, K, cfg=237, set_id=0)
    xb = synth.x_f16(batch, K, cfg=237, set_id=0)
    sg = synth.rht_signs(K, cfg=237, set_id=0)
    gb = synth.rmsnorm_gamma(K, cfg=237, set_id=0)
    y = run(w, xb, "f16", sg, gb, 1e-6).cpu().numpy()
    r = np.random.default_rng(N + K + batch)
    rows = np.unique(np.concatenate([r.choice(N, nsample, replace=False), [0, N - 1]]))
    yr, a, _ = oracle.mirai_gemv_rht(w, xb, "f16", sg, gb, 1e-6, rows=rows)
    assert_within(y[:, rows], yr, a, name)
