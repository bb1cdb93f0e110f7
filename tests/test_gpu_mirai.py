"""GPU parity of qgemv_mirai_m / qgemv_mirai_l against the fp64 oracle.

Formats (uzu page on discuss.pytorch.kr, section on model conversion and
the Mirai quantization formats): Mirai-M = 4-bit codes, bf16 scale and
4-bit zero point per group of 64, w = s*(q - z); Mirai-L = signed 8-bit
codes, bf16 scale per group of 64, w = s*q.

Bar: |y_gpu - y_ref| <= 1e-4 * sum_k |w_k x_k| + 1e-6 per output; bit-exact
where the exact answer is representable in fp32 (one-hot and zero
activations).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within, dev_bf16, dev_codes, dev_half

qd = pytest.importorskip("affine_quantized_gemv_qgemv_amd")

pytestmark = pytest.mark.gpu


def dev_mirai(w):
    z = None if w.zeros is None else dev_codes(w.zeros)
    return dev_codes(w.wq), dev_bf16(w.scales), z


def run(w, xb, xdt="f16", out=None):
    wq, s, z = dev_mirai(w)
    x = dev_half(xb) if xdt == "f16" else dev_bf16(xb)
    if w.fmt == "M":
        y = qd.qgemv_mirai_m(wq, s, z, x, out=out)
    else:
        y = qd.qgemv_mirai_l(wq, s, x, out=out)
    torch.cuda.synchronize()
    return y


def draw_x(T, K, xdt, seed):
    return synth.x_f16(T, K, cfg=220, set_id=seed) if xdt == "f16" else synth.x_bf16(T, K, cfg=220, set_id=seed)


SMALL = [(1, 64), (3, 128), (17, 704), (5, 2112), (129, 2816), (33, 4096), (70, 8192), (9, 14336)]


@pytest.mark.parametrize("fmt", ["M", "L"])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("N,K", SMALL)
def test_small_shapes(fmt, xdt, N, K):
    for batch in (1, 3, 8):
        seed = N * 7 + K + batch
        w = synth.mirai_weights(fmt, N, K, cfg=220, set_id=seed)
        xb = draw_x(batch, K, xdt, seed)
        print(f"mirai-{fmt} {xdt} N={N} K={K} batch={batch}", flush=True)
        y = run(w, xb, xdt).cpu().numpy()
        yr, a = oracle.mirai_gemv_x(w, xb, xdt)
        assert_within(y, yr, a, f"mirai-{fmt} {xdt} N={N} K={K} batch={batch}")


@pytest.mark.parametrize("fmt", ["M", "L"])
@pytest.mark.parametrize("batch", [1, 2, 4, 5, 6, 7, 8])
def test_every_batch_size(fmt, batch):
    w = synth.mirai_weights(fmt, 100, 1024, cfg=221, set_id=batch)
    xb = draw_x(batch, 1024, "f16", batch)
    y = run(w, xb).cpu().numpy()
    yr, a = oracle.mirai_gemv_x(w, xb)
    assert_within(y, yr, a, f"mirai-{fmt} batch={batch}")


@pytest.mark.parametrize("fmt", ["M", "L"])
def test_one_hot_is_bit_exact(fmt):
    N, K = 64, 2048
    w = synth.mirai_weights(fmt, N, K, cfg=222, set_id=0)
    one = np.float16(1.0).view(np.uint16)
    for k in (0, 1, 7, 31, 32, 63, 64, 100, 1000, 2047):
        xb = np.zeros((1, K), np.uint16)
        xb[0, k] = one
        y = run(w, xb).cpu().numpy().astype(np.float64)
        yr, _ = oracle.mirai_gemv_x(w, xb)
        assert np.array_equal(y, yr), f"mirai-{fmt} k={k}"


@pytest.mark.parametrize("fmt", ["M", "L"])
def test_zero_activation_gives_zero(fmt):
    w = synth.mirai_weights(fmt, 40, 1024, cfg=223, set_id=0)
    y = run(w, np.zeros((3, 1024), np.uint16)).cpu().numpy()
    assert np.all(y == 0.0)


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_mirai_m_extreme_codes_and_zero_points(xdt):
    # code == zero point makes every weight exactly zero (w = s (q - z)), so
    # the bar reduces to |y| <= 1e-6
    K = 1088   # 17 groups: the second zero-point word has 7 padding nibbles
    for code, zero in ((15, 0), (0, 15), (15, 15), (0, 0), (7, 8), (8, 8), (3, 3)):
        w = synth.mirai_weights("M", 50, K, cfg=224, set_id=code * 16 + zero, codes="const",
                                const_code=code, zeros="const", const_zero=zero)
        for batch in (1, 8):
            xb = draw_x(batch, K, xdt, code + batch)
            y = run(w, xb, xdt).cpu().numpy()
            yr, a = oracle.mirai_gemv_x(w, xb, xdt)
            assert_within(y, yr, a, f"code {code} zero {zero} batch {batch} {xdt}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_mirai_near_zero_weights(xdt):
    # Mirai-M: codes at and next to the zero point (w = 0 or +-s); Mirai-L:
    # signed codes -1, 0, 1; every K from one group to 4096, batch 1 and 8
    for K in (64, 128, 704, 4096):
        for z in (0, 8, 15):
            cs = [v for v in (z - 1, z, z + 1) if 0 <= v <= 15]
            for only_z in (True, False):
                w = synth.mirai_weights("M", 130, K, cfg=229, set_id=K + z, codes="set",
                                        code_set=[z] if only_z else cs, zeros="const", const_zero=z)
                for batch in (1, 8):
                    xb = draw_x(batch, K, xdt, K + z + batch)
                    y = run(w, xb, xdt).cpu().numpy()
                    yr, a = oracle.mirai_gemv_x(w, xb, xdt)
                    assert_within(y, yr, a, f"mirai-M K={K} z={z} codes {cs if not only_z else [z]} b={batch} {xdt}")
        w = synth.mirai_weights("L", 130, K, cfg=229, set_id=K, codes="set", code_set=(-1, 0, 1))
        for batch in (1, 8):
            xb = draw_x(batch, K, xdt, K + batch)
            y = run(w, xb, xdt).cpu().numpy()
            yr, a = oracle.mirai_gemv_x(w, xb, xdt)
            assert_within(y, yr, a, f"mirai-L K={K} codes -1..1 b={batch} {xdt}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_mirai_l_extreme_codes(xdt):
    K = 1024
    for c in (-128, -1, 0, 1, 127):
        w = synth.mirai_weights("L", 70, K, cfg=225, set_id=c + 128, codes="const", const_code=c)
        xb = draw_x(3, K, xdt, c + 128)
        y = run(w, xb, xdt).cpu().numpy()
        yr, a = oracle.mirai_gemv_x(w, xb, xdt)
        assert_within(y, yr, a, f"const {c} {xdt}")


def test_mirai_l_matches_affine8_kernel_bit_for_bit():
    # w = s*q = s*(q XOR 0x80) - 128 s: the affine 8-bit entry point on the
    # flipped codes with b = -128 s (exact in fp16) must give identical bits
    N, K, batch = 300, 2816, 4
    w = synth.mirai_weights("L", N, K, cfg=226, set_id=0)
    xb = draw_x(batch, K, "f16", 0)
    y = run(w, xb).cpu()
    s = oracle.bf16_to_f64(w.scales)
    s16 = s.astype(np.float16)
    b16 = (-128.0 * s).astype(np.float16)
    assert np.array_equal(s16.astype(np.float64), s)
    x = dev_half(xb)
    ya = qd.qgemv_affine8(dev_codes(w.wq ^ np.uint32(0x80808080)), dev_half(s16.view(np.uint16)),
                          dev_half(b16.view(np.uint16)), x)
    torch.cuda.synchronize()
    assert torch.equal(y, ya.cpu())


def test_deterministic_and_no_out_of_bounds_writes():
    for fmt in ("M", "L"):
        N, K, batch = 1000, 4096, 3
        w = synth.mirai_weights(fmt, N, K, cfg=227, set_id=0)
        xb = synth.x_f16(batch, K, cfg=227, set_id=0)
        guard = 4096
        buf = torch.full((guard + batch * N + guard,), float("nan"), device="cuda")
        out = buf[guard:guard + batch * N].view(batch, N)
        y1 = run(w, xb, out=out).clone()
        y2 = run(w, xb).clone()
        assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + batch * N:]).all()
        assert torch.equal(y1, y2)


# --------------------------------------------------------------- full sizes

FULL = [
    ("c2 gate+up 4096->28672", 4096, 28672, 1, 512),
    ("c2 down 14336->4096", 14336, 4096, 1, 256),
    ("c1 4096->4096", 4096, 4096, 1, None),
    ("c5 8192->28672 b8", 8192, 28672, 8, 256),
    ("c5 28672->8192 b2", 28672, 8192, 2, 256),
]


@pytest.mark.parametrize("fmt", ["M", "L"])
@pytest.mark.parametrize("name,K,N,batch,nsample", FULL, ids=[f[0] for f in FULL])
def test_full_size(fmt, name, K, N, batch, nsample):
    print(f"mirai-{fmt} {name}", flush=True)
    w = synth.mirai_weights(fmt, N, K, cfg=228, set_id=0)
    xb = synth.x_f16(batch, K, cfg=228, set_id=0)
    y = run(w, xb).cpu().numpy()
    if nsample is None:
        yr, a = oracle.mirai_gemv_x(w, xb)
        assert_within(y, yr, a, name)
    else:
        r = np.random.default_rng(N + K + batch)
        rows = np.unique(np.concatenate([r.choice(N, nsample, replace=False), [0, N - 1]]))
        yr, a = oracle.mirai_gemv_x(w, xb, rows=rows)
        assert_within(y[:, rows], yr, a, name)
