"""GPU parity of qgemv_affine4 / qgemv_affine8 against the fp64 oracle.

Bar: |y_gpu - y_ref| <= 1e-4 * sum_k |w_k x_k| + 1e-6 per output, and
bit-exact results for the special inputs whose exact answer is
representable in fp32 (one-hot activations, zero activations,
power-of-two scaling).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within, dev_bf16, dev_half, dev_weights

qd = pytest.importorskip("affine_quantized_gemv_qgemv_amd")

pytestmark = pytest.mark.gpu


def run_gemv(bits, w, xb, xdt="f16", out=None):
    wq, s, b = dev_weights(w)
    x = dev_half(xb) if xdt == "f16" else dev_bf16(xb)
    fn = qd.qgemv_affine4 if bits == 4 else qd.qgemv_affine8
    y = fn(wq, s, b, x, out=out)
    torch.cuda.synchronize()
    return y


def ref_gemv(w, xb, xdt="f16", rows=None):
    return oracle.gemv_f16(w, xb, rows) if xdt == "f16" else oracle.gemm_chunk(w, xb, rows)


def draw_x(T, K, xdt, seed):
    return synth.x_f16(T, K, cfg=200, set_id=seed) if xdt == "f16" else synth.x_bf16(T, K, cfg=200, set_id=seed)


SMALL = [(1, 64), (3, 128), (17, 704), (5, 2112), (129, 2816), (33, 4096), (70, 8192), (9, 14336)]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("N,K", SMALL)
def test_small_shapes(bits, xdt, N, K):
    for batch in (1, 3, 8):
        seed = N * 7 + K + batch
        w = synth.affine_weights(bits, N, K, cfg=200, set_id=seed)
        xb = draw_x(batch, K, xdt, seed)
        y = run_gemv(bits, w, xb, xdt).cpu().numpy()
        yr, a = ref_gemv(w, xb, xdt)
        print(f"bits={bits} xdt={xdt} N={N} K={K} batch={batch}", flush=True)
        assert_within(y, yr, a, f"bits={bits} {xdt} N={N} K={K} batch={batch}")


@pytest.mark.parametrize("batch", [1, 2, 4, 5, 6, 7, 8])
def test_every_batch_size(batch):
    w = synth.affine_weights(4, 100, 1024, cfg=201, set_id=batch)
    xb = draw_x(batch, 1024, "f16", batch)
    y = run_gemv(4, w, xb).cpu().numpy()
    yr, a = ref_gemv(w, xb)
    assert_within(y, yr, a, f"batch={batch}")


def test_router_prefill_batch_128():
    w = synth.affine_weights(8, 128, 2816, cfg=202, set_id=0)
    for xdt in ("f16", "bf16"):
        xb = draw_x(128, 2816, xdt, 1)
        y = run_gemv(8, w, xb, xdt).cpu().numpy()
        yr, a = ref_gemv(w, xb, xdt)
        assert_within(y, yr, a, f"router T=128 {xdt}")


# 8-bit weights over more than 8 tokens take the matrix-core path: ragged
# token / output tiles (32 x 32) and group counts that leave some of the
# 8 K-waves with fewer groups or none.
@pytest.mark.parametrize("T", [9, 16, 33, 100])
@pytest.mark.parametrize("N,K", [(1, 64), (37, 704), (128, 2112), (200, 4096)])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_int8_token_chunk(T, N, K, xdt):
    w = synth.affine_weights(8, N, K, cfg=210, set_id=T * 7 + N)
    xb = draw_x(T, K, xdt, T * 13 + N)
    y = run_gemv(8, w, xb, xdt).cpu().numpy()
    yr, a = ref_gemv(w, xb, xdt)
    print(f"int8 chunk T={T} N={N} K={K} {xdt}", flush=True)
    assert_within(y, yr, a, f"int8 chunk T={T} N={N} K={K} {xdt}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_int8_token_chunk_extreme_codes(xdt):
    K, T = 1024, 24
    for kind, c in (("zero", 0), ("const", 15), ("const", 16), ("const", 255)):
        w = synth.affine_weights(8, 70, K, cfg=211, set_id=c, codes=kind, const_code=c)
        xb = draw_x(T, K, xdt, c)
        y = run_gemv(8, w, xb, xdt).cpu().numpy()
        yr, a = ref_gemv(w, xb, xdt)
        assert_within(y, yr, a, f"{kind} {c} {xdt}")


def test_int8_token_chunk_deterministic_and_in_bounds():
    N, K, T = 130, 2816, 45
    w = synth.affine_weights(8, N, K, cfg=212, set_id=0)
    xb = draw_x(T, K, "bf16", 3)
    guard = 4096
    buf = torch.full((guard + T * N + guard,), float("nan"), device="cuda")
    out = buf[guard:guard + T * N].view(T, N)
    y1 = run_gemv(8, w, xb, "bf16", out=out).clone()
    y2 = run_gemv(8, w, xb, "bf16").clone()
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + T * N:]).all()
    assert torch.equal(y1, y2)
    yr, a = ref_gemv(w, xb, "bf16")
    assert_within(y1.cpu().numpy(), yr, a, "int8 chunk")


@pytest.mark.parametrize("N", [16385, 16387, 16390])
def test_ragged_last_tile_of_two_row_tiles(N):
    # N >= 16384 with whole groups per lane takes two-row tiles: the last tile
    # holds one valid row (or two of four) and its other rows are clamped
    K = 4096
    w = synth.affine_weights(4, N, K, cfg=210, set_id=N)
    xb = draw_x(1, K, "f16", N)
    print(f"N={N} K={K}", flush=True)
    y = run_gemv(4, w, xb).cpu().numpy()
    r = np.random.default_rng(N)
    rows = np.unique(np.concatenate([r.choice(N, 256, replace=False), np.arange(N - 8, N), [0]]))
    yr, a = ref_gemv(w, xb, rows=rows)
    assert_within(y[:, rows], yr, a, f"N={N}")


@pytest.mark.parametrize("bits", [4, 8])
def test_largest_k(bits):
    # K = 2^22, the largest the ABI accepts: rows are addressed with 32-bit
    # offsets from a tile's first row, and x is streamed through LDS in
    # about a hundred K slices
    K, N = 1 << 22, 3
    w = synth.affine_weights(bits, N, K, cfg=209, set_id=bits)
    for batch in (1, 2):
        xb = draw_x(batch, K, "f16", 40 + batch)
        print(f"bits={bits} N={N} K={K} batch={batch}", flush=True)
        y = run_gemv(bits, w, xb).cpu().numpy()
        yr, a = ref_gemv(w, xb)
        assert_within(y, yr, a, f"bits={bits} K=2^22 batch={batch}")


@pytest.mark.parametrize("bits", [4, 8])
def test_one_hot_is_bit_exact(bits):
    N, K = 64, 2048
    w = synth.affine_weights(bits, N, K, cfg=203, set_id=bits)
    one = np.float16(1.0).view(np.uint16)
    for k in (0, 1, 7, 31, 32, 63, 64, 100, 1000, 2047):
        xb = np.zeros((1, K), np.uint16)
        xb[0, k] = one
        y = run_gemv(bits, w, xb).cpu().numpy().astype(np.float64)
        yr, _ = ref_gemv(w, xb)
        assert np.array_equal(y, yr), f"k={k}"
    # several one-hot vectors in one launch (batch 3..8 of 4-bit codes runs
    # on the matrix core): each result is s q + b, exact in fp32
    ks = (0, 9, 63, 64, 127, 128, 1000, 2047)
    for batch in (3, 8):
        xb = np.zeros((batch, K), np.uint16)
        for i in range(batch):
            xb[i, ks[i]] = one
        y = run_gemv(bits, w, xb).cpu().numpy().astype(np.float64)
        yr, _ = ref_gemv(w, xb)
        assert np.array_equal(y, yr), f"batch={batch}"


def test_zero_activation_gives_zero():
    w = synth.affine_weights(4, 40, 1024, cfg=204, set_id=0)
    y = run_gemv(4, w, np.zeros((3, 1024), np.uint16)).cpu().numpy()
    assert np.all(y == 0.0)


def test_power_of_two_scaling_is_exact():
    N, K = 300, 4096
    w = synth.affine_weights(4, N, K, cfg=205, set_id=0)
    xb = synth.x_f16(2, K, cfg=205, set_id=0)
    x = xb.view(np.float16)
    y1 = run_gemv(4, w, xb).cpu().numpy()
    for j in (1, 3):
        xs = (x.astype(np.float32) * 2.0 ** j).astype(np.float16).view(np.uint16)
        yj = run_gemv(4, w, xs).cpu().numpy()
        assert np.array_equal(yj, y1 * np.float32(2.0 ** j)), f"2^{j}"
    # the matrix-core path (batch 3..8)
    xb = synth.x_f16(6, K, cfg=205, set_id=1)
    x = xb.view(np.float16)
    y1 = run_gemv(4, w, xb).cpu().numpy()
    for j in (1, 3):
        xs = (x.astype(np.float32) * 2.0 ** j).astype(np.float16).view(np.uint16)
        yj = run_gemv(4, w, xs).cpu().numpy()
        assert np.array_equal(yj, y1 * np.float32(2.0 ** j)), f"batch 6, 2^{j}"


@pytest.mark.parametrize("bits", [4, 8])
def test_constant_and_zero_codes(bits):
    K = 1024
    for kind, c in (("zero", 0), ("const", 5), ("const", (1 << bits) - 1)):
        w = synth.affine_weights(bits, 50, K, cfg=206, set_id=c, codes=kind, const_code=c)
        for batch in (2, 5):
            xb = synth.x_f16(batch, K, cfg=206, set_id=c + batch)
            y = run_gemv(bits, w, xb).cpu().numpy()
            yr, a = ref_gemv(w, xb)
            assert_within(y, yr, a, f"{kind} {c} batch={batch}")


# Weights at and near zero (TurboFieldfare article, section "성능과 제약":
# w = s*q + b; with b close to -c*s a code q = c gives a weight close to
# zero, where real weights cluster). The bar is the same relative bar, so
# the kernel's rounding must follow |w x|, not s*q or b separately.
NEAR_ZERO = {
    4: [("all 8, b ~ -8s", "const", 8, None, 8), ("codes 7..9, b ~ -8s", "set", 0, (7, 8, 9), 8),
        ("all 0, b ~ 0", "const", 0, None, 0), ("all 15, b ~ -15s", "const", 15, None, 15),
        ("all 3, b ~ -3s", "const", 3, None, 3), ("all 12, b ~ -12s", "const", 12, None, 12)],
    8: [("all 128, b ~ -128s", "const", 128, None, 128),
        ("codes 127..129, b ~ -128s", "set", 0, (127, 128, 129), 128),
        ("all 0, b ~ 0", "const", 0, None, 0), ("all 255, b ~ -255s", "const", 255, None, 255),
        ("all 40, b ~ -40s", "const", 40, None, 40)],
}


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [4, 8])
def test_near_zero_weights(bits, xdt):
    N = 300
    for name, kind, c, cset, bc in NEAR_ZERO[bits]:
        for K in (64, 128, 704, 4096):
            seed = K + c + bc
            w = synth.affine_weights(bits, N, K, cfg=230, set_id=seed, codes=kind, const_code=c,
                                     code_set=cset, bias_code=bc)
            for batch in (1, 8):
                xb = draw_x(batch, K, xdt, seed + batch)
                print(f"near-zero bits={bits} {name} K={K} batch={batch} {xdt}", flush=True)
                y = run_gemv(bits, w, xb, xdt).cpu().numpy()
                yr, a = ref_gemv(w, xb, xdt)
                assert_within(y, yr, a, f"near-zero bits={bits} {name} K={K} batch={batch} {xdt}")


# Shapes whose activations are streamed through LDS in K slices (more than
# half the CU's LDS): the partial rows are summed in a fixed order, so two
# runs must agree bit for bit, and nothing outside y may be written.
SLICED = [(28672, 1000, 2), (28672, 1000, 4), (28672, 1000, 8), (8192, 3000, 8), (1 << 22, 3, 1),
          (1 << 22, 5, 2), (65536, 700, 1)]


@pytest.mark.parametrize("K,N,batch", SLICED)
def test_sliced_k_is_deterministic_and_in_bounds(K, N, batch):
    print(f"sliced K={K} N={N} batch={batch}", flush=True)
    w = synth.affine_weights(4, N, K, cfg=231, set_id=K + batch)
    xb = synth.x_f16(batch, K, cfg=231, set_id=batch)
    guard = 4096
    buf = torch.full((guard + batch * N + guard,), float("nan"), device="cuda")
    out = buf[guard:guard + batch * N].view(batch, N)
    y1 = run_gemv(4, w, xb, out=out).clone()
    y2 = run_gemv(4, w, xb).clone()
    y3 = run_gemv(4, w, xb).clone()
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + batch * N:]).all()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    rows = np.unique(np.concatenate([np.random.default_rng(K + N).choice(N, min(N, 64), replace=False),
                                     [0, N - 1]]))
    yr, a = ref_gemv(w, xb, rows=rows)
    assert_within(y1.cpu().numpy()[:, rows], yr, a, f"sliced K={K} N={N} batch={batch}")


# The matrix-core path (batch 3..8, fp16, K a multiple of 512) streams K
# through LDS in slices whose length is a multiple of (waves per tile) x 4
# steps of 128 inputs; when K / 128 is not a multiple of it the last slice is
# ragged and some waves have no step in it, while every wave still meets the
# same barriers. Ragged last tiles (N not a multiple of 16) as well.
RAGGED_SLICES = [(4608, 33, 3), (4608, 300, 8), (5632, 16, 5), (9728, 17, 8), (512, 40, 8),
                 (14848, 1, 3)]


@pytest.mark.parametrize("K,N,batch", RAGGED_SLICES)
def test_matrix_core_ragged_slices(K, N, batch):
    print(f"matrix-core K={K} N={N} batch={batch}", flush=True)
    w = synth.affine_weights(4, N, K, cfg=232, set_id=K + N + batch)
    xb = synth.x_f16(batch, K, cfg=232, set_id=batch)
    guard = 4096
    buf = torch.full((guard + batch * N + guard,), float("nan"), device="cuda")
    out = buf[guard:guard + batch * N].view(batch, N)
    y1 = run_gemv(4, w, xb, out=out).clone()
    y2 = run_gemv(4, w, xb).clone()
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + batch * N:]).all()
    assert torch.equal(y1, y2)
    yr, a = ref_gemv(w, xb)
    assert_within(y1.cpu().numpy(), yr, a, f"matrix-core K={K} N={N} batch={batch}")


def test_deterministic_and_no_out_of_bounds_writes():
    N, K, batch = 1000, 4096, 3
    w = synth.affine_weights(4, N, K, cfg=207, set_id=0)
    xb = synth.x_f16(batch, K, cfg=207, set_id=0)
    guard = 4096
    buf = torch.full((guard + batch * N + guard,), float("nan"), device="cuda")
    out = buf[guard:guard + batch * N].view(batch, N)
    y1 = run_gemv(4, w, xb, out=out).clone()
    y2 = run_gemv(4, w, xb).clone()
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + batch * N:]).all()
    assert torch.equal(y1, y2)


# --------------------------------------------------------------- full sizes

FULL = [
    ("c1 4096->4096", 4096, 4096, 1, None),
    ("c2 gate+up 4096->28672", 4096, 28672, 1, None),
    ("c2 down 14336->4096", 14336, 4096, 1, None),
    ("c5 8192->28672 b1", 8192, 28672, 1, 512),
    ("c5 28672->8192 b1", 28672, 8192, 1, 512),
    ("c5 8192->28672 b8", 8192, 28672, 8, 384),
    ("c5 28672->8192 b2", 28672, 8192, 2, 384),
    ("c5 28672->8192 b4", 28672, 8192, 4, 384),
    ("c5 28672->8192 b8", 28672, 8192, 8, 384),
]


@pytest.mark.parametrize("name,K,N,batch,nsample", FULL, ids=[f[0] for f in FULL])
def test_full_size(name, K, N, batch, nsample):
    print(name, flush=True)
    w = synth.affine_weights(4, N, K, cfg=5, set_id=0)
    xb = synth.x_f16(batch, K, cfg=5, set_id=0)
    y = run_gemv(4, w, xb).cpu().numpy()
    if nsample is None:
        yr, a = ref_gemv(w, xb)
        assert_within(y, yr, a, name)
    else:
        r = np.random.default_rng(N + K + batch)
        rows = np.unique(np.concatenate([r.choice(N, nsample, replace=False), [0, N - 1]]))
        yr, a = ref_gemv(w, xb, rows=rows)
        assert_within(y[:, rows], yr, a, name)
