"""GPU parity of qgemm_affine4_verify_i8 (the verification GEMM on per-token
int8 activations) against the oracle.

Source: uzu page on discuss.pytorch.kr, section on speculative decoding (16
to 32 drafted tokens checked in one pass on the int8 matrix path, the
activations quantized to 8 bits as it goes); the scheme is the oracle's
reading: scale max|x| / 127, codes round(x / scale) with ties to even, both
in fp32. The quantized codes and scales decide integers, so they are
compared bit for bit (read back from the workspace, whose layout the kernel
source documents); Y within |Y_gpu - Y_ref| <= 1e-4 * sum_k |w x^| + 1e-6,
x^ = scale * code (exact in fp64).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within, dev_half, dev_weights

qd = pytest.importorskip("affine_quantized_gemv_qgemv_amd")

pytestmark = pytest.mark.gpu

PERM = [0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15]


def _al(v):
    return (v + 255) // 256 * 256


def read_workspace(ws, M, K):
    """Codes [M][K] int8, group sums [M][K/64] and scales [M] from the
    workspace: codes int8 [G][Mp][64] (16-input blocks permuted by PERM),
    sums fp32 [G][Mp], scales fp32 [Mp], each part 256-byte aligned."""
    Mp, G = (M + 15) // 16 * 16, K // 64
    raw = ws.cpu().numpy()
    q = raw[:Mp * K].view(np.int8).reshape(G, Mp, 4, 16)
    codes = np.empty((Mp, G, 4, 16), np.int8)
    codes[..., PERM] = q.transpose(1, 0, 2, 3)
    o = _al(Mp * K)
    xs = raw[o:o + G * Mp * 4].view(np.float32).reshape(G, Mp).T
    o += _al(G * Mp * 4)
    sx = raw[o:o + Mp * 4].view(np.float32)
    return codes.reshape(Mp, K)[:M], xs[:M], sx[:M], (codes.reshape(Mp, K)[M:], xs[M:], sx[M:])


def run(w, xb, out=None, workspace=None):
    wq, s, b = dev_weights(w)
    y = qd.qgemm_affine4_verify_i8(wq, s, b, dev_half(xb), out=out, workspace=workspace)
    torch.cuda.synchronize()
    return y


def draw_x(M, K, seed):
    return synth.x_f16(M, K, cfg=520, set_id=seed)


@pytest.mark.parametrize("M", [1, 3, 16, 17, 32])
@pytest.mark.parametrize("K", [64, 704, 4096])
def test_codes_sums_and_scales_are_the_oracles(M, K):
    print(f"verify_i8 quantize M={M} K={K}", flush=True)
    w = synth.affine_weights(4, 40, K, cfg=520, set_id=K)
    xb = draw_x(M, K, M + K)
    ws = torch.full((qd.verify_i8_workspace_bytes(M, K),), 0x55, dtype=torch.uint8, device="cuda")
    run(w, xb, workspace=ws)
    codes, xs, sx, (pad_q, pad_xs, pad_sx) = read_workspace(ws, M, K)
    q_ref, sc_ref = oracle.quant_i8(xb)
    assert np.array_equal(sx.view(np.uint32), sc_ref.view(np.uint32))
    assert np.array_equal(codes, q_ref)
    sums = q_ref.astype(np.int64).reshape(M, K // 64, 64).sum(axis=2)
    assert np.array_equal(xs.astype(np.int64), sums) and np.array_equal(xs, sums.astype(np.float32))
    # the padding rows of the last 16-token block are zero
    assert not pad_q.any() and not pad_xs.any() and not pad_sx.any()


def test_ties_round_to_even_and_extremes():
    # max |x| = 127 gives scale 1 exactly, so x = n + 0.5 is a tie
    M, K = 4, 128
    vals = np.zeros((M, K), np.float32)
    vals[0, :8] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5]
    vals[0, 8] = 127.0
    vals[1, 0] = -65504.0                       # largest fp16 magnitude
    vals[1, 1:4] = [65504.0, 257.0, -258.0]
    vals[2, :] = np.float32(6e-8)               # fp16 subnormals only
    vals[2, 5] = -6e-8
    # row 3 stays zero
    xb = vals.astype(np.float16).view(np.uint16)
    w = synth.affine_weights(4, 16, K, cfg=521, set_id=0)
    ws = torch.zeros(qd.verify_i8_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    y = run(w, xb, workspace=ws).cpu().numpy()
    codes, _, sx, _ = read_workspace(ws, M, K)
    q_ref, sc_ref = oracle.quant_i8(xb)
    assert np.array_equal(codes, q_ref) and np.array_equal(sx, sc_ref)
    assert list(codes[0, :9]) == [0, 2, 2, 0, -2, -2, 126, -126, 127]
    assert codes.min() >= -127 and codes.max() <= 127
    assert np.array_equal(y[3], np.zeros(16, np.float32))
    yr, a = oracle.verify_i8(w, xb)
    assert_within(y, yr, a, "ties and extremes")


@pytest.mark.parametrize("M", [1, 2, 5, 16, 17, 31, 32])
@pytest.mark.parametrize("N,K", [(1, 64), (37, 704), (64, 2112), (100, 1088), (257, 4096)])
def test_small_shapes(M, N, K):
    seed = M * 31 + N + K
    print(f"verify_i8 M={M} N={N} K={K}", flush=True)
    w = synth.affine_weights(4, N, K, cfg=522, set_id=seed)
    xb = draw_x(M, K, seed)
    y = run(w, xb).cpu().numpy()
    yr, a = oracle.verify_i8(w, xb)
    assert_within(y, yr, a, f"verify_i8 M={M} N={N} K={K}")


def test_zero_rows_give_zero_outputs():
    M, N, K = 20, 70, 1024
    w = synth.affine_weights(4, N, K, cfg=523, set_id=0)
    xb = draw_x(M, K, 5)
    xb[[0, 7, 19]] = 0
    xb[3] = np.float16(-0.0).view(np.uint16)
    y = run(w, xb).cpu().numpy()
    for m in (0, 3, 7, 19):
        assert np.array_equal(y[m], np.zeros(N, np.float32)), m
    yr, a = oracle.verify_i8(w, xb)
    assert_within(y, yr, a, "zero rows")


def test_extreme_and_near_zero_weights():
    K, M, N = 1024, 24, 70
    cases = [("zero", 0, None, 8), ("const", 15, None, 8), ("const", 0, None, 0), ("const", 8, None, 8),
             ("set", 0, (7, 8, 9), 8), ("const", 12, None, 12), ("const", 15, None, 15)]
    for kind, c, cset, bc in cases:
        w = synth.affine_weights(4, N, K, cfg=524, set_id=c + bc, codes=kind, const_code=c,
                                 code_set=cset, bias_code=bc)
        xb = draw_x(M, K, c)
        print(f"verify_i8 weights {kind} c={c} set={cset} b~-{bc}s", flush=True)
        y = run(w, xb).cpu().numpy()
        yr, a = oracle.verify_i8(w, xb)
        assert_within(y, yr, a, f"{kind} {c} {cset} {bc}")


def test_one_hot_weights_return_the_quantized_activation():
    # row n of W is e_n (code 9, scale 1, bias -8 at input n; code 8 else):
    # Y[m][n] = fp32(scale[m] * code[m][n]) exactly
    M, K = 32, 256
    N = K
    q = np.full((N, K), 8, np.uint32)
    q[np.arange(N), np.arange(N)] = 9
    words = np.zeros((N, K // 8), np.uint32)
    for i in range(8):
        words |= q[:, i::8] << np.uint32(4 * i)
    one = np.float16(1.0).view(np.uint16)
    s = np.full((N, K // 64), one, np.uint16)
    b = np.full((N, K // 64), np.float16(-8.0).view(np.uint16), np.uint16)
    w = synth.AffineWeights(bits=4, N=N, K=K, wq=words, scales=s, biases=b)
    xb = draw_x(M, K, 9)
    y = run(w, xb).cpu().numpy()
    q_ref, sc_ref = oracle.quant_i8(xb)
    assert np.array_equal(y, (sc_ref[:, None] * q_ref.astype(np.float32)).astype(np.float32))


def test_deterministic_guarded_and_workspace_reused():
    # one workspace (left holding the previous call's contents) serves a
    # 32-token call and then a 5-token one; nothing past y or the workspace
    # is written, and repeated calls agree bit for bit
    N, K = 1000, 2048
    w = synth.affine_weights(4, N, K, cfg=525, set_id=0)
    need = qd.verify_i8_workspace_bytes(32, K)
    g = 1 << 14
    wsbuf = torch.full((need + g,), 0x7F, dtype=torch.uint8, device="cuda")
    ws = wsbuf[:need]
    for M in (32, 5, 32):
        xb = draw_x(M, K, 100 + M)
        ybuf = torch.full((g + M * N + g,), float("nan"), device="cuda")
        out = ybuf[g:g + M * N].view(M, N)
        outs = []
        for _ in range(2):
            run(w, xb, out=out, workspace=ws)
            outs.append(out.clone())
        assert torch.equal(outs[0], outs[1])
        assert torch.isnan(ybuf[:g]).all() and torch.isnan(ybuf[g + M * N:]).all()
        assert bool((wsbuf[need:] == 0x7F).all()), "write past the workspace"
        yr, a = oracle.verify_i8(w, xb)
        assert_within(outs[0].cpu().numpy(), yr, a, f"reuse M={M}")


@pytest.mark.parametrize("M", [16, 32])
def test_full_size_sampled_rows(M):
    # the benchmarked shape: 7B FFN up projection, K = 4096 -> N = 14336
    N, K = 14336, 4096
    w = synth.affine_weights(4, N, K, cfg=526, set_id=M)
    xb = draw_x(M, K, M)
    print(f"verify_i8 full M={M}", flush=True)
    y = run(w, xb).cpu().numpy()
    rows = np.concatenate([np.arange(0, 64), np.random.default_rng(M).choice(N, 200, replace=False),
                           np.arange(N - 64, N)])
    yr, a = oracle.verify_i8(w, xb, rows)
    assert_within(y[:, rows], yr, a, f"full M={M}")


def test_close_to_the_fp16_verification():
    # int8 activations move each product by at most half a code step:
    # |Y_i8 - Y_f16| <= sum_k |w| * scale / 2 (plus both kernels' rounding)
    M, N, K = 32, 300, 4096
    w = synth.affine_weights(4, N, K, cfg=527, set_id=0)
    xb = draw_x(M, K, 1)
    y8 = run(w, xb).cpu().numpy().astype(np.float64)
    wq, s, b = dev_weights(w)
    y16 = qd.qgemm_affine4_verify(wq, s, b, dev_half(xb)).cpu().numpy().astype(np.float64)
    _, sc = oracle.quant_i8(xb)
    _, wabs = oracle.gemv(w, np.ones((1, K)))     # A of an all-ones input = sum_k |w|
    bound = sc.astype(np.float64)[:, None] * 0.5 * wabs[0][None, :] * 1.001 + 1e-3 * np.abs(y16) + 1e-5
    assert np.all(np.abs(y8 - y16) <= bound)


# Shapes that select each workgroup shape of the GEMM (tiles per workgroup
# 4 / 2 / 1, 4 or 8 waves, scales staged in LDS or read per group), all with
# a ragged last tile; checked on sampled rows that include the tail.
TILE_SHAPES = [(16400, 4096, 16), (16400, 8192, 16), (8200, 4096, 32), (8200, 8192, 20),
               (4100, 14336, 16), (4100, 4096, 5), (300, 32768, 16), (300, 32768, 32), (300, 32896, 3)]


@pytest.mark.parametrize("N,K,M", TILE_SHAPES)
def test_workgroup_shapes_on_sampled_rows(N, K, M):
    print(f"verify_i8 tiles N={N} K={K} M={M}", flush=True)
    w = synth.affine_weights(4, N, K, cfg=528, set_id=N + K + M)
    xb = draw_x(M, K, N + M)
    y = run(w, xb).cpu().numpy()
    rng = np.random.default_rng(N + K)
    rows = np.unique(np.concatenate([np.arange(0, 40), rng.choice(N, 120, replace=False),
                                     np.arange(N - 80, N)]))
    yr, a = oracle.verify_i8(w, xb, rows)
    assert_within(y[:, rows], yr, a, f"tiles N={N} K={K} M={M}")
