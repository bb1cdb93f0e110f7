"""GPU parity of qgemm_affine4_chunk (bf16 MFMA prefill chunk) against the
fp64 oracle: |Y_gpu - Y_ref| <= 1e-4 * sum_k |w x| + 1e-6 per output."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within, dev_bf16, dev_weights

qd = pytest.importorskip("affine_quantized_gemv_qgemv_amd")

pytestmark = pytest.mark.gpu


def run_chunk(w, xb, out=None):
    wq, s, b = dev_weights(w)
    y = qd.qgemm_affine4_chunk(wq, s, b, dev_bf16(xb), out=out)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M", [1, 7, 33, 128])
@pytest.mark.parametrize("N,K", [(1, 64), (17, 704), (64, 2112), (100, 2816), (257, 4096)])
def test_small_shapes(M, N, K):
    w = synth.affine_weights(4, N, K, cfg=500, set_id=M * 31 + N)
    xb = synth.x_bf16(M, K, cfg=500, set_id=M * 31 + N)
    y = run_chunk(w, xb).cpu().numpy()
    yr, a = oracle.gemm_chunk(w, xb)
    print(f"M={M} N={N} K={K}", flush=True)
    assert_within(y, yr, a, f"M={M} N={N} K={K}")


def test_one_hot_rows_are_exact():
    N, K, M = 96, 1024, 16
    w = synth.affine_weights(4, N, K, cfg=501, set_id=0)
    xb = np.zeros((M, K), np.uint16)
    one = synth.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    cols = [0, 1, 7, 63, 64, 100, 511, 512, 777, 1000, 1023, 5, 9, 300, 640, 900]
    for m, k in enumerate(cols):
        xb[m, k] = one
    y = run_chunk(w, xb).cpu().numpy().astype(np.float64)
    yr, _ = oracle.gemm_chunk(w, xb)
    assert np.array_equal(y, yr)


def test_rows_match_the_gemv():
    N, K, M = 300, 2048, 9
    w = synth.affine_weights(4, N, K, cfg=502, set_id=0)
    xb = synth.x_bf16(M, K, cfg=502, set_id=0)
    y = run_chunk(w, xb).cpu().numpy()
    wq, s, b = dev_weights(w)
    yv = qd.qgemv_affine4(wq, s, b, dev_bf16(xb[:8])).cpu().numpy()
    yr, a = oracle.gemm_chunk(w, xb)
    assert_within(y, yr, a, "chunk")
    assert_within(yv, yr[:8], a[:8], "gemv rows")


def test_deterministic_and_in_bounds():
    N, K, M = 200, 1024, 100
    w = synth.affine_weights(4, N, K, cfg=503, set_id=0)
    xb = synth.x_bf16(M, K, cfg=503, set_id=0)
    guard = 1024
    buf = torch.full((guard + M * N + guard,), float("nan"), device="cuda")
    out = buf[guard:guard + M * N].view(M, N)
    y1 = run_chunk(w, xb, out=out).clone()
    y2 = run_chunk(w, xb).clone()
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + M * N:]).all()
    assert torch.equal(y1, y2)


def test_full_size_dense_chunk():
    c = synth.CONFIGS["c4_chunk"]
    M, K, N = c["M"], c["K"], c["N"]
    print("c4 dense chunk", flush=True)
    w = synth.affine_weights(4, N, K, cfg=4, set_id=0)
    xb = synth.x_bf16(M, K, cfg=4, set_id=0)
    y = run_chunk(w, xb).cpu().numpy()
    rows = np.unique(np.concatenate([np.random.default_rng(1).choice(N, 256, replace=False), [0, N - 1]]))
    yr, a = oracle.gemm_chunk(w, xb, rows=rows)
    assert_within(y[:, rows], yr, a, "c4 dense")


def test_full_size_7b_down_projection_split_k():
    # the prefill down projection K=14336 -> N=4096 over a 128-token chunk: 64 column
    # tiles, so K is split across workgroups; sampled rows against the oracle, two
    # calls bitwise equal, Y written only inside its bounds
    K, N, M = 14336, 4096, 128
    assert qd.chunk_workspace_bytes(M, N, K) > 0
    w = synth.affine_weights(4, N, K, cfg=503, set_id=1)
    xb = synth.x_bf16(M, K, cfg=503, set_id=1)
    print("chunk down projection 128 x 14336 -> 4096", flush=True)
    guard = 4096
    buf = torch.full((guard + M * N + guard,), float("nan"), device="cuda")
    out = buf[guard:guard + M * N].view(M, N)
    y1 = run_chunk(w, xb, out=out).clone()
    y2 = run_chunk(w, xb)
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + M * N:]).all()
    assert torch.equal(y1, y2)
    rows = np.unique(np.concatenate([np.random.default_rng(3).choice(N, 96, replace=False), [0, N - 1]]))
    yr, a = oracle.gemm_chunk(w, xb, rows)
    assert_within(y1.cpu().numpy()[:, rows], yr, a, "chunk down projection")
