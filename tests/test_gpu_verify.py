"""GPU parity of qgemm_affine4_verify (the verification GEMM over drafted
tokens: fp16 activations on the token kernel, bf16 on the staged chunk
kernel) against the fp64 oracle: |Y_gpu - Y_ref| <= 1e-4 * sum_k |w x| + 1e-6.

Source of the regime: uzu page on discuss.pytorch.kr, speculative-decoding
section (16 to 32 drafted tokens checked in one forward pass)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within, dev_bf16, dev_half, dev_weights

qd = pytest.importorskip("affine_quantized_gemv_qgemv_amd")

pytestmark = pytest.mark.gpu


def draw_x(M, K, xdt, seed):
    return synth.x_f16(M, K, cfg=510, set_id=seed) if xdt == "f16" else synth.x_bf16(M, K, cfg=510, set_id=seed)


def run(w, xb, xdt, out=None):
    wq, s, b = dev_weights(w)
    x = dev_half(xb) if xdt == "f16" else dev_bf16(xb)
    y = qd.qgemm_affine4_verify(wq, s, b, x, out=out)
    torch.cuda.synchronize()
    return y


def ref(w, xb, xdt, rows=None):
    return oracle.gemv_f16(w, xb, rows) if xdt == "f16" else oracle.gemm_chunk(w, xb, rows)


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("M", [1, 9, 16, 17, 32, 33, 64, 100, 128])
@pytest.mark.parametrize("N,K", [(1, 64), (37, 704), (64, 2112), (257, 4096)])
def test_small_shapes(xdt, M, N, K):
    seed = M * 31 + N + K
    w = synth.affine_weights(4, N, K, cfg=510, set_id=seed)
    xb = draw_x(M, K, xdt, seed)
    print(f"verify {xdt} M={M} N={N} K={K}", flush=True)
    y = run(w, xb, xdt).cpu().numpy()
    yr, a = ref(w, xb, xdt)
    assert_within(y, yr, a, f"{xdt} M={M} N={N} K={K}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_extreme_codes(xdt):
    K, M = 1024, 24
    for kind, c in (("zero", 0), ("const", 15), ("const", 7)):
        w = synth.affine_weights(4, 70, K, cfg=511, set_id=c, codes=kind, const_code=c)
        xb = draw_x(M, K, xdt, c)
        y = run(w, xb, xdt).cpu().numpy()
        yr, a = ref(w, xb, xdt)
        assert_within(y, yr, a, f"{kind} {c} {xdt}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_one_hot_rows_are_exact(xdt):
    N, K, M = 96, 1024, 16
    w = synth.affine_weights(4, N, K, cfg=512, set_id=0)
    xb = np.zeros((M, K), np.uint16)
    one = np.float16(1.0).view(np.uint16) if xdt == "f16" else synth.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    for m, k in enumerate([0, 1, 7, 63, 64, 100, 511, 512, 777, 1000, 1023, 5, 9, 300, 640, 900]):
        xb[m, k] = one
    y = run(w, xb, xdt).cpu().numpy().astype(np.float64)
    yr, _ = ref(w, xb, xdt)
    assert np.array_equal(y, yr)


def test_rows_match_the_gemv():
    # the first 8 tokens of a verification batch equal the batch-8 GEMV's rows
    N, K, M = 300, 2048, 20
    w = synth.affine_weights(4, N, K, cfg=513, set_id=0)
    xb = draw_x(M, K, "f16", 0)
    y = run(w, xb, "f16").cpu().numpy()
    wq, s, b = dev_weights(w)
    yv = qd.qgemv_affine4(wq, s, b, dev_half(xb[:8])).cpu().numpy()
    yr, a = ref(w, xb, "f16")
    assert_within(y, yr, a, "verify")
    assert_within(yv, yr[:8], a[:8], "gemv rows")


def test_deterministic_and_in_bounds():
    for xdt in ("f16", "bf16"):
        N, K, M = 200, 1024, 29
        w = synth.affine_weights(4, N, K, cfg=514, set_id=0)
        xb = draw_x(M, K, xdt, 3)
        guard = 4096
        buf = torch.full((guard + M * N + guard,), float("nan"), device="cuda")
        out = buf[guard:guard + M * N].view(M, N)
        y1 = run(w, xb, xdt, out=out).clone()
        y2 = run(w, xb, xdt).clone()
        assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + M * N:]).all()
        assert torch.equal(y1, y2)


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("M", [16, 32])
def test_full_size_7b_ffn(xdt, M):
    K, N = 4096, 14336
    print(f"verify full {xdt} M={M}", flush=True)
    w = synth.affine_weights(4, N, K, cfg=515, set_id=0)
    xb = draw_x(M, K, xdt, 5)
    y = run(w, xb, xdt).cpu().numpy()
    rows = np.unique(np.concatenate([np.random.default_rng(M).choice(N, 256, replace=False), [0, N - 1]]))
    yr, a = ref(w, xb, xdt, rows)
    assert_within(y[:, rows], yr, a, f"full {xdt} M={M}")


# K split: shapes with fewer than 128 column x row tiles spread K over
# workgroups and add the slices in a second pass (the workspace)

@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("M", [1, 16, 32, 33, 64, 65, 128])
@pytest.mark.parametrize("N,K", [(130, 3200), (64, 2368), (4096, 2048)])
def test_split_k_ragged(xdt, M, N, K):
    ws = qd.verify_workspace_bytes(M, N, K)
    splits = ws // (4 * M * N)
    assert splits >= 2
    seed = 7 * M + N + K
    w = synth.affine_weights(4, N, K, cfg=516, set_id=seed)
    xb = draw_x(M, K, xdt, seed)
    print(f"verify split {xdt} M={M} N={N} K={K} splits={splits}", flush=True)
    y = run(w, xb, xdt).cpu().numpy()
    if N * M <= 64 * 1088 * 2:
        yr, a = ref(w, xb, xdt)
        assert_within(y, yr, a, f"split {xdt} M={M} N={N} K={K}")
    else:
        rows = np.unique(np.concatenate([np.random.default_rng(seed).choice(N, 200, replace=False), [0, N - 1]]))
        yr, a = ref(w, xb, xdt, rows)
        assert_within(y[:, rows], yr, a, f"split {xdt} M={M} N={N} K={K}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_split_k_extreme_and_near_zero_codes(xdt):
    N, K, M = 96, 4096, 20
    for kind, c in (("zero", 0), ("const", 15), ("const", 8)):
        w = synth.affine_weights(4, N, K, cfg=517, set_id=c, codes=kind, const_code=c)
        xb = draw_x(M, K, xdt, c)
        y = run(w, xb, xdt).cpu().numpy()
        yr, a = ref(w, xb, xdt)
        assert_within(y, yr, a, f"split {kind} {c} {xdt}")


def test_split_k_deterministic_and_in_bounds():
    # two calls bitwise equal; Y and the workspace written only inside their
    # bounds; a workspace holding stale values from another shape changes nothing
    for xdt in ("f16", "bf16"):
        N, K, M = 4096, 14336, 32
        ws = qd.verify_workspace_bytes(M, N, K)
        assert ws > 0
        w = synth.affine_weights(4, N, K, cfg=518, set_id=0)
        xb = draw_x(M, K, xdt, 4)
        wq, s, b = dev_weights(w)
        x = dev_half(xb) if xdt == "f16" else dev_bf16(xb)
        guard = 4096
        ybuf = torch.full((guard + M * N + guard,), float("nan"), device="cuda")
        wbuf = torch.full((guard + ws // 4 + guard,), float("nan"), device="cuda")
        out = ybuf[guard:guard + M * N].view(M, N)
        wsp = wbuf[guard:guard + ws // 4].view(torch.uint8)
        y1 = qd.qgemm_affine4_verify(wq, s, b, x, out=out, workspace=wsp).clone()
        torch.cuda.synchronize()
        assert torch.isnan(ybuf[:guard]).all() and torch.isnan(ybuf[guard + M * N:]).all()
        assert torch.isnan(wbuf[:guard]).all() and torch.isnan(wbuf[guard + ws // 4:]).all()
        # stale contents from a smaller split shape, then the same call again
        x2 = x[:7].contiguous()
        qd.qgemm_affine4_verify(wq, s, b, x2, workspace=wsp)
        y2 = qd.qgemm_affine4_verify(wq, s, b, x, workspace=wsp)
        y3 = qd.qgemm_affine4_verify(wq, s, b, x)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(y1, y3)
        with pytest.raises(qd.QDecodeError):
            qd.qgemm_affine4_verify(wq, s, b, x, workspace=wsp[:ws - 16])


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("M", [16, 32, 128])
def test_full_size_7b_down_projection(xdt, M):
    K, N = 14336, 4096
    print(f"verify full down {xdt} M={M}", flush=True)
    w = synth.affine_weights(4, N, K, cfg=519, set_id=0)
    xb = draw_x(M, K, xdt, 6)
    y = run(w, xb, xdt).cpu().numpy()
    rows = np.unique(np.concatenate([np.random.default_rng(M + 1).choice(N, 128, replace=False), [0, N - 1]]))
    yr, a = ref(w, xb, xdt, rows)
    assert_within(y[:, rows], yr, a, f"full down {xdt} M={M}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_split_k_at_the_largest_k(xdt):
    # K = 2^22 on 3 rows: 256 splits of 256 groups; M N = 6 is not a multiple
    # of 4 (the adding pass's element-wise tail)
    K, N, M = 1 << 22, 3, 2
    ws = qd.verify_workspace_bytes(M, N, K)
    assert ws // (4 * M * N) == 256
    w = synth.affine_weights(4, N, K, cfg=520, set_id=0)
    xb = draw_x(M, K, xdt, 8)
    print(f"verify split K=2^22 {xdt}", flush=True)
    y = run(w, xb, xdt).cpu().numpy()
    yr, a = ref(w, xb, xdt)
    assert_within(y, yr, a, f"split K=2^22 {xdt}")


def test_split_k_ragged_elementwise_tail():
    # M N odd on a split shape: every element, including the last, written once
    for M, N, K in ((3, 7, 2048), (5, 65, 4096)):
        ws = qd.verify_workspace_bytes(M, N, K)
        assert ws > 0 and (M * N) % 4 != 0
        w = synth.affine_weights(4, N, K, cfg=521, set_id=M)
        xb = draw_x(M, K, "f16", M)
        guard = 64
        buf = torch.full((guard + M * N + guard,), float("nan"), device="cuda")
        out = buf[guard:guard + M * N].view(M, N)
        y = run(w, xb, "f16", out=out).cpu().numpy()
        assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + M * N:]).all()
        yr, a = ref(w, xb, "f16")
        assert_within(y, yr, a, f"split tail M={M} N={N}")
