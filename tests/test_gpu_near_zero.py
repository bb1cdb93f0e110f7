"""Weights at and near zero on the matrix-core paths (the prefill chunk GEMM,
the verification GEMM, the 8-bit router over a token chunk and the MoE
experts over a prefill chunk).

TurboFieldfare article, section "성능과 제약": w = s*q + b; with b close to
-c*s, codes at c give weights close to zero, where real weights cluster. The
bar is the workload's relative bar, |y - y_ref| <= 1e-4 * sum_k |w_k x_k| +
1e-6, so each kernel's rounding must follow |w x|, not s*q or b separately.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within, dev_bf16, dev_half, dev_moe, dev_weights

qd = pytest.importorskip("affine_quantized_gemv_qgemv_amd")

pytestmark = pytest.mark.gpu

FAMILIES = {
    4: [("all 8, b ~ -8s", "const", 8, None, 8), ("codes 7..9, b ~ -8s", "set", 0, (7, 8, 9), 8),
        ("all 0, b ~ 0", "const", 0, None, 0), ("all 15, b ~ -15s", "const", 15, None, 15),
        ("all 3, b ~ -3s", "const", 3, None, 3)],
    8: [("all 128, b ~ -128s", "const", 128, None, 128),
        ("codes 127..129, b ~ -128s", "set", 0, (127, 128, 129), 128),
        ("all 255, b ~ -255s", "const", 255, None, 255), ("all 0, b ~ 0", "const", 0, None, 0)],
}


def _x(T, K, xdt, seed):
    return synth.x_f16(T, K, cfg=240, set_id=seed) if xdt == "f16" else synth.x_bf16(T, K, cfg=240, set_id=seed)


@pytest.mark.parametrize("M", [1, 37, 128])
def test_chunk_gemm(M):
    N = 130
    for name, kind, c, cset, bc in FAMILIES[4]:
        for K in (64, 128, 704, 4096):
            w = synth.affine_weights(4, N, K, cfg=240, set_id=K + c, codes=kind, const_code=c,
                                     code_set=cset, bias_code=bc)
            xb = _x(M, K, "bf16", K + M)
            print(f"chunk M={M} K={K} {name}", flush=True)
            y = qd.qgemm_affine4_chunk(*dev_weights(w), dev_bf16(xb)).cpu().numpy()
            yr, a = oracle.gemm_chunk(w, xb)
            assert_within(y, yr, a, f"chunk M={M} K={K} {name}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("M", [9, 32, 64])
def test_verify_gemm(M, xdt):
    N = 130
    for name, kind, c, cset, bc in FAMILIES[4]:
        for K in (64, 704, 4096):
            w = synth.affine_weights(4, N, K, cfg=241, set_id=K + c, codes=kind, const_code=c,
                                     code_set=cset, bias_code=bc)
            xb = _x(M, K, xdt, K + M)
            x = dev_half(xb) if xdt == "f16" else dev_bf16(xb)
            print(f"verify M={M} K={K} {name} {xdt}", flush=True)
            y = qd.qgemm_affine4_verify(*dev_weights(w), x).cpu().numpy()
            yr, a = oracle.gemv_f16(w, xb) if xdt == "f16" else oracle.gemm_chunk(w, xb)
            assert_within(y, yr, a, f"verify M={M} K={K} {name} {xdt}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("T", [9, 128])
def test_int8_token_chunk(T, xdt):
    N = 130
    for name, kind, c, cset, bc in FAMILIES[8]:
        for K in (64, 704, 2816):
            w = synth.affine_weights(8, N, K, cfg=242, set_id=K + c, codes=kind, const_code=c,
                                     code_set=cset, bias_code=bc)
            xb = _x(T, K, xdt, K + T)
            x = dev_half(xb) if xdt == "f16" else dev_bf16(xb)
            print(f"int8 chunk T={T} K={K} {name} {xdt}", flush=True)
            y = qd.qgemv_affine8(*dev_weights(w), x).cpu().numpy()
            yr, a = oracle.gemv_f16(w, xb) if xdt == "f16" else oracle.gemm_chunk(w, xb)
            assert_within(y, yr, a, f"int8 chunk T={T} K={K} {name} {xdt}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_moe_prefill(xdt):
    # every expert matrix (routed and shared) near zero; 11 input groups
    # (ragged stages), routing fixed so that the experts see many rows
    T, k = 37, 3
    for name, kind, c, cset, bc in FAMILIES[4]:
        mw = synth.moe_weights(E=8, H=704, I=128, Is=192, cfg=243, layer=c,
                               expert_codes=dict(codes=kind, const_code=c, code_set=cset, bias_code=bc))
        xb = _x(T, 704, xdt, c)
        x = dev_half(xb) if xdt == "f16" else dev_bf16(xb)
        idx = (np.arange(T)[:, None] * 5 + np.arange(k)[None, :] * 3) % 8
        p = np.tile(np.array([0.5, 0.3, 0.2]), (T, 1))
        print(f"moe prefill T={T} {name} {xdt}", flush=True)
        y = qd.qmoe_expert_gemv(dev_moe(mw), torch.tensor(idx, dtype=torch.int32, device="cuda"),
                                torch.tensor(p, dtype=torch.float32, device="cuda"), x).cpu().numpy()
        xd = oracle.f16_to_f64(xb) if xdt == "f16" else oracle.bf16_to_f64(xb)
        yr, a = oracle.moe_experts(mw, xd, idx, p)
        assert_within(y, yr, a, f"moe prefill T={T} {name} {xdt}")
