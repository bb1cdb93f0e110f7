"""The nibble-to-byte permutes that feed the fp8 converter (csrc/mfma.h).

v_perm_b32(src0, src1, sel) builds each result byte from an 8-byte pool
(bytes 0..3 of src1, then bytes 0..3 of src0) by the selector byte. The
kernels spread the 8 codes of a word w to bytes as t = w & 0x0F0F0F0F
(codes 0, 2, 4, 6) and u = (w >> 4) & 0x0F0F0F0F (codes 1, 3, 5, 7), then
permute. This test models the instruction and checks the selectors read
from the header against the orders the activations are staged in: natural
(chunk GEMM) and [0, 4, 1, 5, 2, 6, 3, 7] (MoE prefill). No GPU needed.
"""
import os
import re

import numpy as np

HDR = os.path.join(os.path.dirname(__file__), "..", "affine_quantized_gemv_qgemv_amd", "csrc", "mfma.h")


def v_perm(src0, src1, sel):
    pool = [(src1 >> (8 * i)) & 0xFF for i in range(4)] + [(src0 >> (8 * i)) & 0xFF for i in range(4)]
    out = 0
    for i in range(4):
        s = (sel >> (8 * i)) & 0xFF
        assert s < 8, "selector outside the byte pool"
        out |= pool[s] << (8 * i)
    return out


def selectors(func):
    src = open(HDR).read()
    body = src[src.index(func):]
    body = body[:body.index("\n}\n")]
    return [int(v, 16) for v in re.findall(r"__builtin_amdgcn_perm\(u, t, (0x[0-9A-Fa-f]+)u\)", body)]


def spread(func, w):
    t = w & 0x0F0F0F0F
    u = (w >> 4) & 0x0F0F0F0F
    out = []
    for sel in selectors(func):
        v = v_perm(u, t, sel)
        out += [(v >> (8 * i)) & 0xFF for i in range(4)]
    return out


def test_natural_order():
    rng = np.random.default_rng(11)
    for w in rng.integers(0, 2**32, size=500, dtype=np.uint64):
        w = int(w)
        q = [(w >> (4 * i)) & 0xF for i in range(8)]
        assert spread("uint2 codes_to_bytes(", w) == q


def test_interleaved_order():
    rng = np.random.default_rng(12)
    for w in rng.integers(0, 2**32, size=500, dtype=np.uint64):
        w = int(w)
        q = [(w >> (4 * i)) & 0xF for i in range(8)]
        assert spread("uint2 codes_to_bytes_p(", w) == [q[i] for i in (0, 4, 1, 5, 2, 6, 3, 7)]


def test_model_catches_a_swapped_selector():
    # the mistake this guards against: one selector byte off
    w = 0x76543210
    t, u = w & 0x0F0F0F0F, (w >> 4) & 0x0F0F0F0F
    v = v_perm(u, t, 0x05040200)
    assert [(v >> (8 * i)) & 0xFF for i in range(4)] != [0, 4, 1, 5]
