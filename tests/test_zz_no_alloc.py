"""GPU check of qmoe_layer_decode_noalloc, the allocation-free variant of the
decode MoE layer: through the C ABI, its outputs must equal those of
qmoe_layer_decode (same kernels, a caller workspace instead of the library's
per-device scratch) bit for bit, and meet the oracle's bar, on consecutive
calls whose activations shrink and grow again (the scratch keeps the previous
call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within, dev_half, dev_moe

qd = pytest.importorskip("affine_quantized_gemv_qgemv_amd")

pytestmark = pytest.mark.gpu

SHAPES = [dict(E=128, H=2816, I=704, Is=2112, k=8),    # the decode workload's layer
          dict(E=64, H=1024, I=256, Is=512, k=4),      # smaller activations
          dict(E=16, H=256, I=64, Is=128, k=2)]


def _layer(mw, w, x, k):
    """qmoe_layer_decode through the C ABI with a caller workspace."""
    L = qd.lib()
    st = w.cstruct()
    need = int(L.qmoe_expert_workspace_bytes(ctypes.byref(st), 1, k))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    logits = torch.empty((1, mw.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, k), dtype=torch.int32, device="cuda")
    p = torch.empty((1, k), dtype=torch.float32, device="cuda")
    y = torch.empty((1, mw.H), dtype=torch.float32, device="cuda")
    rc = L.qmoe_layer_decode(ctypes.byref(st), w.router_q.data_ptr(), w.router_s.data_ptr(),
                             w.router_b.data_ptr(), k, x.data_ptr(), 0, logits.data_ptr(),
                             idx.data_ptr(), p.data_ptr(), y.data_ptr(), ws.data_ptr(), need, None)
    assert rc == qd.QD_OK, qd.last_error()
    return logits, idx, p, y


def _noalloc(mw, w, x, k):
    """qmoe_layer_decode_noalloc through the C ABI (outputs poisoned first)."""
    L = qd.lib()
    st = w.cstruct()
    logits = torch.full((1, mw.E), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((1, k), -7, dtype=torch.int32, device="cuda")
    p = torch.full((1, k), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((1, mw.H), float("nan"), dtype=torch.float32, device="cuda")
    rc = L.qmoe_layer_decode_noalloc(ctypes.byref(st), w.router_q.data_ptr(), w.router_s.data_ptr(),
                                     w.router_b.data_ptr(), k, x.data_ptr(), 0, logits.data_ptr(),
                                     idx.data_ptr(), p.data_ptr(), y.data_ptr(), None)
    assert rc == qd.QD_OK, qd.last_error()
    return logits, idx, p, y


def test_noalloc_layer_matches_the_workspace_call():
    layers = []
    for i, sh in enumerate(SHAPES):
        mw = synth.moe_weights(E=sh["E"], H=sh["H"], I=sh["I"], Is=sh["Is"], cfg=700, layer=i)
        layers.append((sh, mw, dev_moe(mw)))
    # large, smaller, smallest, then the large one again over the stale scratch
    for n, j in enumerate((0, 1, 2, 0)):
        sh, mw, w = layers[j]
        k = sh["k"]
        xb = synth.x_f16(1, sh["H"], cfg=700, set_id=n)
        x = dev_half(xb)
        print(f"noalloc call {n}: E={sh['E']} H={sh['H']} I={sh['I']} Is={sh['Is']} k={k}", flush=True)
        got = _noalloc(mw, w, x, k)
        ref = _layer(mw, w, x, k)
        torch.cuda.synchronize()
        for g, r, name in zip(got, ref, ("logits", "idx", "weights", "y")):
            assert torch.equal(g, r), f"call {n}: {name} differs from qmoe_layer_decode"
        # and the oracle's bar on the GPU's own routing
        yr, a = oracle.moe_experts(mw, oracle.f16_to_f64(xb), got[1].cpu().numpy(),
                                   got[2].cpu().numpy().astype(np.float64))
        assert_within(got[3].cpu().numpy(), yr, a, f"noalloc call {n}")
