"""GPU parity of the MoE layer: int8 router GEMV -> top-k routing -> expert
block (qmoe_expert_gemv), against the fp64 oracle.

Expert ids and their order must match bit for bit; outputs must satisfy
|y_gpu - y_ref| <= 1e-4 * A + 1e-6 with
A = sum_j p_j sum_k |W_dn[e_j] h_j| + sum_k |W_sdn h_s| (oracle values).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within, dev_bf16, dev_half, dev_moe

qd = pytest.importorskip("affine_quantized_gemv_qgemv_amd")

pytestmark = pytest.mark.gpu


def x_dev(xb, xdt):
    return dev_half(xb) if xdt == "f16" else dev_bf16(xb)


def x_ref(xb, xdt):
    return oracle.f16_to_f64(xb) if xdt == "f16" else oracle.bf16_to_f64(xb)


def run_layer(w, xb, k, xdt="f16"):
    x = x_dev(xb, xdt)
    T = x.shape[0]
    logits = torch.empty((T, w.E), dtype=torch.float32, device="cuda")
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    p = torch.full((T, k), -7.0, dtype=torch.float32, device="cuda")
    y = qd.qmoe_layer(w, x, k=k, logits=logits, idx=idx, weights=p)
    torch.cuda.synchronize()
    return logits, idx, p, y


def check_layer(mw, xb, k, act=0, xdt="f16", tokens=None, what=""):
    w = dev_moe(mw, act)
    logits, il, pl, yl = run_layer(w, xb, k, xdt)
    # routing on the GPU's own logits: ids bit-exact
    idx, p = qd.qmoe_route_topk(logits, k)
    y = qd.qmoe_expert_gemv(w, idx, p, x_dev(xb, xdt))
    torch.cuda.synchronize()
    # the one-call layer (decode: ranking inside gate+up) equals the separate calls
    assert torch.equal(il, idx), f"{what}: layer ids differ from qmoe_route_topk"
    assert torch.equal(pl, p), f"{what}: layer weights differ from qmoe_route_topk"
    assert torch.equal(yl, y), f"{what}: layer output differs from qmoe_expert_gemv"
    L = logits.cpu().numpy()
    ir, pr = oracle.route_topk(L.astype(np.float64), k)
    ig, pg = idx.cpu().numpy(), p.cpu().numpy()
    assert np.array_equal(ig, ir), f"{what}: routing ids differ"
    assert np.max(np.abs(pg - pr)) <= 1e-6
    xd = x_ref(xb, xdt)
    # router logits against the oracle's fp64 logits
    lr, la = oracle.gemv(mw.router, xd)
    assert_within(L, lr, la, f"{what} logits")
    rows = np.arange(xd.shape[0]) if tokens is None else np.asarray(tokens)
    yr, a = oracle.moe_experts(mw, xd[rows], ig[rows], pg[rows].astype(np.float64), act)
    r = assert_within(y.cpu().numpy()[rows], yr, a, f"{what} y")
    # end to end: ids against the oracle's own fp64 routing, away from near-ties
    ie, _ = oracle.route_topk(lr, k)
    srt = -np.sort(-lr, axis=1)[:, :k + 1]
    gaps = np.min(np.abs(np.diff(srt, axis=1)), axis=1)
    clear = gaps > 1e-6 * la.max(axis=1)
    assert np.array_equal(ig[clear], ie[clear]), f"{what}: end-to-end routing differs"
    return r


TINY = dict(E=6, H=128, I=64, Is=128)


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("T", [1, 2, 5])
def test_tiny_layer(act, xdt, T):
    mw = synth.moe_weights(**TINY, cfg=400, layer=T)
    xb = (synth.x_f16 if xdt == "f16" else synth.x_bf16)(T, TINY["H"], cfg=400, set_id=T)
    check_layer(mw, xb, 3, act, xdt, what=f"tiny T={T} {xdt} act={act}")


def test_odd_shapes():
    mw = synth.moe_weights(E=9, H=192, I=128, Is=320, cfg=401, layer=0)
    xb = synth.x_f16(1, 192, cfg=401, set_id=0)
    check_layer(mw, xb, 9, what="k=E")
    check_layer(mw, xb, 1, what="k=1")


def test_down_row_over_several_rounds():
    # k*I/32 + Is/32 = 260 chunks: more than one round of the down kernel
    mw = synth.moe_weights(E=16, H=128, I=1024, Is=128, cfg=407, layer=0)
    xb = synth.x_f16(1, 128, cfg=407, set_id=0)
    check_layer(mw, xb, 8, what="two rounds")


def test_identical_experts_ignore_routing():
    mw = synth.moe_weights(**TINY, cfg=402, layer=0, identical_experts=True)
    w = dev_moe(mw)
    xb = synth.x_f16(1, TINY["H"], cfg=402, set_id=0)
    x = dev_half(xb)
    i1 = torch.tensor([[0, 1, 2]], dtype=torch.int32, device="cuda")
    p1 = torch.tensor([[0.5, 0.3, 0.2]], dtype=torch.float32, device="cuda")
    i2 = torch.tensor([[5, 3, 4]], dtype=torch.int32, device="cuda")
    p2 = torch.tensor([[0.6, 0.25, 0.15]], dtype=torch.float32, device="cuda")
    ya = qd.qmoe_expert_gemv(w, i1, p1, x).cpu().numpy()
    yb = qd.qmoe_expert_gemv(w, i2, p2, x).cpu().numpy()
    yr, a = oracle.moe_experts(mw, oracle.f16_to_f64(xb), np.array([[2]]), np.array([[1.0]]))
    assert_within(ya, yr, a, "identical a")
    assert_within(yb, yr, a, "identical b")


@pytest.mark.parametrize("E,k,flat", [(1, 1, False), (64, 8, False), (200, 32, False),
                                      (256, 8, False), (128, 8, True), (96, 32, True)])
def test_decode_layer_ranking_in_gateup(E, k, flat):
    """qmoe_layer_decode against router GEMV + qmoe_route_topk + qmoe_expert_gemv
    (flat: every logit ties, so the ids are 0..k-1 and the weights 1/k)."""
    mw = synth.moe_weights(E=E, H=256, I=64, Is=128, cfg=406, layer=E, flat_router=flat)
    w = dev_moe(mw)
    L = qd.lib()
    for s in range(3):
        xb = synth.x_f16(1, 256, cfg=406, set_id=s)
        x = dev_half(xb)
        logits = torch.empty((1, E), dtype=torch.float32, device="cuda")
        idx = torch.full((1, k), -7, dtype=torch.int32, device="cuda")
        p = torch.full((1, k), -7.0, dtype=torch.float32, device="cuda")
        y = torch.full((1, 256), float("nan"), dtype=torch.float32, device="cuda")
        st = w.cstruct()
        need = int(L.qmoe_expert_workspace_bytes(ctypes.byref(st), 1, k))
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        rc = L.qmoe_layer_decode(ctypes.byref(st), w.router_q.data_ptr(), w.router_s.data_ptr(),
                                 w.router_b.data_ptr(), k, x.data_ptr(), 0, logits.data_ptr(),
                                 idx.data_ptr(), p.data_ptr(), y.data_ptr(), ws.data_ptr(), need,
                                 None)
        assert rc == qd.QD_OK, qd.last_error()
        lr = qd.qgemv_affine8(w.router_q, w.router_s, w.router_b, x)
        ir, pr = qd.qmoe_route_topk(lr, k)
        yr = qd.qmoe_expert_gemv(w, ir, pr, x)
        torch.cuda.synchronize()
        assert torch.equal(logits, lr)
        assert torch.equal(idx, ir), (idx, ir)
        assert torch.equal(p, pr)
        assert torch.equal(y, yr)
        if flat:
            assert np.array_equal(idx.cpu().numpy()[0], np.arange(k))
            assert np.allclose(p.cpu().numpy(), 1.0 / k, rtol=1e-6)


def test_flat_router_routes_first_k_evenly():
    mw = synth.moe_weights(**TINY, cfg=403, layer=0, flat_router=True)
    w = dev_moe(mw)
    xb = synth.x_f16(3, TINY["H"], cfg=403, set_id=0)
    logits = qd.qgemv_affine8(w.router_q, w.router_s, w.router_b, dev_half(xb))
    idx, p = qd.qmoe_route_topk(logits, 4)
    torch.cuda.synchronize()
    assert np.all(idx.cpu().numpy() == np.arange(4))
    assert np.allclose(p.cpu().numpy(), 0.25, atol=1e-7)


def test_invalid_expert_ids_contribute_nothing():
    mw = synth.moe_weights(**TINY, cfg=404, layer=0)
    w = dev_moe(mw)
    xb = synth.x_f16(1, TINY["H"], cfg=404, set_id=0)
    idx = torch.tensor([[2, -1, 7]], dtype=torch.int32, device="cuda")
    p = torch.tensor([[0.5, 0.3, 0.2]], dtype=torch.float32, device="cuda")
    y = qd.qmoe_expert_gemv(w, idx, p, dev_half(xb)).cpu().numpy()
    yr, a = oracle.moe_experts(mw, oracle.f16_to_f64(xb), np.array([[2]]), np.array([[0.5]]))
    assert_within(y, yr, a, "invalid ids")


def test_prefill_long_rows():
    # H / 64 = 65 groups: more than the gate+up kernel copies into LDS, so its
    # scales and biases come per lane from global memory (every shorter layer
    # here takes the LDS copy)
    mw = synth.moe_weights(E=4, H=4160, I=64, Is=64, cfg=409, layer=0)
    xb = synth.x_f16(3, 4160, cfg=409, set_id=0)
    check_layer(mw, xb, 2, what="H=4160")


def test_deterministic():
    mw = synth.moe_weights(**TINY, cfg=405, layer=0)
    w = dev_moe(mw)
    xb = synth.x_f16(1, TINY["H"], cfg=405, set_id=0)
    y1 = qd.qmoe_layer(w, dev_half(xb), k=3).clone()
    y2 = qd.qmoe_layer(w, dev_half(xb), k=3).clone()
    assert torch.equal(y1, y2)


# ---------------------------------------------------------------- full size

@pytest.fixture(scope="module")
def full_layer():
    c = synth.CONFIGS["c3_moe_decode"]
    return synth.moe_weights(c["E"], c["H"], c["I"], c["Is"], cfg=3, layer=0)


def test_full_decode_layer(full_layer):
    print("moe decode full layer", flush=True)
    for s in range(4):
        xb = synth.x_f16(1, full_layer.H, cfg=3, set_id=100 + s)
        check_layer(full_layer, xb, 8, what=f"c3 decode token {s}")


def test_full_prefill_chunk(full_layer):
    print("moe prefill chunk T=128", flush=True)
    for xdt in ("bf16", "f16"):
        xb = (synth.x_bf16 if xdt == "bf16" else synth.x_f16)(128, full_layer.H, cfg=4, set_id=7)
        check_layer(full_layer, xb, 8, xdt=xdt, tokens=[0, 1, 31, 64, 127], what=f"c4 moe {xdt}")


# ------------------------------------------------- prefill layer (one call)

@pytest.mark.parametrize("E,H,T,k", [(300, 1088, 37, 5), (128, 2816, 9, 8), (40, 512, 2, 32),
                                     (600, 704, 1, 8)])
def test_prefill_layer_split_router(E, H, T, k):
    """qmoe_layer_prefill: the router split over H (1088 = 17 groups: two splits
    of 9 and 8; 2816: five of 9; 512: one), its slices added by the routing; ids
    and weights equal qmoe_route_topk on the logits it wrote, y equals
    qmoe_expert_gemv, logits and y within the bar of the oracle. E > 256 takes
    the prefill call for a single token too."""
    mw = synth.moe_weights(E=E, H=H, I=64, Is=128, cfg=410, layer=E)
    xb = synth.x_bf16(T, H, cfg=410, set_id=T)
    print(f"prefill layer E={E} H={H} T={T} k={k}", flush=True)
    check_layer(mw, xb, k, xdt="bf16", what=f"prefill E={E} H={H} T={T}")


def test_prefill_layer_deterministic_and_in_bounds():
    mw = synth.moe_weights(E=128, H=2816, I=64, Is=128, cfg=411, layer=0)
    w = dev_moe(mw)
    T, k = 50, 8
    xb = synth.x_f16(T, 2816, cfg=411, set_id=0)
    x = dev_half(xb)
    need = qd.qmoe_workspace_bytes(w, T, k)
    guard = 4096
    wbuf = torch.full((guard + need + guard,), 0x5A, dtype=torch.uint8, device="cuda")
    ybuf = torch.full((guard + T * 2816 + guard,), float("nan"), device="cuda")
    ws = wbuf[guard:guard + need]
    out = ybuf[guard:guard + T * 2816].view(T, 2816)
    y1 = qd.qmoe_layer(w, x, k=k, workspace=ws, out=out).clone()
    y2 = qd.qmoe_layer(w, x, k=k, workspace=ws).clone()
    torch.cuda.synchronize()
    assert (wbuf[:guard] == 0x5A).all() and (wbuf[guard + need:] == 0x5A).all()
    assert torch.isnan(ybuf[:guard]).all() and torch.isnan(ybuf[guard + T * 2816:]).all()
    assert torch.equal(y1, y2)
