"""GPU parity of qattn_decode (exact split decode attention over circular and
linear fp16 KV) against the fp64 oracle.

Source: jeff.news/article/5193 (TurboFieldfare), internals section: circular
KV storage for sliding-window layers, linear for full attention, exact
decode attention. Bar per output: |out_gpu - out_ref| <= 1e-4 * sum_j p_j
|v_j| + 1e-6 (the value-weighted analogue of the GEMV rule); the cache
update is checked bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_within, dev_half, host_bits

qd = pytest.importorskip("affine_quantized_gemv_qgemv_amd")

pytestmark = pytest.mark.gpu


def f64(bits):
    return oracle.f16_to_f64(bits)


def run_case(Hq, Hkv, D, cap, window, pos, seed, scale_q=1.0):
    t = synth.attn_inputs(Hq, Hkv, D, cap, cfg=600, set_id=seed, scale_q=scale_q)
    scale = D ** -0.5
    dev = {k: dev_half(v) for k, v in t.items()}
    y = qd.qattn_decode(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"], pos,
                        window, scale)
    torch.cuda.synchronize()
    ref, a = oracle.attn_decode(f64(t["q"]), f64(t["k_new"]), f64(t["v_new"]), f64(t["k_cache"]),
                                f64(t["v_cache"]), window, pos, scale)
    # the caches afterwards: the inputs with the token's slot replaced, bit for bit
    slot = pos % window if window else pos
    kc, vc = t["k_cache"].copy(), t["v_cache"].copy()
    kc[:, slot], vc[:, slot] = t["k_new"], t["v_new"]
    assert np.array_equal(host_bits(dev["k_cache"]), kc)
    assert np.array_equal(host_bits(dev["v_cache"]), vc)
    return y.cpu().numpy(), ref, a


CASES = [
    # Hq, Hkv, D, cap, window, pos
    (16, 8, 128, 4096, 0, 0), (16, 8, 128, 4096, 0, 1), (16, 8, 128, 4096, 0, 100),
    (16, 8, 128, 4096, 0, 4095), (16, 8, 128, 1024, 1024, 5), (16, 8, 128, 1024, 1024, 1023),
    (16, 8, 128, 1024, 1024, 1024), (16, 8, 128, 1024, 1024, 3000), (8, 8, 64, 300, 0, 299),
    (32, 4, 64, 777, 777, 2000), (4, 1, 256, 200, 0, 150), (8, 2, 256, 513, 513, 513),
    (16, 2, 128, 48, 0, 17), (2, 1, 128, 1, 1, 9),
    # ragged split counts with one query head per key/value head
    (4, 4, 256, 2049, 0, 2047), (4, 4, 256, 2049, 0, 2048), (8, 4, 64, 2048, 2048, 5000),
]


@pytest.mark.parametrize("Hq,Hkv,D,cap,window,pos", CASES)
def test_decode_attention(Hq, Hkv, D, cap, window, pos):
    print(f"attn Hq={Hq} Hkv={Hkv} D={D} cap={cap} window={window} pos={pos}", flush=True)
    y, ref, a = run_case(Hq, Hkv, D, cap, window, pos, seed=Hq + D + cap + pos)
    assert_within(y, ref, a, f"Hq={Hq} Hkv={Hkv} D={D} cap={cap} window={window} pos={pos}")


def test_sharp_softmax_and_large_scores():
    # scores in the hundreds: the running max keeps every exponent finite
    y, ref, a = run_case(16, 8, 128, 2048, 0, 2047, seed=7, scale_q=40.0)
    assert np.all(np.isfinite(y))
    assert_within(y, ref, a, "sharp")


def test_first_token_is_its_value_exactly():
    Hq, Hkv, D, cap = 16, 8, 128, 64
    t = synth.attn_inputs(Hq, Hkv, D, cap, cfg=601, set_id=0)
    dev = {k: dev_half(v) for k, v in t.items()}
    y = qd.qattn_decode(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"], 0, 0)
    torch.cuda.synchronize()
    expect = np.repeat(f64(t["v_new"]), Hq // Hkv, axis=0)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), expect)


def test_successive_steps_fill_a_circular_cache():
    # 40 decode steps through a window of 16: each step's output matches the
    # oracle run on the cache as the previous steps left it
    Hq, Hkv, D, W = 8, 4, 64, 16
    rng = np.random.default_rng(3)
    kc = np.zeros((Hkv, W, D), np.float16)
    vc = np.zeros((Hkv, W, D), np.float16)
    dk, dv = dev_half(kc.view(np.uint16)), dev_half(vc.view(np.uint16))
    for pos in range(40):
        q = rng.standard_normal((Hq, D)).astype(np.float16)
        kn = rng.standard_normal((Hkv, D)).astype(np.float16)
        vn = rng.standard_normal((Hkv, D)).astype(np.float16)
        y = qd.qattn_decode(dev_half(q.view(np.uint16)), dev_half(kn.view(np.uint16)),
                            dev_half(vn.view(np.uint16)), dk, dv, pos, W, 0.125)
        torch.cuda.synchronize()
        ref, a = oracle.attn_decode(q.astype(np.float64), kn.astype(np.float64), vn.astype(np.float64),
                                    kc.astype(np.float64), vc.astype(np.float64), W, pos, 0.125)
        assert_within(y.cpu().numpy(), ref, a, f"pos {pos}")
        kc[:, pos % W], vc[:, pos % W] = kn, vn
        assert np.array_equal(host_bits(dk), kc.view(np.uint16))


def test_deterministic_and_in_bounds():
    Hq, Hkv, D, cap = 16, 8, 128, 4096
    t = synth.attn_inputs(Hq, Hkv, D, cap, cfg=602, set_id=0)
    guard = 1024
    buf = torch.full((guard + Hq * D + guard,), float("nan"), device="cuda")
    out = buf[guard:guard + Hq * D].view(Hq, D)
    outs = []
    for rep in range(2):
        dev = {k: dev_half(v) for k, v in t.items()}
        qd.qattn_decode(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"], 3000, 0,
                        out=out)
        torch.cuda.synchronize()
        outs.append(out.clone())
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + Hq * D:]).all()
    assert torch.equal(outs[0], outs[1])


def test_one_workspace_across_calls_with_different_split_counts():
    # one workspace (sized for the full cache, left holding the previous
    # call's partial sums) serves calls whose split counts differ
    Hq, Hkv, D, cap = 16, 8, 128, 4096
    t = synth.attn_inputs(Hq, Hkv, D, cap, cfg=603, set_id=0)
    ws = torch.full((qd.qattn_workspace_bytes(Hq, Hkv, D, cap),), 255, dtype=torch.uint8, device="cuda")
    for pos in (4095, 0, 37, 1000, 15, 4095, 2048):
        dev = {k: dev_half(v) for k, v in t.items()}
        y = qd.qattn_decode(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"], pos, 0,
                            workspace=ws)
        torch.cuda.synchronize()
        ref, a = oracle.attn_decode(f64(t["q"]), f64(t["k_new"]), f64(t["v_new"]), f64(t["k_cache"]),
                                    f64(t["v_cache"]), 0, pos, D ** -0.5)
        assert_within(y.cpu().numpy(), ref, a, f"pos {pos}")


@pytest.mark.parametrize("Hq,Hkv,D,cap,pos", [(16, 8, 128, 2049, 2047), (32, 16, 64, 1025, 1023),
                                             (8, 4, 128, 4097, 4095), (16, 8, 128, 2049, 2048)])
def test_workspace_guard_band_at_ragged_split_counts(Hq, Hkv, D, cap, pos):
    # occupancies just below a multiple of the split size take more splits
    # than the full cache: the workspace (sized for the cache) must still
    # hold them, and nothing past it may be written
    print(f"attn guard Hq={Hq} Hkv={Hkv} D={D} cap={cap} pos={pos}", flush=True)
    t = synth.attn_inputs(Hq, Hkv, D, cap, cfg=604, set_id=cap + pos)
    need = qd.qattn_workspace_bytes(Hq, Hkv, D, cap)
    guard = 1 << 16
    buf = torch.full((need + guard,), 0x7F, dtype=torch.uint8, device="cuda")
    dev = {k: dev_half(v) for k, v in t.items()}
    y = qd.qattn_decode(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"], pos, 0,
                        workspace=buf[:need])
    torch.cuda.synchronize()
    assert bool((buf[need:] == 0x7F).all()), "write past the workspace"
    ref, a = oracle.attn_decode(f64(t["q"]), f64(t["k_new"]), f64(t["v_new"]), f64(t["k_cache"]),
                                f64(t["v_cache"]), 0, pos, D ** -0.5)
    assert_within(y.cpu().numpy(), ref, a, f"guard cap={cap} pos={pos}")
