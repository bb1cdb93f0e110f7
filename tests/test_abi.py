"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad arguments with the documented status before
touching the HIP runtime (errors as values, as the uzu walk-through at
fiv.co.kr/repos/uzu-deep-dive.html sections 4-4 and 7-1 describes)."""
import ctypes
import os
import re

import pytest

import affine_quantized_gemv_qgemv_amd as qd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qdecode.h")

A = 1 << 20      # a fake, 16-byte aligned "device" address (never dereferenced)
MIS = A + 4      # misaligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for fn in ("qgemv_affine4", "qgemv_affine8", "qmoe_route_topk", "qmoe_expert_gemv",
               "qgemm_affine4_chunk"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    L = qd.lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing
    assert set(qd.EXPORTS) <= set(declared_functions())


def test_status_strings():
    assert qd.status_name(qd.QD_OK) == "QD_OK"
    assert qd.status_name(qd.QD_ERR_MISALIGNED) == "QD_ERR_MISALIGNED"
    assert qd.status_name(99) == "QD_UNKNOWN_STATUS"


def gemv(fn="qgemv_affine4", wq=A, s=A, b=A, x=A, dt=0, y=A, N=16, K=128, batch=1, g=64):
    return getattr(qd.lib(), fn)(wq, s, b, x, dt, y, N, K, batch, g, None)


@pytest.mark.parametrize("fn", ["qgemv_affine4", "qgemv_affine8"])
def test_gemv_argument_errors(fn):
    E = qd
    assert gemv(fn, g=32) == E.QD_ERR_UNSUPPORTED
    assert "group_size" in qd.last_error()
    assert gemv(fn, K=100) == E.QD_ERR_INVALID_ARGUMENT
    assert gemv(fn, K=0) == E.QD_ERR_INVALID_ARGUMENT
    assert gemv(fn, N=0) == E.QD_ERR_INVALID_ARGUMENT
    assert gemv(fn, batch=0) == E.QD_ERR_INVALID_ARGUMENT
    assert gemv(fn, batch=129) == E.QD_ERR_INVALID_ARGUMENT
    assert gemv(fn, wq=None) == E.QD_ERR_INVALID_ARGUMENT
    assert "wq" in qd.last_error()
    assert gemv(fn, y=None) == E.QD_ERR_INVALID_ARGUMENT
    assert gemv(fn, x=MIS) == E.QD_ERR_MISALIGNED
    assert gemv(fn, s=MIS) == E.QD_ERR_MISALIGNED
    assert gemv(fn, dt=7) == E.QD_ERR_UNSUPPORTED
    # rows are addressed with 32-bit offsets: K is capped at 2^22
    assert gemv(fn, K=(1 << 22) + 64) == E.QD_ERR_UNSUPPORTED
    assert "4194304" in qd.last_error()


def test_affine4_batch_limit_is_eight():
    assert gemv("qgemv_affine4", batch=9) == qd.QD_ERR_INVALID_ARGUMENT


def mirai_l(wq=A, s=A, x=A, dt=0, y=A, N=16, K=128, batch=1, g=64):
    return qd.lib().qgemv_mirai_l(wq, s, x, dt, y, N, K, batch, g, None)


def test_mirai_argument_errors():
    E = qd
    # Mirai-M: the third pointer is the zero-point array
    assert gemv("qgemv_mirai_m", g=128) == E.QD_ERR_UNSUPPORTED
    assert gemv("qgemv_mirai_m", K=96) == E.QD_ERR_INVALID_ARGUMENT
    assert gemv("qgemv_mirai_m", batch=9) == E.QD_ERR_INVALID_ARGUMENT
    assert gemv("qgemv_mirai_m", b=None) == E.QD_ERR_INVALID_ARGUMENT
    assert "zeros" in qd.last_error()
    assert gemv("qgemv_mirai_m", b=MIS) == E.QD_ERR_MISALIGNED
    assert gemv("qgemv_mirai_m", s=None) == E.QD_ERR_INVALID_ARGUMENT
    assert gemv("qgemv_mirai_m", dt=2) == E.QD_ERR_UNSUPPORTED
    # Mirai-L
    assert mirai_l(g=32) == E.QD_ERR_UNSUPPORTED
    assert mirai_l(N=0) == E.QD_ERR_INVALID_ARGUMENT
    assert mirai_l(batch=0) == E.QD_ERR_INVALID_ARGUMENT
    assert mirai_l(batch=9) == E.QD_ERR_INVALID_ARGUMENT
    assert mirai_l(wq=None) == E.QD_ERR_INVALID_ARGUMENT
    assert mirai_l(x=MIS) == E.QD_ERR_MISALIGNED
    assert mirai_l(dt=5) == E.QD_ERR_UNSUPPORTED


def test_route_argument_errors():
    L = qd.lib()
    assert L.qmoe_route_topk(A, 0, 128, 8, A, A, None) == qd.QD_ERR_INVALID_ARGUMENT
    assert L.qmoe_route_topk(A, 1, 0, 8, A, A, None) == qd.QD_ERR_INVALID_ARGUMENT
    assert L.qmoe_route_topk(A, 1, 4, 8, A, A, None) == qd.QD_ERR_INVALID_ARGUMENT
    assert L.qmoe_route_topk(A, 1, 2048, 8, A, A, None) == qd.QD_ERR_INVALID_ARGUMENT
    assert L.qmoe_route_topk(A, 1, 128, 33, A, A, None) == qd.QD_ERR_INVALID_ARGUMENT
    assert L.qmoe_route_topk(None, 1, 128, 8, A, A, None) == qd.QD_ERR_INVALID_ARGUMENT
    assert L.qmoe_route_topk(A, 1, 128, 8, MIS, A, None) == qd.QD_ERR_MISALIGNED


def moe_struct(**kw):
    f = dict(E=128, H=2816, I=704, I_shared=2112, group_size=64, act=0)
    f.update({n: A for n in ("gu_q", "dn_q", "sgu_q", "sdn_q", "gu_s", "gu_b", "dn_s", "dn_b",
                            "sgu_s", "sgu_b", "sdn_s", "sdn_b")})
    f.update(kw)
    return qd.MoeWeightsC(**f)


def moe_call(st, T=1, k=8, ws=A, ws_bytes=1 << 30, x=A, dt=0):
    return qd.lib().qmoe_expert_gemv(ctypes.byref(st), A, A, T, k, x, dt, A, ws, ws_bytes, None)


def test_prefill_layer_argument_errors():
    L = qd.lib()
    st = moe_struct()
    need = L.qmoe_layer_prefill_workspace_bytes(ctypes.byref(st), 128, 8)
    # the expert block's workspace plus the router's split slices (at least one T x E slice)
    assert need >= L.qmoe_expert_workspace_bytes(ctypes.byref(st), 128, 8) + 128 * 128 * 4
    assert L.qmoe_layer_prefill_workspace_bytes(ctypes.byref(st), 0, 8) == 0
    assert L.qmoe_layer_prefill_workspace_bytes(ctypes.byref(st), 129, 8) == 0
    assert L.qmoe_layer_prefill_workspace_bytes(None, 16, 8) == 0

    def f(w=st, rq=A, k=8, T=128, x=A, dt=1, lg=A, ws=A, wsb=need):
        return L.qmoe_layer_prefill(ctypes.byref(w) if w is not None else None, rq, A, A, k, T, x, dt, lg,
                                    A, A, A, ws, wsb, None)

    assert f(w=None) == qd.QD_ERR_INVALID_ARGUMENT
    assert f(T=0) == qd.QD_ERR_INVALID_ARGUMENT
    assert f(T=129) == qd.QD_ERR_INVALID_ARGUMENT
    assert f(k=0) == qd.QD_ERR_INVALID_ARGUMENT
    assert f(k=33) == qd.QD_ERR_INVALID_ARGUMENT
    assert f(w=moe_struct(E=1025)) == qd.QD_ERR_UNSUPPORTED
    assert f(dt=2) == qd.QD_ERR_UNSUPPORTED
    assert f(rq=None) == qd.QD_ERR_INVALID_ARGUMENT
    assert f(lg=None) == qd.QD_ERR_INVALID_ARGUMENT
    assert f(x=MIS) == qd.QD_ERR_MISALIGNED
    assert f(ws=None) == qd.QD_ERR_WORKSPACE
    assert f(wsb=need - 1) == qd.QD_ERR_WORKSPACE
    assert f(ws=MIS) == qd.QD_ERR_MISALIGNED


def test_moe_argument_errors():
    L = qd.lib()
    assert L.qmoe_expert_gemv(None, A, A, 1, 8, A, 0, A, A, 1 << 30, None) == qd.QD_ERR_INVALID_ARGUMENT
    assert moe_call(moe_struct(group_size=128)) == qd.QD_ERR_UNSUPPORTED
    assert moe_call(moe_struct(H=100)) == qd.QD_ERR_INVALID_ARGUMENT
    assert moe_call(moe_struct(act=5)) == qd.QD_ERR_UNSUPPORTED
    assert moe_call(moe_struct(dn_s=None)) == qd.QD_ERR_INVALID_ARGUMENT
    assert moe_call(moe_struct(sgu_q=MIS)) == qd.QD_ERR_MISALIGNED
    assert moe_call(moe_struct(), T=0) == qd.QD_ERR_INVALID_ARGUMENT
    assert moe_call(moe_struct(), T=129) == qd.QD_ERR_INVALID_ARGUMENT
    assert moe_call(moe_struct(), k=0) == qd.QD_ERR_INVALID_ARGUMENT
    assert moe_call(moe_struct(E=4), k=8) == qd.QD_ERR_INVALID_ARGUMENT
    assert moe_call(moe_struct(), ws=None) == qd.QD_ERR_WORKSPACE
    assert moe_call(moe_struct(), ws_bytes=16) == qd.QD_ERR_WORKSPACE
    assert moe_call(moe_struct(), ws=MIS) == qd.QD_ERR_MISALIGNED
    assert moe_call(moe_struct(), dt=3) == qd.QD_ERR_UNSUPPORTED


def layer_call(st, k=8, ws=A, ws_bytes=1 << 30, x=A, dt=0, rq=A, logits=A):
    return qd.lib().qmoe_layer_decode(ctypes.byref(st), rq, A, A, k, x, dt, logits, A, A, A, ws,
                                      ws_bytes, None)


def test_moe_layer_decode_argument_errors():
    L = qd.lib()
    assert L.qmoe_layer_decode(None, A, A, A, 8, A, 0, A, A, A, A, A, 1 << 30,
                               None) == qd.QD_ERR_INVALID_ARGUMENT
    assert layer_call(moe_struct(group_size=128)) == qd.QD_ERR_UNSUPPORTED
    assert layer_call(moe_struct(E=257)) == qd.QD_ERR_UNSUPPORTED
    assert layer_call(moe_struct(), k=0) == qd.QD_ERR_INVALID_ARGUMENT
    assert layer_call(moe_struct(), k=33) == qd.QD_ERR_INVALID_ARGUMENT
    assert layer_call(moe_struct(E=4), k=8) == qd.QD_ERR_INVALID_ARGUMENT
    assert layer_call(moe_struct(), dt=2) == qd.QD_ERR_UNSUPPORTED
    assert layer_call(moe_struct(), rq=None) == qd.QD_ERR_INVALID_ARGUMENT
    assert layer_call(moe_struct(), logits=MIS) == qd.QD_ERR_MISALIGNED
    assert layer_call(moe_struct(), ws=None) == qd.QD_ERR_WORKSPACE
    assert layer_call(moe_struct(), ws_bytes=16) == qd.QD_ERR_WORKSPACE
    assert layer_call(moe_struct(), ws=MIS) == qd.QD_ERR_MISALIGNED


def test_moe_workspace_size_grows_with_tokens():
    st = moe_struct()
    L = qd.lib()
    w1 = L.qmoe_expert_workspace_bytes(ctypes.byref(st), 1, 8)
    w128 = L.qmoe_expert_workspace_bytes(ctypes.byref(st), 128, 8)
    assert 0 < w1 < w128
    assert L.qmoe_expert_workspace_bytes(None, 1, 8) == 0


def test_chunk_argument_errors():
    L = qd.lib()
    f = lambda **kw: L.qgemm_affine4_chunk(kw.get("wq", A), A, A, kw.get("x", A), A, kw.get("M", 128),
                                           kw.get("N", 256), kw.get("K", 256), kw.get("g", 64),
                                           kw.get("w", None), kw.get("wsb", 0), None)
    assert f(M=0) == qd.QD_ERR_INVALID_ARGUMENT
    assert f(M=129) == qd.QD_ERR_INVALID_ARGUMENT
    assert f(K=96) == qd.QD_ERR_INVALID_ARGUMENT
    assert f(K=(1 << 22) + 64) == qd.QD_ERR_UNSUPPORTED
    assert f(g=128) == qd.QD_ERR_UNSUPPORTED
    assert f(wq=None) == qd.QD_ERR_INVALID_ARGUMENT
    assert f(x=MIS) == qd.QD_ERR_MISALIGNED
    # the prefill down projection (64 column tiles) splits K, with the verification GEMM's plan
    ws = qd.chunk_workspace_bytes(128, 4096, 14336)
    assert ws > 0 and ws == qd.verify_workspace_bytes(128, 4096, 14336)
    assert qd.chunk_workspace_bytes(128, 14336, 4096) == 0 and qd.chunk_workspace_bytes(129, 4096, 14336) == 0
    assert f(N=4096, K=14336) == qd.QD_ERR_WORKSPACE
    assert f(N=4096, K=14336, w=A, wsb=ws - 1) == qd.QD_ERR_WORKSPACE
    assert f(N=4096, K=14336, w=MIS, wsb=ws) == qd.QD_ERR_MISALIGNED


def test_mirai_rht_argument_errors():
    E = qd
    L = qd.lib()

    def m(wq=A, s=A, z=A, sg=A, g=A, eps=1e-6, x=A, dt=0, y=A, N=16, K=128, batch=1, gs=64):
        return L.qgemv_mirai_m_rht(wq, s, z, sg, g, eps, x, dt, y, N, K, batch, gs, None)

    def l(wq=A, s=A, sg=A, g=A, eps=1e-6, x=A, dt=1, y=A, N=16, K=128, batch=1, gs=64):
        return L.qgemv_mirai_l_rht(wq, s, sg, g, eps, x, dt, y, N, K, batch, gs, None)

    assert m(eps=-1.0) == E.QD_ERR_INVALID_ARGUMENT
    assert "eps" in qd.last_error()
    assert m(eps=float("nan")) == E.QD_ERR_INVALID_ARGUMENT
    assert m(eps=float("inf")) == E.QD_ERR_INVALID_ARGUMENT
    assert m(sg=MIS) == E.QD_ERR_MISALIGNED
    assert m(g=MIS) == E.QD_ERR_MISALIGNED
    assert m(z=None) == E.QD_ERR_INVALID_ARGUMENT
    assert m(batch=9) == E.QD_ERR_INVALID_ARGUMENT
    assert m(K=32) == E.QD_ERR_INVALID_ARGUMENT
    assert m(gs=32) == E.QD_ERR_UNSUPPORTED
    assert l(eps=-0.5) == E.QD_ERR_INVALID_ARGUMENT
    assert l(g=MIS) == E.QD_ERR_MISALIGNED
    assert l(dt=3) == E.QD_ERR_UNSUPPORTED
    assert l(y=None) == E.QD_ERR_INVALID_ARGUMENT


def test_verify_argument_errors():
    E = qd
    L = qd.lib()

    def v(wq=A, s=A, b=A, x=A, dt=0, y=A, M=16, N=16, K=128, gs=64, w=None, wsb=0):
        return L.qgemm_affine4_verify(wq, s, b, x, dt, y, M, N, K, gs, w, wsb, None)

    assert v(M=0) == E.QD_ERR_INVALID_ARGUMENT
    assert v(M=129) == E.QD_ERR_INVALID_ARGUMENT
    assert v(K=100) == E.QD_ERR_INVALID_ARGUMENT
    assert v(gs=128) == E.QD_ERR_UNSUPPORTED
    assert v(dt=2) == E.QD_ERR_UNSUPPORTED
    assert v(b=None) == E.QD_ERR_INVALID_ARGUMENT
    assert v(x=MIS) == E.QD_ERR_MISALIGNED
    # a down projection (N = 4096, 64 column tiles) splits K; a wide matrix does not
    ws = qd.verify_workspace_bytes(32, 4096, 14336)
    assert ws > 0 and ws % (32 * 4096 * 4) == 0
    assert qd.verify_workspace_bytes(32, 28672, 4096) == 0
    assert qd.verify_workspace_bytes(0, 4096, 14336) == 0 and qd.verify_workspace_bytes(129, 4096, 14336) == 0
    assert qd.verify_workspace_bytes(16, 4096, 100) == 0
    assert v(M=32, N=4096, K=14336) == E.QD_ERR_WORKSPACE
    assert v(M=32, N=4096, K=14336, w=A, wsb=ws - 1) == E.QD_ERR_WORKSPACE
    assert v(M=32, N=4096, K=14336, w=MIS, wsb=ws) == E.QD_ERR_MISALIGNED


def test_verify_split_plan_covers_k_once():
    # every split shape: at least two slices of at least 16 groups each, and the
    # workspace holds splits x M x N fp32
    for M in (1, 16, 32, 33, 64, 65, 128):
        for N in (1, 64, 100, 4096, 8192):
            for K in (64, 1024, 2048, 4096, 14336, 1 << 22):
                ws = qd.verify_workspace_bytes(M, N, K)
                if ws == 0:
                    continue
                splits = ws // (4 * M * N)
                assert ws == splits * 4 * M * N and 2 <= splits
                assert splits <= (K // 64) // 16


def test_verify_i8_argument_errors():
    E = qd
    L = qd.lib()
    ws = qd.verify_i8_workspace_bytes(32, 4096)
    assert ws >= 32 * 4096 + 64 * 32 * 4 + 32 * 4
    assert qd.verify_i8_workspace_bytes(33, 4096) == 0 and qd.verify_i8_workspace_bytes(1, 100) == 0
    assert qd.verify_i8_workspace_bytes(16, 4096) < ws

    def v(wq=A, s=A, b=A, x=A, y=A, M=32, N=16, K=4096, gs=64, w=A, wsb=ws):
        return L.qgemm_affine4_verify_i8(wq, s, b, x, y, M, N, K, gs, w, wsb, None)

    assert v(M=0) == E.QD_ERR_INVALID_ARGUMENT
    assert v(M=33) == E.QD_ERR_INVALID_ARGUMENT
    assert v(K=100) == E.QD_ERR_INVALID_ARGUMENT
    assert v(N=0) == E.QD_ERR_INVALID_ARGUMENT
    assert v(gs=32) == E.QD_ERR_UNSUPPORTED
    assert v(s=None) == E.QD_ERR_INVALID_ARGUMENT
    assert v(x=MIS) == E.QD_ERR_MISALIGNED
    assert v(w=None) == E.QD_ERR_WORKSPACE
    assert v(w=MIS) == E.QD_ERR_MISALIGNED
    assert v(wsb=ws - 1) == E.QD_ERR_WORKSPACE
    assert "workspace" in qd.last_error()


def test_attention_argument_errors():
    E = qd
    L = qd.lib()
    ws = qd.qattn_workspace_bytes(16, 8, 128, 4096)
    assert ws > 0

    def at(q=A, kn=A, vn=A, kc=A, vc=A, Hq=16, Hkv=8, D=128, cap=4096, window=0, pos=10,
           scale=0.088, out=A, w=A, wsb=ws):
        return L.qattn_decode(q, kn, vn, kc, vc, Hq, Hkv, D, cap, window, pos, scale, out, w, wsb, None)

    assert at(D=96) == E.QD_ERR_UNSUPPORTED
    assert at(Hq=12) == E.QD_ERR_INVALID_ARGUMENT     # 12 is not a multiple of 8
    assert "multiple" in qd.last_error()
    assert at(Hq=24, Hkv=8) == E.QD_ERR_UNSUPPORTED   # groups of 3
    assert at(pos=4096) == E.QD_ERR_INVALID_ARGUMENT
    assert at(pos=-1) == E.QD_ERR_INVALID_ARGUMENT
    assert at(window=1024) == E.QD_ERR_INVALID_ARGUMENT   # circular storage needs cap == window
    assert at(scale=float("nan")) == E.QD_ERR_INVALID_ARGUMENT
    assert at(kc=None) == E.QD_ERR_INVALID_ARGUMENT
    assert at(q=MIS) == E.QD_ERR_MISALIGNED
    assert at(w=None) == E.QD_ERR_WORKSPACE
    assert at(wsb=ws - 1) == E.QD_ERR_WORKSPACE
    # circular storage accepts any position
    assert qd.qattn_workspace_bytes(16, 8, 128, 1024) <= ws


def _attn_splits(n, Hkv, cus=256, maxsplit=256):
    """The split rule of the decode-attention launch, written out: about two
    workgroups per CU over the key/value heads, at most 256 splits, splits of
    a multiple of 32 rows."""
    want = max(1, min((2 * cus + Hkv - 1) // Hkv, maxsplit, (n + 31) // 32))
    chunk = -(-n // want)
    chunk = (chunk + 31) // 32 * 32
    return -(-n // chunk)


@pytest.mark.parametrize("Hkv", [1, 2, 4, 8, 16])
def test_attention_workspace_covers_every_position(Hkv):
    # the split count is not monotonic in the occupancy n (the chunk is
    # rounded up to 32 rows), so the workspace for a cache of `cap` slots
    # must cover the largest split count of any n <= cap
    Hq, D = 2 * Hkv, 128
    per_split = Hq * (D + 2) * 4
    caps = sorted(set(list(range(1, 4200, 7)) + [1025, 2049, 4097, 8193, 16385, 20000]))
    worst = 0
    for cap in caps:
        ws = qd.qattn_workspace_bytes(Hq, Hkv, D, cap)
        need = max(_attn_splits(n, Hkv) for n in range(max(1, cap - 1200), cap + 1))
        worst = max(worst, need)
        assert ws >= need * per_split, (cap, ws, need)
        # a larger cache never needs less
        assert ws >= qd.qattn_workspace_bytes(Hq, Hkv, D, max(1, cap - 1))
    # the case that overran the old cap-based size (Hkv 8, cap 2049, n 2048)
    if Hkv == 8:
        assert _attn_splits(2048, 8) > _attn_splits(2049, 8)
        assert qd.qattn_workspace_bytes(16, 8, 128, 2049) >= _attn_splits(2048, 8) * 16 * 130 * 4


def test_moe_layer_decode_noalloc_argument_errors():
    # the allocation-free decode layer: same checks as qmoe_layer_decode, and
    # a layer whose activations exceed the library's 4 MiB scratch is refused
    # before any launch
    L = qd.lib()

    def call(st, k=8, dt=0, rq=A, logits=A):
        return L.qmoe_layer_decode_noalloc(ctypes.byref(st), rq, A, A, k, A, dt, logits, A, A, A, None)

    assert L.qmoe_layer_decode_noalloc(None, A, A, A, 8, A, 0, A, A, A, A, None) == qd.QD_ERR_INVALID_ARGUMENT
    assert call(moe_struct(group_size=128)) == qd.QD_ERR_UNSUPPORTED
    assert call(moe_struct(E=257)) == qd.QD_ERR_UNSUPPORTED
    assert call(moe_struct(), k=0) == qd.QD_ERR_INVALID_ARGUMENT
    assert call(moe_struct(), dt=2) == qd.QD_ERR_UNSUPPORTED
    assert call(moe_struct(), rq=None) == qd.QD_ERR_INVALID_ARGUMENT
    assert call(moe_struct(), logits=MIS) == qd.QD_ERR_MISALIGNED
    # 32 slots of I = 32768 plus the shared expert: 4 MiB + 4 KiB of activations
    assert call(moe_struct(E=64, I=32768, I_shared=1024), k=32) == qd.QD_ERR_WORKSPACE
    assert "scratch" in qd.last_error()
