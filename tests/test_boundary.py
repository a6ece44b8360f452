"""C-ABI boundary on the CPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments before any HIP call (so these
run without a GPU). Fake device pointers are only passed where validation must
fail; the module is skipped where a GPU is visible."""
import ctypes
import os
import re

import pytest
import torch

import autoround_signsgd_rounding_amd as ar

pytestmark = pytest.mark.skipif(
    torch.cuda.is_available(),
    reason="validation-only tests pass fake device pointers; they run on a host without a GPU")

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "autoround_hip.h")
OK, INV, UNSUP, SHAPE, WS = 0, 1, 2, 3, 4
P = ctypes.c_void_p(0x100000)          # fake, 16-byte aligned, never dereferenced
P_MIS = ctypes.c_void_p(0x100004)      # misaligned
NULL = None


def cfg(**kw):
    c = ar.Config(**kw).c()
    return ctypes.byref(c), c


def test_exports_every_header_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:ar_status|const char\*)\s+(ar_\w+)\s*\(", text, re.M))
    assert declared == set(ar.EXPORTS)
    lib = ctypes.CDLL(ar.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_config_default_and_strings():
    c = ar.ArConfig()
    assert ar.lib.ar_config_default(ctypes.byref(c)) == OK
    assert (c.bits, c.group_size, c.sym, c.nsamples, c.seqlen, c.batch_samples, c.iters) == \
        (4, 128, 0, 128, 2048, 8, 200)
    assert abs(c.lr - 0.005) < 1e-9 and c.minmax_lr < 0 and c.minmax_shrink == 1.0
    assert (c.clip_lo, c.clip_hi) == (0.5, 1.0)
    assert (c.init_scale, c.mse_grid, c.check_finite) == (0, 100, 0)
    assert ar.lib.ar_config_default(None) == INV
    for s in (0, 1, 2, 3, 4, 5, 6, 99):
        assert len(ar.lib.ar_status_string(s)) > 0
    assert b"NaN" in ar.lib.ar_status_string(5)
    assert ar.STATUS[5] == "AR_ERR_NONFINITE"


def test_check_finite_flag_validation():
    """check_finite is 0 or 1; any other value is refused before any HIP call."""
    c, cc = cfg()
    cc.check_finite = 2
    assert rtn(ctypes.byref(cc)) == INV
    cc.check_finite = 1
    assert rtn(ctypes.byref(cc), N=0) == OK


def rtn(c, wdt=1, W=P, N=8, K=128, Wq=NULL, codes=NULL):
    return ar.lib.ar_rtn_quant(c, wdt, W, N, K, codes, NULL, NULL, Wq, NULL)


def test_rtn_validation():
    c, _ = cfg()
    assert rtn(None) == INV
    for bits in (1, 5, 6, 16):
        assert rtn(cfg(bits=bits)[0]) == UNSUP
    assert rtn(cfg(group_size=0)[0]) == INV
    assert rtn(cfg(group_size=-2)[0]) == INV
    assert rtn(cfg(group_size=12)[0], K=96) == UNSUP
    assert rtn(cfg(group_size=64)[0], K=96) == SHAPE
    assert rtn(cfg(group_size=-1)[0], K=100) == SHAPE
    assert rtn(cfg(sym=2)[0]) == INV
    assert rtn(cfg(minmax_shrink=0.0)[0]) == INV
    assert rtn(c, N=-1) == SHAPE
    assert rtn(c, wdt=7) == UNSUP
    assert rtn(c, W=NULL) == INV
    assert rtn(c, W=P_MIS) == INV
    assert rtn(c, Wq=P_MIS) == INV
    assert rtn(c, N=0) == OK          # empty: no-op, nothing launched
    assert rtn(c, K=0) == OK


def test_init_scale_validation():
    assert rtn(cfg(init="mse")[0], N=0) == OK
    c, cc = cfg(init="mse")
    cc.init_scale = 2
    assert rtn(ctypes.byref(cc)) == INV
    assert rtn(cfg(init="mse", mse_grid=0)[0]) == INV
    assert rtn(cfg(init="mse", clip_lo=0.91, clip_hi=0.99, minmax_shrink=0.95, mse_grid=10)[0]) == INV
    assert rtn(cfg(init="mse", clip_lo=0.0)[0]) == INV
    # min-max init ignores the grid (validation only: the workspace query launches nothing)
    assert _ws(cfg(mse_grid=0)[0])[0] == OK
    assert _ws(cfg(init="mse", mse_grid=0)[0])[0] == INV
    f = ar.lib.ar_init_clip
    assert f(cfg(init="mse")[0], 1, P, 8, 128, NULL, P, NULL) == INV
    assert f(cfg(init="mse")[0], 1, P_MIS, 8, 128, P, P, NULL) == INV
    assert f(cfg(init="mse")[0], 1, P, 0, 128, P, P, NULL) == OK


def test_fakequant_validation():
    c, _ = cfg()
    f = ar.lib.ar_fakequant_fwd
    assert f(c, 1, P, 8, 128, NULL, P, P, P, NULL, NULL, NULL, NULL) == INV
    assert f(c, 1, P, 8, 128, P, NULL, P, P, NULL, NULL, NULL, NULL) == INV
    assert f(c, 1, P, 8, 128, P_MIS, P, P, P, NULL, NULL, NULL, NULL) == INV
    assert f(cfg(bits=16)[0], 1, P, 8, 128, P, P, P, P, NULL, NULL, NULL, NULL) == UNSUP
    assert f(c, 1, P, 0, 128, P, P, P, P, NULL, NULL, NULL, NULL) == OK


def _ws(c, N=4096, K=4096, ydt=1):
    out = ctypes.c_size_t()
    st = ar.lib.ar_workspace_size(c, N, K, ydt, ctypes.byref(out))
    return st, out.value


def test_workspace_size():
    c, cc = cfg()
    st, n = _ws(c)
    assert st == OK
    M, Tb, N, K = 128 * 2048, 8 * 2048, 4096, 4096
    # blocked copies of X (two layouts) and Y for every minibatch, the residual
    # and weight operands, gradient, offsets + best offsets, four clip arrays
    big = 2 * M * K * 2 + M * N * 2 + N * Tb * 2 + N * K * 2 + 3 * N * K * 4 + \
        4 * N * (K // 128) * 4
    assert big <= n <= big + 64 * 1024
    assert _ws(cfg(nsamples=10, batch_samples=4)[0])[0] == SHAPE
    assert _ws(cfg(seqlen=3, batch_samples=1, nsamples=2)[0])[0] == SHAPE
    assert _ws(cfg(lr=float("nan"))[0])[0] == INV
    assert _ws(cfg(lr=-1.0)[0])[0] == INV
    assert _ws(cfg(minmax_lr=float("inf"))[0])[0] == INV
    assert _ws(cfg(minmax_shrink=0.3)[0])[0] == INV
    assert _ws(cfg(clip_lo=0.0)[0])[0] == INV
    assert _ws(cfg(clip_lo=0.9, clip_hi=0.8, minmax_shrink=0.85)[0])[0] == INV
    assert _ws(cfg(iters=-1)[0])[0] == INV
    assert _ws(c, ydt=5)[0] == UNSUP
    assert _ws(c, N=0)[0] == SHAPE
    out = ctypes.c_size_t()
    assert ar.lib.ar_step_workspace_size(c, 4096, 4096, 16384, 1, ctypes.byref(out)) == OK
    assert out.value >= 16384 * 4096 * 2 * 3 + 4096 * 4096 * 6
    assert ar.lib.ar_step_workspace_size(c, 4096, 4096, 12, 1, ctypes.byref(out)) == SHAPE
    assert ar.lib.ar_step_workspace_size(c, 4096, 4096, 16, 1, None) == INV


def _state(**kw):
    d = dict(W=0x100000, wdt=1, N=8, K=128, V=0x200000, alpha=0x300000, beta=0x400000,
             best_V=None, best_alpha=None, best_beta=None, best_loss=None)
    d.update(kw)
    return ar.ArState(**d)


def test_tune_step_validation():
    c, _ = cfg()
    need = ctypes.c_size_t()
    assert ar.lib.ar_step_workspace_size(c, 8, 128, 64, 1, ctypes.byref(need)) == OK

    def step(st, Tb=64, loss=P, ws=P, ws_bytes=None, Xb=P):
        nb = need.value if ws_bytes is None else ws_bytes
        return ar.lib.ar_tune_step(c, ctypes.byref(st), Xb, P, 1, Tb, loss, NULL, NULL, NULL, 1,
                                   ws, nb, NULL)
    assert step(_state(), ws_bytes=need.value - 1) == WS
    assert step(_state(best_V=0x500000)) == INV          # best_* all-or-none
    assert step(_state(), loss=NULL) == INV
    assert step(_state(), Xb=NULL) == INV
    assert step(_state(), Tb=60) == SHAPE
    assert step(_state(), Tb=0) == SHAPE
    assert step(_state(V=0x200008)) == INV
    assert step(_state(wdt=3)) == UNSUP
    assert ar.lib.ar_tune_step(c, None, P, P, 1, 64, P, NULL, NULL, NULL, 1, P, need.value,
                               NULL) == INV


def test_tune_linear_validation():
    c, _ = cfg(nsamples=2, seqlen=64, batch_samples=1, iters=3)
    st, need = _ws(c, N=8, K=128)
    assert st == OK

    def run(codes=P, ws_bytes=need, W=P, cref=c):
        return ar.lib.ar_tune_linear(cref, 1, W, 8, 128, P, P, 1, codes, P, P, NULL, NULL, NULL,
                                     NULL, NULL, P, ws_bytes, None, NULL)
    assert run(ws_bytes=need - 1) == WS
    assert run(codes=NULL) == INV
    assert run(W=NULL) == INV
    assert run(cref=cfg(bits=7)[0]) == UNSUP
    assert run(codes=ctypes.c_void_p(0x100004)) == INV                  # codes 8-byte aligned
    assert run(cref=cfg(nsamples=3, seqlen=64, batch_samples=2, iters=3)[0]) == SHAPE
    assert run(cref=cfg(nsamples=2, seqlen=64, batch_samples=1, group_size=48)[0]) == SHAPE
    assert run(cref=cfg(nsamples=2, seqlen=64, batch_samples=1, group_size=12)[0]) == UNSUP
    assert ar.lib.ar_tune_linear(c, 1, P, 8, 128, P_MIS, P, 1, P, P, P, NULL, NULL, NULL, NULL,
                                 NULL, P, need, None, NULL) == INV      # X misaligned


def test_gram_validation():
    """The Gram-form entry points check their arguments as the token form does."""
    c, _ = cfg(nsamples=2, seqlen=64, batch_samples=1, iters=3)
    n = ctypes.c_size_t()
    assert ar.lib.ar_gram_workspace_size(c, 1, 8, 128, 1, ctypes.byref(n)) == OK
    need = n.value
    assert need > 0
    assert ar.lib.ar_gram_workspace_size(c, 1, 8, 128, 1, None) == INV
    assert ar.lib.ar_gram_workspace_size(c, 5, 8, 128, 1, ctypes.byref(n)) == UNSUP
    assert ar.lib.ar_gram_workspace_size(cfg(nsamples=3, seqlen=64, batch_samples=2)[0], 1, 8,
                                         128, 1, ctypes.byref(n)) == SHAPE
    sn = ctypes.c_size_t()
    assert ar.lib.ar_gram_step_workspace_size(c, 1, 8, 128, 64, 1, ctypes.byref(sn)) == OK
    assert ar.lib.ar_gram_step_workspace_size(c, 1, 8, 128, 60, 1, ctypes.byref(sn)) == SHAPE
    assert ar.lib.ar_gram_step_workspace_size(c, 1, 8, 128, 64, 7, ctypes.byref(sn)) == UNSUP

    def step(st, Tb=64, loss=P, ws_bytes=None, Xb=P):
        nb = sn.value if ws_bytes is None else ws_bytes
        return ar.lib.ar_tune_step_gram(c, ctypes.byref(st), Xb, P, 1, Tb, loss, NULL, NULL,
                                        NULL, 1, P, nb, NULL)
    assert step(_state(), ws_bytes=sn.value - 1) == WS
    assert step(_state(best_V=0x500000)) == INV
    assert step(_state(), loss=NULL) == INV
    assert step(_state(), Xb=P_MIS) == INV
    assert step(_state(), Tb=60) == SHAPE
    assert step(_state(wdt=3)) == UNSUP
    assert ar.lib.ar_tune_step_gram(c, None, P, P, 1, 64, P, NULL, NULL, NULL, 1, P, sn.value,
                                    NULL) == INV

    def run(codes=P, ws_bytes=need, X=P, cref=c):
        return ar.lib.ar_tune_linear_gram(cref, 1, P, 8, 128, X, P, 1, codes, P, P, NULL, NULL,
                                          NULL, NULL, NULL, P, ws_bytes, None, NULL)
    assert run(ws_bytes=need - 1) == WS
    assert run(codes=NULL) == INV
    assert run(X=P_MIS) == INV
    assert run(cref=cfg(bits=7, nsamples=2, seqlen=64, batch_samples=1)[0]) == UNSUP


def test_pack_validation():
    pk = ar.lib.ar_pack
    assert pk(5, P, NULL, 8, 128, 1, P, NULL, NULL) == UNSUP
    assert pk(3, P, NULL, 8, 48, 1, P, NULL, NULL) == SHAPE      # 48*3 % 32 != 0
    assert pk(4, P, P, 8, 128, 1, P, NULL, NULL) == INV          # zp without qzeros
    assert pk(3, P, P, 8, 128, 1, P, P, NULL) == SHAPE           # N*3 % 32 != 0
    assert pk(4, NULL, NULL, 8, 128, 1, P, NULL, NULL) == INV
    assert pk(4, P, NULL, 0, 128, 1, P, NULL, NULL) == OK
    assert ar.lib.ar_unpack(16, P, NULL, 8, 128, 1, P, NULL, NULL) == UNSUP


def dq_ws(bits=4, g=128, M=1, N=4096, K=4096):
    n = ctypes.c_size_t(12345)
    st = ar.lib.ar_dequant_gemm_workspace_size(bits, g, M, N, K, ctypes.byref(n))
    return st, n.value


def test_dequant_workspace_validation():
    assert dq_ws(bits=5)[0] == UNSUP
    assert dq_ws(g=0)[0] == INV
    assert dq_ws(g=12)[0] == UNSUP            # groups must be a multiple of 8
    assert dq_ws(g=64, K=96)[0] == SHAPE      # K % group
    assert dq_ws(K=12)[0] == SHAPE            # K % 8
    assert dq_ws(M=0) == (OK, 0)
    assert ar.lib.ar_dequant_gemm_workspace_size(4, 128, 1, 64, 128, None) == INV
    for M in (1, 16, 17, 300):
        st, n = dq_ws(M=M)
        assert st == OK and n > 0 and n % 256 == 0
    # small M: one float32 partial per (slice, row, column), a whole number of slices
    st1, n1 = dq_ws(M=1, N=4096)
    assert n1 % (4096 * 4) == 0 and n1 // (4096 * 4) >= 1
    st2, n2 = dq_ws(M=2, N=4096)
    assert n2 % (2 * 4096 * 4) == 0


def dq(X=P, M=1, K=4096, qw=P, qz=P, sc=P, N=4096, Y=P, ydt=0, ws=P, wsb=1 << 30, g=128, bits=4):
    return ar.lib.ar_dequant_gemm(bits, g, X, M, K, qw, qz, sc, N, Y, ydt, ws, wsb, NULL)


def test_dequant_validation():
    assert dq(X=NULL) == INV
    assert dq(Y=NULL) == INV
    assert dq(qw=NULL) == INV
    assert dq(X=P_MIS) == INV
    assert dq(ydt=7) == UNSUP
    assert dq(bits=6) == UNSUP
    assert dq(g=-2) == INV
    assert dq(wsb=16) == WS
    assert dq(N=30, qz=P, bits=3) == SHAPE     # zero-point words need N*bits % 32 == 0
    assert dq(M=0) == OK and dq(N=0) == OK     # no-ops


def test_attention_validation():
    d = ar.block_dims(256, 4, 512, 64, 2)
    A = ar.lib.ar_attention
    assert A(None, P, P, P, P, NULL) == INV
    assert A(ctypes.byref(d), NULL, P, P, P, NULL) == INV
    assert A(ctypes.byref(d), P, P, P_MIS, P, NULL) == INV
    bad = ar.block_dims(384, 4, 512, 64, 2)    # head dim 96
    assert A(ctypes.byref(bad), P, P, P, P, NULL) == UNSUP
    assert A(ctypes.byref(ar.block_dims(256, 3, 512, 64, 2)), P, P, P, P, NULL) == SHAPE
