"""Python binding of libautoround_hip.so (AutoRound per-Linear tuning on gfx950).

Argument marshalling only: torch tensors provide device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
Importing this package loads the library and fails loudly if it is missing.
Entry points mirror include/autoround_hip.h.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libautoround_hip.so")

AR_F32, AR_BF16 = 0, 1
SUPPORTED_BITS = (2, 3, 4, 8)

STATUS = {
    0: "AR_OK", 1: "AR_ERR_INVALID_ARG", 2: "AR_ERR_UNSUPPORTED", 3: "AR_ERR_SHAPE",
    4: "AR_ERR_WORKSPACE", 5: "AR_ERR_NONFINITE", 6: "AR_ERR_HIP",
}

# every symbol declared in include/autoround_hip.h
EXPORTS = (
    "ar_config_default", "ar_status_string", "ar_workspace_size", "ar_step_workspace_size",
    "ar_rtn_quant", "ar_fakequant_fwd", "ar_tune_step", "ar_tune_linear", "ar_pack", "ar_unpack",
    "ar_gram_workspace_size", "ar_gram_step_workspace_size", "ar_tune_step_gram",
    "ar_tune_linear_gram", "ar_init_clip", "ar_resolve_layer_config", "ar_resolve_fused_config",
    "ar_dequant_gemm_workspace_size", "ar_dequant_gemm", "ar_block_workspace_size",
    "ar_block_forward", "ar_tune_block", "ar_attention", "ar_tune_step_noalloc",
)

# fixed scratch of ar_tune_step_noalloc per GPU (AR_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


class ArConfig(ctypes.Structure):
    _fields_ = [
        ("bits", ctypes.c_int32), ("group_size", ctypes.c_int32), ("sym", ctypes.c_int32),
        ("nsamples", ctypes.c_int32), ("seqlen", ctypes.c_int32),
        ("batch_samples", ctypes.c_int32), ("iters", ctypes.c_int32),
        ("lr", ctypes.c_float), ("minmax_lr", ctypes.c_float),
        ("minmax_shrink", ctypes.c_float), ("clip_lo", ctypes.c_float),
        ("clip_hi", ctypes.c_float), ("init_scale", ctypes.c_int32),
        ("mse_grid", ctypes.c_int32), ("check_finite", ctypes.c_int32),
    ]


class ArState(ctypes.Structure):
    _fields_ = [
        ("W", ctypes.c_void_p), ("wdt", ctypes.c_int32), ("N", ctypes.c_int64),
        ("K", ctypes.c_int64), ("V", ctypes.c_void_p), ("alpha", ctypes.c_void_p),
        ("beta", ctypes.c_void_p), ("best_V", ctypes.c_void_p),
        ("best_alpha", ctypes.c_void_p), ("best_beta", ctypes.c_void_p),
        ("best_loss", ctypes.c_void_p),
    ]


class ArKernelTimes(ctypes.Structure):
    _fields_ = [
        ("sample_every", ctypes.c_int32),
        ("fwd_gemm_ms", ctypes.c_double), ("wgrad_gemm_ms", ctypes.c_double),
        ("ste_update_ms", ctypes.c_double),
        ("steps", ctypes.c_int64),
    ]


class ArLayerRule(ctypes.Structure):
    _fields_ = [("key", ctypes.c_char_p), ("bits", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("sym", ctypes.c_int32)]


class ArLayerQConfig(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("sym", ctypes.c_int32)]


class ArBlockDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int64), ("heads", ctypes.c_int64), ("inter", ctypes.c_int64),
                ("seqlen", ctypes.c_int64), ("nsamples", ctypes.c_int64),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


class ArBlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("Wq", "Wk", "Wv", "Wo", "Wg", "Wu", "Wd",
                                               "norm_attn", "norm_mlp")]


class ArBlockOutputs(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p * 7), ("scale", ctypes.c_void_p * 7),
                ("zp", ctypes.c_void_p * 7), ("Wq", ctypes.c_void_p * 7),
                ("losses", ctypes.c_void_p * 7), ("out_fp", ctypes.c_void_p),
                ("out_q", ctypes.c_void_p)]


BLOCK_LINEARS = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python autoround_signsgd_rounding_amd/build.py` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(ArConfig)
    sig = {
        "ar_config_default": [cfgp],
        "ar_workspace_size": [cfgp, i64, i64, i32, ctypes.POINTER(sz)],
        "ar_step_workspace_size": [cfgp, i64, i64, i64, i32, ctypes.POINTER(sz)],
        "ar_rtn_quant": [cfgp, i32, vp, i64, i64, vp, vp, vp, vp, vp],
        "ar_init_clip": [cfgp, i32, vp, i64, i64, vp, vp, vp],
        "ar_fakequant_fwd": [cfgp, i32, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp],
        "ar_tune_step": [cfgp, ctypes.POINTER(ArState), vp, vp, i32, i64, vp, vp, vp, vp, i32,
                         vp, sz, vp],
        "ar_tune_step_noalloc": [cfgp, ctypes.POINTER(ArState), vp, vp, i32, i64, vp, vp, vp,
                                 vp, i32, vp],
        "ar_tune_linear": [cfgp, i32, vp, i64, i64, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                           vp, sz, ctypes.POINTER(ArKernelTimes), vp],
        "ar_gram_workspace_size": [cfgp, i32, i64, i64, i32, ctypes.POINTER(sz)],
        "ar_gram_step_workspace_size": [cfgp, i32, i64, i64, i64, i32, ctypes.POINTER(sz)],
        "ar_tune_step_gram": [cfgp, ctypes.POINTER(ArState), vp, vp, i32, i64, vp, vp, vp, vp,
                              i32, vp, sz, vp],
        "ar_tune_linear_gram": [cfgp, i32, vp, i64, i64, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                vp, vp, sz, ctypes.POINTER(ArKernelTimes), vp],
        "ar_resolve_layer_config": [ctypes.POINTER(ArLayerRule), i32,
                                    ctypes.POINTER(ArLayerQConfig), i32, ctypes.c_char_p,
                                    ctypes.POINTER(ArLayerQConfig)],
        "ar_resolve_fused_config": [ctypes.POINTER(ArLayerRule), i32,
                                    ctypes.POINTER(ArLayerQConfig), i32, ctypes.c_char_p,
                                    ctypes.POINTER(ctypes.c_char_p), i32,
                                    ctypes.POINTER(ArLayerQConfig)],
        "ar_dequant_gemm_workspace_size": [i32, i32, i64, i64, i64, ctypes.POINTER(sz)],
        "ar_dequant_gemm": [i32, i32, vp, i64, i64, vp, vp, vp, i64, vp, i32, vp, sz, vp],
        "ar_block_workspace_size": [cfgp, ctypes.POINTER(ArBlockDims), ctypes.POINTER(sz)],
        "ar_block_forward": [ctypes.POINTER(ArBlockDims), ctypes.POINTER(ArBlockWeights), vp, vp,
                             vp, sz, vp],
        "ar_attention": [ctypes.POINTER(ArBlockDims), vp, vp, vp, vp, vp],
        "ar_tune_block": [cfgp, ctypes.POINTER(ArBlockDims), ctypes.POINTER(ArBlockWeights), vp,
                          vp, i32, ctypes.POINTER(ArBlockOutputs), vp, sz, vp],
        "ar_pack": [i32, vp, vp, i64, i64, i64, vp, vp, vp],
        "ar_unpack": [i32, vp, vp, i64, i64, i64, vp, vp, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int32
    lib.ar_status_string.argtypes = [ctypes.c_int32]
    lib.ar_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


class ArError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.ar_status_string(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


def _check(status: int, where: str):
    if status != 0:
        raise ArError(status, where)


@dataclasses.dataclass
class Config:
    """Tuning hyper-parameters (names of the llm-compressor AutoRoundModifier)."""
    bits: int = 4
    group_size: int = 128
    sym: bool = False
    nsamples: int = 128
    seqlen: int = 2048
    batch_samples: int = 8
    iters: int = 200
    lr: float = 0.005
    minmax_lr: float | None = None
    minmax_shrink: float = 1.0
    clip_lo: float = 0.5
    clip_hi: float = 1.0
    init: str = "minmax"       # initial scale: "minmax" or "mse"
    mse_grid: int = 100
    check_finite: bool = False  # scan the inputs first; NaN/Inf -> AR_ERR_NONFINITE

    def c(self) -> ArConfig:
        if self.init not in ("minmax", "mse"):
            raise ValueError(f"init must be 'minmax' or 'mse', not {self.init!r}")
        return ArConfig(self.bits, self.group_size, int(self.sym), self.nsamples, self.seqlen,
                        self.batch_samples, self.iters, self.lr,
                        -1.0 if self.minmax_lr is None else self.minmax_lr,
                        self.minmax_shrink, self.clip_lo, self.clip_hi,
                        1 if self.init == "mse" else 0, self.mse_grid, int(self.check_finite))

    def G(self, K: int) -> int:
        return 1 if self.group_size == -1 else K // self.group_size


# ------------------------------------------------------------------ torch marshalling
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return AR_F32
    if t.dtype == torch.bfloat16:
        return AR_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _need(t, name, shape, dtypes):
    """ValueError unless t is a contiguous GPU tensor of this shape and one of
    these dtypes (the library indexes every buffer by the shapes it is given,
    so a mismatch would read or write out of bounds)."""
    if t is None:
        raise ValueError(f"{name} is required")
    _dev(t)
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if tuple(t.shape) != tuple(shape) or t.dtype not in dtypes:
        want = "/".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name} must be {want} {list(shape)}, got {t.dtype} {list(t.shape)}")


def _weight(W, name="W"):
    """(N, K) of a 2-D float32 / bf16 weight on the GPU."""
    torch = _torch()
    if W is None or W.dim() != 2:
        raise ValueError(f"{name} must be a 2-D [N, K] tensor")
    _need(W, name, W.shape, (torch.float32, torch.bfloat16))
    return W.shape


def _groups(group_size: int, K: int) -> int:
    return 1 if group_size == -1 else (K // group_size if group_size > 0 else 0)


def workspace_size(cfg: Config, N: int, K: int, ydtype) -> int:
    out = ctypes.c_size_t()
    cc = cfg.c()
    _check(lib.ar_workspace_size(ctypes.byref(cc), N, K, ydtype, ctypes.byref(out)),
           "ar_workspace_size")
    return out.value


def step_workspace_size(cfg: Config, N: int, K: int, Tb: int, ydtype) -> int:
    out = ctypes.c_size_t()
    cc = cfg.c()
    _check(lib.ar_step_workspace_size(ctypes.byref(cc), N, K, Tb, ydtype, ctypes.byref(out)),
           "ar_step_workspace_size")
    return out.value


def gram_workspace_size(cfg: Config, wdt: int, N: int, K: int, ydtype) -> int:
    out = ctypes.c_size_t()
    cc = cfg.c()
    _check(lib.ar_gram_workspace_size(ctypes.byref(cc), wdt, N, K, ydtype, ctypes.byref(out)),
           "ar_gram_workspace_size")
    return out.value


def gram_step_workspace_size(cfg: Config, wdt: int, N: int, K: int, Tb: int, ydtype) -> int:
    out = ctypes.c_size_t()
    cc = cfg.c()
    _check(lib.ar_gram_step_workspace_size(ctypes.byref(cc), wdt, N, K, Tb, ydtype,
                                           ctypes.byref(out)), "ar_gram_step_workspace_size")
    return out.value


def init_clip(W, cfg: Config, stream=None):
    """Initial clip factors (alpha, beta) [N, G] float32 (Min-Max shrink or MSE search)."""
    torch = _torch()
    N, K = _weight(W)
    G = cfg.G(K)
    alpha = torch.empty((N, G), dtype=torch.float32, device=W.device)
    beta = torch.empty_like(alpha)
    cc = cfg.c()
    _check(lib.ar_init_clip(ctypes.byref(cc), _dt(W), _ptr(W), N, K, _ptr(alpha), _ptr(beta),
                            _stream(stream)), "ar_init_clip")
    return alpha, beta


def rtn_quant(W, cfg: Config, stream=None, want_wq: bool = True):
    """RTN codes [N,K] u8, scale [N,G] f32, zp [N,G] u8, Wq [N,K] (W's dtype)."""
    torch = _torch()
    N, K = _weight(W)
    G = cfg.G(K)
    codes = torch.empty((N, K), dtype=torch.uint8, device=W.device)
    scale = torch.empty((N, G), dtype=torch.float32, device=W.device)
    zp = torch.empty((N, G), dtype=torch.uint8, device=W.device)
    Wq = torch.empty_like(W) if want_wq else None
    cc = cfg.c()
    _check(lib.ar_rtn_quant(ctypes.byref(cc), _dt(W), _ptr(W), N, K, _ptr(codes), _ptr(scale),
                            _ptr(zp), _ptr(Wq), _stream(stream)), "ar_rtn_quant")
    return codes, scale, zp, Wq


def fakequant_fwd(W, V, alpha, beta, cfg: Config, stream=None):
    """bf16 Ŵ [N,K], codes [N,K] u8, scale [N,G] f32, zp [N,G] u8."""
    torch = _torch()
    N, K = _weight(W)
    G = cfg.G(K)
    _need(V, "V", (N, K), torch.float32)
    _need(alpha, "alpha", (N, G), torch.float32)
    _need(beta, "beta", (N, G), torch.float32)
    Wq = torch.empty((N, K), dtype=torch.bfloat16, device=W.device)
    codes = torch.empty((N, K), dtype=torch.uint8, device=W.device)
    scale = torch.empty((N, G), dtype=torch.float32, device=W.device)
    zp = torch.empty((N, G), dtype=torch.uint8, device=W.device)
    cc = cfg.c()
    _check(lib.ar_fakequant_fwd(ctypes.byref(cc), _dt(W), _ptr(W), N, K, _ptr(V), _ptr(alpha),
                                _ptr(beta), _ptr(Wq), _ptr(codes), _ptr(scale), _ptr(zp),
                                _stream(stream)), "ar_fakequant_fwd")
    return Wq, codes, scale, zp


def tune_step(W, V, alpha, beta, Xb, Yb, cfg: Config, *, best=None, want_grads=True,
              apply_update=True, workspace=None, stream=None, gram=False, noalloc=False):
    """One SignSGD step in place on (V, alpha, beta). ``best`` is an optional
    tuple (best_V, best_alpha, best_beta, best_loss[1]). Returns
    (loss[1] device tensor, gV, galpha, gbeta) with grads None unless wanted.
    ``gram`` selects ar_tune_step_gram; ``noalloc`` selects
    ar_tune_step_noalloc (no workspace: the library's fixed scratch)."""
    torch = _torch()
    N, K = _weight(W)
    G = cfg.G(K)
    if Xb is None or Xb.dim() != 2:
        raise ValueError("Xb must be a 2-D [Tb, K] tensor")
    Tb = Xb.shape[0]
    _need(Xb, "Xb", (Tb, K), torch.bfloat16)
    _need(Yb, "Yb", (Tb, N), (torch.float32, torch.bfloat16))
    _need(V, "V", (N, K), torch.float32)
    _need(alpha, "alpha", (N, G), torch.float32)
    _need(beta, "beta", (N, G), torch.float32)
    if best is not None:
        bV, bA, bB, bL = best
        _need(bV, "best_V", (N, K), torch.float32)
        _need(bA, "best_alpha", (N, G), torch.float32)
        _need(bB, "best_beta", (N, G), torch.float32)
        _need(bL, "best_loss", (1,), torch.float32)
    if workspace is not None:
        _need(workspace, "workspace", (workspace.numel(),), torch.uint8)
    ydt = _dt(Yb)
    if noalloc and (gram or workspace is not None):
        raise ValueError("noalloc takes no workspace and has no Gram form")
    if workspace is None and not noalloc:
        need = gram_step_workspace_size(cfg, _dt(W), N, K, Tb, ydt) if gram else \
            step_workspace_size(cfg, N, K, Tb, ydt)
        workspace = torch.empty(need, dtype=torch.uint8, device=W.device)
    loss = torch.empty(1, dtype=torch.float32, device=W.device)
    gV = torch.empty_like(V) if want_grads else None
    ga = torch.empty_like(alpha) if want_grads else None
    gb = torch.empty_like(beta) if want_grads else None
    bV, bA, bB, bL = best if best is not None else (None, None, None, None)
    st = ArState(W.data_ptr(), _dt(W), N, K, V.data_ptr(), alpha.data_ptr(), beta.data_ptr(),
                 None if bV is None else bV.data_ptr(), None if bA is None else bA.data_ptr(),
                 None if bB is None else bB.data_ptr(), None if bL is None else bL.data_ptr())
    cc = cfg.c()
    if noalloc:
        _check(lib.ar_tune_step_noalloc(ctypes.byref(cc), ctypes.byref(st), _ptr(Xb), _ptr(Yb),
                                        ydt, Tb, _ptr(loss), _ptr(gV), _ptr(ga), _ptr(gb),
                                        int(apply_update), _stream(stream)),
               "ar_tune_step_noalloc")
        return loss, gV, ga, gb
    fn, name = (lib.ar_tune_step_gram, "ar_tune_step_gram") if gram else \
        (lib.ar_tune_step, "ar_tune_step")
    _check(fn(ctypes.byref(cc), ctypes.byref(st), _ptr(Xb), _ptr(Yb), ydt, Tb, _ptr(loss),
              _ptr(gV), _ptr(ga), _ptr(gb), int(apply_update), _ptr(workspace),
              workspace.numel(), _stream(stream)), name)
    return loss, gV, ga, gb


@dataclasses.dataclass
class TuneOutput:
    codes: object
    scale: object
    zp: object
    Wq: object
    V: object
    alpha: object
    beta: object
    losses: object
    times: ArKernelTimes | None


def tune_linear(W, X, Y, cfg: Config, *, want_state=True, want_wq=False, timed=False,
                time_every=1, workspace=None, stream=None, gram=False) -> TuneOutput:
    """The whole tuning loop of one Linear (X [nsamples*seqlen, K] bf16,
    Y [nsamples*seqlen, N] bf16/f32). ``timed`` records HIP events around the
    kernels of every ``time_every``-th step. ``gram`` selects
    ar_tune_linear_gram."""
    torch = _torch()
    N, K = _weight(W)
    M = cfg.nsamples * cfg.seqlen
    _need(X, "X", (M, K), torch.bfloat16)
    _need(Y, "Y", (M, N), (torch.float32, torch.bfloat16))
    if workspace is not None:
        _need(workspace, "workspace", (workspace.numel(),), torch.uint8)
    G = cfg.G(K)
    ydt = _dt(Y)
    dev = W.device
    if workspace is None:
        need = gram_workspace_size(cfg, _dt(W), N, K, ydt) if gram else \
            workspace_size(cfg, N, K, ydt)
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
    scale = torch.empty((N, G), dtype=torch.float32, device=dev)
    zp = torch.empty((N, G), dtype=torch.uint8, device=dev)
    Wq = torch.empty_like(W) if want_wq else None
    V = torch.empty((N, K), dtype=torch.float32, device=dev) if want_state else None
    a = torch.empty((N, G), dtype=torch.float32, device=dev) if want_state else None
    b = torch.empty((N, G), dtype=torch.float32, device=dev) if want_state else None
    losses = torch.empty(max(cfg.iters, 1), dtype=torch.float32, device=dev)
    times = ArKernelTimes() if timed else None
    if times is not None:
        times.sample_every = time_every
    cc = cfg.c()
    fn, name = (lib.ar_tune_linear_gram, "ar_tune_linear_gram") if gram else \
        (lib.ar_tune_linear, "ar_tune_linear")
    _check(fn(ctypes.byref(cc), _dt(W), _ptr(W), N, K, _ptr(X), _ptr(Y), ydt, _ptr(codes),
              _ptr(scale), _ptr(zp), _ptr(Wq), _ptr(V), _ptr(a), _ptr(b), _ptr(losses),
              _ptr(workspace), workspace.numel(), ctypes.byref(times) if timed else None,
              _stream(stream)), name)
    return TuneOutput(codes, scale, zp, Wq, V, a, b, losses[:cfg.iters], times)


def dequant_gemm_workspace_size(bits: int, group_size: int, M: int, N: int, K: int) -> int:
    need = ctypes.c_size_t()
    _check(lib.ar_dequant_gemm_workspace_size(bits, group_size, M, N, K, ctypes.byref(need)),
           "ar_dequant_gemm_workspace_size")
    return need.value


def dequant_gemm(X, qweight, qzeros, scale, bits: int, group_size: int, N: int, *,
                 out_dtype=None, out=None, workspace=None, stream=None):
    """Y [M, N] = X·bf16(Ŵ)ᵀ from the packed format (ar_dequant_gemm). X [M, K]
    bf16; qzeros None for the symmetric grid; scale [N, G] float32. ``out`` and
    ``workspace`` may be given to avoid allocations."""
    torch = _torch()
    if X is None or X.dim() != 2:
        raise ValueError("X must be a 2-D [M, K] tensor")
    M, K = X.shape
    _need(X, "X", (M, K), torch.bfloat16)
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"bits must be one of {SUPPORTED_BITS}")
    G = _groups(group_size, K)
    _need(qweight, "qweight", (K * bits // 32, N), torch.int32)
    if qzeros is not None:
        _need(qzeros, "qzeros", (G, N * bits // 32), torch.int32)
    _need(scale, "scale", (N, G), torch.float32)
    if out is None:
        out_dtype = torch.float32 if out_dtype is None else out_dtype
        Y = torch.empty((M, N), dtype=out_dtype, device=X.device)
    else:
        _need(out, "out", (M, N), (torch.float32, torch.bfloat16))
        Y = out
    if workspace is not None:
        _need(workspace, "workspace", (workspace.numel(),), torch.uint8)
    if workspace is None:
        need = dequant_gemm_workspace_size(bits, group_size, M, N, K)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=X.device)
    _check(lib.ar_dequant_gemm(bits, group_size, _ptr(X), M, K, _ptr(qweight), _ptr(qzeros),
                               _ptr(scale), N, _ptr(Y), _dt(Y), _ptr(workspace),
                               workspace.numel(), _stream(stream)), "ar_dequant_gemm")
    return Y


def pack(codes, zp, bits: int, stream=None, out=None):
    """qweight [K*bits/32, N] int32 and qzeros [G, N*bits/32] int32 (or None).
    ``out`` = (qweight, qzeros) writes into given tensors instead."""
    torch = _torch()
    if codes is None or codes.dim() != 2:
        raise ValueError("codes must be a 2-D [N, K] uint8 tensor")
    N, K = codes.shape
    _need(codes, "codes", (N, K), torch.uint8)
    if zp is not None:
        if zp.dim() != 2 or zp.shape[0] != N:
            raise ValueError("zp must be a 2-D [N, G] uint8 tensor")
        _need(zp, "zp", (N, zp.shape[1]), torch.uint8)
    G = 0 if zp is None else zp.shape[1]
    if out is not None:
        qw, qz = out
        _dev(qw, qz)
        if tuple(qw.shape) != (K * bits // 32, N) or qw.dtype != torch.int32 or \
                (zp is not None and (qz is None or tuple(qz.shape) != (G, N * bits // 32)
                                     or qz.dtype != torch.int32)):
            raise ValueError("out tensors do not match the packed shapes")
    else:
        qw = torch.empty((K * bits // 32, N), dtype=torch.int32, device=codes.device)
        qz = None
        if zp is not None:
            qz = torch.empty((G, N * bits // 32), dtype=torch.int32, device=codes.device)
    _check(lib.ar_pack(bits, _ptr(codes), _ptr(zp), N, K, G, _ptr(qw), _ptr(qz),
                       _stream(stream)), "ar_pack")
    return qw, qz


def unpack(qweight, qzeros, bits: int, N: int, K: int, G: int, stream=None):
    torch = _torch()
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"bits must be one of {SUPPORTED_BITS}")
    _need(qweight, "qweight", (K * bits // 32, N), torch.int32)
    if qzeros is not None:
        _need(qzeros, "qzeros", (G, N * bits // 32), torch.int32)
    codes = torch.empty((N, K), dtype=torch.uint8, device=qweight.device)
    zp = torch.empty((N, G), dtype=torch.uint8, device=qweight.device) if qzeros is not None \
        else None
    _check(lib.ar_unpack(bits, _ptr(qweight), _ptr(qzeros), N, K, G, _ptr(codes), _ptr(zp),
                         _stream(stream)), "ar_unpack")
    return codes, zp


# ------------------------------------------------------------------ per-layer config
def _rules(rules):
    """[(key, {"bits", "group_size", "sym"} subset), ...] -> ctypes array."""
    arr = (ArLayerRule * max(len(rules), 1))()
    for i, (key, cfg) in enumerate(rules):
        arr[i] = ArLayerRule(key.encode(), int(cfg.get("bits", -1)),
                             int(cfg.get("group_size", 0)),
                             int(cfg["sym"]) if "sym" in cfg else -1)
    return arr


def resolve_layer_config(rules, defaults, quantized: bool, name: str):
    """(bits, group_size, sym) of one layer (ar_resolve_layer_config)."""
    arr = _rules(rules)
    d = ArLayerQConfig(*[int(x) for x in defaults])
    out = ArLayerQConfig()
    _check(lib.ar_resolve_layer_config(arr, len(rules), ctypes.byref(d), int(quantized),
                                       name.encode(), ctypes.byref(out)),
           "ar_resolve_layer_config")
    return out.bits, out.group_size, bool(out.sym)


def resolve_fused_config(rules, defaults, quantized: bool, layer_name: str, sub_names=None):
    """Config of a fused layer (ar_resolve_fused_config); ArError when its
    sub-layers disagree."""
    arr = _rules(rules)
    d = ArLayerQConfig(*[int(x) for x in defaults])
    out = ArLayerQConfig()
    # None selects the fused-expert rule (sub-layers from the rule keys); an
    # explicit list, even an empty one, is the sub-layer set itself
    if sub_names is None:
        names, nsub = None, 0
    else:
        subs = list(sub_names)
        names = (ctypes.c_char_p * max(len(subs), 1))(*[n.encode() for n in subs])
        nsub = len(subs)
    _check(lib.ar_resolve_fused_config(arr, len(rules), ctypes.byref(d), int(quantized),
                                       layer_name.encode(), names, nsub,
                                       ctypes.byref(out)), "ar_resolve_fused_config")
    return out.bits, out.group_size, bool(out.sym)


# ------------------------------------------------------------------ decoder block
def block_dims(D, H, F, seqlen, nsamples, rms_eps=1e-6, rope_theta=10000.0) -> ArBlockDims:
    return ArBlockDims(D, H, F, seqlen, nsamples, rms_eps, rope_theta)


def _block_shapes(dims: ArBlockDims):
    """[out, in] of each Linear of the block and the token count."""
    D, F = dims.hidden, dims.inter
    shapes = {"q_proj": (D, D), "k_proj": (D, D), "v_proj": (D, D), "o_proj": (D, D),
              "gate_proj": (F, D), "up_proj": (F, D), "down_proj": (D, F)}
    return shapes, dims.nsamples * dims.seqlen


def _block_weights(W: dict, norms, dims: ArBlockDims):
    torch = _torch()
    shapes, _ = _block_shapes(dims)
    for n in BLOCK_LINEARS:
        _need(W.get(n), n, shapes[n], torch.bfloat16)
    if len(norms) != 2:
        raise ValueError("norms = (attention norm, MLP norm)")
    for i, t in enumerate(norms):
        _need(t, f"norms[{i}]", (dims.hidden,), torch.bfloat16)
    return ArBlockWeights(*[W[n].data_ptr() for n in BLOCK_LINEARS],
                          norms[0].data_ptr(), norms[1].data_ptr())


def block_forward(h, W: dict, norms, dims: ArBlockDims, stream=None):
    """The decoder block's forward (ar_block_forward): h [M, D] bf16, W maps
    the Linear names to bf16 [out, in] tensors, norms = (attention, MLP) bf16 [D]."""
    torch = _torch()
    _need(h, "h", (_block_shapes(dims)[1], dims.hidden), torch.bfloat16)
    bw = _block_weights(W, norms, dims)
    need = ctypes.c_size_t()
    _check(lib.ar_block_workspace_size(None, ctypes.byref(dims), ctypes.byref(need)),
           "ar_block_workspace_size")
    ws = torch.empty(need.value, dtype=torch.uint8, device=h.device)
    out = torch.empty_like(h)
    _check(lib.ar_block_forward(ctypes.byref(dims), ctypes.byref(bw), _ptr(h), _ptr(out),
                                _ptr(ws), ws.numel(), _stream(stream)), "ar_block_forward")
    return out


def attention(q, k, v, dims: ArBlockDims, out=None, stream=None):
    """The block's causal attention step (ar_attention) on rotated q, k and v
    [nsamples·seqlen, hidden] bf16; returns out of the same shape."""
    torch = _torch()
    shape = (_block_shapes(dims)[1], dims.hidden)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, shape, torch.bfloat16)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", shape, torch.bfloat16)
    _check(lib.ar_attention(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                            _stream(stream)), "ar_attention")
    return out


def tune_block(h, W: dict, norms, dims: ArBlockDims, cfg: Config, *, quanted_input=True,
               h_q=None, stream=None):
    """Sequential tuning of the block's Linears (ar_tune_block). Returns a dict
    name -> (codes, scale, zp, Wq, losses) and the block outputs (fp, quantized)."""
    torch = _torch()
    shape = (_block_shapes(dims)[1], dims.hidden)
    _need(h, "h", shape, torch.bfloat16)
    if h_q is not None:
        _need(h_q, "h_q", shape, torch.bfloat16)
    dev = h.device
    bw = _block_weights(W, norms, dims)
    cc = cfg.c()
    need = ctypes.c_size_t()
    _check(lib.ar_block_workspace_size(ctypes.byref(cc), ctypes.byref(dims),
                                       ctypes.byref(need)), "ar_block_workspace_size")
    ws = torch.empty(need.value, dtype=torch.uint8, device=dev)
    res = {}
    outs = ArBlockOutputs()
    for i, n in enumerate(BLOCK_LINEARS):
        N, K = W[n].shape
        G = cfg.G(K)
        t = (torch.empty((N, K), dtype=torch.uint8, device=dev),
             torch.empty((N, G), dtype=torch.float32, device=dev),
             torch.empty((N, G), dtype=torch.uint8, device=dev),
             torch.empty((N, K), dtype=torch.bfloat16, device=dev),
             torch.empty(max(cfg.iters, 1), dtype=torch.float32, device=dev))
        res[n] = t
        outs.codes[i], outs.scale[i], outs.zp[i], outs.Wq[i], outs.losses[i] = \
            [x.data_ptr() for x in t]
    out_fp = torch.empty_like(h)
    out_q = torch.empty_like(h)
    outs.out_fp, outs.out_q = out_fp.data_ptr(), out_q.data_ptr()
    _check(lib.ar_tune_block(ctypes.byref(cc), ctypes.byref(dims), ctypes.byref(bw), _ptr(h),
                             _ptr(h_q), int(quanted_input), ctypes.byref(outs), _ptr(ws),
                             ws.numel(), _stream(stream)), "ar_tune_block")
    res = {n: (c, s, z, w, l[:cfg.iters]) for n, (c, s, z, w, l) in res.items()}
    return res, out_fp, out_q

