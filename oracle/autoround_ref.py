"""Plain CPU oracle of AutoRound's per-Linear SignSGD tuning loop.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The HIP library
and its Python binding never import it, and it imports nothing from them: the
two implementations share no code. The only common module is ``synth`` (seeded
input draws, none of the method's arithmetic).

Sources, cited by page title and section:
  [LLMC]  "[llm-compressor] AutoRound: 부호 경사 하강법으로 라운딩 최적화"
          - "논문 핵심 내용" (paper core): RTN equation, learnable-offset
            equation, offset range, output-reconstruction loss, SignSGD equation
          - "AutoRoundModifier 생성자 파라미터" (constructor parameter table)
          - "on_event with SEQUENTIAL_EPOCH_END" (the per-module tuning loop)
          - "_fake_quantize_with_offset" (quantize / clamp / dequantize)
  [INTEL] "Introducing AutoRound: Intel's Advanced Quantization for LLMs and VLMs"
          - section 2 (joint optimisation of rounding and clipping range)
          - section 4 (iters = 0 falls back to RTN; 8/4/3/2-bit)
  [SGL]   "[SGLang] AutoRound: 자동 라운딩 최적화 양자화"
          - "1. AutoRoundConfig" (SUPPORTED_BITS, pack_factor = Fraction(32, bits))
          - "설계 근거" (reuse of GPTQ/AWQ packing)
  [ADMMQ] ADMM-Q page, "1. 문제 공식화" (Hessian-weighted layer objective with
          H = XᵀX), used only as an independent identity in the tests.

Precision: the per-module loop upcasts W to float before quantizing ([LLMC]
tuning loop), so every elementwise quantizer step (scale, zero-point, divide,
offset add, round, clamp, dequantize) is IEEE float32 here, in the order stated
below. AMP is on by default ([LLMC] parameter table), read as bf16 GEMM
operands; the oracle evaluates the two contractions in float64 on those bf16
operands (``amp=True``) or on unrounded float64 operands (``amp=False``), and
accumulates the loss and the straight-through sums in float64.

Every function here is pinned by a CPU test against something other than
itself (hand-derived vectors, a nearest-grid search, brute force, torch
autograd, the Gram identity, big-integer packing); see ``tests/test_oracle_pins.py``.
Where the pages are silent or garbled, the reading taken is stated in the
function that takes it.
"""
from __future__ import annotations

import dataclasses
import re
import math

import numpy as np

F32 = np.float32
F64 = np.float64

SUPPORTED_BITS = (2, 3, 4, 8)      # [SGL] "1. AutoRoundConfig"


@dataclasses.dataclass
class Config:
    """Tuning hyper-parameters, named as on the [LLMC] parameter table."""
    bits: int = 4
    group_size: int = 128          # -1: one group per row
    sym: bool = False
    nsamples: int = 128
    seqlen: int = 2048
    batch_samples: int = 8         # samples per SignSGD step
    iters: int = 200
    lr: float = 0.005
    minmax_lr: float | None = None  # None: same as lr
    minmax_shrink: float = 1.0     # initial alpha = beta
    clip_lo: float = 0.5           # alpha/beta clamp range
    clip_hi: float = 1.0
    init: str = "minmax"           # initial scale: "minmax" or "mse"
    mse_grid: int = 100            # shrink grid steps per unit for init = "mse"

    @property
    def maxq(self) -> int:
        return 2 ** self.bits - 1

    @property
    def mlr(self) -> float:
        return self.lr if self.minmax_lr is None else self.minmax_lr

    def g(self, K: int) -> int:
        return K if self.group_size == -1 else self.group_size


# ------------------------------------------------------------------ bf16
def bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even mantissa);
    the result is returned as float32. NaN stays NaN."""
    x32 = np.ascontiguousarray(x, dtype=F32)
    bits = x32.view(np.uint32)
    upper = bits >> np.uint32(16)
    low = bits & np.uint32(0xFFFF)
    up = (low > 0x8000) | ((low == 0x8000) & ((upper & np.uint32(1)) == 1))
    upper = upper + up.astype(np.uint32)
    out = (upper << np.uint32(16)).view(F32)
    return np.where(np.isnan(x32), F32(np.nan), out)


# ------------------------------------------------------------------ S1
def group_minmax(W: np.ndarray, group_size: int):
    """Per-(row, group) min and max of W (the Min-Max initial range of
    [LLMC] tuning loop). Groups are ``group_size`` contiguous input channels
    of one output row; ``group_size == -1`` is the whole row."""
    N, K = W.shape
    g = K if group_size == -1 else group_size
    Wg = np.asarray(W, dtype=F32).reshape(N, K // g, g)
    return Wg.min(axis=2), Wg.max(axis=2)


# ------------------------------------------------------------------ S2
@dataclasses.dataclass
class QParams:
    s: np.ndarray          # float32 [N, G]
    zp: np.ndarray         # float32 [N, G], integer-valued
    lo: np.ndarray | None  # asym: clipped range low end
    hi: np.ndarray | None
    zero: np.ndarray       # bool [N, G]: degenerate (zero-range) group, s forced to 1


def qparams(wmin, wmax, alpha, beta, bits: int, sym: bool) -> QParams:
    """Scale and zero-point from the clipped min/max ([INTEL] section 2:
    rounding and clipping range tuned together; alpha scales the group min,
    beta the group max). All steps float32, in this order.

    asym: lo = min(alpha*wmin, 0); hi = max(beta*wmax, 0); s = (hi-lo)/maxq;
          zp = clamp(rint(-lo/s), 0, maxq)
    sym:  amax = max(|alpha*wmin|, |beta*wmax|); s = (2*amax)/maxq; zp = 2^(bits-1)
    A zero-range group gets s = 1.
    """
    maxq = F32(2 ** bits - 1)
    wmin = np.asarray(wmin, F32)
    wmax = np.asarray(wmax, F32)
    alpha = np.asarray(alpha, F32)
    beta = np.asarray(beta, F32)
    if sym:
        amax = np.maximum(np.abs(alpha * wmin), np.abs(beta * wmax))
        s = (F32(2.0) * amax) / maxq
        zero = s == 0
        s = np.where(zero, F32(1.0), s).astype(F32)
        zp = np.full(s.shape, F32(2 ** (bits - 1)), dtype=F32)
        return QParams(s=s, zp=zp, lo=None, hi=None, zero=zero)
    lo = np.minimum(alpha * wmin, F32(0.0))
    hi = np.maximum(beta * wmax, F32(0.0))
    s = (hi - lo) / maxq
    zero = s == 0
    s = np.where(zero, F32(1.0), s).astype(F32)
    zp = np.clip(np.rint(-lo / s), F32(0.0), maxq).astype(F32)
    return QParams(s=s, zp=zp, lo=lo, hi=hi, zero=zero)


# ------------------------------------------------------------------ S3
@dataclasses.dataclass
class FakeQuant:
    t: np.ndarray      # W/s                   float32 [N, K]
    q: np.ndarray      # clamped integer code  float32 [N, K]
    m: np.ndarray      # in-range mask         bool [N, K]
    what: np.ndarray   # s*(q - zp)            float32 [N, K]
    s_e: np.ndarray    # s broadcast           float32 [N, K]
    zp_e: np.ndarray   # zp broadcast          float32 [N, K]


def fake_quant(W, V, qp: QParams, bits: int, group_size: int) -> FakeQuant:
    """Learnable-offset rounding ([LLMC] paper core; _fake_quantize_with_offset).

    t = W/s; r = rint(t + V); c = r + zp; q = clamp(c, 0, maxq);
    Ŵ = s*(q - zp). rint rounds half to even. The zero-point is added after
    rounding (the offset equation rounds W/s + V); the in-range mask
    m = [0 <= c <= maxq] is what a straight-through backward passes.
    """
    W = np.asarray(W, F32)
    V = np.asarray(V, F32)
    N, K = W.shape
    g = K if group_size == -1 else group_size
    maxq = F32(2 ** bits - 1)
    s_e = np.repeat(qp.s, g, axis=1)
    zp_e = np.repeat(qp.zp, g, axis=1)
    t = W / s_e
    u = t + V
    r = np.rint(u)
    c = r + zp_e
    q = np.clip(c, F32(0.0), maxq)
    m = (c >= 0) & (c <= maxq)
    what = s_e * (q - zp_e)
    return FakeQuant(t=t, q=q, m=m, what=what, s_e=s_e, zp_e=zp_e)


# ------------------------------------------------------------------ initial scale
def mse_grid_points(cfg: Config) -> np.ndarray:
    """Shrink candidates of the MSE initial scale, largest first: the values
    p_j = float32(1 - j/mse_grid) (formed in float64, rounded once), j = 0, 1,
    ..., that lie in [clip_lo, clip_hi] (float32 comparisons), so every
    candidate is a valid clip factor. ValueError when there is none."""
    lo, hi = F32(cfg.clip_lo), F32(cfg.clip_hi)
    if cfg.mse_grid < 1:
        raise ValueError("mse_grid must be >= 1")
    pts = []
    j = 0
    while True:
        p = F32(1.0 - j / cfg.mse_grid)
        if p < lo:
            break
        if p <= hi:
            pts.append(p)
        j += 1
    if not pts:
        raise ValueError("no MSE grid point inside [clip_lo, clip_hi]")
    return np.array(pts, F32)


def mse_shrink(W, cfg: Config) -> np.ndarray:
    """MSE initial scale ([LLMC] tuning loop: initial scale / zero-point by
    "Min-Max or MSE"): per group, the shrink p of the grid whose round-to-
    nearest quantization (V = 0, alpha = beta = p) has the smallest sum of
    squared weight errors. Errors are formed in float32 (w - Ŵ, squared) and
    summed in float64; ties go to the earlier, larger p. Returns p [N, G]."""
    W = np.asarray(W, F32)
    N, K = W.shape
    g = cfg.g(K)
    Gn = K // g
    wmin, wmax = group_minmax(W, cfg.group_size)
    V0 = np.zeros((N, K), F32)
    errs = []
    pts = mse_grid_points(cfg)
    for p in pts:
        a = np.full(wmin.shape, p, F32)
        qp = qparams(wmin, wmax, a, a, cfg.bits, cfg.sym)
        fq = fake_quant(W, V0, qp, cfg.bits, cfg.group_size)
        d = (W - fq.what).astype(F32)
        e = (d * d).astype(F32)
        errs.append(e.astype(F64).reshape(N, Gn, g).sum(axis=2))
    best = np.argmin(np.stack(errs), axis=0)          # first minimum on ties
    return pts[best]


def init_clip(W, cfg: Config):
    """Initial clip factors (alpha, beta) [N, G]: minmax_shrink everywhere
    (init = "minmax"), or the MSE shrink of each group (init = "mse")."""
    N, K = np.shape(W)
    Gn = K // cfg.g(K)
    if cfg.init == "mse":
        p = mse_shrink(W, cfg)
        return p.copy(), p.copy()
    a = np.full((N, Gn), F32(cfg.minmax_shrink), F32)
    return a, a.copy()


# ------------------------------------------------------------------ S4-S7
def forward_backward(Xb, Yb, what, *, amp: bool = True, n_scale: int | None = None):
    """Output-reconstruction loss and its gradient with respect to Ŵ.

    Y' = Xb·Ŵᵀ; R = Y' - Yb; L = sum(R²)/(T·N)   (mean over the minibatch, as
    the [LLMC] loop's ``pow(2).mean()``);
    dL/dŴ = (2/(T·N))·dYᵀ·Xb with dY = R.
    amp=True: Ŵ and Xb are bf16 operands and dY is rounded to bf16 from its
    float32 value; the products are summed in float64.
    ``n_scale`` replaces N in the normalisation when only some rows are given
    (rows of Ŵ are independent except for this constant).
    Returns (L, G[N, K] float64, sum(R²)).
    """
    T = Xb.shape[0]
    N = what.shape[0]
    if T == 0 or N == 0:
        raise ValueError("the loss is a mean over tokens and outputs: needs T > 0 and N > 0")
    Nn = N if n_scale is None else n_scale
    X64 = np.asarray(Xb, F64)
    Wq = bf16(what) if amp else np.asarray(what, F32)
    Yp = X64 @ Wq.astype(F64).T
    R = Yp - np.asarray(Yb, F64)
    loss_sum = float(np.sum(R * R))
    dY = bf16(R.astype(F32)).astype(F64) if amp else R
    G = (2.0 / (T * Nn)) * (dY.T @ X64)
    return loss_sum / (T * Nn), G, loss_sum


# ------------------------------------------------------------------ Gram form
@dataclasses.dataclass
class GramStats:
    """Minibatch statistics of the Gram form: H = Xbᵀ·Xb [K, K], Cn = Eᵀ·Xb
    [N, K] and e2 = sum(E²), where E = Xb·Wᵀ − Yb is the target's deviation from
    the unquantized layer on these tokens. All float64."""
    H: np.ndarray
    Cn: np.ndarray
    e2: float
    T: int


def gram_stats(Xb, Yb, W) -> GramStats:
    """H = XᵀX is the weight of the layer-wise objective on the ADMM-Q page
    ("1. 문제 공식화"); Cn and e2 carry the part of the target that the
    unquantized weight does not reproduce (zero when Yb = Xb·Wᵀ exactly)."""
    X64 = np.asarray(Xb, F64)
    E = X64 @ np.asarray(W, F64).T - np.asarray(Yb, F64)
    return GramStats(H=X64.T @ X64, Cn=E.T @ X64, e2=float(np.sum(E * E)), T=X64.shape[0])


def forward_backward_gram(st: GramStats, W, what, *, n_scale: int | None = None):
    """The loss and Ŵ-gradient of ``forward_backward`` (bf16 Ŵ operand),
    evaluated through the minibatch's Gram matrix, with the residual kept
    unrounded. With D = bf16(Ŵ) − W, the residual is R = Xb·Dᵀ + E, so
      sum(R²)  = Σ D∘(D·H) + 2·Σ D∘Cn + e2,
      dL/dŴ    = (2/(T·N))·Rᵀ·Xb = (2/(T·N))·(D·H + Cn).
    float64. Returns (L, G[N, K], sum(R²))."""
    N = what.shape[0]
    Nn = N if n_scale is None else n_scale
    D = bf16(what).astype(F64) - np.asarray(W, F64)
    P = D @ st.H
    loss_sum = float(np.sum(D * P) + 2.0 * np.sum(D * st.Cn) + st.e2)
    G = (2.0 / (st.T * Nn)) * (P + st.Cn)
    return loss_sum / (st.T * Nn), G, loss_sum


# ------------------------------------------------------------------ S8
def ste_grads(G, W, fq: FakeQuant, qp: QParams, wmin, wmax, alpha, beta,
              bits: int, sym: bool, group_size: int):
    """Straight-through gradients of the loss w.r.t. V, alpha and beta.

    Rounding is passed through with slope 1 (the literal listing would give
    zero slope, which leaves V fixed); the clamp passes gradient where
    0 <= c <= maxq. With dŴ = G:
      dL/dV  = G·s·m
      A      = Σ_group G·((q - zp) - m·t)      (dL/ds at fixed zp)
      B      = -s·Σ_group G·[not m]            (dL/dzp, through the rounding)
    asym (zp = -lo/s before rounding, s = (hi-lo)/maxq):
      D = A + B·lo/s²;  dL/dlo = -D/maxq - B/s;  dL/dhi = D/maxq
      dL/dalpha = dL/dlo·wmin·[wmin < 0];  dL/dbeta = dL/dhi·wmax·[wmax > 0]
    sym (s = 2·amax/maxq, zp fixed):
      dL/damax = 2A/maxq, routed to alpha (·|wmin|) when |alpha·wmin| > |beta·wmax|,
      else to beta (·|wmax|).
    Zero-range groups get no alpha/beta gradient. Sums are float64.
    """
    N, K = W.shape
    g = K if group_size == -1 else group_size
    Gn = K // g
    maxq = float(2 ** bits - 1)
    G64 = np.asarray(G, F64)
    m = fq.m
    gV = G64 * fq.s_e.astype(F64) * m
    qz = (fq.q - fq.zp_e).astype(F64)
    A = np.sum((G64 * (qz - m * fq.t.astype(F64))).reshape(N, Gn, g), axis=2)
    Bsum = np.sum((G64 * (~m)).reshape(N, Gn, g), axis=2)
    s64 = qp.s.astype(F64)
    B = -s64 * Bsum
    wmin64 = np.asarray(wmin, F64)
    wmax64 = np.asarray(wmax, F64)
    if sym:
        damax = 2.0 * A / maxq
        to_alpha = np.abs(np.asarray(alpha, F32) * np.asarray(wmin, F32)) > \
            np.abs(np.asarray(beta, F32) * np.asarray(wmax, F32))
        ga = np.where(to_alpha, damax * np.abs(wmin64), 0.0)
        gb = np.where(to_alpha, 0.0, damax * np.abs(wmax64))
    else:
        lo64 = qp.lo.astype(F64)
        D = A + B * lo64 / (s64 * s64)
        dlo = -D / maxq - B / s64
        dhi = D / maxq
        ga = dlo * wmin64 * (wmin64 < 0)
        gb = dhi * wmax64 * (wmax64 > 0)
    ga = np.where(qp.zero, 0.0, ga)
    gb = np.where(qp.zero, 0.0, gb)
    return gV, ga, gb


# ------------------------------------------------------------------ S9
def sgn(x) -> np.ndarray:
    """Sign as float32 in {-1, 0, 1}; NaN counts as 0."""
    x = np.asarray(x)
    return ((x > 0).astype(F32) - (x < 0).astype(F32))


def signsgd_update(V, alpha, beta, gV, ga, gb, cfg: Config):
    """SignSGD step with clamping ([LLMC] paper core; tuning loop):
    V <- clamp(V - lr·sgn(dL/dV), -0.5, 0.5); alpha and beta move by
    minmax_lr (lr when unset) and stay within [clip_lo, clip_hi]. float32."""
    lr = F32(cfg.lr)
    mlr = F32(cfg.mlr)
    Vn = np.clip(np.asarray(V, F32) - lr * sgn(gV), F32(-0.5), F32(0.5))
    an = np.clip(np.asarray(alpha, F32) - mlr * sgn(ga), F32(cfg.clip_lo), F32(cfg.clip_hi))
    bn = np.clip(np.asarray(beta, F32) - mlr * sgn(gb), F32(cfg.clip_lo), F32(cfg.clip_hi))
    return Vn.astype(F32), an.astype(F32), bn.astype(F32)


# ------------------------------------------------------------------ one step
@dataclasses.dataclass
class StepResult:
    loss: float
    loss_sum: float
    gV: np.ndarray
    galpha: np.ndarray
    gbeta: np.ndarray
    V: np.ndarray          # updated state
    alpha: np.ndarray
    beta: np.ndarray
    what: np.ndarray       # fake-quantized weight of the state the loss was taken at


def tune_step(W, V, alpha, beta, wmin, wmax, Xb, Yb, cfg: Config, *, amp: bool = True,
              n_scale: int | None = None, gram: GramStats | None = None) -> StepResult:
    """One SignSGD iteration from state (V, alpha, beta) on one minibatch.
    With ``gram`` (the minibatch's ``gram_stats``), loss and gradient come from
    ``forward_backward_gram`` and Xb, Yb are not used."""
    qp = qparams(wmin, wmax, alpha, beta, cfg.bits, cfg.sym)
    fq = fake_quant(W, V, qp, cfg.bits, cfg.group_size)
    if gram is not None:
        L, G, loss_sum = forward_backward_gram(gram, W, fq.what, n_scale=n_scale)
    else:
        L, G, loss_sum = forward_backward(Xb, Yb, fq.what, amp=amp, n_scale=n_scale)
    gV, ga, gb = ste_grads(G, W, fq, qp, wmin, wmax, alpha, beta,
                           cfg.bits, cfg.sym, cfg.group_size)
    Vn, an, bn = signsgd_update(V, alpha, beta, gV, ga, gb, cfg)
    return StepResult(loss=L, loss_sum=loss_sum, gV=gV, galpha=ga, gbeta=gb,
                      V=Vn, alpha=an, beta=bn, what=fq.what)


# ------------------------------------------------------------------ whole loop
@dataclasses.dataclass
class TuneResult:
    codes: np.ndarray      # uint8 [N, K]
    scale: np.ndarray      # float32 [N, G]
    zp: np.ndarray         # uint8 [N, G]
    what: np.ndarray       # float32 [N, K]
    V: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    losses: list
    best_loss: float
    best_step: int         # -1 when no step was evaluated (iters = 0)


def quantize_state(W, V, alpha, beta, wmin, wmax, cfg: Config):
    """Codes, scale, zero-point and Ŵ of a state (final write-back of the
    [LLMC] tuning loop: weight, weight_scale, weight_zero_point)."""
    qp = qparams(wmin, wmax, alpha, beta, cfg.bits, cfg.sym)
    fq = fake_quant(W, V, qp, cfg.bits, cfg.group_size)
    return fq.q.astype(np.uint8), qp.s, qp.zp.astype(np.uint8), fq.what


def rtn_quant(W, cfg: Config):
    """Round-to-nearest: V = 0 and the initial clip factors ([LLMC] RTN
    equation; [INTEL] section 4: zero iterations give RTN)."""
    N, K = W.shape
    wmin, wmax = group_minmax(W, cfg.group_size)
    a, b = init_clip(W, cfg)
    return quantize_state(W, np.zeros((N, K), F32), a, b, wmin, wmax, cfg)


def tune_linear(W, minibatch, nb: int, cfg: Config, *, amp: bool = True,
                n_scale: int | None = None, on_step=None, gram: bool = False) -> TuneResult:
    """The per-Linear tuning loop ([LLMC] tuning loop) with a best-loss snapshot.

    ``minibatch(b)`` returns (Xb, Yb) for minibatch b; step i uses
    b = i mod nb. The state (V, alpha, beta) whose loss is strictly below the
    best so far is snapshotted before its update; after ``iters`` steps the
    best state is restored and quantized. iters = 0 returns the initial state
    (RTN with minmax_shrink). ``gram=True`` evaluates every step in the Gram
    form (``forward_backward_gram``) from per-minibatch ``gram_stats``.
    """
    N, K = W.shape
    W = np.asarray(W, F32)
    stats = {}
    wmin, wmax = group_minmax(W, cfg.group_size)
    V = np.zeros((N, K), F32)
    alpha, beta = init_clip(W, cfg)
    best = (V.copy(), alpha.copy(), beta.copy())
    best_loss, best_step = math.inf, -1
    losses = []
    for i in range(cfg.iters):
        Xb, Yb = minibatch(i % nb)
        st = None
        if gram:
            if i % nb not in stats:
                stats[i % nb] = gram_stats(Xb, Yb, W)
            st = stats[i % nb]
        r = tune_step(W, V, alpha, beta, wmin, wmax, Xb, Yb, cfg, amp=amp, n_scale=n_scale,
                      gram=st)
        losses.append(r.loss)
        if r.loss < best_loss:
            best_loss, best_step = r.loss, i
            best = (V.copy(), alpha.copy(), beta.copy())
        if on_step is not None:
            on_step(i, r)
        V, alpha, beta = r.V, r.alpha, r.beta
    if cfg.iters >= 1:
        V, alpha, beta = best
    codes, scale, zp, what = quantize_state(W, V, alpha, beta, wmin, wmax, cfg)
    return TuneResult(codes=codes, scale=scale, zp=zp, what=what, V=V, alpha=alpha,
                      beta=beta, losses=losses, best_loss=best_loss, best_step=best_step)


# ------------------------------------------------------------------ S11
def _pack_axis0(vals: np.ndarray, bits: int) -> np.ndarray:
    """Concatenate ``bits``-wide fields along axis 0, least significant bit
    first, into 32-bit words; a field that crosses a word boundary is split."""
    L, C = vals.shape
    assert (L * bits) % 32 == 0
    out = np.zeros((L * bits // 32, C), dtype=np.uint64)
    v = np.asarray(vals, np.uint64)
    for k in range(L):
        w, off = divmod(k * bits, 32)
        out[w] |= (v[k] << np.uint64(off)) & np.uint64(0xFFFFFFFF)
        if off + bits > 32:
            out[w + 1] |= v[k] >> np.uint64(32 - off)
    return out.astype(np.uint32)


def _unpack_axis0(words: np.ndarray, bits: int, L: int) -> np.ndarray:
    C = words.shape[1]
    w64 = np.asarray(words, np.uint64)
    mask = np.uint64((1 << bits) - 1)
    out = np.zeros((L, C), dtype=np.uint64)
    for k in range(L):
        w, off = divmod(k * bits, 32)
        val = w64[w] >> np.uint64(off)
        if off + bits > 32:
            val |= w64[w + 1] << np.uint64(32 - off)
        out[k] = val & mask
    return out.astype(np.uint8)


def pack(codes: np.ndarray, zp: np.ndarray, bits: int):
    """GPTQ-style int32 packing ([SGL] pack_factor = Fraction(32, bits);
    packing reuse in "설계 근거"): 32/bits codes per word, exact for 3 bits
    (32 codes in 3 words).
    qweight [K·bits/32, N]: column n holds row n's codes along K, LSB first.
    qzeros  [G, N·bits/32]: row j holds group j's zero-points along N.
    Returned as uint32 bit patterns."""
    qweight = _pack_axis0(np.asarray(codes).T, bits)
    qzeros = _pack_axis0(np.asarray(zp), bits).T.copy()
    return qweight, qzeros


def unpack(qweight, qzeros, bits: int, N: int, K: int):
    codes = _unpack_axis0(qweight, bits, K).T.copy()
    zp = _unpack_axis0(np.asarray(qzeros).T, bits, N)
    return codes, zp


# ------------------------------------------------------------------ W{2,3,4,8}A16 product
def dequantize(qweight, qzeros, scale, bits: int, group_size: int, N: int, K: int):
    """Ŵ [N, K] float32 from the packed format ([SGL] "설계 근거": AutoRound
    checkpoints reuse GPTQ/AWQ packing; the dequantisation Ŵ = s·(q - zp) of
    [LLMC] _fake_quantize_with_offset): codes and zero-points unpacked (zp =
    2^(bits-1) when qzeros is None, the symmetric grid), scale [N, G] float32,
    then s·(q - zp) in float32."""
    g = K if group_size == -1 else group_size
    if qzeros is None:   # symmetric grid: no zero-point words, N need not fill words
        codes = _unpack_axis0(qweight, bits, K).T.copy()
        zp = np.full((N, K // g), 2 ** (bits - 1), np.int64)
    else:
        codes, zp = unpack(qweight, qzeros, bits, N, K)
    s_e = np.repeat(np.asarray(scale, F32), g, axis=1)
    zp_e = np.repeat(np.asarray(zp, F32), g, axis=1)
    return (s_e * (codes.astype(F32) - zp_e)).astype(F32)


def dequant_matmul(X, qweight, qzeros, scale, bits: int, group_size: int, N: int, K: int):
    """Y = X·bf16(Ŵ)ᵀ [M, N] in float64 (bf16 Ŵ: the operand the tuning loop's
    forward product uses; X is taken as given, bf16 values)."""
    what = dequantize(qweight, qzeros, scale, bits, group_size, N, K)
    return np.asarray(X, F64) @ bf16(what).astype(F64).T


# ------------------------------------------------------------------ brute force
def brute_force_rounding(W, X, Y, qp: QParams, bits: int, group_size: int):
    """Exhaustive optimum over every floor/ceil choice of W/s (the rounding
    choices an offset in [-0.5, 0.5] can reach for non-half-integer W/s) with
    s and zp fixed. Rows are independent; returns (per-row minimum of
    ||X·ŵ_nᵀ - Y[:, n]||², best codes). float64, small inputs only."""
    W = np.asarray(W, F32)
    N, K = W.shape
    g = K if group_size == -1 else group_size
    maxq = 2 ** bits - 1
    s_e = np.repeat(qp.s, g, axis=1).astype(F64)
    zp_e = np.repeat(qp.zp, g, axis=1).astype(F64)
    t = (W / np.repeat(qp.s, g, axis=1)).astype(F64)
    fl = np.floor(t)
    X64 = np.asarray(X, F64)
    Y64 = np.asarray(Y, F64)
    best_val = np.full(N, np.inf)
    best_codes = np.zeros((N, K), np.uint8)
    for n in range(N):
        for mask in range(1 << K):
            up = np.array([(mask >> k) & 1 for k in range(K)], F64)
            c = np.clip(fl[n] + up + zp_e[n], 0, maxq)
            w_hat = s_e[n] * (c - zp_e[n])
            val = float(np.sum((X64 @ w_hat - Y64[:, n]) ** 2))
            if val < best_val[n]:
                best_val[n] = val
                best_codes[n] = c.astype(np.uint8)
    return best_val, best_codes


# ------------------------------------------------------------------ per-layer config
# A rule key is a pattern when it holds one of these characters; the set has
# to be the same for every implementation, since it decides which keys match.
REGEX_SPECIAL_CHARS = frozenset("*+?^$()[]{}|\\")
_FIELDS = ("bits", "group_size", "sym")
_UNQUANTIZED = (16, -1, True)       # "leave the layer unquantized"


def _merge(rule_cfg: dict, fallback) -> tuple:
    """(bits, group_size, sym): the rule's value where it sets one, else the
    fallback's."""
    return tuple(rule_cfg[f] if f in rule_cfg else fb for f, fb in zip(_FIELDS, fallback))


def _whole_name_match(key: str, name: str) -> bool:
    """True when ``key`` is a pattern that compiles and matches all of ``name``."""
    if REGEX_SPECIAL_CHARS.isdisjoint(key):
        return False
    try:
        return re.compile(key).fullmatch(name) is not None
    except re.error:
        return False


def resolve_layer_config(rules, defaults, quantized: bool, name: str):
    """(bits, group_size, sym) of one layer from per-layer rules ([SGL]
    "2. 레이어별 개별 설정" and "3. 정규식 기반 레이어 매칭"). ``rules`` is an
    ordered list of (key, cfg dict with optional "bits", "group_size", "sym").
    The fallback is the defaults, or (16, -1, True) for a layer outside the
    quantized set (16 bits: leave it unquantized).
      - no rules: the fallback;
      - a key equal to the name (the first such rule): its values, the
        missing ones from the fallback;
      - else the first key that is a pattern (holds a regular-expression
        special character) and matches the whole name: its values, the
        missing ones from the defaults; keys that do not compile never match;
      - else the fallback."""
    fallback = tuple(defaults) if quantized else _UNQUANTIZED
    if not rules:
        return fallback
    by_key = {}
    for key, cfg in rules:
        by_key.setdefault(key, cfg)
    if name in by_key:
        return _merge(by_key[name], fallback)
    hit = next((cfg for key, cfg in rules if _whole_name_match(key, name)), None)
    return fallback if hit is None else _merge(hit, tuple(defaults))


def resolve_fused_config(rules, defaults, quantized: bool, layer_name: str, sub_names=None):
    """Config of a fused layer ([SGL] "4. FusedMoE와 Fused QKV 처리"): all of its
    sub-layers must resolve to one config, else ValueError. With ``sub_names``
    (a fused q/k/v-style layer) those names are the sub-layers; without (a
    fused expert layer) they are the rule keys that start with the layer's
    name, and a layer with no such key resolves as itself."""
    if sub_names is not None:
        members = list(sub_names)
    else:
        members = [key for key, _ in rules if key.startswith(layer_name)]
        if not members:
            return resolve_layer_config(rules, defaults, quantized, layer_name)
    resolved = {resolve_layer_config(rules, defaults, quantized, m) for m in members}
    if len(resolved) != 1:
        raise ValueError(f"fused layer {layer_name!r}: sub-layers resolve to {sorted(resolved)}")
    return resolved.pop()

