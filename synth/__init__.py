"""Seeded synthetic inputs for the per-Linear AutoRound tuning workloads.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It only *draws* data: Gaussian weights and activations with outlier
columns/channels, and the reference layer output Y_true = X·Wᵀ that the tuning
loop is given as its target. It holds none of the quantization method's
arithmetic (no scales, rounding offsets, losses or gradients).

The workloads stand in for the calibration setting described on the
llm-compressor AutoRound walk-through (AutoRoundModifier parameters: 128
samples of 2048 tokens) and for the Qwen2.5-72B timing mentioned on the
"Introducing AutoRound" page. No model weights or text are used; shapes are
those of the named Linear layers.

Recipe (per workload, one ``numpy.random.default_rng(seed)`` stream):
  1. W outlier column indices: ``round(0.005*K)`` distinct columns (if enabled);
  2. X outlier channel indices: ``round(0.01*K)`` distinct channels (if enabled);
  3. W ~ N(0, sigma_w) as float32 [N, K]; outlier columns ×10;
     cast to bf16 (round-to-nearest-even) when the weight dtype is bf16;
  4. X ~ N(0, 1) float32 [M, K], drawn in row chunks of ``CHUNK_ROWS``; outlier
     channels ×20 per chunk; the tuning input is bf16(X) (RNE);
  5. Y_true = X·Wᵀ accumulated in float64 from the stored operands
     (bf16 X for bf16 workloads, float32 X for float32 ones), rounded to
     float32 and then, for bf16 workloads, to bf16 (RNE).
Because step 5 accumulates in float64, the rounded result does not depend on
the summation order, so a CPU (numpy) and a GPU (torch float64) evaluation give
identical bytes.
"""
from __future__ import annotations

import dataclasses
import numpy as np

CHUNK_ROWS = 16384


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int                  # out features
    K: int                  # in features
    wdtype: str             # "f32" | "bf16"  (model dtype: W and Y_true)
    bits: int
    group_size: int
    sym: bool
    nsamples: int
    seqlen: int
    batch_samples: int      # samples per SignSGD step (minibatch)
    iters: int
    lr: float = 0.005
    minmax_lr: float | None = None   # None: same as lr
    minmax_shrink: float = 1.0
    sigma_w: float = 0.02
    outliers: bool = True
    seed: int = 0

    @property
    def M(self) -> int:
        return self.nsamples * self.seqlen

    @property
    def Tb(self) -> int:
        return self.batch_samples * self.seqlen

    @property
    def flop_per_iter(self) -> int:
        """Forward plus weight-gradient contraction: 2·Tb·K·N each."""
        return 4 * self.Tb * self.K * self.N


WORKLOADS = {
    w.name: w
    for w in (
        Workload("toy_256", N=256, K=256, wdtype="f32", bits=4, group_size=64,
                 sym=False, nsamples=2, seqlen=128, batch_samples=2, iters=20,
                 outliers=False),
        Workload("llama7b_q_proj", N=4096, K=4096, wdtype="bf16", bits=4,
                 group_size=128, sym=False, nsamples=128, seqlen=2048,
                 batch_samples=8, iters=200),
        Workload("llama7b_down_proj", N=4096, K=11008, wdtype="bf16", bits=2,
                 group_size=128, sym=False, nsamples=128, seqlen=2048,
                 batch_samples=8, iters=200, minmax_lr=0.005, minmax_shrink=1.0),
        Workload("llama7b_gate_proj", N=11008, K=4096, wdtype="bf16", bits=3,
                 group_size=128, sym=True, nsamples=128, seqlen=2048,
                 batch_samples=8, iters=200),
        Workload("qwen72b_up_proj", N=29568, K=8192, wdtype="bf16", bits=4,
                 group_size=128, sym=False, nsamples=128, seqlen=2048,
                 batch_samples=8, iters=200, sigma_w=0.015),
    )
}


# ---------------------------------------------------------------- bf16 casts
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u.astype(np.uint64) + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- generators
@dataclasses.dataclass
class Case:
    """Host copies of one workload's inputs.

    W       float32 [N, K]  weight values (bf16-representable for bf16 weights)
    W_bits  uint16 [N, K]   bf16 bit patterns, or None for float32 weights
    X_bits  uint16 [M, K]   bf16 calibration inputs (the tuning GEMM operand)
    X_f32   float32 [M, K]  float32 inputs (only for float32 workloads, used for Y_true)
    """
    N: int
    K: int
    M: int
    wdtype: str
    W: np.ndarray
    W_bits: np.ndarray | None
    X_bits: np.ndarray
    X_f32: np.ndarray | None


def make_case(N: int, K: int, M: int, *, wdtype: str = "bf16", sigma_w: float = 0.02,
              outliers: bool = True, seed: int = 0) -> Case:
    """Draw W and X following the module recipe (steps 1-4)."""
    rng = np.random.default_rng(seed)
    w_cols = x_chs = None
    if outliers:
        w_cols = np.sort(rng.choice(K, size=int(np.rint(0.005 * K)), replace=False))
        x_chs = np.sort(rng.choice(K, size=int(np.rint(0.01 * K)), replace=False))
    W = rng.normal(0.0, sigma_w, size=(N, K)).astype(np.float32)
    if w_cols is not None and len(w_cols):
        W[:, w_cols] *= np.float32(10.0)
    W_bits = None
    if wdtype == "bf16":
        W_bits = f32_to_bf16_bits(W)
        W = bf16_bits_to_f32(W_bits)
    X_bits = np.empty((M, K), dtype=np.uint16)
    X_f32 = np.empty((M, K), dtype=np.float32) if wdtype == "f32" else None
    for r0 in range(0, M, CHUNK_ROWS):
        r1 = min(M, r0 + CHUNK_ROWS)
        xc = rng.standard_normal(size=(r1 - r0, K), dtype=np.float32)
        if x_chs is not None and len(x_chs):
            xc[:, x_chs] *= np.float32(20.0)
        X_bits[r0:r1] = f32_to_bf16_bits(xc)
        if X_f32 is not None:
            X_f32[r0:r1] = xc
    return Case(N=N, K=K, M=M, wdtype=wdtype, W=W, W_bits=W_bits, X_bits=X_bits, X_f32=X_f32)


def make_workload_case(w: Workload, nsamples: int | None = None) -> Case:
    """Inputs of a named workload; ``nsamples`` truncates the sample count
    (the first samples are identical to those of the full draw)."""
    M = (nsamples if nsamples is not None else w.nsamples) * w.seqlen
    return make_case(w.N, w.K, M, wdtype=w.wdtype, sigma_w=w.sigma_w,
                     outliers=w.outliers, seed=w.seed)


def reference_outputs(case: Case, rows: slice | None = None) -> np.ndarray:
    """Y_true = X·Wᵀ (recipe step 5) with numpy float64 accumulation.

    Returns float32 [M, N] for float32 workloads, bf16 bit patterns uint16
    [M, N] for bf16 workloads.
    """
    rows = rows if rows is not None else slice(0, case.M)
    r0, r1 = rows.start, rows.stop
    W64 = case.W.astype(np.float64)
    bf = case.wdtype == "bf16"
    out = np.empty((r1 - r0, case.N), dtype=np.uint16 if bf else np.float32)
    for c0 in range(r0, r1, CHUNK_ROWS):
        c1 = min(r1, c0 + CHUNK_ROWS)
        if bf:
            xc = bf16_bits_to_f32(case.X_bits[c0:c1]).astype(np.float64)
        else:
            xc = case.X_f32[c0:c1].astype(np.float64)
        y = (xc @ W64.T).astype(np.float32)
        out[c0 - r0:c1 - r0] = f32_to_bf16_bits(y) if bf else y
    return out


def reference_outputs_torch(case: Case, device, rows: slice | None = None):
    """Same as :func:`reference_outputs` but evaluated with torch float64
    matmuls on ``device``; returns a torch tensor on ``device``
    (bfloat16 for bf16 workloads, float32 otherwise)."""
    import torch
    rows = rows if rows is not None else slice(0, case.M)
    r0, r1 = rows.start, rows.stop
    bf = case.wdtype == "bf16"
    W64 = torch.from_numpy(case.W).to(device=device, dtype=torch.float64)
    out = torch.empty((r1 - r0, case.N), dtype=torch.bfloat16 if bf else torch.float32,
                      device=device)
    for c0 in range(r0, r1, CHUNK_ROWS):
        c1 = min(r1, c0 + CHUNK_ROWS)
        if bf:
            xb = torch.from_numpy(case.X_bits[c0:c1].view(np.int16)).to(device)
            xc = xb.view(torch.bfloat16).to(torch.float64)
        else:
            xc = torch.from_numpy(case.X_f32[c0:c1]).to(device=device, dtype=torch.float64)
        y = (xc @ W64.T).to(torch.float32)
        out[c0 - r0:c1 - r0] = y.to(torch.bfloat16) if bf else y
    return out


# ---------------------------------------------------------------- decoder block
@dataclasses.dataclass(frozen=True)
class BlockDims:
    """A Llama-style decoder block: hidden D, heads H (head_dim D/H), MLP width
    F; calibration of nsamples sequences of seqlen tokens."""
    name: str
    D: int
    H: int
    F: int
    seqlen: int
    nsamples: int
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    sigma_w: float = 0.02
    seed: int = 0

    @property
    def M(self) -> int:
        return self.nsamples * self.seqlen

    @property
    def Dh(self) -> int:
        return self.D // self.H


BLOCKS = {
    b.name: b
    for b in (
        BlockDims("toy_block", D=256, H=4, F=512, seqlen=64, nsamples=4),
        BlockDims("llama7b_block", D=4096, H=32, F=11008, seqlen=2048, nsamples=16),
    )
}

# Linear layers of the block in tuning order: (name, out features, in features)
BLOCK_LINEARS = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")


def block_linear_shape(b: BlockDims, name: str):
    return {"q_proj": (b.D, b.D), "k_proj": (b.D, b.D), "v_proj": (b.D, b.D),
            "o_proj": (b.D, b.D), "gate_proj": (b.F, b.D), "up_proj": (b.F, b.D),
            "down_proj": (b.D, b.F)}[name]


@dataclasses.dataclass
class BlockCase:
    dims: BlockDims
    W_bits: dict          # name -> bf16 bits [out, in]
    norm_bits: tuple      # (attention norm, MLP norm) bf16 bits [D]
    H_bits: np.ndarray    # block input hidden states, bf16 bits [M, D]


def make_block_case(b: BlockDims, nsamples: int | None = None) -> BlockCase:
    """Draw one block's weights and its calibration input (one stream, in this
    order): the seven Linear weights N(0, sigma_w) in BLOCK_LINEARS order, each
    with rint(0.005·in) outlier input columns ×10; the two RMSNorm weights
    1 + N(0, 0.05); the hidden states N(0, 1) [M, D] with rint(0.01·D) outlier
    channels ×20, drawn in row chunks. Everything is cast to bf16 (RNE)."""
    rng = np.random.default_rng(b.seed)
    W = {}
    for name in BLOCK_LINEARS:
        N, K = block_linear_shape(b, name)
        cols = rng.choice(K, size=int(np.rint(0.005 * K)), replace=False)
        w = rng.normal(0.0, b.sigma_w, size=(N, K)).astype(np.float32)
        w[:, cols] *= np.float32(10.0)
        W[name] = f32_to_bf16_bits(w)
    norms = tuple(f32_to_bf16_bits((1.0 + 0.05 * rng.standard_normal(b.D)).astype(np.float32))
                  for _ in range(2))
    M = (nsamples if nsamples is not None else b.nsamples) * b.seqlen
    chs = rng.choice(b.D, size=int(np.rint(0.01 * b.D)), replace=False)
    Hb = np.empty((M, b.D), dtype=np.uint16)
    for r0 in range(0, M, CHUNK_ROWS):
        r1 = min(M, r0 + CHUNK_ROWS)
        hc = rng.standard_normal(size=(r1 - r0, b.D), dtype=np.float32)
        hc[:, chs] *= np.float32(20.0)
        Hb[r0:r1] = f32_to_bf16_bits(hc)
    return BlockCase(dims=b, W_bits=W, norm_bits=norms, H_bits=Hb)
