"""Plain CPU oracle of sequential block-wise tuning with quantized inputs.

TEST INFRASTRUCTURE ONLY (imported by ``tests/`` and nothing in the product).

Sources:
  [LLMC] "[llm-compressor] AutoRound: 부호 경사 하강법으로 라운딩 최적화":
         the per-subgraph loop (each Linear of a subgraph tuned in turn on its
         captured inputs and targets), the parameter table
         (``enable_quanted_input``: use the previous layers' quantized output
         as input), the "enable_quanted_input 모드" section and design point 3
         (layer-by-layer, as in GPTQ's sequential pipeline).

The pages do not show the decoder block itself. A Llama-style block is
assumed (LLaMA-2-7B is the pages' model). It runs RMSNorm, the q/k/v
projections, rotary embedding (rotate-half), causal softmax attention and
o_proj with a residual, then RMSNorm, gate/up projections, SiLU(gate)·up and
down_proj with a residual. Activations are bf16 between operations, as in a
bf16 model; each operation works in float32 or float64 as stated per function,
then rounds its output to bf16 (RNE).

Sequential tuning of one block:
  - full-precision pipeline: the block with its original weights;
  - quantized pipeline: the same ops with every already-tuned Linear replaced
    by bf16(Ŵ);
  - Linears tuned in order q, k, v, o, gate, up, down. Each is tuned with
    ``autoround_ref.tune_linear`` on input X and target Y, where Y is that
    Linear's full-precision output on its full-precision input, and X is its
    input in the quantized pipeline (``quanted_input=True``) or in the
    full-precision pipeline (``False``).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import autoround_ref as R

F32, F64 = np.float32, np.float64
LINEARS = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")


def b16(x) -> np.ndarray:
    """Round to bf16 (RNE), returned as float32 values."""
    return R.bf16(np.asarray(x, F32))


# ------------------------------------------------------------------ operations
def rmsnorm(x, w, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x²) + eps) · w per row; mean and root in float64,
    the two products in float32 (x·r, then ·w); bf16 output."""
    x = np.asarray(x, F32)
    ms = np.mean(x.astype(F64) ** 2, axis=1, keepdims=True)
    r = (1.0 / np.sqrt(ms + eps)).astype(F32)
    return b16((x * r).astype(F32) * np.asarray(w, F32))


def linear(x, W) -> np.ndarray:
    """y = x·Wᵀ summed in float64, rounded to float32, then bf16."""
    return b16((np.asarray(x, F64) @ np.asarray(W, F64).T).astype(F32))


def rope_table(seqlen: int, Dh: int, theta: float):
    """cos/sin [seqlen, Dh/2] of angle p·theta^(−2j/Dh), in float64 rounded to
    float32."""
    j = np.arange(Dh // 2, dtype=F64)
    inv = theta ** (-2.0 * j / Dh)
    ang = np.arange(seqlen, dtype=F64)[:, None] * inv[None, :]
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def rope(x, seqlen: int, H: int, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding per head: for the two halves (a, b) of a
    head vector at position p (token index within its sequence),
    (a·cos − b·sin, b·cos + a·sin), each product and difference in float32;
    bf16 output."""
    x = np.asarray(x, F32)
    M, D = x.shape
    Dh = D // H
    c, s = rope_table(seqlen, Dh, theta)
    pos = np.arange(M) % seqlen
    c, s = c[pos][:, None, :], s[pos][:, None, :]
    xh = x.reshape(M, H, Dh)
    a, b = xh[..., :Dh // 2], xh[..., Dh // 2:]
    out = np.concatenate([(a * c).astype(F32) - (b * s).astype(F32),
                          (b * c).astype(F32) + (a * s).astype(F32)], axis=-1)
    return b16(out.reshape(M, D))


def attention(q, k, v, seqlen: int, H: int) -> np.ndarray:
    """Causal softmax attention per sequence and head:
    softmax(q·kᵀ / sqrt(Dh)) · v, with the scores formed in float64, the
    softmax and the weighted sum in float64; bf16 output [M, D]."""
    q, k, v = (np.asarray(t, F64) for t in (q, k, v))
    M, D = q.shape
    Dh = D // H
    out = np.empty((M, D), F64)
    mask = np.triu(np.ones((seqlen, seqlen), bool), 1)
    for s0 in range(0, M, seqlen):
        for h in range(H):
            sl = slice(h * Dh, (h + 1) * Dh)
            S = (q[s0:s0 + seqlen, sl] @ k[s0:s0 + seqlen, sl].T) / np.sqrt(Dh)
            S[mask] = -np.inf
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P /= P.sum(axis=1, keepdims=True)
            out[s0:s0 + seqlen, sl] = P @ v[s0:s0 + seqlen, sl]
    return b16(out.astype(F32))


def silu_mul(g, u) -> np.ndarray:
    """SiLU(g)·u = g/(1 + exp(−g))·u in float64; bf16 output."""
    g, u = np.asarray(g, F64), np.asarray(u, F64)
    return b16((g / (1.0 + np.exp(-g)) * u).astype(F32))


def add(a, b) -> np.ndarray:
    """bf16(a + b), the sum in float32."""
    return b16(np.asarray(a, F32) + np.asarray(b, F32))


# ------------------------------------------------------------------ block
def block_forward(h, W: dict, norms, dims) -> dict:
    """One block's forward on hidden states h [M, D]; W maps each Linear's name
    to its (bf16-valued) weight. Returns every intermediate by name, and
    "out"."""
    t = {"h": np.asarray(h, F32)}
    t["a"] = rmsnorm(t["h"], norms[0], dims.rms_eps)
    for n in ("q_proj", "k_proj", "v_proj"):
        t[n] = linear(t["a"], W[n])
    t["q_rope"] = rope(t["q_proj"], dims.seqlen, dims.H, dims.rope_theta)
    t["k_rope"] = rope(t["k_proj"], dims.seqlen, dims.H, dims.rope_theta)
    t["attn"] = attention(t["q_rope"], t["k_rope"], t["v_proj"], dims.seqlen, dims.H)
    t["o_proj"] = linear(t["attn"], W["o_proj"])
    t["h1"] = add(t["h"], t["o_proj"])
    t["m"] = rmsnorm(t["h1"], norms[1], dims.rms_eps)
    t["gate_proj"] = linear(t["m"], W["gate_proj"])
    t["up_proj"] = linear(t["m"], W["up_proj"])
    t["z"] = silu_mul(t["gate_proj"], t["up_proj"])
    t["down_proj"] = linear(t["z"], W["down_proj"])
    t["out"] = add(t["h1"], t["down_proj"])
    return t


# input activation of each Linear, by name of the intermediate
LINEAR_INPUT = {"q_proj": "a", "k_proj": "a", "v_proj": "a", "o_proj": "attn",
                "gate_proj": "m", "up_proj": "m", "down_proj": "z"}


@dataclasses.dataclass
class BlockTuneResult:
    results: dict        # name -> autoround_ref.TuneResult
    Wq: dict             # name -> bf16(Ŵ) used in the quantized pipeline
    out_fp: np.ndarray   # full-precision block output
    out_q: np.ndarray    # quantized block output
    err: float           # mean squared difference of the two outputs


def tune_block(h, W: dict, norms, dims, cfg: R.Config, *, quanted_input: bool = True,
               h_q=None) -> BlockTuneResult:
    """Sequential tuning of the block's Linears (module docstring). ``h_q`` is
    the block input in the quantized pipeline (the previous block's quantized
    output); it defaults to h. ``cfg`` gives nsamples / seqlen /
    batch_samples over the M = nsamples·seqlen tokens."""
    fp = block_forward(h, W, norms, dims)
    Tb = cfg.batch_samples * cfg.seqlen
    nb = cfg.nsamples // cfg.batch_samples
    Wq = dict(W)
    results = {}
    hq = fp["h"] if h_q is None else np.asarray(h_q, F32)
    q = None
    for name in LINEARS:
        # the quantized pipeline up to this Linear's input, with the Linears tuned so far
        q = block_forward(hq, Wq, norms, dims)
        X = q[LINEAR_INPUT[name]] if quanted_input else fp[LINEAR_INPUT[name]]
        Y = fp[name]
        res = R.tune_linear(np.asarray(W[name], F32),
                            lambda b: (X[b * Tb:(b + 1) * Tb], Y[b * Tb:(b + 1) * Tb]), nb, cfg)
        results[name] = res
        Wq[name] = b16(res.what)
    q = block_forward(hq, Wq, norms, dims)
    err = float(np.mean((q["out"].astype(F64) - fp["out"].astype(F64)) ** 2))
    return BlockTuneResult(results=results, Wq=Wq, out_fp=fp["out"], out_q=q["out"], err=err)
