"""Helpers shared by the GPU parity tests: host <-> device conversions and the
oracle's view of the same inputs. Imports the binding and the oracle side by
side; neither imports the other."""
import numpy as np
import torch

import oracle as O
import synth

F32 = np.float32


def dev():
    return torch.device("cuda:0")


def bf16_dev(bits_u16: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(dev()).view(
        torch.bfloat16)


def weight_dev(case):
    if case.wdtype == "bf16":
        return bf16_dev(case.W_bits)
    return torch.from_numpy(case.W).to(dev())


def to_np(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def bf16_bits_of(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def targets_dev(case, rows=None):
    """Y_true on the GPU (torch float64 accumulation, same bytes as numpy)."""
    return synth.reference_outputs_torch(case, dev(), rows=rows)


def oracle_cfg(c):
    return O.Config(bits=c.bits, group_size=c.group_size, sym=bool(c.sym), nsamples=c.nsamples,
                    seqlen=c.seqlen, batch_samples=c.batch_samples, iters=c.iters, lr=c.lr,
                    minmax_lr=c.minmax_lr, minmax_shrink=c.minmax_shrink, clip_lo=c.clip_lo,
                    clip_hi=c.clip_hi, init=c.init, mse_grid=c.mse_grid)


def rel_norm(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def log(msg):
    print(msg, flush=True)
