"""Seeded synthetic inputs for the MoE layer workloads.

Holds no arithmetic of the MoE layer: it only draws the tensors a workload
needs (x, router weight, expert weights, upstream gradient, router bias) from a
counter-based generator implemented in ``gen.c``. The same arrays feed the CPU
oracle and the GPU library.

Recipe (all seeded; stream ids are (tensor << 32) | expert):
  * x, dY ~ N(0, 1)
  * Wr [E, H], W1 [E, 2I, H] ~ N(0, 1/H) (std 1/sqrt(fan_in)); W2 [E, H, I] ~ N(0, 1/I)
  * N(0,1) is the Irwin-Hall(12) approximation in exact integer arithmetic.
  * imbalanced workloads add a fixed router-logit bias: experts get a seeded
    random Zipf rank rho in 1..E; the hottest 7E/8 ranks get
    b = -alpha * s * ln(rho) with s = 1.2, the coldest E/8 get -30 so that they
    receive no tokens. alpha is a per-workload constant chosen so that the
    busiest expert holds about 8x the mean number of routed rows.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "libmokgen.so")

T_X, T_WR, T_W1, T_W2, T_DY, T_BIAS = 0, 1, 2, 3, 4, 5


def build_generator(force: bool = False) -> str:
    """Compile gen.c into libmokgen.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _gen_lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build_generator())
        _lib.mok_gen_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                        ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        _lib.mok_gen_normal.restype = None
        _lib.mok_gen_words.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                       ctypes.c_void_p]
        _lib.mok_gen_words.restype = None
    return _lib


def normal(seed: int, stream: int, offset: int, n: int, scale: float, dtype: str) -> torch.Tensor:
    """n deviates of N(0, scale^2) as a 1-D CPU tensor of dtype 'f32' or 'bf16'."""
    if dtype == "bf16":
        out = torch.empty(n, dtype=torch.int16)
        _gen_lib().mok_gen_normal(seed, stream, offset, n, scale, 1, out.data_ptr())
        return out.view(torch.bfloat16)
    out = torch.empty(n, dtype=torch.float32)
    _gen_lib().mok_gen_normal(seed, stream, offset, n, scale, 0, out.data_ptr())
    return out


def words(seed: int, stream: int, offset: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _gen_lib().mok_gen_words(seed, stream, offset, n, out.ctypes.data)
    return out


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    T: int
    H: int
    E: int
    k: int
    I: int
    act: str            # activation / weight storage dtype: 'f32' or 'bf16'
    gemm: str           # expert-GEMM operand format: 'f32', 'bf16', 'mxfp8' or 'mxfp4'
    backward: bool
    zipf: bool          # imbalanced routing via the Zipf-ranked router bias
    micro_batches: int = 1

    @property
    def seed(self) -> int:
        return 0x4D6F4B00 + self.index

    @property
    def R(self) -> int:
        return self.T * self.k


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 0, 64, 128, 8, 2, 256, "f32", "f32", False, False),
        Workload("small_bf16", 1, 2048, 1024, 32, 2, 512, "bf16", "bf16", True, False),
        Workload("imbalanced_bf16", 2, 2048, 1024, 32, 2, 512, "bf16", "bf16", True, True),
        Workload("kimi_k2_bf16", 3, 16384, 7168, 384, 8, 2048, "bf16", "bf16", True, False),
        Workload("kimi_k2_mxfp8_stream", 4, 16384, 7168, 384, 8, 2048, "bf16", "mxfp8", True, True, 8),
    ]
}

# Bias scale alpha per imbalanced workload. Chosen by oracle/calibrate_imbalance.py
# (bisection on the oracle's router over the whole token set) so that the
# busiest expert receives about 8x the mean number of routed rows.
ZIPF_ALPHA = {
    "imbalanced_bf16": 0.5996,          # max/mean 8.000, 4 of 32 experts get no tokens
    "kimi_k2_mxfp8_stream": 0.1862,     # max/mean 7.989, 48 of 384 experts get no tokens
}
ZIPF_S = 1.2
COLD_BIAS = -30.0


def _std(fan_in: int) -> float:
    return float(np.float32(1.0 / math.sqrt(fan_in)))


def replace(w: Workload, **kw) -> Workload:
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)


def make_x(w: Workload, t0: int = 0, n: Optional[int] = None) -> torch.Tensor:
    """Tokens t0 .. t0+n-1 of x as [n, H]."""
    n = w.T - t0 if n is None else n
    return normal(w.seed, T_X << 32, t0 * w.H, n * w.H, 1.0, w.act).view(n, w.H)


def make_dy(w: Workload, t0: int = 0, n: Optional[int] = None) -> torch.Tensor:
    n = w.T - t0 if n is None else n
    return normal(w.seed, T_DY << 32, t0 * w.H, n * w.H, 1.0, w.act).view(n, w.H)


def make_wr(w: Workload) -> torch.Tensor:
    return normal(w.seed, T_WR << 32, 0, w.E * w.H, _std(w.H), w.act).view(w.E, w.H)


def make_w1(w: Workload, e: int) -> torch.Tensor:
    """Expert e's first-layer weight [2I, H]: rows 0..I-1 gate, I..2I-1 up."""
    return normal(w.seed, (T_W1 << 32) | e, 0, 2 * w.I * w.H, _std(w.H), w.act).view(2 * w.I, w.H)


def make_w2(w: Workload, e: int) -> torch.Tensor:
    """Expert e's second-layer weight [H, I]."""
    return normal(w.seed, (T_W2 << 32) | e, 0, w.H * w.I, _std(w.I), w.act).view(w.H, w.I)


def zipf_ranks(w: Workload) -> np.ndarray:
    """Seeded random permutation giving each expert a Zipf rank in 1..E (Fisher-Yates)."""
    order = np.arange(w.E)
    r = words(w.seed, T_BIAS << 32, 0, w.E)
    for i in range(w.E - 1, 0, -1):
        j = int(r[i] % np.uint64(i + 1))
        order[i], order[j] = order[j], order[i]
    rank = np.empty(w.E, dtype=np.int64)
    rank[order] = np.arange(1, w.E + 1)
    return rank


def make_bias(w: Workload, alpha: Optional[float] = None) -> Optional[torch.Tensor]:
    """Router-logit bias [E] float32, or None for balanced workloads."""
    if not w.zipf:
        return None
    if alpha is None:
        alpha = ZIPF_ALPHA[w.name]
        if alpha is None:
            raise RuntimeError("no calibrated Zipf bias scale for %s" % w.name)
    rank = zipf_ranks(w)
    n_cold = w.E // 8
    b = np.empty(w.E, dtype=np.float32)
    for e in range(w.E):
        if rank[e] > w.E - n_cold:
            b[e] = COLD_BIAS
        else:
            b[e] = np.float32(-alpha * ZIPF_S * math.log(rank[e]))
    return torch.from_numpy(b)
