"""Seeded synthetic workloads for the MoE dispatch/combine path.

This module only draws random inputs; it holds none of the method's
arithmetic, and it is the one module that both the HIP path's tests/bench and
the CPU oracle are fed from.  Everything is generated on the host with numpy
``Generator(PCG64)``; each tensor has its own sub-stream spawned from one
``SeedSequence(seed)``, so a tensor's values do not depend on which other
tensors were drawn.  fp32 -> bf16 uses torch's CPU conversion
(round-to-nearest-even).

Workload shapes follow the problem statement of the reference pages: T
tokens, hidden H, E experts (E/R per virtual rank), top-k.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from fractions import Fraction

import numpy as np

# sub-stream ids under SeedSequence(seed).spawn(...)
_S_HIDDEN = 0
_S_OUTLIER_ROWS = 1
_S_LOGITS0 = 2  # layer l uses _S_LOGITS0 + l
_N_STREAMS = 16


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    R: int
    chunks: int = 1                # 0: fitted per payload (driver.fit_chunks)
    layers: int = 1
    quant: tuple = (0,)            # per-layer payload: 0 = bf16, 1 = int8
    capacity_factor: Fraction | None = None
    zipf_s: float | None = None    # per-expert logit bias ln p_e, p_e ~ (e+1)^-s
    outlier_frac: float = 0.0      # fraction of hidden rows scaled by outlier_scale
    outlier_scale: float = 50.0
    streams: int = 1
    seed: int = 0
    note: str = field(default="", compare=False)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload("tiny", T=256, H=512, E=8, k=2, R=2, chunks=1, quant=(0,),
                     note="hidden N(0,1) bf16, logits N(0,1) fp32, bf16 send buffer, "
                          "stand-in expert x*(1+e/8)"),
    "mid": Workload("mid", T=4096, H=4096, E=64, k=8, R=8, chunks=1, quant=(1,),
                    note="per-token dynamic int8 send buffer, one chunk"),
    "dsv3": Workload("dsv3", T=16384, H=7168, E=256, k=8, R=32, chunks=0, quant=(0,),
                     zipf_s=1.1, outlier_frac=0.01,
                     note="DeepSeek-V3-like; 1% rows x50; Zipf(1.1) expert bias; "
                          "int8 on and off; chunks fitted to the last-level cache "
                          "(8 for bf16, 4 for int8)"),
    "qwen3": Workload("qwen3", T=32768, H=2048, E=128, k=8, R=16, chunks=8, layers=4,
                      quant=(0, 1, 1, 0), capacity_factor=Fraction(5, 4), streams=2,
                      note="Qwen3-30B-A3B-like 4-layer stack, 8 chunks on 2 streams, "
                           "int8 on middle layers, capacity 1.25 drop by token id"),
    "large": Workload("large", T=131072, H=8192, E=64, k=8, R=8, chunks=4, quant=(0,),
                      note="bf16 (~17.2 GB per direction) and int8, 4 chunks"),
}


def _streams(seed: int):
    return np.random.SeedSequence(seed).spawn(_N_STREAMS)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_streams(seed)[stream]))


def zipf_bias(E: int, s: float) -> np.ndarray:
    """Per-expert logit bias ln p_e with p_e proportional to (e+1)^-s; the
    normalising constant is dropped (a common shift of a token's logits)."""
    return (-s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)


def make_logits(wl: Workload, layer: int = 0) -> np.ndarray:
    """Router logits, fp32 [T, E]: N(0,1), plus the Zipf bias if configured."""
    rng = _rng(wl.seed, _S_LOGITS0 + layer)
    z = rng.standard_normal((wl.T, wl.E), dtype=np.float32)
    if wl.zipf_s:
        z += zipf_bias(wl.E, wl.zipf_s)[None, :]
    return z


def outlier_rows(wl: Workload) -> np.ndarray:
    n = int(round(wl.outlier_frac * wl.T))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    rng = _rng(wl.seed, _S_OUTLIER_ROWS)
    return np.sort(rng.choice(wl.T, size=n, replace=False))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (torch CPU, nearest-even); returns the uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_hidden(wl: Workload, rows_per_block: int = 8192) -> np.ndarray:
    """Hidden states, bf16 bits uint16 [T, H]: N(0,1) drawn in fp32, outlier
    rows scaled in fp32, then rounded to bf16.  Drawn block by block from one
    stream so large T never holds a full fp32 copy."""
    rng = _rng(wl.seed, _S_HIDDEN)
    out = np.empty((wl.T, wl.H), dtype=np.uint16)
    rows = outlier_rows(wl)
    for r0 in range(0, wl.T, rows_per_block):
        r1 = min(wl.T, r0 + rows_per_block)
        blk = rng.standard_normal((r1 - r0, wl.H), dtype=np.float32)
        sel = rows[(rows >= r0) & (rows < r1)] - r0
        if sel.size:
            blk[sel] *= np.float32(wl.outlier_scale)
        out[r0:r1] = f32_to_bf16_bits(blk)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32 (bit placement, no rounding)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
