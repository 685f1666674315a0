"""Seeded synthetic inputs for the attention forward path.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no attention arithmetic: only random draws, dtype casts, the fp8
quantiser that prepares fp8 inputs (outside any timed region) and the
workload descriptions.  Neither the HIP library nor the CPU reference imports
it; callers hand the same tensors to both.

Recipe: ``torch.Generator().manual_seed(seed)`` draws fp32 N(0, 1) values in
the order Q, K, V (large tensors in fixed chunks of 2**24 elements), which are
then cast with round-to-nearest-even to the storage dtype.  FP8 inputs are
quantised per tensor to OCP e4m3fn with descale = amax(|x|) / 448, the stored
value being round(x / descale).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

CHUNK = 1 << 24
FP8_MAX = 448.0

TORCH_DTYPE = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "fp8_e4m3": torch.float8_e4m3fn,
}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}


def randn(gen: torch.Generator, shape, device="cpu") -> torch.Tensor:
    """fp32 N(0,1) of ``shape`` drawn in fixed chunks from ``gen``."""
    n = math.prod(shape)
    out = torch.empty(n, dtype=torch.float32, device=device)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        out[s:e] = torch.randn(e - s, generator=gen, dtype=torch.float32,
                               device=device)
    return out.view(*shape)


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor fp8 e4m3fn quantisation: returns (codes, descale)."""
    amax = float(x.abs().max()) if x.numel() else 0.0
    descale = amax / FP8_MAX if amax > 0 else 1.0
    codes = (x / descale).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes, descale


def cast(x: torch.Tensor, dtype: str):
    """Cast fp32 draws to ``dtype``; returns (tensor, descale)."""
    if dtype == "fp8_e4m3":
        return quantize_e4m3(x)
    return x.to(TORCH_DTYPE[dtype]), 1.0


def raw_bits(t: torch.Tensor) -> np.ndarray:
    """Contiguous numpy view of a CPU tensor's storage bits."""
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"no raw view for {t.dtype}")


def cu_seqlens(lengths) -> np.ndarray:
    """[0, s0, s0+s1, ...] as int32."""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    assert out[-1] < 2**31
    return out.astype(np.int32)


@dataclasses.dataclass
class Problem:
    """One attention problem: tensors in packed [tokens, heads, dim] layout."""
    name: str
    dtype: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    q_descale: float
    k_descale: float
    v_descale: float
    lens_q: list
    lens_k: list
    varlen_q: bool
    varlen_k: bool
    hq: int
    hkv: int
    dqk: int
    dv: int
    causal: bool = False
    window: tuple = (-1, -1)

    @property
    def batch(self):
        return len(self.lens_q)

    @property
    def cu_q(self):
        return cu_seqlens(self.lens_q) if self.varlen_q else None

    @property
    def cu_k(self):
        return cu_seqlens(self.lens_k) if self.varlen_k else None

    @property
    def max_seqlen_q(self):
        return max(self.lens_q) if self.lens_q else 0

    @property
    def max_seqlen_k(self):
        return max(self.lens_k) if self.lens_k else 0


def make_problem(name, *, dtype, lens_q, lens_k, hq, hkv, dqk, dv, seed,
                 varlen_q=None, varlen_k=None, causal=False, window=(-1, -1),
                 device="cpu", shape_draws=None) -> Problem:
    """Draw Q, K, V for the given per-sequence lengths (packed along tokens).

    ``shape_draws(q32, k32, v32)``, when given, may overwrite the fp32 draws in
    place before the cast (a caller-supplied input structure, e.g. keys placed
    at chosen score heights by a test); this module computes nothing with it.
    """
    lens_q = [int(x) for x in lens_q]
    lens_k = [int(x) for x in lens_k]
    if varlen_q is None:
        varlen_q = len(set(lens_q)) > 1
    if varlen_k is None:
        varlen_k = len(set(lens_k)) > 1
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    tq, tk = sum(lens_q), sum(lens_k)
    q32 = randn(gen, (tq, hq, dqk), device)
    k32 = randn(gen, (tk, hkv, dqk), device)
    v32 = randn(gen, (tk, hkv, dv), device)
    if shape_draws is not None:
        shape_draws(q32, k32, v32)
    q, qd = cast(q32, dtype)
    del q32
    k, kd = cast(k32, dtype)
    del k32
    v, vd = cast(v32, dtype)
    del v32
    return Problem(name, dtype, q, k, v, qd, kd, vd, lens_q, lens_k, varlen_q,
                   varlen_k, hq, hkv, dqk, dv, causal, tuple(window))


# ---- the workloads ---------------------------------------------------------

GQA_DECODE_LEN_RANGE = (1024, 32768)
VARLEN_SKEWED = [4096, 512, 3072, 1024, 2560, 1536, 2048, 1536]
VARLEN_EQUAL = [2048] * 8
EDGE_LENGTHS = [1, 0, 63, 64, 65, 128, 129, 700]


def many_lengths(seed=6, batch=128, lo=64, hi=2048):
    """Lengths of a many-sequence varlen batch: uniform integers in [lo, hi]."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi, size=batch, endpoint=True)]


def gqa_decode_lengths(seed=2, batch=16):
    rng = np.random.default_rng(seed)
    lo, hi = GQA_DECODE_LEN_RANGE
    return [int(x) for x in rng.integers(lo, hi, size=batch, endpoint=True)]


def tiny(dtype="bf16", device="cpu"):
    """B=1, Hq=Hkv=4, Q=1, K=1024, D=64, seed 0."""
    return make_problem("tiny", dtype=dtype, lens_q=[1], lens_k=[1024], hq=4,
                        hkv=4, dqk=64, dv=64, seed=0, device=device)


def long_decode(device="cpu", seqlen_k=131072):
    """B=1, Q=1, K=131072, Hq=Hkv=32, D=128, bf16, seed 1."""
    return make_problem("long_decode", dtype="bf16", lens_q=[1],
                        lens_k=[seqlen_k], hq=32, hkv=32, dqk=128, dv=128,
                        seed=1, device=device)


def gqa_decode(device="cpu"):
    """B=16, Q=1, Hq=32, Hkv=8, D=128, bf16, KV lengths U[1024, 32768], seed 2."""
    lens_k = gqa_decode_lengths()
    return make_problem("gqa_decode", dtype="bf16", lens_q=[1] * 16,
                        lens_k=lens_k, hq=32, hkv=8, dqk=128, dv=128, seed=2,
                        varlen_q=False, varlen_k=True, device=device)


def fp8_prefix(seqlen_k=16384, device="cpu"):
    """B=1, Q=70, H=12, Dqk=192, Dv=128, fp8 e4m3 per-tensor scales, seed 3."""
    return make_problem(f"fp8_prefix_{seqlen_k}", dtype="fp8_e4m3", lens_q=[70],
                        lens_k=[seqlen_k], hq=12, hkv=12, dqk=192, dv=128,
                        seed=3, device=device)


def varlen_prefill(lengths="skewed", causal=False, device="cpu"):
    """fp16, Hq=Hkv=16, D=128, packed lengths (16384 tokens), seed 4."""
    lens = VARLEN_SKEWED if lengths == "skewed" else VARLEN_EQUAL
    return make_problem(f"varlen_prefill_{lengths}", dtype="f16", lens_q=lens,
                        lens_k=lens, hq=16, hkv=16, dqk=128, dv=128, seed=4,
                        varlen_q=True, varlen_k=True, causal=causal,
                        device=device)


def edge_set(causal=False, window=(128, 0), dtype="bf16", device="cpu"):
    """Lengths [1,0,63,64,65,128,129,700], Hq=8, Hkv=2, D=128, seed 5."""
    return make_problem("edge_set", dtype=dtype, lens_q=EDGE_LENGTHS,
                        lens_k=EDGE_LENGTHS, hq=8, hkv=2, dqk=128, dv=128,
                        seed=5, varlen_q=True, varlen_k=True, causal=causal,
                        window=window, device=device)
