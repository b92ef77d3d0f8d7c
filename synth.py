"""Seeded synthetic inputs for the N-rank reduction -- shared by tests, the
benchmark and the oracle checks.

This module only draws random data; it holds none of the reduction's
arithmetic.  Rank r of a workload is drawn from its own generator seeded with
``seed0 + r``.  Floating-point data is drawn in float32 by torch and converted
to the storage type with torch's own cast; FP8 E4M3B15 data is a uniform draw
over the 240 codes whose exponent field is not all ones (the finite codes,
every one of them in [-0.9375, 0.9375]).
"""
from __future__ import annotations

import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
                "fp8": torch.uint8, "fp8fn": torch.uint8}
ELEM_SIZE = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "fp8fn": 1}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(t: str, count: int, seed: int, device="cpu") -> torch.Tensor:
    """~N(0,1) drawn in float32, stored as type t."""
    x = torch.randn(count, dtype=torch.float32, generator=_gen(seed, device), device=device)
    return x.to(TORCH_DTYPES[t])


def uniform(t: str, count: int, seed: int, lo=-1.0, hi=1.0, device="cpu") -> torch.Tensor:
    """~U(lo, hi) drawn in float32, stored as type t."""
    x = torch.rand(count, dtype=torch.float32, generator=_gen(seed, device), device=device)
    return (x * (hi - lo) + lo).to(TORCH_DTYPES[t])


def fp8_finite_codes(count: int, seed: int, device="cpu") -> torch.Tensor:
    """Uniform over the 240 finite FP8 E4M3B15 codes: 0x00..0x77, 0x80..0xF7."""
    j = torch.randint(0, 240, (count,), generator=_gen(seed, device), device=device,
                      dtype=torch.int32)
    codes = torch.where(j < 120, j, j - 120 + 0x80)
    return codes.to(torch.uint8)


def fp8fn_finite_codes(count: int, seed: int, device="cpu") -> torch.Tensor:
    """Uniform over the 254 finite OCP FP8 E4M3FN codes (all but 0x7F, 0xFF)."""
    j = torch.randint(0, 254, (count,), generator=_gen(seed, device), device=device,
                      dtype=torch.int32)
    codes = torch.where(j < 127, j, j - 127 + 0x80)
    return codes.to(torch.uint8)


def rank_inputs(kind: str, t: str, nranks: int, count: int, seed0: int = 0,
                device="cpu") -> list[torch.Tensor]:
    """One buffer per simulated rank; rank r uses seed seed0 + r.

    kind: "normal" (~N(0,1)), "uniform" (~U(-1,1)) or "fp8codes" (uniform over
    the finite codes of t = "fp8" (E4M3B15) or "fp8fn" (OCP E4M3FN)).
    """
    out = []
    for r in range(nranks):
        if kind == "normal":
            out.append(normal(t, count, seed0 + r, device))
        elif kind == "uniform":
            out.append(uniform(t, count, seed0 + r, device=device))
        elif kind == "fp8codes":
            assert t in ("fp8", "fp8fn")
            gen = fp8_finite_codes if t == "fp8" else fp8fn_finite_codes
            out.append(gen(count, seed0 + r, device))
        else:
            raise ValueError(kind)
    return out


def to_bits_numpy(x: torch.Tensor):
    """Raw bits of a CPU/GPU tensor as a numpy array (float32 stays float32,
    16-bit types become uint16 codes, FP8 stays uint8)."""
    x = x.detach().contiguous().cpu()
    if x.dtype in (torch.float16, torch.bfloat16):
        return x.view(torch.int16).numpy().view("uint16")
    return x.numpy()
