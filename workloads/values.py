"""Seeded synthetic gradient and shard values.

Gradients are bf16. Each value is an fp32 draw rounded to bf16 with
round-to-nearest-even. The distributions follow the workloads' description:
N(0, sigma) with sigma = 1e-3 for the model-shaped groups, N(0, 1) for the
worked example, and for the padding stress group N(0, 1) where each element
independently (probability 0.01) is replaced by sign * 65504 * u with a fair
random sign and u ~ U[0.5, 1) (65504 is the fp16 maximum; it rounds to 65536 in
bf16).

Draw order is contributor-major, then parameter order, so a group's values
depend only on (shapes, L, seed, distribution).

Host generators use numpy's PCG64 (``default_rng``); device generators use a
seeded ``torch.Generator`` on the GPU. The two streams differ, so each test
takes its inputs from one of them and hands the same bits to both sides.
"""
from typing import List, Sequence, Tuple

import numpy as np

OUTLIER_SCALE = 65504.0


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the uint16 bits.

    NaN inputs are not produced by the generators here; infinities pass
    through unchanged.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def _draw_values(rng: np.random.Generator, n: int, sigma: float,
                 outlier_frac: float) -> np.ndarray:
    x = rng.standard_normal(n, dtype=np.float32) * np.float32(sigma)
    if outlier_frac > 0.0:
        m = rng.random(n) < outlier_frac
        sign = rng.integers(0, 2, n).astype(np.float32) * 2.0 - 1.0
        u = rng.uniform(0.5, 1.0, n).astype(np.float32)
        x = np.where(m, sign * np.float32(OUTLIER_SCALE) * u, x).astype(np.float32)
    return fp32_to_bf16_bits(x)


def host_grads(shapes: Sequence[Tuple[int, int]], L: int, seed: int,
               sigma: float = 1.0, outlier_frac: float = 0.0) -> List[List[np.ndarray]]:
    """grads[c][p] = flat uint16 array of T_p * K_p bf16 bits (contributor c)."""
    rng = np.random.default_rng(seed)
    return [[_draw_values(rng, t * k, sigma, outlier_frac) for (t, k) in shapes]
            for _ in range(L)]


def host_special_grads(shapes: Sequence[Tuple[int, int]], L: int, seed: int,
                       allow_inf: bool = True) -> List[List[np.ndarray]]:
    """Adversarial bf16 bit patterns: uniformly random non-NaN bit patterns
    (so subnormals, huge values and both zeros all occur), mixed with small
    integers, exact zeros of both signs and, optionally, infinities."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(L):
        row = []
        for (t, k) in shapes:
            n = t * k
            bits = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
            exp = (bits >> 7) & 0xFF
            nan = (exp == 0xFF) & ((bits & 0x7F) != 0)
            bits[nan] &= np.uint16(0x807F)             # NaN -> subnormal pattern
            kind = rng.integers(0, 8, n)
            small_int = fp32_to_bf16_bits(rng.integers(-256, 257, n).astype(np.float32))
            bits = np.where(kind == 0, small_int, bits)
            bits = np.where(kind == 1, np.uint16(0x0000), bits)
            bits = np.where(kind == 2, np.uint16(0x8000), bits)
            sub = (rng.integers(1, 0x80, n) | (rng.integers(0, 2, n) << 15)).astype(np.uint16)
            bits = np.where(kind == 3, sub, bits)
            if not allow_inf:
                inf = ((bits >> 7) & 0xFF) == 0xFF
                bits[inf] &= np.uint16(0x807F)
            row.append(bits.astype(np.uint16))
        out.append(row)
    return out


def host_rank_major_bits(count: int, seed: int) -> np.ndarray:
    """Random bf16 values (N(0,1)) for a rank-major all-gather input buffer."""
    rng = np.random.default_rng(seed)
    return fp32_to_bf16_bits(rng.standard_normal(count, dtype=np.float32))


def device_grads(shapes: Sequence[Tuple[int, int]], L: int, seed: int,
                 sigma: float = 1.0, outlier_frac: float = 0.0, device="cuda",
                 progress=None):
    """grads[c][p] = a separately allocated bf16 (T_p, K_p) tensor on `device`.

    Drawn on the device from one seeded torch.Generator, contributor-major.
    `progress(c)`, if given, is called once contributor c's tensors are drawn.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for _ in range(L):
        row = []
        for (t, k) in shapes:
            x = torch.randn((t, k), generator=g, device=device, dtype=torch.float32)
            x.mul_(sigma)
            if outlier_frac > 0.0:
                m = torch.rand((t, k), generator=g, device=device) < outlier_frac
                sign = torch.randint(0, 2, (t, k), generator=g, device=device,
                                     dtype=torch.int32).to(torch.float32).mul_(2.0).sub_(1.0)
                u = torch.rand((t, k), generator=g, device=device).mul_(0.5).add_(0.5)
                x = torch.where(m, sign * OUTLIER_SCALE * u, x)
                del m, sign, u
            row.append(x.to(torch.bfloat16))
            del x
        out.append(row)
        if progress is not None:
            progress(len(out) - 1)
    return out


def device_rank_major_bits(count: int, seed: int, device="cuda"):
    """A bf16 rank-major all-gather input of `count` elements, N(0,1) values."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(count, generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)
