"""Helpers shared by the GPU tests: moving seeded bits between numpy and
torch device tensors, and misaligned device views."""
import sys

import numpy as np
import torch

SENTINEL_F32 = np.float32(-1234.5)          # never a sum of the test inputs
SENTINEL_BF16 = np.uint16(0xBEEF)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def bf16_view(buf: torch.Tensor, offset: int, n: int, shape):
    """A bf16 tensor of `n` elements starting `offset` elements into `buf`."""
    return buf[offset:offset + n].view(shape)


def to_dev_bf16(bits: np.ndarray, shape, offset: int = 0) -> torch.Tensor:
    n = int(np.prod(shape)) if len(shape) else 1
    buf = torch.empty(n + offset + 8, dtype=torch.bfloat16, device=dev())
    t = bf16_view(buf, offset, n, shape)
    src = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16).copy())
    t.view(-1).view(torch.int16).copy_(src.to(dev()))
    return t


def bits_of(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.detach().reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.detach().reshape(-1).cpu().numpy()
    raise TypeError(t.dtype)


def same_f32(got: np.ndarray, want: np.ndarray, what=""):
    got = np.ascontiguousarray(got, dtype=np.float32).reshape(-1)
    want = np.ascontiguousarray(want, dtype=np.float32).reshape(-1)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    gn, wn = np.isnan(got), np.isnan(want)
    bad = np.flatnonzero((gn != wn) | ((got.view(np.uint32) != want.view(np.uint32)) & ~wn))
    assert bad.size == 0, "%s: %d mismatches, first at %d: got %r want %r" % (
        what, bad.size, bad[0], got[bad[0]], want[bad[0]])


def same_u16(got: np.ndarray, want: np.ndarray, what=""):
    got = np.ascontiguousarray(got, dtype=np.uint16).reshape(-1)
    want = np.ascontiguousarray(want, dtype=np.uint16).reshape(-1)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, "%s: %d mismatches, first at %d: got %#x want %#x" % (
        what, bad.size, bad[0], got[bad[0]], want[bad[0]])
