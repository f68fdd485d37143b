"""Shared helpers of the GPU parity tests: running the ops through the C-ABI
binding and comparing with the CPU oracle.

Tolerance for floating-point outputs: |got - ref| <= 1e-2 + 1e-2 * |ref|
elementwise, with ref the oracle's exact (float64) value. Copies must be
bit-exact.
"""
import numpy as np
import torch

import oracle

TOL_ABS = 1e-2
TOL_REL = 1e-2


def note(msg: str) -> None:
    print(msg, flush=True)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def empty(shape, fill=float("nan")) -> torch.Tensor:
    """Device output pre-filled with NaN so that an unwritten element fails."""
    return torch.full(shape, fill, dtype=torch.float16, device="cuda")


def assert_close(got, ref: np.ndarray, what: str) -> None:
    g = (host(got) if isinstance(got, torch.Tensor) else np.asarray(got)).astype(np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    err = np.abs(g - ref)
    bound = TOL_ABS + TOL_REL * np.abs(ref)
    bad = ~(err <= bound)  # NaN counts as bad
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(np.isnan(err), np.inf, err - bound)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside "
                             f"|d| <= {TOL_ABS} + {TOL_REL}|ref|; worst at {idx}: "
                             f"got {g[idx]!r}, ref {ref[idx]!r}")


def assert_bits_equal(a: torch.Tensor, b, what: str) -> None:
    av = host(a).view(np.uint16)
    bv = (host(b) if isinstance(b, torch.Tensor) else np.asarray(b)).view(np.uint16)
    if not np.array_equal(av, bv):
        diff = np.argwhere(av != bv)
        raise AssertionError(f"{what}: {len(diff)} elements differ bitwise, first at {tuple(diff[0])}")


def assert_same_bits(a: torch.Tensor, b: torch.Tensor, what: str) -> None:
    """Two device tensors hold the same bits (compared on the device)."""
    ai, bi = a.view(torch.int16), b.view(torch.int16)
    if not torch.equal(ai, bi):
        n = int((ai != bi).sum().item())
        raise AssertionError(f"{what}: {n} elements differ bitwise")


def assert_exact(got: torch.Tensor, ref: np.ndarray, what: str) -> None:
    """Integer-exact case: the fp16 result must equal the exact value."""
    assert np.all(np.abs(ref) <= 2048), f"{what}: exact values exceed the fp16 integer range"
    enc = oracle.f16_encode(ref)
    assert_bits_equal(got, enc.view(np.float16), what)
