"""Helpers shared by the GPU parity tests: device transfer, poisoned outputs, checks."""
import sys

import numpy as np
import torch

import oracle

SENTINEL = 12345.0  # guard-band value after every output buffer


def announce(msg: str) -> None:
    """Print what the next GPU step is, flushed, before it runs."""
    print(f"\n[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.require(a, requirements=["C", "W"])).to("cuda")  # writable copy if needed


def poisoned(n_elems: int, guard: int = 64):
    """Output buffer of n_elems NaNs followed by a guard band of sentinels."""
    buf = torch.full((n_elems + guard,), float("nan"), dtype=torch.float32, device="cuda")
    buf[n_elems:] = SENTINEL
    return buf


def guard_intact(buf: torch.Tensor, n_elems: int) -> bool:
    return bool((buf[n_elems:] == SENTINEL).all().item())


def check_linear(got: np.ndarray, ref: np.ndarray, S: np.ndarray, what: str) -> None:
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output (unwritten element?)"
    err = np.abs(got - ref)
    tol = oracle.tol_linear(S)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} ref {ref[tuple(i)]!r} tol {tol[tuple(i)]!r}")


def check_swiglu(got, h_ref, g, u, Sg, Su, what):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - h_ref)
    tol = oracle.tol_swiglu(g, u, Sg, Su)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} out of tolerance; first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} ref {h_ref[tuple(i)]!r} tol {tol[tuple(i)]!r}")


def sample_rows(M: int, n: int, seed: int) -> np.ndarray:
    """First, last and n random rows (sorted, unique)."""
    g = np.random.default_rng(seed)
    rows = set([0, 1, M - 1, M - 2] + list(g.integers(0, M, size=n)))
    return np.array(sorted(r for r in rows if 0 <= r < M), dtype=np.int64)


def check_residual(got, ref, S, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output (unwritten element?)"
    err = np.abs(got - ref)
    tol = oracle.tol_residual(S, ref)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} ref {ref[tuple(i)]!r} tol {tol[tuple(i)]!r}")
