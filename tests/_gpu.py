"""Helpers shared by the GPU parity tests (device transfer, bf16 views, the tolerance rule)."""
import numpy as np
import torch

import oracle

TOL = 2e-3   # max |err| per output <= TOL * sum |scale * w * x| over that output's row


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev())


def empty_bf16(*shape):
    return torch.empty(shape, dtype=torch.int16, device=dev())


def bits(t) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def check_within(y_bits, ref, l1, what=""):
    """Asserts the float-path tolerance element by element; zero bound requires +-0."""
    y = oracle.bf16_to_f64(np.asarray(y_bits))
    err = np.abs(y - ref)
    # NaN fails unless the oracle's value is NaN too
    bad = ~(err <= TOL * l1) & ~(np.isnan(y) & np.isnan(ref))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outputs out of tolerance; first at {tuple(i)}: "
            f"gpu={y[tuple(i)]!r} ref={ref[tuple(i)]!r} l1={l1[tuple(i)]!r}")
    return float((err / np.maximum(l1, 1e-300)).max()) if err.size else 0.0


def bf16_ordinal(b):
    """Monotone integer order of bf16 bit patterns (for 'within one ulp' comparisons)."""
    b = np.asarray(b).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)
