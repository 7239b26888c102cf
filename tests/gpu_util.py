"""Helpers for GPU parity tests: host <-> device transfers and the tolerance rule."""

import numpy as np
import torch


def dev_bf16(a):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on cuda:0."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    return t.detach().cpu().numpy()


def host_bf16_bits(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_close_rms(got, ref, frac=1e-2, what="output"):
    """max |got - ref| <= frac * RMS(ref) over the whole tensor (the parity bar for outputs)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(got - ref).max()
    print(f"[parity] {what}: max|err|/RMS = {err / rms:.3e} (bar {frac})")
    assert err <= frac * rms, f"{what}: max|err| {err:.3e} > {frac} * RMS {rms:.3e} (ratio {err / rms:.2e})"
    return err / rms


def assert_lse_close(got, ref, tol=1e-3, rel=0.0):
    """|got - ref| <= tol + rel * max|ref| over the finite entries (the -inf pattern must match).

    ``rel`` scales the bound with the logits for workloads whose logits are far
    from O(1) (their fp32 logits carry an error relative to their size)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    assert (np.isfinite(got) == fin).all(), "lse: -inf pattern differs"
    if fin.any():
        err = np.abs(got[fin] - ref[fin]).max()
        bound = tol + rel * np.abs(ref[fin]).max()
        print(f"[parity] lse: max|err| = {err:.3e} (bound {bound:.3e}, max|lse| {np.abs(ref[fin]).max():.1f})")
        assert err <= bound, f"lse: max|err| {err:.3e} > {bound:.3e}"
