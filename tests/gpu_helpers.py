"""Shared helpers of the GPU parity tests: device selection, tolerance checks
and readback of the decode layer's workspace intermediates."""
from __future__ import annotations

import numpy as np
import pytest


def cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_step_attention_layer_amd import ck

    ck.load()          # fails loudly if libck.so is missing
    return torch.device("cuda:0")


def rms(a) -> float:
    a = np.asarray(a, np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def assert_close_rms(got, ref, rel, what=""):
    """max |got - ref| <= rel * RMS(ref), NaN-free."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    bound = rel * rms(ref)
    assert err <= bound, f"{what}: max|err| {err:.3e} > {rel:g} * RMS {rms(ref):.3e}"
    return err / max(rms(ref), 1e-30)


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def ws_slice(ws, off, nbytes, dtype):
    import torch

    raw = ws[off: off + nbytes]
    a = raw.cpu().numpy()
    return a.view(dtype)
