"""Shared helpers of the GPU parity tests (comparison against the fp64 oracle)."""

import math

import numpy as np
import pytest
import torch

# Tolerances: fp32 inputs -> 1e-5 on O and LSE; bf16 inputs with fp32
# accumulation -> 2e-2 on O, 1e-3 on LSE (max abs error over compared elements).
TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_flashattention_amd as eta

    eta.library()  # raises if libattn.so is missing: no silent skip of the HIP path
    return torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def to_f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def max_err(got, ref):
    """Max |got - ref| over entries where ref is not NaN; equal infinities count as 0."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    sel = ~np.isnan(ref)
    g = got[sel]
    r = ref[sel]
    both_inf = np.isinf(g) & np.isinf(r) & (np.sign(g) == np.sign(r))
    with np.errstate(invalid="ignore"):
        d = np.abs(g - r)
    d[both_inf] = 0.0
    if d.size == 0:
        return 0.0
    return float(np.nanmax(np.where(np.isnan(d), np.inf, d)))


def check(o_gpu, O_ref, lse_gpu, L_ref, dtype, what=""):
    tol_o, tol_l = TOL[dtype]
    og = to_f64(o_gpu)
    lg = to_f64(lse_gpu)
    assert np.isfinite(og).all(), f"{what}: non-finite output"
    eo = max_err(og, O_ref)
    el = max_err(lg, L_ref)
    print(f"    {what} max|dO|={eo:.3e} (tol {tol_o}) max|dLSE|={el:.3e} (tol {tol_l})", flush=True)
    assert eo <= tol_o, f"{what}: O error {eo}"
    assert el <= tol_l, f"{what}: LSE error {el}"
    return eo, el


def nan_guarded(shape, dtype, device, pad=64):
    """A contiguous tensor of `shape` carved from a NaN-filled buffer with guard bands."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=dtype, device=device)
    return buf, buf[pad:pad + n].view(shape)


def guards_intact(buf, pad=64):
    head = buf[:pad].float()
    tail = buf[-pad:].float()
    return bool(torch.isnan(head).all()) and bool(torch.isnan(tail).all())


def scale_of(d):
    return 1.0 / math.sqrt(d)
