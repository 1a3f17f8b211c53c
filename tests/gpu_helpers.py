"""Device marshalling and tolerance checks shared by the GPU tests."""
from __future__ import annotations

import numpy as np

import seeded_inputs as si

# Tolerances of the parity bar: max |gpu - oracle| <= TOL * rms(oracle) over a tensor.
TOL = {"bf16": 2e-2, "f32": 1e-5}


def torch():
    import torch as _t
    return _t


def dev(a: np.ndarray, io: str):
    """Host float32 array (already exact in the io type) -> device tensor of the io type."""
    t = torch()
    a = np.ascontiguousarray(a, dtype=np.float32)
    if io == "bf16":
        bits = si.bf16_bits(a).view(np.int16)
        return t.from_numpy(bits).view(t.bfloat16).cuda()
    return t.from_numpy(a).cuda()


def dev32(a: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t) -> np.ndarray:
    """Device tensor -> exact float64 host array."""
    tt = torch()
    return t.detach().to(tt.float32).cpu().numpy().astype(np.float64)


def empty(shape, io: str):
    t = torch()
    return t.empty(shape, dtype=t.bfloat16 if io == "bf16" else t.float32, device="cuda")


def rms(a) -> float:
    return float(np.sqrt(np.mean(np.square(a, dtype=np.float64))))


def rel_err(got, ref) -> float:
    """max |got - ref| / rms(ref) (the raw figure, output rounding included)."""
    r = rms(ref)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref))) / (r if r > 0 else 1.0)


def half_ulp(v, io: str):
    """Half the spacing of the io type's grid at |v|: the largest error that rounding
    an exact value to that type (round to nearest even) can make."""
    bits = 8 if io == "bf16" else 24          # significand bits, implicit one included
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - bits), 0.0)


def compute_err(got, ref, io: str, rounded: bool = True) -> float:
    """Error of the computation relative to rms(ref): max over elements of
    |got - ref| minus the rounding of the output to the io type (when ``rounded``),
    divided by rms(ref). The rounding slack is half an ulp at max(|got|, |ref|)."""
    got = np.asarray(got, np.float64)
    d = np.abs(got - ref)
    if rounded:
        d = np.maximum(d - half_ulp(np.maximum(np.abs(got), np.abs(ref)), io), 0.0)
    r = rms(ref)
    return float(np.max(d)) / (r if r > 0 else 1.0) if d.size else 0.0


def assert_close(got, ref, io: str, what: str = "", rounded: bool = True):
    """Parity bar: compute_err <= TOL[io]. ``rounded`` marks outputs stored in the io type
    (y, conv output); fp32 states are compared without slack."""
    e = compute_err(got, ref, io, rounded)
    raw = rel_err(got, ref)
    if e > TOL[io]:
        got_a, ref_a = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        d = np.abs(got_a - ref_a)
        if rounded:
            d = np.maximum(d - half_ulp(np.maximum(np.abs(got_a), np.abs(ref_a)), io), 0.0)
        i = np.unravel_index(int(np.argmax(d)), d.shape)
        where = f"; worst at {tuple(int(v) for v in i)}: got {got_a[i]:.9g}, ref {ref_a[i]:.9g}, " \
                f"max|ref|/rms {np.max(np.abs(ref_a)) / rms(ref_a):.3g}"
    else:
        where = ""
    assert e <= TOL[io], f"{what}: error/rms = {e:.3e} (raw {raw:.3e}) > {TOL[io]:.0e}{where}"
    return e
