"""Shared helpers of the GPU parity tests (no method arithmetic here)."""
import numpy as np

F32_MAX_ABS = 2e-5      # f32 path: max |gpu - oracle|
F32_REL_L2 = 1e-5       # f32 path: ||gpu - oracle||_2 / ||oracle||_2
BF16_MAX_ABS = 2e-2     # bf16-input path: max |gpu - oracle|
# 8-bit session: the bf16 gate, and a relative-L2 bound from its one systematic rounding --
# V dequantised and the weights rounded to bf16, 2^-9 relative each (~2e-3 measured)
Q8_REL_L2 = 4e-3


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / nrm) if nrm > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_f32_parity(got, ref, what=""):
    max_abs, rel = errors(got, ref)
    print(f"{what}: max|err| {max_abs:.3e}  rel L2 {rel:.3e}", flush=True)
    assert max_abs <= F32_MAX_ABS, f"{what}: max abs error {max_abs:.3e} > {F32_MAX_ABS}"
    assert rel <= F32_REL_L2, f"{what}: relative L2 error {rel:.3e} > {F32_REL_L2}"


def assert_bf16_parity(got, ref, what=""):
    max_abs, rel = errors(got, ref)
    print(f"{what}: max|err| {max_abs:.3e}  rel L2 {rel:.3e}", flush=True)
    assert max_abs <= BF16_MAX_ABS, f"{what}: max abs error {max_abs:.3e} > {BF16_MAX_ABS}"


def eps32(w):
    """The eps the library receives (an f32), as the oracle must see it."""
    return float(np.float32(w.rms_eps))


def assert_q8_parity(got, ref, what=""):
    max_abs, rel = errors(got, ref)
    print(f"{what}: max|err| {max_abs:.3e}  rel L2 {rel:.3e}", flush=True)
    assert max_abs <= BF16_MAX_ABS, f"{what}: max abs error {max_abs:.3e} > {BF16_MAX_ABS}"
    assert rel <= Q8_REL_L2, f"{what}: relative L2 error {rel:.3e} > {Q8_REL_L2}"
