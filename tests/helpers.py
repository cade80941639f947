"""Shared helpers of the GPU tests: device transfer of storage-form arrays and error metrics."""
import numpy as np

import st_synth

# Parity bars.  bf16 outputs: max abs error 2e-2 and relative L2 error 1e-2;
# fp32 outputs: 1e-4 for both.
BF16_MAX_ABS, BF16_REL_L2 = 2e-2, 1e-2
F32_MAX_ABS, F32_REL_L2 = 1e-4, 1e-4


def torch():
    import torch as _t
    return _t


def to_dev(a: np.ndarray):
    """Storage-form numpy array (uint16 bf16 bits or float32) -> CUDA tensor (bfloat16 or float32)."""
    t = torch()
    if a.dtype == np.uint16:
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(t.bfloat16)
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def to_host(x) -> np.ndarray:
    """CUDA tensor -> storage-form numpy array."""
    t = torch()
    if x.dtype == t.bfloat16:
        return x.contiguous().view(t.int16).cpu().numpy().view(np.uint16)
    return x.contiguous().cpu().numpy()


def f64(x) -> np.ndarray:
    if not isinstance(x, np.ndarray):
        x = to_host(x)
    return st_synth.to_f64(x)


def empty(shape, bf16=True):
    t = torch()
    return t.empty(shape, dtype=t.bfloat16 if bf16 else t.float32, device="cuda")


def errors(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)) if diff.size else 0.0
    return max_abs, rel


def assert_close_stored(got, ref, what=""):
    """bf16 tensors that are stored values (q, k, v), not attention outputs: rel L2 1e-2, and
    max abs error 2e-2 or one bf16 ulp at the largest magnitude (2^-7 max|ref|), whichever is
    larger -- rounding a value of magnitude |x| to bf16 alone moves it by up to 2^-8 |x|."""
    max_abs, rel = errors(got, ref)
    lim_a = max(BF16_MAX_ABS, 2.0 ** -7 * float(np.max(np.abs(ref))) if np.size(ref) else 0.0)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_abs <= lim_a and rel <= BF16_REL_L2, f"{what}: max_abs={max_abs:.3e} (bar {lim_a:.3e}) rel_l2={rel:.3e}"
    return max_abs, rel


def assert_close(got, ref, bf16=True, what=""):
    max_abs, rel = errors(got, ref)
    lim_a, lim_r = (BF16_MAX_ABS, BF16_REL_L2) if bf16 else (F32_MAX_ABS, F32_REL_L2)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_abs <= lim_a and rel <= lim_r, f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}"
    return max_abs, rel


def bf16_round(a) -> np.ndarray:
    """float64 values rounded to bf16 storage (through fp32, nearest-even), widened back to float64."""
    return st_synth.to_f64(st_synth.f32_to_bf16_bits(np.asarray(a, np.float64).astype(np.float32)))
