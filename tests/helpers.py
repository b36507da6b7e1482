"""Shared helpers for the GPU parity tests: seeded inputs go to both the HIP
path and the oracle; the oracle never sees a value produced on the GPU."""
import numpy as np
import torch

# Parity bar: max |gpu - oracle| <= tol * RMS(oracle), per tensor.
TOL_F32 = 1e-4    # fp32 element type
TOL_BF16 = 2e-2   # bf16 inputs / outputs with an fp32 state


def f32np(t: torch.Tensor) -> np.ndarray:
    """Exact float32 copy of a CPU tensor (bf16 values are exact in float32)."""
    return t.detach().cpu().to(torch.float32).numpy()


def err_ratio(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0:
        return float(np.max(np.abs(gpu)))
    return float(np.max(np.abs(gpu - ref)) / rms)


def assert_parity(name, gpu, ref, tol):
    r = err_ratio(gpu, ref)
    print(f"    {name}: max|err|/rms = {r:.3e} (tol {tol:.0e})", flush=True)
    assert r <= tol, f"{name}: max|err|/rms = {r:.3e} > {tol:.0e}"
    return r


def announce(msg):
    print(f"[gpu] {msg}", flush=True)


def assert_bf16_rounded(name, gpu, ref):
    """Element-wise check of a tensor the GPU stores in bf16: within one bf16 ulp
    (2^-8 relative) of the fp64 value, plus 1e-5 RMS for fp32 arithmetic noise.
    Round-to-nearest-even alone gives at most half an ulp."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    rms = np.sqrt(np.mean(ref * ref))
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * rms
    worst = float(np.max(np.abs(gpu - ref) / bound)) if ref.size else 0.0
    print(f"    {name}: max |err| / (1 bf16 ulp) = {worst:.3f}", flush=True)
    assert worst <= 1.0, f"{name}: error exceeds one bf16 ulp (ratio {worst:.3f})"


def assert_parity_bf16_out(name, gpu, ref, tol):
    """Parity of an output the GPU stores in bf16: within tol * RMS(oracle) plus the
    output's own rounding, one bf16 ulp (2^-8 relative) of the oracle value, per element."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    rms = np.sqrt(np.mean(ref * ref))
    err = np.abs(gpu - ref)
    worst = float(np.max(err / (tol * rms + 2.0 ** -8 * np.abs(ref)))) if ref.size else 0.0
    print(f"    {name}: max|err|/rms = {float(np.max(err)) / rms if ref.size else 0.0:.3e}; "
          f"max err / (tol rms + 1 bf16 ulp) = {worst:.3f} (tol {tol:.0e})", flush=True)
    assert worst <= 1.0, f"{name}: error beyond {tol:.0e} RMS + one bf16 ulp (ratio {worst:.3f})"
