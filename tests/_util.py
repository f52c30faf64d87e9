"""Helpers shared by the GPU tests: device upload of the seeded inputs and
the output tolerance metric."""
import numpy as np

TOL = 1e-2   # max relative error of bf16 outputs against the oracle's float32 epilogue


def to_dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev_to_f32(t) -> np.ndarray:
    import torch
    u = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def max_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max |y - ref| / max(|ref|, 1e-2 * rms(ref)); the floor keeps outputs
    that cancel to ~0 (bias) from dividing by ~0."""
    ref = ref.astype(np.float64)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 1.0
    den = np.maximum(np.abs(ref), 1e-2 * rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(y.astype(np.float64) - ref) / den)) if ref.size else 0.0
