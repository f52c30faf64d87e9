"""Seeded synthetic inputs for the ConvRot-quantized linear.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds only random-number draws and the bf16 storage cast; none
of the method's arithmetic (rotation, scales, quantisation, GEMM, epilogue)
lives here.

Workloads (shapes and distributions) stand in for the real models the model
cards measure (Qwen-Image-Edit-2511 DiT, Qwen3-VL-4B text encoder, Z-Image
Turbo), whose weights and prompts are not available:

* ``tiny``      x [64,512] N(0,1), 4 outlier channels x30; W [256,512] N(0,0.02)
* ``te``        x [M,2560] N(0,1), 0.5% outlier channels x40; W gate/up
                [9728,2560], down [2560,9728] N(0,0.02); M in {76, 1220}
* ``dit``       x [4096,3072] Student-t(nu=3), 1% outlier channels x50;
                W1 [12288,3072], W2 [3072,12288] N(0,0.02); bias N(0,0.01)
* ``int8tw``    x N(0,1), W N(0,0.02): V/O [3072,3072] at M=4096, and a
                K=2688 layer (2688 is not a multiple of 256) with N=2688
* ``w4a8``      x [4096,3840] N(0,1); W [10240,3840] N(0,0.02)

Draw order per (workload, layer) with a fresh ``np.random.default_rng(seed)``:
W, then x, then the outlier column indices (``choice(K, n, replace=False)``,
n = round(p*K)), then the bias.  Values are drawn in float64, stored as float32
(round to nearest even) and then as bf16 (round to nearest even on the float32
bit pattern).  bf16 tensors are carried as ``uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses

import numpy as np


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Storage cast float32 -> bf16 bit pattern, round to nearest even.

    Inputs are finite (the generators draw no NaN/Inf)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> float32 (exact widening)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class LayerInputs:
    """One linear layer's synthetic inputs (bf16 bit patterns)."""
    name: str
    x: np.ndarray          # uint16 [M, K]
    w: np.ndarray          # uint16 [N, K]
    bias: np.ndarray | None  # uint16 [N] or None

    @property
    def M(self) -> int:
        return self.x.shape[0]

    @property
    def K(self) -> int:
        return self.x.shape[1]

    @property
    def N(self) -> int:
        return self.w.shape[0]


def _outlier_count(frac: float, K: int) -> int:
    return int(round(frac * K))


def make_layer(name: str, M: int, K: int, N: int, *, seed: int,
               x_dist: str = "normal", outlier_frac: float = 0.0,
               outlier_count: int | None = None, outlier_scale: float = 1.0,
               w_std: float = 0.02, bias_std: float | None = None,
               t_nu: float = 3.0) -> LayerInputs:
    """Draw one layer: W, then x, then outlier columns, then bias."""
    rng = np.random.default_rng(seed)
    w = rng.normal(0.0, w_std, size=(N, K)).astype(np.float32)
    if x_dist == "normal":
        x = rng.normal(0.0, 1.0, size=(M, K)).astype(np.float32)
    elif x_dist == "student_t":
        x = rng.standard_t(t_nu, size=(M, K)).astype(np.float32)
    else:
        raise ValueError(f"unknown x distribution {x_dist!r}")
    n_out = outlier_count if outlier_count is not None else _outlier_count(outlier_frac, K)
    if n_out > 0:
        cols = rng.choice(K, n_out, replace=False)
        x[:, cols] *= np.float32(outlier_scale)
    bias = None
    if bias_std is not None:
        bias = f32_to_bf16_bits(rng.normal(0.0, bias_std, size=(N,)).astype(np.float32))
    return LayerInputs(name, f32_to_bf16_bits(x), f32_to_bf16_bits(w), bias)


# ---------------------------------------------------------------------------
# The workloads.
# ---------------------------------------------------------------------------

def tiny(seed: int = 0) -> LayerInputs:
    return make_layer("tiny", 64, 512, 256, seed=seed, outlier_count=4, outlier_scale=30.0)


def te_gate_up(M: int = 76, seed: int = 0) -> LayerInputs:
    return make_layer(f"te_gate_up_M{M}", M, 2560, 9728, seed=seed,
                      outlier_frac=0.005, outlier_scale=40.0)


def te_down(M: int = 76, seed: int = 1) -> LayerInputs:
    return make_layer(f"te_down_M{M}", M, 9728, 2560, seed=seed,
                      outlier_frac=0.005, outlier_scale=40.0)


def te_attn_proj(M: int = 76, seed: int = 2) -> LayerInputs:
    """Stand-in for a text-encoder attention projection in the ConvRot INT8
    row-scaled format: square, at the encoder's hidden width (the pages give
    the format's role, not the layer dimensions)."""
    return make_layer(f"te_attn_proj_M{M}", M, 2560, 2560, seed=seed,
                      outlier_frac=0.005, outlier_scale=40.0)


def te_mlp(M: int = 76):
    """Text-encoder MLP block inputs (hidden 2560, intermediate 9728): x and the
    gate weight from te_gate_up(M), the up weight from te_gate_up(M, seed=3),
    the down weight from te_down(M).  Returns (x, w_gate, w_up, w_down) as bf16
    bit patterns."""
    g = te_gate_up(M)
    return g.x, g.w, te_gate_up(M, seed=3).w, te_down(M).w


def dit_w1(M: int = 4096, seed: int = 0) -> LayerInputs:
    return make_layer(f"dit_w1_M{M}", M, 3072, 12288, seed=seed, x_dist="student_t",
                      outlier_frac=0.01, outlier_scale=50.0, bias_std=0.01)


def dit_w2(M: int = 4096, seed: int = 1) -> LayerInputs:
    return make_layer(f"dit_w2_M{M}", M, 12288, 3072, seed=seed, x_dist="student_t",
                      outlier_frac=0.01, outlier_scale=50.0, bias_std=0.01)


def int8tw_vo(M: int = 4096, seed: int = 0) -> LayerInputs:
    return make_layer(f"int8tw_vo_M{M}", M, 3072, 3072, seed=seed)


def int8tw_k2688(M: int = 4096, seed: int = 1) -> LayerInputs:
    return make_layer(f"int8tw_k2688_M{M}", M, 2688, 2688, seed=seed)


def w4a8_layer(M: int = 4096, seed: int = 0) -> LayerInputs:
    return make_layer(f"w4a8_M{M}", M, 3840, 10240, seed=seed)


def random_layer(M: int, K: int, N: int, seed: int, *, bias: bool = False,
                 outlier_count: int = 0, outlier_scale: float = 30.0) -> LayerInputs:
    """Small generic layer for parity sweeps over ragged shapes."""
    return make_layer(f"rand_M{M}_K{K}_N{N}", M, K, N, seed=seed,
                      outlier_count=min(outlier_count, K), outlier_scale=outlier_scale,
                      bias_std=0.01 if bias else None)


def random_w4a8_format(N: int, K: int, seed: int):
    """Random tensors in the W4A8 storage format (for shape/edge tests).

    Returns (idx packed uint8 [N, K/2] low nibble = even k, s_rel e4m3 bytes
    [N, K/16], codebook float32 [16] sorted, s_channel float32 [N]).
    The e4m3 bytes are drawn from positive, finite codes 0x20..0x5F
    (2^-3 .. 2^4 range), the codebook levels from N(0, 0.5)."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s_rel = rng.integers(0x20, 0x60, size=(N, K // 16), dtype=np.uint8)
    cb = np.sort(rng.normal(0.0, 0.5, size=16).astype(np.float32))
    s_ch = np.abs(rng.normal(0.0, 1e-3, size=N)).astype(np.float32) + np.float32(1e-5)
    return idx, s_rel, cb, s_ch
