"""ConvRot-quantized linear forward on MI355X (gfx950).

Thin ctypes binding over ``libconvrot.so`` (C ABI in ``include/convrot.h``).
Every step of the computation runs in the library's HIP kernels; this module
only checks tensors, passes device pointers and the current stream, and uses
torch as the device-memory allocator.  There is no CPU fallback: if the
library is missing or the device is not a gfx950, calls raise.

Formats (model cards cited by title and section):
  * W4A4 ConvRot  - [QIE] "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4
    (+ConvRot, mixed int8 fallback)", intro: INT4 weights two per byte with a
    group-256 Hadamard rotation, INT4 activations quantised in the kernel.
  * int8_tensorwise - same card, intro; [REB] "Rebels_w4a8s", "Mixed formats
    where the kernel demands it": used for layers whose K is not a multiple
    of 256.
  * asym W4A8 codebook - [REB] "What's inside a file".
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

__all__ = [
    "W4A4", "INT8TW", "W4A8", "INT8ROT", "W4A4_G64", "W4A4_G16", "W4A4_RH", "ConvRotError", "lib", "packed_bytes", "workspace_bytes",
    "pack_weight_w4", "pack_weight_int8tw", "pack_weight_w4a8", "pack_weight_int8rot",
    "linear_w4a4", "linear_int8tw", "linear_w4a8", "linear_int8rot",
    "pack_weight_w4_regular", "linear_w4a4_regular",
    "mlp_workspace_bytes", "mlp_w4a4", "dbg_quant_swiglu", "dbg_silu_mul",
    "dbg_quant_act", "dbg_unpack_weight", "dbg_linear_acc",
    "quantize_activations", "gemm_quantized",
    "PackedWeight", "pack_linear", "linear",
    "probe_mfma_i8", "probe_read", "probe_copy", "probe_wall_clock_khz",
    "linear_w4a4_noalloc", "NOALLOC_SCRATCH_BYTES",
    "encode_w4a8", "encode_w4a8_workspace_bytes", "dbg_e4m3_encode",
    "dbg_fused_config", "dbg_fused_timeouts", "dbg_big_plan", "dbg_small_plan",
]

W4A4, INT8TW, W4A8, INT8ROT, W4A4_G64, W4A4_G16, W4A4_RH = 0, 1, 2, 3, 4, 5, 6
# W4A4 kind of each rotation group size
W4_GROUP_KIND = {256: W4A4, 64: W4A4_G64, 16: W4A4_G16}
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libconvrot.so")
_LIB = None

_STATUS = {0: "CR_OK", 1: "CR_ERR_NULL", 2: "CR_ERR_SHAPE", 3: "CR_ERR_GROUP", 4: "CR_ERR_ALIGN",
           5: "CR_ERR_WORKSPACE", 6: "CR_ERR_DEVICE", 7: "CR_ERR_LAUNCH", 8: "CR_ERR_KIND"}

EXPORTS = [
    "cr_packed_bytes", "cr_workspace_bytes", "cr_pack_weight_w4", "cr_linear_w4a4",
    "cr_pack_weight_int8tw", "cr_linear_int8tw", "cr_pack_weight_w4a8", "cr_linear_w4a8",
    "cr_status_str", "cr_last_error", "cr_dbg_quant_act", "cr_dbg_unpack_weight",
    "cr_dbg_linear_acc", "cr_quantize_activations", "cr_gemm_quantized",
    "cr_pack_weight_int8rot", "cr_linear_int8rot",
    "cr_pack_weight_w4_group", "cr_linear_w4a4_group",
    "cr_pack_weight_w4_regular", "cr_linear_w4a4_regular",
    "cr_mlp_workspace_bytes", "cr_mlp_w4a4", "cr_dbg_quant_swiglu", "cr_dbg_silu_mul",
    # measurement probes (include/convrot_probe.h)
    "cr_probe_mfma_i8", "cr_probe_read", "cr_probe_copy", "cr_probe_wall_clock_khz",
    "cr_linear_w4a4_noalloc",
    "cr_encode_w4a8_workspace_bytes", "cr_encode_w4a8", "cr_dbg_e4m3_encode",
    "cr_dbg_fused_config", "cr_dbg_fused_timeouts", "cr_dbg_big_plan", "cr_dbg_small_plan",
]


class ConvRotError(RuntimeError):
    """A library call returned a non-OK status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libconvrot.so (built in-tree by ``build_lib``)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m rotated_bit_quantized_convrot_amd.build_lib`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "cr_packed_bytes": (sz, [i, i, i]),
        "cr_workspace_bytes": (sz, [i, i, i, i]),
        "cr_pack_weight_w4": (i, [vp, i, i, vp, vp, vp]),
        "cr_pack_weight_int8tw": (i, [vp, i, i, vp, vp, vp]),
        "cr_pack_weight_w4a8": (i, [vp, vp, vp, i, i, vp, vp]),
        "cr_pack_weight_int8rot": (i, [vp, i, i, vp, vp, vp]),
        "cr_linear_int8rot": (i, [vp, i, i, vp, vp, i, vp, vp, vp, sz, vp]),
        "cr_pack_weight_w4_group": (i, [vp, i, i, i, vp, vp, vp]),
        "cr_linear_w4a4_group": (i, [vp, i, i, i, vp, vp, i, vp, vp, vp, sz, vp]),
        "cr_pack_weight_w4_regular": (i, [vp, i, i, vp, vp, vp]),
        "cr_linear_w4a4_regular": (i, [vp, i, i, vp, vp, i, vp, vp, vp, sz, vp]),
        "cr_mlp_workspace_bytes": (sz, [i, i, i, i]),
        "cr_mlp_w4a4": (i, [vp, i, i, vp, vp, vp, vp, i, vp, vp, i, vp, vp, sz, vp]),
        "cr_dbg_quant_swiglu": (i, [vp, vp, i, i, vp, vp, vp]),
        "cr_dbg_silu_mul": (i, [vp, vp, sz, vp, vp]),
        "cr_linear_w4a4": (i, [vp, i, i, vp, vp, i, vp, vp, vp, sz, vp]),
        "cr_linear_w4a4_noalloc": (i, [vp, i, i, vp, vp, i, vp, vp, vp]),
        "cr_encode_w4a8_workspace_bytes": (sz, [i, i]),
        "cr_encode_w4a8": (i, [vp, i, i, i, vp, vp, vp, vp, vp, sz, vp]),
        "cr_dbg_e4m3_encode": (i, [vp, sz, vp, vp]),
        "cr_dbg_fused_config": (i, [i, i]),
        "cr_dbg_fused_timeouts": (i, [vp]),
        "cr_dbg_big_plan": (i, [i, i]),
        "cr_dbg_small_plan": (i, [i]),
        "cr_linear_int8tw": (i, [vp, i, i, vp, vp, i, vp, vp, vp, sz, vp]),
        "cr_linear_w4a8": (i, [vp, i, i, vp, vp, i, vp, vp, vp, sz, vp]),
        "cr_status_str": (ctypes.c_char_p, [i]),
        "cr_last_error": (ctypes.c_char_p, []),
        "cr_dbg_quant_act": (i, [i, vp, i, i, vp, vp, vp]),
        "cr_dbg_unpack_weight": (i, [i, vp, i, i, vp, vp]),
        "cr_dbg_linear_acc": (i, [i, vp, i, i, vp, i, vp, vp, sz, vp]),
        "cr_quantize_activations": (i, [i, vp, i, i, vp, sz, vp]),
        "cr_gemm_quantized": (i, [i, i, i, vp, vp, i, vp, vp, vp, sz, vp]),
        "cr_probe_mfma_i8": (i, [i, i, vp, vp, vp]),
        "cr_probe_read": (i, [vp, sz, vp, vp]),
        "cr_probe_copy": (i, [vp, vp, sz, vp]),
        "cr_probe_wall_clock_khz": (i, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _LIB = L
    return L


def _check(status: int):
    if status != 0:
        raise ConvRotError(status, lib().cr_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def packed_bytes(kind: int, N: int, K: int) -> int:
    return int(lib().cr_packed_bytes(kind, N, K))


def workspace_bytes(kind: int, M: int, N: int, K: int) -> int:
    return int(lib().cr_workspace_bytes(kind, M, N, K))


def _empty_u8(n: int, device) -> torch.Tensor:
    return torch.empty(max(int(n), 16), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# Weight preparation (offline)
# ---------------------------------------------------------------------------

def pack_weight_w4(w: torch.Tensor, group: int = 256):
    """bf16 [N,K] -> (packed uint8, scale float32[1]) in the W4A4 format,
    rotated in groups of ``group`` (256, 64 or 16)."""
    _dev(w, "w", torch.bfloat16)
    N, K = w.shape
    nb = packed_bytes(W4A4, N, K)
    if nb == 0:
        _check(lib().cr_pack_weight_w4(_ptr(w), N, K, None, None, None) or 2)
    out = _empty_u8(nb, w.device)
    scale = torch.empty(4, dtype=torch.float32, device=w.device)
    if group == 256:
        _check(lib().cr_pack_weight_w4(_ptr(w), N, K, _ptr(out), _ptr(scale), _stream()))
    else:
        _check(lib().cr_pack_weight_w4_group(_ptr(w), N, K, group, _ptr(out), _ptr(scale), _stream()))
    return out, scale


def pack_weight_w4_regular(w: torch.Tensor):
    """bf16 [N,K] -> (packed uint8, scale float32[1]) in the W4A4 format with
    the group-256 regular Hadamard rotation."""
    _dev(w, "w", torch.bfloat16)
    N, K = w.shape
    nb = packed_bytes(W4A4_RH, N, K)
    if nb == 0:
        _check(lib().cr_pack_weight_w4_regular(_ptr(w), N, K, None, None, None) or 2)
    out = _empty_u8(nb, w.device)
    scale = torch.empty(4, dtype=torch.float32, device=w.device)
    _check(lib().cr_pack_weight_w4_regular(_ptr(w), N, K, _ptr(out), _ptr(scale), _stream()))
    return out, scale


def pack_weight_int8tw(w: torch.Tensor):
    """bf16 [N,K] -> (packed uint8, scale float32[1]) in the int8_tensorwise format."""
    _dev(w, "w", torch.bfloat16)
    N, K = w.shape
    nb = packed_bytes(INT8TW, N, K)
    if nb == 0:
        _check(lib().cr_pack_weight_int8tw(_ptr(w), N, K, None, None, None) or 2)
    out = _empty_u8(nb, w.device)
    scale = torch.empty(4, dtype=torch.float32, device=w.device)
    _check(lib().cr_pack_weight_int8tw(_ptr(w), N, K, _ptr(out), _ptr(scale), _stream()))
    return out, scale


def pack_weight_int8rot(w: torch.Tensor):
    """bf16 [N,K] -> (packed uint8, row scales float32[N]) in the ConvRot INT8
    row-scaled format (K % 256 == 0)."""
    _dev(w, "w", torch.bfloat16)
    N, K = w.shape
    nb = packed_bytes(INT8ROT, N, K)
    if nb == 0:
        _check(lib().cr_pack_weight_int8rot(_ptr(w), N, K, None, None, None) or 2)
    out = _empty_u8(nb, w.device)
    scale = torch.empty(max(N, 4), dtype=torch.float32, device=w.device)
    _check(lib().cr_pack_weight_int8rot(_ptr(w), N, K, _ptr(out), _ptr(scale), _stream()))
    return out, scale


def pack_weight_w4a8(idx: torch.Tensor, s_rel: torch.Tensor, codebook: torch.Tensor, N: int, K: int):
    """Stored W4A8 tensors -> packed uint8 (index nibbles [N,K/2], e4m3 scale
    codes [N,K/16] as uint8, codebook float32[16])."""
    _dev(idx, "idx", torch.uint8)
    _dev(s_rel, "s_rel", torch.uint8)
    _dev(codebook, "codebook", torch.float32)
    if idx.numel() != N * K // 2 or s_rel.numel() != N * K // 16 or codebook.numel() != 16:
        raise ValueError("W4A8 tensor sizes do not match N, K")
    nb = packed_bytes(W4A8, N, K)
    if nb == 0:
        _check(lib().cr_pack_weight_w4a8(_ptr(idx), _ptr(s_rel), _ptr(codebook), N, K, None, None) or 2)
    out = _empty_u8(nb, idx.device)
    _check(lib().cr_pack_weight_w4a8(_ptr(idx), _ptr(s_rel), _ptr(codebook), N, K, _ptr(out), _stream()))
    return out


def encode_w4a8_workspace_bytes(N: int, K: int) -> int:
    return int(lib().cr_encode_w4a8_workspace_bytes(N, K))


def encode_w4a8(w: torch.Tensor, iters: int = 100, workspace=None):
    """bf16 [N,K] -> the stored W4A8 tensors (idx uint8 [N,K/2], s_rel e4m3
    uint8 [N,K/16], codebook float32 [16], s_channel float32 [N]), encoded on
    the GPU with at most ``iters`` Lloyd-Max iterations."""
    _dev(w, "w", torch.bfloat16)
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    N, K = w.shape
    need = encode_w4a8_workspace_bytes(N, K)
    if workspace is None:
        workspace = _empty_u8(max(need, 256), w.device)
    else:
        _dev(workspace, "workspace", torch.uint8)
        _same_device(w, workspace=workspace)
    idx = torch.empty((N, max(K // 2, 1)), dtype=torch.uint8, device=w.device)
    s_rel = torch.empty((N, max(K // 16, 1)), dtype=torch.uint8, device=w.device)
    cb = torch.empty(16, dtype=torch.float32, device=w.device)
    sch = torch.empty(max(N, 1), dtype=torch.float32, device=w.device)
    _check(lib().cr_encode_w4a8(_ptr(w), N, K, iters, _ptr(idx), _ptr(s_rel), _ptr(cb), _ptr(sch),
                                _ptr(workspace), workspace.numel(), _stream()))
    return idx, s_rel, cb, sch[:N]


def dbg_e4m3_encode(v: torch.Tensor) -> torch.Tensor:
    """E4M3FN codes (uint8) of non-negative float32 values <= 448, as the
    encoder rounds its group scales."""
    _dev(v, "v", torch.float32)
    out = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _check(lib().cr_dbg_e4m3_encode(_ptr(v), v.numel(), _ptr(out), _stream()))
    return out


def dbg_fused_config(mode: int, spin_limit: int = -1) -> None:
    """Path of the small-M W4A4 linear: 1 = one launch that quantises its own
    activations where it applies and M <= 8 (the default), 2 = that launch
    wherever it applies, 0 = always the activation quantiser and the GEMM;
    ``spin_limit >= 0`` sets the polls of the fused launch's bounded wait."""
    _check(lib().cr_dbg_fused_config(int(mode), int(spin_limit)))


def dbg_big_plan(bn: int = 0, splits: int = 0) -> None:
    """Large-M GEMM plan for later calls: block tiles 256 x ``bn`` (256, 192,
    128 or 64) and ``splits`` K slices across blocks; 0 keeps the planner's
    choice.  Size workspaces after setting it."""
    _check(lib().cr_dbg_big_plan(int(bn), int(splits)))


def dbg_small_plan(splits: int = 0) -> None:
    """Small-M GEMM plan for later calls: ``splits`` K slices across blocks
    where that count fits the plan; 0 keeps the planner's choice.  Size
    workspaces after setting it."""
    _check(lib().cr_dbg_small_plan(int(splits)))


def dbg_fused_timeouts() -> int:
    """GEMM blocks of the fused linear whose wait ran out, on the current
    device, since the library was loaded (synchronises the device)."""
    n = ctypes.c_uint32(0)
    _check(lib().cr_dbg_fused_timeouts(ctypes.byref(n)))
    return int(n.value)


# ---------------------------------------------------------------------------
# Linears
# ---------------------------------------------------------------------------

def _same_device(first: torch.Tensor, **others):
    """Every tensor passed must live on ``first``'s device: the kernels take
    raw pointers and would fault on another GPU's memory."""
    for name, t in others.items():
        if t is not None and t.device != first.device:
            raise ValueError(f"{name} is on {t.device}, expected {first.device}")


def _check_weight(kind: int, packed, scale, N: int, K: int):
    """Refuse packed weights and scales smaller than the layout of (kind, N,
    K) needs: the kernels would read past their end.  (Shapes the library
    rejects give 0 bytes here and are left to its own error.)"""
    need = packed_bytes(kind, N, K)
    if need and packed.numel() < need:
        raise ValueError(f"packed weight has {packed.numel()} bytes, kind {kind} N={N} K={K} needs {need}")
    per_row = kind in (W4A8, INT8ROT)
    if scale is not None and scale.numel() < (N if per_row else 1):
        raise ValueError(f"scale has {scale.numel()} values, needs {N if per_row else 1}")


def _linear(fn_name: str, kind: int, x, packed, scale, N, bias, out, workspace, group=None):
    _dev(x, "x", torch.bfloat16)
    _dev(packed, "packed", torch.uint8)
    _dev(scale, "scale", torch.float32)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    _check_weight(kind, packed, scale, N, K)
    _same_device(x, packed=packed, scale=scale, bias=bias, out=out, workspace=workspace)
    if bias is not None:
        _dev(bias, "bias", torch.bfloat16)
        if bias.numel() != N:
            raise ValueError("bias must have N elements")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _dev(out, "out", torch.bfloat16)
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N]")
    need = workspace_bytes(kind, M, N, K)
    if need == 0:  # invalid shapes: let the library report the reason
        need = 256
    if workspace is None:
        workspace = _empty_u8(need, x.device)
    else:
        _dev(workspace, "workspace", torch.uint8)
    fn = getattr(lib(), fn_name)
    lead = (_ptr(x), M, K) if group is None else (_ptr(x), M, K, group)
    _check(fn(*lead, _ptr(packed), _ptr(scale), N, _ptr(bias), _ptr(out),
              _ptr(workspace), workspace.numel(), _stream()))
    return out


def linear_w4a4(x, packed, scale, N, bias=None, out=None, workspace=None, group: int = 256):
    """y = ConvRot W4A4 linear (x bf16 [M,K], K % 256 == 0), rotation groups
    of ``group`` (the group the weight was packed with)."""
    if group == 256:
        return _linear("cr_linear_w4a4", W4A4, x, packed, scale, N, bias, out, workspace)
    return _linear("cr_linear_w4a4_group", W4_GROUP_KIND.get(group, W4A4), x, packed, scale, N, bias, out,
                   workspace, group=group)


NOALLOC_SCRATCH_BYTES = 8 << 20


def linear_w4a4_noalloc(x, packed, scale, N, bias=None, out=None):
    """cr_linear_w4a4_noalloc: the W4A4 linear with the library's static
    scratch as its workspace (the C call allocates nothing; ``out`` is
    allocated here when not given).  Shapes whose workspace exceeds
    NOALLOC_SCRATCH_BYTES raise."""
    _dev(x, "x", torch.bfloat16)
    _dev(packed, "packed", torch.uint8)
    _dev(scale, "scale", torch.float32)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    _check_weight(W4A4, packed, scale, N, K)
    _same_device(x, packed=packed, scale=scale, bias=bias, out=out)
    if bias is not None:
        _dev(bias, "bias", torch.bfloat16)
        if bias.numel() != N:
            raise ValueError("bias must have N elements")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _dev(out, "out", torch.bfloat16)
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N]")
    _check(lib().cr_linear_w4a4_noalloc(_ptr(x), M, K, _ptr(packed), _ptr(scale), N, _ptr(bias), _ptr(out),
                                        _stream()))
    return out


def linear_w4a4_regular(x, packed, scale, N, bias=None, out=None, workspace=None):
    """y = W4A4 linear with the group-256 regular Hadamard rotation (weight from
    pack_weight_w4_regular)."""
    return _linear("cr_linear_w4a4_regular", W4A4_RH, x, packed, scale, N, bias, out, workspace)


def linear_int8tw(x, packed, scale, N, bias=None, out=None, workspace=None):
    """y = int8_tensorwise linear (any K)."""
    return _linear("cr_linear_int8tw", INT8TW, x, packed, scale, N, bias, out, workspace)


def linear_int8rot(x, packed, scale, N, bias=None, out=None, workspace=None):
    """y = ConvRot INT8 row-scaled linear (K % 256 == 0); scale float32 [N]."""
    return _linear("cr_linear_int8rot", INT8ROT, x, packed, scale, N, bias, out, workspace)


def linear_w4a8(x, packed, s_channel, N, bias=None, out=None, workspace=None):
    """y = asym W4A8 codebook linear; s_channel float32 [N]."""
    return _linear("cr_linear_w4a8", W4A8, x, packed, s_channel, N, bias, out, workspace)


# ---------------------------------------------------------------------------
# Text-encoder MLP block
# ---------------------------------------------------------------------------

def mlp_workspace_bytes(M: int, K: int, F: int, N: int) -> int:
    return int(lib().cr_mlp_workspace_bytes(M, K, F, N))


def mlp_w4a4(x, wg, sg, wu, su, F, wd, sd, N, out=None, workspace=None):
    """y = down(silu(gate(x)) * up(x)) with W4A4 ConvRot linears (weights from
    pack_weight_w4: gate and up [F,K], down [N,F]; no biases)."""
    _dev(x, "x", torch.bfloat16)
    for t, n in ((wg, "wg"), (wu, "wu"), (wd, "wd")):
        _dev(t, n, torch.uint8)
    for t, n in ((sg, "sg"), (su, "su"), (sd, "sd")):
        _dev(t, n, torch.float32)
    M, K = x.shape
    _check_weight(W4A4, wg, sg, F, K)
    _check_weight(W4A4, wu, su, F, K)
    _check_weight(W4A4, wd, sd, N, F)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    _same_device(x, wg=wg, sg=sg, wu=wu, su=su, wd=wd, sd=sd, out=out, workspace=workspace)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _dev(out, "out", torch.bfloat16)
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N]")
    need = max(mlp_workspace_bytes(M, K, F, N), 256)
    if workspace is None:
        workspace = _empty_u8(need, x.device)
    else:
        _dev(workspace, "workspace", torch.uint8)
    _check(lib().cr_mlp_w4a4(_ptr(x), M, K, _ptr(wg), _ptr(sg), _ptr(wu), _ptr(su), F, _ptr(wd), _ptr(sd), N,
                             _ptr(out), _ptr(workspace), workspace.numel(), _stream()))
    return out


def dbg_quant_swiglu(g: torch.Tensor, u: torch.Tensor):
    """Codes int8 [M,K] and scales [M] of h = silu(g) * u, as the MLP block
    quantises the down projection's input."""
    _dev(g, "g", torch.bfloat16)
    _dev(u, "u", torch.bfloat16)
    if g.dim() != 2 or g.shape != u.shape:
        raise ValueError("g and u must be [M, K] of the same shape")
    _same_device(g, u=u)
    M, K = g.shape
    codes = torch.empty((M, K), dtype=torch.int8, device=g.device)
    scales = torch.empty(max(M, 1), dtype=torch.float32, device=g.device)
    _check(lib().cr_dbg_quant_swiglu(_ptr(g), _ptr(u), M, K, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales[:M]


def dbg_silu_mul(g: torch.Tensor, u: torch.Tensor) -> torch.Tensor:
    """h = silu(g) * u (bf16, same shape), as the MLP block forms it."""
    _dev(g, "g", torch.bfloat16)
    _dev(u, "u", torch.bfloat16)
    if g.shape != u.shape:
        raise ValueError("g and u must have the same shape")
    _same_device(g, u=u)
    h = torch.empty_like(g)
    _check(lib().cr_dbg_silu_mul(_ptr(g), _ptr(u), g.numel(), _ptr(h), _stream()))
    return h


# ---------------------------------------------------------------------------
# Two-phase form: quantise x once, run GEMMs against one or more weights
# ---------------------------------------------------------------------------

def quantize_activations(kind: int, x: torch.Tensor, workspace: torch.Tensor):
    """Rotate (W4A4, W4A8, ConvRot INT8) and quantise x [M,K] into ``workspace``."""
    _dev(x, "x", torch.bfloat16)
    _dev(workspace, "workspace", torch.uint8)
    M, K = x.shape
    _check(lib().cr_quantize_activations(kind, _ptr(x), M, K, _ptr(workspace), workspace.numel(),
                                         _stream()))


def gemm_quantized(kind: int, M: int, K: int, packed, scale, N: int, workspace, bias=None, out=None):
    """GEMM + epilogue from a workspace filled by :func:`quantize_activations`."""
    _dev(packed, "packed", torch.uint8)
    _dev(scale, "scale", torch.float32)
    _check_weight(kind, packed, scale, N, K)
    _dev(workspace, "workspace", torch.uint8)
    _same_device(packed, scale=scale, workspace=workspace, bias=bias, out=out)
    if bias is not None:
        _dev(bias, "bias", torch.bfloat16)
        if bias.numel() != N:
            raise ValueError("bias must have N elements")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=packed.device)
    else:
        _dev(out, "out", torch.bfloat16)
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N]")
    _check(lib().cr_gemm_quantized(kind, M, K, _ptr(packed), _ptr(scale), N, _ptr(bias), _ptr(out),
                                   _ptr(workspace), workspace.numel(), _stream()))
    return out


# ---------------------------------------------------------------------------
# Inspection hooks
# ---------------------------------------------------------------------------

def dbg_quant_act(kind: int, x: torch.Tensor):
    """Activation codes int8 [M,K] and scales float32 [M] of the linear `kind`."""
    _dev(x, "x", torch.bfloat16)
    M, K = x.shape
    codes = torch.empty((M, K), dtype=torch.int8, device=x.device)
    scales = torch.empty(max(M, 1), dtype=torch.float32, device=x.device)
    _check(lib().cr_dbg_quant_act(kind, _ptr(x), M, K, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales[:M]


def dbg_unpack_weight(kind: int, packed: torch.Tensor, N: int, K: int):
    """Canonical int8 weight codes [N,K] held by a packed weight."""
    _dev(packed, "packed", torch.uint8)
    _check_weight(kind, packed, None, N, K)
    codes = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    _check(lib().cr_dbg_unpack_weight(kind, _ptr(packed), N, K, _ptr(codes), _stream()))
    return codes


def dbg_linear_acc(kind: int, x: torch.Tensor, packed: torch.Tensor, N: int, workspace=None):
    """int32 accumulators [M,N] of the linear `kind`."""
    _dev(x, "x", torch.bfloat16)
    _dev(packed, "packed", torch.uint8)
    _check_weight(kind, packed, None, N, x.shape[1])
    M, K = x.shape
    acc = torch.empty((M, N), dtype=torch.int32, device=x.device)
    need = max(workspace_bytes(kind, M, N, K), 256)
    if workspace is None:
        workspace = _empty_u8(need, x.device)
    _check(lib().cr_dbg_linear_acc(kind, _ptr(x), M, K, _ptr(packed), N, _ptr(acc),
                                   _ptr(workspace), workspace.numel(), _stream()))
    return acc


# ---------------------------------------------------------------------------
# Layer-level convenience
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class PackedWeight:
    """A packed weight and what its linear needs besides x."""
    kind: int
    N: int
    K: int
    packed: torch.Tensor
    scale: torch.Tensor              # tensor scale (W4A4, int8tw), s_channel (W4A8), row scales (INT8ROT)
    bias: Optional[torch.Tensor] = None


def pack_linear(w: torch.Tensor, bias: Optional[torch.Tensor] = None, int8: bool = False,
                group: int = 256, regular: bool = False) -> PackedWeight:
    """Pack a bf16 [N,K] weight: W4A4 ConvRot when K % 256 == 0 (ConvRot INT8
    row-scaled instead with ``int8=True``, the format [Q3N] gives attention
    projections; ``group`` picks the W4A4 rotation group: 256, 64 or 16, and
    ``regular=True`` the group-256 regular Hadamard),
    otherwise int8_tensorwise ([REB] "Mixed formats where the
    kernel demands it")."""
    N, K = w.shape
    if K % 256 == 0 and int8:
        p, s = pack_weight_int8rot(w)
        return PackedWeight(INT8ROT, N, K, p, s, bias)
    if K % 256 == 0 and regular:
        p, s = pack_weight_w4_regular(w)
        return PackedWeight(W4A4_RH, N, K, p, s, bias)
    if K % 256 == 0:
        p, s = pack_weight_w4(w, group)
        return PackedWeight(W4_GROUP_KIND.get(group, W4A4), N, K, p, s, bias)
    p, s = pack_weight_int8tw(w)
    return PackedWeight(INT8TW, N, K, p, s, bias)


def linear(x: torch.Tensor, pw: PackedWeight, out=None, workspace=None) -> torch.Tensor:
    if pw.kind in (W4A4_G64, W4A4_G16):
        group = 64 if pw.kind == W4A4_G64 else 16
        return linear_w4a4(x, pw.packed, pw.scale, pw.N, pw.bias, out, workspace, group=group)
    fn = {W4A4: linear_w4a4, INT8TW: linear_int8tw, W4A8: linear_w4a8, INT8ROT: linear_int8rot,
          W4A4_RH: linear_w4a4_regular}[pw.kind]
    return fn(x, pw.packed, pw.scale, pw.N, pw.bias, out, workspace)


# ---------------------------------------------------------------------------
# Measurement probes (include/convrot_probe.h): ceilings of the machine at
# hand, not part of the method
# ---------------------------------------------------------------------------

PROBE_SINK_WORDS = 4096


def probe_mfma_i8(blocks: int, iters: int, sink: torch.Tensor, stamps: torch.Tensor):
    """Launch the int8 matrix-core probe: blocks * 8 * iters * 4 * 65536 int
    ops; ``sink`` int32 [blocks * 512], ``stamps`` int64 [4] (shader clock
    counter start/end, real-time counter start/end)."""
    _dev(sink, "sink", torch.int32)
    _dev(stamps, "stamps", torch.int64)
    if sink.numel() < blocks * 512 or stamps.numel() < 4:
        raise ValueError("sink needs blocks * 512 words and stamps 4")
    _check(lib().cr_probe_mfma_i8(blocks, iters, _ptr(sink), _ptr(stamps), _stream()))


def probe_read(src: torch.Tensor, sink: torch.Tensor):
    """One kernel reading all of ``src`` (bytes a multiple of 16)."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    _dev(sink, "sink", torch.int32)
    if sink.numel() < PROBE_SINK_WORDS:
        raise ValueError(f"sink needs {PROBE_SINK_WORDS} words")
    _check(lib().cr_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream()))


def probe_copy(src: torch.Tensor, dst: torch.Tensor):
    """dst = src, one kernel with 16-byte loads and stores."""
    for t, n in ((src, "src"), (dst, "dst")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous device tensor")
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nb:
        raise ValueError("dst is smaller than src")
    _check(lib().cr_probe_copy(_ptr(src), _ptr(dst), nb, _stream()))


def probe_wall_clock_khz() -> int:
    return int(lib().cr_probe_wall_clock_khz())
