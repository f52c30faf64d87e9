"""CPU oracle for the ConvRot-quantized linear forward.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this module.  The GPU library never calls it and shares no code with
it: the two meet only through the seeded inputs of ``synthetic_inputs``.

Plain NumPy, written for a reader to check against the pages by eye.  Vector
operations run over independent rows / groups; the arithmetic order inside one
output follows the definitions below and nothing is blocked, fused or
reordered.

Sources (web pages; cited by title and section):

* [QIE]  "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4 (+ConvRot, mixed int8
         fallback)" model card: intro paragraph (signed 4-bit weight codes
         two to a byte, a group-256 Hadamard rotation named "regular",
         activations rotated and quantised to 4 bits per row at run time,
         no calibration); "Speed" table (one kernel for the rotation, the
         s4 MMA and the rank-one rescale; int8_tensorwise kernels).
* [Q3N]  "qwen3-4b-nvfp4-convrot" asset page: file table and converter
         flags (ConvRot INT8 row-scaled, group size 256).
* [QVL]  "Qwen3-VL-4B-W4A8-ConvRot" model page: file table
         (asym_w4a8_int8, group 16, convrot_groupsize 256).
* [REB]  "Rebels_w4a8s" collection page: "What's inside a file" table (4-bit
         codebook indices two to a byte, an fp8 scale for each 16 weights, a
         scale for each output row, a 16-level Lloyd-Max codebook); "Mixed
         formats where the kernel demands it" (the W4 kernel takes only
         groups of 256, int8_tensorwise covers other widths);
         "Why W4A8 instead of GGUF" (int8 GEMM, ~0.56 B/param, ~7% weight
         error).
* [ZIT]  "Z-Image-Turbo-W4A4-ConvRot" model card: "Where Z-Image sits"
         (convrot_groupsize sweep 256 / 64 / 16; a size-N rotation spreads
         an outlier over N channels).

Readings taken where the pages are silent (each also listed, under the same
number, in the design notes of the repository; R11-R16 there concern the
GPU library's interface and tolerance, not this module's arithmetic):

R1  Hadamard: Sylvester order-256 matrix H[i,j] = (-1)^popcount(i&j), scaled
    by 1/16 so it is orthonormal.  ("regular-Hadamard" read as the standard
    Sylvester construction.)
R2  Rotation arithmetic: float32, fast Walsh-Hadamard butterflies with strides
    1,2,4,...,128 in that order, each (a, b) -> (a+b, a-b), then one multiply
    by 0.0625 (exact).  The rotated value stays float32 until quantised.
R3  Activation scale: per row over the full K, s = absmax / 7 in float32
    (IEEE division); code = clip(rint(v / s), -8, 7) with round-half-even.
    A row of zeros has s = 0 and codes 0.
R4  Weight scale (W4A4): one per tensor, absmax of the *rotated* weight / 7.
R5  Accumulation: exact integer sum over the full K (int32 range).
R6  Epilogue: y = fl(fl(float32(acc) * s_x[m]) * s_w) + float32(bias[n]),
    in float32; the GPU result is this value rounded to bf16.
R7  int8_tensorwise: no rotation; x per row absmax/127, W per tensor
    absmax/127, codes clip(rint(v/s), -128, 127); any K.
R8  W4A8 decode: w8 = clip(rint(float32(cb[idx]) * e4m3(s_rel)), -127, 127)
    with one float32 multiply; one int32 accumulation over the full K; the
    epilogue uses s_channel[n] in place of s_w.  Activations: rotated, per
    row absmax/127, clip [-128, 127].
R9  fp8 is OCP E4M3FN (bias 7, no infinities, 0x7F/0xFF are NaN, max 448).
R10 W4A8 encode (offline): s_channel[n] = absmax_k |W~[n,:]| / 127;
    s_rel[n,g] = e4m3_rne(min(absmax_{k in g} |W~| / s_channel[n], 127));
    u = W~ / (s_channel * s_rel) (0 where the divisor is 0); 16-level
    Lloyd-Max quantiser of all u of the tensor (as float32): levels start
    evenly spread over [min u, max u], cells by the midpoints of adjacent
    levels (a value on a midpoint goes to the lower level), each level moved
    to its cell's exact mean (samples summed as the integers rint(u 2^24),
    one float64 division), at most 100 iterations or until no level moves;
    the codebook is the levels rounded to float32; idx = the cell of u by
    the midpoints of the float32 codebook.  (The pages fix only "16
    Lloyd-Max levels fit to the tensor"; the start and the exact sums make
    the fit one definite result that a parallel encoder reproduces bit for
    bit.)
R17 ConvRot INT8 row-scaled ([Q3N] file table: INT8 with group-256 Hadamard
    rotation and row-wise scaling; converter flags: int8, row scaling,
    dynamic ConvRot, group 256): the weight is rotated like R2, then
    quantised per output row, s_w[n] = absmax_k |W~[n,k]| / 127, codes
    clip(rint(W~ / s_w[n]), -128, 127); the activations are rotated online
    and quantised per row as in R8; one int32 accumulation over the full K;
    the epilogue takes s_w[n] per output column (as s_channel in R8).
R18 Smaller rotation groups ([ZIT] "Where Z-Image sits": the sweep over
    group sizes 256, 64 and 16): the same butterflies as R2 over groups of
    G = 64 or 16 consecutive k (strides 1 .. G/2 ascending), i.e. a
    block-diagonal rotation, then one multiply by 1/sqrt(G) (0.125 or
    0.25, exact); everything after the rotation is R3-R6 unchanged.  K
    stays a multiple of 256 (the layer eligibility rule of [REB] "Mixed
    formats" is kept whatever the group).
R19 Regular Hadamard ([QIE] intro: "regular-Hadamard" rotation, no
    construction given): the group-256 matrix (J - 2I)^(x4) / 16, the fourth
    Kronecker power of the 4x4 regular Hadamard matrix J - 2I (every row of
    which sums to 2, so every row of the normalised H sums to 1).  Applied
    by four radix-4 stages (digit strides 1, 4, 16, 64 ascending); a stage
    maps the group x0..x3 to t - 2 x_k, t = (x0 + x1) + (x2 + x3), in
    float32; then one multiply by 0.0625.  Everything after the rotation is
    R3-R6 unchanged.  An alternative to R1, not the default.  (The other
    4x4 regular Hadamard matrix, 2I - J = -(J - 2I), gives the same
    256-matrix: the four sign flips cancel.)
R20 Text-encoder MLP block ([Q3N] file table and the "qwen3vl_4b" page:
    the decoder blocks' gate_proj, up_proj and down_proj Linears; the
    pages do not state the activation): the gated MLP of this model family,
    h = silu(gate(x)) * up(x), silu(v) = v / (1 + exp(-v)), then
    y = down(h).  Each Linear is the W4A4 linear of R1-R6 (bf16 out, no
    bias); h is computed from the bf16 g and u in float64, rounded to
    float32 and then to bf16 (round to nearest even), and enters the down
    linear as its bf16 input.
R21 Canonical 4-bit storage: two values per byte, low nibble = even k;
    signed codes in two's complement, codebook indices unsigned.

Parity notes: the Lloyd-Max fit (R10) is defined to be deterministic (exact
integer cell sums, a fixed start), so the GPU encoder is compared with it bit
for bit; it is pinned by the closed-form optimum of a uniform source, the
textbook 16-level Gaussian quantiser, non-increasing distortion and the
pages' ~7% weight error.
"""
from __future__ import annotations

import numpy as np

GROUP = 256
F32 = np.float32


# ---------------------------------------------------------------------------
# bf16 <-> float32
# ---------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32; exact."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits.

    NaN maps to a quiet NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    r = r.astype(np.uint16)
    nan = np.isnan(a)
    if np.any(nan):
        r[nan] = np.uint16(0x7FC0)
    return r


# ---------------------------------------------------------------------------
# The rotation  [QIE intro: group-256 regular-Hadamard ConvRot; ZIT "Where
# Z-Image sits": rotation of size N spreads an outlier over N channels]
# ---------------------------------------------------------------------------

def hadamard(n: int = GROUP) -> np.ndarray:
    """Closed form of the normalised Sylvester Hadamard matrix (float64).

    H[i, j] = (-1)^popcount(i & j) / sqrt(n)   (reading R1)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    bits = np.bitwise_and(i, j)
    pop = np.zeros_like(bits)
    b = bits.copy()
    while np.any(b):
        pop += b & 1
        b >>= 1
    return np.where(pop % 2 == 0, 1.0, -1.0) / np.sqrt(n)


def fwht(v: np.ndarray, group: int = GROUP, dtype=np.float32) -> np.ndarray:
    """Group-wise rotation along the last axis: each contiguous block of
    ``group`` values is multiplied by the normalised Sylvester Hadamard.

    Reading R2: butterflies with strides 1, 2, 4, ... group/2 in that order,
    each pair (i, i+h) with i & h == 0 becoming (a+b, a-b), computed in
    ``dtype``; then one multiply by 1/sqrt(group) (a power of two for the
    group sizes used: 16, 64, 256)."""
    v = np.asarray(v)
    K = v.shape[-1]
    if K % group != 0:
        raise ValueError(f"K={K} is not a multiple of the rotation group {group}")
    lead = v.shape[:-1]
    y = np.array(v, dtype=dtype).reshape(-1, K // group, group)
    R, G = y.shape[0], y.shape[1]
    h = 1
    while h < group:
        y = y.reshape(R, G, group // (2 * h), 2, h)
        a = y[:, :, :, 0, :].copy()
        b = y[:, :, :, 1, :].copy()
        y[:, :, :, 0, :] = a + b
        y[:, :, :, 1, :] = a - b
        h *= 2
    y = y.reshape(R, G, group)
    scale = dtype(1.0 / np.sqrt(group))
    y = y * scale
    return y.reshape(*lead, K).astype(dtype)


def regular_hadamard() -> np.ndarray:
    """Closed form of the normalised group-256 regular Hadamard matrix of
    reading R19 (float64): with A = J - 2I the 4x4 matrix of ones less twice
    the identity (every row sums to 2), H[i, j] = prod_d A[i_d, j_d] / 16 over
    the four base-4 digits of i and j.  Every row of H sums to 1."""
    A = np.ones((4, 4)) - 2.0 * np.eye(4)
    H = A
    for _ in range(3):
        H = np.kron(H, A)
    return H / 16.0


def rht(v: np.ndarray, dtype=np.float32) -> np.ndarray:
    """Group-256 rotation by the regular Hadamard matrix along the last axis.

    Reading R19: four radix-4 stages over the base-4 digits of the index
    (strides 1, 4, 16, 64 in that order); a stage replaces the four values
    x0..x3 of a group (index order) by t - 2 x_k with t = (x0 + x1) + (x2 + x3),
    computed in ``dtype``; then one multiply by 1/16 (exact)."""
    v = np.asarray(v)
    K = v.shape[-1]
    if K % GROUP != 0:
        raise ValueError(f"K={K} is not a multiple of the rotation group {GROUP}")
    lead = v.shape[:-1]
    y = np.array(v, dtype=dtype).reshape(-1, K // GROUP, GROUP)
    R, G = y.shape[0], y.shape[1]
    s = 1
    while s < GROUP:
        y = y.reshape(R, G, GROUP // (4 * s), 4, s)
        x = [y[:, :, :, k, :].copy() for k in range(4)]
        t = (x[0] + x[1]) + (x[2] + x[3])
        for k in range(4):
            y[:, :, :, k, :] = t - dtype(2) * x[k]
        s *= 4
    y = y.reshape(R, G, GROUP) * dtype(0.0625)
    return y.reshape(*lead, K).astype(dtype)


# ---------------------------------------------------------------------------
# Symmetric quantisation  [QIE intro: activations "dynamically quantized to
# INT4"; weights packed signed INT4, tensorwise]
# ---------------------------------------------------------------------------

def _quant_with_scale(v: np.ndarray, amax: np.ndarray, qmax: int, lo: int, hi: int):
    """s = fl(amax / qmax); q = clip(rint(v / s), lo, hi); s == 0 -> q = 0.

    ``amax`` broadcasts against ``v`` (per row: shape [R, 1]; per tensor: a
    scalar)."""
    amax = np.asarray(amax, dtype=F32)
    s = (amax / F32(qmax)).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(v.astype(F32) / s)
    r = np.where(s == 0, F32(0), r)
    q = np.clip(r, lo, hi).astype(np.int8)
    return q, s


def quant_rows(v: np.ndarray, qmax: int, lo: int, hi: int):
    """Per-row dynamic symmetric quantisation (readings R3, R7).

    Returns (codes int8 [R, K], scales float32 [R])."""
    v = np.asarray(v, dtype=F32)
    amax = np.max(np.abs(v), axis=1, keepdims=True) if v.shape[1] else np.zeros((v.shape[0], 1), F32)
    q, s = _quant_with_scale(v, amax, qmax, lo, hi)
    return q, s.reshape(-1)


def quant_tensor(v: np.ndarray, qmax: int, lo: int, hi: int):
    """Tensorwise symmetric quantisation (readings R4, R7).

    Returns (codes int8, scale float32 scalar)."""
    v = np.asarray(v, dtype=F32)
    amax = np.max(np.abs(v)) if v.size else F32(0)
    q, s = _quant_with_scale(v, F32(amax), qmax, lo, hi)
    return q, F32(s)


# --- W4A4 ----------------------------------------------------------------

def quant_act_w4a4(x_bits: np.ndarray, group: int = GROUP):
    """Online rotation + dynamic per-row INT4 codes of the activations."""
    xr = fwht(bf16_to_f32(x_bits), group)
    return quant_rows(xr, 7, -8, 7)


def quant_weight_w4(w_bits: np.ndarray, group: int = GROUP):
    """Offline rotation + tensorwise INT4 codes of the weight [N, K]."""
    wr = fwht(bf16_to_f32(w_bits), group)
    return quant_tensor(wr, 7, -8, 7)


# --- int8_tensorwise -------------------------------------------------------

def quant_act_w4a4_regular(x_bits: np.ndarray):
    """W4A4 activations rotated by the regular Hadamard matrix (R19)."""
    return quant_rows(rht(bf16_to_f32(x_bits)), 7, -8, 7)


def quant_weight_w4_regular(w_bits: np.ndarray):
    """W4 weight rotated by the regular Hadamard matrix (R19), tensorwise."""
    return quant_tensor(rht(bf16_to_f32(w_bits)), 7, -8, 7)


def quant_act_int8(x_bits: np.ndarray):
    """int8_tensorwise activations: no rotation, per row absmax/127."""
    return quant_rows(bf16_to_f32(x_bits), 127, -128, 127)


def quant_weight_int8tw(w_bits: np.ndarray):
    """int8_tensorwise weight: no rotation, per tensor absmax/127."""
    return quant_tensor(bf16_to_f32(w_bits), 127, -128, 127)


# --- W4A8 activations ------------------------------------------------------

def quant_act_w4a8(x_bits: np.ndarray, group: int = GROUP):
    """W4A8 activations: group-256 rotation, then per-row int8 (absmax/127)."""
    xr = fwht(bf16_to_f32(x_bits), group)
    return quant_rows(xr, 127, -128, 127)


# --- ConvRot INT8, row-scaled (reading R17) --------------------------------

def quant_act_int8rot(x_bits: np.ndarray, group: int = GROUP):
    """ConvRot INT8 activations: group-256 rotation (dynamic ConvRot), then
    per-row int8 codes (absmax/127)."""
    xr = fwht(bf16_to_f32(x_bits), group)
    return quant_rows(xr, 127, -128, 127)


def quant_weight_int8rot(w_bits: np.ndarray, group: int = GROUP):
    """ConvRot INT8 row-scaled weight [N, K]: group-256 rotation, then one
    int8 scale per output row (absmax of the rotated row / 127)."""
    wr = fwht(bf16_to_f32(w_bits), group)
    return quant_rows(wr, 127, -128, 127)


# ---------------------------------------------------------------------------
# Canonical nibble packing (reading R21)
# ---------------------------------------------------------------------------

def pack_int4(q: np.ndarray) -> np.ndarray:
    """int4 codes [R, K] (values in [-8, 7]) -> bytes [R, K/2], low nibble =
    even k, two's complement."""
    q = np.asarray(q, dtype=np.int8)
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_int4` (signed codes)."""
    p = np.asarray(p, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def unpack_uint4(p: np.ndarray) -> np.ndarray:
    """Unsigned nibbles (codebook indices) [R, K/2] -> [R, K], low = even k."""
    p = np.asarray(p, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def pack_uint4(idx: np.ndarray) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.uint8)
    return (idx[:, 0::2] | (idx[:, 1::2] << 4)).astype(np.uint8)


# ---------------------------------------------------------------------------
# Integer GEMM and rank-one epilogue  [QIE "Speed": rank-one s4 MMA]
# ---------------------------------------------------------------------------

def int_gemm(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k qx[m, k] * qw[n, k], exact (reading R5).

    Computed with a float64 matrix product on integer-valued operands: every
    product and partial sum is an integer of magnitude below 2^53 for the
    sizes used (|code| <= 128, K < 2^30 / 2^14), so the float64 result is the
    exact integer.  Raises if the result leaves the int32 range."""
    qx = np.asarray(qx)
    qw = np.asarray(qw)
    K = qx.shape[1]
    assert qw.shape[1] == K
    bound = int(np.max(np.abs(qx.astype(np.int64)), initial=0)) * \
        int(np.max(np.abs(qw.astype(np.int64)), initial=0)) * K
    if bound >= 2 ** 53:
        raise OverflowError("float64 product would not be exact")
    acc = qx.astype(np.float64) @ qw.astype(np.float64).T
    acc = acc.astype(np.int64)
    if acc.size and (acc.max() > 2 ** 31 - 1 or acc.min() < -2 ** 31):
        raise OverflowError("accumulator leaves int32")
    return acc.astype(np.int32)


def epilogue(acc: np.ndarray, s_x: np.ndarray, s_w, bias_bits: np.ndarray | None):
    """Rank-one rescale (reading R6): fl(fl(float32(acc)*s_x[m])*s_w) + bias[n].

    ``s_w`` is a scalar (tensorwise) or a per-column vector (W4A8 s_channel).
    Returns float32 [M, N] (not rounded to bf16)."""
    a = np.asarray(acc).astype(F32)
    y = (a * np.asarray(s_x, dtype=F32)[:, None]).astype(F32)
    sw = np.asarray(s_w, dtype=F32)
    y = (y * (sw[None, :] if sw.ndim == 1 else sw)).astype(F32)
    if bias_bits is not None:
        y = (y + bf16_to_f32(bias_bits)[None, :]).astype(F32)
    return y


# ---------------------------------------------------------------------------
# End-to-end linears (float32 pre-bf16 output)
# ---------------------------------------------------------------------------

def linear_w4a4(x_bits, w_bits, bias_bits=None, group: int = GROUP):
    """ConvRot W4A4 linear [QIE intro + "Speed"].

    Returns dict with codes, scales, acc and the float32 output."""
    qx, sx = quant_act_w4a4(x_bits, group)
    qw, sw = quant_weight_w4(w_bits, group)
    acc = int_gemm(qx, qw)
    return dict(qx=qx, sx=sx, qw=qw, sw=sw, acc=acc, y=epilogue(acc, sx, sw, bias_bits))


def linear_w4a4_regular(x_bits, w_bits, bias_bits=None):
    """W4A4 linear with the regular Hadamard rotation (R19): R3-R6 after the
    rotation, as in linear_w4a4."""
    qx, sx = quant_act_w4a4_regular(x_bits)
    qw, sw = quant_weight_w4_regular(w_bits)
    acc = int_gemm(qx, qw)
    return dict(qx=qx, sx=sx, qw=qw, sw=sw, acc=acc, y=epilogue(acc, sx, sw, bias_bits))


# --- Text-encoder MLP block  [Q3N / "qwen3vl_4b" pages: the decoder
# blocks' {gate,up,down}_proj Linears, all W4A4 ConvRot in the W4A4 file]

def silu_mul_bf16(g_bits: np.ndarray, u_bits: np.ndarray) -> np.ndarray:
    """h = silu(g) * u of two bf16 tensors (reading R20): in float64,
    silu(v) = v / (1 + exp(-v)), the product rounded to float32 and then to
    bf16 (both round to nearest even).  Returns bf16 bits."""
    g = bf16_to_f32(g_bits).astype(np.float64)
    u = bf16_to_f32(u_bits).astype(np.float64)
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * u
    return f32_to_bf16_rne(h.astype(F32))


def mlp_w4a4(x_bits, wg_bits, wu_bits, wd_bits, group: int = GROUP):
    """Gated MLP block of W4A4 ConvRot linears (reading R20): g and u the bf16
    outputs of the gate and up linears of x, h = silu_mul_bf16(g, u), y the
    W4A4 linear of h with the down weight (no biases).  Returns the
    intermediates and the float32 output of the down linear."""
    g = f32_to_bf16_rne(linear_w4a4(x_bits, wg_bits, None, group)["y"])
    u = f32_to_bf16_rne(linear_w4a4(x_bits, wu_bits, None, group)["y"])
    h = silu_mul_bf16(g, u)
    d = linear_w4a4(h, wd_bits, None, group)
    return dict(g=g, u=u, h=h, qh=d["qx"], sh=d["sx"], acc=d["acc"], y=d["y"])


def linear_int8tw(x_bits, w_bits, bias_bits=None):
    """int8_tensorwise linear [QIE intro "stock int8_tensorwise"; REB "Mixed
    formats": no group constraint]."""
    qx, sx = quant_act_int8(x_bits)
    qw, sw = quant_weight_int8tw(w_bits)
    acc = int_gemm(qx, qw)
    return dict(qx=qx, sx=sx, qw=qw, sw=sw, acc=acc, y=epilogue(acc, sx, sw, bias_bits))


def linear_int8rot(x_bits, w_bits, bias_bits=None, group: int = GROUP):
    """ConvRot INT8 row-scaled linear [Q3N file table and converter flags]:
    rotated per-row int8 activations, rotated row-scaled int8 weight, exact
    int32 accumulation, epilogue with the weight scale of each output column."""
    qx, sx = quant_act_int8rot(x_bits, group)
    qw, sw = quant_weight_int8rot(w_bits, group)
    acc = int_gemm(qx, qw)
    return dict(qx=qx, sx=sx, qw=qw, sw=sw, acc=acc, y=epilogue(acc, sx, sw, bias_bits))


# ---------------------------------------------------------------------------
# OCP E4M3FN  (reading R9; [REB] "fp8 scale, one per group of 16")
# ---------------------------------------------------------------------------

def e4m3_to_f32(code: np.ndarray) -> np.ndarray:
    """Decode E4M3FN bytes: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    exponent 0: subnormal m/8 * 2^-6; S.1111.111 is NaN; no infinities."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = sign * val
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return val.astype(F32)


def _e4m3_positive_table() -> np.ndarray:
    return e4m3_to_f32(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float64)  # 0x00..0x7E


def f32_to_e4m3_rne(v: np.ndarray) -> np.ndarray:
    """Encode finite values of magnitude <= 448 to E4M3FN, nearest value,
    ties to the even code (even mantissa).  Raises on larger magnitudes."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > 448.0):
        raise ValueError("value outside the finite E4M3FN range")
    table = _e4m3_positive_table()          # increasing, codes 0..126
    a = np.abs(v)
    hi = np.searchsorted(table, a, side="left")          # first table >= a
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    dlo = a - table[lo]
    dhi = table[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = np.where(v < 0, 0x80, 0).astype(np.uint8)
    return (code | sign).astype(np.uint8)


# ---------------------------------------------------------------------------
# W4A8 codebook format  ([REB] "What's inside a file"; [QVL] group 16,
# convrot_groupsize 256)
# ---------------------------------------------------------------------------

def w4a8_decode(idx: np.ndarray, s_rel: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """Decode to int8 weights (reading R8).

    idx: uint8 codebook indices [N, K] (already unpacked); s_rel: e4m3 bytes
    [N, K/16]; codebook: float32 [16].  w8 = clip(rint(cb[idx]*s), -127, 127)
    with one float32 multiply."""
    idx = np.asarray(idx)
    N, K = idx.shape
    cb = np.asarray(codebook, dtype=F32)
    s = e4m3_to_f32(s_rel)                         # [N, K/16]
    s_full = np.repeat(s, 16, axis=1)              # [N, K]
    prod = (cb[idx] * s_full).astype(F32)
    prod = np.where(np.isnan(prod), F32(0), prod)
    return np.clip(np.rint(prod), -127, 127).astype(np.int8)


def linear_w4a8(x_bits, idx_packed, s_rel, codebook, s_channel, bias_bits=None,
                group: int = GROUP):
    """Asym W4A8 codebook linear ([REB] "Why W4A8 instead of GGUF": the GEMM
    runs on the int8 matrix units with no dequantisation to a float type;
    reading R8)."""
    qx, sx = quant_act_w4a8(x_bits, group)
    w8 = w4a8_decode(unpack_uint4(idx_packed), s_rel, codebook)
    acc = int_gemm(qx, w8)
    return dict(qx=qx, sx=sx, w8=w8, acc=acc,
                y=epilogue(acc, sx, np.asarray(s_channel, F32), bias_bits))


LLOYD_FRAC_BITS = 24        # samples enter the cell sums as integers rint(u * 2^24)


def lloyd_max_16(u: np.ndarray, iters: int = 100):
    """16-level Lloyd-Max scalar quantiser of the samples ``u`` (reading R10).

    The samples are taken as float32.  Levels start evenly spread over
    [min u, max u]: c_j = lo + (j + 1/2) * ((hi - lo) / 16) in float64.  An
    iteration assigns every sample to a cell by the midpoints t_j =
    (c_j + c_{j+1}) / 2 (float64; a sample on a midpoint goes to the lower
    cell) and moves every non-empty cell's level to the cell mean, taken
    exactly: each sample enters the sum as the integer q = rint(u * 2^24)
    (exact for float32 |u| < 2^29), so the sums are exact integers and do not
    depend on the order of summation, and the level is
    fl(float64(S) / float64(n)) * 2^-24.  Empty cells keep their level; the
    levels are then sorted.  Stops when an iteration changes no level, or
    after ``iters`` iterations.  Returns (levels float32 [16], list of the
    distortion at each iteration).

    Computed here on the sorted samples with prefix sums (of q, exact in
    int64), which gives the same cells and sums as visiting every sample."""
    u32 = np.asarray(u, dtype=np.float32).ravel()
    n = u32.size
    if n == 0:
        return np.zeros(16, F32), []
    if np.max(np.abs(u32)) >= 2.0 ** 28:
        raise ValueError("samples too large for the exact fixed-point sums")
    s = np.sort(u32.astype(np.float64))
    q = np.rint(np.sort(u32) * F32(2.0 ** LLOYD_FRAC_BITS)).astype(np.int64)
    cq = np.concatenate([[0], np.cumsum(q)])                  # exact int64 prefix sums
    if abs(int(cq[-1])) >= 2 ** 53 or int(np.sum(np.abs(q))) >= 2 ** 53:
        raise ValueError("too many samples for exact float64 sums")
    csum = np.concatenate([[0.0], np.cumsum(s)])             # distortion bookkeeping only
    csq = np.concatenate([[0.0], np.cumsum(s * s)])
    lo, hi = s[0], s[-1]
    w = (hi - lo) / 16.0
    levels = np.array([lo + (j + 0.5) * w for j in range(16)], dtype=np.float64)
    hist = []

    def cells(lv):
        thr = 0.5 * (lv[:-1] + lv[1:])
        # a sample equal to a midpoint belongs to the lower cell
        return np.concatenate([[0], np.searchsorted(s, thr, side="right"), [n]])

    for _ in range(iters):
        b = cells(levels)
        cnt = b[1:] - b[:-1]
        sums = csum[b[1:]] - csum[b[:-1]]
        sq = csq[b[1:]] - csq[b[:-1]]
        hist.append(float(np.sum(sq - 2 * levels * sums + cnt * levels ** 2)))
        qs = cq[b[1:]] - cq[b[:-1]]                           # exact integer cell sums
        mean = qs.astype(np.float64) / np.maximum(cnt, 1).astype(np.float64) * 2.0 ** -LLOYD_FRAC_BITS
        new = np.sort(np.where(cnt > 0, mean, levels))
        if np.array_equal(new, levels):
            break
        levels = new
    return levels.astype(F32), hist


def w4a8_encode(w_bits: np.ndarray, group: int = GROUP, iters: int = 100):
    """Offline W4A8 encode of a bf16 weight [N, K] (reading R10).

    Returns dict(idx_packed uint8 [N,K/2], s_rel e4m3 [N,K/16], codebook
    float32 [16], s_channel float32 [N], distortion history)."""
    wr = fwht(bf16_to_f32(w_bits), group)                       # float32 [N, K]
    N, K = wr.shape
    if K % 16 != 0:
        raise ValueError("K must be a multiple of 16")
    s_ch = (np.max(np.abs(wr), axis=1) / F32(127)).astype(F32)  # [N]
    gmax = np.max(np.abs(wr).reshape(N, K // 16, 16), axis=2)   # [N, K/16]
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(s_ch[:, None] > 0, gmax / s_ch[:, None], F32(0)).astype(F32)
    rel = np.minimum(rel, F32(127))
    s_rel = f32_to_e4m3_rne(rel)
    s_rel_f = e4m3_to_f32(s_rel)
    div = (np.repeat(s_rel_f, 16, axis=1) * s_ch[:, None]).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(div > 0, wr / div, F32(0)).astype(F32)
    cb, hist = lloyd_max_16(u, iters)
    thr = 0.5 * (cb[:-1].astype(np.float64) + cb[1:].astype(np.float64))
    idx = np.searchsorted(thr, u.astype(np.float64).ravel(), side="left").reshape(N, K)
    idx = idx.astype(np.uint8)
    return dict(idx_packed=pack_uint4(idx), idx=idx, s_rel=s_rel, codebook=cb,
                s_channel=s_ch, distortion=hist, w_rot=wr)
