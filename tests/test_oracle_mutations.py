"""Plant plausible mistakes in the oracle (on the CPU, by monkeypatching) and
check that the pins in test_oracle_pins catch every one of them."""
import numpy as np
import pytest

from oracle import convrot_oracle as O
import tests.test_oracle_pins as P

F32 = np.float32
_real_fwht = O.fwht
_real_quant = O._quant_with_scale


def _fwht_generic(v, group=256, dtype=np.float32, order="asc", sign_swap=False, scale=True):
    v = np.asarray(v)
    K = v.shape[-1]
    lead = v.shape[:-1]
    y = np.array(v, dtype=dtype).reshape(-1, K // group, group)
    R, G = y.shape[0], y.shape[1]
    hs = []
    h = 1
    while h < group:
        hs.append(h)
        h *= 2
    if order == "desc":
        hs = hs[::-1]
    for h in hs:
        y = y.reshape(R, G, group // (2 * h), 2, h)
        a = y[:, :, :, 0, :].copy()
        b = y[:, :, :, 1, :].copy()
        y[:, :, :, 0, :] = a + b
        y[:, :, :, 1, :] = (b - a) if sign_swap else (a - b)
    y = y.reshape(R, G, group)
    if scale:
        y = y * dtype(1.0 / np.sqrt(group))
    return y.reshape(*lead, K).astype(dtype)


def _quant_floor(v, amax, qmax, lo, hi):
    amax = np.asarray(amax, dtype=F32)
    s = (amax / F32(qmax)).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.trunc(v.astype(F32) / s)
    r = np.where(s == 0, F32(0), r)
    return np.clip(r, lo, hi).astype(np.int8), s


def _quant_qmax8(v, amax, qmax, lo, hi):
    return _real_quant(v, amax, qmax + 1 if qmax == 7 else qmax, lo, hi)


def _quant_rows_tensor_scale(v, qmax, lo, hi):
    v = np.asarray(v, dtype=F32)
    amax = np.full((v.shape[0], 1), np.max(np.abs(v)), F32)
    q, s = _real_quant(v, amax, qmax, lo, hi)
    return q, s.reshape(-1)


def _gemm_reversed_k(qx, qw):
    return (qx.astype(np.float64) @ qw[:, ::-1].astype(np.float64).T).astype(np.int64).astype(np.int32)


def _epilogue_no_sw(acc, s_x, s_w, bias_bits):
    a = np.asarray(acc).astype(F32)
    y = (a * np.asarray(s_x, F32)[:, None]).astype(F32)
    if bias_bits is not None:
        y = y + O.bf16_to_f32(bias_bits)[None, :]
    return y


def _e4m3_bias8(code):
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -7, (1.0 + m / 8.0) * np.exp2(e - 8.0))
    val = np.where((e == 15) & (m == 7), np.nan, sign * val)
    return val.astype(F32)


def _decode_clamp128(idx, s_rel, codebook):
    cb = np.asarray(codebook, F32)
    s = np.repeat(O.e4m3_to_f32(s_rel), 16, axis=1)
    return np.clip(np.rint((cb[np.asarray(idx)] * s).astype(F32)), -128, 127).astype(np.int8)


def _int8rot_weight_tensor_scale(w_bits, group=256):
    wr = _real_fwht(O.bf16_to_f32(w_bits), group)
    q, s = O.quant_tensor(wr, 127, -128, 127)
    return q, np.full(wr.shape[0], s, F32)


def _int8rot_weight_unrotated(w_bits, group=256):
    return O.quant_rows(O.bf16_to_f32(w_bits), 127, -128, 127)


def _pack_high_first(q):
    u = (np.asarray(q, np.int8).astype(np.int16) & 0xF).astype(np.uint8)
    return (u[:, 1::2] | (u[:, 0::2] << 4)).astype(np.uint8)


def _fwht_group_ignored(v, group=256, dtype=np.float32):
    return _fwht_generic(v, 256, dtype)


def _fwht_norm_of_256(v, group=256, dtype=np.float32):
    return (_fwht_generic(v, group, dtype, scale=False) * dtype(1.0 / 16.0)).astype(dtype)


def _rht_generic(v, dtype=np.float32, order="asc", seq_sum=False, half_weight=False):
    v = np.asarray(v)
    K = v.shape[-1]
    lead = v.shape[:-1]
    y = np.array(v, dtype=dtype).reshape(-1, K // 256, 256)
    R, G = y.shape[0], y.shape[1]
    strides = [1, 4, 16, 64] if order == "asc" else [64, 16, 4, 1]
    for s in strides:
        y = y.reshape(R, G, 256 // (4 * s), 4, s)
        x = [y[:, :, :, k, :].copy() for k in range(4)]
        t = (((x[0] + x[1]) + x[2]) + x[3]) if seq_sum else ((x[0] + x[1]) + (x[2] + x[3]))
        for k in range(4):
            y[:, :, :, k, :] = (t - x[k]) if half_weight else (t - dtype(2) * x[k])
    return (y.reshape(R, G, 256) * dtype(0.0625)).reshape(*lead, K).astype(dtype)


def _rot_act_unrotated(x_bits, group=256):
    return O.quant_rows(O.bf16_to_f32(x_bits), 127, -128, 127)


def _rot_act_div7(x_bits, group=256):
    return O.quant_rows(_real_fwht(O.bf16_to_f32(x_bits), group), 7, -8, 7)


def _pack_uint4_high_first(idx):
    idx = np.asarray(idx, dtype=np.uint8)
    return (idx[:, 1::2] | (idx[:, 0::2] << 4)).astype(np.uint8)


def _unpack_uint4_high_first(p):
    p = np.asarray(p, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 1::2] = p & 0xF
    out[:, 0::2] = p >> 4
    return out


def _silu_mul_sigmoid(g_bits, u_bits):
    g = O.bf16_to_f32(g_bits).astype(np.float64)
    u = O.bf16_to_f32(u_bits).astype(np.float64)
    return O.f32_to_bf16_rne((1.0 / (1.0 + np.exp(-g)) * u).astype(F32))


def _silu_no_up(g_bits, u_bits):
    g = O.bf16_to_f32(g_bits).astype(np.float64)
    return O.f32_to_bf16_rne((g / (1.0 + np.exp(-g))).astype(F32))


_real_lloyd = O.lloyd_max_16


def _lloyd_ties_up(u, iters=100):
    """R10 with a sample on a midpoint sent to the upper cell."""
    real_ss = np.searchsorted

    def ss(a, v, side="left", sorter=None):
        return real_ss(a, v, side="left" if side == "right" else "right", sorter=sorter)
    np.searchsorted = ss
    try:
        return _real_lloyd(u, iters)
    finally:
        np.searchsorted = real_ss


def _lloyd_float_sums(u, iters=100):
    """R10 with float32 cell means in place of the exact integer sums."""
    u32 = np.sort(np.asarray(u, np.float32).ravel())
    lo, hi = float(u32[0]), float(u32[-1])
    lv = np.array([lo + (j + 0.5) * ((hi - lo) / 16.0) for j in range(16)])
    for _ in range(iters):
        thr = 0.5 * (lv[:-1] + lv[1:])
        cell = np.searchsorted(thr, u32.astype(np.float64), side="left")
        new = np.array([u32[cell == j].mean(dtype=np.float32) if np.any(cell == j) else lv[j] for j in range(16)],
                       dtype=np.float64)
        new = np.sort(new)
        if np.array_equal(new, lv):
            break
        lv = new
    return lv.astype(F32), [0.0]


MUTATIONS = {
    "fwht_descending_order": ("fwht", lambda v, group=256, dtype=np.float32:
                              _fwht_generic(v, group, dtype, order="desc")),
    "fwht_sign_swapped": ("fwht", lambda v, group=256, dtype=np.float32:
                          _fwht_generic(v, group, dtype, sign_swap=True)),
    "fwht_missing_normalisation": ("fwht", lambda v, group=256, dtype=np.float32:
                                   _fwht_generic(v, group, dtype, scale=False)),
    "quant_truncates": ("_quant_with_scale", _quant_floor),
    "quant_divides_by_8": ("_quant_with_scale", _quant_qmax8),
    "act_scale_per_tensor": ("quant_rows", _quant_rows_tensor_scale),
    "gemm_reversed_k": ("int_gemm", _gemm_reversed_k),
    "epilogue_drops_weight_scale": ("epilogue", _epilogue_no_sw),
    "e4m3_wrong_bias": ("e4m3_to_f32", _e4m3_bias8),
    "w4a8_clamp_128": ("w4a8_decode", _decode_clamp128),
    "pack_nibble_order": ("pack_int4", _pack_high_first),
    "int8rot_weight_scale_per_tensor": ("quant_weight_int8rot", _int8rot_weight_tensor_scale),
    "int8rot_weight_unrotated": ("quant_weight_int8rot", _int8rot_weight_unrotated),
    "fwht_group_ignored": ("fwht", _fwht_group_ignored),
    "fwht_group_norm_of_256": ("fwht", _fwht_norm_of_256),
    "rht_descending_stages": ("rht", lambda v, dtype=np.float32: _rht_generic(v, dtype, order="desc")),
    "rht_left_to_right_sum": ("rht", lambda v, dtype=np.float32: _rht_generic(v, dtype, seq_sum=True)),
    "rht_diagonal_weight_1": ("rht", lambda v, dtype=np.float32: _rht_generic(v, dtype, half_weight=True)),
    "mlp_sigmoid_not_silu": ("silu_mul_bf16", _silu_mul_sigmoid),
    "mlp_gate_without_up": ("silu_mul_bf16", _silu_no_up),
    "int8rot_act_unrotated": ("quant_act_int8rot", _rot_act_unrotated),
    "int8rot_act_div7": ("quant_act_int8rot", _rot_act_div7),
    "w4a8_act_unrotated": ("quant_act_w4a8", _rot_act_unrotated),
    "w4a8_act_div7": ("quant_act_w4a8", _rot_act_div7),
    # both directions swapped consistently: a round trip alone cannot see it
    "lloyd_ties_to_upper_cell": ("lloyd_max_16", _lloyd_ties_up),
    "lloyd_float32_means": ("lloyd_max_16", _lloyd_float_sums),
    "uint4_high_first": [("pack_uint4", _pack_uint4_high_first), ("unpack_uint4", _unpack_uint4_high_first)],
}

PINS = [
    P.test_hadamard_orthonormal_exact,
    P.test_fwht_unit_vectors_give_hadamard_rows,
    P.test_fwht_float64_equals_dense_product,
    P.test_fwht_float32_within_error_bound,
    P.test_fwht_stage_order_fixture,
    P.test_exact_identity_before_quantisation,
    P.test_one_hot_row_codes,
    lambda: P.test_constant_row_codes(0.5),
    P.test_zero_row_and_bias_only_output,
    P.test_quant_invariants,
    P.test_pack_roundtrip,
    P.test_acc_brute_force_python_ints_tiny,
    P.test_epilogue_exact_for_power_of_two_scales,
    P.test_end_to_end_close_to_float_linear,
    P.test_e4m3_decode_matches_torch,
    P.test_w4a8_decode_hand_cases,
    P.test_int8rot_row_scale_invariance,
    P.test_int8rot_one_hot_weight_rows,
    P.test_int8rot_acc_brute_force_python_ints,
    lambda: P.test_fwht_group_unit_vectors_block_diagonal(16),
    lambda: P.test_fwht_group_float64_equals_dense_block_product(64),
    lambda: P.test_group_one_hot_row_codes(64),
    lambda: P.test_group_constant_row_codes(16, 0.5),
    lambda: P.test_group_weight_one_hot_codes(16),
    P.test_rht_unit_vectors_give_rows,
    P.test_rht_float64_equals_dense_product,
    P.test_rht_pairwise_sum_fixture,
    P.test_rht_stage_order_fixture,
    lambda: P.test_rht_constant_row_stays_constant(0.5),
    P.test_rht_one_hot_row_codes,
    P.test_silu_mul_matches_library_logistic,
    P.test_silu_mul_special_values,
    P.test_mlp_block_close_to_float_mlp,
    lambda: P.test_rotated_int8_act_one_hot_rows("int8rot"),
    lambda: P.test_rotated_int8_act_one_hot_rows("w4a8"),
    lambda: P.test_rotated_int8_act_constant_rows("int8rot", 0.75),
    lambda: P.test_rotated_int8_act_constant_rows("w4a8", -2.0),
    P.test_linear_int8rot_close_to_float_linear,
    P.test_uint4_nibble_order_hand_bytes,
    P.test_lloyd_max_hand_fixture,
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    plants = MUTATIONS[name]
    for attr, bad in (plants if isinstance(plants, list) else [plants]):
        monkeypatch.setattr(O, attr, bad)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:
            caught.append(getattr(pin, "__name__", "lambda"))
    assert caught, f"no pin caught the planted mistake {name}"
