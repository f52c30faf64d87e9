"""Pins of the CPU oracle against facts that do not come from the oracle
itself: closed forms, exact identities, hand-derived fixtures, library
routines (torch's float8 cast), brute-force integer sums, and the figures the
model cards print.  CPU only."""
import json
import os

import numpy as np
import pytest

import synthetic_inputs as si
from oracle import convrot_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _popcount(v: int) -> int:
    return bin(v).count("1")


# ---------------------------------------------------------------------------
# Hadamard closed form
# ---------------------------------------------------------------------------

def test_hadamard_orthonormal_exact():
    H = O.hadamard(256)
    assert np.array_equal(H @ H.T, np.eye(256))      # exact in float64
    assert np.array_equal(H, H.T)


def test_hadamard_matches_sylvester_recursion():
    # H_1 = [1]; H_2n = [[H, H], [H, -H]]  (unnormalised), an independent
    # construction of the same matrix
    h = np.array([[1.0]])
    while h.shape[0] < 256:
        h = np.block([[h, h], [h, -h]])
    assert np.array_equal(O.hadamard(256) * 16.0, h)
    for n in (16, 64):
        g = np.array([[1.0]])
        while g.shape[0] < n:
            g = np.block([[g, g], [g, -g]])
        assert np.allclose(O.hadamard(n) * np.sqrt(n), g, rtol=0, atol=0)


def test_fwht_unit_vectors_give_hadamard_rows():
    eye = np.eye(256, dtype=F32)
    got = O.fwht(eye)                         # row j = e_j rotated
    want = np.array([[(-1.0) ** _popcount(i & j) / 16 for j in range(256)] for i in range(256)])
    assert np.array_equal(got.astype(np.float64), want)


def test_fwht_float64_equals_dense_product():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(5, 1024))
    got = O.fwht(x, 256, dtype=np.float64)
    H = O.hadamard(256)
    want = (x.reshape(5, 4, 256) @ H).reshape(5, 1024)
    assert np.max(np.abs(got - want)) <= 1e-14 * np.max(np.abs(want))


def test_fwht_float32_within_error_bound():
    rng = np.random.default_rng(4)
    x32 = rng.standard_t(3, size=(8, 512)).astype(F32)
    got = O.fwht(x32).astype(np.float64)
    H = O.hadamard(256)
    want = (x32.astype(np.float64).reshape(8, 2, 256) @ H).reshape(8, 512)
    l1 = np.abs(x32.astype(np.float64)).reshape(8, 2, 256).sum(-1)            # ||x_g||_1
    bound = 8 * 2.0 ** -24 * l1 / 16 * 1.0001
    err = np.abs(got - want).reshape(8, 2, 256)
    assert np.all(err <= bound[:, :, None])


def test_fwht_stage_order_fixture():
    g = _golden("fwht_order_case.json")
    x = np.zeros((1, 256), dtype=np.uint16)
    for k, h in g["input_bf16_hex"].items():
        x[0, int(k)] = int(h, 16)
    y = O.fwht(O.bf16_to_f32(x))
    want = np.array([int(h, 16) for h in g["expected_rotated_f32_hex_by_k_mod_4"]], dtype=np.uint32)
    assert np.array_equal(y.view(np.uint32)[0], np.tile(want, 64))
    q, s = O.quant_act_w4a4(x)
    assert np.array_equal(q[0], np.tile(np.array(g["expected_int4_codes_by_k_mod_4"], np.int8), 64))
    assert s.view(np.uint32)[0] == int(g["expected_scale_f32_hex"], 16)


def test_exact_identity_before_quantisation():
    L = si.tiny()
    x = O.bf16_to_f32(L.x).astype(np.float64)
    w = O.bf16_to_f32(L.w).astype(np.float64)
    xr = O.fwht(x, 256, dtype=np.float64)
    wr = O.fwht(w, 256, dtype=np.float64)
    lhs = xr @ wr.T
    rhs = x @ w.T
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs))


# ---------------------------------------------------------------------------
# Special cases of the quantiser
# ---------------------------------------------------------------------------

def test_one_hot_row_codes():
    K, j, g = 512, 37, 1
    x = np.zeros((1, K), F32)
    x[0, 256 * g + j] = 3.0
    q, s = O.quant_act_w4a4(si.f32_to_bf16_bits(x))
    sign = np.array([1 if _popcount(j & k) % 2 == 0 else -1 for k in range(256)])
    assert np.array_equal(q[0, 256 * g:], (7 * sign).astype(np.int8))
    assert np.all(q[0, :256] == 0)
    assert s[0] == F32(F32(3.0 / 16) / F32(7))
    assert list(q[0, 256:264]) == [7, -7, 7, -7, -7, 7, -7, 7]


@pytest.mark.parametrize("c", [0.5, -2.0, 1.0])
def test_constant_row_codes(c):
    K = 768
    x = np.full((1, K), c, F32)
    q, s = O.quant_act_w4a4(si.f32_to_bf16_bits(x))
    want = np.zeros(K, np.int8)
    want[0::256] = 7 if c > 0 else -7
    assert np.array_equal(q[0], want)
    assert s[0] == F32(F32(16 * abs(c)) / F32(7))


def test_zero_row_and_bias_only_output():
    L = si.random_layer(4, 512, 32, seed=5, bias=True)
    L.x[2, :] = 0
    r = O.linear_w4a4(L.x, L.w, L.bias)
    assert r["sx"][2] == 0 and np.all(r["qx"][2] == 0)
    assert np.array_equal(r["y"][2], O.bf16_to_f32(L.bias))


def test_quant_invariants():
    L = si.tiny()
    qx, sx = O.quant_act_w4a4(L.x)
    xr = O.fwht(O.bf16_to_f32(L.x))
    assert qx.min() >= -8 and qx.max() <= 7
    assert np.all(np.max(np.abs(qx), axis=1) == 7)
    err = np.abs(xr.astype(np.float64) - sx[:, None].astype(np.float64) * qx)
    assert np.all(err <= sx[:, None] * 0.5 * (1 + 1e-6))
    qw, sw = O.quant_weight_w4(L.w)
    assert np.max(np.abs(qw)) == 7 and qw.min() >= -8
    q8, s8 = O.quant_act_int8(L.x)
    assert np.all(np.max(np.abs(q8.astype(np.int32)), axis=1) == 127)


def test_w4_codes_never_reach_minus_8_on_bf16_inputs():
    """The clip bound -8 is never reached from bf16 inputs, however small.

    A nonzero rotated bf16 value is a multiple of 2^-137 (bf16's smallest
    subnormal is 2^-133 and every rotation divides by at most 16), so the
    scale amax / 7 >= 2^-139.8 keeps at least nine significant bits and
    |v / s| <= 7 (1 + 2^-9) < 7.5 before rounding.  Rows of the smallest
    bf16 subnormals, with every rotation, stay in [-7, 7]; the same
    quantiser on raw fp32 subnormals (below that grid) does give -8, so the
    check is not vacuous."""
    rng = np.random.default_rng(17)
    K = 512
    rows = []
    for sign in (0x0000, 0x8000):
        r = np.zeros(K, np.uint16)
        r[3] = sign | 0x0001                                   # one +-2^-133
        rows.append(r)
    rows.append((rng.integers(1, 128, K) | (rng.integers(0, 2, K) << 15)).astype(np.uint16))   # all subnormal
    r = np.zeros(K, np.uint16)
    r[::7] = 0x8001
    r[5] = 0x007F
    rows.append(r)
    x = np.stack(rows)
    cases = [O.quant_act_w4a4(x, g) for g in (256, 64, 16)] + [O.quant_act_w4a4_regular(x)]
    for q, sc in cases:
        assert q.min() >= -7 and q.max() <= 7
        assert np.all(sc > 0)
    vs = O.fwht(O.bf16_to_f32(x)).astype(np.float64)
    _, sx = O.quant_act_w4a4(x)
    assert np.max(np.abs(vs / sx.astype(np.float64)[:, None])) < 7.5
    for g in (256, 64, 16):
        qw, sw = O.quant_weight_w4(x, g)
        assert qw.min() >= -7 and qw.max() <= 7 and sw > 0
    # raw fp32 subnormals: amax = 10 ulps, s = fl(10/7 ulp) = 1 ulp, v / s = -10
    tiny = np.zeros((1, 8), np.float32)
    tiny[0, 2] = -np.float32(10 * 2.0 ** -149)
    q, sc = O.quant_rows(tiny, 7, -8, 7)
    assert sc[0] == np.float32(2.0 ** -149) and q[0, 2] == -8


def test_pack_roundtrip():
    rng = np.random.default_rng(1)
    q = rng.integers(-8, 8, size=(7, 64)).astype(np.int8)
    p = O.pack_int4(q)
    assert p.shape == (7, 32)
    assert np.array_equal(O.unpack_int4(p), q)
    # low nibble = even k, two's complement: codes (-1, 3) -> 0x3F
    assert O.pack_int4(np.array([[-1, 3]], np.int8))[0, 0] == 0x3F
    assert O.pack_int4(np.array([[-8, 7]], np.int8))[0, 0] == 0x78


# ---------------------------------------------------------------------------
# Integer accumulation
# ---------------------------------------------------------------------------

def test_acc_brute_force_python_ints_tiny():
    L = si.tiny()
    r = O.linear_w4a4(L.x, L.w)
    qx, qw, acc = r["qx"], r["qw"], r["acc"]
    for m in (0, 5, 63):
        for n in (0, 17, 255):
            s = 0
            for k in range(qx.shape[1]):
                s += int(qx[m, k]) * int(qw[n, k])
            assert acc[m, n] == s
    full = (qx[:, None, :].astype(np.int64) * qw[None, :, :].astype(np.int64)).sum(-1)
    assert np.array_equal(acc.astype(np.int64), full)
    assert np.max(np.abs(acc)) <= 64 * qx.shape[1]


def test_acc_brute_force_int8_k2688():
    L = si.random_layer(7, 2688, 7, seed=9)
    r = O.linear_int8tw(L.x, L.w)
    qx, qw = r["qx"].astype(np.int64), r["qw"].astype(np.int64)
    for m in range(7):
        for n in range(7):
            assert r["acc"][m, n] == sum(int(a) * int(b) for a, b in zip(qx[m], qw[n]))


def test_epilogue_exact_for_power_of_two_scales():
    acc = np.array([[3, -5], [1000, 0]], np.int32)
    sx = np.array([2.0 ** -3, 2.0 ** 4], F32)
    sw = F32(2.0 ** -7)
    bias = si.f32_to_bf16_bits(np.array([0.5, -0.25], F32))
    y = O.epilogue(acc, sx, sw, bias)
    want = np.array([[3 / 1024 + 0.5, -5 / 1024 - 0.25], [1000 / 8 + 0.5, -0.25]])
    assert np.array_equal(y.astype(np.float64), want)
    y2 = O.epilogue(acc, sx, np.array([2.0 ** -1, 2.0 ** 2], F32), None)
    assert np.array_equal(y2.astype(np.float64),
                          np.array([[3 / 16, -5 / 2], [1000 * 8, 0]]))


def test_end_to_end_close_to_float_linear():
    L = si.random_layer(32, 1024, 64, seed=2, bias=True, outlier_count=6)
    r = O.linear_w4a4(L.x, L.w, L.bias)
    ref = O.bf16_to_f32(L.x).astype(np.float64) @ O.bf16_to_f32(L.w).astype(np.float64).T \
        + O.bf16_to_f32(L.bias)
    rel = np.linalg.norm(r["y"] - ref) / np.linalg.norm(ref)
    assert 0.02 < rel < 0.35
    r8 = O.linear_int8tw(L.x, L.w, L.bias)
    rel8 = np.linalg.norm(r8["y"] - ref) / np.linalg.norm(ref)
    assert rel8 < 0.1 and rel8 < rel


def test_rotation_and_group_size_reduce_error():
    """[ZIT] 'Where Z-Image sits': a rotation of size N spreads an outlier
    over N channels, so the error falls as the group grows."""
    L = si.random_layer(64, 2048, 128, seed=11, outlier_count=10, outlier_scale=40.0)
    x = O.bf16_to_f32(L.x).astype(np.float64)
    w = O.bf16_to_f32(L.w).astype(np.float64)
    ref = x @ w.T

    def err(group):
        if group is None:
            qx, sx = O.quant_rows(O.bf16_to_f32(L.x), 7, -8, 7)
            qw, sw = O.quant_tensor(O.bf16_to_f32(L.w), 7, -8, 7)
        else:
            qx, sx = O.quant_act_w4a4(L.x, group)
            qw, sw = O.quant_weight_w4(L.w, group)
        y = O.epilogue(O.int_gemm(qx, qw), sx, sw, None)
        return np.linalg.norm(y - ref) / np.linalg.norm(ref)

    e_none, e16, e64, e256 = err(None), err(16), err(64), err(256)
    assert e256 < e64 < e16 < e_none


def test_int8tw_weight_error_near_page_figure():
    facts = _golden("page_facts.json")
    L = si.random_layer(1, 3072, 512, seed=6)
    qw, sw = O.quant_weight_int8tw(L.w)
    w = O.bf16_to_f32(L.w).astype(np.float64)
    rel = np.linalg.norm(qw * np.float64(sw) - w) / np.linalg.norm(w)
    assert 0.3 * facts["int8_tensorwise_weight_error"]["value"] < rel < \
        3 * facts["int8_tensorwise_weight_error"]["value"]


# ---------------------------------------------------------------------------
# E4M3 and the W4A8 format
# ---------------------------------------------------------------------------

def test_e4m3_decode_matches_torch():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = O.e4m3_to_f32(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(0, 448, 20000), rng.uniform(0, 0.05, 20000),
                        -rng.uniform(0, 200, 2000),
                        O.e4m3_to_f32(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)])
    v = v.astype(F32)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.f32_to_e4m3_rne(v)
    assert np.array_equal(got, want)


def test_w4a8_decode_hand_cases():
    cb = np.linspace(-1.0, 1.0, 16).astype(F32)
    idx = np.zeros((1, 32), np.uint8)
    idx[0, :16] = np.arange(16)
    idx[0, 16:] = 15
    s_rel = np.array([[0x38, 0x67]], np.uint8)     # 1.0 and 0x67 = 2^5 * 1.875 = 60
    w8 = O.w4a8_decode(idx, s_rel, cb)
    assert np.array_equal(w8[0, :16], np.rint(cb).astype(np.int8))
    assert np.all(w8[0, 16:] == 60)
    s_big = np.array([[0x78, 0x78]], np.uint8)     # 256: 1.0 * 256 clamps to 127
    assert np.all(O.w4a8_decode(idx, s_big, cb)[0, 16:] == 127)
    assert O.w4a8_decode(idx, s_big, cb)[0, 0] == -127


def test_w4a8_storage_matches_page_bytes_per_param():
    facts = _golden("page_facts.json")
    K = 3840
    bytes_per_row = K / facts["int4_codes_per_byte"]["value"] + K / facts["w4a8_scale_group"]["value"]
    assert bytes_per_row / K == pytest.approx(0.5625)
    assert abs(bytes_per_row / K - facts["w4a8_bytes_per_param"]["value"]) < 0.01


def test_lloyd_max_uniform_closed_form():
    # the optimal 16-level quantiser of U(-1, 1) is uniform: levels (2j+1)/16 - 1
    rng = np.random.default_rng(0)
    u = rng.uniform(-1, 1, 400_000)
    cb, hist = O.lloyd_max_16(u, iters=300)
    want = (2 * np.arange(16) + 1) / 16 - 1
    assert np.max(np.abs(cb - want)) < 0.01
    assert all(b <= a * (1 + 1e-12) for a, b in zip(hist, hist[1:]))


def test_lloyd_max_gaussian_textbook_levels():
    # Max (1960), 16-level minimum-MSE quantiser for N(0,1): positive levels
    want = np.array([0.1284, 0.3881, 0.6568, 0.9424, 1.2562, 1.6181, 2.0690, 2.7326])
    rng = np.random.default_rng(1)
    cb, _ = O.lloyd_max_16(rng.normal(size=1_000_000), iters=500)
    assert np.all(np.diff(cb) > 0)
    assert np.max(np.abs(np.sort(np.abs(cb[8:])) - want)) < 0.03
    assert np.max(np.abs(cb[:8][::-1] + want)) < 0.03


def test_lloyd_max_hand_fixture():
    """R10 by hand: samples 0..31 and 1.9375 (float32).  lo = 0, hi = 31, so
    the start is c_j = (j + 1/2) * 1.9375 with midpoints (j + 1) * 1.9375;
    the sample 1.9375 sits on the first midpoint and goes to the lower cell:
    after one iteration cell 0 = {0, 1, 1.9375} (mean 2.9375 / 3), cell j >= 1
    = {2j, 2j + 1} (mean 2j + 1/2).  Then the first midpoint drops to
    (2.9375/3 + 2.5) / 2 < 1.9375 and the sample moves up: cell 0 = {0, 1}
    (0.5), cell 1 = {1.9375, 2, 3} (6.9375 / 3 = 2.3125), and nothing moves
    after that."""
    u = np.concatenate([np.arange(32), [1.9375]]).astype(F32)
    one, _ = O.lloyd_max_16(u, iters=1)
    want1 = np.array([2.9375 / 3] + [2 * j + 0.5 for j in range(1, 16)])
    assert np.array_equal(one, want1.astype(F32))
    cb, hist = O.lloyd_max_16(u, iters=100)
    want = np.array([0.5, 2.3125] + [2 * j + 0.5 for j in range(2, 16)])
    assert np.array_equal(cb, want.astype(F32))
    assert len(hist) == 3                     # two moves, then a pass that changes nothing


def test_w4a8_encode_weight_error_near_page_figure():
    facts = _golden("page_facts.json")
    L = si.random_layer(1, 1024, 256, seed=8)
    enc = O.w4a8_encode(L.w)
    w8 = O.w4a8_decode(enc["idx"], enc["s_rel"], enc["codebook"])
    rec = w8.astype(np.float64) * enc["s_channel"][:, None]
    wr = enc["w_rot"].astype(np.float64)
    rel = np.linalg.norm(rec - wr) / np.linalg.norm(wr)
    page = facts["w4a8_weight_rel_l2"]["value"]
    assert 0.5 * page < rel < 1.7 * page
    assert np.all(np.diff(enc["codebook"]) > 0)
    assert np.array_equal(O.unpack_uint4(enc["idx_packed"]), enc["idx"])
    h = enc["distortion"]
    assert all(b <= a * (1 + 1e-12) for a, b in zip(h, h[1:]))


def test_w4a8_linear_runs_and_is_close():
    L = si.random_layer(16, 512, 64, seed=12, bias=True)
    enc = O.w4a8_encode(L.w)
    r = O.linear_w4a8(L.x, enc["idx_packed"], enc["s_rel"], enc["codebook"], enc["s_channel"], L.bias)
    ref = O.bf16_to_f32(L.x).astype(np.float64) @ O.bf16_to_f32(L.w).astype(np.float64).T \
        + O.bf16_to_f32(L.bias)
    rel = np.linalg.norm(r["y"] - ref) / np.linalg.norm(ref)
    assert rel < 0.15
    assert np.max(np.abs(r["w8"].astype(np.int32))) <= 127


def test_bf16_rne():
    v = np.array([1.0, 1.00390625, 1.005859375, -3.0e38, 1e-40], F32)
    got = O.f32_to_bf16_rne(v)
    # 1+2^-8 is a tie -> 1.0 (even); 1+3*2^-9 rounds up to 1+2^-7
    assert got[0] == 0x3F80 and got[1] == 0x3F80 and got[2] == 0x3F81
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    w = (rng.normal(size=10000) * 10).astype(F32)
    want = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_rne(w), want)


# ---------------------------------------------------------------------------
# ConvRot INT8, row-scaled (reading R17)
# ---------------------------------------------------------------------------

def test_int8rot_row_scale_invariance():
    """Rows that are power-of-two multiples of one row: the rotation and the
    per-row scale commute with the power of two, so every row gets the same
    codes and its scale is the base scale times that power, exactly.  (One
    scale for the whole tensor would give the small rows other codes.)"""
    rng = np.random.default_rng(11)
    K = 512
    base = O.bf16_to_f32(si.f32_to_bf16_bits(rng.standard_normal((1, K)).astype(F32)))
    ks = [0, -3, 2, 5, -1]
    w = np.concatenate([base * F32(2.0 ** k) for k in ks]).astype(F32)
    wb = si.f32_to_bf16_bits(w)
    assert np.array_equal(O.bf16_to_f32(wb), w)
    q, s = O.quant_weight_int8rot(wb)
    for i, k in enumerate(ks):
        assert np.array_equal(q[i], q[0])
        assert s[i] == F32(s[0] * F32(2.0 ** k))
    assert np.max(np.abs(q[0])) == 127


def test_int8rot_one_hot_weight_rows():
    """A weight row c * e_j in group g rotates to c/16 times row j of the
    Sylvester matrix in group g: codes +-127 in that sign pattern there, 0 in
    the other groups, scale fl(fl(|c|/16)/127)."""
    K = 768
    rows = [(2.0, 37, 1), (-0.75, 0, 0), (5.0, 255, 2)]
    w = np.zeros((len(rows), K), F32)
    for n, (c, j, g) in enumerate(rows):
        w[n, 256 * g + j] = c
    q, s = O.quant_weight_int8rot(si.f32_to_bf16_bits(w))
    for n, (c, j, g) in enumerate(rows):
        sign = np.array([1 if _popcount(j & k) % 2 == 0 else -1 for k in range(256)])
        want = np.zeros(K, np.int8)
        want[256 * g:256 * (g + 1)] = (127 * sign * (1 if c > 0 else -1)).astype(np.int8)
        assert np.array_equal(q[n], want)
        assert s[n] == F32(F32(abs(c) / 16) / F32(127))


def test_int8rot_acc_brute_force_python_ints():
    """acc[m, n] = sum_k qx[m, k] * qw[n, k] over Python integers, and the
    epilogue's scale of column n is the weight row n's scale."""
    L = si.random_layer(3, 256, 5, seed=21, bias=True, outlier_count=3)
    r = O.linear_int8rot(L.x, L.w, L.bias)
    qx, qw = r["qx"].astype(int), r["qw"].astype(int)
    for m in range(3):
        for n in range(5):
            assert int(r["acc"][m, n]) == sum(int(qx[m, k]) * int(qw[n, k]) for k in range(256))
    b = O.bf16_to_f32(L.bias)
    for m in range(3):
        for n in range(5):
            want = F32(F32(F32(r["acc"][m, n]) * r["sx"][m]) * r["sw"][n]) + b[n]
            assert r["y"][m, n] == want


def test_int8rot_row_scaling_beats_tensorwise_on_uneven_rows():
    """Weights whose rows differ in magnitude by 2^6: per-row scales keep every
    row at full int8 resolution, one tensor scale does not."""
    rng = np.random.default_rng(3)
    N, K = 32, 1024
    w = rng.normal(0, 0.02, (N, K)).astype(F32)
    w[::4] *= 64
    wb = si.f32_to_bf16_bits(w)
    wr = O.fwht(O.bf16_to_f32(wb))
    q, s = O.quant_weight_int8rot(wb)
    err_row = np.linalg.norm(q * s[:, None] - wr) / np.linalg.norm(wr)
    qt, st = O.quant_tensor(wr, 127, -128, 127)
    small = np.arange(N) % 4 != 0
    err_small_row = np.linalg.norm((q * s[:, None] - wr)[small]) / np.linalg.norm(wr[small])
    err_small_t = np.linalg.norm((qt * st - wr)[small]) / np.linalg.norm(wr[small])
    assert err_small_row < 0.02 and err_small_t > 4 * err_small_row
    assert err_row < 0.02


# --- the rotated int8 activations of ConvRot INT8 (R17) and W4A8 (R8) -------
# Both formats rotate x online with the group-256 Sylvester matrix and take
# per-row int8 codes with absmax / 127.  A one-hot row c * e_j of group g
# rotates to c/16 times row j of the Sylvester matrix in that group, so every
# code there is +-127 in that row's sign pattern (popcount(j & k) parity), 0
# in the other groups, and the scale is fl(fl(|c| / 16) / 127).  A constant
# row c rotates to 16 c at each group's k = 0 and 0 elsewhere.

_ROT_INT8_ACT = [("int8rot", lambda xb: O.quant_act_int8rot(xb)),
                 ("w4a8", lambda xb: O.quant_act_w4a8(xb))]


@pytest.mark.parametrize("fmt", [f for f, _ in _ROT_INT8_ACT])
def test_rotated_int8_act_one_hot_rows(fmt):
    quant = dict(_ROT_INT8_ACT)[fmt]
    K = 768
    rows = [(3.0, 37, 1), (-0.5, 0, 0), (1.25, 255, 2), (-6.0, 170, 0)]
    x = np.zeros((len(rows), K), F32)
    for m, (c, j, g) in enumerate(rows):
        x[m, 256 * g + j] = c
    q, s = quant(si.f32_to_bf16_bits(x))
    for m, (c, j, g) in enumerate(rows):
        sign = np.array([1 if _popcount(j & k) % 2 == 0 else -1 for k in range(256)])
        want = np.zeros(K, np.int8)
        want[256 * g:256 * (g + 1)] = (127 * sign * (1 if c > 0 else -1)).astype(np.int8)
        assert np.array_equal(q[m], want)
        assert s[m] == F32(F32(abs(c) / 16) / F32(127))
    # row 0 (j = 37 = 0b100101) by hand: k = 0..7 -> + - + - - + - +
    assert list(q[0, 256:264]) == [127, -127, 127, -127, -127, 127, -127, 127]


@pytest.mark.parametrize("fmt", [f for f, _ in _ROT_INT8_ACT])
@pytest.mark.parametrize("c", [0.75, -2.0])
def test_rotated_int8_act_constant_rows(fmt, c):
    quant = dict(_ROT_INT8_ACT)[fmt]
    K = 512
    q, s = quant(si.f32_to_bf16_bits(np.full((1, K), c, F32)))
    want = np.zeros(K, np.int8)
    want[0::256] = 127 if c > 0 else -127
    assert np.array_equal(q[0], want)
    assert s[0] == F32(F32(16 * abs(c)) / F32(127))


def test_linear_int8rot_close_to_float_linear():
    """ConvRot INT8 against the float64 x W^T + b: both operands at int8
    resolution after the rotation has spread the outlier channels, so the
    relative error sits near 1e-2, far below the 4-bit linear's (~0.2) and
    below int8_tensorwise without rotation (~0.05) on the same inputs."""
    for seed, (M, K, N) in enumerate([(32, 1024, 64), (16, 2560, 128)]):
        L = si.random_layer(M, K, N, seed=30 + seed, bias=True, outlier_count=4)
        ref = O.bf16_to_f32(L.x).astype(np.float64) @ O.bf16_to_f32(L.w).astype(np.float64).T \
            + O.bf16_to_f32(L.bias)
        rel = lambda y: np.linalg.norm(y - ref) / np.linalg.norm(ref)   # noqa: E731
        e_rot = rel(O.linear_int8rot(L.x, L.w, L.bias)["y"])
        e_w4 = rel(O.linear_w4a4(L.x, L.w, L.bias)["y"])
        assert e_rot < 0.02
        assert e_rot < 0.1 * e_w4


def test_uint4_nibble_order_hand_bytes():
    """Codebook indices (R8 storage): low nibble = even k, unsigned.  Hand
    bytes: indices (1, 2) -> 0x21, (15, 0) -> 0x0F, (0, 15) -> 0xF0."""
    idx = np.array([[1, 2, 15, 0, 0, 15]], np.uint8)
    p = O.pack_uint4(idx)
    assert list(p[0]) == [0x21, 0x0F, 0xF0]
    assert list(O.unpack_uint4(np.array([[0x21, 0x0F, 0xF0, 0x9A]], np.uint8))[0]) == [1, 2, 15, 0, 0, 15, 10, 9]


# ---------------------------------------------------------------------------
# Smaller rotation groups ([ZIT] "Where Z-Image sits": group sizes 64 and 16)
# ---------------------------------------------------------------------------

def _sylvester(n):
    g = np.array([[1.0]])
    while g.shape[0] < n:
        g = np.block([[g, g], [g, -g]])
    return g


@pytest.mark.parametrize("G", [16, 64])
def test_fwht_group_unit_vectors_block_diagonal(G):
    """e_j rotated in groups of G: (-1)^popcount((j % G) & (k % G)) / sqrt(G)
    inside j's group, zero in every other group."""
    K = 256
    got = O.fwht(np.eye(K, dtype=F32), G).astype(np.float64)
    want = np.zeros((K, K))
    for j in range(K):
        for k in range(K):
            if j // G == k // G:
                want[j, k] = (-1.0) ** _popcount((j % G) & (k % G)) / np.sqrt(G)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("G", [16, 64])
def test_fwht_group_float64_equals_dense_block_product(G):
    rng = np.random.default_rng(G)
    x = rng.normal(size=(3, 512))
    got = O.fwht(x, G, dtype=np.float64)
    H = _sylvester(G) / np.sqrt(G)
    want = (x.reshape(3, 512 // G, G) @ H).reshape(3, 512)
    assert np.max(np.abs(got - want)) <= 1e-14 * np.max(np.abs(want))


@pytest.mark.parametrize("G", [16, 64])
def test_fwht_group_float32_within_error_bound(G):
    rng = np.random.default_rng(40 + G)
    x32 = rng.standard_t(3, size=(6, 512)).astype(F32)
    got = O.fwht(x32, G).astype(np.float64)
    H = _sylvester(G) / np.sqrt(G)
    want = (x32.astype(np.float64).reshape(6, 512 // G, G) @ H).reshape(6, 512)
    stages = int(np.log2(G))
    l1 = np.abs(x32.astype(np.float64)).reshape(6, 512 // G, G).sum(-1)
    bound = stages * 2.0 ** -24 * l1 / np.sqrt(G) * 1.0001
    err = np.abs(got - want).reshape(6, 512 // G, G)
    assert np.all(err <= bound[:, :, None])


@pytest.mark.parametrize("G", [16, 64])
def test_group_one_hot_row_codes(G):
    """x = 3 e_j: codes 7 (-1)^popcount((j % G) & (k % G)) in j's group, 0
    elsewhere; scale fl(fl(3 / sqrt(G)) / 7)."""
    K, j = 512, 300
    x = np.zeros((1, K), F32)
    x[0, j] = 3.0
    q, s = O.quant_act_w4a4(si.f32_to_bf16_bits(x), G)
    want = np.zeros(K, np.int8)
    g0 = (j // G) * G
    for k in range(G):
        want[g0 + k] = 7 if _popcount((j % G) & k) % 2 == 0 else -7
    assert np.array_equal(q[0], want)
    assert s[0] == F32(F32(3.0 / np.sqrt(G)) / F32(7))


@pytest.mark.parametrize("G", [16, 64])
@pytest.mark.parametrize("c", [0.5, -2.0])
def test_group_constant_row_codes(G, c):
    """A constant row rotates to sqrt(G) c at the first k of every group and 0
    elsewhere: codes +-7 there, scale fl(fl(sqrt(G) |c|) / 7)."""
    K = 768
    x = np.full((1, K), c, F32)
    q, s = O.quant_act_w4a4(si.f32_to_bf16_bits(x), G)
    want = np.zeros(K, np.int8)
    want[0::G] = 7 if c > 0 else -7
    assert np.array_equal(q[0], want)
    assert s[0] == F32(F32(np.sqrt(G) * abs(c)) / F32(7))


@pytest.mark.parametrize("G", [16, 64])
def test_group_exact_identity_before_quantisation(G):
    L = si.tiny()
    x = O.bf16_to_f32(L.x).astype(np.float64)
    w = O.bf16_to_f32(L.w).astype(np.float64)
    lhs = O.fwht(x, G, dtype=np.float64) @ O.fwht(w, G, dtype=np.float64).T
    rhs = x @ w.T
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs))


@pytest.mark.parametrize("G", [16, 64])
def test_group_weight_one_hot_codes(G):
    """A weight whose largest entry is c e_j in row n: that row's codes are
    7 (-1)^popcount(...) in j's group (the tensor absmax comes from it)."""
    N, K, n, j = 4, 256, 2, 77
    w = np.zeros((N, K), F32)
    w[n, j] = -5.0
    w[0, 3] = 1.0
    q, s = O.quant_weight_w4(si.f32_to_bf16_bits(w), G)
    g0 = (j // G) * G
    for k in range(G):
        sign = 1 if _popcount((j % G) & k) % 2 == 0 else -1
        assert q[n, g0 + k] == -7 * sign
    assert np.all(q[n, :g0] == 0) and np.all(q[n, g0 + G:] == 0)
    assert s == F32(F32(5.0 / np.sqrt(G)) / F32(7))


# ---------------------------------------------------------------------------
# Regular Hadamard rotation (R19; [QIE] intro "regular-Hadamard")
# ---------------------------------------------------------------------------

def _regular_entry(i, j):
    """prod over the four base-4 digits of (1 - 2 [i_d == j_d]), written out
    digit by digit (the entries of (J - 2I) x (J - 2I) x ...)."""
    e = 1
    for _ in range(4):
        e *= -1 if (i % 4) == (j % 4) else 1
        i //= 4
        j //= 4
    return e


def _sigma(d):
    # sign a one-hot group picks up in a radix-4 stage: position 0 of the
    # group gets t - 2 x0 = -x0, the others t = x0
    return -1.0 if d == 0 else 1.0


def test_regular_hadamard_closed_form_orthonormal_regular():
    H = O.regular_hadamard()
    want = np.array([[_regular_entry(i, j) / 16.0 for j in range(256)] for i in range(256)])
    assert np.array_equal(H, want)
    assert np.array_equal(H @ H.T, np.eye(256))
    assert np.array_equal(H, H.T)
    assert np.array_equal(H.sum(axis=1), np.ones(256))      # every row sums to 1 (regular)


def test_rht_unit_vectors_give_rows():
    got = O.rht(np.eye(256, dtype=F32)).astype(np.float64)
    want = np.array([[_regular_entry(i, j) / 16.0 for j in range(256)] for i in range(256)])
    assert np.array_equal(got, want)


def test_rht_float64_equals_dense_product():
    rng = np.random.default_rng(14)
    x = rng.normal(size=(4, 768))
    got = O.rht(x, dtype=np.float64)
    H = np.array([[_regular_entry(i, j) / 16.0 for j in range(256)] for i in range(256)])
    want = (x.reshape(4, 3, 256) @ H).reshape(4, 768)
    assert np.max(np.abs(got - want)) <= 1e-14 * np.max(np.abs(want))


def test_rht_float32_within_error_bound():
    """Error of the float32 stages against the exact product, u = 2^-24.  An
    output of a stage, t - 2 x_k with t = (x0 + x1) + (x2 + x3), takes four
    roundings (the two pair sums, t, the output), together below u times
    |x0 + x1| + |x2 + x3| + |t| + |t - 2 x_k| <= 5 ||x_4||_1 <= 10 ||x_4||_2
    over its 4-group (first order in u), so one stage adds an error of L2
    norm <= 20 u ||x||_2 over the 256-group; the exact stage (J - 2I per
    digit, (J - 2I)^T (J - 2I) = 4 I) doubles L2 norms, so four stages give
    <= 20 u (8 + 8 + 8 + 8) ||x||_2 = 640 u ||x||_2, i.e. 40 u ||x_g||_2
    after the 1/16: a bound on every element's error."""
    rng = np.random.default_rng(15)
    x32 = rng.standard_t(3, size=(8, 512)).astype(F32)
    got = O.rht(x32).astype(np.float64)
    H = np.array([[_regular_entry(i, j) / 16.0 for j in range(256)] for i in range(256)])
    want = (x32.astype(np.float64).reshape(8, 2, 256) @ H).reshape(8, 512)
    l2 = np.sqrt((x32.astype(np.float64).reshape(8, 2, 256) ** 2).sum(-1))
    err = np.abs(got - want).reshape(8, 2, 256)
    assert np.all(err <= (40 * 2.0 ** -24 * l2)[:, :, None])
    assert np.max(err) > 0                                   # float32 arithmetic really ran


def test_rht_pairwise_sum_fixture():
    """x0 = 1, x2 = x3 = e = 2^-24 (bf16 values): the first stage's sum is
    (1 + 0) + (e + e) = 1 + 2^-23 exactly (a left-to-right sum would round
    1 + e to 1 twice), so that group becomes (t - 2, t, t - 2e, t) =
    (-1 + 2^-23, 1 + 2^-23, 1, 1); the later stages see one non-zero value
    per group and only apply the signs sigma(d)."""
    e = 2.0 ** -24
    x = np.zeros(256, F32)
    x[0], x[2], x[3] = 1.0, e, e
    w = [-1 + 2.0 ** -23, 1 + 2.0 ** -23, 1.0, 1.0]
    want = np.array([w[i % 4] * _sigma((i // 4) % 4) * _sigma((i // 16) % 4) * _sigma(i // 64) / 16
                     for i in range(256)], np.float64).astype(F32)
    assert np.array_equal(O.rht(x).view(np.uint32), want.view(np.uint32))


def test_rht_stage_order_fixture():
    """x0 = 1, x5 = e = 2^-24 with the stages in ascending stride order.
    Stride 1: (1,0,0,0) -> (-1,1,1,1) at 0..3 and (0,e,0,0) -> (e,-e,e,e) at
    4..7.  Stride 4, groups (r, 4+r, 8+r, 12+r) holding (P0[r], P1[r], 0, 0),
    t = P0[r] + P1[r]:
      r=0: t = -1 + e (exact) -> (t+2, t-2e, t, t) = (1, -1, -1+e, -1+e)
           (1 + e and -1 - e are ties that round to the even 1 and -1);
      r=1: t = 1 - e -> (t-2, t+2e, t, t) = (-1, 1, 1-e, 1-e);
      r=2, 3: t = 1 + e rounds to 1 -> (-1, 1 - 2e, 1, 1).
    Strides 16 and 64 then apply sigma(d2) sigma(d3).  Descending strides
    would meet 1 and e only in the last stage and give -(1 - e) at 2, 3."""
    e = 2.0 ** -24
    x = np.zeros(256, F32)
    x[0], x[5] = 1.0, e
    u = np.zeros(16)
    u[[0, 4, 8, 12]] = [1, -1, -1 + e, -1 + e]
    u[[1, 5, 9, 13]] = [-1, 1, 1 - e, 1 - e]
    for r in (2, 3):
        u[[r, 4 + r, 8 + r, 12 + r]] = [-1, 1 - 2 * e, 1, 1]
    want = np.array([u[i % 16] * _sigma((i // 16) % 4) * _sigma(i // 64) / 16 for i in range(256)],
                    np.float64).astype(F32)
    assert np.array_equal(O.rht(x).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("c", [0.5, -3.0])
def test_rht_constant_row_stays_constant(c):
    """Every row of the regular matrix sums to 1, so a constant row rotates to
    itself (each stage maps (c,c,c,c) to (2c,...): 16c, then x 1/16): codes
    +-7 everywhere, scale fl(|c| / 7) - unlike the Sylvester rotation, which
    moves it all to the first k of each group."""
    K = 512
    x = np.full((1, K), c, F32)
    q, s = O.quant_act_w4a4_regular(si.f32_to_bf16_bits(x))
    assert np.all(q[0] == (7 if c > 0 else -7))
    assert s[0] == F32(F32(abs(c)) / F32(7))


def test_rht_one_hot_row_codes():
    j, g = 201, 1
    x = np.zeros((1, 512), F32)
    x[0, 256 * g + j] = -2.0
    q, s = O.quant_act_w4a4_regular(si.f32_to_bf16_bits(x))
    want = np.array([-7 * _regular_entry(j, k) for k in range(256)], np.int8)
    assert np.array_equal(q[0, 256 * g:], want) and np.all(q[0, :256] == 0)
    assert s[0] == F32(F32(2.0 / 16) / F32(7))


def test_rht_exact_identity_before_quantisation():
    L = si.tiny()
    x = O.bf16_to_f32(L.x).astype(np.float64)
    w = O.bf16_to_f32(L.w).astype(np.float64)
    lhs = O.rht(x, dtype=np.float64) @ O.rht(w, dtype=np.float64).T
    rhs = x @ w.T
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs))


# ---------------------------------------------------------------------------
# Text-encoder MLP block (R20)
# ---------------------------------------------------------------------------

def test_silu_mul_matches_library_logistic():
    """silu(g) * u against scipy's logistic function (an independent
    implementation): g * expit(g) * u in float64, rounded to float32, then
    bf16.  The two float64 values differ by an ulp or so; a bf16 rounding
    could only differ within ~1e-16 of a boundary, which 2e5 random values
    do not hit."""
    from scipy.special import expit
    rng = np.random.default_rng(16)
    g = si.f32_to_bf16_bits((rng.standard_t(3, size=200_000) * 2).astype(F32))
    u = si.f32_to_bf16_bits(rng.standard_normal(200_000).astype(F32))
    g64 = O.bf16_to_f32(g).astype(np.float64)
    u64 = O.bf16_to_f32(u).astype(np.float64)
    want = O.f32_to_bf16_rne((g64 * expit(g64) * u64).astype(F32))
    assert np.array_equal(O.silu_mul_bf16(g, u), want)


def test_silu_mul_special_values():
    bits = lambda a: si.f32_to_bf16_bits(np.array(a, F32))
    f = lambda h: O.bf16_to_f32(h)
    # silu(0) = 0; u = 0 gives 0
    assert np.all(f(O.silu_mul_bf16(bits([0.0, 0.0]), bits([3.0, -1.0]))) == 0)
    assert np.all(f(O.silu_mul_bf16(bits([2.5, -7.0]), bits([0.0, 0.0]))) == 0)
    # large positive g: silu(g) = g to float32 precision; large negative: 0
    h = f(O.silu_mul_bf16(bits([96.0, -200.0, -1000.0]), bits([0.5, 1.0, 1.0])))
    assert h[0] == 48.0 and h[1] == 0 and h[2] == 0
    # silu(1) = 1 / (1 + e^-1) = 0.7310585786...; bf16 nearest is 0.73046875
    assert f(O.silu_mul_bf16(bits([1.0]), bits([1.0])))[0] == np.float32(0.73046875)


def test_silu_odd_part_identity():
    """silu(v) - silu(-v) = v exactly in real arithmetic: with u = 1 the bf16
    results satisfy it within two bf16 roundings."""
    v = np.linspace(-8, 8, 1601).astype(F32)
    vb = si.f32_to_bf16_bits(v)
    nb = si.f32_to_bf16_bits(-O.bf16_to_f32(vb))
    one = si.f32_to_bf16_bits(np.ones_like(v))
    hp = O.bf16_to_f32(O.silu_mul_bf16(vb, one)).astype(np.float64)
    hn = O.bf16_to_f32(O.silu_mul_bf16(nb, one)).astype(np.float64)
    vv = O.bf16_to_f32(vb).astype(np.float64)
    assert np.all(np.abs((hp - hn) - vv) <= 2.0 ** -8 * (np.abs(hp) + np.abs(hn)) + 1e-30)


def test_mlp_block_close_to_float_mlp():
    """The W4A4 MLP block against the float64 gated MLP of the same bf16
    inputs: the error of three 4-bit linears, and the intermediates are the
    bf16 outputs of the gate and up linears."""
    rng = np.random.default_rng(17)
    M, K, F, N = 24, 512, 768, 512
    x = si.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(F32))
    wg = si.f32_to_bf16_bits((rng.standard_normal((F, K)) * 0.05).astype(F32))
    wu = si.f32_to_bf16_bits((rng.standard_normal((F, K)) * 0.05).astype(F32))
    wd = si.f32_to_bf16_bits((rng.standard_normal((N, F)) * 0.05).astype(F32))
    r = O.mlp_w4a4(x, wg, wu, wd)
    assert np.array_equal(r["g"], O.f32_to_bf16_rne(O.linear_w4a4(x, wg)["y"]))
    x64 = O.bf16_to_f32(x).astype(np.float64)
    g = x64 @ O.bf16_to_f32(wg).astype(np.float64).T
    u = x64 @ O.bf16_to_f32(wu).astype(np.float64).T
    h = g / (1 + np.exp(-g)) * u
    ref = h @ O.bf16_to_f32(wd).astype(np.float64).T
    rel = np.linalg.norm(r["y"] - ref) / np.linalg.norm(ref)
    # three 4-bit linears in a row (about 0.43 here; the "qwen3vl_4b" page
    # reports ~0.5 relative RMSE for the whole W4A4 encoder at 76 tokens)
    assert 0.1 < rel < 0.6
