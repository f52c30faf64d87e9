"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact: activation codes and scales, weight codes and scales, int32
accumulators.  bf16 outputs: within max relative error 1e-2 of the oracle's
float32 epilogue (they are expected to equal its bf16 rounding)."""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import convrot_oracle as O
from tests._util import TOL, bf16_dev_to_f32, max_rel_err, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def crp():
    import rotated_bit_quantized_convrot_amd as m
    m.lib()
    return m


def _sync():
    torch.cuda.synchronize()


KIND_ORACLE_ACT = {
    0: O.quant_act_w4a4,
    1: O.quant_act_int8,
    2: O.quant_act_w4a8,
    3: O.quant_act_int8rot,
}


# ---------------------------------------------------------------------------
# Activation quantisation
# ---------------------------------------------------------------------------

ACT_CASES = [
    (0, 64, 512), (0, 76, 2560), (0, 33, 9728), (0, 3, 256), (0, 5, 12288), (0, 2, 65536),
    (0, 33, 512), (0, 17, 768), (0, 9, 1024), (0, 7, 1280), (0, 3, 32768), (0, 300, 3072),
    (1, 64, 2688), (1, 9, 100), (1, 17, 3072), (1, 1, 7),
    (1, 33, 512), (1, 5, 4096), (1, 130, 1000), (1, 4, 4104),
    # int8_tensorwise rows held in registers: 1 to 4 chunks of 8 per thread
    (1, 40, 8192), (1, 3, 6144), (1, 2049, 3072), (1, 2050, 4096),
    # rotated int8 codes (and unpacked W4A4 codes) four rows per block at M >= 2048
    (3, 2049, 2560), (3, 2050, 8192), (2, 2051, 256), (0, 2052, 3072),
    (2, 40, 3840), (2, 3, 256),
    # grids larger than the chip holds at once: two groups per lane (rotated)
    # or two waves per row (int8_tensorwise)
    (2, 2100, 3840), (0, 1100, 8192), (1, 2100, 640),
    # M >= 2048 with more than 32 groups per row: one row per block
    (0, 2050, 9216),
    (3, 76, 2560), (3, 300, 512), (3, 5, 9728),
]


@pytest.mark.parametrize("kind,M,K", ACT_CASES)
def test_quant_act_bitexact(crp, kind, M, K):
    L = si.random_layer(M, K, 1, seed=100 + M + K, outlier_count=min(8, K), outlier_scale=40.0)
    x = L.x.copy()
    if M >= 3:
        x[1, :] = 0                                  # zero row
        x[2, :] = si.f32_to_bf16_bits(np.full(K, 0.75, np.float32))   # constant row
    q, s = crp.dbg_quant_act(kind, to_dev_bf16(x))
    _sync()
    q_ref, s_ref = KIND_ORACLE_ACT[kind](x)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def _rows_from_rotated(y_rows):
    """bf16 rows x with rotate(x) == y exactly: x = H y per 256-group (the
    normalised Sylvester Hadamard is symmetric and its own inverse); asserts
    that every x is exactly a bf16 value."""
    H = O.hadamard(256)
    y = np.asarray(y_rows, np.float64)
    R, K = y.shape
    x = (y.reshape(R, K // 256, 256) @ H.T).reshape(R, K)
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x)
    bits = si.f32_to_bf16_bits(x32)
    assert np.array_equal(si.bf16_bits_to_f32(bits).astype(np.float64), x)
    return bits


@pytest.mark.parametrize("kind", [0, 2])
def test_quant_act_exact_ties(crp, kind):
    """Rotated values exactly on half-integer multiples of the scale (round
    half to even decides) next to the row maximum."""
    qmax = 7 if kind == 0 else 127
    K = 256 * 8
    rows = []
    for e in (-3, 0, 5):
        y = np.zeros(K)
        for g in range(8):
            y[g * 256] = qmax * 2.0 ** e                  # the row maximum: scale 2^e
            if kind == 0:
                k = g % 7
                y[g * 256 + 1 + g] = (-1) ** g * (k + 0.5) * 2.0 ** e
            else:
                y[g * 256 + 1 + g] = (-1) ** g * 0.5 * 2.0 ** e
        rows.append(y)
    x = _rows_from_rotated(rows)
    q, s = crp.dbg_quant_act(kind, to_dev_bf16(x))
    _sync()
    q_ref, s_ref = KIND_ORACLE_ACT[kind](x)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_quant_act_extreme_magnitudes(crp, kind):
    """Rows whose max lies outside [2^-100, 2^100] before the 1/16 (tiny,
    huge, subnormal bf16) next to ordinary rows."""
    rng = np.random.default_rng(7)
    K = 512
    base = rng.standard_normal((6, K)).astype(np.float32)
    scales = [1.0, 1e-33, 1e33, 1e-39, 3e-38, 1.0]
    x = si.f32_to_bf16_bits(base * np.array(scales, np.float32)[:, None])
    q, s = crp.dbg_quant_act(kind, to_dev_bf16(x))
    _sync()
    q_ref, s_ref = KIND_ORACLE_ACT[kind](x)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_quant_act_int8_exact_ties(crp):
    """int8_tensorwise rows whose values sit exactly on half-integer multiples
    of the scale (s = 2^e exactly): round half to even decides."""
    K = 1024
    rows = []
    for e in (-6, 0, 3):
        r = np.zeros(K, np.float32)
        r[0] = 127.0 * 2.0 ** e                           # the row maximum: scale 2^e
        for i in range(1, 40):
            r[i] = (-1) ** i * ((i % 9) + 0.5) * 2.0 ** e
        rows.append(r)
    x = si.f32_to_bf16_bits(np.stack(rows))
    assert np.array_equal(si.bf16_bits_to_f32(x), np.stack(rows))
    q, s = crp.dbg_quant_act(1, to_dev_bf16(x))
    _sync()
    q_ref, s_ref = KIND_ORACLE_ACT[1](x)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_quant_act_stage_order_fixture(crp):
    """The hand-derived stage-order case: codes and scale bits."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fwht_order_case.json")))
    x = np.zeros((1, 256), np.uint16)
    for k, h in g["input_bf16_hex"].items():
        x[0, int(k)] = int(h, 16)
    q, s = crp.dbg_quant_act(0, to_dev_bf16(x))
    _sync()
    assert np.array_equal(q.cpu().numpy()[0], np.tile(np.array(g["expected_int4_codes_by_k_mod_4"], np.int8), 64))
    assert s.cpu().numpy().view(np.uint32)[0] == int(g["expected_scale_f32_hex"], 16)


# ---------------------------------------------------------------------------
# Weight packing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(256, 512), (100, 512), (33, 256), (64, 2560)])
def test_pack_w4_bitexact(crp, N, K):
    L = si.random_layer(1, K, N, seed=N * 7 + K)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    codes = crp.dbg_unpack_weight(0, p, N, K)
    _sync()
    q_ref, s_ref = O.quant_weight_w4(L.w)
    assert np.array_equal(codes.cpu().numpy(), q_ref)
    assert s.cpu().numpy()[:1].view(np.uint32)[0] == np.float32(s_ref).view(np.uint32)


@pytest.mark.parametrize("N,K", [(256, 512), (7, 100), (64, 2688), (40, 3072)])
def test_pack_int8tw_bitexact(crp, N, K):
    L = si.random_layer(1, K, N, seed=N * 5 + K)
    p, s = crp.pack_weight_int8tw(to_dev_bf16(L.w))
    codes = crp.dbg_unpack_weight(1, p, N, K)
    _sync()
    q_ref, s_ref = O.quant_weight_int8tw(L.w)
    assert np.array_equal(codes.cpu().numpy(), q_ref)
    assert s.cpu().numpy()[:1].view(np.uint32)[0] == np.float32(s_ref).view(np.uint32)


def _w4a8_dev(crp, idx_packed, s_rel, cb, N, K):
    return crp.pack_weight_w4a8(to_dev(idx_packed), to_dev(s_rel), to_dev(cb.astype(np.float32)), N, K)


@pytest.mark.parametrize("N,K", [(256, 512), (50, 768)])
def test_pack_w4a8_decode_bitexact(crp, N, K):
    L = si.random_layer(1, K, N, seed=N + K)
    enc = O.w4a8_encode(L.w)
    p = _w4a8_dev(crp, enc["idx_packed"], enc["s_rel"], enc["codebook"], N, K)
    codes = crp.dbg_unpack_weight(2, p, N, K)
    _sync()
    assert np.array_equal(codes.cpu().numpy(), O.w4a8_decode(enc["idx"], enc["s_rel"], enc["codebook"]))


def test_pack_w4a8_random_format_bitexact(crp):
    """Random stored tensors, including scale codes that saturate at 127."""
    N, K = 96, 512
    idx, s_rel, cb, _ = si.random_w4a8_format(N, K, seed=3)
    s_rel[0, :] = 0x78                                  # 256: every |cb| >= 0.5 saturates
    s_rel[1, :4] = np.array([0x00, 0x01, 0x7F, 0xFF], np.uint8)   # zero, subnormal, NaN codes
    p = _w4a8_dev(crp, idx, s_rel, cb, N, K)
    codes = crp.dbg_unpack_weight(2, p, N, K)
    _sync()
    assert np.array_equal(codes.cpu().numpy(), O.w4a8_decode(O.unpack_uint4(idx), s_rel, cb))


# ---------------------------------------------------------------------------
# Accumulators and outputs
# ---------------------------------------------------------------------------

def _run_w4a4(crp, L, acc=True):
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    bias = to_dev_bf16(L.bias) if L.bias is not None else None
    y = crp.linear_w4a4(x, p, s, L.N, bias)
    a = crp.dbg_linear_acc(0, x, p, L.N) if acc else None
    _sync()
    return y, a


SHAPES = [
    (64, 512, 256), (1, 256, 64), (33, 512, 100), (76, 2560, 512), (128, 1024, 256),
    (129, 512, 256), (300, 768, 384), (257, 256, 96), (96, 2048, 2560), (2, 9728, 64),
    # the four-rows-per-block activation quantiser (M >= 2048), with a partial quad
    (2049, 512, 64), (2048, 1024, 96), (2050, 2304, 64),
    # 256 x 192 block tiles, full ones included (odd M: with bias)
    (1025, 512, 768),
]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w4a4_acc_and_output(crp, M, K, N):
    L = si.random_layer(M, K, N, seed=M * 3 + K + N, bias=(M % 2 == 1), outlier_count=6)
    y, a = _run_w4a4(crp, L)
    r = O.linear_w4a4(L.x, L.w, L.bias)
    assert np.array_equal(a.cpu().numpy(), r["acc"])
    yd = bf16_dev_to_f32(y)
    assert max_rel_err(yd, r["y"]) <= TOL
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), O.f32_to_bf16_rne(r["y"]))


@pytest.mark.parametrize("M,K,N", [(64, 2688, 256), (7, 2688, 7), (130, 100, 40), (76, 3072, 384),
                                   (5, 7, 9), (200, 192, 64), (2048, 256, 1536)])
def test_int8tw_acc_and_output(crp, M, K, N):
    L = si.random_layer(M, K, N, seed=M + K * 3 + N, bias=True)
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_int8tw(to_dev_bf16(L.w))
    y = crp.linear_int8tw(x, p, s, N, to_dev_bf16(L.bias))
    a = crp.dbg_linear_acc(1, x, p, N)
    _sync()
    r = O.linear_int8tw(L.x, L.w, L.bias)
    assert np.array_equal(a.cpu().numpy(), r["acc"])
    assert max_rel_err(bf16_dev_to_f32(y), r["y"]) <= TOL


@pytest.mark.parametrize("M,K,N", [(64, 512, 256), (76, 768, 96), (200, 512, 160), (3, 256, 33),
                                   # M >= 2048: weight decoded to int8 per call, int8 GEMM
                                   (2050, 512, 160), (2048, 1024, 300)])
def test_w4a8_acc_and_output(crp, M, K, N):
    L = si.random_layer(M, K, N, seed=M + K + N * 11, bias=True)
    enc = O.w4a8_encode(L.w)
    x = to_dev_bf16(L.x)
    p = _w4a8_dev(crp, enc["idx_packed"], enc["s_rel"], enc["codebook"], N, K)
    sch = to_dev(enc["s_channel"])
    y = crp.linear_w4a8(x, p, sch, N, to_dev_bf16(L.bias))
    a = crp.dbg_linear_acc(2, x, p, N)
    _sync()
    r = O.linear_w4a8(L.x, enc["idx_packed"], enc["s_rel"], enc["codebook"], enc["s_channel"], L.bias)
    assert np.array_equal(a.cpu().numpy(), r["acc"])
    assert max_rel_err(bf16_dev_to_f32(y), r["y"]) <= TOL


# Shapes with few 256 x 256 output tiles and a long K: the large-M path splits
# K across blocks and adds the int32 partial tiles in a second kernel.
# Ragged M, N (N % 8 != 0, N % 4 != 0) and K (int8: K % 64 != 0) included.
SPLIT_CASES = [
    (0, 300, 4096, 512, False), (0, 520, 2560, 300, True),
    (1, 260, 2688, 200, True), (1, 300, 1000, 37, False),
    (2, 400, 1024, 264, True),
]


@pytest.mark.parametrize("kind,M,K,N,bias", SPLIT_CASES)
def test_split_k_acc_and_output(crp, kind, M, K, N, bias):
    tiles = -(-M // 256) * -(-N // 256)
    # the workspace holds at least two slices of int32 partial tiles
    assert crp.workspace_bytes(kind, M, N, K) >= 2 * tiles * 256 * 256 * 4
    L = si.random_layer(M, K, N, seed=M * 5 + K + N + kind, bias=bias, outlier_count=6)
    x = to_dev_bf16(L.x)
    b = to_dev_bf16(L.bias) if bias else None
    if kind == 0:
        p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
        y = crp.linear_w4a4(x, p, s, N, b)
        r = O.linear_w4a4(L.x, L.w, L.bias)
    elif kind == 1:
        p, s = crp.pack_weight_int8tw(to_dev_bf16(L.w))
        y = crp.linear_int8tw(x, p, s, N, b)
        r = O.linear_int8tw(L.x, L.w, L.bias)
    else:
        enc = O.w4a8_encode(L.w)
        p = _w4a8_dev(crp, enc["idx_packed"], enc["s_rel"], enc["codebook"], N, K)
        y = crp.linear_w4a8(x, p, to_dev(enc["s_channel"]), N, b)
        r = O.linear_w4a8(L.x, enc["idx_packed"], enc["s_rel"], enc["codebook"], enc["s_channel"], L.bias)
    a = crp.dbg_linear_acc(kind, x, p, N)
    _sync()
    assert np.array_equal(a.cpu().numpy(), r["acc"])
    assert max_rel_err(bf16_dev_to_f32(y), r["y"]) <= TOL
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), O.f32_to_bf16_rne(r["y"]))


@pytest.mark.parametrize("N,K", [(256, 512), (100, 2560), (33, 256)])
def test_pack_int8rot_bitexact(crp, N, K):
    """ConvRot INT8 row-scaled weight: codes and per-row scales bit-exact."""
    L = si.random_layer(1, K, N, seed=N + 3 * K, outlier_count=4)
    L.w[min(5, N - 1), :] = 0                               # a zero row: scale 0, codes 0
    p, s = crp.pack_weight_int8rot(to_dev_bf16(L.w))
    codes = crp.dbg_unpack_weight(3, p, N, K)
    _sync()
    q_ref, s_ref = O.quant_weight_int8rot(L.w)
    assert np.array_equal(codes.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy()[:N].view(np.uint32), s_ref.view(np.uint32))


# small M, K split across blocks at large M, full 256 x 192 tiles, ragged N
@pytest.mark.parametrize("M,K,N,bias", [(76, 2560, 512, False), (7, 256, 33, True), (300, 4096, 512, True),
                                        (1025, 512, 768, True), (260, 2560, 200, False)])
def test_int8rot_acc_and_output(crp, M, K, N, bias):
    L = si.random_layer(M, K, N, seed=M + K + N, bias=bias, outlier_count=6)
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_int8rot(to_dev_bf16(L.w))
    b = to_dev_bf16(L.bias) if bias else None
    y = crp.linear_int8rot(x, p, s, N, b)
    a = crp.dbg_linear_acc(3, x, p, N)
    _sync()
    r = O.linear_int8rot(L.x, L.w, L.bias)
    assert np.array_equal(a.cpu().numpy(), r["acc"])
    assert max_rel_err(bf16_dev_to_f32(y), r["y"]) <= TOL
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), O.f32_to_bf16_rne(r["y"]))


def test_tiny_config_end_to_end(crp):
    L = si.tiny()
    y, a = _run_w4a4(crp, L)
    r = O.linear_w4a4(L.x, L.w)
    assert np.array_equal(a.cpu().numpy(), r["acc"])
    assert max_rel_err(bf16_dev_to_f32(y), r["y"]) <= TOL


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------

def test_zero_rows_give_bias(crp):
    L = si.random_layer(40, 512, 64, seed=1, bias=True)
    L.x[[0, 17, 39], :] = 0
    y, a = _run_w4a4(crp, L)
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    for m in (0, 17, 39):
        assert np.array_equal(yb[m], L.bias)
        assert np.all(a.cpu().numpy()[m] == 0)


def test_m_zero_noop(crp):
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    p, s = crp.pack_weight_w4(to_dev_bf16(si.random_layer(1, 256, 32, seed=0).w))
    y = crp.linear_w4a4(x, p, s, 32)
    _sync()
    assert tuple(y.shape) == (0, 32)


def test_group_error_raises(crp):
    w = to_dev_bf16(si.random_layer(1, 2688, 64, seed=0).w)
    with pytest.raises(crp.ConvRotError) as e:
        crp.pack_weight_w4(w)
    assert e.value.status == 3
    pw = crp.pack_linear(w)        # routed to int8_tensorwise
    assert pw.kind == crp.INT8TW


def test_short_workspace_raises(crp):
    L = si.random_layer(8, 512, 64, seed=2)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(crp.ConvRotError) as e:
        crp.linear_w4a4(to_dev_bf16(L.x), p, s, 64, workspace=ws)
    assert e.value.status == 5


def test_repeat_runs_identical_and_workspace_reuse(crp):
    L = si.random_layer(76, 2560, 1024, seed=4)
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    ws = torch.empty(crp.workspace_bytes(0, 76, 1024, 2560), dtype=torch.uint8, device="cuda")
    ws.fill_(0xAB)
    y1 = crp.linear_w4a4(x, p, s, 1024, workspace=ws).clone()
    y2 = crp.linear_w4a4(x, p, s, 1024, workspace=ws).clone()
    _sync()
    assert torch.equal(y1, y2)


def test_no_dequantized_weight_buffer(crp):
    """The quantised path never materialises a dequantised weight: its
    workspace holds the activation codes and small partial sums only."""
    M, N, K = 76, 9728, 2560
    assert crp.workspace_bytes(0, M, N, K) < N * K   # far below a bf16 N*K copy


def test_two_phase_matches_linear_and_reuses_quantisation(crp):
    """One quantisation feeding GEMMs against two weights (different N, split
    K on the small-M path), each repeated: identical to the one-call linear."""
    M, K = 76, 2560
    A = si.random_layer(M, K, 640, seed=21, bias=True)
    B = si.random_layer(M, K, 1152, seed=22)
    x = to_dev_bf16(A.x)
    pa, sa = crp.pack_weight_w4(to_dev_bf16(A.w))
    pb, sb = crp.pack_weight_w4(to_dev_bf16(B.w))
    ba = to_dev_bf16(A.bias)
    ya = crp.linear_w4a4(x, pa, sa, 640, ba)
    yb = crp.linear_w4a4(x, pb, sb, 1152)
    ws = torch.empty(crp.workspace_bytes(0, M, 1152, K), dtype=torch.uint8, device="cuda")
    crp.quantize_activations(0, x, ws)
    outs = []
    for _ in range(2):
        outs.append(crp.gemm_quantized(0, M, K, pa, sa, 640, ws, bias=ba))
        outs.append(crp.gemm_quantized(0, M, K, pb, sb, 1152, ws))
    _sync()
    for i in (0, 2):
        assert torch.equal(outs[i], ya)
        assert torch.equal(outs[i + 1], yb)
    r = O.linear_w4a4(A.x, A.w, A.bias)
    assert max_rel_err(bf16_dev_to_f32(ya), r["y"]) <= TOL


def test_two_phase_large_m(crp):
    M, K, N = 300, 1024, 512
    L = si.random_layer(M, K, N, seed=23)
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_int8tw(to_dev_bf16(L.w))
    y = crp.linear_int8tw(x, p, s, N)
    ws = torch.empty(crp.workspace_bytes(1, M, N, K), dtype=torch.uint8, device="cuda")
    crp.quantize_activations(1, x, ws)
    y2 = crp.gemm_quantized(1, M, K, p, s, N, ws)
    _sync()
    assert torch.equal(y, y2)


def test_short_packed_weight_or_scale_raises(crp):
    """The binding refuses packed weights and scales smaller than the layout
    needs, before anything is launched."""
    M, K, N = 8, 512, 64
    L = si.random_layer(M, K, N, seed=12)
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    with pytest.raises(ValueError, match="packed weight"):
        crp.linear_w4a4(x, p[:-16], s, N)
    with pytest.raises(ValueError, match="packed weight"):
        crp.linear_w4a4(x, p, s, N + 32)
    pr, sr = crp.pack_weight_int8rot(to_dev_bf16(L.w))
    with pytest.raises(ValueError, match="scale"):
        crp.linear_int8rot(x, pr, sr[: N // 2], N)
    ws = torch.empty(crp.workspace_bytes(0, M, N, K), dtype=torch.uint8, device="cuda")
    crp.quantize_activations(0, x, ws)
    with pytest.raises(ValueError, match="packed weight"):
        crp.gemm_quantized(0, M, K, p[:100], s, N, ws)
    _sync()
