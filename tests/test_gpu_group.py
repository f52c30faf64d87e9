"""W4A4 with rotation groups of 64 and 16 ([ZIT] "Where Z-Image sits": the
ConvRot group-size sweep): the HIP path through the C ABI against the oracle
run with the same group.  Activation and weight codes, scales and int32
accumulators bit-exact; bf16 outputs equal to the oracle's bf16 rounding
(and within the 1e-2 relative bound).  The cases cover every activation
quantiser path (segmented rows, one row per block with one, two and four
256-blocks per lane, four rows per block), both GEMM paths, split K, bias,
ragged M and N."""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import convrot_oracle as O
from tests._util import TOL, bf16_dev_to_f32, max_rel_err, to_dev_bf16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

KIND = {64: 4, 16: 5}


@pytest.fixture(scope="module")
def crp():
    import rotated_bit_quantized_convrot_amd as m
    m.lib()
    return m


def _sync():
    torch.cuda.synchronize()


ACT_CASES = [(64, 512), (33, 768), (76, 2560), (5, 12288), (2, 65536), (1100, 8192), (2049, 512),
             (2050, 3840), (300, 3072)]


@pytest.mark.parametrize("G", [64, 16])
@pytest.mark.parametrize("M,K", ACT_CASES)
def test_group_quant_act_bitexact(crp, G, M, K):
    L = si.random_layer(M, K, 1, seed=200 + M + K + G, outlier_count=min(8, K), outlier_scale=40.0)
    x = L.x.copy()
    x[1, :] = 0
    if M >= 3:
        x[2, :] = si.f32_to_bf16_bits(np.full(K, 0.75, np.float32))
    q, s = crp.dbg_quant_act(KIND[G], to_dev_bf16(x))
    _sync()
    q_ref, s_ref = O.quant_act_w4a4(x, G)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def _rows_from_rotated(y_rows, G):
    """bf16 rows x with rotate_G(x) == y exactly (x = H_G y per group; the
    normalised Sylvester Hadamard is symmetric and its own inverse)."""
    H = O.hadamard(G)
    y = np.asarray(y_rows, np.float64)
    R, K = y.shape
    x = (y.reshape(R, K // G, G) @ H.T).reshape(R, K)
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x)
    bits = si.f32_to_bf16_bits(x32)
    assert np.array_equal(si.bf16_bits_to_f32(bits).astype(np.float64), x)
    return bits


@pytest.mark.parametrize("G", [64, 16])
def test_group_quant_act_exact_ties(crp, G):
    """Rotated values exactly on half-integer multiples of the scale next to
    the row maximum, one per group: round half to even decides."""
    K = 256 * 4
    rows = []
    for e in (-3, 0, 5):
        y = np.zeros(K)
        y[0] = 7 * 2.0 ** e                               # the row maximum: scale 2^e
        for g in range(K // G):
            y[g * G + 1 + g % (G - 1)] = (-1) ** g * ((g % 7) + 0.5) * 2.0 ** e
        rows.append(y)
    x = _rows_from_rotated(rows, G)
    q, s = crp.dbg_quant_act(KIND[G], to_dev_bf16(x))
    _sync()
    q_ref, s_ref = O.quant_act_w4a4(x, G)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("G", [64, 16])
def test_group_quant_act_extreme_magnitudes(crp, G):
    rng = np.random.default_rng(9 + G)
    K = 512
    base = rng.standard_normal((6, K)).astype(np.float32)
    scales = [1.0, 1e-33, 1e33, 1e-39, 3e-38, 1.0]
    x = si.f32_to_bf16_bits(base * np.array(scales, np.float32)[:, None])
    q, s = crp.dbg_quant_act(KIND[G], to_dev_bf16(x))
    _sync()
    q_ref, s_ref = O.quant_act_w4a4(x, G)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("G", [64, 16])
@pytest.mark.parametrize("N,K", [(256, 512), (33, 256), (64, 2560), (40, 8192)])
def test_group_pack_w4_bitexact(crp, G, N, K):
    L = si.random_layer(1, K, N, seed=N * 11 + K + G, outlier_count=4)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w), group=G)
    codes = crp.dbg_unpack_weight(KIND[G], p, N, K)
    _sync()
    q_ref, s_ref = O.quant_weight_w4(L.w, G)
    assert np.array_equal(codes.cpu().numpy(), q_ref)
    assert s.cpu().numpy()[:1].view(np.uint32)[0] == np.float32(s_ref).view(np.uint32)


SHAPES = [(64, 512, 256), (1, 256, 64), (76, 2560, 512), (33, 512, 100), (300, 4096, 512),
          (2049, 512, 64), (1025, 512, 768), (2050, 2304, 96)]


@pytest.mark.parametrize("G", [64, 16])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_group_acc_and_output(crp, G, M, K, N):
    L = si.random_layer(M, K, N, seed=M + 5 * K + N + G, bias=(M % 2 == 1), outlier_count=6)
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w), group=G)
    bias = to_dev_bf16(L.bias) if L.bias is not None else None
    y = crp.linear_w4a4(x, p, s, N, bias, group=G)
    a = crp.dbg_linear_acc(KIND[G], x, p, N)
    _sync()
    r = O.linear_w4a4(L.x, L.w, L.bias, G)
    assert np.array_equal(a.cpu().numpy(), r["acc"])
    assert max_rel_err(bf16_dev_to_f32(y), r["y"]) <= TOL
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), O.f32_to_bf16_rne(r["y"]))


@pytest.mark.parametrize("G", [64, 16])
def test_group_two_phase_and_pack_linear(crp, G):
    """The generic two-phase calls with the group kinds, and the layer-level
    pack_linear / linear, equal the one-call group linear."""
    M, K, N = 76, 2560, 640
    L = si.random_layer(M, K, N, seed=31 + G, bias=True)
    x = to_dev_bf16(L.x)
    b = to_dev_bf16(L.bias)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w), group=G)
    y = crp.linear_w4a4(x, p, s, N, b, group=G)
    ws = torch.empty(crp.workspace_bytes(KIND[G], M, N, K), dtype=torch.uint8, device="cuda")
    crp.quantize_activations(KIND[G], x, ws)
    y2 = crp.gemm_quantized(KIND[G], M, K, p, s, N, ws, bias=b)
    pw = crp.pack_linear(to_dev_bf16(L.w), b, group=G)
    y3 = crp.linear(x, pw)
    _sync()
    assert pw.kind == KIND[G]
    assert torch.equal(y2, y) and torch.equal(y3, y)


def test_group_sizes_differ_and_bad_group_raises(crp):
    """The three groups give different codes on the same input (the group
    reaches the kernels), and a group outside {256, 64, 16} is refused."""
    L = si.random_layer(8, 512, 32, seed=3)
    x = to_dev_bf16(L.x)
    q256, _ = crp.dbg_quant_act(0, x)
    q64, _ = crp.dbg_quant_act(4, x)
    q16, _ = crp.dbg_quant_act(5, x)
    _sync()
    assert not torch.equal(q256, q64) and not torch.equal(q64, q16)
    with pytest.raises(crp.ConvRotError, match="CR_ERR_GROUP"):
        crp.pack_weight_w4(to_dev_bf16(L.w), group=32)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w), group=64)
    with pytest.raises(crp.ConvRotError, match="CR_ERR_GROUP"):
        crp.linear_w4a4(x, p, s, 32, group=128)


def _subnormal_rows(K, seed):
    """Rows of the smallest bf16 subnormals (one +-2^-133, all-subnormal
    random rows, a sparse mix), where the scales are fp32 subnormals too."""
    rng = np.random.default_rng(seed)
    rows = []
    for sign in (0x0000, 0x8000):
        r = np.zeros(K, np.uint16)
        r[3] = sign | 0x0001
        rows.append(r)
    rows.append((rng.integers(1, 128, K) | (rng.integers(0, 2, K) << 15)).astype(np.uint16))
    r = np.zeros(K, np.uint16)
    r[::7] = 0x8001
    r[5] = 0x007F
    rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("kind", [0, 4, 5, 6])
@pytest.mark.parametrize("M,K", [(4, 512), (36, 3072), (2052, 512)])
def test_subnormal_rows_quant_act_bitexact(crp, kind, M, K):
    """Activation codes and scales of subnormal-only rows, every rotation,
    across the quantiser's row layouts; the codes stay in [-7, 7]."""
    base = _subnormal_rows(K, seed=M + K + kind)
    x = np.tile(base, ((M + 3) // 4, 1))[:M]
    q, s = crp.dbg_quant_act(kind, to_dev_bf16(x))
    _sync()
    q_ref, s_ref = O.quant_act_w4a4_regular(x) if kind == 6 else O.quant_act_w4a4(x, {0: 256, 4: 64, 5: 16}[kind])
    qn = q.cpu().numpy()
    assert np.array_equal(qn, q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert qn.min() >= -7 and qn.max() <= 7


@pytest.mark.parametrize("G", [256, 64, 16])
def test_subnormal_weight_pack_bitexact(crp, G):
    """A weight of subnormal bf16 values only: tensor scale and codes."""
    w = np.tile(_subnormal_rows(512, seed=G), (9, 1))[:33]
    p, s = crp.pack_weight_w4(to_dev_bf16(w), group=G)
    codes = crp.dbg_unpack_weight({256: 0, 64: 4, 16: 5}[G], p, 33, 512)
    _sync()
    q_ref, s_ref = O.quant_weight_w4(w, G)
    assert np.array_equal(codes.cpu().numpy(), q_ref)
    assert s.cpu().numpy()[:1].view(np.uint32)[0] == np.float32(s_ref).view(np.uint32)
