"""W4A4 with the group-256 regular Hadamard rotation ([QIE] intro:
"regular-Hadamard"; the construction (J - 2I)^(x4) / 16 is the oracle's
reading R19): the HIP path through the C ABI against the oracle.  Codes,
scales and int32 accumulators bit-exact; bf16 outputs equal to the oracle's
bf16 rounding.  Cases cover every activation quantiser path and both GEMM
paths, with ragged M and N, bias and split K."""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import convrot_oracle as O
from tests._util import TOL, bf16_dev_to_f32, max_rel_err, to_dev_bf16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

RH = 6


@pytest.fixture(scope="module")
def crp():
    import rotated_bit_quantized_convrot_amd as m
    m.lib()
    return m


def _sync():
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,K", [(64, 512), (33, 768), (76, 2560), (5, 12288), (2, 65536), (1100, 8192),
                                 (2049, 512), (2050, 3840), (300, 3072)])
def test_regular_quant_act_bitexact(crp, M, K):
    L = si.random_layer(M, K, 1, seed=300 + M + K, outlier_count=min(8, K), outlier_scale=40.0)
    x = L.x.copy()
    x[1, :] = 0
    if M >= 3:
        x[2, :] = si.f32_to_bf16_bits(np.full(K, -1.25, np.float32))     # constant row: codes -7
    q, s = crp.dbg_quant_act(RH, to_dev_bf16(x))
    _sync()
    q_ref, s_ref = O.quant_act_w4a4_regular(x)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_regular_quant_act_exact_ties(crp):
    """Rows x = H y (H symmetric, its own inverse) with y on half-integer
    multiples of the scale next to the row maximum: round half to even
    decides.  y has three non-zeros per 256-block, so every value of x and of
    the stages is exact."""
    H = O.regular_hadamard()
    K = 1024
    rows = []
    for e in (-2, 0, 4):
        y = np.zeros(K)
        y[0] = 7 * 2.0 ** e
        for g in range(K // 256):
            y[g * 256 + 3 + 17 * g] = (-1) ** g * ((g % 7) + 0.5) * 2.0 ** e
            y[g * 256 + 200] = 2.0 ** e
        rows.append(y)
    y = np.array(rows)
    x = (y.reshape(3, 4, 256) @ H.T).reshape(3, K)
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x)
    bits = si.f32_to_bf16_bits(x32)
    assert np.array_equal(si.bf16_bits_to_f32(bits).astype(np.float64), x)
    assert np.array_equal(O.rht(si.bf16_bits_to_f32(bits)).astype(np.float64), y)
    q, s = crp.dbg_quant_act(RH, to_dev_bf16(bits))
    _sync()
    q_ref, s_ref = O.quant_act_w4a4_regular(bits)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_regular_quant_act_extreme_magnitudes(crp):
    rng = np.random.default_rng(61)
    K = 512
    base = rng.standard_normal((6, K)).astype(np.float32)
    scales = [1.0, 1e-33, 1e33, 1e-39, 3e-38, 1.0]
    x = si.f32_to_bf16_bits(base * np.array(scales, np.float32)[:, None])
    q, s = crp.dbg_quant_act(RH, to_dev_bf16(x))
    _sync()
    q_ref, s_ref = O.quant_act_w4a4_regular(x)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("N,K", [(256, 512), (33, 256), (64, 2560), (40, 8192)])
def test_regular_pack_w4_bitexact(crp, N, K):
    L = si.random_layer(1, K, N, seed=N * 13 + K, outlier_count=4)
    p, s = crp.pack_weight_w4_regular(to_dev_bf16(L.w))
    codes = crp.dbg_unpack_weight(RH, p, N, K)
    _sync()
    q_ref, s_ref = O.quant_weight_w4_regular(L.w)
    assert np.array_equal(codes.cpu().numpy(), q_ref)
    assert s.cpu().numpy()[:1].view(np.uint32)[0] == np.float32(s_ref).view(np.uint32)


@pytest.mark.parametrize("M,K,N", [(64, 512, 256), (1, 256, 64), (76, 2560, 512), (33, 512, 100),
                                   (300, 4096, 512), (2049, 512, 64), (1025, 512, 768), (7, 9728, 40)])
def test_regular_acc_and_output(crp, M, K, N):
    L = si.random_layer(M, K, N, seed=M + 7 * K + N, bias=(M % 2 == 1), outlier_count=6)
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_w4_regular(to_dev_bf16(L.w))
    bias = to_dev_bf16(L.bias) if L.bias is not None else None
    y = crp.linear_w4a4_regular(x, p, s, N, bias)
    a = crp.dbg_linear_acc(RH, x, p, N)
    _sync()
    r = O.linear_w4a4_regular(L.x, L.w, L.bias)
    assert np.array_equal(a.cpu().numpy(), r["acc"])
    assert max_rel_err(bf16_dev_to_f32(y), r["y"]) <= TOL
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), O.f32_to_bf16_rne(r["y"]))


def test_regular_two_phase_pack_linear_and_differs_from_sylvester(crp):
    M, K, N = 76, 2560, 640
    L = si.random_layer(M, K, N, seed=41, bias=True)
    x = to_dev_bf16(L.x)
    b = to_dev_bf16(L.bias)
    p, s = crp.pack_weight_w4_regular(to_dev_bf16(L.w))
    y = crp.linear_w4a4_regular(x, p, s, N, b)
    ws = torch.empty(crp.workspace_bytes(RH, M, N, K), dtype=torch.uint8, device="cuda")
    crp.quantize_activations(RH, x, ws)
    y2 = crp.gemm_quantized(RH, M, K, p, s, N, ws, bias=b)
    pw = crp.pack_linear(to_dev_bf16(L.w), b, regular=True)
    y3 = crp.linear(x, pw)
    q_rh, _ = crp.dbg_quant_act(RH, x)
    q_sy, _ = crp.dbg_quant_act(0, x)
    _sync()
    assert pw.kind == RH
    assert torch.equal(y2, y) and torch.equal(y3, y)
    assert not torch.equal(q_rh, q_sy)
