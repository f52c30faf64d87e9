"""Text-encoder MLP block (gate/up -> silu(g) * u -> rotate + quantise ->
down; the oracle's reading R20) through the C ABI against the oracle.  The
fused kernel's codes and scales are compared bit-exactly with the oracle's
quantisation of silu_mul_bf16(g, u) (h is computed in float64 on both sides
and rounded to float32, then bf16: the two float64 exp implementations can
only disagree on h within ~1e-16 of a rounding boundary); the block's bf16
output equals the oracle's bf16 rounding."""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import convrot_oracle as O
from tests._util import TOL, bf16_dev_to_f32, max_rel_err, to_dev_bf16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def crp():
    import rotated_bit_quantized_convrot_amd as m
    m.lib()
    return m


def _sync():
    torch.cuda.synchronize()


def _gu(M, F, seed):
    rng = np.random.default_rng(seed)
    g = (rng.standard_t(3, size=(M, F)) * 2.0).astype(np.float32)
    u = rng.standard_normal((M, F)).astype(np.float32)
    g[0, :8] = [0.0, -0.0, 60.0, -60.0, -800.0, 1e-30, -3.5, 2.0]        # saturating and tiny values
    return si.f32_to_bf16_bits(g), si.f32_to_bf16_bits(u)


@pytest.mark.parametrize("M,F", [(76, 9728), (3, 256), (33, 768), (1220, 2560), (2049, 512), (5, 12288)])
def test_swiglu_quant_bitexact(crp, M, F):
    g, u = _gu(M, F, seed=M + F)
    q, s = crp.dbg_quant_swiglu(to_dev_bf16(g), to_dev_bf16(u))
    _sync()
    h = O.silu_mul_bf16(g, u)
    q_ref, s_ref = O.quant_act_w4a4(h)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def _weights(K, F, N, seed):
    rng = np.random.default_rng(seed)
    wg = si.f32_to_bf16_bits((rng.standard_normal((F, K)) * 0.02).astype(np.float32))
    wu = si.f32_to_bf16_bits((rng.standard_normal((F, K)) * 0.02).astype(np.float32))
    wd = si.f32_to_bf16_bits((rng.standard_normal((N, F)) * 0.02).astype(np.float32))
    return wg, wu, wd


@pytest.mark.parametrize("M,K,F,N", [(76, 2560, 9728, 2560), (7, 512, 768, 300), (300, 1024, 1536, 512),
                                     (1025, 512, 1024, 768)])
def test_mlp_block_output(crp, M, K, F, N):
    L = si.random_layer(M, K, 1, seed=M + K + F, outlier_count=min(13, K))
    wg, wu, wd = _weights(K, F, N, seed=F + N)
    x = to_dev_bf16(L.x)
    pg, sg = crp.pack_weight_w4(to_dev_bf16(wg))
    pu, su = crp.pack_weight_w4(to_dev_bf16(wu))
    pd, sd = crp.pack_weight_w4(to_dev_bf16(wd))
    y = crp.mlp_w4a4(x, pg, sg, pu, su, F, pd, sd, N)
    # the same block from the separate linears (bit-identical by construction)
    g = crp.linear_w4a4(x, pg, sg, F)
    u = crp.linear_w4a4(x, pu, su, F)
    _sync()
    r = O.mlp_w4a4(L.x, wg, wu, wd)
    assert np.array_equal(g.view(torch.int16).cpu().numpy().view(np.uint16), r["g"])
    assert np.array_equal(u.view(torch.int16).cpu().numpy().view(np.uint16), r["u"])
    assert max_rel_err(bf16_dev_to_f32(y), r["y"]) <= TOL
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), O.f32_to_bf16_rne(r["y"]))


def test_mlp_block_repeat_and_m_zero(crp):
    M, K, F, N = 76, 512, 768, 256
    L = si.random_layer(M, K, 1, seed=5)
    wg, wu, wd = _weights(K, F, N, seed=6)
    x = to_dev_bf16(L.x)
    pg, sg = crp.pack_weight_w4(to_dev_bf16(wg))
    pu, su = crp.pack_weight_w4(to_dev_bf16(wu))
    pd, sd = crp.pack_weight_w4(to_dev_bf16(wd))
    ws = torch.empty(crp.mlp_workspace_bytes(M, K, F, N), dtype=torch.uint8, device="cuda")
    y1 = crp.mlp_w4a4(x, pg, sg, pu, su, F, pd, sd, N, workspace=ws).clone()
    y2 = crp.mlp_w4a4(x, pg, sg, pu, su, F, pd, sd, N, workspace=ws)
    y0 = crp.mlp_w4a4(x[:0], pg, sg, pu, su, F, pd, sd, N)
    _sync()
    assert torch.equal(y1, y2) and y0.shape == (0, N)


def test_silu_mul_bits_including_fallback_cases(crp):
    """h = silu(g) * u bit-exact against the oracle, on random values and on
    the hard ones: values whose float64 result lies near a bf16 rounding
    midpoint (picked from 4e6 random pairs by the oracle's own value), |g|
    beyond the float32 range of exp(-g), and tiny results."""
    rng = np.random.default_rng(23)
    g = si.f32_to_bf16_bits((rng.standard_t(3, size=4_000_000) * 3).astype(np.float32))
    u = si.f32_to_bf16_bits(rng.standard_normal(4_000_000).astype(np.float32))
    g64 = O.bf16_to_f32(g).astype(np.float64)
    u64 = O.bf16_to_f32(u).astype(np.float64)
    with np.errstate(over="ignore"):
        h32 = (g64 / (1.0 + np.exp(-g64)) * u64).astype(np.float32)
    lo = h32.view(np.uint32) & 0xFFFF
    # within 2048 float32 ulps of a bf16 rounding midpoint
    near = np.nonzero(np.abs(lo.astype(np.int64) - 0x8000) <= 2048)[0][:100_000]
    big = si.f32_to_bf16_bits(np.array([65.0, -65.0, 88.0, -88.5, -90.0, -100.0, -103.0, -150.0, 300.0, -800.0],
                                       np.float32))
    tiny_u = si.f32_to_bf16_bits(np.array([1e-30, -3e-38, 1e-39, 2.0, 0.5, -1.0, 1e-38, 7.0, 1.0, 1.0], np.float32))
    gs = np.concatenate([g[:200_000], g[near], big, big])
    us = np.concatenate([u[:200_000], u[near], tiny_u, u[:10]])
    assert len(near) > 1000
    h = crp.dbg_silu_mul(to_dev_bf16(gs), to_dev_bf16(us))
    _sync()
    got = h.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, O.silu_mul_bf16(gs, us))
