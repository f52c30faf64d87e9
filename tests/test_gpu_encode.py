"""On-GPU W4A8 encoder (cr_encode_w4a8; [REB] "Rebels_w4a8s", "What's inside
a file") against the oracle's encode (reading R10): every output compared -
index bytes, E4M3 scale bytes, the float32 codebook and the per-channel
scales bit for bit - on small ragged shapes with edge rows, several
iteration budgets, and the full W4A8 benchmark layer."""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import convrot_oracle as O
from tests._util import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def crp():
    import rotated_bit_quantized_convrot_amd as m
    m.lib()
    return m


def test_e4m3_encode_matches_oracle(crp):
    """Nearest E4M3 with ties to the even code: every code value, every
    midpoint between neighbours (exact ties), one float32 ulp either side,
    random values over the range the encoder uses and the subnormal range."""
    vals = O.e4m3_to_f32(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    m32 = mids.astype(np.float32)
    rng = np.random.default_rng(5)
    v = np.concatenate([vals.astype(np.float32), m32, np.nextafter(m32, np.float32(0)),
                        np.nextafter(m32, np.float32(np.inf)),
                        rng.uniform(0, 127, 50000).astype(np.float32),
                        rng.uniform(0, 2.0 ** -6, 20000).astype(np.float32),
                        np.array([0.0, 127.0, 448.0, 2.0 ** -10, 2.0 ** -9 * 0.5], np.float32)])
    got = crp.dbg_e4m3_encode(to_dev(v)).cpu().numpy()
    assert np.array_equal(got, O.f32_to_e4m3_rne(v))


def _compare(crp, wb, iters):
    N, K = wb.shape
    idx, s_rel, cb, sch = crp.encode_w4a8(to_dev_bf16(wb), iters=iters)
    torch.cuda.synchronize()
    ref = O.w4a8_encode(wb, iters=iters)
    assert np.array_equal(sch.cpu().numpy().view(np.uint32), ref["s_channel"].view(np.uint32))
    assert np.array_equal(s_rel.cpu().numpy(), ref["s_rel"])
    assert np.array_equal(cb.cpu().numpy(), ref["codebook"])          # values (a zero's sign may differ)
    got_idx = idx.cpu().numpy()
    bad = np.count_nonzero(got_idx != ref["idx_packed"])
    assert bad == 0, f"{bad} index bytes differ"
    return ref


def _edge_weight(N, K, seed):
    rng = np.random.default_rng(seed)
    w = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    w[1] = 0.0                                            # zero row: s_channel 0, u = 0
    w[2, :16] *= 1e-4                                     # tiny group: subnormal or zero scale code
    w[2, 16:32] *= 3e-3
    w[3, 5] = 4.0                                         # one large value in the row
    w[4] = np.linspace(-1, 1, K)                          # a smooth row
    return si.f32_to_bf16_bits(w)


@pytest.mark.parametrize("N,K,iters", [(64, 256, 100), (37, 512, 1), (37, 512, 3), (100, 1024, 100),
                                       (9, 2560, 7)])
def test_encode_small_shapes(crp, N, K, iters):
    print(f"[encode] N={N} K={K} iters={iters}", flush=True)
    _compare(crp, _edge_weight(N, K, seed=N + K), iters)


def test_encode_full_w4a8_layer(crp):
    """The W4A8 benchmark layer (10240 x 3840, N(0, 0.02)): 39.3 M weights,
    100 Lloyd iterations, every output equal to the oracle's; the encoded
    weight then decodes to the oracle's int8 weights."""
    print("[encode] W4A8 layer 10240 x 3840", flush=True)
    L = si.w4a8_layer()
    ref = _compare(crp, L.w, 100)
    w8 = O.w4a8_decode(ref["idx"], ref["s_rel"], ref["codebook"])
    rec = w8.astype(np.float64) * ref["s_channel"][:, None]
    wr = ref["w_rot"].astype(np.float64)
    assert 0.05 < np.linalg.norm(rec - wr) / np.linalg.norm(wr) < 0.1


def test_encode_rejects_bad_shapes(crp):
    w = to_dev_bf16(si.f32_to_bf16_bits(np.zeros((4, 300), np.float32)))
    with pytest.raises(crp.ConvRotError):
        crp.encode_w4a8(w)
