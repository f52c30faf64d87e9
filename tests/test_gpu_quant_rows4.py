"""W4A4 activation quantisation of many rows (M >= 2048, K <= 8192: four rows
per block, every block resident at once): the linear's int32 accumulators
and bf16 outputs equal the oracle's bit for bit (so do the codes, scales and
correction sums they are made from), for one and two 256-groups per lane,
1 to 32 groups per row, ragged M (a partial last block of rows), zero,
constant and negative constant rows, and the group-64 / group-16 /
regular-Hadamard rotations."""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import convrot_oracle as O
from tests._util import to_dev_bf16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def crp():
    import rotated_bit_quantized_convrot_amd as m
    m.lib()
    return m


def _bits(y):
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("M,K", [(2048, 256), (2051, 1024), (2300, 1792), (4097, 2048), (4096, 3072),
                                 (2049, 4096), (2050, 6144), (3001, 8192)])
def test_rows4_quantiser_linear_bitexact(crp, M, K):
    print(f"[quant-rows4] M={M} K={K}", flush=True)
    N = 96
    L = si.random_layer(M, K, N, seed=M + K, bias=True, outlier_count=min(8, K // 64), outlier_scale=40.0)
    x = L.x.copy()
    x[1, :] = 0                                                   # zero row
    x[2, :] = si.f32_to_bf16_bits(np.full(K, 0.75, np.float32))   # constant row
    x[M - 1, :] = si.f32_to_bf16_bits(np.full(K, -3.0, np.float32))
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    xd = to_dev_bf16(x)
    y = crp.linear_w4a4(xd, p, s, N, to_dev_bf16(L.bias))
    acc = crp.dbg_linear_acc(0, xd, p, N)
    torch.cuda.synchronize()
    ref = O.linear_w4a4(x, L.w, L.bias)
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    assert np.array_equal(_bits(y), O.f32_to_bf16_rne(ref["y"]))


@pytest.mark.parametrize("variant", ["group64", "group16", "regular"])
def test_rows4_quantiser_rotation_variants(crp, variant):
    M, K, N = 2053, 3072, 64
    print(f"[quant-rows4] {variant} M={M} K={K}", flush=True)
    L = si.random_layer(M, K, N, seed=17, bias=False, outlier_count=8, outlier_scale=40.0)
    xd, wd = to_dev_bf16(L.x), to_dev_bf16(L.w)
    if variant == "regular":
        p, s = crp.pack_weight_w4_regular(wd)
        y = crp.linear_w4a4_regular(xd, p, s, N)
        ref = O.linear_w4a4_regular(L.x, L.w, None)
    else:
        g = 64 if variant == "group64" else 16
        p, s = crp.pack_weight_w4(wd, group=g)
        y = crp.linear_w4a4(xd, p, s, N, group=g)
        ref = O.linear_w4a4(L.x, L.w, None, group=g)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), O.f32_to_bf16_rne(ref["y"]))
