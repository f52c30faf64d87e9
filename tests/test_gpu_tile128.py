"""Large-M GEMM on 256 x 128 block tiles (taken for layers with few output
tiles), with and without K split across blocks: bf16 outputs and int32
accumulators against the oracle, bit for bit, for W4A4, int8_tensorwise and
ConvRot INT8.  (M, K, N) chosen so the planner picks that tile: 1000 x 1024 x
2560 whole tiles, 600 x 4096 x 1280 with K slices, 1220 x 2560 x 2560 the
ConvRot INT8 attention projection's shape."""
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


@pytest.mark.parametrize("kind", [0, 1, 3])
@pytest.mark.parametrize("M,K,N", [(1000, 1024, 2560), (600, 4096, 1280), (1220, 2560, 2560)])
def test_tile128_output_and_acc(crp, kind, M, K, N):
    print(f"[tile128] kind={kind} M={M} K={K} N={N}", flush=True)
    L = si.random_layer(M, K, N, seed=M + K + kind, bias=True, outlier_count=7)
    w = to_dev_bf16(L.w)
    x = to_dev_bf16(L.x)
    b = to_dev_bf16(L.bias)
    if kind == 0:
        p, s = crp.pack_weight_w4(w)
        y = crp.linear_w4a4(x, p, s, N, b)
        ref = O.linear_w4a4(L.x, L.w, L.bias)
    elif kind == 1:
        p, s = crp.pack_weight_int8tw(w)
        y = crp.linear_int8tw(x, p, s, N, b)
        ref = O.linear_int8tw(L.x, L.w, L.bias)
    else:
        p, s = crp.pack_weight_int8rot(w)
        y = crp.linear_int8rot(x, p, s, N, b)
        ref = O.linear_int8rot(L.x, L.w, L.bias)
    acc = crp.dbg_linear_acc(kind, x, p, N)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), O.f32_to_bf16_rne(ref["y"]))
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
