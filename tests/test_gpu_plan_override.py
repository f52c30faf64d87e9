"""Large-M GEMMs on plans the planner would not take, forced with
cr_dbg_big_plan: other block tile widths (256, 192, 128, 64) and K splits (2..8
slices, added by the second kernel), on ragged shapes, for W4A4,
int8_tensorwise, ConvRot INT8 and W4A8.  The int32 sums are exact, so the
outputs and accumulators must equal the oracle's bit for bit whatever the
plan."""
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
    yield m
    m.dbg_big_plan(0, 0)


def _bits(y):
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


# (kind, M, K, N, bn, splits)
CASES = [
    (0, 300, 4096, 512, 128, 2), (0, 520, 2560, 300, 192, 4), (0, 1220, 2560, 2560, 256, 2),
    (0, 257, 9728, 1024, 128, 8), (1, 260, 2688, 200, 128, 3), (1, 300, 1000, 37, 192, 2),
    (3, 1220, 2560, 2560, 128, 4), (3, 700, 1536, 900, 256, 3), (2, 400, 1024, 264, 256, 2),
    # 256 x 64 tiles: whole tiles and K slices, ragged M and N (N % 8 != 0)
    (3, 1220, 2560, 2560, 64, 1), (0, 1220, 9728, 2560, 64, 1), (1, 300, 1000, 37, 64, 2),
    (0, 520, 2560, 300, 64, 1), (1, 4096, 3072, 3072, 64, 1), (0, 257, 9728, 1024, 64, 4),
]


@pytest.mark.parametrize("kind,M,K,N,bn,splits", CASES)
def test_forced_plan_output_and_acc(crp, kind, M, K, N, bn, splits):
    print(f"[plan] kind={kind} M={M} K={K} N={N} bn={bn} splits={splits}", flush=True)
    L = si.random_layer(M, K, N, seed=M + K + N + 7 * kind + splits, bias=True, outlier_count=5)
    x, b = to_dev_bf16(L.x), to_dev_bf16(L.bias)
    if kind == 2:
        enc = O.w4a8_encode(L.w)
        p = crp.pack_weight_w4a8(to_dev(enc["idx_packed"]), to_dev(enc["s_rel"]), to_dev(enc["codebook"]), N, K)
        s = to_dev(enc["s_channel"])
        ref = O.linear_w4a8(L.x, enc["idx_packed"], enc["s_rel"], enc["codebook"], enc["s_channel"], L.bias)
    else:
        w = to_dev_bf16(L.w)
        p, s = {0: crp.pack_weight_w4, 1: crp.pack_weight_int8tw, 3: crp.pack_weight_int8rot}[kind](w)
        ref = {0: O.linear_w4a4, 1: O.linear_int8tw, 3: O.linear_int8rot}[kind](L.x, L.w, L.bias)
    fn = {0: crp.linear_w4a4, 1: crp.linear_int8tw, 2: crp.linear_w4a8, 3: crp.linear_int8rot}[kind]
    crp.dbg_big_plan(bn, splits)
    try:
        ws = torch.empty(crp.workspace_bytes(kind, M, N, K), dtype=torch.uint8, device="cuda")
        ws.fill_(0xA5)
        y = fn(x, p, s, N, b, workspace=ws)
        acc = crp.dbg_linear_acc(kind, x, p, N, workspace=ws)
        torch.cuda.synchronize()
    finally:
        crp.dbg_big_plan(0, 0)
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    assert np.array_equal(_bits(y), O.f32_to_bf16_rne(ref["y"]))
