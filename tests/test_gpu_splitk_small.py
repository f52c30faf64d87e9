"""Small-M GEMMs whose K is split across blocks and finished inside the
kernel by the last block of each weight block to arrive (arrival counters in
the workspace, zeroed by the activation quantiser, left zero by the GEMM).
Several calls in a row on one workspace that starts as garbage, each with
new activations: a stale partial tile or counter from an earlier call would
change the result, which must stay the oracle's bit for bit."""
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


# (kind, M, K, N, bias): few weight blocks and a long K, so the plan splits K
CASES = [(0, 76, 9728, 640, True), (0, 33, 9728, 2560, False), (3, 76, 2560, 512, False),
         (3, 76, 2560, 2560, True), (1, 50, 4096, 300, True), (2, 40, 3840, 256, True)]


def _weights(crp, kind, L):
    w = to_dev_bf16(L.w)
    if kind == 0:
        return crp.pack_weight_w4(w), lambda xb: O.linear_w4a4(xb, L.w, L.bias)
    if kind == 1:
        return crp.pack_weight_int8tw(w), lambda xb: O.linear_int8tw(xb, L.w, L.bias)
    if kind == 3:
        return crp.pack_weight_int8rot(w), lambda xb: O.linear_int8rot(xb, L.w, L.bias)
    enc = O.w4a8_encode(L.w)
    p = crp.pack_weight_w4a8(to_dev(enc["idx_packed"]), to_dev(enc["s_rel"]), to_dev(enc["codebook"]), L.N, L.K)
    ref = lambda xb: O.linear_w4a8(xb, enc["idx_packed"], enc["s_rel"], enc["codebook"], enc["s_channel"], L.bias)  # noqa: E731
    return (p, to_dev(enc["s_channel"])), ref


@pytest.mark.parametrize("kind,M,K,N,bias", CASES)
def test_small_m_split_k_calls_in_a_row(crp, kind, M, K, N, bias):
    print(f"[splitk-small] kind={kind} M={M} K={K} N={N}", flush=True)
    L = si.random_layer(M, K, N, seed=M + K + N + kind, bias=bias, outlier_count=5)
    (p, s), ref = _weights(crp, kind, L)
    b = to_dev_bf16(L.bias) if bias else None
    fn = {0: crp.linear_w4a4, 1: crp.linear_int8tw, 2: crp.linear_w4a8, 3: crp.linear_int8rot}[kind]
    ws = torch.empty(crp.workspace_bytes(kind, M, N, K), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)                                        # garbage counters and partials
    xs = [si.random_layer(M, K, 1, seed=100 * r + kind, outlier_count=5).x for r in range(3)]
    ys = [fn(to_dev_bf16(xb), p, s, N, b, workspace=ws).clone() for xb in xs]
    acc = crp.dbg_linear_acc(kind, to_dev_bf16(xs[-1]), p, N, workspace=ws)
    torch.cuda.synchronize()
    for xb, y in zip(xs, ys):
        r = ref(xb)
        assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), O.f32_to_bf16_rne(r["y"]))
    assert np.array_equal(acc.cpu().numpy(), ref(xs[-1])["acc"])


# forced split counts (cr_dbg_small_plan), including ones the planner would
# not take: 2 to 16 slices
FORCED = [(0, 76, 9728, 2560, True, 3), (0, 76, 9728, 2560, False, 8), (3, 76, 2560, 2560, True, 2),
          (3, 76, 2560, 2560, False, 5), (0, 76, 2560, 9728, True, 2), (1, 50, 4096, 300, True, 16),
          (2, 40, 3840, 256, False, 6)]


@pytest.mark.parametrize("kind,M,K,N,bias,splits", FORCED)
def test_small_m_forced_splits(crp, kind, M, K, N, bias, splits):
    print(f"[splitk-small-forced] kind={kind} M={M} K={K} N={N} splits={splits}", flush=True)
    L = si.random_layer(M, K, N, seed=M + K + N + kind + splits, bias=bias, outlier_count=5)
    (p, s), ref = _weights(crp, kind, L)
    b = to_dev_bf16(L.bias) if bias else None
    fn = {0: crp.linear_w4a4, 1: crp.linear_int8tw, 2: crp.linear_w4a8, 3: crp.linear_int8rot}[kind]
    crp.dbg_small_plan(splits)
    try:
        ws = torch.empty(crp.workspace_bytes(kind, M, N, K), dtype=torch.uint8, device="cuda")
        ws.fill_(0xA5)
        xs = [L.x, si.random_layer(M, K, 1, seed=7 + kind, outlier_count=5).x]
        ys = [fn(to_dev_bf16(xb), p, s, N, b, workspace=ws).clone() for xb in xs]
        acc = crp.dbg_linear_acc(kind, to_dev_bf16(xs[0]), p, N, workspace=ws)
        torch.cuda.synchronize()
    finally:
        crp.dbg_small_plan(0)
    for xb, y in zip(xs, ys):
        assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), O.f32_to_bf16_rne(ref(xb)["y"]))
    assert np.array_equal(acc.cpu().numpy(), ref(xs[0])["acc"])
