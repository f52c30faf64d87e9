"""The fused small-M W4A4 linear: one launch whose first blocks rotate and
quantise the activation rows while the GEMM blocks load their weights and
then wait (bounded) for the rows.  Its outputs must be the oracle's bit for
bit and those of the two-launch path (activation quantiser, then GEMM), on
a workspace that starts as garbage, over several calls in a row with new
activations (a stale code, scale or counter of an earlier call would show).
The fused launch is forced (mode 2) at every size; by default it is taken
at M <= 8 only.  The timeout branch is forced from the host (a wait of zero
polls): every GEMM block then exits without writing, and the next call is
correct again."""
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
    yield m
    m.dbg_fused_config(1, 1 << 22)


def _bits(y):
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


# (M, K, N, bias): one row to 128 rows (ragged activation tiles), two rows per
# producer block (K <= 4096) and one (K > 4096), one 256-group per producer
# lane (K <= 8192) and two (up to K = 16384, ragged second pass), one weight
# tile to many, K split across blocks; N = 1030 is not a multiple of 4 and
# takes the two-launch path (the comparison still holds)
CASES = [(1, 256, 4, False), (1, 3072, 3072, True), (16, 4096, 640, True), (17, 4352, 1028, False),
         (33, 8192, 256, True), (76, 3072, 3072, True), (76, 3072, 8192, False), (76, 8192, 3072, True),
         (100, 1280, 2560, True), (128, 2560, 1024, False), (76, 9728, 640, True), (40, 16384, 512, True),
         (76, 2560, 1030, True)]


@pytest.mark.parametrize("M,K,N,bias", CASES)
def test_fused_matches_oracle_and_two_launch_path(crp, M, K, N, bias):
    print(f"[fused-small] M={M} K={K} N={N} bias={bias}", flush=True)
    L = si.random_layer(M, K, N, seed=3 * M + K + N, bias=bias, outlier_count=5)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    b = to_dev_bf16(L.bias) if bias else None
    ws = torch.empty(crp.workspace_bytes(0, M, N, K), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)
    xs = [si.random_layer(M, K, 1, seed=1000 + 7 * r + M, outlier_count=5).x for r in range(3)]
    xs[1][M // 2] = 0                                     # a zero row: scale 0, codes 0
    crp.dbg_fused_config(2)
    fused = [crp.linear_w4a4(to_dev_bf16(xb), p, s, N, b, workspace=ws).clone() for xb in xs]
    acc = crp.dbg_linear_acc(0, to_dev_bf16(xs[-1]), p, N, workspace=ws)
    crp.dbg_fused_config(0)
    two = [crp.linear_w4a4(to_dev_bf16(xb), p, s, N, b, workspace=ws).clone() for xb in xs]
    crp.dbg_fused_config(1)
    torch.cuda.synchronize()
    assert crp.dbg_fused_timeouts() == 0
    for xb, yf, y2 in zip(xs, fused, two):
        ref = O.f32_to_bf16_rne(O.linear_w4a4(xb, L.w, L.bias)["y"])
        assert np.array_equal(_bits(yf), ref)
        assert np.array_equal(_bits(y2), ref)
    assert np.array_equal(acc.cpu().numpy(), O.linear_w4a4(xs[-1], L.w, L.bias)["acc"])


def test_fused_timeout_forced_from_host(crp):
    """A wait of zero polls: the GEMM blocks leave y as it was and count their
    timeouts; the producers still finish, the slot is reset, and the next
    call (normal wait) is the oracle's again."""
    M, K, N = 76, 3072, 1024
    L = si.random_layer(M, K, N, seed=77, bias=True)
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    b = to_dev_bf16(L.bias)
    ws = torch.empty(crp.workspace_bytes(0, M, N, K), dtype=torch.uint8, device="cuda")
    y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    before = crp.dbg_fused_timeouts()
    crp.dbg_fused_config(2, 0)
    try:
        crp.linear_w4a4(x, p, s, N, b, out=y, workspace=ws)
        torch.cuda.synchronize()
    finally:
        crp.dbg_fused_config(1, 1 << 22)
    assert crp.dbg_fused_timeouts() > before
    assert bool((y == 3.0).all())
    after = crp.dbg_fused_timeouts()
    ref = O.f32_to_bf16_rne(O.linear_w4a4(L.x, L.w, L.bias)["y"])
    crp.dbg_fused_config(2)
    try:
        for _ in range(2):
            y2 = crp.linear_w4a4(x, p, s, N, b, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(_bits(y2), ref)
    finally:
        crp.dbg_fused_config(1)
    assert crp.dbg_fused_timeouts() == after


def _w(shape, seed):
    rng = np.random.default_rng(seed)
    return si.f32_to_bf16_bits((rng.standard_normal(shape) * 0.02).astype(np.float32))


@pytest.mark.parametrize("M,K,F,N", [(76, 2560, 9728, 2560), (33, 4352, 8448, 512), (1, 256, 512, 256)])
def test_fused_mlp_block(crp, M, K, F, N):
    """The MLP block with its gate GEMM quantising x and its down GEMM forming
    and quantising h = silu(g) * u in their own launches: the oracle's output
    bit for bit, and the five-launch block's."""
    print(f"[fused-mlp] M={M} K={K} F={F} N={N}", flush=True)
    L = si.random_layer(M, K, 1, seed=M + F, outlier_count=5)
    wg, wu, wd = _w((F, K), 1), _w((F, K), 2), _w((N, F), 3)
    x = to_dev_bf16(L.x)
    (pg, sg), (pu, su), (pd, sd) = [crp.pack_weight_w4(to_dev_bf16(w)) for w in (wg, wu, wd)]
    ws = torch.empty(crp.mlp_workspace_bytes(M, K, F, N), dtype=torch.uint8, device="cuda")
    ws.fill_(0x5A)
    crp.dbg_fused_config(2)
    yf = [crp.mlp_w4a4(x, pg, sg, pu, su, F, pd, sd, N, workspace=ws).clone() for _ in range(2)]
    crp.dbg_fused_config(0)
    y5 = crp.mlp_w4a4(x, pg, sg, pu, su, F, pd, sd, N, workspace=ws).clone()
    crp.dbg_fused_config(1)
    torch.cuda.synchronize()
    ref = O.f32_to_bf16_rne(O.mlp_w4a4(L.x, wg, wu, wd)["y"])
    for y in yf + [y5]:
        assert np.array_equal(_bits(y), ref)


def test_default_routing_by_m(crp):
    """Mode 1 (the default) takes the fused launch at M <= 8 and two launches
    above: with a wait of zero polls only the fused launch counts timeouts."""
    K, N = 3072, 1024
    L = si.random_layer(16, K, N, seed=5)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    crp.dbg_fused_config(1, 0)
    try:
        for M, fused in ((1, True), (8, True), (9, False), (16, False)):
            x = to_dev_bf16(L.x[:M])
            before = crp.dbg_fused_timeouts()
            crp.linear_w4a4(x, p, s, N)
            torch.cuda.synchronize()
            assert (crp.dbg_fused_timeouts() > before) == fused, M
    finally:
        crp.dbg_fused_config(1, 1 << 22)


@pytest.mark.parametrize("M", [1, 5, 8])
def test_fused_under_graph_capture(crp, M):
    """The fused launch (its counter slot fixed at capture) in a replayed
    graph, eager work and synchronisation between replays, every replay equal
    to the eager result and to the oracle; the MLP block too."""
    K, N = 2560, 3072
    L = si.random_layer(M, K, N, seed=40 + M, bias=True, outlier_count=5)
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    b = to_dev_bf16(L.bias)
    ws = torch.empty(crp.workspace_bytes(0, M, N, K), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ref = crp.linear_w4a4(x, p, s, N, b).clone()
    torch.cuda.synchronize()
    assert np.array_equal(_bits(ref), O.f32_to_bf16_rne(O.linear_w4a4(L.x, L.w, L.bias)["y"]))
    F = 768
    wg, wu, wd = _w((F, K), 7), _w((F, K), 8), _w((N, F), 9)
    (pg, sg), (pu, su), (pd, sd) = [crp.pack_weight_w4(to_dev_bf16(w)) for w in (wg, wu, wd)]
    wsm = torch.empty(crp.mlp_workspace_bytes(M, K, F, N), dtype=torch.uint8, device="cuda")
    ym = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    refm = crp.mlp_w4a4(x, pg, sg, pu, su, F, pd, sd, N).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        crp.linear_w4a4(x, p, s, N, b, out=y, workspace=ws)
        crp.mlp_w4a4(x, pg, sg, pu, su, F, pd, sd, N, out=ym, workspace=wsm)
    for i in range(4):
        y.zero_()
        ym.zero_()
        crp.linear_w4a4(x, p, s, N, None)       # eager fused launches between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref) and torch.equal(ym, refm), f"replay {i}"
    assert np.array_equal(_bits(refm), O.f32_to_bf16_rne(O.mlp_w4a4(L.x, wg, wu, wd)["y"]))
