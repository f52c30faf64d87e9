"""The linears under HIP graph capture: every replay equals the eager result,
with other eager work and synchronisation between replays.  Shapes cover the
small-M path, the large-M path with whole tiles (256- and 192-wide) and the
large-M path with K split across blocks (two kernels per GEMM)."""
import numpy as np
import pytest

import synthetic_inputs as si
from tests._util import to_dev_bf16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("M,K,N", [(76, 2560, 1024), (300, 512, 256), (300, 4096, 512), (1025, 512, 768)])
def test_graph_replays_match_eager(M, K, N):
    import rotated_bit_quantized_convrot_amd as crp
    L = si.random_layer(M, K, N, seed=M + N, bias=True)
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    b = to_dev_bf16(L.bias)
    ws = torch.empty(crp.workspace_bytes(0, M, N, K), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ref = crp.linear_w4a4(x, p, s, N, b).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        crp.linear_w4a4(x, p, s, N, b, out=y, workspace=ws)
        crp.linear_w4a4(x, p, s, N, b, out=y, workspace=ws)
    for i in range(4):
        y.zero_()
        other = crp.linear_w4a4(x, p, s, N, None)   # eager work on another output
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {i}"
        assert not torch.equal(other, ref)


def test_graph_mlp_block_and_rotation_variants():
    """The MLP block (five launches, workspace-resident g and u) and the group /
    regular-Hadamard linears under capture: every replay equals eager."""
    import rotated_bit_quantized_convrot_amd as crp
    M, K, F, N = 76, 512, 768, 256
    xb, _, _, _ = si.te_mlp(M)
    L = si.random_layer(M, K, N, seed=9)
    rng = np.random.default_rng(10)
    ws_ = [si.f32_to_bf16_bits((rng.standard_normal(s) * 0.02).astype(np.float32)) for s in ((F, K), (F, K), (N, F))]
    x = to_dev_bf16(L.x)
    (pg, sg), (pu, su), (pd, sd) = [crp.pack_weight_w4(to_dev_bf16(w)) for w in ws_]
    p64, s64 = crp.pack_weight_w4(to_dev_bf16(L.w), group=64)
    prh, srh = crp.pack_weight_w4_regular(to_dev_bf16(L.w))
    wsm = torch.empty(crp.mlp_workspace_bytes(M, K, F, N), dtype=torch.uint8, device="cuda")
    wsl = torch.empty(crp.workspace_bytes(0, M, N, K), dtype=torch.uint8, device="cuda")
    ym = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y64 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    yrh = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ref = [crp.mlp_w4a4(x, pg, sg, pu, su, F, pd, sd, N).clone(),
           crp.linear_w4a4(x, p64, s64, N, group=64).clone(),
           crp.linear_w4a4_regular(x, prh, srh, N).clone()]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        crp.mlp_w4a4(x, pg, sg, pu, su, F, pd, sd, N, out=ym, workspace=wsm)
        crp.linear_w4a4(x, p64, s64, N, out=y64, workspace=wsl, group=64)
        crp.linear_w4a4_regular(x, prh, srh, N, out=yrh, workspace=wsl)
    for i in range(4):
        for t in (ym, y64, yrh):
            t.zero_()
        crp.linear_w4a4(x, p64, s64, N)           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ym, ref[0]) and torch.equal(y64, ref[1]) and torch.equal(yrh, ref[2]), f"replay {i}"


def test_graph_w4a8_large_m_decode_route():
    """W4A8 at M >= 2048 (weight decoded into the workspace, then the int8
    GEMM) under capture: every replay equals eager."""
    import rotated_bit_quantized_convrot_amd as crp
    from tests._util import to_dev
    M, K, N = 2048, 512, 320
    L = si.random_layer(M, K, N, seed=31, bias=True)
    idx, s_rel, cb, s_ch = si.random_w4a8_format(N, K, seed=5)
    p = crp.pack_weight_w4a8(to_dev(idx), to_dev(s_rel), to_dev(cb), N, K)
    sch = to_dev(s_ch)
    x = to_dev_bf16(L.x)
    b = to_dev_bf16(L.bias)
    ws = torch.empty(crp.workspace_bytes(2, M, N, K), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ref = crp.linear_w4a8(x, p, sch, N, b).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        crp.linear_w4a8(x, p, sch, N, b, out=y, workspace=ws)
    for i in range(4):
        y.zero_()
        ws.fill_(0x5A)                                  # the decoded copy must be rebuilt each replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {i}"
