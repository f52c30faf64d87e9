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
