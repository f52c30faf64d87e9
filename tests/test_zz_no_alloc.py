"""cr_linear_w4a4_noalloc (the W4A4 linear on the library's static scratch,
for callers that cannot allocate) against cr_linear_w4a4 with a caller
workspace, through the C ABI: bf16 outputs bit-identical on two calls in a
row on one stream, the second with a smaller input (the scratch keeps the
first call's contents), both also against the oracle's accumulators and
rounding."""
import ctypes

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


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _case(crp, M, K, N, seed, bias):
    L = si.random_layer(M, K, N, seed=seed, bias=bias, outlier_count=5)
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    b = to_dev_bf16(L.bias) if bias else None
    return L, x, p, s, b


def _ref_bits(L):
    r = O.linear_w4a4(L.x, L.w, L.bias)
    return O.f32_to_bf16_rne(r["y"])


def test_noalloc_matches_linear_two_calls(crp):
    lib = crp.lib()
    st = torch.cuda.current_stream().cuda_stream
    # first call: the large-M path (ragged M and N tiles, bias); second call:
    # a smaller input on the small-M path, issued right behind the first
    cases = [(2050, 3072, 3000, 41, True), (70, 1024, 520, 42, False)]
    for M, K, N, _, _ in cases:
        assert crp.workspace_bytes(crp.W4A4, M, N, K) <= crp.NOALLOC_SCRATCH_BYTES
    prepared = [_case(crp, *c) for c in cases]
    outs = []
    for (L, x, p, s, b) in prepared:
        print(f"[noalloc] M={L.M} K={L.K} N={L.N}", flush=True)
        y = torch.empty((L.M, L.N), dtype=torch.bfloat16, device="cuda")
        rc = lib.cr_linear_w4a4_noalloc(x.data_ptr(), L.M, L.K, p.data_ptr(), s.data_ptr(), L.N,
                                        None if b is None else b.data_ptr(), y.data_ptr(), st)
        assert rc == 0, lib.cr_last_error()
        outs.append(y)
    torch.cuda.synchronize()
    for (L, x, p, s, b), y in zip(prepared, outs):
        ws = torch.empty(crp.workspace_bytes(crp.W4A4, L.M, L.N, L.K), dtype=torch.uint8, device="cuda")
        yref = torch.empty_like(y)
        rc = lib.cr_linear_w4a4(x.data_ptr(), L.M, L.K, p.data_ptr(), s.data_ptr(), L.N,
                                None if b is None else b.data_ptr(), yref.data_ptr(), ws.data_ptr(),
                                ws.numel(), st)
        assert rc == 0, lib.cr_last_error()
        torch.cuda.synchronize()
        got = _bits(y)
        assert np.array_equal(got, _bits(yref))
        assert np.array_equal(got, _ref_bits(L))


def test_noalloc_full_dit_w1_then_smaller(crp):
    """The headline layer (workspace 6.3 MB of the 8 MiB scratch), then a
    smaller one, through the binding's wrapper of the same C call."""
    L = si.dit_w1()
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    b = to_dev_bf16(L.bias)
    print("[noalloc] DiT W1", flush=True)
    y1 = crp.linear_w4a4_noalloc(x, p, s, L.N, b)
    L2, x2, p2, s2, b2 = _case(crp, 2050, 1536, 4100, 43, True)
    y2 = crp.linear_w4a4_noalloc(x2, p2, s2, L2.N, b2)
    torch.cuda.synchronize()
    ref1 = crp.linear_w4a4(x, p, s, L.N, b)
    ref2 = crp.linear_w4a4(x2, p2, s2, L2.N, b2)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y1), _bits(ref1))
    assert np.array_equal(_bits(y2), _bits(ref2))
    assert np.array_equal(_bits(y2), _ref_bits(L2))


def test_noalloc_rejects_sizes_beyond_the_scratch(crp):
    lib = crp.lib()
    vp = ctypes.c_void_p(16)
    # K = 9728 at M = 4096: 20 MB of activation codes alone
    need = crp.workspace_bytes(crp.W4A4, 4096, 2560, 9728)
    assert need > crp.NOALLOC_SCRATCH_BYTES
    assert lib.cr_linear_w4a4_noalloc(vp, 4096, 9728, vp, vp, 2560, None, vp, None) == 5   # CR_ERR_WORKSPACE
    assert b"static scratch" in lib.cr_last_error()
