"""Seeded sweep of random layer shapes for every format, through the C ABI,
against the oracle: int32 accumulators bit-exact and bf16 outputs equal to
the oracle's float32 epilogue rounded to bf16.  The shapes land on every
path the planners choose between (small M with and without a K split, large
M with 256- or 192-wide tiles, with and without a K split) with ragged M, N
and K tails."""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import convrot_oracle as O
from tests._util import TOL, bf16_dev_to_f32, max_rel_err, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _shapes(kind, n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.choice([int(rng.integers(1, 129)), int(rng.integers(129, 700))]))
        N = int(rng.integers(1, 900))
        if kind == 1:
            K = int(rng.integers(1, 3000))
        else:
            K = 256 * int(rng.integers(1, 13))
        if M * N * K <= 120_000_000:
            out.append((M, K, N))
    return out


CASES = [(kind, *shape) for kind, seed in ((0, 101), (1, 202), (2, 303), (3, 404))
         for shape in _shapes(kind, 6, seed)]


@pytest.fixture(scope="module")
def crp():
    import rotated_bit_quantized_convrot_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("kind,M,K,N", CASES)
def test_random_shape(crp, kind, M, K, N):
    print(f"[random] kind={kind} M={M} K={K} N={N}", flush=True)
    L = si.random_layer(M, K, N, seed=M * 7 + K * 3 + N + kind, bias=(N % 2 == 0), outlier_count=5)
    x = to_dev_bf16(L.x)
    b = to_dev_bf16(L.bias) if L.bias is not None else None
    if kind == 0:
        p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
        y = crp.linear_w4a4(x, p, s, N, b)
        r = O.linear_w4a4(L.x, L.w, L.bias)
    elif kind == 1:
        p, s = crp.pack_weight_int8tw(to_dev_bf16(L.w))
        y = crp.linear_int8tw(x, p, s, N, b)
        r = O.linear_int8tw(L.x, L.w, L.bias)
    elif kind == 2:
        enc = O.w4a8_encode(L.w, iters=20)
        p = crp.pack_weight_w4a8(to_dev(enc["idx_packed"]), to_dev(enc["s_rel"]),
                                 to_dev(enc["codebook"].astype(np.float32)), N, K)
        y = crp.linear_w4a8(x, p, to_dev(enc["s_channel"]), N, b)
        r = O.linear_w4a8(L.x, enc["idx_packed"], enc["s_rel"], enc["codebook"], enc["s_channel"], L.bias)
    else:
        p, s = crp.pack_weight_int8rot(to_dev_bf16(L.w))
        y = crp.linear_int8rot(x, p, s, N, b)
        r = O.linear_int8rot(L.x, L.w, L.bias)
    a = crp.dbg_linear_acc(kind, x, p, N)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy(), r["acc"])
    assert max_rel_err(bf16_dev_to_f32(y), r["y"]) <= TOL
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), O.f32_to_bf16_rne(r["y"]))
