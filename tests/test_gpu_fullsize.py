"""Full-size parity for every workload, in the launch configuration the
benchmark times: the GPU computes the whole layer and the oracle recomputes
every row of it (a few seconds of float64 BLAS per layer), compared bit-exact
on the int32 accumulators and on the bf16 output bits (the oracle's float32
epilogue rounded to nearest even), and within 1e-2 relative error.  Only the
M = 131071 case checks a sample of rows."""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import convrot_oracle as O
from tests._util import TOL, bf16_dev_to_f32, max_rel_err, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def crp():
    import rotated_bit_quantized_convrot_amd as m
    m.lib()
    return m


def _rows(M, n=None, seed=0):
    """All rows, or (n given) a seeded sample that keeps the first, middle
    and last rows."""
    if n is None or M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    fixed = [0, 1, M // 2, M - 2, M - 1]
    rest = rng.choice(np.setdiff1d(np.arange(M), fixed), n - len(fixed), replace=False)
    return np.sort(np.concatenate([fixed, rest]))


def _take(t, rows):
    if len(rows) == t.shape[0]:
        return t
    return t.index_select(0, torch.from_numpy(rows).cuda())


def _check(y, acc, rows, ref_acc, ref_y):
    a = _take(acc, rows).cpu().numpy()
    bad = np.argwhere(a != ref_acc)
    assert bad.size == 0, f"{len(bad)} accumulators differ, first at (row, col) {tuple(bad[0])}"
    yt = _take(y, rows)
    ybits = yt.view(torch.int16).cpu().numpy().view(np.uint16)
    want = O.f32_to_bf16_rne(ref_y)
    nbad = int(np.count_nonzero(ybits != want))
    assert nbad == 0, f"{nbad} bf16 outputs differ from the oracle's rounding"
    assert max_rel_err(bf16_dev_to_f32(yt), ref_y) <= TOL


W4A4_LAYERS = {
    "dit_w1": lambda: si.dit_w1(),
    "dit_w2": lambda: si.dit_w2(),
    "te_gate_up_M76": lambda: si.te_gate_up(76),
    "te_down_M76": lambda: si.te_down(76),
    "te_gate_up_M1220": lambda: si.te_gate_up(1220),
    "te_down_M1220": lambda: si.te_down(1220),
}


@pytest.mark.parametrize("name", list(W4A4_LAYERS))
def test_w4a4_full_size(crp, name):
    print(f"[fullsize] {name}", flush=True)
    L = W4A4_LAYERS[name]()
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    bias = to_dev_bf16(L.bias) if L.bias is not None else None
    ws = torch.empty(crp.workspace_bytes(0, L.M, L.N, L.K), dtype=torch.uint8, device="cuda")
    y = crp.linear_w4a4(x, p, s, L.N, bias, workspace=ws)
    acc = crp.dbg_linear_acc(0, x, p, L.N, workspace=ws)
    torch.cuda.synchronize()
    rows = _rows(L.M)
    qw, sw = O.quant_weight_w4(L.w)
    assert s.cpu().numpy()[:1].view(np.uint32)[0] == np.float32(sw).view(np.uint32)
    qx, sx = O.quant_act_w4a4(L.x[rows])
    ref_acc = O.int_gemm(qx, qw)
    _check(y, acc, rows, ref_acc, O.epilogue(ref_acc, sx, sw, L.bias))


INT8ROT_LAYERS = {"int8rot_attn_M76": lambda: si.te_attn_proj(76),
                  "int8rot_attn_M1220": lambda: si.te_attn_proj(1220)}


@pytest.mark.parametrize("name", list(INT8ROT_LAYERS))
def test_int8rot_full_size(crp, name):
    print(f"[fullsize] {name}", flush=True)
    L = INT8ROT_LAYERS[name]()
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_int8rot(to_dev_bf16(L.w))
    ws = torch.empty(crp.workspace_bytes(3, L.M, L.N, L.K), dtype=torch.uint8, device="cuda")
    y = crp.linear_int8rot(x, p, s, L.N, workspace=ws)
    acc = crp.dbg_linear_acc(3, x, p, L.N, workspace=ws)
    torch.cuda.synchronize()
    rows = _rows(L.M)
    qw, sw = O.quant_weight_int8rot(L.w)
    assert np.array_equal(s.cpu().numpy()[:L.N].view(np.uint32), sw.view(np.uint32))
    qx, sx = O.quant_act_int8rot(L.x[rows])
    ref_acc = O.int_gemm(qx, qw)
    _check(y, acc, rows, ref_acc, O.epilogue(ref_acc, sx, sw, None))


INT8_LAYERS = {"int8tw_vo": lambda: si.int8tw_vo(), "int8tw_k2688": lambda: si.int8tw_k2688()}


@pytest.mark.parametrize("name", list(INT8_LAYERS))
def test_int8tw_full_size(crp, name):
    print(f"[fullsize] {name}", flush=True)
    L = INT8_LAYERS[name]()
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_int8tw(to_dev_bf16(L.w))
    y = crp.linear_int8tw(x, p, s, L.N)
    acc = crp.dbg_linear_acc(1, x, p, L.N)
    torch.cuda.synchronize()
    rows = _rows(L.M)
    qw, sw = O.quant_weight_int8tw(L.w)
    qx, sx = O.quant_act_int8(L.x[rows])
    ref_acc = O.int_gemm(qx, qw)
    _check(y, acc, rows, ref_acc, O.epilogue(ref_acc, sx, sw, None))


def test_w4a8_full_size(crp):
    print("[fullsize] w4a8", flush=True)
    L = si.w4a8_layer()
    enc = O.w4a8_encode(L.w)
    x = to_dev_bf16(L.x)
    p = crp.pack_weight_w4a8(to_dev(enc["idx_packed"]), to_dev(enc["s_rel"]),
                             to_dev(enc["codebook"]), L.N, L.K)
    sch = to_dev(enc["s_channel"])
    y = crp.linear_w4a8(x, p, sch, L.N)
    acc = crp.dbg_linear_acc(2, x, p, L.N)
    torch.cuda.synchronize()
    rows = _rows(L.M)
    w8 = O.w4a8_decode(enc["idx"], enc["s_rel"], enc["codebook"])
    qx, sx = O.quant_act_w4a8(L.x[rows])
    ref_acc = O.int_gemm(qx, w8)
    _check(y, acc, rows, ref_acc, O.epilogue(ref_acc, sx, enc["s_channel"], None))


W4_VARIANTS = {"dit_w1_group64": 4, "dit_w1_group16": 5, "dit_w1_regular": 6}


@pytest.mark.parametrize("name", list(W4_VARIANTS))
def test_w4a4_rotation_variants_full_size(crp, name):
    """DiT W1 with the other rotations, as the benchmark rows run them."""
    print(f"[fullsize] {name}", flush=True)
    kind = W4_VARIANTS[name]
    L = si.dit_w1()
    x = to_dev_bf16(L.x)
    w = to_dev_bf16(L.w)
    if kind == 6:
        p, s = crp.pack_weight_w4_regular(w)
        y = crp.linear_w4a4_regular(x, p, s, L.N, to_dev_bf16(L.bias))
        qw, sw = O.quant_weight_w4_regular(L.w)
        qx, sx = O.quant_act_w4a4_regular(L.x[_rows(L.M)])
    else:
        G = 64 if kind == 4 else 16
        p, s = crp.pack_weight_w4(w, group=G)
        y = crp.linear_w4a4(x, p, s, L.N, to_dev_bf16(L.bias), group=G)
        qw, sw = O.quant_weight_w4(L.w, G)
        qx, sx = O.quant_act_w4a4(L.x[_rows(L.M)], G)
    acc = crp.dbg_linear_acc(kind, x, p, L.N)
    torch.cuda.synchronize()
    assert s.cpu().numpy()[:1].view(np.uint32)[0] == np.float32(sw).view(np.uint32)
    ref_acc = O.int_gemm(qx, qw)
    _check(y, acc, _rows(L.M), ref_acc, O.epilogue(ref_acc, sx, sw, L.bias))


@pytest.mark.parametrize("M", [76, 1220])
def test_mlp_block_full_size(crp, M):
    """The text-encoder MLP block at the benchmark's shapes: the GPU runs the
    whole block, the oracle follows every row through it and the bf16
    outputs must be equal."""
    print(f"[fullsize] te_mlp_M{M}", flush=True)
    xb, wg, wu, wd = si.te_mlp(M)
    F, N = wg.shape[0], wd.shape[0]
    packs = [crp.pack_weight_w4(to_dev_bf16(w)) for w in (wg, wu, wd)]
    (pg, sg), (pu, su), (pd, sd) = packs
    y = crp.mlp_w4a4(to_dev_bf16(xb), pg, sg, pu, su, F, pd, sd, N)
    torch.cuda.synchronize()
    rows = _rows(M)
    qg, s_g = O.quant_weight_w4(wg)
    qu, s_u = O.quant_weight_w4(wu)
    qd, s_d = O.quant_weight_w4(wd)
    qx, sx = O.quant_act_w4a4(xb[rows])
    g = O.f32_to_bf16_rne(O.epilogue(O.int_gemm(qx, qg), sx, s_g, None))
    u = O.f32_to_bf16_rne(O.epilogue(O.int_gemm(qx, qu), sx, s_u, None))
    qh, sh = O.quant_act_w4a4(O.silu_mul_bf16(g, u))
    ref_y = O.epilogue(O.int_gemm(qh, qd), sh, s_d, None)
    got = y.index_select(0, torch.from_numpy(rows).cuda())
    assert max_rel_err(bf16_dev_to_f32(got), ref_y) <= TOL
    assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), O.f32_to_bf16_rne(ref_y))


def test_w4a4_very_large_m(crp):
    """M = 131071 (512 row tiles, ragged last one): workspace and tile
    arithmetic far past the benchmark shapes; sampled rows checked."""
    print("[fullsize] very large M", flush=True)
    M, K, N = 131071, 256, 96
    L = si.random_layer(M, K, N, seed=77, bias=True, outlier_count=4)
    x = to_dev_bf16(L.x)
    p, s = crp.pack_weight_w4(to_dev_bf16(L.w))
    ws = torch.empty(crp.workspace_bytes(0, M, N, K), dtype=torch.uint8, device="cuda")
    y = crp.linear_w4a4(x, p, s, N, to_dev_bf16(L.bias), workspace=ws)
    acc = crp.dbg_linear_acc(0, x, p, N, workspace=ws)
    torch.cuda.synchronize()
    rows = _rows(M, n=4096, seed=3)
    qw, sw = O.quant_weight_w4(L.w)
    qx, sx = O.quant_act_w4a4(L.x[rows])
    ref_acc = O.int_gemm(qx, qw)
    _check(y, acc, rows, ref_acc, O.epilogue(ref_acc, sx, sw, L.bias))
