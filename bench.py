#!/usr/bin/env python3
"""Benchmark of the ConvRot-quantized linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--prewarm-ms MS] [--no-cpu-baseline]
                    [--rows all|none|name,name] [--repeat R]

Headline ("step"): one W4A4 ConvRot linear of the DiT image-token MLP (W1,
x bf16 [4096,3072], W [12288,3072], bias) - activation rotation +
quantisation kernel, then the int-MFMA GEMM with the rank-one epilogue - on
inputs resident in HBM, weights packed beforehand (offline).  value = int
TOPS (2*M*N*K / wall time per step over the K timed steps, after an untimed
run of --prewarm-ms for the clock ramp and W warm-up steps); K further steps
with HIP events around each GEMM launch give its average launch duration for
the roofline.

Also measured in the same run, each by replaying a HIP graph of repeated
calls and timing it with HIP events on the launch stream:
  * the GEMM kernel alone (roofline: int8 MFMA peak 5.0 POPS dense) and the
    activation kernel alone (roofline: HBM 8 TB/s);
  * every other row of the hot path (the W4A8 layer's weight encoded from
    its bf16 values by the library's GPU encoder): DiT W2, text-encoder gate/up and down
    at M=76 (weight-stream GB/s with cold weights cycled through 48 copies,
    more than twice the 256 MB last-level cache) and M=1220, the
    int8_tensorwise V/O and K=2688 layers, the W4A8 codebook layer, and the
    ConvRot INT8 row-scaled format on a square text-encoder projection
    (K=N=2560) at M=76 and M=1220, and the DiT W1 layer with W4A4 rotation
    groups of 64 and 16 and with the group-256 regular Hadamard;
  * the text-encoder MLP block (cr_mlp_w4a4: gate and up 2560 -> 9728,
    silu(g) * u, down 9728 -> 2560) at M=76 (cold weights) and M=1220.
The CPU oracle (NumPy) is timed on a row sample of the headline layer.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0        # MI355X dense int8 MFMA, 5.0 POPS
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
COLD_COPIES = 48
COPY_BYTES = 512 << 20         # plain device copy used to calibrate the HBM byte counters


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sources_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rotated_bit_quantized_convrot_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# Rows of the hot path
# ---------------------------------------------------------------------------

def row_specs():
    import synthetic_inputs as si
    return {
        "dit_w1": dict(kind=0, gen=lambda: si.dit_w1(), cold=False),
        "dit_w2": dict(kind=0, gen=lambda: si.dit_w2(), cold=False),
        "dit_w1_group64": dict(kind=4, gen=lambda: si.dit_w1(), cold=False),
        "dit_w1_group16": dict(kind=5, gen=lambda: si.dit_w1(), cold=False),
        "dit_w1_regular": dict(kind=6, gen=lambda: si.dit_w1(), cold=False),
        "te_gate_up_M1": dict(kind=0, gen=lambda: si.te_gate_up(1), cold=True),
        "te_down_M1": dict(kind=0, gen=lambda: si.te_down(1), cold=True),
        "te_gate_up_M76": dict(kind=0, gen=lambda: si.te_gate_up(76), cold=True),
        "te_down_M76": dict(kind=0, gen=lambda: si.te_down(76), cold=True),
        "te_gate_up_M1220": dict(kind=0, gen=lambda: si.te_gate_up(1220), cold=False),
        "te_down_M1220": dict(kind=0, gen=lambda: si.te_down(1220), cold=False),
        "int8tw_vo": dict(kind=1, gen=lambda: si.int8tw_vo(), cold=False),
        "int8tw_k2688": dict(kind=1, gen=lambda: si.int8tw_k2688(), cold=False),
        "w4a8": dict(kind=2, gen=lambda: si.w4a8_layer(), cold=False),
        "int8rot_attn_M76": dict(kind=3, gen=lambda: si.te_attn_proj(76), cold=True),
        "int8rot_attn_M1220": dict(kind=3, gen=lambda: si.te_attn_proj(1220), cold=False),
    }


class Layer:
    """A layer's device buffers: x, packed weight(s), scale, bias, y, workspace."""

    def __init__(self, crp, torch, L, kind, copies=1):
        import synthetic_inputs as si
        dev = "cuda"
        self.crp, self.torch, self.kind = crp, torch, kind
        self.M, self.K, self.N = L.M, L.K, L.N
        self.x = torch.from_numpy(L.x.view(np.int16)).view(torch.bfloat16).to(dev)
        self.bias = None
        if L.bias is not None:
            self.bias = torch.from_numpy(L.bias.view(np.int16)).view(torch.bfloat16).to(dev)
        self.encode_ms = None
        if kind == 2:
            # the layer's own weight, encoded on the GPU (Lloyd-Max codebook,
            # E4M3 group scales, channel scales), then laid out for the GEMM
            w = torch.from_numpy(L.w.view(np.int16)).view(torch.bfloat16).to(dev)
            ews = torch.empty(crp.encode_w4a8_workspace_bytes(L.N, L.K), dtype=torch.uint8, device=dev)
            crp.encode_w4a8(w, workspace=ews)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            idx, s_rel, cb, s_ch = crp.encode_w4a8(w, workspace=ews)
            e1.record()
            torch.cuda.synchronize()
            self.encode_ms = e0.elapsed_time(e1)
            del ews, w
            p = crp.pack_weight_w4a8(idx, s_rel, cb, L.N, L.K)
            s = s_ch
        else:
            w = torch.from_numpy(L.w.view(np.int16)).view(torch.bfloat16).to(dev)
            p, s = {0: crp.pack_weight_w4, 1: crp.pack_weight_int8tw, 3: crp.pack_weight_int8rot,
                    4: lambda t: crp.pack_weight_w4(t, group=64),
                    5: lambda t: crp.pack_weight_w4(t, group=16), 6: crp.pack_weight_w4_regular}[kind](w)
            del w
        self.packed = [p] + [p.clone() for _ in range(copies - 1)]
        self.scale = s
        self.y = torch.empty((L.M, L.N), dtype=torch.bfloat16, device=dev)
        self.ws = torch.empty(crp.workspace_bytes(kind, L.M, L.N, L.K), dtype=torch.uint8, device=dev)
        self.fn = {0: crp.linear_w4a4, 1: crp.linear_int8tw, 2: crp.linear_w4a8, 3: crp.linear_int8rot,
                   4: lambda *a: crp.linear_w4a4(*a, group=64),
                   5: lambda *a: crp.linear_w4a4(*a, group=16), 6: crp.linear_w4a4_regular}[kind]
        self.w4 = kind in (0, 4, 5, 6)

    def linear(self, i=0):
        return self.fn(self.x, self.packed[i], self.scale, self.N, self.bias, self.y, self.ws)

    def quant(self):
        self.crp.quantize_activations(self.kind, self.x, self.ws)

    def gemm(self, i=0):
        self.crp.gemm_quantized(self.kind, self.M, self.K, self.packed[i], self.scale, self.N, self.ws,
                                self.bias, self.y)

    # algorithmic quantities
    def ops(self):
        return 2.0 * self.M * self.N * self.K

    def weight_bytes(self):
        if self.w4:
            return self.N * self.K / 2
        if self.kind == 1:
            return self.N * self.K
        if self.kind == 3:
            return self.N * self.K + 4 * self.N
        return self.N * self.K / 2 + self.N * self.K / 16 + 4 * self.N

    def gemm_bytes(self):
        qx = self.M * self.K / 2 if self.w4 else self.M * self.K    # activation codes
        y = self.M * self.N * 2
        b = self.N * 2 if self.bias is not None else 0
        return qx + self.weight_bytes() + y + b + 4 * self.M

    def quant_bytes(self):
        if self.w4:             # 4-bit codes, scale and correction sum per row
            return self.M * self.K * 2 + self.M * self.K / 2 + 8 * self.M
        return self.M * self.K * 2 + self.M * self.K + 4 * self.M

    def linear_bytes(self):
        return self.M * self.K * 2 + self.weight_bytes() + self.M * self.N * 2 + \
            (self.N * 2 if self.bias is not None else 0)


def graph_time_us(torch, fn_list, min_us=4000.0):
    """Average time per call of the calls in fn_list, replayed as one HIP graph.

    The graph is replayed until at least min_us of GPU time is timed, so that
    short kernels are measured over a long enough window."""
    for f in fn_list:          # eager warm-up (first-call checks happen outside capture)
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fn_list:
            f()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        g.replay()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1) * 1e3, 1.0)
    iters = int(min(2000, max(5, min_us // one + 1)))
    e0.record()
    for _ in range(iters):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (iters * len(fn_list))
    del g
    return us


def measure_row(torch, lay: Layer, cold: bool, reps: int):
    n = len(lay.packed)
    calls = max(reps, n)
    out = {}
    out["linear_us"] = graph_time_us(torch, [lambda i=i: lay.linear(i % n) for i in range(calls)])
    lay.quant()
    out["gemm_us"] = graph_time_us(torch, [lambda i=i: lay.gemm(i % n) for i in range(calls)])
    out["quant_us"] = graph_time_us(torch, [lay.quant for _ in range(reps)])
    out["linear_tops"] = lay.ops() / (out["linear_us"] * 1e-6) / 1e12
    out["gemm_tops"] = lay.ops() / (out["gemm_us"] * 1e-6) / 1e12
    out["gemm_frac_int8_peak"] = out["gemm_tops"] / PEAK_INT8_TOPS
    out["weight_gbs"] = lay.weight_bytes() / (out["gemm_us"] * 1e-6) / 1e9
    out["gemm_alg_gbs"] = lay.gemm_bytes() / (out["gemm_us"] * 1e-6) / 1e9
    out["linear_alg_gbs"] = lay.linear_bytes() / (out["linear_us"] * 1e-6) / 1e9
    out["quant_gbs"] = lay.quant_bytes() / (out["quant_us"] * 1e-6) / 1e9
    out["cold_weights"] = bool(cold)
    if lay.encode_ms is not None:
        out["encode_ms"] = lay.encode_ms     # offline: the GPU encoder of this layer's weight
    out["shape"] = {"M": lay.M, "K": lay.K, "N": lay.N}
    return out


def measure_mlp(torch, crp, M: int, cold: bool, reps: int):
    """The text-encoder MLP block (K=2560, F=9728, N=2560; inputs
    synthetic_inputs.te_mlp) through cr_mlp_w4a4, by graph replay; cold: the
    three packed weights cycled through enough copies to exceed the
    last-level cache."""
    import synthetic_inputs as si
    K, F, N = 2560, 9728, 2560
    xb, wg, wu, wd = si.te_mlp(M)
    dev = "cuda"
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    packs = []
    for w in (wg, wu, wd):
        t = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev)
        packs.append(crp.pack_weight_w4(t))
        del t
    copies = max(1, COLD_COPIES // 3) if cold else 1
    sets = [[(p.clone(), s) for (p, s) in packs] for _ in range(copies - 1)] + [packs]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(crp.mlp_workspace_bytes(M, K, F, N), dtype=torch.uint8, device=dev)

    def call(i):
        (pg, sg), (pu, su), (pd, sd) = sets[i % len(sets)]
        crp.mlp_w4a4(x, pg, sg, pu, su, F, pd, sd, N, out=y, workspace=ws)

    calls = max(reps, len(sets))
    us = graph_time_us(torch, [lambda i=i: call(i) for i in range(calls)])
    ops = 2.0 * M * K * F * 2 + 2.0 * M * F * N
    wbytes = (2 * F * K + N * F) / 2
    return {"mlp_us": us, "tops": ops / (us * 1e-6) / 1e12, "weight_gbs": wbytes / (us * 1e-6) / 1e9,
            "cold_weights": bool(cold), "shape": {"M": M, "K": K, "F": F, "N": N},
            # gate and down GEMMs quantise their own inputs at M <= 8
            "launches": 3 if M <= 8 else 5}


# ---------------------------------------------------------------------------
# Ceilings of the machine at hand (probe kernels of the library, not the
# method): int8 matrix-core rate, cold single-kernel read, plain copy; and the
# shader clock, from the kernels' own cycle and real-time counters
# ---------------------------------------------------------------------------

def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _sclk_mhz(stamps, wall_khz):
    """Shader clock (MHz) from a probe's cycle and real-time counter stamps."""
    c0, c1, w0, w1 = [int(v) for v in stamps]
    if wall_khz <= 0 or w1 <= w0:
        return None
    return (c1 - c0) / ((w1 - w0) / (wall_khz * 1e3)) / 1e6


def clock_sample(torch, crp):
    """Shader clock right now: a one-block matrix-core probe of ~0.1 ms,
    enqueued behind whatever the stream is running."""
    sink = torch.empty(512, dtype=torch.int32, device="cuda")
    stamps = torch.zeros(4, dtype=torch.int64, device="cuda")
    crp.probe_mfma_i8(1, 2000, sink, stamps)
    torch.cuda.synchronize()
    return _sclk_mhz(stamps.cpu().tolist(), crp.probe_wall_clock_khz())


def measure_ceilings(torch, crp, read_bytes: int, copies: int):
    """Probe ceilings: the int8 matrix-core rate (8 and 16 waves per CU, at the
    chip's power limit after a warm-up of the same launch), the rate of one
    kernel reading a cold buffer of ``read_bytes`` (cycled through ``copies``
    distinct buffers, by graph replay, as the cold-weight rows are), and a
    512 MiB device copy."""
    dev = "cuda"
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    khz = crp.probe_wall_clock_khz()
    out = {"wall_clock_khz": khz, "cus": ncu}
    sink = torch.empty(2 * ncu * 512, dtype=torch.int32, device=dev)
    stamps = torch.zeros(4, dtype=torch.int64, device=dev)
    best = None
    for blocks, iters in ((ncu, 400), (2 * ncu, 200)):
        for _ in range(3):                              # warm-up: clock settles under this load
            crp.probe_mfma_i8(blocks, iters, sink, stamps)
        torch.cuda.synchronize()
        runs = []
        for _ in range(3):
            e0, e1 = _events(torch)
            e0.record()
            crp.probe_mfma_i8(blocks, iters, sink, stamps)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3
            runs.append((us, _sclk_mhz(stamps.cpu().tolist(), khz)))
        us, mhz = sorted(runs)[1]
        ops = blocks * 8.0 * iters * 4 * 65536
        r = {"waves_per_cu": 8 * blocks // ncu, "us": round(us, 1), "tops": round(ops / (us * 1e-6) / 1e12, 1),
             "sclk_mhz": round(mhz, 1) if mhz else None}
        out[f"mfma_i8_{r['waves_per_cu']}w"] = r
        if best is None or r["tops"] > best["tops"]:
            best = r
    out["mfma_i8_tops"] = best["tops"]
    out["mfma_i8_sclk_mhz"] = best["sclk_mhz"]
    del sink

    n16 = read_bytes // 16 * 16
    bufs = [torch.empty(n16, dtype=torch.uint8, device=dev).fill_(i & 0xFF) for i in range(copies)]
    rsink = torch.empty(crp.PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
    read_us = graph_time_us(torch, [lambda i=i: crp.probe_read(bufs[i], rsink) for i in range(copies)])
    out["cold_read"] = {"bytes": n16, "copies": copies, "us": round(read_us, 3),
                        "gbs": round(n16 / (read_us * 1e-6) / 1e9, 1)}
    del bufs
    src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    crp.probe_copy(src, dst)
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(5):
        crp.probe_copy(src, dst)
    e1.record()
    torch.cuda.synchronize()
    cus = e0.elapsed_time(e1) * 1e3 / 5
    out["copy"] = {"bytes": COPY_BYTES, "us": round(cus, 1), "gbs_read_plus_write": round(2 * COPY_BYTES / (cus * 1e-6) / 1e9, 1)}
    del src, dst
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a row sample of the headline layer
# ---------------------------------------------------------------------------

def cpu_baseline(L, rows: int, min_seconds: float = 10.0):
    """The oracle on blocks of `rows` rows of the headline layer, taken in turn
    (wrapping around) until at least min_seconds of CPU time have been spent."""
    from oracle import convrot_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    qw, sw = O.quant_weight_w4(L.w)           # offline weight preparation: not timed
    bias = L.bias
    done_rows = 0
    blocks = 0
    t0 = time.perf_counter()
    while True:
        r0 = (blocks * rows) % L.M
        xs = L.x[r0:r0 + rows]
        qx, sx = O.quant_act_w4a4(xs)
        acc = O.int_gemm(qx, qw)
        O.epilogue(acc, sx, sw, bias)
        done_rows += xs.shape[0]
        blocks += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or dt > 30.0:
            break
    ops = 2.0 * done_rows * L.N * L.K
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"DiT W1 W4A4 linear (K={L.K}, N={L.N}), {blocks} blocks of {rows} rows "
                      f"({done_rows} rows, the {L.M}-row input taken in turn); rotation+quantisation of x, "
                      "exact integer GEMM (float64 BLAS), epilogue; weight preparation excluded "
                      "(offline on both sides)"}


def load_traffic(kernel_hash: str):
    """HBM traffic per GEMM launch from committed rocprofv3 --pmc runs, if they
    were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "gemm_w4a4_dit_w1_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_sources_hash") != kernel_hash:
        return None
    return d.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--repeat", type=int, default=20, help="calls per captured graph")
    ap.add_argument("--rows", default="all", help="all | none | comma-separated row names")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the probe ceilings")
    ap.add_argument("--cpu-rows", type=int, default=512)
    ap.add_argument("--prewarm-ms", type=float, default=150.0,
                    help="untimed run of the step before the warm-up steps (clock ramp)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only launch the headline GEMM 5 times and a 512 MiB device copy 5 times "
                         "(for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs), then exit")
    ap.add_argument("--traffic-row", default="dit_w1", choices=sorted(row_specs()),
                    help="row whose GEMM --traffic-probe launches (a cold row uses a different weight "
                         "copy for each of the 5 launches)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(the linear would shard by rows with no communication); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import rotated_bit_quantized_convrot_amd as crp
    crp.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    khash = kernel_sources_hash()

    specs = row_specs()
    _log("generating DiT W1 inputs")
    Lh = specs["dit_w1"]["gen"]()
    head = Layer(crp, torch, Lh, 0)

    if args.traffic_probe:
        probe = head
        if args.traffic_row != "dit_w1":
            spec = specs[args.traffic_row]
            probe = Layer(crp, torch, spec["gen"](), spec["kind"], copies=5 if spec["cold"] else 1)
        probe.quant()
        for i in range(5):
            probe.gemm(i % len(probe.packed))
        if probe.kind == 0 and probe.M <= 8:
            # the whole linear too: one fused launch at this size
            for i in range(5):
                probe.linear(i % len(probe.packed))
        torch.cuda.synchronize()
        src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": True, "row": args.traffic_row, "gemm_launches": 5,
                          "copy_launches": 5, "copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES,
                          "gemm_algorithmic_bytes": probe.gemm_bytes()}), flush=True)
        return

    # --- headline: K timed steps of the whole linear -----------------------
    # The GPU raises its clocks only after some tens of milliseconds of
    # sustained work (an idle gap of ~0.5 s drops them again), so the step
    # first runs untimed for at least --prewarm-ms of wall time, then the W
    # warm-up steps, then exactly K timed steps.
    torch.cuda.synchronize()
    t_pw = time.perf_counter()
    prewarm_steps = 0
    while (time.perf_counter() - t_pw) * 1e3 < args.prewarm_ms:
        for _ in range(20):
            head.linear()
        prewarm_steps += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        head.linear()
    torch.cuda.synchronize()
    # Timed region: exactly K steps of the linear, bracketed by synchronize.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        head.linear()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    value = head.ops() / (ms_per_step * 1e-3) / 1e12

    # Kernel durations, live: right after, K more steps as the linear's two
    # halves (cr_quantize_activations then cr_gemm_quantized: the same
    # kernels and bits as cr_linear_w4a4) with HIP events on the launch
    # stream around each GEMM launch (each event record costs ~3 us of GPU
    # time, which is why the value pass above has none).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(args.steps):
        head.quant()
        evs[k][0].record()
        head.gemm()
        evs[k][1].record()
    torch.cuda.synchronize()
    step_gemm_us = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e3
    sclk_headline = clock_sample(torch, crp)
    _log(f"headline: {ms_per_step * 1e3:.1f} us/step wall, {ev_ms * 1e3:.1f} us/step events; "
         f"GEMM {step_gemm_us:.1f} us per launch")
    # --- kernels of the headline step: GEMM and activation kernel -----------
    hrow = measure_row(torch, head, False, args.repeat)
    _log(f"dit_w1 gemm {hrow['gemm_us']:.1f} us = {hrow['gemm_tops']:.0f} TOPS; "
         f"quant {hrow['quant_us']:.1f} us")

    rows = {"dit_w1": hrow}
    wanted = [] if args.rows == "none" else (
        [r for r in specs if r != "dit_w1"] if args.rows == "all" else
        [r for r in args.rows.split(",") if r != "dit_w1" and r in specs])
    for name in wanted:
        sp = specs[name]
        _log(f"row {name}")
        lay = Layer(crp, torch, sp["gen"](), sp["kind"], COLD_COPIES if sp["cold"] else 1)
        rows[name] = measure_row(torch, lay, sp["cold"], args.repeat)
        r = rows[name]
        _log(f"  linear {r['linear_us']:.2f} us ({r['linear_tops']:.0f} TOPS), gemm {r['gemm_us']:.2f} us "
             f"({r['gemm_tops']:.0f} TOPS, weights {r['weight_gbs']:.0f} GB/s), quant {r['quant_us']:.2f} us")
        del lay
        torch.cuda.empty_cache()

    for name, M, cold in (("te_mlp_M1", 1, True), ("te_mlp_M76", 76, True), ("te_mlp_M1220", 1220, False)):
        if args.rows == "all" or name in args.rows.split(","):
            _log(f"row {name}")
            rows[name] = measure_mlp(torch, crp, M, cold, args.repeat)
            _log(f"  MLP block {rows[name]['mlp_us']:.2f} us ({rows[name]['tops']:.0f} TOPS, "
                 f"weights {rows[name]['weight_gbs']:.0f} GB/s)")
            torch.cuda.empty_cache()

    ceil = None
    if not args.no_ceilings:
        _log("ceilings: int8 matrix-core probe, cold read, copy")
        ceil = measure_ceilings(torch, crp, int(9728 * 2560 // 2), COLD_COPIES)
        _log(f"  mfma {ceil['mfma_i8_tops']} TOPS at {ceil['mfma_i8_sclk_mhz']} MHz; cold read "
             f"{ceil['cold_read']['us']} us = {ceil['cold_read']['gbs']} GB/s; copy {ceil['copy']['gbs_read_plus_write']} GB/s")

    achieved = head.ops() / (step_gemm_us * 1e-6) / 1e12
    roofline = {
        "bound": "mfma",
        "kernel": "k_gemm_big<W4> (DiT W1, M=4096 K=3072 N=12288)",
        "achieved": round(achieved, 2),
        "peak": PEAK_INT8_TOPS,
        "unit": "TOP/s",
        "frac": round(achieved / PEAK_INT8_TOPS, 4),
        "ceiling": ceil["mfma_i8_tops"] if ceil else None,
        "frac_of_ceiling": round(achieved / ceil["mfma_i8_tops"], 4) if ceil else None,
        "ceiling_note": "ceiling: int8 matrix-core probe of the library (register operands, no memory "
                        "traffic, 8 or 16 waves per CU, best), measured in this run at the chip's power limit",
        "traffic": load_traffic(khash),
        "algorithmic_bytes": head.gemm_bytes(),
        "avg_launch_us": round(step_gemm_us, 3),
        "graph_replay_us": round(hrow["gemm_us"], 3),
        "note": "int8 MFMA ops (2*M*N*K per launch) / the GEMM's average launch duration, from HIP "
                "events on the launch stream around each GEMM launch of K steps run right after the "
                "timed ones; unit: tera integer ops per second.  graph_replay_us: the same kernel over "
                "a replayed graph of back-to-back launches",
    }
    small = rows.get("te_gate_up_M76")
    small_m = None
    if small is not None:
        small_m = {
            "workload": "text-encoder gate/up W4A4, M=76 K=2560 N=9728, cold weights",
            "bound": "hbm",
            "weight_gbs": round(small["weight_gbs"], 1),
            "gemm_alg_gbs": round(small["gemm_alg_gbs"], 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(small["weight_gbs"] / PEAK_HBM_GBS, 4),
            "gemm_us": round(small["gemm_us"], 3),
            "linear_us": round(small["linear_us"], 3),
            "ceiling": ceil["cold_read"]["gbs"] if ceil else None,
            "frac_of_ceiling": round(small["weight_gbs"] / ceil["cold_read"]["gbs"], 4) if ceil else None,
            "floor_us": ceil["cold_read"]["us"] if ceil else None,
            "ceiling_note": "ceiling: one probe kernel of the library reading a cold 12.45 MB buffer (the "
                            "gate/up weight's size), cycled over 48 copies by graph replay like the GEMM",
        }

    cpu = None
    if not args.no_cpu_baseline:
        _log(f"cpu baseline on {args.cpu_rows} rows")
        cpu = cpu_baseline(Lh, args.cpu_rows)

    out = {
        "metric": "fused ConvRot W4A4 linear TOPS (% int8 MFMA peak) + small-M HBM GB/s",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded; shapes and distributions of the DiT image-token MLP W1)",
        "config": {
            "workload": "DiT image-token MLP W1, W4A4 ConvRot linear: x bf16 [4096,3072] Student-t(3) "
                        "with 1% outlier channels x50, W [12288,3072] N(0,0.02), bias, group 256",
            "M": head.M, "K": head.K, "N": head.N, "parallelism": "single GPU",
        },
        "roofline": roofline,
        "small_m": small_m,
        "cpu_baseline": cpu,
        "step_events_us": round(ev_ms * 1e3, 3),
        "clocks": {"sclk_mhz_after_headline": round(sclk_headline, 1) if sclk_headline else None,
                   "sclk_mhz_mfma_probe": ceil["mfma_i8_sclk_mhz"] if ceil else None,
                   "note": "shader clock from the probe kernels' cycle counter over the real-time "
                           "counter: right after the headline's event-timed steps (same stream), and "
                           "under the full-chip matrix-core probe"},
        "ceilings": ceil,
        "prewarm": {"ms": args.prewarm_ms, "steps": prewarm_steps},
        "rows": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                 for k, v in rows.items()},
        "kernel_sources_hash": khash,
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
