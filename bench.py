"""Benchmark of the SVDQuant W4A4 + rank-32 linear layer on one MI355X.

Workload: the FLUX.1 MLP pair at 1024x1024 (4096 image + 512 text tokens):
fc1 4608 x 3072 -> 12288 and fc2 4608 x 12288 -> 3072, both rank 32, INT4
groups of 64, bias.  One step runs both layers through the two fused kernels
each (quantize + down projection, then 4-bit GEMM + up projection).  The fc2
input is GELU(fc1 output) computed once before timing (not inside the step).

Inputs are synthetic (seeded FLUX-shaped activations with planted outlier
channels, random weights packed by the library's offline pack) and resident
in HBM; four copies of every buffer are rotated so that the 256 MB
Infinity Cache cannot hold a step's working set.

Prints one JSON line.  `value` is the whole step's effective throughput
(2*M*N*K summed over both layers / step time) in TOPS.  `roofline` is that
of the dominant kernel, the 4-bit GEMM + up projection: its algorithmic
ops (2*M*N*K, the same for fc1 and fc2) over its average launch time,
timed with HIP events on the stream the library launches on, against the
dense 8-bit matrix-core peak (int8 and fp8 run at the same rate).

The `mxfp4` object times the same two layers packed in MXFP4 (E2M1 codes,
E8M0 scales per 32 k) outside the timed step, against the dense FP4
matrix-core peak.  The `w4a16` object times the same weights as a 4-bit
weight-only layer (bf16 activations, one kernel) against the dense bf16
matrix-core peak, the comparison the pages quote W4A4 speedups against.

Each roofline object also carries `measured_ceiling`: the dense rate the
matrix core sustains here on independent MFMAs of the same instruction
(FP8, or FP4 for MXFP4), and the fraction of it achieved.

`--calibrate-copy` instead runs a plain elementwise copy of 1 GiB a few
times; its FETCH_SIZE / WRITE_SIZE counters give the factor that turns the
counters read on the GEMM into HBM bytes.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("fused W4A4+LoRA-r32 linear: µs/layer, TOPS & % INT8-MFMA roofline (FLUX MLP)")
EV_EVERY = 4          # timed steps per step that carries the per-layer events
INT8_PEAK_TOPS = 5033.0        # 256 CU x 2.4 GHz x 8192 int8/fp8 ops/clk/CU (dense)
FP4_PEAK_TOPS = 10066.0        # 256 CU x 2.4 GHz x 16384 fp4 ops/clk/CU (dense)
BF16_PEAK_TFLOPS = 2517.0      # 256 CU x 2.4 GHz x 4096 bf16 flops/clk/CU (dense)
HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "bit_quantized_diffusion_amd", "csrc", "svdq_kernels.hip")
TRAFFIC = os.path.join(ROOT, "profiles", "k2_gemm_int4_flux_mlp_hbm_traffic.md")
TRAFFIC_NOTE = ("rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, scaled by the elementwise-copy "
                "calibration (profiles/k2_gemm_int4_flux_mlp_hbm_traffic.md)")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha() -> str:
    with open(KERNEL_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--sets", type=int, default=4, help="rotated buffer sets")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ablation", action="store_true",
                   help="skip the fused-vs-unfused (four kernel) comparison")
    p.add_argument("--no-mxfp4", action="store_true", help="skip the MXFP4 timing of the same layers")
    p.add_argument("--no-mlp", action="store_true", help="skip the fused-MLP timing")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-config layer timings (QKV, fc1 r48, tiny, M=576 shares)")
    p.add_argument("--no-w4a16", action="store_true",
                   help="skip the W4A16 (4-bit weight, bf16 activation) comparison timing")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="time budget of the oracle sample (whole chunks of rows)")
    p.add_argument("--cpu-chunk", type=int, default=96, help="token rows per oracle chunk")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run a 1 GiB elementwise copy (counter calibration) and exit")
    return p.parse_args()


def calibrate_copy():
    """A plain copy of known size: 2^28 fp32 read and 2^28 fp32 written per
    launch (torch.neg into a second buffer, one elementwise kernel)."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "elementwise copy", "bytes_read_per_launch": 4 * n,
                      "bytes_written_per_launch": 4 * n, "launches": 5}), flush=True)


def read_traffic():
    """HBM bytes per GEMM launch from the committed counter summary, if it
    was taken on the current kernel source."""
    import re
    if not os.path.exists(TRAFFIC):
        return None, None
    text = open(TRAFFIC).read()
    sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != kernel_sha():
        return None, "stale" if sha else None
    return float(val.group(1)), "fresh"


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus above 1 is not supported "
                          "(token rows shard across GPUs with no exchange; see the design notes)"}))
        sys.exit(2)

    import numpy as np
    import torch

    import bit_quantized_diffusion_amd as bq
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if not bq.device_check(0):
        raise SystemExit(bq.status_string(bq.SVDQ_ERR_UNSUPPORTED_DEVICE))
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    def to_dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---------------- inputs and offline packs ----------------------------
    s1, s2 = synth.layer_spec("fc1"), synth.layer_spec("fc2")
    lay1 = synth.gen_layer(s1)
    x1 = to_dev_bf16(lay1["x"])
    ax1 = x1.float().abs().amax(dim=0).cpu().numpy().astype(np.float32)
    t0 = time.time()
    pk1 = bq.pack_weights(lay1["w"], ax1, s1.rank)
    pack_s = {"fc1": round(time.time() - t0, 2)}
    log(f"bench: packed fc1 ({s1.K}x{s1.N}, rank {s1.rank}) in {pack_s['fc1']:.1f} s")
    L1 = bq.PackedLinear.from_host(pk1, lay1["bias"], s1.rank, device=dev)
    y1 = bq.linear(x1, L1)
    x2 = torch.nn.functional.gelu(y1.float(), approximate="tanh").to(torch.bfloat16)
    ax2 = x2.float().abs().amax(dim=0).cpu().numpy().astype(np.float32)
    idx2 = np.sort(np.argsort(-ax2, kind="stable")[: s2.n_outliers])
    w2 = synth.gen_w(s2, idx2)
    t0 = time.time()
    pk2 = bq.pack_weights(w2, ax2, s2.rank)
    pack_s["fc2"] = round(time.time() - t0, 2)
    log(f"bench: packed fc2 ({s2.K}x{s2.N}, rank {s2.rank}) in {pack_s['fc2']:.1f} s")
    L2 = bq.PackedLinear.from_host(pk2, synth.gen_bias(s2), s2.rank, device=dev)
    torch.cuda.synchronize()

    M = s1.M

    def clone_layer(L):
        return bq.PackedLinear(L.K, L.N, L.rank, L.precision, L.smooth_inv.clone(),
                               L.lora_down.clone(), L.lora_up.clone(), L.wq.clone(), L.ws.clone(),
                               None if L.bias is None else L.bias.clone())

    def buffers(L, x):
        G = L.K // 64
        return dict(L=clone_layer(L), x=x.clone(),
                    xq=torch.empty((M, L.K // 2), dtype=torch.uint8, device=dev),
                    xs=torch.empty((G, M), dtype=torch.float16, device=dev),
                    la=torch.empty((M, L.rank), dtype=torch.float32, device=dev),
                    y=torch.empty((M, L.N), dtype=torch.bfloat16, device=dev))

    sets = [(buffers(L1, x1), buffers(L2, x2)) for _ in range(args.sets)]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    # HIP events on the library's stream, created before the timed region and
    # recorded on every EV_EVERY-th step only (the other steps run bare, so
    # that the markers cost the timed region little): one before the step,
    # one after each layer's kernel 1 and one after its kernel 2
    n_rec = (args.steps + EV_EVERY - 1) // EV_EVERY
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_rec)]
    ev = {"fc1": [], "fc2": []}

    def run_layer(b, e1=None, e2=None):
        L = b["L"]
        bq.quantize_act_lora_down(b["x"], L.smooth_inv, L.lora_down, L.rank, xq=b["xq"], xs=b["xs"],
                                  lora_act=b["la"])
        if e1 is not None:
            e1.record(stream)
        bq.gemm_w4a4_lora_up(b["xq"], b["xs"], L.wq, L.ws, b["la"], L.lora_up, L.bias, M, L.N, L.K,
                             L.rank, y=b["y"])
        if e2 is not None:
            e2.record(stream)

    def step(i, record):
        b1, b2 = sets[i % len(sets)]
        if record and i % EV_EVERY == 0:
            m = marks[i // EV_EVERY]
            m[0].record(stream)
            run_layer(b1, m[1], m[2])
            run_layer(b2, m[3], m[4])
        else:
            run_layer(b1)
            run_layer(b2)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    log(f"bench: warmup {args.warmup} steps done")

    # timed region: host clock around exactly `steps` steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"bench: timed {args.steps} steps in {elapsed * 1e3:.2f} ms")
    for m in marks:
        ev["fc1"].append((m[0], m[1], m[2]))
        ev["fc2"].append((m[2], m[3], m[4]))

    def avg_us(tag, a, b):
        return 1e3 * float(np.mean([x[a].elapsed_time(x[b]) for x in ev[tag]]))

    per = {}
    ops_total = 0.0
    for tag, s in (("fc1", s1), ("fc2", s2)):
        k1 = avg_us(tag, 0, 1)
        k2 = avg_us(tag, 1, 2)
        ops = 2.0 * s.M * s.N * s.K
        ops_total += ops
        per[tag] = {"M": s.M, "K": s.K, "N": s.N, "rank": s.rank,
                    "us_k1": round(k1, 2), "us_k2": round(k2, 2), "us_layer": round(k1 + k2, 2),
                    "tops": round(ops / ((k1 + k2) * 1e-6) / 1e12, 1),
                    "pct_int8_roofline": round(100 * ops / ((k1 + k2) * 1e-6) / 1e12 / INT8_PEAK_TOPS, 2)}
    ms_per_step = elapsed * 1e3 / args.steps
    value = ops_total / (ms_per_step * 1e-3) / 1e12

    # roofline of the dominant kernel: the 4-bit GEMM + up projection, over
    # all its launches (fc1 and fc2 carry the same 2*M*N*K)
    k2_us = float(np.mean([x[1].elapsed_time(x[2]) for t in ("fc1", "fc2") for x in ev[t]])) * 1e3
    k2_ops = 2.0 * s1.M * s1.N * s1.K
    assert k2_ops == 2.0 * s2.M * s2.N * s2.K
    achieved = k2_ops / (k2_us * 1e-6) / 1e12
    traffic, traffic_state = read_traffic()
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS,
                "unit": "TFLOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": traffic,
                "kernel": "k2_gemm_int4 (fc1 4608x3072->12288 and fc2 4608x12288->3072)",
                "avg_launch_us": round(k2_us, 2), "ops_per_launch": k2_ops,
                "peak_basis": "dense int8/fp8 matrix-core rate, 256 CU x 2.4 GHz x 8192 ops/clk",
                "traffic_source": TRAFFIC_NOTE if traffic is not None else
                ("counter summary taken on older kernel source" if traffic_state == "stale" else None)}

    ceil8 = mfma_ceiling(bq, torch, stream, bq.INT4)
    roofline["measured_ceiling"] = ceil8
    roofline["frac_of_measured_ceiling"] = round(achieved / ceil8["tops"], 4)

    ablation = None
    if not args.no_ablation:
        ablation = fusion_ablation(bq, torch, np, sets, M, (s1, s2), per, stream, reps=10)

    mlp = None
    if not args.no_mlp:
        mlp = mlp_fusion(bq, torch, np, sets, M, stream, reps=10)

    mx = None
    if not args.no_mxfp4:
        mx = mxfp4_layers(bq, torch, np, dev, (s1, s2), (lay1["w"], w2), (ax1, ax2),
                          (lay1["bias"], synth.gen_bias(s2)), (x1, x2), args.sets, stream, reps=20)
        ceil4 = mfma_ceiling(bq, torch, stream, bq.MXFP4)
        mx["roofline"]["measured_ceiling"] = ceil4
        mx["roofline"]["frac_of_measured_ceiling"] = round(mx["roofline"]["achieved"] / ceil4["tops"], 4)

    w16 = None
    if not args.no_w4a16:
        w16 = w4a16_layers(bq, torch, np, dev, (s1, s2), (lay1["w"], w2), (lay1["bias"], synth.gen_bias(s2)),
                           (x1, x2), args.sets, stream, per, reps=20)

    configs = None
    if not args.no_configs:
        configs = config_lines(bq, torch, np, dev, synth, stream, pk1, lay1, (L1, x1), (L2, x2))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(lay1, pk1, s1, args.cpu_seconds, args.cpu_chunk)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int4",
        "data": "synthetic",
        "config": {"workload": "FLUX.1 MLP pair at 1024x1024: fc1 4608x3072->12288 + fc2 4608x12288->3072, "
                               "rank 32, int4 g64 W4A4, bf16 in/out, bias",
                   "M": s1.M, "layers": per, "rotated_sets": args.sets, "parallelism": "single GPU"},
        "us_per_layer": {k: v["us_layer"] for k, v in per.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fusion_ablation": ablation,
        "mxfp4": mx,
        "mlp_fusion": mlp,
        "w4a16": w16,
        "configs": configs,
        "offline_pack_s": pack_s,
    }
    print(json.dumps(out), flush=True)


def layer_bytes(M, K, N, r, bias=True):
    """Algorithmic HBM bytes of one layer: fused (two kernels) and unfused
    (quantize, down projection, 4-bit GEMM, up projection)."""
    x, sinv, l1, l2 = M * K * 2, K * 4, r * K * 2, N * r * 2
    xq, xs, wq, ws, la = M * K // 2, (K // 64) * M * 2, N * K // 2, (K // 64) * N * 2, M * r * 4
    b, y = (N * 2 if bias else 0), M * N * 2
    k1 = x + sinv + l1 + xq + xs + la
    k2 = xq + xs + wq + ws + la + l2 + b + y
    quant = x + sinv + xq + xs
    down = x + sinv + l1 + la
    gemm = xq + xs + wq + ws + y
    up = la + l2 + b + y + y
    return k1 + k2, quant + down + gemm + up


def fusion_ablation(bq, torch, np, sets, M, specs, per, stream, reps):
    """Times the unfused four-kernel layer on the same buffers as the fused
    one (outside the timed step), next to the fused per-layer times."""
    out = {}
    for li, (tag, s) in enumerate(zip(("fc1", "fc2"), specs)):
        for i in range(3):
            b = sets[i % len(sets)][li]
            bq.unfused_linear(b["x"], b["L"], y=b["y"], xq=b["xq"], xs=b["xs"], lora_act=b["la"])
        torch.cuda.synchronize()
        evs = []
        for i in range(reps):
            b = sets[i % len(sets)][li]
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            bq.unfused_linear(b["x"], b["L"], y=b["y"], xq=b["xq"], xs=b["xs"], lora_act=b["la"])
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        us_unfused = 1e3 * float(np.mean([a.elapsed_time(c) for a, c in evs]))
        fused_b, unfused_b = layer_bytes(s.M, s.K, s.N, s.rank)
        us_fused = per[tag]["us_layer"]
        out[tag] = {"us_fused": us_fused, "us_unfused": round(us_unfused, 2),
                    "unfused_over_fused": round(us_unfused / us_fused, 3),
                    "algorithmic_mb_fused": round(fused_b / 1e6, 1),
                    "algorithmic_mb_unfused": round(unfused_b / 1e6, 1),
                    "mb_saved_by_fusion": round((unfused_b - fused_b) / 1e6, 1)}
    log(f"bench: fusion ablation {json.dumps(out)}")
    return out


def mlp_fusion(bq, torch, np, sets, M, stream, reps):
    """The MLP pair fc2(GELU(fc1(x))) two ways, outside the timed step, on
    the same buffers: GELU fused into fc1's GEMM epilogue with X2 written and
    read back by fc2's first kernel (4 launches), and GELU plus fc2's first
    kernel fused into fc1's GEMM epilogue (3 launches, no X2 in memory)."""
    def gelu_path(b1, b2):
        L1, L2 = b1["L"], b2["L"]
        bq.quantize_act_lora_down(b1["x"], L1.smooth_inv, L1.lora_down, L1.rank, xq=b1["xq"], xs=b1["xs"],
                                  lora_act=b1["la"])
        bq.gemm_w4a4_lora_up_gelu(b1["xq"], b1["xs"], L1.wq, L1.ws, b1["la"], L1.lora_up, L1.bias, M, L1.N, L1.K,
                                  L1.rank, y=b1["y"])
        bq.quantize_act_lora_down(b1["y"], L2.smooth_inv, L2.lora_down, L2.rank, xq=b2["xq"], xs=b2["xs"],
                                  lora_act=b2["la"])
        bq.gemm_w4a4_lora_up(b2["xq"], b2["xs"], L2.wq, L2.ws, b2["la"], L2.lora_up, L2.bias, M, L2.N, L2.K,
                             L2.rank, y=b2["y"])

    def fused_path(b1, b2):
        L1, L2 = b1["L"], b2["L"]
        bq.quantize_act_lora_down(b1["x"], L1.smooth_inv, L1.lora_down, L1.rank, xq=b1["xq"], xs=b1["xs"],
                                  lora_act=b1["la"])
        bq.mlp_gemm_gelu_quant(b1["xq"], b1["xs"], L1.wq, L1.ws, b1["la"], L1.lora_up, L1.bias, M, L1.N, L1.K,
                               L1.rank, L2.smooth_inv, L2.lora_down, L2.rank, xq2=b2["xq"], xs2=b2["xs"],
                               lora_act2=b2["la"])
        bq.gemm_w4a4_lora_up(b2["xq"], b2["xs"], L2.wq, L2.ws, b2["la"], L2.lora_up, L2.bias, M, L2.N, L2.K,
                             L2.rank, y=b2["y"])

    out = {}
    for name, fn in (("gelu_in_fc1_epilogue_us", gelu_path), ("gelu_and_fc2_kernel1_in_fc1_epilogue_us", fused_path)):
        for i in range(3):
            fn(*sets[i % len(sets)])
        torch.cuda.synchronize()
        evs = []
        for i in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(*sets[i % len(sets)])
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        out[name] = round(1e3 * float(np.mean([a.elapsed_time(b) for a, b in evs])), 2)
    out["speedup"] = round(out["gelu_in_fc1_epilogue_us"] / out["gelu_and_fc2_kernel1_in_fc1_epilogue_us"], 3)
    out["note"] = "MLP pair fc1 4608x3072->12288, GELU(tanh), fc2 12288->3072, both rank 32, INT4"
    log(f"bench: mlp fusion {json.dumps(out)}")
    return out


def mxfp4_layers(bq, torch, np, dev, specs, ws, axs, biases, xs, n_sets, stream, reps):
    """The same fc1 / fc2 layers (same weights, activations and bias) packed
    in MXFP4; both kernels timed per launch with HIP events on the library's
    stream, over rotated buffer sets, outside the timed step."""
    out = {}
    k2_all = []
    for tag, s, w, ax, bias, x in zip(("fc1", "fc2"), specs, ws, axs, biases, xs):
        pk = bq.pack_weights(w, ax, s.rank, precision=bq.MXFP4)
        L = bq.PackedLinear.from_host(pk, bias, s.rank, precision=bq.MXFP4, device=dev)
        sets = []
        for _ in range(n_sets):
            sets.append(dict(x=x.clone(), wq=L.wq.clone(), ws=L.ws.clone(),
                             xq=torch.empty((s.M, s.K // 2), dtype=torch.uint8, device=dev),
                             xs=torch.empty((s.K // 32, s.M), dtype=torch.uint8, device=dev),
                             la=torch.empty((s.M, s.rank), dtype=torch.float32, device=dev),
                             y=torch.empty((s.M, s.N), dtype=torch.bfloat16, device=dev)))

        def run(b, record, evs):
            if record:
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                gpu_lead(torch)
                e[0].record(stream)
            bq.quantize_act_lora_down(b["x"], L.smooth_inv, L.lora_down, s.rank, bq.MXFP4, xq=b["xq"], xs=b["xs"],
                                      lora_act=b["la"])
            if record:
                e[1].record(stream)
            bq.gemm_w4a4_lora_up(b["xq"], b["xs"], b["wq"], b["ws"], b["la"], L.lora_up, L.bias, s.M, s.N, s.K,
                                 s.rank, bq.MXFP4, y=b["y"])
            if record:
                e[2].record(stream)
                evs.append(e)

        for i in range(3):
            run(sets[i % n_sets], False, None)
        torch.cuda.synchronize()
        evs = []
        for i in range(reps):
            run(sets[i % n_sets], True, evs)
        torch.cuda.synchronize()
        k1 = 1e3 * float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        k2 = 1e3 * float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        k2_all += [e[1].elapsed_time(e[2]) for e in evs]
        ops = 2.0 * s.M * s.N * s.K
        out[tag] = {"us_k1": round(k1, 2), "us_k2": round(k2, 2), "us_layer": round(k1 + k2, 2),
                    "tops": round(ops / ((k1 + k2) * 1e-6) / 1e12, 1),
                    "pct_fp4_roofline": round(100 * ops / ((k1 + k2) * 1e-6) / 1e12 / FP4_PEAK_TOPS, 2)}
        del sets
    k2_us = 1e3 * float(np.mean(k2_all))
    ops = 2.0 * specs[0].M * specs[0].N * specs[0].K
    achieved = ops / (k2_us * 1e-6) / 1e12
    out["roofline"] = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP4_PEAK_TOPS, "unit": "TFLOP/s",
                       "frac": round(achieved / FP4_PEAK_TOPS, 4), "kernel": "k2_gemm_mxfp4 (fc1 and fc2)",
                       "avg_launch_us": round(k2_us, 2),
                       "peak_basis": "dense fp4 matrix-core rate, 256 CU x 2.4 GHz x 16384 ops/clk"}
    log(f"bench: mxfp4 {json.dumps(out)}")
    return out


def w4a16_layers(bq, torch, np, dev, specs, ws, biases, xs, n_sets, stream, per, reps):
    """The same fc1 / fc2 weights as W4A16 (INT4 codes, fp16 scales per 64 k,
    bf16 activations, no smoothing or low-rank branch): one kernel per layer,
    timed per launch with HIP events on the library's stream over rotated
    buffer sets, outside the timed step.  `w4a4_speedup` = W4A16 time over
    the fused W4A4 layer's time (both kernels) from the timed step.  A plain
    bf16 torch.matmul of the unquantized weights is timed beside it for
    context."""
    out = {}
    k_all = []
    for tag, s, w, bias, x in zip(("fc1", "fc2"), specs, ws, biases, xs):
        wq, wsc = bq.pack_w4a16(w)
        b = torch.from_numpy(np.ascontiguousarray(bias).view(np.int16)).view(torch.bfloat16).to(dev)
        wd = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).view(torch.bfloat16).to(dev)
        sets = []
        for _ in range(n_sets):
            sets.append(dict(x=x.clone(), wq=torch.from_numpy(wq).to(dev), ws=torch.from_numpy(wsc).to(dev),
                             w=wd.clone(), y=torch.empty((s.M, s.N), dtype=torch.bfloat16, device=dev)))
        del wd

        def run(bset, kind):
            if kind == "w4a16":
                bq.gemm_w4a16(bset["x"], bset["wq"], bset["ws"], b, s.N, y=bset["y"])
            else:
                torch.addmm(b, bset["x"], bset["w"].t(), out=bset["y"])

        res = {}
        for kind in ("w4a16", "bf16"):
            for i in range(3):
                run(sets[i % n_sets], kind)
            torch.cuda.synchronize()
            evs = []
            for i in range(reps):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record(stream)
                run(sets[i % n_sets], kind)
                e[1].record(stream)
                evs.append(e)
            torch.cuda.synchronize()
            res[kind] = [e[0].elapsed_time(e[1]) for e in evs]
        k_all += res["w4a16"]
        us = 1e3 * float(np.mean(res["w4a16"]))
        us_bf16 = 1e3 * float(np.mean(res["bf16"]))
        ops = 2.0 * s.M * s.N * s.K
        out[tag] = {"us_layer": round(us, 2), "tops": round(ops / (us * 1e-6) / 1e12, 1),
                    "w4a4_speedup": round(us / per[tag]["us_layer"], 3),
                    "us_bf16_torch_matmul": round(us_bf16, 2)}
        del sets
    us = 1e3 * float(np.mean(k_all))
    ops = 2.0 * specs[0].M * specs[0].N * specs[0].K
    achieved = ops / (us * 1e-6) / 1e12
    out["roofline"] = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                       "kernel": "k2_gemm_w4a16 (fc1 and fc2)", "avg_launch_us": round(us, 2),
                       "peak_basis": "dense bf16 matrix-core rate, 256 CU x 2.4 GHz x 4096 flops/clk"}
    log(f"bench: w4a16 {json.dumps(out)}")
    return out


def mfma_ceiling(bq, torch, stream, precision, reps=3):
    """Dense matrix-core rate this GPU sustains: svdq_bench_mfma_ceiling
    (independent 32x32x64 scaled MFMAs, FP8 or FP4 operands, 2 waves per
    SIMD), timed with HIP events on the library's stream."""
    ops, out = bq.mfma_ceiling(precision)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        bq.mfma_ceiling(precision, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    tops = ops / min(ts) / 1e12
    name = "FP8" if precision == bq.INT4 else "FP4"
    res = {"tops": round(tops, 1), "kernel": f"k_mfma_ceiling ({name} 32x32x64 scaled MFMA, 8 independent "
                                             "accumulators per wave, 2 waves per SIMD)"}
    log(f"bench: measured {name} matrix-core ceiling {res['tops']} TOPS")
    return res


def gpu_lead(torch, us=300):
    """Queue a short spin kernel on the current stream, so that the GPU is
    still busy while the host enqueues the timed calls after it: the event
    intervals then hold device time only, not host launch gaps (a layer whose
    kernels run shorter than the Python call overhead would otherwise show
    the host's pace)."""
    torch.cuda._sleep(int(us * 2400))


def time_layer(bq, torch, np, stream, L, xs_list, M, reps):
    """Mean K1 and K2 times (HIP events on the library's stream) of the INT4
    layer L over `reps` calls rotating through the inputs xs_list."""
    dev = xs_list[0].device
    G = L.K // 64
    bufs = [dict(x=x, xq=torch.empty((M, L.K // 2), dtype=torch.uint8, device=dev),
                 xs=torch.empty((G, M), dtype=torch.float16, device=dev),
                 la=torch.empty((M, L.rank), dtype=torch.float32, device=dev),
                 y=torch.empty((M, L.N), dtype=torch.bfloat16, device=dev)) for x in xs_list]

    def call(b):
        bq.quantize_act_lora_down(b["x"], L.smooth_inv, L.lora_down, L.rank, xq=b["xq"], xs=b["xs"], lora_act=b["la"])
        bq.gemm_w4a4_lora_up(b["xq"], b["xs"], L.wq, L.ws, b["la"], L.lora_up, L.bias, M, L.N, L.K, L.rank, y=b["y"])

    for i in range(3):
        call(bufs[i % len(bufs)])
    torch.cuda.synchronize()
    evs = []
    for i in range(reps):
        b = bufs[i % len(bufs)]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        gpu_lead(torch)
        e[0].record(stream)
        bq.quantize_act_lora_down(b["x"], L.smooth_inv, L.lora_down, L.rank, xq=b["xq"], xs=b["xs"], lora_act=b["la"])
        e[1].record(stream)
        bq.gemm_w4a4_lora_up(b["xq"], b["xs"], L.wq, L.ws, b["la"], L.lora_up, L.bias, M, L.N, L.K, L.rank, y=b["y"])
        e[2].record(stream)
        evs.append(e)
    torch.cuda.synchronize()
    k1 = [1e3 * e[0].elapsed_time(e[1]) for e in evs]
    k2 = [1e3 * e[1].elapsed_time(e[2]) for e in evs]
    lay = [a + b for a, b in zip(k1, k2)]
    ops = 2.0 * M * L.N * L.K
    us = float(np.mean(lay))
    return {"M": M, "K": L.K, "N": L.N, "rank": L.rank, "us_k1": round(float(np.mean(k1)), 2),
            "us_k2": round(float(np.mean(k2)), 2), "us_layer": round(us, 2),
            "us_layer_median": round(float(np.median(lay)), 2),
            "tops": round(ops / (us * 1e-6) / 1e12, 1),
            "pct_int8_roofline": round(100 * ops / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 2)}


def config_lines(bq, torch, np, dev, synth, stream, pk1, lay1, fc1, fc2):
    """The other configurations one GPU can show, timed outside the step:
    the fused QKV projection (4608x3072->9216, rank 32), fc1 with a rank-16
    LoRA merged into its branch (rank 48), the tiny case (256x512->512, rank
    16), and fc1 / fc2 at M = 576 (the token rows one of eight GPUs holds
    when the 4608 rows are split).  Each call is timed on the device behind a
    spin kernel (gpu_lead), so short layers report kernel time, not the
    host's launch pace; the median over calls is reported beside the mean."""
    out = {}

    def to_dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # C1: fused QKV
    sq = synth.layer_spec("qkv")
    lq = synth.gen_layer(sq)
    xq_ = to_dev_bf16(lq["x"])
    axq = xq_.float().abs().amax(dim=0).cpu().numpy().astype(np.float32)
    Lq = bq.PackedLinear.from_host(bq.pack_weights(lq["w"], axq, sq.rank), lq["bias"], sq.rank, device=dev)
    out["qkv"] = time_layer(bq, torch, np, stream, Lq, [xq_, xq_.clone()], sq.M, reps=20)
    del Lq, xq_
    # C3: fc1 + rank-16 LoRA merged (rank 48)
    sl = synth.layer_spec("fc1_lora")
    a_bits, b_bits = synth.gen_lora(sl)
    down, up = bq.merge_lora(pk1["lora_down"], pk1["lora_up"], pk1["smooth_inv"], a_bits, b_bits)
    pk48 = dict(pk1, lora_down=down, lora_up=up)
    L48 = bq.PackedLinear.from_host(pk48, lay1["bias"], down.shape[0], device=dev)
    x1 = fc1[1]
    out["fc1_lora_r48"] = time_layer(bq, torch, np, stream, L48, [x1, x1.clone()], x1.shape[0], reps=20)
    del L48
    # C0: tiny
    st = synth.layer_spec("tiny")
    lt = synth.gen_layer(st)
    xt = to_dev_bf16(lt["x"])
    axt = xt.float().abs().amax(dim=0).cpu().numpy().astype(np.float32)
    Lt = bq.PackedLinear.from_host(bq.pack_weights(lt["w"], axt, st.rank), lt["bias"], st.rank, device=dev)
    out["tiny"] = time_layer(bq, torch, np, stream, Lt, [xt], st.M, reps=50)
    # per-GPU share of the MLP pair
    for tag, (L, x) in (("fc1_m576", fc1), ("fc2_m576", fc2)):
        xs_ = [x[:576].contiguous(), x[576:1152].contiguous()]
        out[tag] = time_layer(bq, torch, np, stream, L, xs_, 576, reps=30)
    log(f"bench: configs {json.dumps(out)}")
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_tiny(reps=5):
    """The oracle's online path on the whole tiny case (256x512->512, rank
    16): median of `reps` runs on all threads, and one run on one thread."""
    import numpy as np
    import oracle as O
    import synth
    st = synth.layer_spec("tiny")
    lt = synth.gen_layer(st)
    ax = np.abs(O.bf16_bits_to_f32(lt["x"])).max(axis=0).astype(np.float32)
    pk = O.pack_weights(lt["w"], ax, st.rank)

    def once():
        t0 = time.perf_counter()
        a = O.quantize_act_lora_down(lt["x"], pk["smooth_inv"], pk["l1"])
        O.gemm_w4a4_lora_up(a["xq"], a["xs"], pk["wq"], pk["ws"], a["t"], pk["l2"], lt["bias"])
        return time.perf_counter() - t0

    ts = sorted(once() for _ in range(reps))
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            one = once()
    except Exception:
        pass
    return {"us_median_of_5_all_threads": round(ts[len(ts) // 2] * 1e6, 1),
            "us_one_thread": None if one is None else round(one * 1e6, 1)}


def cpu_baseline(lay1, pk1, spec, seconds, chunk):
    """The oracle's online path (both fused kernels' steps) on whole chunks
    of fc1 token rows, spread over the token range, until `seconds` of host
    time are spent; scaled to TOPS."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    l1 = np.ascontiguousarray(pk1["lora_down"].T)
    l2 = np.ascontiguousarray(pk1["lora_up"].T)
    n_chunks = spec.M // chunk
    order = np.random.default_rng(0).permutation(n_chunks)
    rows = 0
    t0 = time.perf_counter()
    for c in order:
        x = np.ascontiguousarray(lay1["x"][c * chunk:(c + 1) * chunk])
        a = O.quantize_act_lora_down(x, pk1["smooth_inv"], l1)
        O.gemm_w4a4_lora_up(a["xq"], a["xs"], pk1["wq"], pk1["ws"], a["t"], l2, lay1["bias"])
        rows += chunk
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    ops = 2.0 * rows * spec.N * spec.K
    log(f"bench: cpu oracle {rows} rows of fc1 in {dt:.1f} s")
    tiny = cpu_tiny()
    log(f"bench: cpu oracle tiny case {json.dumps(tiny)}")
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "tiny_case": tiny,
            "sample": f"{rows} of {spec.M} token rows of fc1 ({spec.K}->{spec.N}, rank {spec.rank}) in "
                      f"chunks of {chunk}: quantize+down and per-group GEMM+up, {dt:.1f} s",
            "us_per_layer_equiv": round(dt / rows * spec.M * 1e6, 1)}


if __name__ == "__main__":
    main()
