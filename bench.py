#!/usr/bin/env python3
"""Bench: packed-weight HBM GB/s (and % of the 8 TB/s peak) plus decode tok/s-equivalent of the
27B-shaped Q1_0_g128 decode-step weight stream at batch 1 on one MI355X.

A step is one decode step of the whole stream: 64 layers x (q, o 5120x5120; k, v 1024x5120;
gate, up 17408x5120; down 5120x17408) Q1_0_g128 GEMVs with the RMS rescales between them
(lbq_decode_step_q1g128), over seeded synthetic weights (sign bits Bernoulli(0.5), fp16 scales
|N(0, 0.02)|) and a bf16 N(0, 1) input, all resident in HBM before timing starts. At batch 1 a
step is two stage-kernel launches per layer and a final one; larger batches run the
per-projection launches. Either is captured once in a HIP graph and replayed (--no-graph runs it
eagerly). W untimed warm-up steps precede exactly K timed steps bracketed by device
synchronisation.

With --gemm the bench times the many-row products on the matrix cores instead (prefill and
large batch: Q1 MLP and INT4 layer shapes at 32, 128 and 512 activation rows) and reports
TFLOP/s against the bf16 matrix-core peak. With --i4-layer it times the seven projections of a
Qwen3-8B-shaped INT4 g128 layer at B = 1 and 8 through the bf16-activation GEMV and the
int8-activation GEMV (integer dot products) and reports packed-weight GB/s against HBM. With
--z80-chat it times the Z80-uLM character loop (1024 prompts, replies of up to 32 characters,
one launch) and reports generated characters per second. With --tern-layer it times the seven
projections of one 27B-shaped layer with ternary g160 weights (1.7 bits per weight) at B = 1
and 8 and reports packed-weight GB/s against HBM.

Printed: one JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "q1_stage_decode_64L.md")
I4_PROFILE = os.path.join(ROOT, "profiles", "i4_layer_gemv.md")
TERN_PROFILE = os.path.join(ROOT, "profiles", "tern_layer_gemv.md")
I4_KERNELS = [os.path.join(ROOT, "packed_weight_gemv_amd", "csrc", f)
              for f in ("lbq_kernels.hip", "lbq_q1mb.hip")]
STEP_SOURCES = [os.path.join(ROOT, "packed_weight_gemv_amd", "csrc", f)
                for f in ("lbq_stage.hip", "lbq_internal.h")]


def measured_traffic(layers: int, batch: int):
    """HBM bytes per decode step from the committed PMC summary (FETCH_SIZE + WRITE_SIZE summed
    over the step's launches, each scaled by a plain copy of known size), or None when the
    stage-kernel sources changed since it was taken or the workload differs from the profiled
    one (64 layers, batch 1)."""
    import hashlib
    if layers != 64 or batch != 1 or not os.path.exists(TRAFFIC_PROFILE):
        return None
    h = hashlib.sha256()
    for f in STEP_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    sha, traffic = None, None
    with open(TRAFFIC_PROFILE) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("step-source-sha256:"):
                sha = line.split(":", 1)[1].strip()
            elif line.startswith("traffic-bytes-per-step:"):
                traffic = int(line.split(":", 1)[1].strip())
    return traffic if sha == h.hexdigest() else None


def i4_layer_traffic(key: str, profile: str = None):
    """HBM bytes per layer of the layer GEMVs (`key` like "i8act-B1") from a committed PMC
    summary, or None when the kernel sources changed since it was taken."""
    import hashlib
    profile = profile or I4_PROFILE
    if not os.path.exists(profile):
        return None
    h = hashlib.sha256()
    for f in I4_KERNELS:
        with open(f, "rb") as fh:
            h.update(fh.read())
    cur = h.hexdigest()
    sha, traffic = None, None
    with open(profile) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("kernels-source-sha256:"):
                sha = line.split(":", 1)[1].strip()
            elif line.startswith(f"traffic-bytes-per-layer-{key}:"):
                traffic = int(line.split(":", 1)[1].strip())
    return traffic if sha == cur else None


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_cpu():
    """(cores this process may run on, CPU model name from /proc/cpuinfo)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def oracle_rows(fn, signs, scales, x, n, threads, rows=None):
    """The oracle GEMV `fn` over `rows` (default: all n) split across `threads` host threads (the
    oracle is a plain C function; ctypes releases the interpreter lock while it runs). Returns
    (y, l1) as the oracle does."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    rows = np.arange(n, dtype=np.int32) if rows is None else np.asarray(rows, dtype=np.int32)
    chunks = [c for c in np.array_split(rows, max(1, min(threads, rows.size))) if c.size]
    with ThreadPoolExecutor(len(chunks)) as ex:
        res = list(ex.map(lambda r: fn(signs, scales, x, rows=r), chunks))
    return (np.concatenate([r[0] for r in res], axis=1),
            np.concatenate([r[1] for r in res], axis=1))


def hbm_achievable(torch, lbq, dev, gib: int = 4):
    """Best read bandwidth (GB/s) of the streaming-read probe over a `gib` GiB buffer (best of
    several workgroup counts, three passes each), the reference for "% of achievable HBM"."""
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    best = 0.0
    for wgs in (1024, 2048, 4096, 8192):
        lbq.lbq_hbm_read_probe(buf, sink, wgs)
        torch.cuda.synchronize()
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            lbq.lbq_hbm_read_probe(buf, sink, wgs)
            e1.record()
            torch.cuda.synchronize()
            best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf, sink
    torch.cuda.empty_cache()
    return best


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--no-graph", action="store_true", help="launch steps eagerly")
    ap.add_argument("--cpu-layers", type=int, default=40,
                    help="layers of the stream the CPU oracle baseline runs on all host cores "
                         "(0 = skip the baseline, the sampled parity and the chain check)")
    ap.add_argument("--rounds", type=int, default=3,
                    help="extra timed rounds of --steps steps each (min and median reported)")
    ap.add_argument("--no-chain", action="store_true",
                    help="skip the oracle chain over all layers (batch 1) and its cosine")
    ap.add_argument("--no-hbm-probe", action="store_true",
                    help="skip the 4 GiB streaming-read reference of achievable bandwidth")
    ap.add_argument("--kernel-steps", type=int, default=3,
                    help="instrumented steps timing each GEMV launch with HIP events")
    ap.add_argument("--q1-gemv", action="store_true",
                    help="time single Q1_0_g128 GEMVs instead: 5120x5120 at batch 1, and gate/up "
                         "17408x5120 and down 5120x17408 at batch 1, 4 and 16")
    ap.add_argument("--mlp2bit", action="store_true",
                    help="time the 2-bit integer MLP (1024 vectors through 256-192-128-40) instead")
    ap.add_argument("--tern-layer", action="store_true",
                    help="time the ternary g160 GEMVs of one 27B-shaped layer instead")
    ap.add_argument("--z80-chat", action="store_true",
                    help="time the Z80-uLM character loop (1024 prompts, replies up to 32) instead")
    ap.add_argument("--i4-layer", action="store_true",
                    help="time the INT4 layer GEMVs (float and int8-activation paths) instead")
    ap.add_argument("--gemm", action="store_true",
                    help="instead of the decode step, time the many-row products on the matrix "
                         "cores (Q1 MLP and INT4 layer shapes, 32 to 512 activation rows)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the reference for "
                         "scaling HBM byte counters), then exit")
    return ap.parse_args()


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sharding is described in DESIGN.md); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n,
                          "bytes_written_per_copy": n, "copies": 5}), flush=True)
        return 0

    from packed_weight_gemv_amd import build as lbq_build
    if not os.path.exists(lbq_build.LIB):
        import __graft_entry__
        __graft_entry__.build()
    import packed_weight_gemv_amd as lbq
    from packed_weight_gemv_amd import synth

    lbq.load()
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), CUs {props.multi_processor_count}")
    if args.gemm:
        return gemm_bench(args, lbq, synth, torch, np, dev)
    if args.i4_layer:
        return i4_layer_bench(args, lbq, synth, torch, np, dev)
    if args.z80_chat:
        return chat_bench(args, lbq, synth, torch, np, dev)
    if args.tern_layer:
        return tern_layer_bench(args, lbq, synth, torch, np, dev)
    if args.q1_gemv:
        return q1_gemv_bench(args, lbq, synth, torch, np, dev)
    if args.mlp2bit:
        return mlp2bit_bench(args, lbq, synth, torch, np, dev)

    L, B = args.layers, args.batch
    hid, kv, ffn = synth.STREAM_HIDDEN, synth.STREAM_KV, synth.STREAM_FFN
    shapes = {nm: synth.stream_shape(nm) for nm in synth.STREAM_MATRICES}
    bytes_per_layer = synth.stream_bytes_per_layer()
    bytes_per_step = bytes_per_layer * L

    # ---- weights resident in HBM -------------------------------------------------------------
    t0 = time.time()
    layers = []
    for l in range(L):
        d = {}
        for nm in synth.STREAM_MATRICES:
            m = synth.stream_matrix(l, nm)
            d[nm] = torch.from_numpy(lbq.lbq_pack_q1g128(m.signs, m.scales)).to(dev)
        layers.append(d)
        if l % 8 == 7 or l == L - 1:
            log(f"packed and uploaded {l + 1}/{L} layers ({time.time() - t0:.1f} s)")
    arr = lbq.make_layers(layers)
    x0_np = synth.activations(B, hid, workload=synth.W_Q1_STREAM)
    x0 = torch.from_numpy(x0_np.view(np.int16)).to(dev)
    act = torch.zeros(lbq.lbq_decode_act_elems(L, hid, kv, ffn, B), dtype=torch.int16, device=dev)

    def step():
        lbq.lbq_decode_step_q1g128(arr, L, hid, kv, ffn, x0, act)

    # ---- warm-up, graph capture, timed steps -------------------------------------------------
    # warm-up runs on the stream the graph is captured on: the library's per-stream workspace
    # is allocated by the first call on a stream, which cannot happen inside a capture
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for _ in range(max(1, args.warmup)):
            step()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            step()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
    run = graph.replay if graph is not None else step
    log(f"timing {args.steps} steps ({'graph' if graph is not None else 'eager'})")
    # every step is bracketed by its own event pair on the launch stream, inside the timed
    # region: at batch 1 a step is the 2 x layers + 1 stage-kernel launches and nothing else, so
    # these give the step's kernel time
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        evs[i][0].record(stream)
        run()
        evs[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    gbs = bytes_per_step / (ms * 1e-3) / 1e9
    step_kernel_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    # further rounds of K steps each, after the timed region (run-to-run spread)
    round_ms = []
    for _ in range(max(0, args.rounds)):
        r0 = torch.cuda.Event(enable_timing=True)
        r1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        r0.record(stream)
        for _ in range(args.steps):
            run()
        r1.record(stream)
        torch.cuda.synchronize()
        round_ms.append(r0.elapsed_time(r1) / args.steps)
    achievable = None if args.no_hbm_probe else hbm_achievable(torch, lbq, dev)
    if achievable:
        log(f"achievable HBM read bandwidth (4 GiB streaming read): {achievable:.0f} GB/s")

    # ---- dominant kernel ---------------------------------------------------------------------
    if B == 1:
        kern_name = ("stage_kernel (whole decode step: two launches per layer and a final one, "
                     f"{2 * L + 1} launches)")
        kern_avg_ms, kern_bytes = step_kernel_ms, bytes_per_step
    else:
        # batched step: each projection's GEMV timed on its own, as a HIP graph of back-to-back
        # calls over different layers' weights (so every call streams its weights from HBM and
        # no host gap falls between the launches)
        kern_name = ("q1_mb_kernel (the batched matrix-core GEMV; each projection of the step "
                     "launched alone, back to back over the layers)")
        src = {"q": "x", "k": "x", "v": "x", "gate": "x", "up": "x", "o": "xo", "down": "xd"}
        gemv_ms, gemv_bytes, launches = 0.0, 0, 0
        cap = torch.cuda.Stream()
        for nm in ("q", "k", "v", "gate", "up", "o", "down"):
            n, k = shapes[nm]
            calls = [(layers[l][nm], lbq.act_view(act, src[nm], l, L, hid, kv, ffn, B),
                      lbq.act_view(act, nm, l, L, hid, kv, ffn, B)) for l in range(L)]
            with torch.cuda.stream(cap):
                for w_, xin, yout in calls:
                    lbq.lbq_gemv_q1g128(w_, n, k, xin, yout, stream=cap)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for w_, xin, yout in calls:
                    lbq.lbq_gemv_q1g128(w_, n, k, xin, yout, stream=cap)
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            reps = max(1, args.kernel_steps)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            gemv_ms += e0.elapsed_time(e1) / reps
            gemv_bytes += L * (n * k * 9 // 64)
            launches += L
            del g
        kern_avg_ms = gemv_ms / launches
        kern_bytes = gemv_bytes / launches
        run()   # restore the activation record of a full step for the parity check below
        torch.cuda.synchronize()
    kern_gbs = kern_bytes / (kern_avg_ms * 1e-3) / 1e9

    # ---- oracle legs: sampled teacher-forced parity, all-core baseline, chain cosine ---------
    cpu, parity, chain = None, None, None
    if args.cpu_layers > 0:
        import oracle
        from tests._gpu import check_within  # the tolerance rule shared with the tests
        cores, cpu_model = host_cpu()
        src = {"q": "x", "k": "x", "v": "x", "gate": "x", "up": "x", "o": "xo", "down": "xd"}
        view = lambda slot, l: lbq.act_view(act, slot, l, L, hid, kv, ffn, B).cpu().numpy().view(np.uint16)
        # (1) teacher-forced parity on sampled rows of every GEMV of layers 0, 1, L/2 - 1, L - 1
        #     (each GEMV fed the GPU's own input), and the rescales of those layers
        check_layers = sorted({l for l in (0, 1, L // 2 - 1, L - 1) if 0 <= l < L})
        worst, checked = 0.0, 0
        for l in check_layers:
            for nm in synth.STREAM_MATRICES:
                m = synth.stream_matrix(l, nm)
                n = m.shape[0]
                rows = np.unique(np.concatenate([np.linspace(0, n - 1, 384).astype(np.int32),
                                                 [n - 1]])).astype(np.int32)
                ref, l1 = oracle_rows(oracle.gemv_q1g128, m.signs, m.scales, view(src[nm], l), n,
                                      cores, rows)
                worst = max(worst, check_within(view(nm, l)[:, rows], ref, l1,
                                                f"bench layer {l} {nm}"))
                checked += rows.size * B
            from tests._gpu import bf16_ordinal
            nxt = (view("x", l + 1) if l + 1 < L else lbq.act_view(
                act, "final", L, L, hid, kv, ffn, B).cpu().numpy().view(np.uint16))
            for yname, y2name, got in (("q", None, view("xo", l)), ("gate", "up", view("xd", l)),
                                       ("down", None, nxt)):
                xr, _ = oracle.rms_rescale(view(yname, l),
                                           None if y2name is None else view(y2name, l))
                dd = np.abs(bf16_ordinal(xr) - bf16_ordinal(got))
                assert dd.max() <= 1, f"bench layer {l} rescale of {yname}: {dd.max()} ulp"
        parity = {"layers": check_layers, "gemv_rows_checked": int(checked),
                  "worst_err_over_l1": float(f"{worst:.3e}"), "tolerance": "2e-3 * sum|s*w*x|",
                  "rescales": "within 1 bf16 ulp"}
        log(f"parity: layers {check_layers}, sampled rows of all 7 GEMVs within 2e-3*L1 "
            f"(worst |err|/L1 = {worst:.2e}); rescales within 1 ulp")
        # (2) the oracle as it stands on all host cores (rows split across threads), on every
        #     row of every GEMV of the first --cpu-layers layers
        cpu_s, cpu_bytes = 0.0, 0
        sample_layers = list(range(min(args.cpu_layers, L)))
        for l in sample_layers:
            for nm in synth.STREAM_MATRICES:
                m = synth.stream_matrix(l, nm)
                xin = view(src[nm], l)
                t = time.perf_counter()
                oracle_rows(oracle.gemv_q1g128, m.signs, m.scales, xin, m.shape[0], cores)
                cpu_s += time.perf_counter() - t
                cpu_bytes += m.shape[0] * m.shape[1] * 9 // 64 * B
        log(f"oracle baseline: {cpu_bytes / 1e6:.0f} MB in {cpu_s:.1f} s on {cores} cores ({cpu_model})")
        cpu = {"value": round(cpu_bytes / cpu_s / 1e9, 6), "unit": "GB/s", "cores": cores,
               "kind": "oracle", "cpu_model": cpu_model,
               "sample": f"{len(sample_layers)} of {L} layers (all 7 GEMVs of each, every row, "
                         f"batch {B}), plain scalar C oracle in float64, rows split over "
                         f"{cores} threads; {cpu_bytes / 1e6:.1f} MB of packed weights in "
                         f"{cpu_s:.1f} s",
               "tok_s_equiv": round(B * cpu_bytes / bytes_per_step / cpu_s, 6)}
        # (3) the whole chain in the oracle (batch 1): x_{l+1} = rms(down(rms(gate * up))) from
        #     the same x0, every row, compared with the GPU's chain by cosine similarity
        #     (reported, not gated: the two chains drift apart by rounding)
        if B == 1 and not args.no_chain:
            t = time.perf_counter()
            x = x0_np.reshape(1, hid)
            cos = []
            for l in range(L):
                g = synth.stream_matrix(l, "gate")
                u = synth.stream_matrix(l, "up")
                dn = synth.stream_matrix(l, "down")
                yg, _ = oracle_rows(oracle.gemv_q1g128, g.signs, g.scales, x, ffn, cores)
                yu, _ = oracle_rows(oracle.gemv_q1g128, u.signs, u.scales, x, ffn, cores)
                xd, _ = oracle.rms_rescale(oracle.round_bf16(yg), oracle.round_bf16(yu))
                yd, _ = oracle_rows(oracle.gemv_q1g128, dn.signs, dn.scales, xd, hid, cores)
                x, _ = oracle.rms_rescale(oracle.round_bf16(yd))
                gpu_x = (view("x", l + 1) if l + 1 < L else lbq.act_view(
                    act, "final", L, L, hid, kv, ffn, B).cpu().numpy().view(np.uint16))
                a = oracle.bf16_to_f64(x).ravel()
                b = oracle.bf16_to_f64(gpu_x).ravel()
                cos.append(float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b))))
            marks = [m for m in (1, 2, 4, 8, 16, 32, 64) if m <= L]
            chain = {"layers": L, "cosine_final_x": round(cos[-1], 6),
                     "cosine_by_layer": {str(m): round(cos[m - 1], 6) for m in marks},
                     "note": "x_l of the GPU chain vs x_l of the oracle chain from the same x0; "
                             "random 1-bit layers amplify rounding differences, so the chains "
                             "decorrelate with depth (reported, not gated)",
                     "oracle_seconds": round(time.perf_counter() - t, 1), "threads": cores}
            log(f"chain: cosine of x_l (GPU vs oracle chain) by layer: {chain['cosine_by_layer']} "
                f"({chain['oracle_seconds']} s)")

    out = {
        "metric": f"packed-weight HBM GB/s (% of peak) + decode tok/s-equiv, batch {B}, 27B-shape",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tok_s_equiv": round(B / (ms * 1e-3), 2),
        "config": {
            "workload": (f"27B-shaped Q1_0_g128 decode-step weight stream: {L} layers x "
                         f"(q,o {hid}x{hid}; k,v {kv}x{hid}; gate,up {ffn}x{hid}; down {hid}x{ffn}) "
                         f"+ RMS rescales, batch {B}"),
            "layers": L, "batch": B, "packed_bytes_per_step": bytes_per_step,
            "launch": "HIP graph" if graph is not None else "eager",
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(kern_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(L, B) if B == 1 else None,
            "traffic_unit": ("bytes per step (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)"
                             if B == 1 else "bytes per launch"),
            "kernel": kern_name,
            "avg_launch_us": round(kern_avg_ms * 1e3, 3),
            "bytes_per_launch": round(kern_bytes),
        },
        "cpu_baseline": cpu,
        "rounds": {"count": len(round_ms), "steps_each": args.steps,
                   "ms_per_step_min": round(min(round_ms), 4) if round_ms else None,
                   "ms_per_step_median": round(sorted(round_ms)[len(round_ms) // 2], 4)
                   if round_ms else None},
        "hbm_achievable": None if achievable is None else {
            "gbs": round(achievable, 1), "pct_of_peak": round(100.0 * achievable / HBM_PEAK_GBS, 2),
            "probe": "4 GiB streaming read, 16-byte nontemporal loads (lbq_hbm_read_probe)",
            "value_pct_of_achievable": round(100.0 * gbs / achievable, 2)},
        "parity": parity,
        "chain": chain,
    }
    print(json.dumps(out), flush=True)
    return 0


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak


# 2-bit MACs per evaluation of the 256-192-128-40 network
Z80_MACS_PER_EVAL = 256 * 192 + 192 * 128 + 128 * 40
# int16 dot2 issue rate of the chip: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz x 2 MACs
ALU_DOT2_PEAK_TMACS = 256 * 4 * 16 * 2.4e9 * 2 / 1e12


def graph_time_us(torch, fn, pool, args, cap, stream):
    """Per-call time of fn(w) over a HIP graph of >= 64 launches rotating through `pool`."""
    calls = len(pool) * max(1, 64 // len(pool))
    with torch.cuda.stream(cap):
        for i in range(max(len(pool), args.warmup)):
            fn(pool[i % len(pool)])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for i in range(calls):
            fn(pool[i % len(pool)])
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) * 1e3 / (args.steps * calls)


def q1_gemv_bench(args, lbq, synth, torch, np, dev) -> int:
    """Single Q1_0_g128 GEMVs through lbq_gemv_q1g128: 5120x5120 at batch 1, and the MLP
    projections gate/up 17408x5120 and down 5120x17408 at batch 1, 4 and 16. Weights rotate
    through >= 1 GiB of copies (no reuse from the 256 MB last-level cache); the calls are
    replayed from one HIP graph. Algorithmic bytes per call: packed weights (1.125 bits per
    weight) plus bf16 activations in and out. The headline value is 5120x5120 at batch 1."""
    stream = torch.cuda.current_stream()
    cap = torch.cuda.Stream()
    import oracle
    from tests._gpu import check_within
    cores, cpu_model = host_cpu()
    cases, head = [], None
    worst = 0.0
    for name, n, k, batches in (("square", 5120, 5120, (1,)), ("gate", 17408, 5120, (1, 4, 16)),
                                ("down", 5120, 17408, (1, 4, 16))):
        m = synth.q1_matrix(n, k, workload=synth.W_Q1_SQUARE if name == "square"
                            else synth.W_Q1_MLP, matrix={"square": 0, "gate": 4, "down": 6}[name])
        packed = lbq.lbq_pack_q1g128(m.signs, m.scales)
        host = torch.from_numpy(packed)
        pool = [host.to(dev) for _ in range(max(2, -(-(1 << 30) // packed.nbytes)))]
        for batch in batches:
            xh = synth.activations(batch, k, workload=synth.W_Q1_MLP, extra=200 + batch)
            x = torch.from_numpy(xh.view(np.int16)).to(dev)
            y = torch.empty((batch, n), dtype=torch.int16, device=dev)
            us = graph_time_us(torch, lambda w: lbq.lbq_gemv_q1g128(w, n, k, x, y, stream=cap),
                               pool, args, cap, stream)
            nbytes = packed.nbytes + 2 * batch * (n + k)
            rows = np.unique(np.linspace(0, n - 1, 256).astype(np.int32))
            ref, l1 = oracle_rows(oracle.gemv_q1g128, m.signs, m.scales, xh, n, cores, rows)
            worst = max(worst, check_within(y.cpu().numpy().view(np.uint16)[:, rows], ref, l1,
                                            f"q1 {name} B={batch}"))
            case = {"matrix": name, "n": n, "k": k, "batch": batch, "us_per_call": round(us, 2),
                    "gbs": round(nbytes / us / 1e3, 1),
                    "pct_of_hbm_peak": round(100.0 * nbytes / us / 1e3 / HBM_PEAK_GBS, 2)}
            cases.append(case)
            if head is None:
                head = (us, nbytes)
            log(f"q1 {name} {n}x{k} B={batch}: {us:.2f} us, {nbytes / us / 1e3:.0f} GB/s")
        del pool
        torch.cuda.empty_cache()
    us, nbytes = head
    gbs = nbytes / us / 1e3
    # the oracle on all host cores: every row of the 5120x5120 matrix at batch 1
    m = synth.q1_matrix(5120, 5120, workload=synth.W_Q1_SQUARE, matrix=0)
    xh = synth.activations(1, 5120, workload=synth.W_Q1_MLP, extra=201)
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < 2.0:
        oracle_rows(oracle.gemv_q1g128, m.signs, m.scales, xh, 5120, cores)
        reps += 1
    dt = time.perf_counter() - t0
    out = {
        "metric": "packed-weight HBM GB/s of single Q1_0_g128 GEMVs (5120x5120 at batch 1)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "gemv_per_s": round(1e6 / us, 1),
        "config": {"workload": "Q1_0_g128 GEMV 5120x5120, batch 1 (and the MLP projections "
                               "gate/up 17408x5120, down 5120x17408 at batch 1, 4, 16 in cases)",
                   "rotation": ">= 1 GiB of weight copies", "launch": "HIP graph",
                   "parallelism": "single GPU"},
        "cases": cases,
        "parity": {"rows_checked_per_case": 256, "worst_err_over_l1": float(f"{worst:.3e}"),
                   "tolerance": "2e-3 * sum|s*w*x|"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "stage1_kernel (the stage-1 lookup kernel, which takes "
                               "batch-1 GEMVs with k <= 7168)",
                     "avg_launch_us": round(us, 3), "bytes_per_launch": nbytes},
        "cpu_baseline": {"value": round(reps * m.shape[0] * m.shape[1] * 9 / 64 / dt / 1e9, 4),
                         "unit": "GB/s", "cores": cores, "kind": "oracle",
                         "cpu_model": cpu_model,
                         "sample": f"{reps} full 5120x5120 batch-1 GEMVs, rows split over "
                                   f"{cores} threads, in {dt:.1f} s"},
    }
    print(json.dumps(out), flush=True)
    return 0


def mlp2bit_bench(args, lbq, synth, torch, np, dev) -> int:
    """The 2-bit integer MLP through lbq_mlp_2bit_i16: 1024 input vectors of 256 int16 bucket
    counts (uniform 0..127) through the 256-192-128-40 network with uniform 2-bit codes, one
    launch per step, launches replayed from a HIP graph; logits and argmax are compared with the
    oracle bit for bit. Also timed, as cases: the same vectors through balanced codes (uniform
    over 1..3, weights -1, 0, +1: the uniform codes' mean weight of -1/2 drives every ReLU input
    negative, so their logits are all zero, and this case shows the time does not depend on the
    values), and 65,536 vectors (throughput context; the first and last 1024 checked)."""
    import oracle
    dims = list(synth.MLP_DIMS)
    layers = synth.mlp2bit_layers()
    balanced = []   # canonical bytes of codes uniform over 1..3 (four per byte, first code lowest)
    for l in range(len(dims) - 1):
        r = synth.rng(synth.W_MLP2BIT, l, 0, synth.KIND_STRESS)
        v = r.integers(1, 4, size=(dims[l + 1], dims[l] // 4, 4)).astype(np.uint8)
        balanced.append((v[..., 0] | v[..., 1] << 2 | v[..., 2] << 4 | v[..., 3] << 6)
                        .astype(np.uint8))
    stream = torch.cuda.current_stream()
    cap = torch.cuda.Stream()
    cases = []
    head = None
    for name, codes, B in (("uniform codes", layers, 1024), ("balanced codes", balanced, 1024),
                           ("uniform codes", layers, 65536)):
        xh = synth.mlp2bit_inputs(batch=B)
        lw = [torch.from_numpy(lbq.lbq_pack_2bit(c)).to(dev) for c in codes]
        x = torch.from_numpy(xh).to(dev)
        logits = torch.empty((B, dims[-1]), dtype=torch.int16, device=dev)
        am = torch.empty((B,), dtype=torch.int32, device=dev)
        # one launch per step, 32 steps per replay of a HIP graph
        us = graph_time_us(torch, lambda w: lbq.lbq_mlp_2bit_i16(w, dims, x, logits, am,
                                                                 stream=cap),
                           [lw] * 32, args, cap, stream)
        rows = np.arange(B) if B <= 1024 else np.r_[0:1024, B - 1024:B]
        t0 = time.perf_counter()
        ref_logits, ref_am = oracle.mlp_2bit(codes, dims, xh[rows])
        dt = time.perf_counter() - t0
        assert np.array_equal(logits.cpu().numpy()[rows], ref_logits), f"2-bit MLP logits differ ({name})"
        assert np.array_equal(am.cpu().numpy()[rows], ref_am), f"2-bit MLP argmax differs ({name})"
        tmacs = B * Z80_MACS_PER_EVAL / (us * 1e-6) / 1e12
        log(f"mlp2bit {name}, {B} vectors: {us:.2f} us per launch, {tmacs:.3f} T MAC/s, "
            f"bit-exact on {rows.size} vectors")
        cases.append({"codes": name, "vectors": B, "us_per_launch": round(us, 3),
                      "evals_per_s": round(B / (us * 1e-6), 1), "gmac_per_s": round(tmacs * 1e3, 1),
                      "pct_of_dot2_issue_rate": round(100.0 * tmacs / ALU_DOT2_PEAK_TMACS, 2),
                      "vectors_checked": int(rows.size)})
        if head is None:
            head = (us, B, tmacs, dt)
    us, B, tmacs, dt = head
    out = {
        "metric": "2-bit integer MLP evaluations per second (1024 vectors, 256-192-128-40)",
        "value": round(B / (us * 1e-6), 1),
        "unit": "evals/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int16 x 2-bit -> int32 (mod 2^16)",
        "data": "synthetic",
        "gmac_per_s": round(tmacs * 1e3, 1),
        "config": {"workload": f"Z80-uLM-shaped 2-bit MLP, {B} vectors, 256-192-128-40",
                   "parallelism": "single GPU", "parity": "logits and argmax bit-exact"},
        "cases": cases,
        "roofline": {"bound": "alu", "achieved": round(tmacs, 3), "peak": ALU_DOT2_PEAK_TMACS,
                     "unit": "T 2-bit MAC/s (v_dot2_i32_i16 issue rate)",
                     "frac": round(tmacs / ALU_DOT2_PEAK_TMACS, 4), "traffic": None,
                     "kernel": "mlp2bit_lds_kernel", "avg_launch_us": round(us, 3)},
        "cpu_baseline": {"value": round(B / dt, 1), "unit": "evals/s", "cores": 1,
                         "kind": "oracle", "sample": f"all {B} vectors, one host thread"},
    }
    print(json.dumps(out), flush=True)
    return 0


def tern_layer_bench(args, lbq, synth, torch, np, dev) -> int:
    """The seven projections of one 27B-shaped layer (q, o 5120x5120; k, v 1024x5120; gate, up
    17408x5120; down 5120x17408) with ternary g160 weights through lbq_gemv_tern_g160 at B = 1
    and 8. Weights rotate through >= 1 GiB of copies; each projection's calls are replayed from
    one HIP graph; the time per layer is the sum of the projections' times per call. Algorithmic
    bytes: packed weights (34 bytes per 160 weights) plus bf16 activations in and out."""
    stream = torch.cuda.current_stream()
    cap = torch.cuda.Stream()
    layer = {1: [0.0, 0], 8: [0.0, 0]}
    cases = []
    for name in synth.STREAM_MATRICES:
        n, k = synth.stream_shape(name)
        m = synth.tern_matrix(n, k, matrix=synth.STREAM_MATRICES.index(name))
        packed = lbq.lbq_pack_tern_g160(m.codes, m.scales)
        host = torch.from_numpy(packed)
        pool = [host.to(dev) for _ in range(max(2, -(-(1 << 30) // packed.nbytes)))]
        for batch in (1, 8):
            x = torch.from_numpy(synth.activations(batch, k, workload=synth.W_TERN,
                                                   extra=100 + batch).view(np.int16)).to(dev)
            y = torch.empty((batch, n), dtype=torch.int16, device=dev)
            us = graph_time_us(torch, lambda w: lbq.lbq_gemv_tern_g160(w, n, k, x, y, stream=cap),
                               pool, args, cap, stream)
            nbytes = packed.nbytes + 2 * batch * (n + k)
            layer[batch][0] += us
            layer[batch][1] += nbytes
            cases.append({"proj": name, "n": n, "k": k, "batch": batch, "us_per_call": round(us, 2),
                          "gbs": round(nbytes / us / 1e3, 1)})
            log(f"tern {name} {n}x{k} B={batch}: {us:.1f} us, {nbytes / us / 1e3:.0f} GB/s")
        del pool
        torch.cuda.empty_cache()
    head_us, head_bytes = layer[1]
    gbs = head_bytes / head_us / 1e3
    import oracle
    t0 = time.perf_counter()
    sampled = 0
    for name in synth.STREAM_MATRICES:
        n, k = synth.stream_shape(name)
        m = synth.tern_matrix(n, k, matrix=synth.STREAM_MATRICES.index(name))
        xs = synth.activations(1, k, workload=synth.W_TERN, extra=101)
        oracle.gemv_tern_g160(m.codes, m.scales, xs, rows=np.arange(512, dtype=np.int32))
        sampled += 512 * ((k + 159) // 160) * 34
    dt = time.perf_counter() - t0
    out = {
        "metric": "packed-weight HBM GB/s of the ternary g160 GEMVs of a 27B-shaped layer",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head_us / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (ternary weights, bf16 activations)",
        "data": "synthetic",
        "config": {"workload": "27B-shaped layer (7 projections), ternary g160 weights, B = 1; "
                               "B = 8 in cases",
                   "parallelism": "single GPU",
                   "us_per_layer_b8": round(layer[8][0], 2),
                   "gbs_b8": round(layer[8][1] / layer[8][0] / 1e3, 1)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": i4_layer_traffic("B1", TERN_PROFILE),
                     "traffic_unit": "HBM bytes per layer (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-scaled)",
                     "bytes_per_layer": head_bytes,
                     "kernel": "tern_gemv_kernel<1> (7 launches per layer)"},
        "cpu_baseline": {"value": round(sampled / dt / 1e9, 5), "unit": "GB/s", "cores": 1,
                         "kind": "oracle",
                         "sample": "512 output rows of each of the 7 projections, B = 1"},
        "cases": cases,
    }
    print(json.dumps(out), flush=True)
    return 0


def chat_bench(args, lbq, synth, torch, np, dev) -> int:
    """The Z80-uLM character loop (lbq_z80_chat_2bit): 1024 synthetic prompts of a few words,
    replies of up to 32 characters, random 2-bit weights of the 256-192-128-40 network. A step
    is one launch that generates every reply. Characters per second count the characters
    emitted; evaluations per second count one network evaluation per emitted character plus
    one per reply that ended before the cap."""
    layers = synth.mlp2bit_layers()
    arr, lens = synth.chat_prompts(synth.MLP_BATCH)
    B, R = arr.shape[0], synth.Z80_REPLY
    lw = [torch.from_numpy(lbq.lbq_pack_2bit(c)).to(dev) for c in layers]
    pr = torch.from_numpy(arr).to(dev)
    ln = torch.from_numpy(lens).to(dev)
    reply = torch.empty((B, R), dtype=torch.uint8, device=dev)
    rl = torch.empty((B,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(max(1, args.warmup)):
        lbq.lbq_z80_chat_2bit(lw, synth.MLP_DIMS, pr, ln, reply, rl, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        lbq.lbq_z80_chat_2bit(lw, synth.MLP_DIMS, pr, ln, reply, rl, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    lengths = rl.cpu().numpy()
    chars = int(lengths.sum())
    evals = chars + int((lengths < R).sum())
    tmacs = evals * Z80_MACS_PER_EVAL / (us * 1e-6) / 1e12
    log(f"z80 chat: {us:.1f} us per launch, {chars} characters, {evals} evaluations")
    # the oracle (one host thread) on the first 256 prompts
    import oracle
    nb = 256
    t0 = time.perf_counter()
    _, _, orl = oracle.z80_chat(layers, list(synth.MLP_DIMS),
                                [bytes(arr[b, :lens[b]]) for b in range(nb)], R)
    dt = time.perf_counter() - t0
    out = {
        "metric": "Z80-uLM generated characters per second (whole character loop on the GPU)",
        "value": round(chars / (us * 1e-6), 1),
        "unit": "chars/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int16 x 2-bit -> int32 (mod 2^16)",
        "data": "synthetic",
        "config": {"workload": f"Z80-uLM chat loop, 256-192-128-40 2-bit network, {B} prompts, "
                               f"replies up to {R} characters",
                   "parallelism": "single GPU", "characters": chars, "evaluations": evals},
        "roofline": {"bound": "alu", "achieved": round(tmacs, 3), "peak": ALU_DOT2_PEAK_TMACS,
                     "unit": "T 2-bit MAC/s (v_dot2_i32_i16 issue rate)",
                     "frac": round(tmacs / ALU_DOT2_PEAK_TMACS, 4), "traffic": None,
                     "kernel": "z80_chat_kernel"},
        "cpu_baseline": {"value": round(float(orl.sum()) / dt, 1), "unit": "chars/s", "cores": 1,
                         "kind": "oracle", "sample": f"the first {nb} prompts of the workload"},
    }
    print(json.dumps(out), flush=True)
    return 0


def i4_layer_bench(args, lbq, synth, torch, np, dev) -> int:
    """The seven projections of a Qwen3-8B-shaped INT4 g128 layer (q, o 4096x4096; k, v
    1024x4096; gate, up 12288x4096; down 4096x12288) through lbq_gemv_i4g128 (bf16 activations)
    and lbq_gemv_i4g128_act_i8 (int8 activations quantized in the kernel, integer dot products),
    at B = 1 and 8. Weights rotate through a pool of at least 1 GiB of copies so that every call
    streams them from HBM. Each projection's calls are captured in one HIP graph (64 or more
    launches) so that host launch cost stays out of the figure; the graph is replayed `steps`
    times between HIP events on the replay stream, and the time per layer is the sum of the
    projections' times per call. Algorithmic bytes: the packed weights (33/64 B per weight) plus
    bf16 activations in and out."""
    stream = torch.cuda.current_stream()
    cap = torch.cuda.Stream()
    paths = (("bf16", lbq.lbq_gemv_i4g128), ("i8act", lbq.lbq_gemv_i4g128_act_i8))
    layer = {(p, b): [0.0, 0] for p, _ in paths for b in (1, 8)}
    cases = []
    for name, n, k in synth.I4_SHAPES:
        mat = synth.i4_matrix(n, k, workload=synth.W_I4_LAYER,
                              matrix=synth.STREAM_MATRICES.index(name))
        packed = lbq.lbq_pack_i4g128(mat.nib, mat.scales)
        host = torch.from_numpy(packed)
        pool = [host.to(dev) for _ in range(max(2, -(-(1 << 30) // packed.nbytes)))]
        for batch in (1, 8):
            x = torch.from_numpy(synth.activations(batch, k, workload=synth.W_I4_LAYER,
                                                   extra=100 + batch).view(np.int16)).to(dev)
            y = torch.empty((batch, n), dtype=torch.int16, device=dev)
            nbytes = packed.nbytes + 2 * batch * (n + k)
            for pname, fn in paths:
                # eager warm-up on the capture stream (creates the split-K workspace), then one
                # graph of `calls` launches rotating through the pool
                calls = len(pool) * max(1, 64 // len(pool))
                with torch.cuda.stream(cap):
                    for i in range(max(len(pool), args.warmup)):
                        fn(pool[i % len(pool)], n, k, x, y, stream=cap)
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=cap):
                    for i in range(calls):
                        fn(pool[i % len(pool)], n, k, x, y, stream=cap)
                graph.replay()
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(args.steps):
                    graph.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                del graph
                us = e0.elapsed_time(e1) * 1e3 / (args.steps * calls)
                layer[(pname, batch)][0] += us
                layer[(pname, batch)][1] += nbytes
                cases.append({"path": pname, "proj": name, "n": n, "k": k, "batch": batch,
                              "us_per_call": round(us, 2), "gbs": round(nbytes / us / 1e3, 1)})
                log(f"i4 {pname} {name} {n}x{k} B={batch}: {us:.1f} us, {nbytes / us / 1e3:.0f} GB/s")
        del pool
        torch.cuda.empty_cache()
    summary = {f"{p}_B{b}": {"us_per_layer": round(v[0], 2), "gbs": round(v[1] / v[0] / 1e3, 1)}
               for (p, b), v in layer.items()}
    head_us, head_bytes = layer[("i8act", 1)]
    gbs = head_bytes / head_us / 1e3
    # the oracle (one host thread): quantize and multiply 512 rows of each projection, B = 1
    import oracle
    t0 = time.perf_counter()
    sampled = 0
    for name, n, k in synth.I4_SHAPES:
        mat = synth.i4_matrix(n, k, workload=synth.W_I4_LAYER,
                              matrix=synth.STREAM_MATRICES.index(name))
        xs = synth.activations(1, k, workload=synth.W_I4_LAYER, extra=101)
        q, d = oracle.quant_act_i8g128(xs)
        oracle.gemv_i4g128_i8act(mat.nib, mat.scales, q, d, rows=np.arange(512, dtype=np.int32))
        sampled += 512 * k * 33 // 64
    dt = time.perf_counter() - t0
    out = {
        "metric": "packed-weight HBM GB/s of the INT4 g128 layer GEMVs, int8 activations",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head_us / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 x int4 -> int32, fp32 group scaling",
        "data": "synthetic",
        "config": {"workload": "Qwen3-8B-shaped INT4 g128 layer (7 projections), B = 1, int8 "
                               "activations; bf16 path and B = 8 in cases",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": i4_layer_traffic("i8act-B1"),
                     "traffic_unit": "HBM bytes per layer (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-scaled)",
                     "bytes_per_layer": head_bytes,
                     "kernel": "i4_i8act_gemv_kernel<1> (7 launches per layer)"},
        "cpu_baseline": {"value": round(sampled / dt / 1e9, 5), "unit": "GB/s", "cores": 1,
                         "kind": "oracle",
                         "sample": "quantize + 512 output rows of each of the 7 projections, B = 1"},
        "summary": summary,
        "cases": cases,
    }
    print(json.dumps(out), flush=True)
    return 0


def gemm_bench(args, lbq, synth, torch, np, dev) -> int:
    """Many-row products (prefill / large batch) on the matrix cores: y[m][n] = x[m][k] W^T for
    the Q1 MLP shapes (gate 17408x5120, down 5120x17408) and the INT4 layer shapes (gate
    12288x4096, down 4096x12288) at m = 32, 128, 512 activation rows. Weights rotate through a
    pool of at least 1 GiB of copies so that every call streams them from HBM; times are HIP
    events around `steps` calls after `warmup` calls on the launch stream. Flops = 2 m n k."""
    cases = []
    shapes = [("q1", 17408, 5120), ("q1", 5120, 17408), ("i4", 12288, 4096), ("i4", 4096, 12288)]
    stream = torch.cuda.current_stream()
    for fmt, n, k in shapes:
        wl = synth.W_Q1_MLP if fmt == "q1" else synth.W_I4_LAYER
        mat = (synth.q1_matrix(n, k, workload=wl, matrix=n + k) if fmt == "q1"
               else synth.i4_matrix(n, k, workload=wl, matrix=n + k))
        packed = (lbq.lbq_pack_q1g128(mat.signs, mat.scales) if fmt == "q1"
                  else lbq.lbq_pack_i4g128(mat.nib, mat.scales))
        host = torch.from_numpy(packed)
        pool = [host.to(dev) for _ in range(max(2, -(-(1 << 30) // packed.nbytes)))]
        fn = lbq.lbq_gemm_q1g128 if fmt == "q1" else lbq.lbq_gemm_i4g128
        for m in (32, 128, 512):
            x = torch.from_numpy(synth.activations(m, k, workload=wl, matrix=n + k, extra=m)
                                 .view(np.int16)).to(dev)
            y = torch.empty((m, n), dtype=torch.int16, device=dev)
            it = [0]

            def call():
                fn(pool[it[0] % len(pool)], n, k, x, y, stream=stream)
                it[0] += 1

            for _ in range(max(1, args.warmup)):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / args.steps
            tflops = 2.0 * m * n * k / (us * 1e-6) / 1e12
            cases.append({"format": fmt, "n": n, "k": k, "m": m, "us_per_call": round(us, 2),
                          "tflops": round(tflops, 2), "weight_gbs": round(packed.nbytes / us / 1e3, 1),
                          "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)})
            log(f"gemm {fmt} {n}x{k} m={m}: {us:.1f} us, {tflops:.1f} TFLOP/s")
        del pool
        torch.cuda.empty_cache()
    head = next(c for c in cases if c["format"] == "q1" and c["n"] == 17408 and c["m"] == 512)
    # the oracle (one host thread) on the first 4 activation rows of the head case, all outputs
    import oracle
    mat = synth.q1_matrix(17408, 5120, workload=synth.W_Q1_MLP, matrix=17408 + 5120)
    xs = synth.activations(512, 5120, workload=synth.W_Q1_MLP, matrix=17408 + 5120, extra=512)[:4]
    t0 = time.perf_counter()
    oracle.gemv_q1g128(mat.signs, mat.scales, xs)
    dt = time.perf_counter() - t0
    out = {
        "metric": "packed-weight GEMM TFLOP/s on the matrix cores (prefill / large batch)",
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_call"] / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Q1_0_g128 gate 17408x5120, 512 activation rows (head); Q1 MLP and "
                               "INT4 layer shapes at 32/128/512 rows in cases",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": head["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": head["mfma_frac"], "traffic": None,
                     "kernel": "gemm_kernel<0, 2>"},
        "cpu_baseline": {"value": round(2.0 * 4 * 17408 * 5120 / dt / 1e12, 6), "unit": "TFLOP/s",
                         "cores": 1, "kind": "oracle",
                         "sample": "4 activation rows x all 17408 outputs of the head case"},
        "cases": cases,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
