"""Benchmark of the group-quantized GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

A step is one decode pass of the hidden-2560 MLP pair at M = 1 (the fused
gate/up projection K=2560 -> N=19456, then the down projection K=9728 ->
N=2560), both W4A16 with group-128 INT4 codes and fp16 scales, weights and
activations already resident in HBM. The reported value is achieved HBM
throughput on the algorithmic bytes of the step (codes + scales + x + out).

Weights rotate over enough distinct copies (>= 2 x 256 MiB per shape) that
the 256 MB Infinity Cache cannot serve them, so every step reads HBM. Steps
are captured in HIP graphs (torch.cuda.graph), so the timing measures the GPU
rather than Python launch overhead.

Besides the headline line, the same JSON object carries
  roofline      the dominant kernel (gate/up GEMV), timed live with events,
                with the read-stream ceiling of one launch over the same
                weight copies (the library's read probe) as context;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same step
                (all BLAS threads; single_thread_value on one thread);
  workloads     the other shapes (the tiny 256 x 512 case, M=16
                verification, W8A16 drafter, M=8192 prefill, fp16
                activations, Q_s packing, dense dequantization, the fake
                quantizer, the grouped K+V launch, and the drafter's
                sliding-window attention), each with its roofline fraction
                (none for the tiny case, whose weights stay in cache); the
                prefill rows also carry, as context, the vendor library's
                dense bf16 GEMM (torch.matmul) at the same shape. The M = 16
                W4A16 and W8A16 sets are also run back to back (QKV, gate/up,
                down) for their byte-weighted aggregate rate. Each row carries
                the CPU oracle's figure for the same shape (cpu_oracle).

The headline times exactly --steps steps after about 20 ms of untimed graph
replays, like every other row: a short region timed cold reads up to ~15%
slow while the GPU clocks settle.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("W4A16 GEMM achieved HBM GB/s (M=1,16) and TFLOP/s (M=8192) vs MI355X roofline")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix, published
MALL_BYTES = 256 * 2**20
GRAPH_CHUNK = 20               # steps per captured graph


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only-headline", action="store_true", help="skip the other workloads")
    ap.add_argument("--workload", default="",
                    help="run only the other workloads whose key contains one of these "
                         "comma-separated texts (tiny, verify, drafter, prefill, fp16act, "
                         "pack, dequant, fake_quant, grouped, attention)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_w4a16_gate_up_m1.json")
KERNEL_SOURCES = [os.path.join(ROOT, "int8_group_quantized_amd", "csrc", f)
                  for f in ("gemv.hip", "qg_device.h")]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel sources changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def copy_calibration(torch):
    """A plain 256 MiB device-to-device copy of known size: its byte counters
    scale the GEMM's counter readings to bytes."""
    n = 256 * 2**20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del dst


def alg_bytes(bits, M, K, N):
    codes = K * N * bits // 8
    scales = (K // 128) * N * 2
    return codes + scales + M * K * 2 + M * N * 2


class Weights:
    """Distinct device copies of one packed weight (RTN on the GPU)."""

    def __init__(self, q, torch, cfg, shape_index, copies, act="bf16"):
        import workloads
        w = workloads.WORKLOADS[cfg]
        self.bits, self.M = w["bits"], w["M"]
        self.K, self.N = w["shapes"][shape_index]
        W = workloads.weights(self.K, self.N, workloads.seed_for(cfg, shape_index, 0))
        Wd = torch.from_numpy(W).cuda()
        s = q.rtn_scales(Wd, self.bits)
        p = q.pack_to_grid(Wd, s, self.bits)
        self.W = Wd
        self.copies = copies
        self.packed = [p] + [p.clone() for _ in range(copies - 1)]
        self.scales = [s] + [s.clone() for _ in range(copies - 1)]
        xb = workloads.activations(self.M, self.K, workloads.seed_for(cfg, shape_index, 1), dtype=act)
        xdt = torch.bfloat16 if act == "bf16" else torch.float16
        self.x = torch.from_numpy(xb.view(np.int16)).view(xdt).cuda()
        self.out = torch.empty((self.M, self.N), dtype=xdt, device="cuda")
        self.ws = torch.zeros(max(q.workspace_bytes(self.bits, self.M, self.K, self.N), 1 << 16),
                              dtype=torch.uint8, device="cuda")
        self.cbm = False              # scales in the logical [K/128, N] order
        self.bytes = alg_bytes(self.bits, self.M, self.K, self.N)
        self.flops = 2 * self.M * self.K * self.N

    def call(self, q, i):
        j = i % len(self.packed)
        q.qgemm(self.x, self.packed[j], self.scales[j], self.bits, self.N, out=self.out, ws=self.ws,
                scales_cbm=self.cbm)

    def free(self):
        self.W = None
        self.packed = self.scales = None


def copies_for(bits, K, N):
    per = K * N * bits // 8 + (K // 128) * N * 2
    return max(1, math.ceil(2 * MALL_BYTES / per))


def capture(torch, fn, n):
    """A HIP graph of n calls fn(0..n-1) on a capture stream."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn_range = list(range(n))
        for i in fn_range:        # warm the stream once outside capture
            fn(i)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in fn_range:
                fn(i)
    torch.cuda.synchronize()
    return g


def time_graphs(torch, graphs, reps=1):
    """Milliseconds to replay the list of graphs `reps` times (events on the
    replay stream, synchronised on both sides)."""
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        for g in graphs:
            g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def time_steady(torch, g, reps, warm_ms=20.0):
    """Milliseconds for `reps` replays of graph g, timed after untimed replays
    that keep the GPU busy for about warm_ms: the clocks settle over the
    first milliseconds of work, and a short timed region taken cold reads up
    to ~15% slow at the small-M shapes."""
    first = time_graphs(torch, [g])
    extra = min(1000, int(warm_ms / max(first, 1e-3)))
    if extra:
        time_graphs(torch, [g], reps=extra)
    return time_graphs(torch, [g], reps=reps)


def time_steps(torch, graphs, steps, warm_ms=20.0):
    """Milliseconds per step over exactly `steps` steps (one replay of the
    list of graphs), timed after untimed replays of the same graphs that keep
    the GPU busy for about warm_ms (as time_steady does for one graph)."""
    first = time_graphs(torch, graphs)
    extra = min(1000, int(warm_ms / max(first, 1e-3)))
    if extra:
        time_graphs(torch, graphs, reps=extra)
    return time_graphs(torch, graphs) / steps


def graphs_for_steps(torch, step, steps):
    full, rem = divmod(steps, GRAPH_CHUNK)
    gs = []
    if full:
        g = capture(torch, step, GRAPH_CHUNK)
        gs += [g] * full
    if rem:
        gs.append(capture(torch, step, rem))
    return gs


def kernel_average(torch, wt, q, launches=400):
    """Average duration of one GEMM launch: a graph of back-to-back launches
    on rotating weight copies, timed with events."""
    g = capture(torch, lambda i: wt.call(q, i), 100)
    ms = time_steady(torch, g, reps=launches // 100)
    return ms / (100 * (launches // 100))


def read_stream_ceiling(torch, q, bufs, widths=(1024, 2048, 4096, 8192, 16384)):
    """The library's read-stream probe (a measurement aid: plain 16-byte
    loads, nothing computed) over the rotating buffers bufs, one whole buffer
    per launch, in HIP-graph replays like the GEMV; the fastest of a few
    launch widths. Returns (us per launch, bytes per launch, workgroups)."""
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    nbytes = bufs[0].numel() * bufs[0].element_size()
    best = None
    for wgs in widths:
        g = capture(torch, lambda i: q.read_stream(bufs[i % len(bufs)], wgs, sink), 100)
        us = time_steady(torch, g, reps=4) / 400 * 1e3
        del g
        if best is None or us < best[0]:
            best = (us, nbytes, wgs)
    return best


def measure_decode_cbm(torch, q, steps):
    """The headline's decode step with the scales prepacked column-block-major
    (qg_prepack_scales, done once like the codes): same weights, copies,
    bytes and arithmetic (bit-identical outputs), only the scale order
    differs. Context beside the headline, which uses the logical order."""
    up = Weights(q, torch, 2, 0, copies_for(4, 2560, 19456))
    down = Weights(q, torch, 2, 1, copies_for(4, 9728, 2560))
    up.W = down.W = None
    for wt in (up, down):
        wt.scales = [q.prepack_scales(s) for s in wt.scales]
        wt.cbm = True
    torch.cuda.empty_cache()

    def step(i):
        up.call(q, i)
        down.call(q, i)

    graphs = graphs_for_steps(torch, step, steps)
    ms = time_steps(torch, graphs, steps)       # same steps and warm-up as the headline
    k_ms = kernel_average(torch, up, q)
    step_bytes = up.bytes + down.bytes
    gbs = step_bytes / (ms * 1e-3) / 1e9
    k_gbs = up.bytes / (k_ms * 1e-3) / 1e9
    del graphs
    up.free()
    down.free()
    torch.cuda.empty_cache()
    return {"workload": "decode_w4a16_m1, scales column-block-major (qg_prepack_scales)",
            "us_per_step": round(ms * 1e3, 3), "gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "gate_up_us_per_launch": round(k_ms * 1e3, 3),
            "gate_up_frac_hbm_peak": round(k_gbs / HBM_PEAK_GBS, 4)}


def dense_bf16_reference(torch, M, K, N, reps=10):
    """Context for the prefill rows: milliseconds per call of the vendor
    library's plain dense bf16 GEMM (torch.matmul, contiguous [M,K] x [K,N])
    at the same shape. It is not this library's path and does the same
    matrix-core work without the code expansion and group scales."""
    a = torch.randn(M, K, device="cuda").bfloat16()
    b = torch.randn(K, N, device="cuda").bfloat16()
    for _ in range(25):                  # ~20 ms of warm-up, as for the library's rows
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return ms


def measure_workload(torch, q, cfg, reps=1000, act="bf16"):
    import workloads
    w = workloads.WORKLOADS[cfg]
    rows = []
    for si, (K, N) in enumerate(w["shapes"]):
        prefill = w["M"] > 16
        tiny = K * N <= 1 << 20       # the 256 x 512 case: one resident copy, fixed cost only
        copies = 1 if (prefill or tiny) else copies_for(w["bits"], K, N)
        wt = Weights(q, torch, cfg, si, copies, act=act)
        wt.W = None
        n = 4 if prefill else 100
        g = capture(torch, lambda i: wt.call(q, i), n)
        r = max(1, (20 if prefill else reps) // n)
        ms = time_steady(torch, g, reps=r) / (n * r)
        row = {"shape": workloads.SHAPE_NAMES.get((K, N), "%dx%d" % (K, N)), "M": w["M"],
               "K": K, "N": N, "bits": w["bits"], "us_per_call": round(ms * 1e3, 3)}
        if prefill:
            tf = wt.flops / (ms * 1e-3) / 1e12
            row.update(tflops=round(tf, 1), frac_bf16_peak=round(tf / BF16_PEAK_TFLOPS, 4))
            dense = dense_bf16_reference(torch, w["M"], K, N)
            row.update(dense_bf16_library_us=round(dense * 1e3, 1),
                       dense_bf16_library_tflops=round(wt.flops / (dense * 1e-3) / 1e12, 1))
        elif tiny:
            row.update(weight_copies=1, note="69 KB of weights stay in cache; the time is the "
                                             "launch's fixed cost, no roofline claim")
        else:
            gbs = wt.bytes / (ms * 1e-3) / 1e9
            row.update(gbs=round(gbs, 1), frac_hbm_peak=round(gbs / HBM_PEAK_GBS, 4),
                       weight_copies=copies)
        rows.append(row)
        wt.free()
        del g
        torch.cuda.empty_cache()
    name = w["name"] if act == "bf16" else w["name"].replace("a16", "a16_fp16act")
    return {"workload": name, "shapes": rows}


def measure_set_sequence(torch, q, cfg, reps=400):
    """A verification block's Linear set run back to back (fused QKV, gate/up,
    down at M = 16, each over its own rotating weight copies), as one step
    of a graph: the byte-weighted aggregate rate of the set (total
    algorithmic bytes / time per step, launch gaps included)."""
    import workloads
    w = workloads.WORKLOADS[cfg]
    order = [2, 0, 1]                     # QKV, gate/up, down
    wts = []
    for si in order:
        K, N = w["shapes"][si]
        wt = Weights(q, torch, cfg, si, copies_for(w["bits"], K, N))
        wt.W = None
        wts.append(wt)
    torch.cuda.empty_cache()

    def step(i):
        for wt in wts:
            wt.call(q, i)

    g = capture(torch, step, 50)
    ms = time_steady(torch, g, reps=max(1, reps // 50)) / (50 * max(1, reps // 50))
    nbytes = sum(wt.bytes for wt in wts)
    gbs = nbytes / (ms * 1e-3) / 1e9
    for wt in wts:
        wt.free()
    del g
    torch.cuda.empty_cache()
    return {"workload": w["name"] + " set back to back (QKV, gate/up, down)",
            "M": w["M"], "bits": w["bits"], "bytes_per_step": nbytes,
            "us_per_step": round(ms * 1e3, 3), "gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def measure_pack(torch, q):
    """Q_s packing of the gate/up weight (fp32 W in, INT4 tiles out)."""
    import workloads
    K, N = 2560, 19456
    W = torch.from_numpy(workloads.weights(K, N, workloads.seed_for(3, 0, 0))).cuda()
    s = q.rtn_scales(W, 4)
    packed = torch.empty(K * N // 2, dtype=torch.uint8, device="cuda")
    g = capture(torch, lambda i: q.pack_to_grid(W, s, 4, out=packed), 20)
    ms = time_steady(torch, g, reps=5) / 100
    del g
    nbytes = K * N * 4 + (K // 128) * N * 2 + K * N // 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "pack_to_grid_w4 fp32 W", "K": K, "N": N, "us_per_call": round(ms * 1e3, 2),
            "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def measure_dequant(torch, q):
    """Dense dequantization of the gate/up INT4 weight to bf16 (reads codes
    and scales, writes 2 bytes per weight), over rotating weight copies."""
    K, N = 2560, 19456
    wt = Weights(q, torch, 2, 0, copies_for(4, K, N))
    wt.W = None
    dense = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")
    g = capture(torch, lambda i: q.dequant(wt.packed[i % wt.copies], wt.scales[i % wt.copies], 4,
                                           K, N, out=dense), 20)
    ms = time_steady(torch, g, reps=5) / 100
    nbytes = K * N // 2 + (K // 128) * N * 2 + K * N * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    wt.free()
    del g, dense
    torch.cuda.empty_cache()
    return {"workload": "dequant_w4 -> bf16 dense", "K": K, "N": N, "us_per_call": round(ms * 1e3, 2),
            "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def measure_fake_quant(torch, q):
    """The fixed-grid fake quantizer on the gate/up weight: fp32 W and fp16
    scales in, s (.) Q_s(W) out in bf16."""
    import workloads
    K, N = 2560, 19456
    W = torch.from_numpy(workloads.weights(K, N, workloads.seed_for(2, 0, 0))).cuda()
    s = q.rtn_scales(W, 4)
    out = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")
    g = capture(torch, lambda i: q.fake_quant(W, s, 4, out=out), 20)
    ms = time_steady(torch, g, reps=5) / 100
    nbytes = K * N * 4 + (K // 128) * N * 2 + K * N * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    del g, W, out
    torch.cuda.empty_cache()
    return {"workload": "fake_quant_w4 fp32 W -> bf16", "K": K, "N": N,
            "us_per_call": round(ms * 1e3, 2), "gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def measure_grouped(torch, q, bits):
    """K+V projections of the 5 drafter layers (hidden 2560 -> 2 x 512 each)
    for a 16-token block, as one grouped launch and as 5 separate launches,
    over rotating weight copies."""
    import workloads
    M, K, N, L = 16, 2560, 1024, 5
    sdt = "f16" if bits == 4 else "bf16"
    per = L * (K * N * bits // 8 + (K // 128) * N * 2)
    copies = max(1, math.ceil(2 * MALL_BYTES / per))
    sets = []
    for c in range(copies):
        if c == 0:
            base = []
            for i in range(L):
                codes = torch.from_numpy(workloads.codes(K, N, bits, 7000 + i)).cuda()
                sb = workloads.scales(K // 128, N, sdt, 7100 + i).view(np.int16)
                sc = torch.from_numpy(sb).view(torch.float16 if sdt == "f16" else torch.bfloat16).cuda()
                base.append((q.prepack(codes, bits), sc, N))
            sets.append(base)
        else:
            sets.append([(p.clone(), sc.clone(), n) for p, sc, n in base])
    xb = workloads.activations(M, K, 7200)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    g1 = capture(torch, lambda i: q.qgemm_grouped(x, sets[i % copies], bits, outs=outs, ws=ws), 50)
    g2 = capture(torch, lambda i: [q.qgemm(x, p, sc, bits, n, out=o, ws=ws)
                                   for (p, sc, n), o in zip(sets[i % copies], outs)], 50)
    t1 = time_steady(torch, g1, reps=4) / 200
    t2 = time_steady(torch, g2, reps=4) / 200
    nbytes = per + M * K * 2 + L * M * N * 2
    gbs = nbytes / (t1 * 1e-3) / 1e9
    del g1, g2, sets, base
    torch.cuda.empty_cache()
    return {"workload": "grouped K+V extraction, 5 drafter layers x (2560 -> 1024), W%dA16 M=16" % bits,
            "us_per_call": round(t1 * 1e3, 2), "us_five_separate_calls": round(t2 * 1e3, 2),
            "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def measure_attention(torch, q, window, B=1):
    """The drafter's sliding-window attention for one 16-token block after the
    8,192-token Long context (20 query heads, 4 KV heads of 128), over
    rotating copies of the KV cache so the window rows come from HBM."""
    import workloads
    A = workloads.ATTENTION
    T, Hq, Hkv, D = A["T"], A["Hq"], A["Hkv"], A["D"]
    S = A["context"] + T
    lo = 0 if (window == 0 or S <= window) else max(0, S - T - window // 2)
    kv_read = B * (S - lo) * Hkv * D * 2 * 2           # K and V rows any query sees
    nbytes = kv_read + 2 * B * T * Hq * D * 2           # + q and out
    copies = max(1, math.ceil(2 * MALL_BYTES / kv_read))
    qb, kb, vb = workloads.attention_inputs(B, T, Hq, Hkv, D, S, 6900)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    qt, kt, vt = bf(qb), bf(kb), bf(vb)
    k_all = torch.empty((copies, B, S, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v_all = torch.empty_like(k_all)
    k_all[:, :, lo:] = kt[:, lo:]                      # rows before lo are never read
    v_all[:, :, lo:] = vt[:, lo:]
    lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
    out = torch.empty_like(qt)
    ws = torch.zeros(max(1, q.lib().qg_swa_workspace_bytes(B, T, Hq, Hkv, D, S, window)),
                     dtype=torch.uint8, device="cuda")
    g = capture(torch, lambda i: q.swa_attention(qt, k_all[i % copies], v_all[i % copies], lens,
                                                 window, out=out, ws=ws), 100)
    us = time_steady(torch, g, reps=4) / 400 * 1e3
    del g, k_all, v_all
    torch.cuda.empty_cache()
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "drafter attention, 16-token block over 8192 + 16 cached tokens, "
                        "window %s, batch %d" % (window if window else "none (full)", B),
            "us_per_call": round(us, 2), "bytes_per_call": nbytes, "gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "cache_copies": copies}


def cpu_baseline(seconds):
    """The oracle's product for the headline step, timed on the host."""
    from oracle import gemm, numerics, quant
    import workloads
    blas_threads = _blas_threads()
    cases = []
    nbytes = 0
    for si, (K, N) in enumerate(workloads.WORKLOADS[2]["shapes"]):
        W = workloads.weights(K, N, workloads.seed_for(2, si, 0))
        sb = quant.rtn_scales(W, 4)
        codes = quant.q_s(W, numerics.scale_bits_to_f64(sb, "f16"), 4)
        x = workloads.activations(1, K, workloads.seed_for(2, si, 1))
        cases.append((x, codes, sb))
        nbytes += alg_bytes(4, 1, K, N)
    n = 0
    t0 = time.perf_counter()
    while True:
        for x, codes, sb in cases:
            gemm.gemm_ref(x, codes, sb, "f16")
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    return {"value": round(nbytes * n / dt / 1e9, 3), "unit": "GB/s", "cores": blas_threads,
            "kind": "oracle", "blas_threads": blas_threads, "host_cpus": os.cpu_count() or 0,
            "cpu_model": model,
            "sample": "%d full decode steps (gate/up 2560x19456 + down 9728x2560, M=1): "
                      "float64 dequantization + float64 matmul, %.1f s; host has %d CPUs"
                      % (n, dt, os.cpu_count() or 0)}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def _median_seconds(fn, runs):
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def cpu_oracle_rows(rows_of_prefill=1024):
    """The oracle's product (gemm_ref: exact dequantization and a float64
    library matmul), timed on the host beside each GPU row: per shape of the
    tiny, M = 16 W4A16 and W8A16 workloads, the median of 5 runs on all BLAS
    threads and of 3 on one thread (the decode shapes' single-thread figure
    is here too; their all-thread figure is the headline's cpu_baseline);
    per prefill shape the median of 3 runs on a sample of the first
    `rows_of_prefill` of the 8,192 rows (its GFLOP/s are for that sample).
    Inputs come from the same seeds as the GPU rows."""
    from oracle import gemm, numerics, quant
    import workloads
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    threads = _blas_threads()
    out = {}
    for cfg in (1, 2, 3, 4, 5):
        w = workloads.WORKLOADS[cfg]
        bits, sdt = w["bits"], ("f16" if w["bits"] == 4 else "bf16")
        for si, (K, N) in enumerate(w["shapes"]):
            W = workloads.weights(K, N, workloads.seed_for(cfg, si, 0))
            sb = quant.rtn_scales(W, bits)
            codes = quant.q_s(W, numerics.scale_bits_to_f64(sb, sdt), bits)
            del W
            M = w["M"] if cfg != 5 else rows_of_prefill
            x = workloads.activations(w["M"], K, workloads.seed_for(cfg, si, 1))[:M]
            run = lambda: gemm.gemm_ref(x, codes, sb, sdt)
            key = (cfg, si)
            if cfg == 5:
                t = _median_seconds(run, 3)
                out[key] = {"gflops": round(2 * M * K * N / t / 1e9, 2), "s_per_call": round(t, 4),
                            "threads": threads, "runs": 3,
                            "sample": "first %d of %d rows" % (M, w["M"])}
                continue
            nbytes = alg_bytes(bits, M, K, N)
            rec = {}
            if cfg != 2:
                t = _median_seconds(run, 5)
                rec.update(gbs=round(nbytes / t / 1e9, 4), s_per_call=round(t, 4),
                           threads=threads, runs=5)
            if threadpool_limits is not None:
                with threadpool_limits(limits=1):
                    t1 = _median_seconds(run, 3)
                rec.update(single_thread_gbs=round(nbytes / t1 / 1e9, 4),
                           single_thread_s_per_call=round(t1, 4))
            out[key] = rec
    return out


def attach_cpu_rows(extra, cpu):
    """Put each oracle figure beside its GPU row (same config and shape)."""
    import workloads
    by_name = {workloads.WORKLOADS[c]["name"]: c for c in workloads.WORKLOADS}
    for row in extra:
        cfg = by_name.get(row.get("workload"))
        if cfg is None:
            continue
        for si, shp in enumerate(row.get("shapes", [])):
            rec = cpu.get((cfg, si))
            if rec:
                shp["cpu_oracle"] = rec
    for row in extra:
        name = row.get("workload", "")
        for cfg in (3, 4):
            if name.startswith(workloads.WORKLOADS[cfg]["name"] + " set"):
                recs = [cpu.get((cfg, si)) for si in range(3)]
                if all(r and "s_per_call" in r for r in recs):
                    t = sum(r["s_per_call"] for r in recs)
                    row["cpu_oracle"] = {"gbs": round(row["bytes_per_step"] / t / 1e9, 4),
                                         "s_per_step": round(t, 4), "threads": recs[0]["threads"],
                                         "sample": "sum of the three shapes' medians"}


def log(msg):
    """Progress line on stderr (the JSON result alone goes to stdout)."""
    print("[bench %.1fs] %s" % (time.perf_counter() - _T0, msg), file=sys.stderr, flush=True)


_T0 = time.perf_counter()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the path has no multi-GPU step here "
              "(column or K splits across GPUs are described in the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import int8_group_quantized_amd as q
    q.lib()
    torch.cuda.init()

    up = Weights(q, torch, 2, 0, copies_for(4, 2560, 19456))
    down = Weights(q, torch, 2, 1, copies_for(4, 9728, 2560))
    up.W = down.W = None
    torch.cuda.empty_cache()

    def step(i):
        up.call(q, i)
        down.call(q, i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    graphs = graphs_for_steps(torch, step, args.steps)
    # exactly args.steps steps, timed after ~20 ms of untimed replays of the
    # same graphs (a short region timed cold reads up to ~15% slow while the
    # clocks settle), as every other row is timed
    ms = time_steps(torch, graphs, args.steps)
    step_bytes = up.bytes + down.bytes
    value = step_bytes / (ms * 1e-3) / 1e9

    k_ms = kernel_average(torch, up, q)
    k_gbs = up.bytes / (k_ms * 1e-3) / 1e9
    # Context: what one launch streaming the same weight copies reaches on this
    # GPU (the packed codes, 24.9 MB per launch), and the rate of 256 MiB reads.
    c_us, c_bytes, c_wgs = read_stream_ceiling(torch, q, up.packed)
    big = [torch.empty(1 << 28, dtype=torch.uint8, device="cuda") for _ in range(3)]
    b_us, b_bytes, b_wgs = read_stream_ceiling(torch, q, big)
    del big
    c_gbs, b_gbs = c_bytes / c_us / 1e3, b_bytes / b_us / 1e3
    roofline = {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "kernel": "gemv_kernel<4,...> gate/up K=2560 N=19456 M=1",
                "us_per_launch": round(k_ms * 1e3, 3), "bytes_per_launch": up.bytes,
                "read_stream_ceiling": {
                    "probe": "qg_read_stream, 16-byte nontemporal loads, fastest of "
                             "1024-16384 workgroups",
                    "bytes_per_launch": c_bytes, "us_per_launch": round(c_us, 3),
                    "gbs": round(c_gbs, 1), "workgroups": c_wgs,
                    "frac_of_peak": round(c_gbs / HBM_PEAK_GBS, 4),
                    "gemv_frac_of_ceiling": round(k_gbs / c_gbs, 4),
                    "large_read_bytes": b_bytes, "large_read_gbs": round(b_gbs, 1),
                    "large_read_frac_of_peak": round(b_gbs / HBM_PEAK_GBS, 4)}}
    del graphs
    up.free()
    down.free()
    torch.cuda.empty_cache()

    others = [("decode_cbm", lambda: measure_decode_cbm(torch, q, args.steps)),
              ("tiny", lambda: measure_workload(torch, q, 1)),
              ("verify", lambda: measure_workload(torch, q, 3)),
              ("verify_set", lambda: measure_set_sequence(torch, q, 3)),
              ("drafter_w8a16", lambda: measure_workload(torch, q, 4)),
              ("drafter_w8a16_set", lambda: measure_set_sequence(torch, q, 4)),
              ("prefill", lambda: measure_workload(torch, q, 5)),
              ("fp16act", lambda: measure_workload(torch, q, 2, act="f16")),
              ("pack", lambda: measure_pack(torch, q)),
              ("dequant", lambda: measure_dequant(torch, q)),
              ("fake_quant", lambda: measure_fake_quant(torch, q)),
              ("grouped_w8", lambda: measure_grouped(torch, q, 8)),
              ("grouped_w4", lambda: measure_grouped(torch, q, 4))]
    for B in (1, 8):
        for w in (1024, 2048, 0):
            others.append(("attention_b%d_w%d" % (B, w),
                           lambda w=w, B=B: measure_attention(torch, q, w, B)))
    log("headline %.3f us per step, gate/up %.3f us per launch" % (ms * 1e3, k_ms * 1e3))
    extra = []
    if not args.only_headline:
        for key, fn in others:
            if any(w in key for w in args.workload.split(",")):
                extra.append(fn())
                log("row %s done" % key)

    if args.copy_calibration:
        copy_calibration(torch)
    cpu = None if args.no_cpu else cpu_baseline(args.cpu_seconds)
    if cpu is not None:
        log("cpu baseline done; timing the oracle beside each row")
        rows = cpu_oracle_rows()
        attach_cpu_rows(extra, rows)
        single = rows.get((2, 0), {}), rows.get((2, 1), {})
        if all("single_thread_s_per_call" in r for r in single):
            t1 = sum(r["single_thread_s_per_call"] for r in single)
            cpu["single_thread_value"] = round(step_bytes / t1 / 1e9, 4)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights -> RTN INT4, N(0,1) bf16 activations)",
        "config": {"workload": "decode_w4a16_m1: gate/up K=2560 N=19456 + down K=9728 N=2560, "
                               "M=1, group 128, fp16 scales",
                   "weight_copies": [up.copies, down.copies],
                   "bytes_per_step": step_bytes},
        "roofline": roofline, "cpu_baseline": cpu, "workloads": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
