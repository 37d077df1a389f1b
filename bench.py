"""Benchmark of the W4A16 decode GEMV on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweep] [--set] [--no-cpu]

One step is one call of the fused dequantize GEMV at M = 1, K = N = 8192 (the
LLaMA-65B q/k/v/o projection at batch-1 decode), on inputs already resident in
HBM. The inputs are built by the library itself on the GPU: AWQ channel scale
from 512 calibration tokens, the 1/s fold of x, and the RTN g128 quantize-pack
(timed separately as the offline leg). The calls rotate over 16 copies of the
packed layer (>= 512 MiB) so the 256 MB Infinity Cache cannot serve them.

Prints ONE JSON line (metric, value = achieved GB/s over the timed steps,
ms_per_step = time per call including the gaps between launches, roofline of the
GEMV kernel, read floors of the same bytes, CPU-oracle baseline, and extra legs).
The timed steps are back-to-back launches queued on one stream behind a device-side
delay that outlasts their submission, so the HIP events around them time the GPU,
not the host.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMV achieved HBM GB/s (% of peak) + µs/call at M=1, K=N=8192"
HBM_PEAK_GBS = 8000.0
PEAK_FP16_TFLOPS = 2500.0  # dense fp16 MFMA peak of MI355X
ROTATE_BYTES = 1 << 29  # two Infinity Caches' worth of distinct buffers
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_m1_k8192_n8192.json")


def algorithmic_bytes(m, n, k, group=128, bits=4):
    """Bytes the method must move once: the packed codes (bits / 8 per weight) + fp16 scale
    and zero per group + fp16 x in + fp16 y out."""
    return n * k * bits // 8 + 2 * 2 * n * (k // group) + 2 * m * k + 2 * m * n


def source_hash(*names):
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "w4a16_decode_gemv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--sweep", action="store_true", help="also time the M = 1..64 batch sweep at K = N = 8192 on every kernel")
    p.add_argument("--set", dest="llama_set", action="store_true", help="also time the 7-projection LLaMA-65B set")
    p.add_argument("--block", action="store_true",
                   help="also time a LLaMA2-7B decoder block at M=1: separate projections vs q/k/v and gate/up fused")
    p.add_argument("--serving", action="store_true",
                   help="also time the batched-serving GEMMs (LLaMA2-7B shapes, M=128/256) against dense fp16")
    p.add_argument("--search", action="store_true",
                   help="also time the AWQ scale search (loss kernel and grid points) on the LLaMA2-7B block")
    p.add_argument("--formats", action="store_true",
                   help="also time the 3-bit, group-32/64 and NF4 formats at K = N = 8192")
    p.add_argument("--formats-m", default="1,4,128",
                   help="comma-separated batch sizes of the --formats table")
    p.add_argument("--formats-paths", action="store_true",
                   help="in the --formats table, also time every kernel that can take each shape")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--only-gemv", action="store_true", help="time the headline GEMV only (for profilers)")
    p.add_argument("--only-m", type=int, default=0,
                   help="time only the automatic path (or --path) at this batch M, K = N = 8192 (for profilers)")
    p.add_argument("--path", type=int, default=0,
                   help="with --only-m: the kernel (0 auto, 1 GEMV, 2 tiled MFMA, 3 small-batch MFMA, 4 K-lane MFMA, "
                        "6 x-resident MFMA)")
    p.add_argument("--small-batch-shapes", action="store_true",
                   help="also time M = 4..32 on nine LLaMA layer shapes: the automatic path, the small-batch MFMA "
                        "kernel and the x-resident MFMA kernel")
    p.add_argument("--only-serving", default="",
                   help="time only one LLaMA2-7B serving GEMM, LAYER:M with LAYER in qkvo,gate,down (the 4096->4096, "
                        "4096->11008, 11008->4096 shapes) and M in 128,256, on the tiled, K-lane and split-K kernels "
                        "(for profilers)")
    p.add_argument("--copy-probe", action="store_true",
                   help="after the GEMV, run a plain 64 MiB elementwise copy 5 times (counter calibration)")
    return p.parse_args()


class Layer:
    """One packed layer built on the GPU by the library, replicated `copies` times."""

    def __init__(self, w4, torch, cfg, layer_id, n, k, m, copies, bits=4, group=128):
        import synth

        dev = "cuda:0"
        L = synth.layer(cfg, layer_id, n, k, m)
        self.n, self.k, self.m = n, k, m
        W = torch.from_numpy(L["W"]).to(dev)
        xc = torch.from_numpy(L["x_cal"]).to(dev)
        x = torch.from_numpy(L["x"]).to(dev)
        self.s = w4.channel_scale(xc, 0.5)
        self.x = w4.scale_input(x, self.s)
        qw, sc, zr = w4.quantize_pack(W, self.s, bits=bits, group=group)
        self.bits, self.group = bits, group
        self.W = W
        self.copies = [(self.x.clone(), qw.clone(), sc.clone(), zr.clone()) for _ in range(copies)]
        self.y = [torch.empty((m, n), dtype=torch.float16, device=dev) for _ in range(copies)]
        del qw, sc, zr
        torch.cuda.synchronize()

    def call(self, w4, i, path=0):
        x, qw, sc, zr = self.copies[i % len(self.copies)]
        w4.linear(x, qw, sc, zr, out=self.y[i % len(self.y)], path=path, group=self.group, bits=self.bits)


def copies_for(nbytes):
    return max(2, -(-ROTATE_BYTES // nbytes))


def time_back_to_back(torch, fn, steps, warmup):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per call


_DELAY_MHZ = []


def delay_clock_mhz(torch):
    """Rate of the counter behind torch.cuda._sleep (its cycles), measured once with HIP events
    over a short delay (the counter need not run at the shader clock)."""
    if not _DELAY_MHZ:
        torch.cuda.synchronize()
        cycles = 2_000_000
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(cycles)
        e1.record()
        torch.cuda.synchronize()
        _DELAY_MHZ.append(cycles / max(e0.elapsed_time(e1) * 1e3, 1.0))
    return _DELAY_MHZ[0]


def time_steps_queued(torch, fn, steps, warmup):
    """The timed region: `warmup` untimed calls, then exactly `steps` calls launched back to
    back on the current stream (the stream the kernels run on) and bracketed by two HIP
    events on it, synchronized on both sides. The launches are queued behind a bounded
    device-side delay that lasts longer than the host needs to submit them, so the GPU runs
    them back to back from its queue: the events bracket the kernels and the gaps between
    them, not the host's launch cost (about as long as the kernel from Python) and not a
    graph replay's fixed start-up cost (several microseconds per replay, measured). The delay
    is sized from the host's measured submission rate and checked against its own measured
    length; a run whose submission outlasted the delay is timed again with a longer one.
    Returns ms per call."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    cycles_per_us = delay_clock_mhz(torch)
    probe = max(1, min(steps, 50))
    torch.cuda._sleep(int(20_000 * cycles_per_us))  # 20 ms: the probe's launches queue behind it
    t0 = time.perf_counter()
    for i in range(probe):
        fn(i)
    host_us = (time.perf_counter() - t0) / probe * 1e6
    torch.cuda.synchronize()
    delay_us = 3.0 * steps * host_us + 1000.0
    for _ in range(6):
        es = torch.cuda.Event(enable_timing=True)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        es.record()
        torch.cuda._sleep(int(delay_us * cycles_per_us))
        e0.record()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        e1.record()
        submit_us = (time.perf_counter() - t0) * 1e6
        torch.cuda.synchronize()
        if submit_us < 0.8 * es.elapsed_time(e0) * 1e3:
            return e0.elapsed_time(e1) / steps
        delay_us *= 2.0
    raise RuntimeError("the host could not queue the timed launches ahead of the GPU")


def time_per_launch(torch, fn, steps):
    """Average of per-launch HIP event pairs (start/end around every launch)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    d = sorted(a.elapsed_time(b) for a, b in ev)
    return sum(d) / len(d), d[len(d) // 2]


def time_graph(torch, fn, steps, reps=5, warm_ms=25.0):
    """Launches captured into one HIP graph; ms per launch over `reps` replays, after
    replays that keep the GPU busy for about `warm_ms` (right after host-side set-up the
    first replays run slower: 11 us kernels measured 1.2-1.4 us high on the first of six
    back-to-back timings, settling by the fourth)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)  # warm the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    t0 = time.perf_counter()
    n = 0
    while n < 2 or (time.perf_counter() - t0) * 1e3 < warm_ms:
        g.replay()
        torch.cuda.synchronize()
        n += 1
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * steps)


# grid-stride read shapes (threads, workgroups, 16-byte loads in flight per thread) timed
# beside the GEMV's own pattern: fewer and larger workgroups, persistent grids, other depths
GRID_READS = ((256, 1024, 8), (256, 2048, 4), (256, 4096, 2), (512, 1024, 4), (1024, 256, 8), (1024, 512, 4),
              (256, 512, 16), (64, 8192, 4))


def read_floor_leg(torch, w4, nbytes, copies, gemv_ms, steps, warmup):
    """Single-launch read floors of `nbytes`, each timed like the GEMV (back-to-back launches
    queued behind a device-side delay, over `copies` rotating buffers): the GEMV's own access
    pattern (w4a16_stream_read), grid-stride reads of other shapes (w4a16_stream_read_grid),
    and a device-to-device copy of the same bytes (hipMemcpyAsync through torch, which also
    writes them). The same read and copy of 1 GiB show the streaming rate once launch costs
    are amortised."""
    dev = "cuda:0"
    res = {"bytes": nbytes}
    buf = torch.zeros((copies, nbytes // 4), dtype=torch.int32, device=dev)
    sink = w4.stream_read(buf[0])
    t = time_steps_queued(torch, lambda i: w4.stream_read(buf[i % copies], sink), steps, warmup)
    res["gemv_pattern"] = {"us_per_call": t * 1e3, "GB_s": nbytes / (t * 1e-3) / 1e9}
    best = t
    rows = []
    gsink = torch.empty(8192, dtype=torch.int32, device=dev)
    for threads, blocks, unroll in GRID_READS:
        tg = time_steps_queued(torch, lambda i: w4.stream_read_grid(buf[i % copies], threads, blocks, unroll,
                                                                   gsink[:blocks]), min(steps, 500), 20)
        rows.append({"threads": threads, "workgroups": blocks, "loads_in_flight": unroll, "us_per_call": tg * 1e3,
                     "GB_s": nbytes / (tg * 1e-3) / 1e9})
        best = min(best, tg)
    res["grid_stride"] = rows
    dst = torch.empty_like(buf[0])
    tc = time_steps_queued(torch, lambda i: dst.copy_(buf[i % copies]), min(steps, 500), 20)
    res["copy_d2d"] = {"us_per_call": tc * 1e3, "GB_s_read_plus_write": 2 * nbytes / (tc * 1e-3) / 1e9,
                       "note": "reads and writes the bytes once each"}
    del buf, dst
    big = torch.zeros(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB
    big_dst = torch.empty_like(big)
    tb = time_steps_queued(torch, lambda i: w4.stream_read_grid(big, 256, 2048, 8, gsink[:2048]), 20, 3)
    tbc = time_steps_queued(torch, lambda i: big_dst.copy_(big), 20, 3)
    res["read_1gib"] = {"us_per_call": tb * 1e3, "GB_s": (1 << 30) / (tb * 1e-3) / 1e9,
                        "pattern": "grid-stride, 256 threads x 2048 workgroups x 8 loads"}
    res["copy_1gib"] = {"us_per_call": tbc * 1e3, "GB_s_read_plus_write": 2 * (1 << 30) / (tbc * 1e-3) / 1e9}
    del big, big_dst
    torch.cuda.empty_cache()
    res["best_single_launch_read"] = {"us_per_call": best * 1e3, "GB_s": nbytes / (best * 1e-3) / 1e9,
                                      "frac_of_peak": nbytes / (best * 1e-3) / 1e9 / HBM_PEAK_GBS}
    res["gemv_fraction_of_best_read"] = best / gemv_ms
    res["note"] = ("single-launch reads of the GEMV's bytes by several patterns, timed like the GEMV; the best of "
                   "them is the practical ceiling of one launch of this size on this device")
    return res


def small_batch_shapes_leg(w4, torch):
    """M = 4..32 on nine LLaMA projection shapes (4-bit groups of 128), graph-timed: the automatic
    path with a workspace (the binding's default), the small-batch MFMA kernel and the
    x-resident MFMA kernel. One JSON row per shape and M, also printed to stderr as it lands."""
    shapes = [(8192, 8192), (4096, 4096), (4096, 11008), (11008, 4096), (8192, 22016), (22016, 8192),
              (8192, 28672), (28672, 8192), (8192, 1024)]
    rows = []
    for k, n in shapes:
        for mm in (4, 8, 12, 16, 20, 24, 32):
            b = algorithmic_bytes(mm, n, k)
            L = Layer(w4, torch, 4, 0, n, k, mm, copies_for(b))
            r = {"K": k, "N": n, "M": mm, "bytes": b}
            r["auto_us"] = time_graph(torch, lambda i: L.call(w4, i, 0), 100) * 1e3
            r["small_batch_us"] = time_graph(torch, lambda i: L.call(w4, i, 3), 100) * 1e3
            need = w4.xres_workspace_bytes(mm, n, k)
            ws = torch.empty(max(1, need // 4), dtype=torch.float32, device=L.x.device)
            r["xres_us"] = time_graph(torch, lambda i: w4.linear_xres(*L.copies[i % len(L.copies)], workspace=ws,
                                                                      out=L.y[i % len(L.y)]), 100) * 1e3
            r["xres_ranges"] = -(-k // 2048)
            rows.append(r)
            print(json.dumps(r), file=sys.stderr, flush=True)
            del L, ws
            torch.cuda.empty_cache()
    return rows


def block_leg(w4, torch):
    """A LLaMA2-7B decoder block's quantized part at M = 1: RMSNorm (1/s folded) -> q, k, v ->
    o -> RMSNorm -> gate, up -> down, as 9 launches, against the same with q/k/v and gate/up
    stacked into single launches (6 launches). Attention itself is not part of this path; the
    o and down inputs are synthetic activations already divided by their scales (their 1/s
    folds into the preceding projection's weights)."""
    import synth

    dev = "cuda:0"
    layers = synth.CONFIGS[synth.LLAMA2_7B_BLOCK]["layers"]
    k = layers[0][1]
    eps = 1e-5
    groups = [("qkv", [0, 1, 2]), ("o", [3]), ("gate_up", [4, 5]), ("down", [6])]
    packed_bytes = sum(n * kk // 2 + 4 * n * (kk // 128) for _, kk, n in layers)
    copies = max(2, -(-ROTATE_BYTES // packed_bytes))
    base = {}
    for gname, ids in groups:
        kk = layers[ids[0]][1]
        lead = ids[0]
        s = w4.channel_scale(torch.from_numpy(synth.calibration(2, lead, kk)).to(dev), 0.5)
        W = torch.cat([torch.from_numpy(synth.weights(2, i, layers[i][2], kk)).to(dev) for i in ids], dim=0)
        packed = w4.quantize_pack(W, s)
        del W
        bounds, r0 = [], 0
        for i in ids:
            bounds.append((r0, r0 + layers[i][2]))
            r0 += layers[i][2]
        base[gname] = {"s": s, "packed": packed, "parts": bounds,
                       "x": w4.scale_input(torch.from_numpy(synth.activations(2, lead, 1, kk)).to(dev), s), "n": r0}
    h = [torch.from_numpy(synth.activations(2, 10 + j, 1, k)).to(dev) for j in range(2)]
    gamma = [torch.from_numpy((1.0 + 0.1 * np.random.default_rng(j).standard_normal(k)).astype(np.float16)).to(dev)
             for j in range(2)]
    sets = []
    for c in range(copies):
        st = {g: {"s": b["s"], "parts": b["parts"], "x": b["x"].clone(),
                  "packed": tuple(t.clone() for t in b["packed"]),
                  "y": torch.empty((1, b["n"]), dtype=torch.float16, device=dev)} for g, b in base.items()}
        st["h"], st["gamma"] = [t.clone() for t in h], gamma
        sets.append(st)
    del base
    torch.cuda.synchronize()

    def lin(g, fused):
        qw, sc, zr = g["packed"]
        if fused:
            w4.linear(g["x"], qw, sc, zr, out=g["y"])
        else:
            for a, b in g["parts"]:
                w4.linear(g["x"], qw[a:b], sc[a:b], zr[a:b], out=g["y"][:, a:b])

    def step(i, fused):
        st = sets[i % len(sets)]
        w4.rmsnorm_fold(st["h"][0], st["gamma"][0], st["qkv"]["s"], eps, out=st["qkv"]["x"])
        lin(st["qkv"], fused)
        lin(st["o"], fused)
        w4.rmsnorm_fold(st["h"][1], st["gamma"][1], st["gate_up"]["s"], eps, out=st["gate_up"]["x"])
        lin(st["gate_up"], fused)
        lin(st["down"], fused)

    t_norm = time_graph(torch, lambda i: w4.rmsnorm_fold(sets[i % len(sets)]["h"][0], sets[i % len(sets)]["gamma"][0],
                                                       sets[i % len(sets)]["qkv"]["s"], eps,
                                                       out=sets[i % len(sets)]["qkv"]["x"]), 50)
    t_sep = time_graph(torch, lambda i: step(i, False), 20)
    t_fused = time_graph(torch, lambda i: step(i, True), 20)
    norm_bytes = 2 * (2 * k * 2 + 2 * k + 4 * k + 2 * k)
    nbytes = sum(algorithmic_bytes(1, n, kk) for _, kk, n in layers) + norm_bytes
    return {"launches_separate": 9, "launches_fused": 6, "us_separate": t_sep * 1e3, "us_fused": t_fused * 1e3,
            "GB_s_separate": nbytes / (t_sep * 1e-3) / 1e9, "GB_s_fused": nbytes / (t_fused * 1e-3) / 1e9,
            "bytes": nbytes, "rotating_copies": copies, "us_rmsnorm_fold_one_row": t_norm * 1e3,
            "note": "graph-timed; q/k/v (N=12288) and gate/up (N=22016) stacked row-wise share one launch"}


SEARCH_GRID = tuple(i / 20 for i in range(21))  # the alphas the library's search visits


def search_leg(w4, torch):
    """The AWQ scale search on the LLaMA2-7B block's seven projections with 512 calibration
    tokens: per layer the original output (once per search), the loss kernel alone (one
    candidate scale), one grid point (channel scale, input fold, quantize-pack, loss) and the
    21-point search, graph-timed."""
    import synth

    dev = "cuda:0"
    rows = []
    total_search_us = 0.0
    for lid, (name, kk, nn) in enumerate(synth.CONFIGS[synth.LLAMA2_7B_BLOCK]["layers"]):
        x_cal = torch.from_numpy(synth.calibration(2, lid, kk)).to(dev)
        W = torch.from_numpy(synth.weights(2, lid, nn, kk)).to(dev)
        t_cal = x_cal.shape[0]
        s = w4.channel_scale(x_cal, 0.5)
        xs = w4.scale_input(x_cal, s)
        packed = w4.quantize_pack(W, s)
        ws = torch.empty(w4.alpha_loss_workspace(t_cal, nn), dtype=torch.float64, device=dev)
        loss = torch.empty(len(SEARCH_GRID), dtype=torch.float64, device=dev)
        y_ref = torch.empty((t_cal, nn), dtype=torch.float32, device=dev)
        t_ref = time_graph(torch, lambda i: w4.output_reference(x_cal, W, out=y_ref), 10)
        t_loss = time_graph(torch, lambda i: w4.alpha_loss(xs, *packed, y_ref, workspace=ws,
                                                           out=loss[i % 21:i % 21 + 1]), 21)

        def point(i):
            a = SEARCH_GRID[i % 21]
            w4.channel_scale(x_cal, a, out=s)
            w4.scale_input(x_cal, s, out=xs)
            w4.quantize_pack(W, s, out=packed)
            w4.alpha_loss(xs, *packed, y_ref, workspace=ws, out=loss[i % 21:i % 21 + 1])

        t_point = time_graph(torch, point, 21)
        t_scale = time_graph(torch, lambda i: w4.channel_scale(x_cal, SEARCH_GRID[i % 21], out=s), 21)
        t_fold = time_graph(torch, lambda i: w4.scale_input(x_cal, s, out=xs), 21)
        t_quant = time_graph(torch, lambda i: w4.quantize_pack(W, s, out=packed), 21)
        flop = 2 * t_cal * nn * kk  # one product of 2 T N K
        search_us = (t_ref + 21 * t_point) * 1e3
        rows.append({"layer": name, "T": t_cal, "K": kk, "N": nn, "reference_us": t_ref * 1e3,
                     "reference_TFLOP_s": flop / (t_ref * 1e-3) / 1e12,
                     "loss_us": t_loss * 1e3, "loss_TFLOP_s": flop / (t_loss * 1e-3) / 1e12,
                     "loss_mfma_util": flop / (t_loss * 1e-3) / 1e12 / PEAK_FP16_TFLOPS,
                     "grid_point_us": t_point * 1e3, "channel_scale_us": t_scale * 1e3,
                     "scale_input_us": t_fold * 1e3, "quantize_pack_us": t_quant * 1e3,
                     "search_21_us": search_us})
        total_search_us += search_us
        del x_cal, W, s, xs, packed, ws, y_ref
        torch.cuda.empty_cache()
    return {"layers": rows, "block_search_us": total_search_us,
            "note": "flops = 2 T N K per product; a search = one reference output + 21 grid points; "
                    "graph-timed, inputs resident"}


def copy_probe(torch, out):
    """A plain read-once/write-once kernel of known size (64 MiB in, 64 MiB out), run five times so
    that the HBM counters can be scaled to bytes."""
    a = torch.ones(32 << 20, dtype=torch.float16, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    out["copy_probe_bytes"] = {"read": a.numel() * 2, "write": b.numel() * 2, "kernel": "torch.mul(a, 1.0, out=b)"}


def cpu_baseline(layer, seconds):
    """The oracle on the host: its linear (O-L, NumPy float64) on whole-layer calls for
    about `seconds`, and its quantize-pack (O-Q) of the same layer for about half as long,
    each reported separately. `value` is O-L, the metric's operation."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        blas_threads = max([p.get("num_threads", 1) for p in blas] or [1])
    except Exception:  # threadpoolctl missing: report what numpy would use
        blas_threads = len(os.sched_getaffinity(0))

    def timed(fn, budget):
        n_calls, t_total = 0, 0.0
        t0 = time.perf_counter()
        while True:
            a = time.perf_counter()
            fn()
            t_total += time.perf_counter() - a
            n_calls += 1
            if time.perf_counter() - t0 >= budget and n_calls >= 2:
                return n_calls, t_total

    x = layer.x.cpu().numpy()
    qw, sc, zr = (t.cpu().numpy() for t in layer.copies[0][1:])
    qw = qw.view(np.uint32)
    n_calls, t_total = timed(lambda: oracle.linear(x, qw, sc, zr), seconds)
    us = t_total / n_calls * 1e6
    nbytes = algorithmic_bytes(layer.m, layer.n, layer.k)
    W = layer.W.cpu().numpy()
    s = layer.s.cpu().numpy()
    q_calls, q_total = timed(lambda: oracle.quantize_pack(W, s), seconds / 2)
    q_us = q_total / q_calls * 1e6
    q_bytes = layer.n * layer.k * 2 + layer.k * 4 + layer.n * layer.k // 2 + 2 * 2 * layer.n * (layer.k // 128)
    return {
        "value": nbytes / (us * 1e-6) / 1e9,
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"O-L: {n_calls} whole-layer calls of the float64 NumPy oracle linear (M=1, K=N=8192), "
                  f"{t_total:.1f} s, {us:.0f} us/call; O-Q: {q_calls} whole-layer quantize-pack calls, "
                  f"{q_total:.1f} s, {q_us:.0f} us/call. Dequantize and quantize are single-threaded NumPy, the "
                  f"matvec uses {blas_threads} BLAS threads",
        "us_per_call": us,
        "quantize_pack": {"us_per_call": q_us, "GB_s": q_bytes / (q_us * 1e-6) / 1e9, "bytes": q_bytes,
                          "calls": q_calls, "cores": 1},
    }


def traffic_entry(achieved_bytes_per_launch):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; otherwise null."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash("gemv.hip", "device_utils.h"):
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU leg (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    import torch

    import w4a16_decode_gemv_amd as w4

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    w4.load()
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)

    if args.only_serving:
        import synth

        name, mm = args.only_serving.split(":")
        mm = int(mm)
        layers = {lname.split("_")[0]: (lid, lname, kk, nn) for lid, (lname, kk, nn) in enumerate(synth.CONFIGS[synth.LLAMA2_7B_SERVING]["layers"])}
        lid, lname, kk, nn = layers[name]
        b = algorithmic_bytes(mm, nn, kk)
        L = Layer(w4, torch, 5, lid, nn, kk, mm, copies_for(b))
        ws = torch.empty(w4.splitk_workspace_bytes(mm, nn, kk, 16) // 4, dtype=torch.float32, device=L.x.device)
        t_tiled = time_steps_queued(torch, lambda i: L.call(w4, i, 2), args.steps, args.warmup)
        t_klane = time_steps_queued(torch, lambda i: L.call(w4, i, 4), args.steps, args.warmup)
        t_split = time_steps_queued(torch, lambda i: w4.linear_splitk(*L.copies[i % len(L.copies)], workspace=ws,
                                                                       out=L.y[i % len(L.y)]), args.steps, args.warmup)
        flop = 2 * mm * nn * kk
        res = {"layer": lname, "M": mm, "K": kk, "N": nn, "flop": flop, "algorithmic_bytes": b,
               "tiled_us": t_tiled * 1e3, "klane_us": t_klane * 1e3, "splitk_us": t_split * 1e3,
               "splitk_default_splits": w4.splitk_workspace_bytes(mm, nn, kk, 0) // (4 * mm * nn),
               "tiled_mfma_util": flop / (t_tiled * 1e-3) / 1e12 / PEAK_FP16_TFLOPS,
               "klane_mfma_util": flop / (t_klane * 1e-3) / 1e12 / PEAK_FP16_TFLOPS,
               "splitk_mfma_util": flop / (t_split * 1e-3) / 1e12 / PEAK_FP16_TFLOPS}
        print(json.dumps(res), flush=True)
        return 0

    if args.only_m:
        mm = args.only_m
        b = algorithmic_bytes(mm, 8192, 8192)
        L = Layer(w4, torch, 4, 0, 8192, 8192, mm, copies_for(b))
        if args.path == 6:
            ws = torch.empty(max(1, w4.xres_workspace_bytes(mm, 8192, 8192) // 4), dtype=torch.float32,
                             device=L.x.device)
            t = time_steps_queued(torch, lambda i: w4.linear_xres(*L.copies[i % len(L.copies)], workspace=ws,
                                                                  out=L.y[i % len(L.y)]), args.steps, args.warmup)
        else:
            t = time_steps_queued(torch, lambda i: L.call(w4, i, args.path), args.steps, args.warmup)
        res = {"M": mm, "K": 8192, "N": 8192, "path": args.path, "us_per_call": t * 1e3, "GB_s": b / (t * 1e-3) / 1e9,
               "algorithmic_bytes_per_call": b}
        if args.copy_probe:
            copy_probe(torch, res)
        print(json.dumps(res), flush=True)
        return 0

    n = k = 8192
    m = 1
    nbytes = algorithmic_bytes(m, n, k)
    layer = Layer(w4, torch, 3, 0, n, k, m, copies_for(nbytes))
    fn = lambda i: layer.call(w4, i)  # noqa: E731

    # ---- the timed region: exactly `steps` back-to-back calls, synchronized on both sides
    ms = time_steps_queued(torch, fn, args.steps, args.warmup)
    value = nbytes / (ms * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "W4A16 linear M=1 K=8192 N=8192 (LLaMA-65B q/k/v/o projection, batch-1 decode), "
                        "4-bit g128 asymmetric, fp16 x/y, fp32 accumulate",
            "M": m, "K": k, "N": n, "group": 128,
            "rotating_copies": len(layer.copies),
            "algorithmic_bytes_per_call": nbytes,
            "device": props.name, "cus": props.multi_processor_count,
        },
    }
    if args.copy_probe:
        copy_probe(torch, out)
    if args.only_gemv:
        print(json.dumps(out), flush=True)
        return 0

    # ---- roofline of the GEMV kernel: algorithmic bytes per launch over the
    # average launch duration of the timed region (HIP events on the stream the
    # kernel runs on; back-to-back launches, so any gap between launches counts)
    achieved = nbytes / (ms * 1e-3) / 1e9
    out["roofline"] = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic_entry(nbytes),
        "us_per_launch": ms * 1e3,
        "timing": f"HIP events around the {args.steps} timed GEMV launches, queued back to back behind a device-side "
                  f"delay that outlasts their submission, so that neither host launch cost nor graph start-up is timed",
    }
    # the single-launch read floor of the same bytes, by several read patterns
    out["read_floor"] = read_floor_leg(torch, w4, nbytes, len(layer.copies), ms, args.steps, args.warmup)
    eager_ms = time_back_to_back(torch, fn, args.steps, args.warmup)
    avg_ms, med_ms = time_per_launch(torch, fn, min(args.steps, 400))
    graph_ms = time_graph(torch, fn, 200)
    out["timings_us"] = {
        "timed_region_per_call": ms * 1e3,
        "eager_back_to_back_per_call": eager_ms * 1e3,
        "per_launch_event_pair_mean": avg_ms * 1e3,
        "per_launch_event_pair_median": med_ms * 1e3,
        "graph_per_launch": graph_ms * 1e3,
    }

    # ---- offline leg: quantize-pack of the same layer
    qout = tuple(t.clone() for t in layer.copies[0][1:])
    qfn = lambda i: w4.quantize_pack(layer.W, layer.s, out=qout)  # noqa: E731
    q_ms = time_back_to_back(torch, qfn, 20, 3)
    q_bytes = n * k * 2 + k * 4 + n * k // 2 + 2 * 2 * n * (k // 128)
    out["quantize_pack"] = {"us_per_call": q_ms * 1e3, "GB_s": q_bytes / (q_ms * 1e-3) / 1e9,
                            "bytes": q_bytes, "note": "offline: fp16 W + fp32 s in, packed codes/scales/zeros out"}

    if args.llama_set:
        import synth

        total_bytes, total_us, per = 0, 0.0, []
        for lid, (name, kk, nn) in enumerate(synth.CONFIGS[synth.LLAMA65B_DECODE]["layers"]):
            if name in ("k", "v", "o"):
                continue
            b = algorithmic_bytes(1, nn, kk)
            L = Layer(w4, torch, 3, lid, nn, kk, 1, copies_for(b))
            t = time_graph(torch, lambda i: L.call(w4, i), 100)
            reps = 4 if name == "q" else 1
            per.append({"layer": name, "K": kk, "N": nn, "us": t * 1e3, "GB_s": b / (t * 1e-3) / 1e9, "count": reps})
            total_bytes += reps * b
            total_us += reps * t * 1e3
            del L
            torch.cuda.empty_cache()
        out["llama65b_set"] = {"us": total_us, "GB_s": total_bytes / (total_us * 1e-6) / 1e9, "layers": per}

    if args.sweep:
        import synth

        rows = []
        names = {0: "auto", 1: "gemv", 2: "mfma_tiled", 3: "mfma_small_batch"}
        for mm in (1, 2, 3, 4, 8, 16, 32, 48, 64):
            b = algorithmic_bytes(mm, 8192, 8192)
            L = Layer(w4, torch, 4, 0, 8192, 8192, mm, copies_for(b))
            for path in (1, 3, 2, 0):
                if (path == 1 and mm > w4.gemv_max_m()) or (path == 3 and mm > 32):
                    continue
                t = time_graph(torch, lambda i: L.call(w4, i, path), 100)
                rows.append({"M": mm, "path": names[path], "us": t * 1e3,
                             "GB_s": b / (t * 1e-3) / 1e9, "TFLOP_s": 2 * mm * 8192 * 8192 / (t * 1e-3) / 1e12})
            del L
            torch.cuda.empty_cache()
        out["sweep_k8192_n8192"] = rows

    if args.small_batch_shapes:
        out["small_batch_shapes"] = small_batch_shapes_leg(w4, torch)

    if args.block:
        out["llama2_7b_block"] = block_leg(w4, torch)

    if args.search:
        out["awq_search_llama2_7b"] = search_leg(w4, torch)

    if args.formats:
        ms_list = [int(v) for v in args.formats_m.split(",")]

        def paths_for(mm, bits, group):
            # the kernels that take this shape: GEMV (M <= 8), small-batch MFMA (M <= 32), tiled
            if not args.formats_paths:
                return []
            return ([1] if mm <= 8 else []) + ([3] if mm <= 32 else []) + [2]

        def row(fmt, mm, b, call, paths):
            t = time_graph(torch, lambda i: call(i, 0), 100)
            r = dict(fmt, M=mm, us=t * 1e3, bytes=b, GB_s=b / (t * 1e-3) / 1e9,
                     TFLOP_s=2 * mm * 8192 * 8192 / (t * 1e-3) / 1e12)
            if paths:
                r["us_by_path"] = {str(p): time_graph(torch, lambda i, p=p: call(i, p), 100) * 1e3 for p in paths}
            return r

        rows = []
        for bits, group in ((4, 128), (4, 64), (4, 32), (3, 128), (3, 64), (3, 32)):
            for mm in ms_list:
                b = algorithmic_bytes(mm, 8192, 8192, group, bits)
                L = Layer(w4, torch, 3, 0, 8192, 8192, mm, copies_for(b), bits=bits, group=group)
                rows.append(row({"bits": bits, "group": group}, mm, b, lambda i, p: L.call(w4, i, path=p),
                                paths_for(mm, bits, group)))
                print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
                del L
                torch.cuda.empty_cache()
        # NF4 (blocks of 64, float32 absmax) on the same layer
        import synth

        W = torch.from_numpy(synth.weights(3, 0, 8192, 8192)).to("cuda:0")
        for mm in ms_list:
            b = 8192 * 8192 // 2 + 4 * 8192 * (8192 // 64) + 2 * mm * 8192 * 2
            copies = copies_for(b)
            packs = [w4.nf4_quantize_pack(W, None, block=64) for _ in range(copies)]
            xq = torch.from_numpy(synth.activations(3, 0, mm, 8192)).to("cuda:0")
            yq = torch.empty((mm, 8192), dtype=torch.float16, device="cuda:0")
            rows.append(row({"format": "nf4", "group": 64}, mm, b,
                            lambda i, p: w4.nf4_linear(xq, *packs[i % copies], block=64, out=yq, path=p),
                            paths_for(mm, 4, 64)))
            print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
            del packs
            torch.cuda.empty_cache()
        del W
        out["formats_k8192_n8192"] = rows

    if args.serving:
        import synth

        rows = []
        for lid, (name, kk, nn) in enumerate(synth.CONFIGS[synth.LLAMA2_7B_SERVING]["layers"]):
            for mm in (128, 256):
                b = algorithmic_bytes(mm, nn, kk)
                L = Layer(w4, torch, 5, lid, nn, kk, mm, copies_for(b))
                t = time_graph(torch, lambda i: L.call(w4, i), 50)
                t_tiled = time_graph(torch, lambda i: L.call(w4, i, 2), 50)
                t_klane = time_graph(torch, lambda i: L.call(w4, i, 4), 50)
                # dense fp16 reference product of the same shape: y = x @ W^T with W^T stored [K][N]
                wt = [L.W.t().contiguous() for _ in range(copies_for(nn * kk * 2))]
                xd = L.x
                yd = torch.empty((mm, nn), dtype=torch.float16, device=xd.device)
                td = time_graph(torch, lambda i: torch.matmul(xd, wt[i % len(wt)], out=yd), 50)
                td_lt = None
                try:  # the same product with torch's hipBLASLt backend, where this build has it
                    prev = torch.backends.cuda.preferred_blas_library()
                    torch.backends.cuda.preferred_blas_library("cublaslt")
                    td_lt = time_graph(torch, lambda i: torch.matmul(xd, wt[i % len(wt)], out=yd), 50)
                    torch.backends.cuda.preferred_blas_library(prev)
                except (RuntimeError, AttributeError):
                    pass
                flop = 2 * mm * nn * kk
                ws = torch.empty(w4.splitk_workspace_bytes(mm, nn, kk, 16) // 4, dtype=torch.float32,
                                 device=xd.device)
                split_rows = {}
                for sp in (0, 2, 4, 8, 16):
                    if sp > kk // 128:
                        continue
                    ts = time_graph(torch, lambda i: w4.linear_splitk(*L.copies[i % len(L.copies)], splits=sp,
                                                                       workspace=ws, out=L.y[i % len(L.y)]), 50)
                    split_rows["auto" if sp == 0 else str(sp)] = ts * 1e3
                t_split = split_rows["auto"]
                rows.append({"layer": name, "M": mm, "K": kk, "N": nn, "us": t * 1e3,
                             "tiled_us": t_tiled * 1e3, "klane_us": t_klane * 1e3,
                             "splitk_us": t_split, "splitk_TFLOP_s": flop / (t_split * 1e-6) / 1e12,
                             "splitk_mfma_util": flop / (t_split * 1e-6) / 1e12 / PEAK_FP16_TFLOPS,
                             "splitk_by_splits_us": split_rows,
                             "TFLOP_s": flop / (t * 1e-3) / 1e12, "mfma_util": flop / (t * 1e-3) / 1e12 / PEAK_FP16_TFLOPS,
                             "dense_fp16_us": td * 1e3, "dense_fp16_TFLOP_s": flop / (td * 1e-3) / 1e12,
                             "speedup_vs_dense": td / t,
                             "dense_fp16_hipblaslt_us": None if td_lt is None else td_lt * 1e3,
                             "speedup_vs_dense_hipblaslt": None if td_lt is None else td_lt / t})
                del L, wt, ws
                torch.cuda.empty_cache()
        out["serving_llama2_7b"] = rows

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(layer, args.cpu_seconds)

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
