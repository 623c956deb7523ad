#!/usr/bin/env python
"""Benchmark of the BitNet b1.58 BitLinear forward on one MI355X.

Headline (one JSON line on stdout): decode GB/s of one Llama-3-8B layer at T = 1 --
the seven projections q, k, v, o, gate, up, down -- as % of the 8 TB/s HBM peak.
A step is one pass of the per-token hot path over that layer: one grouped launch of
the fused RMSNorm + absmax int8 quantizer (four distinct inputs: attention input,
attention output, MLP input, MLP middle; attention itself is excluded) and one grouped
launch of the ternary GEMV over the seven projections. Weight quantization runs once
before timing (it is the offline conversion step) and is timed separately. Steps
cycle through 32 distinct copies of the packed layer (1.75 GB) so that the 256 MB
last-level cache cannot serve repeated weights; steps are replayed from a HIP graph.

Also reported, as extra objects of the same line: prefill int8 TOPS (T = 2048,
(N, K) = (14336, 4096) and (4096, 14336)) as % of the 5.0 POPS int8 MFMA peak; the
70B-shape token sweep; the full 32-layer x 7-projection pass at T = 16; the weight
quantizer; and the CPU oracle on a bounded sample of the decode workload.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA
METRIC = "BitLinear decode GB/s (% HBM peak) and prefill int8 TOPS (% MFMA peak)"
REPLICAS = 32


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only-decode", action="store_true", help="skip the extra workloads")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy kernel (counter calibration)")
    ap.add_argument("--counter-pass", type=int, default=0, metavar="N",
                    help="hardware-counter pass: N eager decode steps and the calibration "
                         "copy, no graphs and no JSON line (for rocprofv3 --pmc)")
    ap.add_argument("--prefill-pass", type=int, default=0, metavar="N",
                    help="profiling pass: N eager prefill products per prefill shape, no "
                         "graphs and no JSON line (for rocprofv3 --kernel-trace / --pmc)")
    ap.add_argument("--sweep-pass", type=int, default=0, metavar="N",
                    help="profiling pass: N eager products per 70B sweep point, no JSON line")
    ap.add_argument("--fullpass-pass", type=int, default=0, metavar="N",
                    help="profiling pass: N eager 32-layer T = 16 passes, no JSON line")
    return ap.parse_args()


# ---------------------------------------------------------------- HBM traffic counters

def counted_traffic():
    """HBM bytes per grouped GEMV launch from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE passes scaled by a copy kernel of known size), or None when the kernel, its
    launch plan or its build flags have changed since the counters were taken."""
    import hashlib
    rec_path = os.path.join(ROOT, "profiles", "gemv_kernel_decode8b_counters.json")
    try:
        rec = json.load(open(rec_path))
        checks = rec.get("sources") or {rec["source"]: rec.get("source_sha256")}
        for path, digest in checks.items():
            if hashlib.sha256(open(os.path.join(ROOT, path), "rb").read()).hexdigest() != digest:
                return None
    except (OSError, ValueError, KeyError, AttributeError):
        return None
    return rec.get("traffic_bytes_per_dispatch")


# ---------------------------------------------------------------- timing helpers

def _warm_then_capture(torch, fns):
    """Run fns once eagerly (first-launch setup happens outside capture), then capture
    them, in order, into one HIP graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns[: min(len(fns), 4)]:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def _time_graph(torch, g, reps=1):
    """Average ms per replay of graph g, from HIP events on the replay stream."""
    st = torch.cuda.Event(enable_timing=True)
    en = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    st.record()
    for _ in range(reps):
        g.replay()
    en.record()
    en.synchronize()
    return st.elapsed_time(en) / reps


def _time_graph_samples(torch, g, reps, per):
    """Per-unit ms of each of `reps` replays of graph g (each replay runs `per` units),
    from HIP events on the replay stream."""
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        g.replay()
        ev[i + 1].record()
    ev[-1].synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) / per for i in range(reps)]


def _stats_us(samples_ms):
    """median, p10, p90 (microseconds) of per-unit times."""
    import numpy as np
    a = np.asarray(samples_ms, dtype=np.float64) * 1e3
    return {"median_us": round(float(np.median(a)), 3), "p10_us": round(float(np.percentile(a, 10)), 3),
            "p90_us": round(float(np.percentile(a, 90)), 3), "samples": int(a.size)}


def read_clocks(torch):
    """Current shader (sclk) and memory (mclk) clock levels of the GPU in use, from the
    driver's sysfs files (the level marked with '*'); None where unreadable."""
    import glob
    out = {"sclk_mhz": None, "mclk_mhz": None}
    try:
        p = torch.cuda.get_device_properties(0)
        bus = "%04x:%02x:%02x" % (getattr(p, "pci_domain_id", 0), p.pci_bus_id, p.pci_device_id)
    except Exception:  # noqa: BLE001 (property names differ between builds)
        return out
    for card in glob.glob("/sys/class/drm/card[0-9]*/device"):
        try:
            if bus not in os.path.realpath(card):
                continue
            for key, f in (("sclk_mhz", "pp_dpm_sclk"), ("mclk_mhz", "pp_dpm_mclk")):
                for line in open(os.path.join(card, f)):
                    if "*" in line:
                        out[key] = int(line.split(":")[1].strip().lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            continue
    return out


def gemv_bytes(T, N, K):
    """Algorithmic bytes of one projection's product: packed W, Xq, token scales,
    beta, fp32 outputs."""
    return N * K // 4 + T * K + 4 * T + 4 + 4 * T * N


def act_bytes(T, K):
    """Algorithmic bytes of one activation quantization: fp32 in, int8 + scale out."""
    return 4 * T * K + T * K + 4 * T


# ---------------------------------------------------------------- decode8b (headline)

# The headline layer is laid out as one allocation per replica: q|k|v (rows of q, then k,
# then v), o, gate|up, down, each a [N, K/4] block of packed rows; the fused q|k|v and
# gate|up blocks carry one scale per segment (q's 4096 rows as four 1024-row scale
# groups, k and v one each; gate and up one each), so the grouped product sees four
# projections -- one per distinct input -- instead of seven.
FUSED = (("qkv", ("q", "k", "v"), "attn_in"), ("o", ("o",), "attn_out"),
         ("gateup", ("gate", "up"), "mlp_in"), ("down", ("down",), "mlp_mid"))


def _segments(workloads, parts):
    """Rows per scale group of a fused block (the gcd of its parts' rows) and the part
    each group belongs to."""
    rows = [workloads.LLAMA3_8B[p][0] for p in parts]
    rpg = math.gcd(*rows)
    return rpg, [p for p, n in zip(parts, rows) for _ in range(n // rpg)]


def setup_decode(torch, bl, workloads, T=1):
    dev = torch.device("cuda:0")
    L = workloads.LLAMA3_8B
    Ws = workloads.decode8b_layer(0)
    packed_b = sum(N * K // 4 for (N, K) in L.values())
    # replica 0: the seven projections quantized into their places of one allocation
    buf0 = torch.empty(packed_b, dtype=torch.uint8, device=dev)
    ws = torch.empty(max(bl.bitlinear_weight_workspace_bytes(*L[p]) for p in L), dtype=torch.uint8,
                     device=dev)
    views, betas, off = {}, {}, 0
    blocks = {}
    for name, parts, _ in FUSED:
        start = off
        for p in parts:
            N, K = L[p]
            views[p] = buf0[off: off + N * K // 4].view(N, K // 4)
            betas[p] = torch.empty(1, dtype=torch.float32, device=dev)
            bl.bitlinear_quantize_weights(torch.from_numpy(Ws[p]).to(dev), views[p], betas[p], None, ws)
            off += N * K // 4
        blocks[name] = (start, off)
    torch.cuda.synchronize()
    del ws
    # per-segment scales of the fused blocks (read only, shared by the replicas)
    seg_betas, groups = {}, {}
    for name, parts, _ in FUSED:
        rpg, seg = _segments(workloads, parts)
        seg_betas[name] = torch.cat([betas[p] for p in seg])
        groups[name] = len(seg)
    # distinct copies of the packed layer (same content, distinct HBM addresses)
    bufs = [buf0] + [buf0.clone() for _ in range(REPLICAS - 1)]
    inputs = workloads.decode8b_inputs(T, 100)
    acts = {}
    act_entries = []
    for name, X in inputs.items():
        Xg = torch.from_numpy(X).to(dev)
        Xq = torch.empty(X.shape, dtype=torch.int8, device=dev)
        xs = torch.empty(T, dtype=torch.float32, device=dev)
        acts[name] = (Xq, xs)
        act_entries.append((Xg, None, Xq, xs))
    qa = bl.prepare_quantize_acts_grouped(act_entries, T)
    outs = {name: torch.empty((T, sum(L[p][0] for p in parts)), dtype=torch.float32, device=dev)
            for name, parts, _ in FUSED}
    fws, fws7, layer_views = [], [], []
    for buf in bufs:
        entries = []
        for name, parts, inp in FUSED:
            a, b = blocks[name]
            K = L[parts[0]][1]
            Xq, xs = acts[inp]
            entries.append((Xq, xs, buf[a:b].view(-1, K // 4), seg_betas[name], outs[name], None))
        fws.append(bl.prepare_forward_grouped_scale_groups(entries, [groups[n] for n, _, _ in FUSED], T))
        # the same bytes as seven separate projections (context: the unfused launch)
        e7, v7, off = [], [], 0
        for name, parts, inp in FUSED:
            Xq, xs = acts[inp]
            for p in parts:
                N, K = L[p]
                v = buf[off: off + N * K // 4].view(N, K // 4)
                off += N * K // 4
                v7.append(v)
                e7.append((Xq, xs, v, betas[p], torch.empty((T, N), dtype=torch.float32, device=dev), None))
        fws7.append(bl.prepare_forward_grouped(e7, T))
        layer_views.append(v7)
    gemv_b = sum(gemv_bytes(T, N, K) for (N, K) in L.values())
    act_b = sum(act_bytes(T, L[ps[0]][1]) for ps in workloads.LLAMA3_8B_INPUTS.values())
    return {"qa": qa, "fws": fws, "fws7": fws7, "gemv_bytes": gemv_b, "act_bytes": act_b,
            "packed_bytes": packed_b, "bufs": bufs, "layer_views": layer_views, "Ws": Ws,
            "inputs": inputs, "outs": outs, "acts": acts, "views0": views, "betas": betas}


def run_decode(torch, bl, d, steps, warmup):
    qa, fws = d["qa"], d["fws"]

    def step_fns(n, offset=0):
        out = []
        for i in range(n):
            f = fws[(offset + i) % len(fws)]
            out += [qa, f]
        return out

    g_warm = _warm_then_capture(torch, step_fns(max(warmup, 1)))
    g_main = _warm_then_capture(torch, step_fns(steps, warmup))
    clk0 = read_clocks(torch)
    if warmup > 0:
        g_warm.replay()
    torch.cuda.synchronize()
    ms_total = _time_graph(torch, g_main, 1)   # the K timed steps
    clk1 = read_clocks(torch)
    ms_step = ms_total / steps
    step_stats = _stats_us(_time_graph_samples(torch, g_main, 21, steps))
    # the dominant kernel alone: 256 back-to-back grouped GEMV launches, graph-replayed
    n_k = 256
    g_k = _warm_then_capture(torch, [fws[i % len(fws)] for i in range(n_k)])
    g_k.replay()
    gemv_samples = _time_graph_samples(torch, g_k, 11, n_k)
    ms_gemv = sum(gemv_samples) / len(gemv_samples)
    g_7 = _warm_then_capture(torch, [d["fws7"][i % len(fws)] for i in range(n_k)])
    g_7.replay()
    ms_gemv7 = _time_graph(torch, g_7, 2) / n_k
    g_a = _warm_then_capture(torch, [qa] * 128)
    g_a.replay()
    ms_act = _time_graph(torch, g_a, 2) / 128
    # the read roof of the same bytes: one read of a replica's allocation, and of the
    # seven projection views of it, rotating over the replicas like the products
    # (each of the four block schedules of the read kernel; the fastest is the roof)
    sink = torch.empty(bl.ROOF_READ_SINK_BYTES, dtype=torch.uint8, device="cuda:0")
    bufs = d["bufs"]

    def read_ms(parts):
        best = None
        for sched in (0, 1, 2, 3):
            g_r = _warm_then_capture(torch, [lambda p=parts(i), s=sched: bl.bitlinear_roof_read(p, sink, s)
                                             for i in range(n_k)])
            g_r.replay()
            ms = _time_graph(torch, g_r, 2) / n_k
            best = ms if best is None or ms < best else best
        return best

    ms_read = read_ms(lambda i: [bufs[i % len(bufs)]])
    ms_read7 = read_ms(lambda i: d["layer_views"][i % len(bufs)])
    # eager launches (no graph), for reference
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for f in step_fns(64):
        f()
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / 64
    return {"ms_step": ms_step, "ms_gemv": ms_gemv, "ms_act": ms_act, "ms_eager": ms_eager,
            "ms_gemv7": ms_gemv7, "ms_read": ms_read, "ms_read7": ms_read7,
            "step_stats": step_stats, "gemv_stats": _stats_us(gemv_samples),
            "clocks_before": clk0, "clocks_after": clk1}


def run_decode_per_projection(torch, bl, d, n_k=256):
    """Each decode8b projection launched alone (n_k graph-replayed launches rotating over
    the replicas): us, GB/s and % of HBM. k, v and q, o are too small to stream at full
    rate: their time is mostly the launch."""
    per_proj = {}
    names = [(p, inp) for _, parts, inp in FUSED for p in parts]
    for j, (p, inp) in enumerate(names):
        Xq, xs = d["acts"][inp]
        T = Xq.shape[0]
        v0 = d["layer_views"][0][j]
        N, K = v0.shape[0], v0.shape[1] * 4
        Y = torch.empty((T, N), dtype=torch.float32, device=Xq.device)
        fp = [bl.prepare_forward_grouped([(Xq, xs, views[j], d["betas"][p], Y, None)], T)
              for views in d["layer_views"]]
        g_p = _warm_then_capture(torch, [fp[i % len(fp)] for i in range(n_k)])
        g_p.replay()
        ms_p = _time_graph(torch, g_p, 2) / n_k
        gbs = gemv_bytes(T, N, K) / (ms_p * 1e-3) / 1e9
        per_proj[p] = {"N": N, "K": K, "us": round(ms_p * 1e3, 3), "gbs": round(gbs, 1),
                       "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    return per_proj


def run_mfma_roof(torch, bl, iters=2000):
    """The int8 matrix-core roof measured on the part: 2 workgroups of 4 waves per CU,
    each wave 8 * iters independent 32x32x32 int8 MFMAs; and the shader clock the waves
    saw (s_memtime against the 100 MHz s_memrealtime)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = 2 * cus
    sink = torch.empty(wgs * 256, dtype=torch.int32, device="cuda:0")
    clocks = torch.empty(wgs * 16, dtype=torch.int64, device="cuda:0")
    f = lambda: bl.bitlinear_roof_mfma_i8(iters, wgs, sink, clocks)  # noqa: E731
    f()
    torch.cuda.synchronize()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    for _ in range(3):
        f()
    en.record()
    en.synchronize()
    ms = st.elapsed_time(en) / 3
    ops = float(wgs) * 4 * 8 * iters * 65536
    c = clocks.view(-1, 4).cpu().double()
    ghz = ((c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / 100.0)).median().item() / 1e3
    return {"kernel": "roof_mfma_kernel (v_mfma_i32_32x32x32_i8, register operands)",
            "tops": round(ops / (ms * 1e-3) / 1e12, 1),
            "frac_int8_peak": round(ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
            "shader_clock_ghz": round(ghz, 3), "cus": cus}


# ---------------------------------------------------------------- extra workloads

def run_prefill(torch, bl, workloads):
    dev = torch.device("cuda:0")
    T = workloads.PREFILL_T
    out = []
    for (N, K) in workloads.PREFILL_SHAPES:
        W = torch.from_numpy(workloads.weights(N, K, 7)).to(dev)
        packed, beta = bl.quantize_weights(W)
        del W
        Xs = [torch.from_numpy(workloads.acts_student_t(T, K, 8 + i)).to(dev) for i in range(4)]
        Xq = torch.empty((T, K), dtype=torch.int8, device=dev)
        xs = torch.empty(T, dtype=torch.float32, device=dev)
        Y = torch.empty((T, N), dtype=torch.float32, device=dev)
        qas = [bl.prepare_quantize_acts_grouped([(X, None, Xq, xs)], T) for X in Xs]
        fw = bl.prepare_forward_grouped([(Xq, xs, packed, beta, Y, None)], T)
        qas[0]()
        g = _warm_then_capture(torch, [fw] * 20)
        g.replay()
        ms = _time_graph(torch, g, 3) / 20
        ga = _warm_then_capture(torch, [qas[i % 4] for i in range(16)])
        ga.replay()
        ms_a = _time_graph(torch, ga, 3) / 16
        ops = 2.0 * T * N * K
        tops = ops / (ms * 1e-3) / 1e12
        # context: the library int8 GEMM (torch._int_mm) on the same product with the
        # weights unpacked to one int8 per code (4x the weight bytes)
        lib = None
        try:
            codes = torch.randint(-1, 2, (K, N), dtype=torch.int8, device=dev)
            gl = _warm_then_capture(torch, [lambda: torch._int_mm(Xq, codes)] * 10)
            gl.replay()
            ms_l = _time_graph(torch, gl, 3) / 10
            lib = round(ops / (ms_l * 1e-3) / 1e12, 1)
            del codes
        except (RuntimeError, AttributeError):
            lib = None
        out.append({"T": T, "N": N, "K": K, "kernel": bl.bitlinear_forward_choice(T, N, K),
                    "ms": round(ms, 5), "tops": round(tops, 1),
                    "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
                    "torch_int_mm_tops": lib,
                    "act_quant_ms": round(ms_a, 5),
                    "act_quant_gbs": round(act_bytes(T, K) / (ms_a * 1e-3) / 1e9, 1)})
        del Xs, Xq, Y, packed
        torch.cuda.empty_cache()
    return out


def run_prefill_pass(torch, bl, workloads, n):
    """n eager launches of the prefill product per prefill shape (each dispatch on its own,
    for the profiler); inputs as in run_prefill."""
    dev = torch.device("cuda:0")
    T = workloads.PREFILL_T
    for (N, K) in workloads.PREFILL_SHAPES:
        W = torch.from_numpy(workloads.weights(N, K, 7)).to(dev)
        packed, beta = bl.quantize_weights(W)
        del W
        X = torch.from_numpy(workloads.acts_student_t(T, K, 8)).to(dev)
        Xq, xs = bl.quantize_acts(X)
        Y = torch.empty((T, N), dtype=torch.float32, device=dev)
        fw = bl.prepare_forward_grouped([(Xq, xs, packed, beta, Y, None)], T)
        for _ in range(n):
            fw()
        torch.cuda.synchronize()
        print("prefill pass: %d products at T=%d N=%d K=%d (%s)"
              % (n, T, N, K, bl.bitlinear_forward_choice(T, N, K)), flush=True)
        del X, Xq, Y, packed
        torch.cuda.empty_cache()


def run_sweep_pass(torch, bl, workloads, n):
    """n eager products per 70B sweep point (each dispatch on its own, for the profiler)."""
    run_sweep70b(torch, bl, workloads, eager=n)


def run_sweep70b(torch, bl, workloads, eager=0):
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    out = []
    for which, (N, K) in workloads.LLAMA_70B_SWEEP.items():
        gen.manual_seed(70)
        W = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * workloads.WEIGHT_SIGMA
        packed, beta = bl.quantize_weights(W)
        del W
        reps = [packed] + [packed.clone() for _ in range(7)]   # 8 x 58.7 MB > last-level cache
        for T in workloads.SWEEP_TOKENS:
            X = torch.from_numpy(workloads.acts_normal(T, K, 1000 + T)).to(dev)
            Xq, xs = bl.quantize_acts(X)
            Y = torch.empty((T, N), dtype=torch.float32, device=dev)
            fws = [bl.prepare_forward_grouped([(Xq, xs, p, beta, Y, None)], T) for p in reps]
            if eager:
                for i in range(eager):
                    fws[i % 8]()
                torch.cuda.synchronize()
                print("sweep pass: %d products, %s T=%d (%s)"
                      % (eager, which, T, bl.bitlinear_forward_choice(T, N, K)), flush=True)
                continue
            g = _warm_then_capture(torch, [fws[i % 8] for i in range(64)])
            g.replay()
            samples = _time_graph_samples(torch, g, 5, 64)
            ms = sum(samples) / len(samples)
            b = gemv_bytes(T, N, K)
            gbs = b / (ms * 1e-3) / 1e9
            out.append({"proj": which, "N": N, "K": K, "T": T,
                        "kernel": bl.bitlinear_forward_choice(T, N, K), "us": round(ms * 1e3, 2),
                        "timing": _stats_us(samples),
                        "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                        "tops": round(2.0 * T * N * K / (ms * 1e-3) / 1e12, 2)})
        del reps, packed
        torch.cuda.empty_cache()
    return out


def run_fullpass(torch, bl, workloads, eager=0):
    dev = torch.device("cuda:0")
    T = workloads.FULLPASS_T
    gen = torch.Generator(device=dev)
    fns = []
    keep = []
    total_b = 0
    for layer in range(workloads.LLAMA3_8B_LAYERS):
        packed = {}
        for i, (p, (N, K)) in enumerate(workloads.LLAMA3_8B.items()):
            gen.manual_seed(layer * 16 + i)
            W = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * workloads.WEIGHT_SIGMA
            packed[p] = bl.quantize_weights(W)
            del W
            total_b += gemv_bytes(T, N, K)
        act_entries, acts = [], {}
        for j, (name, ps) in enumerate(workloads.LLAMA3_8B_INPUTS.items()):
            K = workloads.LLAMA3_8B[ps[0]][1]
            X = torch.from_numpy(workloads.acts_normal(T, K, 5000 + 8 * layer + j)).to(dev)
            Xq = torch.empty((T, K), dtype=torch.int8, device=dev)
            xs = torch.empty(T, dtype=torch.float32, device=dev)
            act_entries.append((X, None, Xq, xs))
            acts[name] = (Xq, xs)
            total_b += act_bytes(T, K)
        entries = []
        for name, ps in workloads.LLAMA3_8B_INPUTS.items():
            for p in ps:
                N = workloads.LLAMA3_8B[p][0]
                Y = torch.empty((T, N), dtype=torch.float32, device=dev)
                entries.append((acts[name][0], acts[name][1], packed[p][0], packed[p][1], Y, None))
        fns += [bl.prepare_quantize_acts_grouped(act_entries, T),
                bl.prepare_forward_grouped(entries, T)]
        keep.append((packed, act_entries, entries))
    torch.cuda.synchronize()
    if eager:
        for _ in range(eager):
            for f in fns:
                f()
        torch.cuda.synchronize()
        print("fullpass pass: %d eager passes of %d layers at T=%d done"
              % (eager, workloads.LLAMA3_8B_LAYERS, T), flush=True)
        del keep
        return None
    g = _warm_then_capture(torch, fns)
    g.replay()
    samples = _time_graph_samples(torch, g, 7, 1)
    ms = sum(samples) / len(samples)
    gbs = total_b / (ms * 1e-3) / 1e9
    res = {"layers": workloads.LLAMA3_8B_LAYERS, "T": T, "ms_per_pass": round(ms, 4),
           "timing_pass": _stats_us(samples),
           "tokens_per_s": round(T / (ms * 1e-3), 1), "gbs": round(gbs, 1),
           "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "kernel": bl.bitlinear_forward_choice(T, 4096, 4096)}
    del keep
    torch.cuda.empty_cache()
    return res


def run_weight_quant(torch, bl, workloads):
    dev = torch.device("cuda:0")
    N, K = workloads.LLAMA_70B_SWEEP["down"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    W = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * workloads.WEIGHT_SIGMA
    packed = torch.empty((N, K // 4), dtype=torch.uint8, device=dev)
    beta = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(bl.bitlinear_weight_workspace_bytes(N, K), dtype=torch.uint8, device=dev)
    f = lambda: bl.bitlinear_quantize_weights(W, packed, beta, None, ws)  # noqa: E731
    g = _warm_then_capture(torch, [f] * 4)
    g.replay()
    ms = _time_graph(torch, g, 2) / 4
    n = N * K
    res = {"N": N, "K": K, "ms": round(ms, 4),
           "gbs_algorithmic": round(4.25 * n / (ms * 1e-3) / 1e9, 1),
           "gbs_two_pass": round(8.25 * n / (ms * 1e-3) / 1e9, 1)}
    del W, packed, ws
    torch.cuda.empty_cache()
    return res


def run_sign_decode(torch, bl, workloads, T=1):
    """The 1-bit sign variant on the decode8b layer: grouped act-quant + grouped sign GEMV
    (eight codes per byte), rotating replicas, graph-replayed; and the sign quantizer on
    the 70B down matrix."""
    dev = torch.device("cuda:0")
    Ws = workloads.decode8b_layer(0)
    base = {n: bl.quantize_weights_sign(torch.from_numpy(W).to(dev))[:2] for n, W in Ws.items()}
    reps = [base] + [{n: (b.clone(), s.clone()) for n, (b, s) in base.items()}
                     for _ in range(REPLICAS - 1)]
    inputs = workloads.decode8b_inputs(T, 100)
    acts, act_entries = {}, []
    for name, X in inputs.items():
        Xq = torch.empty(X.shape, dtype=torch.int8, device=dev)
        xs = torch.empty(T, dtype=torch.float32, device=dev)
        acts[name] = (Xq, xs)
        act_entries.append((torch.from_numpy(X).to(dev), None, Xq, xs))
    qa = bl.prepare_quantize_acts_grouped(act_entries, T)
    outs = {p: torch.empty((T, N), dtype=torch.float32, device=dev)
            for p, (N, K) in workloads.LLAMA3_8B.items()}
    fws = []
    for r in reps:
        entries = []
        for name, projs in workloads.LLAMA3_8B_INPUTS.items():
            Xq, xs = acts[name]
            for p in projs:
                bits, b = r[p]
                entries.append((Xq, xs, bits, b, outs[p], None))
        fws.append(bl.prepare_forward_sign_grouped(entries, T))
    n_k = 256
    g_k = _warm_then_capture(torch, [fws[i % len(fws)] for i in range(n_k)])
    g_k.replay()
    ms_gemv = _time_graph(torch, g_k, 2) / n_k
    steps = 256
    fns = []
    for i in range(steps):
        fns += [qa, fws[i % len(fws)]]
    g_s = _warm_then_capture(torch, fns)
    g_s.replay()
    ms_step = _time_graph(torch, g_s, 1) / steps
    gemv_b = sum(N * K // 8 + T * K + 4 * T + 4 + 4 * T * N
                 for (N, K) in workloads.LLAMA3_8B.values())
    act_b = sum(act_bytes(T, workloads.LLAMA3_8B[ps[0]][1])
                for ps in workloads.LLAMA3_8B_INPUTS.values())
    del reps, base
    # sign quantizer on the 70B down matrix (exact signed sum + exact |W| sum + bits)
    N, K = workloads.LLAMA_70B_SWEEP["down"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    W = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * workloads.WEIGHT_SIGMA
    bits = torch.empty((N, K // 8), dtype=torch.uint8, device=dev)
    beta = torch.empty(1, dtype=torch.float32, device=dev)
    alpha = torch.empty(1, dtype=torch.float64, device=dev)
    ws = torch.empty(bl.bitlinear_weight_workspace_bytes(N, K), dtype=torch.uint8, device=dev)
    g_w = _warm_then_capture(torch, [lambda: bl.bitlinear_quantize_weights_sign(
        W, bits, beta, alpha, ws)] * 8)
    g_w.replay()
    ms_wq = _time_graph(torch, g_w, 1) / 8
    wq_bytes = N * K * 4 + N * K // 8
    del W, bits, ws
    torch.cuda.empty_cache()
    return {"workload": "decode8b layer, 1-bit sign weights (27.3 MB)",
            "kernel": "gemv_kernel<1, 1> (grouped, 7 projections)",
            "gemv_us": round(ms_gemv * 1e3, 3), "gemv_bytes": gemv_b,
            "gemv_gbs": round(gemv_b / (ms_gemv * 1e-3) / 1e9, 1),
            "gemv_frac_hbm": round(gemv_b / (ms_gemv * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "step_us": round(ms_step * 1e3, 3),
            "step_gbs": round((gemv_b + act_b) / (ms_step * 1e-3) / 1e9, 1),
            "quantize_weights_70b_down_ms": round(ms_wq, 4),
            "quantize_weights_gbs_algorithmic": round(wq_bytes / (ms_wq * 1e-3) / 1e9, 1)}


def run_scale_groups_decode(torch, bl, workloads, G=8, T=1):
    """Group quantization on the decode8b layer: every projection's weights in G blocks of
    output rows with their own scale (a tensor-parallel shard each), grouped GEMV."""
    dev = torch.device("cuda:0")
    Ws = workloads.decode8b_layer(0)
    base = {n: bl.quantize_weights_scale_groups(torch.from_numpy(W).to(dev), G)
            for n, W in Ws.items()}
    reps = [base] + [{n: (p.clone(), b.clone()) for n, (p, b) in base.items()}
                     for _ in range(REPLICAS - 1)]
    inputs = workloads.decode8b_inputs(T, 100)
    acts = {}
    for name, X in inputs.items():
        acts[name] = bl.quantize_acts(torch.from_numpy(X).to(dev))
    outs = {p: torch.empty((T, N), dtype=torch.float32, device=dev)
            for p, (N, K) in workloads.LLAMA3_8B.items()}
    def timed(groups):
        fws = []
        for r in reps:
            entries = []
            for name, projs in workloads.LLAMA3_8B_INPUTS.items():
                Xq, xs = acts[name]
                for p in projs:
                    pk, b = r[p]
                    entries.append((Xq, xs, pk, b, outs[p], None))
            fws.append(bl.prepare_forward_grouped_scale_groups(entries, [groups] * len(entries), T))
        n_k = 256
        g_k = _warm_then_capture(torch, [fws[i % len(fws)] for i in range(n_k)])
        g_k.replay()
        return _time_graph(torch, g_k, 2) / n_k

    # the same buffers read with one scale (G = 1: the first block's scale for all rows)
    # and with the G block scales: the difference is the cost of the grouping alone
    ms1 = timed(1)
    ms = timed(G)
    gemv_b = sum(gemv_bytes(T, N, K) + 4 * (G - 1) for (N, K) in workloads.LLAMA3_8B.values())
    del reps, base
    torch.cuda.empty_cache()
    return {"workload": "decode8b layer, weights in %d scale groups of output rows" % G,
            "kernel": "gemv_kernel<1, 0> (grouped, 7 projections)", "G": G,
            "gemv_us": round(ms * 1e3, 3), "gemv_us_same_buffers_one_scale": round(ms1 * 1e3, 3),
            "gemv_bytes": gemv_b,
            "gemv_gbs": round(gemv_b / (ms * 1e-3) / 1e9, 1),
            "gemv_frac_hbm": round(gemv_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def run_train_side(torch, bl, workloads):
    """Training-side kernels at training shapes: weight fake quantization of the 70B down
    matrix, activation fake quantization and the RMSNorm backward at T = 2048, K = 4096."""
    dev = torch.device("cuda:0")
    N, K = workloads.LLAMA_70B_SWEEP["down"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    W = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * workloads.WEIGHT_SIGMA
    _, beta = bl.quantize_weights(W)
    Wl = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    g_w = _warm_then_capture(torch, [lambda: bl.bitlinear_fake_quant_weights(W, beta, 0.5, Wl)] * 8)
    g_w.replay()
    ms_w = _time_graph(torch, g_w, 1) / 8
    w_bytes = 6 * N * K + 4
    del W, Wl
    torch.cuda.empty_cache()
    T, K = 2048, 4096
    X = torch.randn((T, K), generator=gen, device=dev, dtype=torch.float32)
    dY = torch.randn((T, K), generator=gen, device=dev, dtype=torch.float32)
    Xq = torch.empty((T, K), dtype=torch.int8, device=dev)
    xs = torch.empty(T, dtype=torch.float32, device=dev)
    Xl = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    r = torch.empty(T, dtype=torch.float64, device=dev)
    dX = torch.empty_like(X)
    g_a = _warm_then_capture(torch, [lambda: bl.bitlinear_fake_quant_acts(
        X, None, 1e-6, 0, 0.5, Xq, xs, Xl, r)] * 8)
    g_a.replay()
    ms_a = _time_graph(torch, g_a, 1) / 8
    a_bytes = T * K * (4 + 1 + 2) + T * (4 + 8)
    g_b = _warm_then_capture(torch, [lambda: bl.bitlinear_rmsnorm_backward(X, None, r, dY, dX)] * 8)
    g_b.replay()
    ms_b = _time_graph(torch, g_b, 1) / 8
    b_bytes = T * K * 12 + T * 8
    del X, dY, Xq, Xl, dX
    torch.cuda.empty_cache()

    def rec(ms, b):
        return {"ms": round(ms, 4), "bytes": b, "gbs": round(b / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    return {"fake_quant_weights_70b_down": rec(ms_w, w_bytes),
            "fake_quant_acts_t2048_k4096": rec(ms_a, a_bytes),
            "rmsnorm_backward_t2048_k4096": rec(ms_b, b_bytes)}


def run_bitdelta(torch, bl, N=8192, M=8192, B=8):
    """BitDelta's Figure 4 shape: one bf16 base matrix and B 1-bit deltas, one token per
    model; rotating replicas of base and deltas (402 MB each pair) so the last-level cache
    cannot serve repeats."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    base = (torch.randn((N, M), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    fines = [base.float() + torch.randn((N, M), generator=gen, device=dev) * 0.001
             for _ in range(B)]
    D, alpha = bl.bitdelta_compress(fines, base)
    ws = torch.empty(bl.bitlinear_weight_workspace_bytes(N, M), dtype=torch.uint8, device=dev)
    g_c = _warm_then_capture(torch, [lambda: bl.bitlinear_bitdelta_compress(
        fines[0], base.view(torch.int16), B, 0, D, alpha, ws)] * 4)
    g_c.replay()
    ms_c = _time_graph(torch, g_c, 1) / 4
    del fines
    reps = 4
    copies = [(base, D)] + [(base.clone(), D.clone()) for _ in range(reps - 1)]
    X = torch.randn((B, M), generator=gen, device=dev)
    Y = torch.empty((B, N), dtype=torch.float32, device=dev)
    n_k = 64
    g = _warm_then_capture(torch, [
        (lambda c=copies[i % reps]: bl.bitlinear_bitdelta_forward(c[0].view(torch.int16), c[1],
                                                                 alpha, X, Y))
        for i in range(n_k)])
    g.replay()
    ms = _time_graph(torch, g, 2) / n_k
    nbytes = N * M * 2 + N * M * B // 8 + B * M * 4 + B * N * 4 + 4 * B
    del copies, base, D
    torch.cuda.empty_cache()
    return {"workload": "BitDelta linear layer, N = M = %d, B = %d models (one token each)" % (N, B),
            "kernel": "bitdelta_kernel", "us": round(ms * 1e3, 3), "bytes": nbytes,
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "compress_one_model_ms": round(ms_c, 4)}


def run_calib_copy(torch, bl=None):
    """Kernels of known traffic for the counter calibration: a torch elementwise multiply
    (reads 256 MiB, writes 256 MiB) and the library's read roof over 256 MiB (reads
    256 MiB, writes one word per wave)."""
    n = 64 * 1024 * 1024  # 256 MiB of fp32
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 1.0, out=b)   # one elementwise kernel: reads 256 MiB, writes 256 MiB
    if bl is not None:
        sink = torch.empty(bl.ROOF_READ_SINK_BYTES, dtype=torch.uint8, device="cuda:0")
        for _ in range(3):
            bl.bitlinear_roof_read([a], sink)
    torch.cuda.synchronize()
    return {"bytes_read": 4 * n, "bytes_written": 4 * n, "kernel": "torch elementwise mul",
            "read_kernel": "roof_read_kernel over 256 MiB" if bl is not None else None}


# ---------------------------------------------------------------- tiny (config 1)

def run_tiny(torch, bl, workloads):
    """The tiny single-layer forward (W [256 x 1024], T = 8): act-quant + product per
    step, graph-replayed (launch-bound: 64 KiB of packed weights)."""
    dev = torch.device("cuda:0")
    N, K = workloads.TINY_W
    T = workloads.TINY_T
    packed, beta = bl.quantize_weights(torch.from_numpy(workloads.weights(N, K, 0)).to(dev))
    X = torch.from_numpy(workloads.acts_normal(T, K, 1)).to(dev)
    Xq = torch.empty((T, K), dtype=torch.int8, device=dev)
    xs = torch.empty(T, dtype=torch.float32, device=dev)
    Y = torch.empty((T, N), dtype=torch.float32, device=dev)
    qa = bl.prepare_quantize_acts_grouped([(X, None, Xq, xs)], T)
    fw = bl.prepare_forward_grouped([(Xq, xs, packed, beta, Y, None)], T)
    g = _warm_then_capture(torch, [qa, fw] * 64)
    g.replay()
    st = _stats_us(_time_graph_samples(torch, g, 11, 64))
    b = gemv_bytes(T, N, K) + act_bytes(T, K)
    return {"workload": "tiny: W [256 x 1024], T = 8 (act-quant + product)",
            "kernel": bl.bitlinear_forward_choice(T, N, K), "step": st,
            "gbs": round(b / (st["median_us"] * 1e-6) / 1e9, 1)}


# ---------------------------------------------------------------- CPU baseline

def _oracle_rate(fn, budget_s, max_n=1000):
    fn()
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= max_n:
            return n, el


def run_cpu_baseline(d, workloads, budget_s=8.0):
    """The oracle (plain C, OpenMP over rows) on the host cores: the decode8b step on all
    cores (the reported value) and on one thread; the tiny forward; the 32-layer T = 16
    pass extrapolated from its first layer."""
    import numpy as np  # noqa: F401
    import oracle

    cores = len(os.sched_getaffinity(0))
    used = oracle.set_threads(cores)
    packed = {p: oracle.quantize_weights(W)[:2] for p, W in d["Ws"].items()}
    inputs = d["inputs"]
    T = next(iter(inputs.values())).shape[0]

    def one_step(ins):
        for name, ps in workloads.LLAMA3_8B_INPUTS.items():
            Xq, s = oracle.quantize_acts(ins[name])
            for p in ps:
                P, beta = packed[p]
                oracle.forward(Xq, s, P, beta)

    b = d["gemv_bytes"] + d["act_bytes"]
    n, el = _oracle_rate(lambda: one_step(inputs), budget_s)
    ms = el * 1e3 / n
    out = {"value": round(b / (ms * 1e-3) / 1e9, 3), "unit": "GB/s", "cores": used,
           "kind": "oracle",
           "sample": "%d passes of the decode8b step (T=%d: act-quant of 4 inputs + 7 "
                     "projections), %.1f s wall, %.2f ms/step" % (n, T, el, ms)}
    oracle.set_threads(1)
    n1, el1 = _oracle_rate(lambda: one_step(inputs), budget_s / 2)
    ms1 = el1 * 1e3 / n1
    out["one_thread"] = {"value": round(b / (ms1 * 1e-3) / 1e9, 3), "unit": "GB/s", "cores": 1,
                         "sample": "%d decode8b steps, %.2f ms/step" % (n1, ms1)}
    # tiny (config 1)
    N, K = workloads.TINY_W
    Tt = workloads.TINY_T
    Pt, bt, _ = oracle.quantize_weights(workloads.weights(N, K, 0))
    Xt = workloads.acts_normal(Tt, K, 1)

    def tiny():
        Xq, s = oracle.quantize_acts(Xt)
        oracle.forward(Xq, s, Pt, bt)

    bt_bytes = gemv_bytes(Tt, N, K) + act_bytes(Tt, K)
    tiny_out = {}
    for th in (cores, 1):
        oracle.set_threads(th)
        nt, elt = _oracle_rate(tiny, 1.0, 5000)
        us = elt * 1e6 / nt
        tiny_out["cores_%d" % th] = {"us_per_step": round(us, 1),
                                     "gbs": round(bt_bytes / (us * 1e-6) / 1e9, 3)}
    out["tiny"] = {"workload": "tiny: W [256 x 1024], T = 8 (act-quant + product)", **tiny_out}
    # 32-layer pass at T = 16: the first layer timed, the pass extrapolated (x 32)
    oracle.set_threads(cores)
    Tf = workloads.FULLPASS_T
    ins16 = workloads.decode8b_inputs(Tf, 5000)
    t0 = time.perf_counter()
    one_step(ins16)
    el16 = time.perf_counter() - t0
    ms_pass = el16 * 1e3 * workloads.LLAMA3_8B_LAYERS
    out["fullpass_extrapolated"] = {
        "ms_per_pass": round(ms_pass, 1), "tokens_per_s": round(Tf / (ms_pass * 1e-3), 2),
        "cores": used,
        "sample": "layer 0 of the 32-layer T = 16 pass (act-quant of 4 inputs + 7 projections) "
                  "timed once, %.2f s; the pass figure is that x 32 (extrapolated)" % el16}
    oracle.set_threads(cores)
    return out


# ---------------------------------------------------------------- main

def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the BitLinear path here has no multi-GPU "
              "mode (requested --gpus %d, WORLD_SIZE %d)" % (a.gpus, world), file=sys.stderr)
        sys.exit(2)
    if a.steps < 1 or a.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    import torch

    import ternary_quantized_linear_amd as bl
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if a.prefill_pass > 0:
        run_prefill_pass(torch, bl, workloads, a.prefill_pass)
        return
    if a.sweep_pass > 0:
        run_sweep_pass(torch, bl, workloads, a.sweep_pass)
        run_calib_copy(torch, bl)
        return
    if a.fullpass_pass > 0:
        run_fullpass(torch, bl, workloads, eager=a.fullpass_pass)
        run_calib_copy(torch, bl)
        return
    T = 1
    d = setup_decode(torch, bl, workloads, T)
    if a.counter_pass > 0:
        # eager launches only: each dispatch is counted on its own
        for i in range(a.counter_pass):
            d["qa"]()
            d["fws"][i % len(d["fws"])]()
        torch.cuda.synchronize()
        run_calib_copy(torch, bl)
        print("counter pass: %d decode steps and the 256 MiB copy done" % a.counter_pass,
              flush=True)
        return
    r = run_decode(torch, bl, d, a.steps, a.warmup)
    step_bytes = d["gemv_bytes"] + d["act_bytes"]
    value = step_bytes / (r["ms_step"] * 1e-3) / 1e9
    achieved = d["gemv_bytes"] / (r["ms_gemv"] * 1e-3) / 1e9
    read_gbs = d["packed_bytes"] / (r["ms_read"] * 1e-3) / 1e9
    read7_gbs = d["packed_bytes"] / (r["ms_read7"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic: seeded 0.02*N(0,1) weights (absmean-ternarized, 2-bit packed), "
                "N(0,1) activations",
        "config": {"workload": "decode8b: one Llama-3-8B layer (q,k,v,o,gate,up,down) at T=1; "
                               "step = grouped RMSNorm+int8 act-quant (4 inputs) + grouped "
                               "ternary GEMV over the layer in one allocation (q|k|v, o, "
                               "gate|up, down with per-segment scales); 32 rotating packed-weight "
                               "replicas; HIP-graph replay",
                   "T": T, "projections": 7, "packed_bytes_per_layer": d["packed_bytes"],
                   "bytes_per_step": step_bytes, "frac_hbm_step": round(value / HBM_PEAK_GBS, 4),
                   "step_timing": r["step_stats"]},
        "roofline": {"bound": "hbm", "kernel": "gemv_kernel<1, 0> (grouped: q|k|v, o, gate|up, down)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counted_traffic(),
                     "bytes_per_launch": d["gemv_bytes"],
                     "avg_launch_us": round(r["ms_gemv"] * 1e3, 3),
                     "launch_timing": r["gemv_stats"],
                     "measured_read_roof": {
                         "gbs_one_allocation": round(read_gbs, 1),
                         "gbs_seven_buffers": round(read7_gbs, 1),
                         "frac_of_peak": round(read_gbs / HBM_PEAK_GBS, 4),
                         "gemv_frac_of_measured": round(achieved / read_gbs, 4),
                         "kernel": "roof_read_kernel (the same packed bytes, read once; fastest "
                                   "of its four block schedules)"},
                     "seven_buffer_launch_us": round(r["ms_gemv7"] * 1e3, 3),
                     "packed_weight_gbs": round(d["packed_bytes"] / (r["ms_gemv"] * 1e-3) / 1e9, 1)},
        "act_quant": {"avg_launch_us": round(r["ms_act"] * 1e3, 3),
                      "bytes_per_launch": d["act_bytes"]},
        "clocks": {"before": r["clocks_before"], "after": r["clocks_after"]},
        "eager_ms_per_step": round(r["ms_eager"], 4),
    }
    if not a.only_decode:
        line["decode8b_per_projection"] = run_decode_per_projection(torch, bl, d)
    del d["bufs"], d["layer_views"], d["fws"], d["fws7"]
    torch.cuda.empty_cache()
    line["mfma_roof"] = run_mfma_roof(torch, bl)
    if not a.only_decode:
        line["tiny"] = run_tiny(torch, bl, workloads)
        line["prefill"] = run_prefill(torch, bl, workloads)
        line["sweep70b"] = run_sweep70b(torch, bl, workloads)
        line["fullpass"] = run_fullpass(torch, bl, workloads)
        line["weight_quant"] = run_weight_quant(torch, bl, workloads)
        line["sign_decode8b"] = run_sign_decode(torch, bl, workloads)
        line["scale_groups_decode8b"] = run_scale_groups_decode(torch, bl, workloads)
        line["train_side"] = run_train_side(torch, bl, workloads)
        line["bitdelta"] = run_bitdelta(torch, bl)
    if a.calib_copy:
        line["calib_copy"] = run_calib_copy(torch, bl)
    line["cpu_baseline"] = None if a.no_cpu else run_cpu_baseline(d, workloads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
