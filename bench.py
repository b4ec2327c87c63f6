#!/usr/bin/env python3
"""Throughput of the DropMatch verify step on one MI355X.

One step = one dm_verify_run over a batch of synthetic inputs already
resident in HBM: masks, the K-head LM head, statistics, JS terms, the rules,
the scan and the emitted token.  Prints one JSON line on stdout.

  python bench.py [--steps K] [--warmup W] [--config C]

The default workload is the batched Llama-3.1-70B-shaped head (B = 32,
gamma = 7, d = 8192, |V| = 128256, K = 5, p_drop = 0.25, JS + majority:
1280 LM-head rows, the largest K = 5 workload on one GPU, where the GEMM is
bound by the matrix cores).  --config picks another workload for
inspection (0: tiny; 1, 2: the 8B and 70B heads at B = 1, bound by HBM;
4: wide vocabulary, mixed rules; 5: naive matching on a 60-node token tree
at the 70B head).
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
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
PROFILES = os.path.join(ROOT, "profiles")


class HipEvents:
    """hipEvent_t handles from the HIP runtime already loaded in the process
    (torch's events are created lazily, so their handles are not usable
    before torch itself records them)."""

    def __init__(self):
        import ctypes

        self.ct = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self) -> int:
        ev = self.ct.c_void_p()
        rc = self.lib.hipEventCreate(self.ct.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.made.append(ev.value)
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = self.ct.c_float()
        rc = self.lib.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for ev in self.made:
            self.lib.hipEventDestroy(ev)
        self.made = []


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_kernel(cfg, panels: bool, n_lossless: int, lossy_pos=None, lossless_pos=None) -> str:
    """Which LM-head kernel the library launches: row-major W takes
    k_gemm_skinny; panel-order W takes k_gemm_panel when the rows fit one
    small tile (4 lane groups of 4 * ms slots, ms = 1..4, a position's K heads
    in one group) and k_gemm_tile otherwise.  The live position counts of a
    ragged batch may be given (default: gamma + 1 per sequence)."""
    if not panels:
        return "k_gemm_skinny"
    T1 = cfg.gamma + 1
    if lossy_pos is None:
        lossy_pos, lossless_pos = (cfg.B - n_lossless) * T1, n_lossless * T1
    best = None
    for ms in range(1, 5):
        S = 4 * ms
        if lossy_pos and S < cfg.K:
            continue
        tl = -(-lossy_pos // (4 * (S // cfg.K))) if lossy_pos else 0
        tn = -(-lossless_pos // (4 * S)) if lossless_pos else 0
        best = tl + tn if best is None else min(best, tl + tn)
    return "k_gemm_tile" if best is None or best > 1 else "k_gemm_panel"


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary
    of this workload, if it was taken on the current source of that kernel."""
    from speculative_decoding_verification_philox_amd.rocprof_summary import kernel_source_hash

    path = os.path.join(PROFILES, f"k_gemm_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel") != kernel or rec.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def ragged_gammas(cfg, seed: int):
    """The per-sequence draft counts of `--ragged SEED`: uniform on
    0..gamma, one per sequence, from numpy's default generator."""
    import numpy as np

    return np.random.default_rng(seed).integers(0, cfg.gamma + 1, cfg.B).astype(np.int32)


def cpu_info():
    """(CPU model string, nproc, CPUs this process may run on)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    nproc = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = nproc
    return model, nproc, avail


def cpu_baseline(w, seed, budget_s):
    """The oracle as it stands, timed on bounded samples of the same workload.

    All threads (at most 16, the host share of one GPU): whole sequences
    (every position of a sequence, all its heads, full vocabulary) in batch
    order until about `budget_s` seconds.  One thread: single positions of
    the same sequences (the sequence cut to its first position through the
    ragged-batch inputs: all heads, full vocabulary) until about a third of
    that."""
    import numpy as np

    import oracle

    model, nproc, avail = cpu_info()
    threads = max(1, min(16, avail))
    B = w.cfg.B

    def sample(n_threads, one_position, budget):
        done, elapsed, calls = 0, 0.0, 0
        while elapsed < budget or calls == 0:
            b = calls % B
            kw = {}
            if one_position:
                kw["seq_gamma"] = np.zeros(B, np.int32)
            t0 = time.perf_counter()
            oracle.run(w.W, w.h, w.draft, w.q_hat, w.modes, w.K, w.p_drop, seed, seqs=np.array([b], np.int32),
                       n_threads=n_threads, tree_parent=w.tree_parent, **kw)
            elapsed += time.perf_counter() - t0
            done += 1 if one_position else w.cfg.gamma + 1
            calls += 1
        return done / elapsed, calls, elapsed

    rate, calls, el = sample(threads, False, budget_s)
    rate1, calls1, el1 = sample(1, True, budget_s / 3.0)
    return {"value": round(rate, 3), "unit": "positions/s", "cores": threads, "kind": "oracle",
            "sample": f"{threads} threads: {calls} oracle call(s) of one whole sequence each "
                      f"({w.cfg.gamma + 1} positions, all heads, full vocabulary) of the same workload, fp64, "
                      f"{el:.1f} s; 1 thread: {calls1} call(s) of one position each, {el1:.1f} s",
            "single_thread_value": round(rate1, 4), "nproc": nproc, "cpus_available": avail, "cpu_model": model}


def graph_replay(torch, step_on, outs, steps, warmup):
    """One step captured into a HIP graph (every enqueue of the step is a
    kernel launch), replayed `steps` times after `warmup` replays.  The
    outputs of the last eager step are kept and compared with those of every
    replay, with the host synchronising between replays."""
    eager = {k: v.clone() for k, v in outs.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_on(torch.cuda.current_stream())
    torch.cuda.synchronize()
    match = True
    for _ in range(max(1, warmup)):
        for v in outs.values():
            v.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        match = match and all(bool(torch.equal(outs[k], eager[k])) for k in eager)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    match = match and all(bool(torch.equal(outs[k], eager[k])) for k in eager)
    return {"ms_per_step": round(start.elapsed_time(stop) / steps, 5), "outputs_match": match}


def copy_probe(nbytes: int, dev) -> None:
    """One plain device-to-device copy of `nbytes`, for calibrating HBM byte
    counters: rocprofv3's FETCH_SIZE / WRITE_SIZE of this dispatch are
    compared with the bytes it must move."""
    import torch

    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy probe: {nbytes} bytes read, {nbytes} bytes written")
    del src, dst


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--p-drop", type=float, default=None)
    ap.add_argument("--temperature", type=float, default=1.0,
                    help="sampling temperature of the target (every rule)")
    ap.add_argument("--top-k", type=int, default=0, help="top-k of the lossless target (0 = off)")
    ap.add_argument("--top-p", type=float, default=1.0, help="top-p of the lossless target (1 = off)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--w-layout", choices=("panels", "rowmajor"), default="panels",
                    help="order of the LM-head weight: panels (packed once before timing, as a model loader "
                         "would) or row-major")
    ap.add_argument("--ragged", type=int, default=0,
                    help="a ragged batch: each sequence's draft count drawn uniformly from 0..gamma with this "
                         "seed (0 = every sequence drafts gamma)")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one step into a HIP graph and time its replays (reported beside the "
                         "direct launches, which stay the headline)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this verify step is built and measured on a single MI355X "
              "(--gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from speculative_decoding_verification_philox_amd import binding as Bd
    from speculative_decoding_verification_philox_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib << 20, dev)

    cfg = wl.CONFIGS[args.config]
    over = {}
    if args.p_drop is not None:
        over["p_drop"] = args.p_drop
    t0 = time.perf_counter()
    w = wl.generate(cfg, **over)
    cfg = w.cfg
    log(f"[bench] generated {cfg.name} in {time.perf_counter() - t0:.1f} s")

    def dev_t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    W, h = dev_t(w.W), dev_t(w.h)
    draft = dev_t(w.draft.astype(np.int32))
    q_hat = dev_t(w.q_hat)
    tree = dev_t(w.tree_parent) if w.tree_parent is not None else None
    dtype_code = Bd.DM_DTYPE_BF16 if cfg.dtype == wl.DTYPE_BF16 else Bd.DM_DTYPE_F32
    ver = Bd.Verifier(d=cfg.d, vocab=cfg.V, max_batch=cfg.B, gamma=cfg.gamma, k_max=cfg.K, dtype=dtype_code)
    seed = wl.perf_seed(cfg.index)
    w_layout = Bd.DM_W_PANELS if args.w_layout == "panels" else Bd.DM_W_ROW_MAJOR
    if w_layout == Bd.DM_W_PANELS:
        W_run = ver.pack_w(W)  # one-time reorder of the fixed weight, outside the timed region
        torch.cuda.synchronize()
        del W
    else:
        W_run = W
    outs = {"accept_len": torch.empty(cfg.B, dtype=torch.int32, device=dev),
            "out_token": torch.empty(cfg.B, dtype=torch.int32, device=dev),
            "accept_pos": torch.empty(cfg.B, dtype=torch.int32, device=dev)}
    stream = torch.cuda.current_stream(dev)

    seq_gamma = None
    if args.ragged:
        seq_gamma = ragged_gammas(cfg, args.ragged)

    def step_on(st):
        ver.run(W_run, h, draft, q_hat, w.modes, cfg.K, cfg.p_drop, seed, stream=st.cuda_stream, outputs=outs,
                w_layout=w_layout, temperature=args.temperature, top_k=args.top_k, top_p=args.top_p,
                tree_parent=tree, seq_gamma=seq_gamma)

    def step():
        step_on(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    hev = HipEvents()
    gemm_ev = [(hev.create(), hev.create()) for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    t_wall = time.perf_counter()
    for i in range(args.steps):
        Bd.dm_verify_profile(ver.handle, gemm_ev[i][0], gemm_ev[i][1])
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / args.steps
    gemm_ms = [hev.elapsed_ms(a, b) for a, b in gemm_ev]
    # per-step durations without extra events: from one step's GEMM start to the next one's
    step_ms = [hev.elapsed_ms(gemm_ev[i][0], gemm_ev[i + 1][0]) for i in range(args.steps - 1)]
    ms_median = float(np.median(step_ms)) if step_ms else ms_step
    hev.close()
    gemm_avg = float(np.mean(gemm_ms))
    log(f"[bench] {args.steps} steps: {ms_step * 1e3:.1f} us/step (events), median {ms_median * 1e3:.1f}, "
        f"wall {wall / args.steps * 1e6:.1f} us/step; GEMM kernel {gemm_avg * 1e3:.1f} us avg, "
        f"min {min(gemm_ms) * 1e3:.1f} us")

    graph = None
    if args.graph:
        graph = graph_replay(torch, step_on, outs, args.steps, args.warmup)
        log(f"[bench] graph replay: {graph['ms_per_step'] * 1e3:.1f} us/step against {ms_step * 1e3:.1f} direct; "
            f"outputs identical to the eager step: {graph['outputs_match']}")

    n_lossless = int((w.modes == wl.LOSSLESS).sum())
    per_seq = (seq_gamma + 1) if seq_gamma is not None else np.full(cfg.B, cfg.gamma + 1)
    lossless_seq = w.modes == wl.LOSSLESS
    positions = int(per_seq.sum())
    value = positions / (ms_step / 1e3)
    rows = int(per_seq[~lossless_seq].sum()) * cfg.K + int(per_seq[lossless_seq].sum())
    elem = 2 if cfg.dtype == wl.DTYPE_BF16 else 4
    alg_bytes = cfg.V * cfg.d * elem + positions * cfg.d * elem
    alg_flops = 2.0 * rows * cfg.d * cfg.V
    intensity = alg_flops / alg_bytes
    dname = "bf16" if cfg.dtype == wl.DTYPE_BF16 else "f32"
    balance = MFMA_PEAK_TFLOPS[dname] * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < balance:
        achieved = alg_bytes / (gemm_avg / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = alg_flops / (gemm_avg / 1e3) / 1e12
        peak = MFMA_PEAK_TFLOPS[dname]
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    roof["kernel"] = gemm_kernel(cfg, w_layout == Bd.DM_W_PANELS, n_lossless, int(per_seq[~lossless_seq].sum()),
                                 int(per_seq[lossless_seq].sum()))
    # the committed counter records cover the full (non-ragged) workloads only
    roof["traffic"] = None if seq_gamma is not None else measured_traffic(cfg.name, roof["kernel"])

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host cores ...")
        cpu = cpu_baseline(w, seed, args.cpu_seconds)
        log(f"[bench] oracle {cpu['value']:.3f} positions/s on {cpu['cores']} threads, "
            f"{cpu['single_thread_value']:.4f} on one")

    modes_desc = {"js": "JS+majority", "naive": "naive", "lossless": "lossless",
                  "half_lossless_naive": "half lossless / half naive",
                  "tree": f"naive matching on a {cfg.gamma}-node, {cfg.tree_depth}-level token tree"}[cfg.modes]
    line = {
        "metric": "verified positions/sec (K=5 dropout heads + accept) and % HBM/MFMA roofline",
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_median": round(ms_median, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dname,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={cfg.B}, gamma={cfg.gamma}, d={cfg.d}, |V|={cfg.V}, K={cfg.K}, "
                               f"p_drop={cfg.p_drop}, {modes_desc}",
                   "batch": cfg.B, "positions_per_step": positions, "gemm_rows": rows, "w_layout": args.w_layout,
                   "ragged_seed": args.ragged or None,
                   "sampling": {"temperature": args.temperature, "top_k": args.top_k, "top_p": args.top_p}},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if graph is not None:
        line["graph_replay"] = graph
    print(json.dumps(line), flush=True)
    ver.close()


if __name__ == "__main__":
    main()
