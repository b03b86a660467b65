"""Throughput of the context K/V chain on one MI355X.

One step = the whole hot path over one batch of synthetic context rows, on
one stream, inputs and outputs resident in HBM. Default path: context_norms ->
context_kv_project -> context_kv_store. --path fused times
context_hidden_norm (hidden norm + per-row layer-norm scale) ->
context_kv_project_fused (layer norms applied while staging the projection's
A tiles) -> context_kv_store instead; --path one-call times context_norms
-> context_kv_project_store (the projection and the store in one call: for
small T the store's kernel adds the split projection's partial sums). The
default workload is
the long-context configuration (L=4 draft layers, T=16384 rows, D=8192,
H=8 KV heads, RoPE table [131072, 64], block size 16, 8192 blocks).

    python bench.py [--steps K] [--warmup W] [--workload long] [--no-cpu-baseline]

Prints ONE JSON line on stdout; progress goes to stderr. Launch durations
come from HIP events recorded on the stream the kernels run on (torch's
current stream, which the binding passes to every call), created as timing
events (hipEventDisableSystemFence: recording one does not write back and
invalidate the caches at system scope, which with default events costs each
event a few microseconds of stall and leaves the next kernel cold). The timed
region records events only around the dominant kernel (two per step); the
per-kernel figures come from a pass of as many steps with events between all
calls, run before it.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
PEAK_CLOCK_GHZ = 2.4           # the engine clock the MFMA peak is quoted at


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipTimer:
    """HIP events for timing only, from the HIP runtime this process has
    loaded (the one torch and libnrc share), created with
    hipEventDisableSystemFence and recorded on torch's current stream."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded in this process")
        self._ct = ctypes
        self._hip = h = ctypes.CDLL(path)
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._events = []

    def event(self):
        e = self._ct.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(self._ct.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self._events.append(e)
        return e

    def record(self, e):
        import torch

        rc = self._hip.hipEventRecord(e, self._ct.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, e0, e1):
        f = self._ct.c_float()
        rc = self._hip.hipEventElapsedTime(self._ct.byref(f), e0, e1)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def close(self):
        for e in self._events:
            self._hip.hipEventDestroy(e)
        self._events = []


def algorithmic_bytes(cfg, slots_np):
    """Per-launch algorithmic HBM bytes of the norms and the store.

    norms: read x once (2 D per row), write L rows (2 L D per row), plus the
           weights once ((1 + L) 2 D, or none when weightless).
    store: the one slot mapping every layer shares, 8 B per row, and with
           RoPE each row's position (8 B, loaded with the slot); per row with
           a slot: its cos/sin row (128 B) once, and per layer K and V read
           (2 N) and written (2 N). Rows with a negative slot read nothing
           else."""
    D, L, T, N = 8192, cfg.L, cfg.T, cfg.N
    w = (1 if cfg.hidden_weighted else 0) * 2 * D + (L if cfg.pre_weighted else 0) * 2 * D
    norms = T * (2 * D + 2 * L * D) + w
    valid = int((slots_np >= 0).sum())  # rows of the shared mapping with a slot
    store = T * (8 + (8 if cfg.rope else 0)) + valid * (128 if cfg.rope else 0) + valid * L * (2 * N + 2 * N)
    flops = 2 * L * T * D * N
    return norms, store, flops


def traffic_from_profiles(kernel_tag):
    """HBM bytes per launch measured with rocprofv3 counters, if a committed
    summary for the current kernel source exists (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_tag)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    from norm_rope_cache_amd import build

    if rec.get("source_hash") != build.source_hash():
        return None
    return rec.get("bytes_per_launch")


def host_cpu():
    """(threads available to this process, CPU model name)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    # a host shared between GPUs states each process's CPU share in
    # OMP_NUM_THREADS; honour it when set
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def cpu_baseline(d, cfg, rows, threads):
    """The CPU oracle as it stands, on the first `rows` rows of the workload,
    stage by stage, each stage's work spread over `threads` host threads
    (the oracle's C routines release the GIL): norms by row blocks, the FP32
    projection by (layer, row block), the store by (layer, row block) into
    that layer's cache (distinct slots: no two tasks write one cell).
    Returns per-stage seconds."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    L, N, H = cfg.L, cfg.N, cfg.H
    x = d["x"][:rows]
    pos = np.ascontiguousarray(d["positions"][:rows])
    slots = np.ascontiguousarray(d["slots"][:, :rows])
    caches = d["caches_host_sample"]
    blk = max(1, -(-rows // (4 * threads)))
    row_blocks = [(r0, min(rows, r0 + blk)) for r0 in range(0, rows, blk)]
    normed = np.empty((L, rows, 8192), dtype=np.uint16)
    kv = np.empty((L, rows, N), dtype=np.uint16)

    def norms(rb):
        r0, r1 = rb
        normed[:, r0:r1] = oracle.context_norms(np.ascontiguousarray(x[r0:r1]), d["hidden_w"], d["pre_w"], L,
                                                d["hidden_eps"], d["pre_eps"])

    def project(task):
        l, (r0, r1) = task
        kv[l, r0:r1] = oracle.bf16(oracle.kv_project(normed[l:l + 1, r0:r1], d["w_kv"][l:l + 1])[0])

    def store(task):
        l, (r0, r1) = task
        oracle.context_kv_store(kv[l:l + 1, r0:r1], H, pos[r0:r1], slots[l:l + 1, r0:r1], d["cos_sin"],
                                caches[l:l + 1], cfg.block_size, d["k_eps"])

    tasks = [(l, rb) for l in range(L) for rb in row_blocks]
    times = {}
    with ThreadPoolExecutor(threads) as ex:
        for name, fn, work in (("norms", norms, row_blocks), ("projection", project, tasks),
                               ("store", store, tasks)):
            t0 = time.perf_counter()
            list(ex.map(fn, work))
            times[name] = time.perf_counter() - t0
    return times


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip timing the norm variants after the chain")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip timing the norms against their traffic twin after the chain")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of the workload the CPU oracle is timed on (the whole chain on those rows); "
                         "default: every row, at most as many as hold the oracle's projection to 1.2 TFLOP")
    ap.add_argument("--path", choices=("fused", "unfused", "one-call"), default="unfused")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="KV heads to project and store (default: the workload's); e.g. 1 for the long workload's "
                         "per-GPU share under 8-way tensor parallelism, which splits the heads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB device-to-device once, a known-size reference for HBM byte counters")
    ap.add_argument("--hipblaslt", action="store_true",
                    help="after the chain, time the projection against hipBLASLt (torch.mm per layer) on the same "
                         "operands, the weight both as given ([L, D, N]) and K-contiguous ([L, N, D])")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} / WORLD_SIZE {world} is not supported "
              "(the chain needs no exchange between GPUs; see the design notes on sharding)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import norm_rope_cache_amd as nrc
    from norm_rope_cache_amd import synth

    cfg = synth.CONFIGS[args.workload]
    if args.kv_heads:
        from dataclasses import replace

        cfg = replace(cfg, H=args.kv_heads)
    log(f"generating {cfg.name}: L={cfg.L} T={cfg.T} H={cfg.H}")
    d = synth.make_inputs(cfg, with_cache=False)
    dev = torch.device("cuda", 0)

    def dv(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x0 = dv(d["x"])
    hw = None if d["hidden_w"] is None else dv(d["hidden_w"])
    pw = None if d["pre_w"] is None else dv(d["pre_w"])
    w_kv = dv(d["w_kv"])
    cos_sin = None if d["cos_sin"] is None else dv(d["cos_sin"])
    positions = dv(d["positions"])
    slots = dv(d["slots"][0])  # the one slot mapping every layer shares
    fused = args.path == "fused"
    one_call = args.path == "one-call"
    # Buffer sets the steps rotate over: a step whose touched bytes (rows in
    # and out, the projection weight, the written cache rows) fit twice in
    # the 256 MB infinity cache would otherwise find them there on the next
    # step; with enough sets (at most 16) each has been evicted before its
    # reuse. The long and larger workloads touch over 1 GB per step: one set.
    touched = (cfg.T * 8192 * 2 * (1 + (1 if fused else cfg.L)) + cfg.L * cfg.T * cfg.N * 2 +
               cfg.L * 8192 * cfg.N * 2 + cfg.L * cfg.T * cfg.H * 256)
    n_sets = min(16, -(-(1 << 30) // touched)) if touched < (512 << 20) else 1
    sets = []
    for i in range(n_sets):
        c = torch.empty((cfg.L, cfg.num_blocks, cfg.H, cfg.block_size, 128), dtype=torch.bfloat16, device=dev)
        c.view(torch.int16).random_(-32768, 32767)
        sets.append({
            "x": x0 if i == 0 else x0.clone(),
            "w": w_kv if i == 0 else w_kv.clone(),
            "caches": c,
            "kv": torch.empty((cfg.L, cfg.T, cfg.N), dtype=torch.bfloat16, device=dev),
            "h": torch.empty((cfg.T, 8192), dtype=torch.bfloat16, device=dev) if fused else None,
            "r": torch.empty((cfg.T,), dtype=torch.float32, device=dev) if fused else None,
            "normed": None if fused else torch.empty((cfg.L, cfg.T, 8192), dtype=torch.bfloat16, device=dev),
        })
    x = x0
    torch.cuda.synchronize()
    log(f"{n_sets} buffer set(s), {touched / 1e6:.1f} MB touched per step")
    names = (["context_hidden_norm", "context_kv_project_fused", "context_kv_store"] if fused else
             ["context_norms", "context_kv_project_store"] if one_call else
             ["context_norms", "context_kv_project", "context_kv_store"])

    step_no = [0]
    nrc._load()
    timer = HipTimer()

    def step(ev=None, around=None):
        """One chain step. ev: four events recorded between the calls (the
        per-kernel pass); around: (call index, event, event) recorded just
        before and after that one call (the timed region)."""
        b = sets[step_no[0] % n_sets]
        step_no[0] += 1

        def mark(i):
            if ev:
                timer.record(ev[i])
            if around and around[0] == i:
                timer.record(around[1])
            if around and around[0] + 1 == i:
                timer.record(around[2])

        mark(0)
        if fused:
            nrc.context_hidden_norm(b["x"], hw, pw, cfg.L, d["hidden_eps"], d["pre_eps"], h=b["h"], r=b["r"])
        else:
            nrc.context_norms(b["x"], hw, pw, cfg.L, d["hidden_eps"], d["pre_eps"], out=b["normed"])
        mark(1)
        if one_call:
            nrc.context_kv_project_store(b["normed"], b["w"], positions, slots, cos_sin, b["caches"], d["k_eps"],
                                         out=b["kv"])
            mark(2)
            return
        if fused:
            nrc.context_kv_project_fused(b["h"], b["r"], pw, b["w"], out=b["kv"])
        else:
            nrc.context_kv_project(b["normed"], b["w"], out=b["kv"])
        mark(2)
        nrc.context_kv_store(b["kv"], positions, slots, cos_sin, b["caches"], cfg.H, d["k_eps"])
        mark(3)

    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev).random_(-32768, 32767)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        log("calibration copy: 1 GiB read + 1 GiB written")
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Per-kernel pass: as many steps as the timed region, events between all
    # calls; its durations give each kernel's figures and pick the dominant
    # kernel (the longest launch).
    log(f"per-kernel pass: {args.steps} steps")
    events = [[timer.event() for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    k_ms = {n: [] for n in names}
    for ev in events:
        for i, n in enumerate(names):
            k_ms[n].append(timer.elapsed_ms(ev[i], ev[i + 1]))
    avg = {k: sum(v) / len(v) for k, v in k_ms.items()}
    dom = max(avg, key=avg.get)
    dom_i = names.index(dom)

    # Timed region: K steps, events only around the dominant kernel's call.
    log(f"timing {args.steps} steps")
    around = [(dom_i, timer.event(), timer.event()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(around=around[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    dom_ms = sum(timer.elapsed_ms(a[1], a[2]) for a in around) / args.steps
    log("per-kernel ms (per-kernel pass): " + ", ".join(f"{k}={v:.4f}" for k, v in avg.items()) +
        f"; timed region: wall/step {ms_step:.4f}, {dom} {dom_ms:.4f}")

    norms_b, store_b, flops = algorithmic_bytes(cfg, d["slots"][0])
    n0, n1 = names[0], names[1]
    if fused:
        # pre-pass: read x, write h and r (plus the hidden weight once)
        norms_b = cfg.T * (2 * 8192 + 2 * 8192 + 4) + (2 * 8192 if cfg.hidden_weighted else 0)
    kernels = {
        n0: {"bound": "hbm", "ms": avg[n0], "bytes": norms_b, "achieved_GBs": norms_b / (avg[n0] * 1e-3) / 1e9},
        n1: {"bound": "mfma", "ms": avg[n1], "flops": flops, "achieved_TFLOPs": flops / (avg[n1] * 1e-3) / 1e12},
    }
    if one_call:
        # the call also does the store's work (its bytes below), rated here
        # by the projection's flops alone
        kernels[n1]["store_bytes"] = store_b
    else:
        n2 = names[2]
        kernels[n2] = {"bound": "hbm", "ms": avg[n2], "bytes": store_b,
                       "achieved_GBs": store_b / (avg[n2] * 1e-3) / 1e9}
    for k, rec in kernels.items():
        if rec["bound"] == "hbm":
            rec["frac"] = rec["achieved_GBs"] / HBM_PEAK_GBS
        else:
            rec["frac"] = rec["achieved_TFLOPs"] / BF16_MFMA_PEAK_TFLOPS
        rec["traffic_bytes"] = traffic_from_profiles(k)

    # Shader clock of the projection (unfused path): ten more chain steps
    # whose projection also stamps each workgroup's shader clock and constant
    # clock counters (the same kernel and bits; the call synchronizes to read
    # them). The MFMA peak is quoted at 2.4 GHz; under this load the chip
    # runs slower, and frac_at_clock rates the projection against the peak
    # scaled to the measured clock.
    if not fused and not one_call:
        clocks = []
        for _ in range(10):
            b = sets[step_no[0] % n_sets]
            step_no[0] += 1
            nrc.context_norms(b["x"], hw, pw, cfg.L, d["hidden_eps"], d["pre_eps"], out=b["normed"])
            _, clk = nrc.context_kv_project_timed(b["normed"], b["w"], out=b["kv"])
            nrc.context_kv_store(b["kv"], positions, slots, cos_sin, b["caches"], cfg.H, d["k_eps"])
            clocks.append(float(clk["shader_ghz"].median()))
        torch.cuda.synchronize()
        ghz = sorted(clocks)[len(clocks) // 2]
        rec = kernels[n1]
        rec["clock_ghz"] = ghz
        rec["frac_at_clock"] = rec["achieved_TFLOPs"] / (BF16_MFMA_PEAK_TFLOPS * ghz / PEAK_CLOCK_GHZ)
        log(f"projection shader clock {ghz:.3f} GHz (median of {len(clocks)} launches' workgroup medians); "
            f"{rec['frac_at_clock']:.3f} of the MFMA peak at that clock")

    # The dominant kernel carries the roofline object, at its average launch
    # duration over the timed region.
    rd = kernels[dom]
    if rd["bound"] == "mfma":
        achieved = rd["flops"] / (dom_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS, "traffic": rd["traffic_bytes"],
                    "kernel": dom, "ms": dom_ms}
        if "clock_ghz" in rd:
            roofline["clock_ghz"] = rd["clock_ghz"]
            roofline["frac_at_clock"] = achieved / (BF16_MFMA_PEAK_TFLOPS * rd["clock_ghz"] / PEAK_CLOCK_GHZ)
    else:
        achieved = rd["bytes"] / (dom_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": rd["traffic_bytes"], "kernel": dom, "ms": dom_ms}

    rows_per_s = cfg.T * args.steps / wall

    # Norm variants (FP32 weights, weights scaling the norms' inputs), timed
    # after the chain on the same rows: not part of the step. Each gets 20
    # warm-up launches (a new kernel path runs slower for its first dozen or
    # so launches on this GPU), then 20 timed launches, each after an untimed
    # read of 1 GiB of other memory: run back to back, the 256 MB infinity
    # cache would keep most of the 268 MB input between launches (nontemporal
    # outputs do not evict it), which the chain never sees.
    def time_launches(run, flush_src, warmup=20, timed=20):
        flush_dst = torch.empty((), dtype=torch.float32, device=dev)
        for _ in range(warmup):
            run()
        total = 0.0
        e0, e1 = timer.event(), timer.event()
        for _ in range(timed):
            torch.sum(flush_src, dim=0, out=flush_dst)
            timer.record(e0)
            run()
            timer.record(e1)
            torch.cuda.synchronize()
            total += timer.elapsed_ms(e0, e1)
        return total / timed

    # The ceiling of the norms' traffic: the norms kernel against its traffic
    # twin (the same reads and writes in the same pattern and grid, no
    # arithmetic) with the norms' streaming stores, with plain stores, and
    # its reads and its writes alone; every launch cold, as in the chain.
    ceiling = {}
    if not args.no_ceiling:
        flush_src = torch.ones(256 << 20, dtype=torch.float32, device=dev)
        twin_out = torch.empty((cfg.L, cfg.T, 8192), dtype=torch.bfloat16, device=dev)
        staged = (1 if hw is not None else 0) + (cfg.L if pw is not None and cfg.L <= 5 else 0)
        per_cu = 1 if staged * 16384 > 65536 else 2  # the norms' workgroups per CU
        nb = cfg.T * 2 * 8192
        runs = {
            "context_norms": (lambda: nrc.context_norms(x, hw, pw, cfg.L, d["hidden_eps"], d["pre_eps"],
                                                        out=twin_out), norms_b),
            "twin, the norms' stores": (lambda: nrc.traffic_twin(x, cfg.L, nrc.TWIN_NORMS_STORES, twin_out, per_cu),
                                        nb * (1 + cfg.L)),
            "twin, plain stores": (lambda: nrc.traffic_twin(x, cfg.L, nrc.TWIN_PLAIN_STORES, twin_out, per_cu),
                                   nb * (1 + cfg.L)),
            "twin, reads only": (lambda: nrc.traffic_twin(x, cfg.L, nrc.TWIN_READS_ONLY, None, per_cu), nb),
            "twin, writes only (the norms' stores)": (
                lambda: nrc.traffic_twin(x, cfg.L, nrc.TWIN_WRITES_ONLY, twin_out, per_cu), nb * cfg.L),
        }
        for name, (run, nbytes) in runs.items():
            ms = time_launches(run, flush_src)
            ceiling[name] = {"ms": ms, "bytes": nbytes, "achieved_GBs": nbytes / (ms * 1e-3) / 1e9,
                             "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        ceiling["workgroups_per_cu"] = per_cu
        del twin_out, flush_src
        log("norms ceiling (cold): " + ", ".join(f"{k} {v['frac']:.3f}" for k, v in ceiling.items()
                                                  if isinstance(v, dict)))

    variants = {}
    if not args.no_variants and hw is not None and pw is not None:
        flush_src = torch.ones(256 << 20, dtype=torch.float32, device=dev)
        hw32, pw32 = hw.float().contiguous(), pw.float().contiguous()
        vout = torch.empty((cfg.L, cfg.T, 8192), dtype=torch.bfloat16, device=dev)
        vb = cfg.T * (2 * 8192 + 2 * cfg.L * 8192) + 4 * 8192 * (1 + cfg.L)
        for his, pis in ((False, False), (True, True)):
            run = lambda: nrc.context_norms_ex(x, hw32, pw32, cfg.L, d["hidden_eps"], d["pre_eps"],
                                               hidden_input_scale=his, pre_input_scale=pis, out=vout)
            ms = time_launches(run, flush_src)
            name = "context_norms_ex[fp32 weights" + (", input-scaled]" if his else "]")
            variants[name] = {"bound": "hbm", "ms": ms, "bytes": vb, "achieved_GBs": vb / (ms * 1e-3) / 1e9,
                              "frac": vb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        # The residual boundary over the same number of rows: bf16 branch, FP32
        # stream in and out, bf16 output, bf16 norm weights.
        s_in = torch.empty((cfg.T, 8192), dtype=torch.float32, device=dev).normal_()
        alpha = torch.full((8192,), 0.9, dtype=torch.float32, device=dev)
        beta = torch.full((8192,), 1.1, dtype=torch.float32, device=dev)
        s_out = torch.empty_like(s_in)
        b_out = torch.empty((cfg.T, 8192), dtype=torch.bfloat16, device=dev)
        run = lambda: nrc.draft_boundary(x, s_in, alpha, beta, hw, pw[0], out=b_out, stream_out=s_out)
        ms = time_launches(run, flush_src)
        bb = cfg.T * 8192 * (2 + 4 + 4 + 2) + 8192 * (4 + 4 + 2 + 2)
        variants["draft_boundary[fp32 stream in/out]"] = {"bound": "hbm", "ms": ms, "bytes": bb,
                                                         "achieved_GBs": bb / (ms * 1e-3) / 1e9,
                                                         "frac": bb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del s_in, s_out, b_out, flush_src
        log("variants: " + ", ".join(f"{k}={v['ms']:.4f} ms" for k, v in variants.items()))

    # The projection against hipBLASLt on the same rows (torch.mm per layer,
    # plain 2-D products), each launch cold as in the chain; for the design
    # notes' comparison, not part of the step.
    blas = {}
    if args.hipblaslt and not fused:
        flush_src = torch.ones(256 << 20, dtype=torch.float32, device=dev)
        a_in = sets[0]["normed"]
        nrc.context_norms(x, hw, pw, cfg.L, d["hidden_eps"], d["pre_eps"], out=a_in)
        c_out = torch.empty((cfg.L, cfg.T, cfg.N), dtype=torch.bfloat16, device=dev)
        w_nd = w_kv.transpose(1, 2).contiguous()  # [L, N, D]
        runs = {
            "context_kv_project [L, D, N]": lambda: nrc.context_kv_project(a_in, w_kv, out=c_out),
            "context_kv_project [L, N, D]": lambda: nrc.context_kv_project(a_in, w_nd, out=c_out, w_layout="nd"),
            "torch.mm [L, D, N]": lambda: [torch.mm(a_in[l], w_kv[l], out=c_out[l]) for l in range(cfg.L)],
            "torch.mm [L, N, D]": lambda: [torch.mm(a_in[l], w_nd[l].t(), out=c_out[l]) for l in range(cfg.L)],
        }
        for name, run in runs.items():
            ms = time_launches(run, flush_src)
            blas[name] = {"ms": ms, "achieved_TFLOPs": flops / (ms * 1e-3) / 1e12,
                          "frac": flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}
        del flush_src, c_out, w_nd
        log("projection vs hipBLASLt (cold): " + ", ".join(f"{k} {v['ms']:.4f} ms" for k, v in blas.items()))

    cpu = None
    if not args.no_cpu_baseline:
        per_row = 2 * cfg.L * 8192 * cfg.N  # projection flop per row, the oracle's dominant stage
        rows = min(cfg.T, args.cpu_rows if args.cpu_rows > 0 else max(1, int(1.2e12 // per_row)))
        threads, model = host_cpu()
        d["caches_host_sample"] = synth.random_bits_u16(cfg.stream(synth.TID_CACHE),
                                                       (cfg.L, cfg.num_blocks, cfg.H, cfg.block_size, 128))
        log(f"cpu baseline: oracle chain on {rows} rows, {threads} threads ({model}, nproc {os.cpu_count()})")
        times = cpu_baseline(d, cfg, rows, threads)
        total = sum(times.values())
        what = "every row" if rows == cfg.T else f"the first {rows} of {cfg.T} rows"
        cpu = {"value": rows / total, "unit": "rows/s", "cores": threads, "kind": "oracle",
               "sample": f"{what} of the {cfg.name} workload, whole chain (norms, FP32 projection, store), "
                         f"plain C oracle, each stage split over {threads} host threads, {total:.1f} s",
               "cpu_model": model, "nproc": os.cpu_count(),
               "stages_s": {k: round(v, 3) for k, v in times.items()},
               "stages_rows_per_s": {k: rows / v for k, v in times.items()}}
        log("cpu baseline: " + ", ".join(f"{k} {v:.2f} s" for k, v in times.items()))

    out = {
        "metric": "context rows/s (T=16K, L=4, D=8192); % HBM BW peak; bmm % MFMA peak",
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: L={cfg.L} T={cfg.T} D=8192 H={cfg.H} N={cfg.N} "
                        f"block_size={cfg.block_size} num_blocks={cfg.num_blocks} "
                        f"rope={'[%d,64]' % cfg.max_position if cfg.rope else 'off'}",
            "global_batch": cfg.T,
            "seq_len": cfg.T,
            "parallelism": "single GPU",
            "path": args.path,
        },
        "roofline": roofline,
        "kernels": kernels,
        "variants": variants,
        "norms_ceiling": ceiling,
        "cpu_baseline": cpu,
    }
    if blas:
        out["hipblaslt"] = blas
    timer.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
