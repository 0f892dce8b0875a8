"""Benchmark of one MoE layer's data path on one MI355X: routing layout +
dispatch + combine, timed through the C ABI.

A step is one pass of the whole path over one batch: moe_layout_dispatch
(the layout's 2 kernels, which also read the token rows ahead into the
Infinity Cache, then the dispatch kernel; one fused kernel for T * K <= 8192)
and moe_combine (1 kernel), with every input already resident in HBM.  The
same work as three calls (moe_get_layout, moe_dispatch, moe_combine) is timed
beside it, with events between the calls for the per-call times.  The expert computation between dispatch and combine
is not part of the path; a stand-in expert output (the dequantized dispatched
rows, or the dispatched bf16 rows) is prepared once, untimed.

Bytes are counted in the form the DeepEP issue "#84 Questions on Profiling
dispatch_t ..." prints bandwidth (bytes / 1e9 / t), counting every copy
including those a rank sends to itself: dispatch N * (H * s + 4 [int8 scale]),
combine N * 2H, with N routed copies and s = 1 (int8) or 2 (bf16) bytes; the
closed form is the one of "Wide-EP / DBO / DeepEP hardware cliff", A short
illustrative example (tokens per rank x k x d x s).

Output: one JSON line (see main()).  --gpus above 1 is refused: the path runs
on one GPU.
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak
METRIC = "dispatch+combine µs/layer and achieved HBM GB/s (% of peak), T=4096 H=7168 k=8"
DEFAULT_WORKLOAD = 2


def comm_bytes(n_rows, hidden, payload_bytes, scale_bytes):
    """Bytes a dispatch or combine moves in the printed-bandwidth accounting:
    every routed copy once, self copies included."""
    return int(n_rows) * (int(hidden) * int(payload_bytes) + int(scale_bytes))


def dispatch_comm_bytes(n_rows, hidden, quant_mode):
    return comm_bytes(n_rows, hidden, 2 if quant_mode == 0 else 1, 4 if quant_mode == 2 else 0)


def combine_comm_bytes(n_rows, hidden):
    return comm_bytes(n_rows, hidden, 2, 0)


def dispatch_hbm_bytes(T, H, K, n_rows, n_tok_sending, quant_mode, smooth_rows):
    """Algorithmic HBM bytes of one dispatch launch: each sending token's row is read once,
    every routed copy written once, plus the slot map, the smooth scales and the per-row scale."""
    rd = n_tok_sending * 2 * H + T * K * 4 + 4 * H * int(smooth_rows)
    wr = n_rows * (H * (2 if quant_mode == 0 else 1) + (4 if quant_mode == 2 else 0))
    return rd + wr


def combine_hbm_bytes(T, H, K, n_rows, n_tok_ori):
    """Algorithmic HBM bytes of one combine launch: every routed expert-output row read
    once, ori_x for tokens with a copy/constant slot, the slot map, one bf16 row written per token."""
    return n_rows * 2 * H + n_tok_ori * 2 * H + T * K * 12 + T * 2 * H


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "combine": ["combine_moe_get_amd/csrc/combine.hip", "combine_moe_get_amd/csrc/moe_internal.hpp"],
    "dispatch": ["combine_moe_get_amd/csrc/dispatch.hip", "combine_moe_get_amd/csrc/dispatch_dev.hpp",
                 "combine_moe_get_amd/csrc/moe_internal.hpp"],
}


def counter_traffic(kernel, workload_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_name}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_h or not m_b or m_h.group(1) != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return float(m_b.group(1))


def hbm_probe(dev, nbytes=2 << 30, reps=5):
    """What library streaming kernels reach on this GPU, on a buffer 8x the Infinity Cache:
    a fill (pure write, sequential addresses) and a device-to-device copy (read + write).
    Context for the roofline, which is quoted against the published 8 TB/s."""
    import torch

    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    half = nbytes // 2

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return float(np.median(ts))

    t_w = timed(lambda: buf.fill_(1))
    t_c = timed(lambda: buf[:half].copy_(buf[half:]))
    del buf
    torch.cuda.empty_cache()
    return dict(write_GBps=round(nbytes / t_w / 1e9, 1), copy_rw_GBps=round(2 * half / t_c / 1e9, 1),
                buffer_bytes=nbytes,
                kernels="torch fill_ (its vectorized elementwise kernel) / copy_ (hipMemcpy device to device)")


def cpu_model_name():
    """The host CPU's model name as lscpu prints it (falls back to /proc/cpuinfo)."""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for ln in out.splitlines():
            if ln.startswith("Model name:"):
                return ln.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        return ""


def host_threads():
    """Worker threads for the all-cores oracle leg: the cores this process may run on, at most
    16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_pass(inp, lo_only=False):
    """One single-threaded oracle pass (layout + dispatch + combine); returns (seconds, comm bytes,
    layout) -- the expert stand-in between dispatch and combine is built outside the timing."""
    import oracle

    c = inp["cfg"]
    sh = oracle.make_shape(c["T"], c["H"], c["K"], c["E"], c["P"], c["Z"], c["C"], c["Kc"], c["num_max"])
    a = time.perf_counter()
    lo = oracle.layout(sh, inp["topk_idx"], inp["mask"])
    oracle.dispatch(sh, c["quant_mode"], inp["x"], lo, smooth=inp["smooth"], topk_idx=inp["topk_idx"])
    b = time.perf_counter()
    y = np.ascontiguousarray(inp["x"][lo["src_info"] // c["K"]])  # expert stand-in, not timed
    e0 = time.perf_counter()
    oracle.combine(sh, y, inp["topk_idx"], inp["topk_weights"], lo, inp["mask"], inp["ori_x"],
                   inp["alpha1"], inp["alpha2"], inp["const_v"])
    dt = (b - a) + (time.perf_counter() - e0)
    n = lo["num_rows"]
    return dt, dispatch_comm_bytes(n, c["H"], c["quant_mode"]) + combine_comm_bytes(n, c["H"])


def _oracle_threaded_pass(inp, nthreads, return_outputs=False):
    """The same pass with the oracle's dispatch and combine run by nthreads host threads, each on
    its own slice of tokens (both are independent per token; the C functions are called
    unchanged on the slice, and ctypes releases the interpreter lock during each call).  The
    layout -- a scan over all tokens -- stays single-threaded.  Returns (seconds, comm bytes)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    c = inp["cfg"]
    T, H, K = c["T"], c["H"], c["K"]
    sh = oracle.make_shape(T, H, K, c["E"], c["P"], c["Z"], c["C"], c["Kc"], c["num_max"])
    L = oracle.lib()
    arr = lambda a, dt: None if a is None else np.ascontiguousarray(a, dtype=dt)
    x = arr(inp["x"], np.uint16)
    topk = arr(inp["topk_idx"], np.int32)
    w = arr(inp["topk_weights"], np.float32)
    mask = arr(inp["mask"], np.uint8)
    smooth = arr(inp["smooth"], np.float32)
    ori, a1, a2, cv = (arr(inp[k], np.uint16) for k in ("ori_x", "alpha1", "alpha2", "const_v"))
    bounds = np.linspace(0, T, nthreads + 1).astype(np.int64)
    qm = c["quant_mode"]

    def ptr(a, off_elems=0):
        return None if a is None else ctypes.c_void_p(a.ctypes.data + int(off_elems) * a.itemsize)

    with ThreadPoolExecutor(nthreads) as pool:
        a = time.perf_counter()
        lo = oracle.layout(sh, topk, mask)
        n = lo["num_rows"]
        dst = np.ascontiguousarray(lo["dst_row"], np.int32)
        ex = np.zeros((max(n, 1), H), np.uint16 if qm == 0 else np.int8)
        ds = np.zeros(max(n, 1), np.float32)
        ew = np.zeros(max(n, 1), np.float32)
        srows = 0 if smooth is None else (1 if smooth.size == H else c["E"])

        def disp(i):
            t0, t1 = int(bounds[i]), int(bounds[i + 1])
            cs = oracle._CShape(*[int(v) for v in sh._replace(num_tokens=t1 - t0)])
            return L.orc_dispatch(ctypes.byref(cs), qm, ptr(x, t0 * H), ptr(smooth), srows, None,
                                  ptr(topk, t0 * K), ptr(dst, t0 * K), ptr(ex), ptr(ds), ptr(ew))

        assert all(r == 0 for r in pool.map(disp, range(nthreads)))
        b = time.perf_counter()
        y = np.ascontiguousarray(x[lo["src_info"] // K])  # expert stand-in, not timed
        out = np.zeros((T, H), np.float64)

        def comb(i):
            t0, t1 = int(bounds[i]), int(bounds[i + 1])
            cs = oracle._CShape(*[int(v) for v in sh._replace(num_tokens=t1 - t0)])
            return L.orc_combine(ctypes.byref(cs), ptr(y if y.size else np.zeros((1, H), np.uint16)),
                                 ptr(topk, t0 * K), ptr(w, t0 * K), ptr(mask, t0), ptr(dst, t0 * K),
                                 ptr(ori, t0 * H), ptr(a1), ptr(a2), ptr(cv), ptr(out, t0 * H))

        e0 = time.perf_counter()
        list(pool.map(comb, range(nthreads)))
        dt = (b - a) + (time.perf_counter() - e0)
    if return_outputs:
        return lo, ex[:n], ds[:n], out
    return dt, dispatch_comm_bytes(n, H, qm) + combine_comm_bytes(n, H)


def cpu_baseline(inp, target_seconds):
    """The oracle, as it stands, timed on this host over whole layout + dispatch + combine passes of
    the same workload: single-threaded (the baseline proper: at least 3 passes and about
    target_seconds of CPU time, median pass), and on all host cores (dispatch and combine split
    over token slices, median of 3 passes)."""
    times, comm = [], 0
    while sum(times) < target_seconds or len(times) < 3:
        dt, comm = _oracle_pass(inp)
        times.append(dt)
    med = float(np.median(times))
    nthr = host_threads()
    par = [_oracle_threaded_pass(inp, nthr) for _ in range(3)]
    pmed = float(np.median([p[0] for p in par]))
    model = cpu_model_name()
    return dict(value=round(comm / 1e9 / med, 3), unit="GB/s", cores=1, kind="oracle", cpu_model=model,
                sample=f"{len(times)} whole passes (layout + dispatch + combine) of the timed workload, "
                       f"{sum(times):.1f} s single-threaded, median pass; oracle combine in float64",
                seconds_per_pass=round(med, 4),
                all_cores=dict(value=round(par[0][1] / 1e9 / pmed, 3), unit="GB/s", cores=nthr,
                               seconds_per_pass=round(pmed, 4),
                               sample=f"median of 3 passes; dispatch and combine of the oracle on {nthr} token "
                                      f"slices in parallel host threads, layout single-threaded"))


def run_dbo(args):
    """Dual-batch overlap ("Wide-EP / DBO / DeepEP hardware cliff", section 1) DBO: hiding the
    wire) on one GPU: the batch is split into two microbatches; each runs layout + dispatch, a
    stand-in expert computation, and combine.  Sequential: everything on one stream.  Overlapped:
    layout/dispatch/combine of the microbatches on a data-movement stream while the other
    microbatch's expert GEMMs run on a compute stream, so t_seq ~ t_comm + t_compute should move
    toward max(t_comm, t_compute).  The page's resource split (VLLM_DBO_COMM_SMS compute units
    for the communication kernels) becomes a cap on the data-movement kernels' grids
    (moe_dispatch_capped / moe_combine_capped with max_workgroups; 0 = uncapped): they then hold a
    bounded number of wave slots and walk their work items, leaving the rest to the GEMMs.  The
    expert stand-in is one dense bf16 GEMM pair per microbatch, rows [N_mb, H] x [H, F] -> relu ->
    [F, H] (hipBLASLt through torch.matmul), the FLOPs of equal-sized experts of intermediate size
    F.  Both streams keep the default priority."""
    import torch

    import combine_moe_get_amd as mg
    from combine_moe_get_amd import workloads

    dev = torch.device("cuda:0")
    cid = args.workload
    inp = workloads.make_inputs(cid, seed=args.seed, T=args.tokens, P=args.ranks)
    c = inp["cfg"]
    T, H, K, E, P = c["T"], c["H"], c["K"], c["E"], c["P"]
    assert T % (2 * P) == 0
    Tm = T // 2
    shape = mg.make_shape(Tm, H, K, E, P, c["Z"], c["C"], c["Kc"], 0)

    def d(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    gen = torch.Generator(device=dev).manual_seed(args.seed)
    caps = [int(v) for v in args.dbo_caps.split(",")]
    results = []
    s_comm, s_comp = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    for F in [int(f) for f in args.dbo_f.split(",")]:
        w1 = (torch.randn((H, F), device=dev, generator=gen) / H ** 0.5).to(torch.bfloat16).contiguous()
        w2 = (torch.randn((F, H), device=dev, generator=gen) / F ** 0.5).to(torch.bfloat16).contiguous()
        mbs = []
        for m in range(2):
            sl = slice(m * Tm, (m + 1) * Tm)
            g = dict(topk=d(inp["topk_idx"][sl]), w=d(inp["topk_weights"][sl]), x=d(inp["x"][sl]),
                     mask=None if inp["mask"] is None else d(inp["mask"][sl]),
                     ori=None if inp["ori_x"] is None else d(inp["ori_x"][sl]))
            g["lay"] = mg.alloc_layout(shape, dev)
            g["ws"] = mg.alloc_workspace(shape, dev)
            g["ex"] = torch.zeros((Tm * K, H), dtype=torch.bfloat16, device=dev)
            g["y"] = torch.zeros((Tm * K, H), dtype=torch.bfloat16, device=dev)
            g["out"] = torch.empty((Tm, H), dtype=torch.bfloat16, device=dev)
            g["c_lay"] = mg.prepare_layout(shape, g["topk"], g["mask"], out=g["lay"], workspace=g["ws"])
            for cap in caps:
                g[("dis", cap)] = mg.prepare_dispatch(shape, 0, g["x"], g["lay"].dst_row, expand_x=g["ex"],
                                                      max_workgroups=cap)
                g[("com", cap)] = mg.prepare_combine(shape, g["y"], g["topk"], g["w"], g["lay"].dst_row, g["mask"],
                                                     g["ori"], d(inp["alpha1"]), d(inp["alpha2"]),
                                                     d(inp["const_v"]), out=g["out"], max_workgroups=cap)
            mbs.append(g)

        def experts(g, st):
            with torch.cuda.stream(st):
                h = torch.matmul(g["ex"], w1)
                h.relu_()
                torch.matmul(h, w2, out=g["y"])

        s_main = torch.cuda.current_stream()
        ev = [torch.cuda.Event() for _ in range(4)]

        def sequential():
            for g in mbs:
                g["c_lay"](s_main)
                g[("dis", 0)](s_main)
                experts(g, s_main)
                g[("com", 0)](s_main)

        def overlapped(cap):
            # data-movement stream: layout + dispatch of both microbatches, then each combine once
            # its microbatch's experts are done; compute stream: the experts
            s_comm.wait_stream(s_main)
            s_comp.wait_stream(s_main)
            for m, g in enumerate(mbs):
                g["c_lay"](s_comm)
                g[("dis", cap)](s_comm)
                ev[m].record(s_comm)
            for m, g in enumerate(mbs):
                s_comp.wait_event(ev[m])
                experts(g, s_comp)
                ev[2 + m].record(s_comp)
            for m, g in enumerate(mbs):
                s_comm.wait_event(ev[2 + m])
                g[("com", cap)](s_comm)
            s_main.wait_stream(s_comm)
            s_main.wait_stream(s_comp)

        def comm_only(cap):
            for g in mbs:
                g["c_lay"](s_main)
                g[("dis", cap)](s_main)
                g[("com", cap)](s_main)

        def compute_only():
            for g in mbs:
                experts(g, s_main)

        def timed(fn):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s_main)
            for _ in range(args.steps):
                fn()
            b.record(s_main)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / args.steps * 1e3

        sequential()
        torch.cuda.synchronize()
        ref = [g["out"].clone() for g in mbs]
        t_comm, t_comp = timed(lambda: comm_only(0)), timed(compute_only)
        t_seq = timed(sequential)
        flops = 2 * 2 * (Tm * K) * H * F * 2  # two microbatches, two GEMMs each
        for cap in caps:
            t_dbo = timed(lambda: overlapped(cap))
            t_comm_cap = timed(lambda: comm_only(cap))
            same = all(torch.equal(g["out"], r) for g, r in zip(mbs, ref))
            results.append(dict(F=F, comm_max_workgroups=cap if cap else "uncapped",
                                t_comm_us=round(t_comm, 1), t_comm_capped_us=round(t_comm_cap, 1),
                                t_compute_us=round(t_comp, 1), t_seq_us=round(t_seq, 1),
                                t_dbo_us=round(t_dbo, 1), ideal_us=round(max(t_comm, t_comp), 1),
                                saved_frac_of_comm=round((t_seq - t_dbo) / max(t_comm, 1e-9), 3),
                                gemm_TFLOPs=round(flops / (t_comp * 1e-6) / 1e12, 1), outputs_equal=same))
            print(json.dumps(results[-1]), file=sys.stderr, flush=True)
        del mbs, w1, w2
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "dual-batch overlap of dispatch/combine with expert GEMMs (t_seq vs t_dbo)",
                      "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "config": {"workload": c["name"], "T": T, "microbatch_tokens": Tm, "H": H, "k": K,
                                 "E": E, "P": P, "dispatch": "bf16"},
                      "results": results}), flush=True)


def run_write_sweep(args):
    """Write-pattern sweep with libmoe_hbm_probe.so: rows of R bytes (1-16 KB) stored at randomly
    permuted row slots (eight rows per workgroup, as the dispatch's copies of one token), against the
    same bytes stored in address order; about 940 MB per launch, far beyond the 256 MB Infinity Cache.
    Prints one JSON line."""
    import torch

    dev = torch.device("cuda:0")
    plib = ctypes.CDLL(PROBE_LIB_PATH)
    plib.moe_probe_scatter_write.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p]
    plib.moe_probe_ordered_write.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    total = 940 << 20
    buf = torch.empty(total + (1 << 20), dtype=torch.uint8, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    gen = torch.Generator(device=dev).manual_seed(args.seed)
    res = []
    for R in (1024, 2048, 4096, 7168, 8192, 14336, 16384):
        nrows = total // R // 8 * 8
        perm = torch.randperm(nrows, generator=gen, device=dev).to(torch.int32).view(nrows // 8, 8).contiguous()

        def t_of(fn):
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3)
            return float(np.median(ts))

        def scat():
            if plib.moe_probe_scatter_write(ctypes.c_void_p(perm.data_ptr()), nrows // 8, 8, R,
                                            ctypes.c_void_p(buf.data_ptr()), st) != 0:
                raise RuntimeError("probe refused its arguments")

        def ordered():
            if plib.moe_probe_ordered_write(nrows, R, ctypes.c_void_p(buf.data_ptr()), st) != 0:
                raise RuntimeError("probe refused its arguments")

        ts, to = t_of(scat), t_of(ordered)
        b = nrows * R
        res.append(dict(row_bytes=R, bytes=b, random_slots_us=round(ts, 1), random_slots_GBps=round(b / ts / 1e3, 1),
                        address_order_us=round(to, 1), address_order_GBps=round(b / to / 1e3, 1)))
        print(json.dumps(res[-1]), file=sys.stderr, flush=True)
        del perm
    print(json.dumps({"metric": "HBM write rate by row size: rows at random slots vs address order",
                      "unit": "GB/s", "n_gpus": 1, "results": res}), flush=True)


MALL_BYTES = 256 << 20  # MI355X Infinity Cache
PROBE_LIB_PATH = os.path.join(ROOT, "combine_moe_get_amd", "libmoe_hbm_probe.so")
# what the path moves and computes in, per quant mode (the JSON line's dtype)
PAYLOAD = {0: "bf16 dispatch and combine", 1: "int8 dispatch (static), bf16 combine",
           2: "int8 dispatch + fp32 row scale, bf16 combine"}
PAYLOAD_DISPATCH = {0: "bf16 rows", 1: "int8 codes (static), fp32 quantization math",
                    2: "int8 codes + one fp32 scale per row, fp32 quantization math"}


def rotation_sets(x_bytes):
    """Input sets the timed loops cycle through so that no token row is still cached when it is
    read again: the x rows of all sets together span twice the Infinity Cache.  (With two sets the
    x rows of both stayed cached between steps -- the other traffic of a step is non-temporal --
    and dispatch read them from the cache: 47 us instead of 59 us at workload 2.)"""
    return int(min(12, max(2, -(-2 * MALL_BYTES // max(int(x_bytes), 1)))))


def measure(args, mg, workloads, dev, tokens=None, ranks=None, copy_probe=False, cid=None, headline=True):
    """One step benchmark of a workload (tokens / ranks override T and P); returns the JSON
    line without cpu_baseline, and the first input set.  headline=False: the workload as named
    (no --quant / --smooth / --rank-stride overrides) and none of the extra measurements."""
    import torch

    cid = args.workload if cid is None else cid
    first = workloads.make_inputs(cid, seed=args.seed, T=tokens, P=ranks)
    n_sets = args.rotate if args.rotate else rotation_sets(first["x"].nbytes)
    sets = [first] + [workloads.make_inputs(cid, seed=args.seed + r, T=tokens, P=ranks) for r in range(1, n_sets)]
    c = sets[0]["cfg"]
    T, H, K, E, P, qm = c["T"], c["H"], c["K"], c["E"], c["P"], c["quant_mode"]
    if args.quant is not None and headline:
        qm = c["quant_mode"] = args.quant
    if args.smooth is not None and headline:
        for r, inp in enumerate(sets):
            rng = workloads.rng_for(args.seed + r, cid, 4)
            inp["smooth"] = (None if args.smooth == "none" else
                             rng.uniform(0.5, 1.5, H if args.smooth == "channel" else (E, H)).astype(np.float32))
        c["smooth"] = args.smooth
    shape = mg.make_shape(T, H, K, E, P, c["Z"], c["C"], c["Kc"], c["num_max"])
    A = 0 if not headline else mg.rank_capacity(shape) if args.rank_stride == "min" else int(args.rank_stride)
    cap = P * A if A > 0 else T * K

    def d(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    gsets = []
    for inp in sets:
        g = dict(topk=d(inp["topk_idx"]), w=d(inp["topk_weights"]), mask=d(inp["mask"]), x=d(inp["x"]),
                 smooth=d(inp["smooth"]), ori=d(inp["ori_x"]), a1=d(inp["alpha1"]), a2=d(inp["alpha2"]),
                 v=d(inp["const_v"]))
        g["lay"] = mg.alloc_layout(shape, dev, A)
        g["ws"] = mg.alloc_workspace(shape, dev)
        g["ex"] = torch.empty((cap, H), dtype=torch.bfloat16 if qm == 0 else torch.int8, device=dev)
        g["ds"] = torch.empty(cap, dtype=torch.float32, device=dev) if qm == 2 else None
        g["out"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        # stand-in expert outputs (untimed): dequantized / copied dispatched rows, or N(0,1)
        mg.layout(shape, g["topk"], g["mask"], out=g["lay"], workspace=g["ws"], rank_stride=A)
        mg.dispatch(shape, qm, g["x"], g["lay"].dst_row, g["smooth"], None, g["topk"], g["ex"], g["ds"])
        torch.cuda.synchronize()
        n = int(g["lay"].expert_offsets[-1])
        used = torch.sort(g["lay"].dst_row[g["lay"].dst_row >= 0]).values.long()  # rows holding a copy
        if c["Kc"] + c["C"] > 0 or qm == 1 or (g["smooth"] is not None and g["smooth"].dim() == 2):
            yv = d(workloads.expert_out_normal(n, H, seed=args.seed, config_id=cid))
        elif qm == 0:
            yv = g["ex"][used]
        else:
            yv = g["ex"][used].float() * g["ds"][used, None]
            if g["smooth"] is not None:
                yv = yv / g["smooth"][None, :]
            yv = yv.to(torch.bfloat16)
        g["y"] = torch.empty((max(cap, 1), H), dtype=torch.bfloat16, device=dev)
        g["y"][used] = yv
        del yv, used
        g["n"] = n
        g["n_send"] = int((g["lay"].dst_row >= 0).any(dim=1).sum())
        ids = g["topk"]
        special_copy = (ids >= E + c["Z"]) & (ids < E + c["Z"] + c["C"] + c["Kc"])
        act = torch.ones(T, dtype=torch.bool, device=dev) if g["mask"] is None else g["mask"].bool()
        g["n_ori"] = int((special_copy.any(dim=1) & act).sum())
        gsets.append(g)
    del sets[1:]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    for g in gsets:  # arguments checked and marshalled once; a step is two bare C calls
        g["c_lay"] = mg.prepare_layout(shape, g["topk"], g["mask"], out=g["lay"], workspace=g["ws"], rank_stride=A)
        g["c_dis"] = mg.prepare_dispatch(shape, qm, g["x"], g["lay"].dst_row, g["smooth"], None, g["topk"],
                                         g["ex"], g["ds"], rows=cap)
        g["c_com"] = mg.prepare_combine(shape, g["y"], g["topk"], g["w"], g["lay"].dst_row, g["mask"], g["ori"],
                                        g["a1"], g["a2"], g["v"], out=g["out"])
        # the same layout + dispatch through the one-call entry point (same output buffers)
        g["c_ld"] = mg.prepare_layout_dispatch(shape, qm, g["x"], g["topk"], g["mask"], g["smooth"], None,
                                               out=g["lay"], expand_x=g["ex"], dynamic_scales=g["ds"],
                                               workspace=g["ws"], rank_stride=A)

    # the timed step is the library's layer path: moe_layout_dispatch (layout and dispatch in one
    # call; one kernel for T * K <= 8192, else the layout kernels, which also read the token rows
    # ahead into the Infinity Cache, then the dispatch) and moe_combine
    def step(g, st=None):
        st = stream if st is None else st
        g["c_ld"](st)
        g["c_com"](st)

    # the same work as three calls, events between them: what each call takes inside a step
    def step3(g, ev=None, st=None):
        st = stream if st is None else st
        if ev is not None:
            ev[0].record(st)
        g["c_lay"](st)
        if ev is not None:
            ev[1].record(st)
        g["c_dis"](st)
        if ev is not None:
            ev[2].record(st)
        g["c_com"](st)
        if ev is not None:
            ev[3].record(st)

    # untimed warmup: W steps, and at least two passes over every rotating input set, so that no
    # buffer is touched for the first time inside a timed loop (measured: with W = 5 and ten sets,
    # the per-expert-scale layer timed 236.7 us against 218.1 us after 50 warmup steps)
    n_warm = max(args.warmup, 2 * len(gsets))
    for i in range(n_warm):
        step(gsets[i % len(gsets)])
        step3(gsets[i % len(gsets)])
    torch.cuda.synchronize()

    graphs = None
    if args.graph:
        # eager reference outputs, then one captured step per input set; every replay below
        # is compared with the eager result
        ref = []
        for g in gsets:
            step(g)
            torch.cuda.synchronize()
            ref.append((g["lay"].dst_row.clone(), g["ex"].clone(), g["out"].clone()))
        graphs = []
        for g in gsets:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step(g, st=torch.cuda.current_stream())
            graphs.append(gr)
        torch.cuda.synchronize()
        for rep in range(3):
            for g, gr, r in zip(gsets, graphs, ref):
                g["out"].zero_()
                gr.replay()
                torch.cuda.synchronize()
                if not (torch.equal(g["lay"].dst_row, r[0]) and torch.equal(g["ex"], r[1])
                        and torch.equal(g["out"], r[2])):
                    raise RuntimeError("graph replay differs from the eager step")
        stream = torch.cuda.current_stream()

    # whole-step timing: K steps between two events, nothing else in between
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        if graphs is not None:
            graphs[i % len(graphs)].replay()
        else:
            step(gsets[i % len(gsets)])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # the same steps as three calls, timed alike (nothing between the calls)
    t_start.record(stream)
    for i in range(args.steps):
        step3(gsets[i % len(gsets)])
    t_end.record(stream)
    torch.cuda.synchronize()
    three_ms = t_start.elapsed_time(t_end) / args.steps

    # per-call timing inside steps: the three-call steps with events between the calls
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step3(gsets[i % len(gsets)], evs[i])
    torch.cuda.synchronize()
    lay_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dis_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    com_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])

    # kernel durations: each hot kernel launched back to back between two events on its
    # launch stream (what a kernel trace reports per dispatch)
    def kernel_avg_ms(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn(gsets[0])
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(args.steps):
            fn(gsets[i % len(gsets)])
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    k_dis = kernel_avg_ms(lambda g: g["c_dis"](stream))
    k_com = kernel_avg_ms(lambda g: g["c_com"](stream))
    k_lay = kernel_avg_ms(lambda g: g["c_lay"](stream))
    status = max(int(g["lay"].status[0]) for g in gsets)

    # the same dispatch kernel writing the same copies in token-major order (row = index of the
    # copy in (token, slot) order): what the expert-major placement the layout prescribes costs
    row_probe = None
    if args.row_probe and headline:
        for g in gsets:
            valid = g["lay"].dst_row >= 0
            tm = torch.cumsum(valid.flatten().to(torch.int32), 0, dtype=torch.int32).view_as(valid) - 1
            g["tm_rows"] = torch.where(valid, tm, torch.full_like(tm, -1)).contiguous()
            g["c_dis_tm"] = mg.prepare_dispatch(shape, qm, g["x"], g["tm_rows"], g["smooth"], None, g["topk"],
                                                g["ex"], g["ds"], rows=cap)
        k_tm = kernel_avg_ms(lambda g: g["c_dis_tm"](stream))
        row_probe = dict(expert_major_us=round(k_dis * 1e3, 2), token_major_us=round(k_tm * 1e3, 2),
                         what="dispatch kernel, same copies and bytes, rows in expert-major (the layout's) "
                              "or token-major order")

    # the dispatch's write pattern alone: the same row map and bytes, stores only, next to the same
    # bytes stored in address order (libmoe_hbm_probe.so)
    write_probe = read_probe = None
    if headline and tokens is None and ranks is None and not args.no_write_probe and os.path.exists(PROBE_LIB_PATH):
        plib = ctypes.CDLL(PROBE_LIB_PATH)
        plib.moe_probe_scatter_write.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_void_p, ctypes.c_void_p]
        plib.moe_probe_ordered_write.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        rowb = H * (2 if qm == 0 else 1)

        def probe_call(rc):
            if rc != 0:
                raise RuntimeError(f"write-pattern probe refused its arguments ({rc})")

        st_ptr = ctypes.c_void_p(stream.cuda_stream)
        k_sc = kernel_avg_ms(lambda g: probe_call(plib.moe_probe_scatter_write(
            ctypes.c_void_p(g["lay"].dst_row.data_ptr()), T, K, rowb, ctypes.c_void_p(g["ex"].data_ptr()), st_ptr)))
        k_or = kernel_avg_ms(lambda g: probe_call(plib.moe_probe_ordered_write(
            g["n"], rowb, ctypes.c_void_p(g["ex"].data_ptr()), st_ptr)))
        # the combine's reads alone: its rows gathered in its launch shape, no output rows written
        plib.moe_probe_gather_read.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        nsl = (2 * H // 16 + 127) // 128
        sink = torch.empty((T * nsl * 64, 4), dtype=torch.int32, device=dev)
        k_rd = kernel_avg_ms(lambda g: probe_call(plib.moe_probe_gather_read(
            ctypes.c_void_p(g["lay"].dst_row.data_ptr()), T, K, 2 * H, ctypes.c_void_p(g["y"].data_ptr()),
            ctypes.c_void_p(sink.data_ptr()), st_ptr)))
        rbytes = float(np.mean([g["n"] for g in gsets])) * 2 * H
        read_probe = dict(row_bytes=2 * H, bytes_per_launch=int(rbytes), gathered_rows_us=round(k_rd * 1e3, 2),
                          gathered_rows_GBps=round(rbytes / 1e9 / (k_rd * 1e-3), 1),
                          combine_kernel_us=round(k_com * 1e3, 2),
                          what="reads only: the combine's expert-output rows gathered in its launch shape (one wave "
                               "per token and 2 KB slice, non-temporal loads), no output rows written")
        del sink
        # the combine's reads and writes with XOR in place of its arithmetic, on its row map and on
        # T K rows read in address order (outputs to a buffer of their own)
        if hasattr(plib, "moe_probe_reduce") and gsets[0]["y"].shape[0] >= T * K:
            plib.moe_probe_reduce.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
            pout = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            k_gr = kernel_avg_ms(lambda g: probe_call(plib.moe_probe_reduce(
                ctypes.c_void_p(g["lay"].dst_row.data_ptr()), T, K, 2 * H, ctypes.c_void_p(g["y"].data_ptr()),
                ctypes.c_void_p(pout.data_ptr()), 1, st_ptr)))
            k_sr = kernel_avg_ms(lambda g: probe_call(plib.moe_probe_reduce(
                None, T, K, 2 * H, ctypes.c_void_p(g["y"].data_ptr()), ctypes.c_void_p(pout.data_ptr()), 0, st_ptr)))
            del pout
            gb = rbytes + T * 2 * H
            sb = float(T * K + T) * 2 * H
            read_probe["reduce"] = dict(
                gathered_us=round(k_gr * 1e3, 2), gathered_GBps=round(gb / 1e9 / (k_gr * 1e-3), 1),
                address_order_us=round(k_sr * 1e3, 2), address_order_GBps=round(sb / 1e9 / (k_sr * 1e-3), 1),
                what="the combine's reads and writes (K rows in, one row out per token, 2 KB slice per wave, "
                     "non-temporal) with XOR instead of its arithmetic: on the combine's row map, and on the "
                     "T K rows in address order")
        wbytes = float(np.mean([g["n"] for g in gsets])) * rowb
        write_probe = dict(
            row_bytes=rowb, bytes_per_launch=int(wbytes),
            scattered_rows_us=round(k_sc * 1e3, 2), scattered_rows_GBps=round(wbytes / 1e9 / (k_sc * 1e-3), 1),
            address_order_us=round(k_or * 1e3, 2), address_order_GBps=round(wbytes / 1e9 / (k_or * 1e-3), 1),
            dispatch_kernel_us=round(k_dis * 1e3, 2),
            what="stores only (no reads): every receive row of the dispatch's own row map, one workgroup per "
                 "token as the int8 dispatch, against the same bytes stored in address order")

    # moe_layout_dispatch alone, and the step as three calls (moe_get_layout, moe_dispatch,
    # moe_combine; the dispatch then reads the token rows from HBM)
    k_ld = kernel_avg_ms(lambda g: g["c_ld"](stream))
    three_call = dict(us_per_layer=round(three_ms * 1e3, 2), layout_dispatch_call_us=round(k_ld * 1e3, 2),
                      layout_dispatch_launches=mg.layout_dispatch_launches(shape, qm),
                      what="us_per_layer: the step as moe_get_layout + moe_dispatch + moe_combine (timed like the "
                           "headline step); layout_dispatch_call_us: moe_layout_dispatch back to back")

    n_avg = float(np.mean([g["n"] for g in gsets]))
    cb_d = dispatch_comm_bytes(n_avg, H, qm)
    cb_c = combine_comm_bytes(n_avg, H)
    hb_d = float(np.mean([dispatch_hbm_bytes(T, H, K, g["n"], g["n_send"], qm,
                                             0 if g["smooth"] is None else g["smooth"].numel() // H)
                          for g in gsets]))
    hb_c = float(np.mean([combine_hbm_bytes(T, H, K, g["n"], g["n_ori"]) for g in gsets]))
    us_layer = ms_per_step * 1e3
    value = (cb_d + cb_c) / 1e9 / (ms_per_step * 1e-3)

    def kstats(k_ms, call_ms, comm, hbm):
        d = dict(kernel_us=round(k_ms * 1e3, 2), in_step_us=round(float(call_ms.mean()) * 1e3, 2),
                 in_step_us_median=round(float(np.median(call_ms)) * 1e3, 2),
                 in_step_us_min=round(float(call_ms.min()) * 1e3, 2),
                 in_step_us_p90=round(float(np.percentile(call_ms, 90)) * 1e3, 2))
        if comm is not None:
            d.update(comm_bytes=int(comm), hbm_bytes=int(hbm),
                     comm_GBps=round(comm / 1e9 / (k_ms * 1e-3), 1), hbm_GBps=round(hbm / 1e9 / (k_ms * 1e-3), 1))
            d["comm_pct_of_peak"] = round(100 * d["comm_GBps"] / HBM_PEAK_GBPS, 1)
            d["hbm_pct_of_peak"] = round(100 * d["hbm_GBps"] / HBM_PEAK_GBPS, 1)
        return d

    kern = {"dispatch": kstats(k_dis, dis_ms, cb_d, hb_d), "combine": kstats(k_com, com_ms, cb_c, hb_c),
            "layout": kstats(k_lay, lay_ms, None, None)}
    kern["dispatch"]["payload"] = PAYLOAD_DISPATCH[qm]
    kern["combine"]["payload"] = "bf16 expert rows in, bf16 out, fp32 accumulation"
    kern["layout"]["payload"] = "int32 ids and indices"
    kern["layout"]["launches"] = mg.layout_launches(shape)
    dom = "combine" if k_com >= k_dis else "dispatch"
    ach = kern[dom]["hbm_GBps"]
    traffic = counter_traffic(dom, c["name"])
    roofline = dict(bound="hbm", kernel=dom, achieved=ach, peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBPS, 4),
                    traffic=None if traffic is None else int(traffic),
                    algorithmic_bytes_per_launch=kern[dom]["hbm_bytes"],
                    kernel_us=kern[dom]["kernel_us"])

    if copy_probe:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": PAYLOAD[qm] + "; fp32 math",
        "data": "synthetic (seeded generators; no dataset or weights)",
        "config": {"workload": c["name"] + ("" if tokens is None and ranks is None else
                                            f" (T={T}, P={P} override)"), "desc": c["desc"], "T": T, "H": H, "k": K, "E": E, "P": P,
                   "zero_copy_const": [c["Z"], c["C"], c["Kc"]], "quant_mode": qm,
                   "smooth": ("expert [E, H]" if sets[0]["smooth"] is not None and sets[0]["smooth"].ndim == 2
                              else "channel [H]" if sets[0]["smooth"] is not None else "none"),
                   "num_max_dispatch_tokens_per_rank": c["num_max"], "seed": args.seed,
                   "rotating_input_sets": len(gsets), "rows_N": n_avg,
                   "launch": "hip_graph" if graphs is not None else "eager",
                   "receive_layout": f"rank windows of {A} rows" if A > 0 else "compact"},
        "us_per_layer": round(us_layer, 2),
        "pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 1),
        "kernels": kern,
        "device_status": status,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    line["three_call_step"] = three_call
    if row_probe is not None:
        line["row_placement_probe"] = row_probe
    if write_probe is not None:
        line["write_pattern_probe"] = write_probe
    if read_probe is not None:
        line["read_pattern_probe"] = read_probe
    return line, sets[0]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--tokens", type=int, default=None, help="override T (a multiple of the rank count)")
    ap.add_argument("--quant", type=int, default=None, choices=[0, 1, 2], help="override the quant mode")
    ap.add_argument("--smooth", default=None, choices=["none", "channel", "expert"],
                    help="override the smooth scales: none, one [H] vector, or [E, H] per expert")
    ap.add_argument("--ranks", type=int, default=None,
                    help="override P; with --tokens equal to one rank's batch this times one rank's share")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input sets cycled through; 0 (default): enough that the token rows of all sets "
                         "span twice the 256 MB Infinity Cache (at most 12)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rank-stride", default="0",
                    help="receive layout: 0 compact rows; 'min' or an integer A >= the rank capacity "
                         "puts rank r's rows in the fixed window [r A, r A + A)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step per input set in a HIP graph and time graph replays "
                         "(every replay is checked bit for bit against the eager step)")
    ap.add_argument("--dbo", action="store_true",
                    help="dual-batch overlap measurement instead of the step benchmark (prints its own JSON line)")
    ap.add_argument("--dbo-f", default="256,512,2048", help="expert intermediate sizes F for --dbo")
    ap.add_argument("--dbo-caps", default="0,512,1024,2048,4096",
                    help="grid caps (max workgroups) of the data-movement kernels in --dbo; 0 = uncapped")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the HBM probe (fill and copy of a 2 GiB buffer with library kernels)")
    ap.add_argument("--no-share", action="store_true",
                    help="skip the extra measurement of one rank's share (T = BS, P = 1)")
    ap.add_argument("--row-probe", action="store_true",
                    help="also time the dispatch kernel with token-major receive rows (write-pattern probe)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, run a plain 512 MiB device copy 3x (counter calibration)")
    ap.add_argument("--no-write-probe", action="store_true",
                    help="skip the access-pattern probes (the dispatch's row map, stores only, vs address order; "
                         "the combine's rows, reads only)")
    ap.add_argument("--write-sweep", action="store_true",
                    help="write-pattern sweep over row sizes (random slots vs address order) instead of the step "
                         "benchmark (prints its own JSON line)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other named workloads (each timed like the headline one, summarized in "
                         "the line's 'workloads' key)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this MoE dispatch/combine path runs on one GPU only; --gpus above 1 is not "
              "supported (the simulated expert-parallel world of P ranks lives on the one GPU).",
              file=sys.stderr, flush=True)
        sys.exit(2)

    if args.dbo:
        run_dbo(args)
        return
    if args.write_sweep:
        run_write_sweep(args)
        return

    import torch

    import combine_moe_get_amd as mg
    from combine_moe_get_amd import workloads

    if not os.path.exists(mg.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    line, inp0 = measure(args, mg, workloads, dev, args.tokens, args.ranks, copy_probe=args.copy_probe)
    if args.tokens is None and args.ranks is None and not args.no_share and not args.graph:
        # one simulated rank's share at its real shape: its BS tokens, all E experts local
        bs = line["config"]["T"] // line["config"]["P"]
        sh, _ = measure(args, mg, workloads, dev, bs, 1)
        line["one_rank_share"] = dict(
            T=bs, P=1, us_per_layer=sh["us_per_layer"],
            kernel_us={k: v["kernel_us"] for k, v in sh["kernels"].items()},
            in_step_us_median={k: v["in_step_us_median"] for k, v in sh["kernels"].items()},
            layout_launches=sh["kernels"]["layout"]["launches"],
            three_call_step=sh.get("three_call_step"))
    overrides = (args.tokens, args.ranks, args.quant, args.smooth) != (None, None, None, None) or \
        args.rank_stride not in ("0", 0) or args.graph
    if not args.no_workloads and not overrides:
        # every other named workload, timed the same way (layout / dispatch / combine kernels back
        # to back over rotating input sets), summarized next to the headline one
        wl = {}
        for cid in (1, 2, 3, 4, 5):
            if cid == args.workload:
                continue
            sub, _ = measure(args, mg, workloads, dev, cid=cid, headline=False)
            k = sub["kernels"]
            cfg = sub["config"]
            wl[cfg["workload"]] = dict(
                T=cfg["T"], H=cfg["H"], k=cfg["k"], E=cfg["E"], P=cfg["P"], zero_copy_const=cfg["zero_copy_const"],
                quant_mode=cfg["quant_mode"], rows_N=cfg["rows_N"], rotating_input_sets=cfg["rotating_input_sets"],
                us_per_layer=sub["us_per_layer"], value_GBps=sub["value"], pct_of_peak=sub["pct_of_peak"],
                three_call_us_per_layer=sub["three_call_step"]["us_per_layer"],
                layout_us=k["layout"]["kernel_us"], layout_launches=k["layout"]["launches"],
                dispatch=dict((f, k["dispatch"][f]) for f in ("kernel_us", "comm_bytes", "hbm_bytes", "comm_GBps",
                                                                "comm_pct_of_peak", "hbm_pct_of_peak", "payload")),
                combine=dict((f, k["combine"][f]) for f in ("kernel_us", "comm_bytes", "hbm_bytes", "comm_GBps",
                                                              "comm_pct_of_peak", "hbm_pct_of_peak")),
                device_status=sub["device_status"])
            print(json.dumps({"workload": cfg["workload"], "us_per_layer": sub["us_per_layer"],
                              "dispatch_us": k["dispatch"]["kernel_us"], "combine_us": k["combine"]["kernel_us"]}),
                  file=sys.stderr, flush=True)
            del sub
            torch.cuda.empty_cache()
        line["workloads"] = wl
    if not args.no_probe:
        line["hbm_probe"] = hbm_probe(dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp0, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
