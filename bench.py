"""Benchmark of the RRS A4W4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload o_proj]

A step is one rrs_linear call (front end + grouped INT4 GEMM) on one batch of
synthetic activations already resident in HBM. Default workload: the
LLaMA-3-8B o_proj prefill shape, M=2048 tokens, K=N=4096, G=128.

Prints one JSON line: effective int TOPS of the whole layer (2MNK per step),
the front end's GB/s, a roofline object for the dominant kernel (the GEMM,
whose int4 x int4 products run on fp8 matrix cores, against the dense fp8
peak, which equals the dense int8 peak) and one for the front end (against
HBM peak), each kernel timed alone with HIP events on the stream it runs on,
and the CPU oracle timed on the host as a reported baseline. The oracle leg
also checks the timed run's own outputs (codes of every token, Y on sampled
rows) and reports the counts.

Before the counted warm-up steps, steps run for --settle-s seconds so that
the shader clock reaches its loaded level; the clock levels are sampled
while the timed loop's work is still running on the GPU.

--ablation times the component switches of the method (Runtime Smooth
alone, the rotation alone, the full method) on the same workload, each
with the oracle's output error, in an "ablation" list of the same line.

HBM traffic per launch ("traffic") comes from rocprofv3 FETCH_SIZE and
WRITE_SIZE counter runs recorded in profiles/traffic.txt, scaled by the
same counters read for a plain copy of known size (``--copy-probe``); it is
reported only while the kernel's source file still hashes to the value the
counters were taken with, else null.

To keep the 256 MB Infinity Cache from serving repeated inputs, the timed
loops rotate over enough independent input/weight/output sets to exceed it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TOPS = 5000.0      # MI355X dense fp8 (and int8) MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=1000, help="untimed steps before the timed ones")
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="seconds of untimed steps before the warm-up steps (the shader clock needs tens of "
                         "milliseconds of load to reach its loaded level)")
    ap.add_argument("--ablation", action="store_true",
                    help="also time Runtime Smooth alone and the rotation alone (and report the oracle's error "
                         "of each variant); every G of the workload")
    ap.add_argument("--workload", default="o_proj")
    ap.add_argument("--G", type=int, default=None)
    ap.add_argument("--signed", action="store_true",
                    help="time the signed rotation X D H (random sign mask) instead of X H")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-gemm-only", action="store_true",
                    help="run only the GEMM loop (for counter collection)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times "
                         "(reference dispatch for scaling HBM counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")
CSRC = os.path.join(ROOT, "rotated_runtime_activation_amd", "csrc")


def source_hash(name):
    import hashlib
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_traffic(kernel, source, workload):
    """Bytes per launch (fetch + write) recorded for this kernel and workload
    with the current source, or None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    sha = source_hash(source)
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 6 and parts[0] == kernel and parts[1] == workload and parts[2] == sha:
                return {"fetch_bytes": int(parts[3]), "write_bytes": int(parts[4]),
                        "bytes": int(parts[3]) + int(parts[4]), "copy_scale": float(parts[5]),
                        "source": f"{source}@{sha}"}
    return None


def sample_clocks():
    """Current shader / memory clock levels from the driver's sysfs tables
    (the level marked with *); no program is started from this process."""
    import glob
    clocks = {}
    try:
        for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_[sm]clk")):
            cur = [l.strip() for l in open(path) if "*" in l]
            if cur:
                clocks[path.split("/")[-3] + ":" + path.rsplit("_", 1)[-1]] = cur[0]
    except Exception:
        pass
    return clocks or None


def copy_probe(mib):
    import torch
    dev = torch.device("cuda:0")
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {args.gpus} is not supported (the layer would shard "
              "by output channels with no exchange: each GPU runs these kernels on its N / p channels)",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import torch
    import rotated_runtime_activation_amd as rra
    import workloads

    wl = workloads.WORKLOADS[args.workload]
    G = args.G or wl.G[len(wl.G) // 2]
    M, K, N = wl.M, wl.K, wl.N
    # recorded counters are per workload, and per G where it sweeps G
    tkey = wl.name if len(wl.G) == 1 else f"{wl.name}_G{G}"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    x = workloads.runtime_x(wl)
    w = workloads.weights(wl)
    xc = workloads.calib_x(wl)

    # calibration reorder and weight preparation on the GPU (offline steps)
    X0 = torch.from_numpy(x).to(dev)
    W0 = torch.from_numpy(w).to(dev)
    perm = torch.empty(K, dtype=torch.int32, device=dev)
    cws = torch.empty(rra.rrs_calibrate_workspace_bytes(K), dtype=torch.uint8, device=dev)
    rra.rrs_calibrate_perm(torch.from_numpy(xc).to(dev), perm, cws)
    wq0 = torch.empty(rra.rrs_weight_bytes(K, N), dtype=torch.uint8, device=dev)
    dsign = None
    if args.signed:
        bits = np.random.default_rng(1234).integers(0, 2**32, size=K // 32, dtype=np.uint64).astype(np.uint32)
        dsign = torch.from_numpy(bits.view(np.int32)).to(dev)
        rra.rrs_calibrate_perm_signed(torch.from_numpy(xc).to(dev), dsign, perm, cws)
        rra.rrs_prepare_weights_signed(W0, perm, dsign, wq0)
    else:
        rra.rrs_prepare_weights(W0, perm, wq0)
    del W0

    ws_bytes = rra.rrs_workspace_bytes(M, K, G)
    set_bytes = X0.numel() * 2 + wq0.numel() + M * N * 4 + ws_bytes
    # enough sets to exceed the Infinity Cache twice (at most 64: tiny
    # shapes would need tens of thousands, and stay cache-resident anyway)
    nsets = min(64, max(3, -(-2 * MALL_BYTES // set_bytes)))
    sets = []
    for _ in range(nsets):
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        rra.rrs_workspace_init(ws)
        sets.append(dict(X=X0.clone(), wq=wq0.clone(), Y=torch.empty(M, N, dtype=torch.float32, device=dev),
                         ws=ws, views=rra.workspace_regions(ws, M, K, G)))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(i):
        s = sets[i % nsets]
        if dsign is None:
            rra.rrs_linear(s["X"], G, perm, s["wq"], s["Y"], s["ws"], stream)
        else:
            rra.rrs_linear_signed(s["X"], G, perm, dsign, s["wq"], s["Y"], s["ws"], stream)

    def fe_step(i):
        s = sets[i % nsets]
        xq, dx, S = s["views"]
        if dsign is None:
            rra.rrs_frontend(s["X"], G, perm, xq, dx, S, s["ws"], 0, stream)
        else:
            rra.rrs_frontend_signed(s["X"], G, perm, dsign, xq, dx, S, s["ws"], 0, stream)

    def gemm_step(i):
        s = sets[i % nsets]
        xq, dx, S = s["views"]
        rra.rrs_gemm(xq, dx, S, G, s["wq"], s["Y"], stream)

    clock_log = {}

    def timed(fn, steps, warmup, tag=None):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(steps):
            fn(i)
        ev1.record(stream)
        if tag is not None:
            # the host has queued the loop; while the GPU still runs it, read
            # the clock levels (and note whether the work was still in flight)
            clk = sample_clocks()
            clock_log[tag] = {"levels": clk, "gpu_busy_at_sample": not ev1.query()}
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return ev0.elapsed_time(ev1) / steps, wall

    def settle(fn, seconds):
        """Untimed steps for `seconds` of wall time (the clock-settle phase)."""
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                fn(n)
                n += 1
            torch.cuda.synchronize()
        return {"seconds": round(time.perf_counter() - t0, 3), "steps": n}

    if args.profile_gemm_only:
        for i in range(nsets):   # codes and scales in every set's workspace first
            step(i)
        ms, _ = timed(gemm_step, args.steps, args.warmup)
        print(json.dumps({"gemm_ms": ms}))
        return

    settled = settle(step, args.settle_s)
    # whole layer: the metric
    ms_step, wall = timed(step, args.steps, args.warmup, tag="layer")
    # each part alone, same kernels, on the same stream
    ms_fe, _ = timed(fe_step, args.steps, args.warmup)
    ms_gemm, _ = timed(gemm_step, args.steps, args.warmup)

    fe_launches = rra.rrs_frontend_passes(M, K, 0)
    fe_src = "rrs_frontend.hip" if (K & (K - 1)) == 0 else "rrs_frontend_kron.hip"
    ops = 2.0 * M * N * K
    tops = ops / (ms_step * 1e-3) / 1e12
    gemm_tops = ops / (ms_gemm * 1e-3) / 1e12
    fe_bytes = 2 * M * K + M * K // 2 + 4 * M + 4 * (K // G)
    fe_gbs = fe_bytes / (ms_fe * 1e-3) / 1e9
    gemm_bytes = M * K // 2 + K * N // 2 + 4 * (M + N) + 4 * (K // G) + 4 * M * N

    if rra.rrs_gemm_form(M, K, N, G) == rra.RRS_GEMM_FEW_TOKENS:
        # few tokens: the weights stream from HBM once; bytes bound the kernel
        gemm_gbs = gemm_bytes / (ms_gemm * 1e-3) / 1e9
        gemm_roofline = {
            "kernel": "gemm_small_kernel (few-token grouped int4 GEMM)",
            "bound": "hbm",
            "achieved": round(gemm_gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gemm_gbs / PEAK_HBM_GBS, 4),
            "traffic": (recorded_traffic("gemm_small", "rrs_gemm_small.hip", tkey) or {}).get("bytes"),
            "traffic_detail": recorded_traffic("gemm_small", "rrs_gemm_small.hip", tkey),
            "algorithmic_bytes": gemm_bytes,
            "ms_per_launch": round(ms_gemm, 5),
        }
    else:
        gemm_roofline = {
            "kernel": "gemm_kernel (tiled grouped int4 GEMM)",
            "bound": "mfma",
            "achieved": round(gemm_tops, 3),
            "peak": PEAK_MFMA_TOPS,
            "unit": "TFLOP/s",
            "op_kind": "2MNK ops of int4 codes on fp8 e4m3 MFMA (exact), against the dense fp8 peak 5.0 PFLOP/s",
            "frac": round(gemm_tops / PEAK_MFMA_TOPS, 4),
            "traffic": (recorded_traffic("gemm", "rrs_gemm.hip", tkey) or {}).get("bytes"),
            "traffic_detail": recorded_traffic("gemm", "rrs_gemm.hip", tkey),
            "algorithmic_bytes": gemm_bytes,
            "ms_per_launch": round(ms_gemm, 5),
        }

    out = {
        "metric": "rrs_linear effective int TOPS + front-end GB/s at M=2048,K=N=4096,G=128",
        "value": round(tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded outlier recipe; stands in for WikiText-2 / QA activations)",
        "config": {"workload": wl.name, "M": M, "K": K, "N": N, "G": G, "input_sets": nsets,
                   "rotation": "signed X D H" if dsign is not None else "X H"},
        "frontend_gbs": round(fe_gbs, 2),
        "gemm_tops": round(gemm_tops, 3),
        "roofline": gemm_roofline,
        "roofline_frontend": {
            "kernel": (("rowsplit_kernel (one row per workgroup: rotate, reorder, group max, grid-wide wait, "
                        "quantise, pack)" if M <= 256 and K in (1024, 2048, 4096, 8192) else
                        "fused_kernel (rotate, reorder, group max, grid-wide wait, quantise, pack)")
                       if fe_launches == 1 else
                       "stats pass, group-max reduce, quantise pass" if (K & (K - 1)) == 0 else
                       "stats pass (keeps the rotated rows), group-max reduce, quantise pass over the stored rows"),
            "launches": fe_launches,
            "bound": "hbm",
            "achieved": round(fe_gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(fe_gbs / PEAK_HBM_GBS, 4),
            "traffic": (recorded_traffic("frontend", fe_src, tkey) or {}).get("bytes"),
            "traffic_detail": recorded_traffic("frontend", fe_src, tkey),
            "algorithmic_bytes": fe_bytes,
            "ms_per_call": round(ms_fe, 5),
        },
        "wall_s_timed_region": round(wall, 4),
        "clock_settle": settled,
    }

    out["device"] = device_info(torch)
    out["device"]["clocks_during_timed_loop"] = clock_log.get("layer")
    if args.ablation:
        out["ablation"] = ablation(args, wl, x, w, xc, timed, dev)
    if not args.no_cpu_baseline:
        s0 = sets[0]
        rra.rrs_linear(s0["X"], G, perm, s0["wq"], s0["Y"], s0["ws"], stream) if dsign is None else \
            rra.rrs_linear_signed(s0["X"], G, perm, dsign, s0["wq"], s0["Y"], s0["ws"], stream)
        torch.cuda.synchronize()
        xq, dx, S = rra.workspace_views(s0["ws"], M, K, G)  # row-major copy of the codes
        codes, dw = rra.weight_views(s0["wq"], K, N)
        gpu = {"perm": perm.cpu().numpy(), "xq": xq.cpu().numpy(), "dx": dx.cpu().numpy(), "S": S.cpu().numpy(),
               "codes": codes.cpu().numpy(), "dw": dw.cpu().numpy(), "Y": s0["Y"].cpu().numpy(),
               "dsign": None if dsign is None else dsign.cpu().numpy().view(np.uint32)}
        out["cpu_baseline"] = cpu_baseline(x, w, G, gpu)

    print(json.dumps(out), flush=True)


def device_info(torch):
    """The device; its clock levels are sampled while the timed loop runs
    (clocks_during_timed_loop) and, for reference, after all loops
    (clocks_after, usually the idle level)."""
    props = torch.cuda.get_device_properties(0)
    return {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
            "clocks_after": sample_clocks()}


def ablation(args, wl, x, w, xc, timed, dev):
    """The component switches on the same kernels (RRS rebuttal page,
    "Incomplete ablation study"): per group size of the workload, the full
    method, Runtime Smooth alone (no rotation on either side) and the
    rotation alone (S = 1, the per-channel A4W4 baseline), each timed as a
    whole layer (rrs_linear_ex), with the oracle's relative output error
    against the float64 product X W when the CPU leg is on."""
    import numpy as np
    import torch
    import rotated_runtime_activation_amd as rra
    M, K, N = wl.M, wl.K, wl.N
    variants = [("rrs", 0), ("rs_only", rra.RRS_FLAG_NO_ROTATE), ("rotation_only", rra.RRS_FLAG_NO_SMOOTH)]
    Gs = (args.G,) if args.G else tuple(wl.G)
    X0 = torch.from_numpy(x).to(dev)
    W0 = torch.from_numpy(w).to(dev)
    XC = torch.from_numpy(xc).to(dev)
    stream = torch.cuda.current_stream()
    ref = None
    if not args.no_cpu_baseline:
        ref = x.astype(np.float64) @ w.astype(np.float64)
    rows = []
    for G in Gs:
        for name, flags in variants:
            nr = flags & rra.RRS_FLAG_NO_ROTATE
            perm = torch.empty(K, dtype=torch.int32, device=dev)
            cws = torch.empty(rra.rrs_calibrate_workspace_bytes(K), dtype=torch.uint8, device=dev)
            rra.rrs_calibrate_perm_ex(XC, None, nr, perm, cws)
            wq = torch.empty(rra.rrs_weight_bytes(K, N), dtype=torch.uint8, device=dev)
            rra.rrs_prepare_weights_ex(W0, perm, None, nr, wq)
            ws_bytes = rra.rrs_workspace_bytes(M, K, G)
            set_bytes = X0.numel() * 2 + wq.numel() + M * N * 4 + ws_bytes
            nsets = min(64, max(3, -(-2 * MALL_BYTES // set_bytes)))
            sets = []
            for _ in range(nsets):
                ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
                rra.rrs_workspace_init(ws)
                sets.append((X0.clone(), wq.clone(), torch.empty(M, N, dtype=torch.float32, device=dev), ws))

            def step(i, sets=sets, G=G, flags=flags, perm=perm):
                X, wq_i, Y, ws = sets[i % len(sets)]
                rra.rrs_linear_ex(X, G, perm, None, flags, wq_i, Y, ws, stream)

            ms, _ = timed(step, args.steps, args.warmup)
            row = {"variant": name, "G": G, "flags": flags, "ms_per_step": round(ms, 5),
                   "tops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 3),
                   "frontend_launches": rra.rrs_frontend_passes(M, K, flags)}
            if ref is not None:
                import oracle
                p_np = perm.cpu().numpy()
                y = oracle.rrs_linear(x, w, p_np, G, rotate=not nr, smooth=not (flags & rra.RRS_FLAG_NO_SMOOTH))["Y"]
                row["oracle_rel_fro_error"] = round(float(np.linalg.norm(y - ref) / np.linalg.norm(ref)), 6)
            rows.append(row)
            del sets
            torch.cuda.empty_cache()
    return rows


def cpu_baseline(x, w, G, gpu, budget_s=10.0):
    """The CPU oracle as it stands, on the host cores: full layer steps
    (front end of all tokens + the grouped GEMM output), weights prepared
    beforehand as on the GPU side, with the GPU's calibration order, repeated
    until about ``budget_s`` seconds of CPU work. Reported for context only.

    It also checks the GPU's outputs of the timed run against this oracle:
    every activation and weight code (exempt within 1e-5 of a .5 boundary,
    reported), and Y on sampled rows, both ways: against the oracle GEMM fed
    the GPU's own codes and scales, and, on outputs whose row and column
    carry no code flip, against the oracle's end-to-end result."""
    import numpy as np
    import oracle
    perm = gpu["perm"]
    d = None if gpu["dsign"] is None else oracle.signs_from_bits(gpu["dsign"], x.shape[1])
    wp = oracle.prepare_weights(w, perm, d)
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    reps = 0
    t0 = time.perf_counter()
    while True:
        fe = oracle.frontend(x, perm, G, d=d)
        y = oracle.linear_out(fe["q"], fe["dx"], fe["S"], wp["qw"], wp["dw"], G)["Y"]
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / reps
    M, K = x.shape
    N = w.shape[1]
    # the method's own quantisation error on this workload (outside the timing)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    qerr = float(np.linalg.norm(y - ref) / np.linalg.norm(ref))
    return {
        "value": round(2.0 * M * N * K / dt / 1e12, 6),
        "unit": "TOPS",
        "cores": len(os.sched_getaffinity(0)),
        "blas_threads": blas,
        "kind": "oracle",
        "sample": (f"{reps} full steps of the same workload (M={M}, K={K}, N={N}, G={G}) in float64 "
                   f"NumPy, {dt:.2f} s each; front end single-threaded, group GEMMs on {blas} BLAS threads "
                   f"({len(os.sched_getaffinity(0))} cores available)"),
        "quant_error": {"rel_fro": round(qerr, 6),
                        "of": "the oracle's Y against the float64 product X W of the same fp16 inputs"},
        "parity": parity_of_timed_run(fe, wp, gpu, G),
    }


def parity_of_timed_run(fe, wp, gpu, G, rows_sampled=64):
    """Counts of the GPU's timed-run outputs against the oracle (see
    cpu_baseline). The Y bound is the fp32 rounding bound of the GEMM chain,
    gamma_n C with n = K/64 (K/32 at G = 32) + 2 K/G + 8, u = 2^-24, widened
    for the flip-free check by the GPU scales' relative deviation."""
    import numpy as np
    import oracle
    M, K = fe["q"].shape
    q = oracle.unpack_codes(gpu["xq"])
    qw = oracle.unpack_codes(gpu["codes"])
    out = {}
    for what, got, want, v in (("activation_codes", q, fe["q"], fe["v"]), ("weight_codes", qw, wp["qw"], wp["uw"])):
        diff = got.astype(np.int16) != want.astype(np.int16)
        ex = oracle.near_half(v, 1e-5)
        out[what] = {"codes": int(want.size), "exempt": int(ex.sum()), "exempt_differ": int((diff & ex).sum()),
                     "nonexempt_differ": int((diff & ~ex).sum())}
    n = K // (32 if G == 32 else 64) + 2 * (K // G) + 8
    tol = n * 2.0 ** -24 / (1 - n * 2.0 ** -24)
    rows = np.linspace(0, M - 1, min(rows_sampled, M)).astype(np.int64)
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    own = oracle.linear_out(q[rows], f64(gpu["dx"][rows]), f64(gpu["S"]), qw, f64(gpu["dw"]), G)
    Yg = f64(gpu["Y"][rows])
    C = np.where(own["C"] > 0, own["C"], 1.0)
    e_own = float((np.abs(Yg - own["Y"]) / C).max())
    ref = oracle.linear_out(fe["q"][rows], fe["dx"][rows], fe["S"], wp["qw"], wp["dw"], G)
    rel = lambda g, r: np.abs(f64(g) - f64(r)) / np.where(f64(r) != 0, np.abs(f64(r)), 1.0)
    dev = (1 + rel(gpu["dx"][rows], fe["dx"][rows])[:, None]) * (1 + rel(gpu["dw"], wp["dw"])[None, :]) * \
        (1 + float(rel(gpu["S"], fe["S"]).max())) - 1
    clean = (~(q[rows] != fe["q"][rows]).any(axis=1))[:, None] & (~(qw != wp["qw"]).any(axis=1))[None, :]
    Cr = np.where(ref["C"] > 0, ref["C"], 1.0)
    e_ref = np.abs(Yg - ref["Y"]) / Cr
    out["Y"] = {"rows_sampled": int(rows.size), "tol_over_C": tol,
                "max_err_over_C_vs_oracle_gemm_of_gpu_codes": e_own,
                "flip_free_outputs": int(clean.sum()),
                "max_err_over_C_flip_free_vs_oracle": float(e_ref[clean].max(initial=0.0)),
                "ok": bool(e_own <= tol and np.all(e_ref[clean] <= (tol + dev[clean]) * (1 + 1e-6)))}
    out["ok"] = bool(out["Y"]["ok"] and out["activation_codes"]["nonexempt_differ"] == 0
                     and out["weight_codes"]["nonexempt_differ"] == 0)
    return out


if __name__ == "__main__":
    main()
