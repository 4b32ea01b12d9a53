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
and the CPU oracle timed on the host as a reported baseline.

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
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps first: the shader clock needs tens of milliseconds of load to settle")
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
        import numpy as np
        bits = np.random.default_rng(1234).integers(0, 2**32, size=K // 32, dtype=np.uint64).astype(np.uint32)
        dsign = torch.from_numpy(bits.view(np.int32)).to(dev)
        rra.rrs_calibrate_perm_signed(torch.from_numpy(xc).to(dev), dsign, perm, cws)
        rra.rrs_prepare_weights_signed(W0, perm, dsign, wq0)
    else:
        rra.rrs_prepare_weights(W0, perm, wq0)
    del W0

    ws_bytes = rra.rrs_workspace_bytes(M, K, G)
    set_bytes = X0.numel() * 2 + wq0.numel() + M * N * 4 + ws_bytes
    nsets = max(3, -(-2 * MALL_BYTES // set_bytes))
    sets = []
    for _ in range(nsets):
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        rra.rrs_workspace_init(ws)
        sets.append(dict(X=X0.clone(), wq=wq0.clone(), Y=torch.empty(M, N, dtype=torch.float32, device=dev),
                         ws=ws, views=rra.workspace_views(ws, M, K, G)))
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

    def timed(fn, steps, warmup):
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
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return ev0.elapsed_time(ev1) / steps, wall

    if args.profile_gemm_only:
        ms, _ = timed(gemm_step, args.steps, args.warmup)
        print(json.dumps({"gemm_ms": ms}))
        return

    # whole layer: the metric
    ms_step, wall = timed(step, args.steps, args.warmup)
    # each part alone, same kernels, on the same stream
    ms_fe, _ = timed(fe_step, args.steps, args.warmup)
    ms_gemm, _ = timed(gemm_step, args.steps, args.warmup)

    fe_launches = rra.rrs_frontend_passes(M, K, 0)
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
            "traffic": (recorded_traffic("gemm_small", "rrs_gemm_small.hip", wl.name) or {}).get("bytes"),
            "traffic_detail": recorded_traffic("gemm_small", "rrs_gemm_small.hip", wl.name),
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
            "traffic": (recorded_traffic("gemm", "rrs_gemm.hip", wl.name) or {}).get("bytes"),
            "traffic_detail": recorded_traffic("gemm", "rrs_gemm.hip", wl.name),
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
            "traffic": (recorded_traffic("frontend", "rrs_frontend.hip", wl.name) or {}).get("bytes"),
            "traffic_detail": recorded_traffic("frontend", "rrs_frontend.hip", wl.name),
            "algorithmic_bytes": fe_bytes,
            "ms_per_call": round(ms_fe, 5),
        },
        "wall_s_timed_region": round(wall, 4),
    }

    out["device"] = device_info(torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, w, xc, G)

    print(json.dumps(out), flush=True)


def device_info(torch):
    """The device and the clock levels the driver reports right after the
    timed loops (the shader clock ramps under load; the level marked with *
    is the one in use). Read from the driver's sysfs tables: no program is
    started from this GPU process."""
    import glob
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
            "clocks": None}
    try:
        clocks = {}
        for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_[sm]clk")):
            cur = [l.strip() for l in open(path) if "*" in l]
            if cur:
                clocks[path.split("/")[-3] + ":" + path.rsplit("_", 1)[-1]] = cur[0]
        info["clocks"] = clocks or None
    except Exception:
        pass
    return info


def cpu_baseline(x, w, xc, G, budget_s=10.0):
    """The CPU oracle as it stands, on the host cores: full layer steps
    (front end of all tokens + the grouped GEMM output), weights prepared
    beforehand as on the GPU side, repeated until about ``budget_s`` seconds
    of CPU work. Reported for context only."""
    import oracle
    perm = oracle.calibrate_perm(xc)
    wp = oracle.prepare_weights(w, perm)
    try:
        from threadpoolctl import threadpool_info
        blas = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    reps = 0
    t0 = time.perf_counter()
    while True:
        fe = oracle.frontend(x, perm, G)
        y = oracle.linear_out(fe["q"], fe["dx"], fe["S"], wp["qw"], wp["dw"], G)["Y"]
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / reps
    M, K = x.shape
    N = w.shape[1]
    # the method's own quantisation error on this workload (outside the timing)
    import numpy as np
    ref = x.astype(np.float64) @ w.astype(np.float64)
    qerr = float(np.linalg.norm(y - ref) / np.linalg.norm(ref))
    return {
        "value": round(2.0 * M * N * K / dt / 1e12, 6),
        "unit": "TOPS",
        "cores": blas,
        "kind": "oracle",
        "sample": (f"{reps} full steps of the same workload (M={M}, K={K}, N={N}, G={G}) in float64 "
                   f"NumPy, {dt:.2f} s each; front end single-threaded, group GEMMs on {blas} BLAS threads"),
        "quant_error": {"rel_fro": round(qerr, 6),
                        "of": "the oracle's Y against the float64 product X W of the same fp16 inputs"},
    }


if __name__ == "__main__":
    main()
