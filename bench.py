"""Benchmark of the affine-Q4 GEMV hot path on one MI355X.

One step = q4mv_prepare_x (activation prep) + q4mv (the GEMV) over one batch of synthetic
inputs already resident in HBM. Weights rotate over R copies whose total exceeds twice the
256 MB Infinity Cache, so every launch streams its weights from HBM.

Prints ONE JSON line (rank 0). `value` is weight GB/s of the whole step (weight bytes of the
matrix / step time). `roofline` is the GEMV kernel alone: algorithmic bytes (weights +
activations read + outputs written) per launch / its average duration, timed with HIP events
around each launch inside the timed region. `cpu_baseline` is the CPU oracle timed on the host
cores on the same workload. `sweep` repeats the kernel timing at the other activation batch
sizes of the metric (NB = 1/4/8, and 16 for the LM head) and on the MLP up projection.
"""
import argparse
import hashlib
import glob
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 600e6  # > 2 x (256 MB Infinity Cache + L2)
METRIC = "affine-Q4 GEMV weight GB/s and % of HBM peak at NB=1/4/8; rows/s"


def kernel_source_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "affine_q4_gemv_amd", "csrc", "*"))):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload, nb):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "q4mv_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = d.get("runs", {}).get(f"{workload}_nb{nb}")
    return None if ent is None else ent.get("hbm_bytes_per_launch")


class Problem:
    """Device buffers of one workload: R rotated weight copies, activations and outputs."""

    def __init__(self, name, nb, rotate=True):
        import numpy as np
        import torch

        import affine_q4_gemv_amd as q4
        import workloads

        self.q4, self.torch = q4, torch
        self.case = workloads.make_case(name, nb=nb)
        c = self.case
        self.n_mat, self.out_dim, self.in_dim, self.nb = c["n_mat"], c["out_dim"], c["in_dim"], nb
        self.weight_bytes = workloads.weight_bytes(self.n_mat, self.out_dim, self.in_dim)
        dev = torch.device("cuda:0")
        codes = torch.from_numpy(c["codes"]).to(dev)
        w0 = q4.q4mv_pack_codes(codes)
        del codes

        def bf16(bits):
            return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

        s0, b0 = bf16(c["scales"]), bf16(c["biases"])
        self.R = max(1, math.ceil(ROTATE_BYTES / self.weight_bytes)) if rotate else 1
        self.w = [w0] + [w0.clone() for _ in range(self.R - 1)]
        self.s = [s0] + [s0.clone() for _ in range(self.R - 1)]
        self.b = [b0] + [b0.clone() for _ in range(self.R - 1)]
        self.x = torch.from_numpy(c["x"].reshape(self.n_mat * nb, self.in_dim)).to(dev)
        self.xe, self.xo, self.xsum = q4.q4mv_prepare_x(self.x)
        self.y = torch.empty((self.n_mat, nb, self.out_dim), dtype=torch.float32, device=dev)
        # algorithmic bytes of one GEMV launch: weights + staged activations read + outputs
        rows = self.n_mat * nb
        self.act_bytes = rows * (self.in_dim * 2 + self.in_dim // 32 * 4)
        self.out_bytes = rows * self.out_dim * 4
        self.algo_bytes = self.weight_bytes + self.act_bytes + self.out_bytes
        torch.cuda.synchronize()

    def prep(self):
        self.q4.q4mv_prepare_x(self.x, self.xe, self.xo, self.xsum)

    def gemv(self, i):
        k = i % self.R
        self.q4.q4mv(self.w[k], self.s[k], self.b[k], self.xe, self.xo, self.xsum, self.nb,
                     y=self.y)

    def time_steps(self, steps, warmup):
        """(ms per full step, avg GEMV kernel ms) with HIP events on the launch stream."""
        torch = self.torch
        for i in range(warmup):
            self.prep()
            self.gemv(i)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for i in range(steps):
            self.prep()
            ev[i][0].record()
            self.gemv(i)
            ev[i][1].record()
        t1.record()
        torch.cuda.synchronize()
        step_ms = t0.elapsed_time(t1) / steps
        kern_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
        return step_ms, kern_ms

    def time_kernel(self, launches, warmup=20):
        """Average GEMV kernel ms over back-to-back launches (activations already prepped)."""
        torch = self.torch
        for i in range(warmup):
            self.gemv(i)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for i in range(launches):
            self.gemv(i)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / launches


def cpu_baseline(name, nb, reps=3):
    import oracle
    import workloads
    c = workloads.make_case(name, nb=nb)
    wbytes = workloads.weight_bytes(c["n_mat"], c["out_dim"], c["in_dim"])
    threads = oracle.default_threads()
    times = []
    for _ in range(reps):
        t = time.perf_counter()
        oracle.gemv(c["codes"], c["scales"], c["biases"], c["x"], nthreads=threads)
        times.append(time.perf_counter() - t)
        if times[-1] > 10.0:
            break
    t = sorted(times)[len(times) // 2]
    return {"value": round(wbytes / t / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"full workload ({c['n_mat']}x{c['out_dim']}x{c['in_dim']}, NB={nb}), "
                      f"double-precision C oracle with {threads} threads, median of "
                      f"{len(times)} runs of {t:.3f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="lm_head")
    ap.add_argument("--nb", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-sweep", action="store_true", help="skip the NB / shape sweep")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (the GEMV shards by output rows "
              "with no cross-GPU step in the kernel); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    prob = Problem(args.workload, args.nb)
    step_ms, kern_ms = prob.time_steps(args.steps, args.warmup)
    value = prob.weight_bytes / (step_ms * 1e-3) / 1e9
    achieved = prob.algo_bytes / (kern_ms * 1e-3) / 1e9
    traffic = load_traffic(args.workload, args.nb)
    import affine_q4_gemv_amd as q4
    path = q4.q4mv_auto_path(prob.in_dim, prob.nb, False)
    kernel_name = {1: "valu_kernel", 2: "valu_kernel", 3: "mfma_kernel"}.get(path, "?")

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload} {prob.n_mat}x{prob.out_dim}x{prob.in_dim} "
                               f"affine-Q4 group 64, NB={prob.nb}",
                   "n_mat": prob.n_mat, "out_dim": prob.out_dim, "in_dim": prob.in_dim,
                   "nb": prob.nb, "group": 64, "weight_bytes": prob.weight_bytes,
                   "rotation_copies": prob.R, "seed": 0,
                   "operands": "u4 codes, bf16 scale+bias per 64, f16 activations, f32 acc"},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "rows_per_s": round(prob.n_mat * prob.out_dim / (step_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": kernel_name,
                     "kernel_us": round(kern_ms * 1e3, 3),
                     "algorithmic_bytes_per_launch": prob.algo_bytes},
    }
    del prob
    torch.cuda.empty_cache()

    if not args.no_sweep:
        sweep = []
        runs = [("lm_head", nb) for nb in (1, 4, 8, 16)] + [("up", nb) for nb in (1, 4, 8)] + \
               [("moe_down", 4), ("dense", 1)]
        for name, nb in runs:
            p = Problem(name, nb)
            ms = p.time_kernel(200)
            sweep.append({"workload": name, "nb": nb, "kernel_us": round(ms * 1e3, 3),
                          "weight_GBps": round(p.weight_bytes / (ms * 1e-3) / 1e9, 1),
                          "pct_hbm_peak": round(100 * p.weight_bytes / (ms * 1e-3) / 1e9 /
                                                HBM_PEAK_GBPS, 1),
                          "rows_per_s": round(p.n_mat * p.out_dim / (ms * 1e-3), 1),
                          "path": q4.q4mv_auto_path(p.in_dim, nb, False)})
            del p
            torch.cuda.empty_cache()
        result["sweep"] = sweep

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args.workload, args.nb)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
