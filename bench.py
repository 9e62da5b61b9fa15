"""Benchmark of the affine-Q4 GEMV hot path on one MI355X.

One step = q4mv_fused over one batch of synthetic inputs already resident in HBM: the GEMV
with the activation prep (f16 rounding, per-chunk sums) done inside its own staging, one
launch, bitwise what q4mv_prepare_x followed by q4mv gives (checked in the run); the
two-launch step is reported next to it in the sweep. Weights rotate over R copies whose total exceeds twice the
256 MB Infinity Cache, so every launch streams its weights from HBM. Timed loops are captured
in a HIP graph (replayed after a warm-up replay), so host launch cost is not measured; a
replay's output is checked bit for bit against an eager call.

Prints ONE JSON line. `value` is weight GB/s of the whole step (weight bytes / step time).
`roofline` is the GEMV kernel alone: algorithmic bytes (weights + activations read + outputs
written) per launch / its average duration, timed with HIP events around a graph of
back-to-back GEMV launches on the launch stream. `cpu_baseline` is the CPU oracle on the host
cores on the same workload. `sweep` repeats the kernel timing at the other batch sizes of the
metric (NB = 1/4/8, 16 for the LM head) and on the other projection shapes.

Profiling helpers (commands recorded in profiles/):
  --eager               time plain launches (for rocprofv3 runs)
  --pmc-probe           a plain 256 MiB streaming kernel (negation), then 10 GEMV launches:
                        the counters of the first calibrate those of the second
  --summarize-trace D   kernel statistics of a rocprofv3 --kernel-trace run directory
  --summarize-pmc F W   HBM traffic per GEMV launch from FETCH_SIZE / WRITE_SIZE run dirs
"""
import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 600e6  # > 2 x (256 MB Infinity Cache + L2)
CALIB_BYTES = 256 << 20
MAX_COPIES = 200  # launches per timed graph
METRIC = "affine-Q4 GEMV weight GB/s and % of HBM peak at NB=1/4/8; rows/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "q4mv_traffic.json")


KERNEL_SOURCES = {"valu_kernel": ["q4mv_valu.hip"], "mfma_kernel": ["q4mv_mfma.hip"]}


def kernel_source_hash(kernel):
    """Hash of the sources that define a kernel and its launch shape."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ["q4mv_device.h", "q4mv_internal.h"]:
        h.update(open(os.path.join(ROOT, "affine_q4_gemv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload, nb, kernel):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current sources of that kernel (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        ent = json.load(open(TRAFFIC_FILE)).get(f"{workload}_nb{nb}")
    except ValueError:
        return None
    if not ent or ent.get("kernel") != kernel or ent.get("source_hash") != kernel_source_hash(kernel):
        return None
    return ent.get("hbm_bytes_per_launch")


class Problem:
    """Device buffers of one workload: R rotated weight copies, activations and outputs."""

    def __init__(self, name, nb, rotate=True, silu_div=None, bits=4, fused=False):
        import numpy as np
        import torch

        import affine_q4_gemv_amd as q4
        import workloads

        self.q4, self.torch = q4, torch
        self.silu_div = silu_div
        self.bits = bits
        self.fused = fused and bits == 4 and silu_div is None
        c = workloads.make_case(name, nb=nb)
        self.name = name
        self.n_mat, self.out_dim, self.in_dim, self.nb = c["n_mat"], c["out_dim"], c["in_dim"], nb
        self.weight_bytes = workloads.weight_bytes(self.n_mat, self.out_dim, self.in_dim)
        if bits != 4:  # code bytes scale with the width; scales and biases do not
            self.weight_bytes = self.n_mat * self.out_dim * (
                self.in_dim // 32 * 4 * bits + self.in_dim // 64 * 4)
        dev = torch.device("cuda:0")
        codes = torch.from_numpy(c["codes"]).to(dev)
        w0 = q4.q4mv_pack_codes(codes) if bits == 4 else q4.q4mv_pack_lowbit(bits, codes)
        del codes

        def bf16(bits):
            return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

        s0, b0 = bf16(c["scales"]), bf16(c["biases"])
        # copies past MAX_COPIES are never read by a graph of that many launches
        self.R = min(MAX_COPIES, max(1, math.ceil(ROTATE_BYTES / self.weight_bytes))) \
            if rotate else 1
        self.w = [w0] + [w0.clone() for _ in range(self.R - 1)]
        self.s = [s0] + [s0.clone() for _ in range(self.R - 1)]
        self.b = [b0] + [b0.clone() for _ in range(self.R - 1)]
        self.x = torch.from_numpy(c["x"].reshape(self.n_mat * nb, self.in_dim)).to(dev)
        self.xe, self.xo, self.xsum = q4.q4mv_prepare_x(self.x)
        self.y = torch.empty((self.n_mat, nb, self.out_dim), dtype=torch.float32, device=dev)
        rows = self.n_mat * nb
        self.algo_bytes = self.algorithmic_bytes(name, nb, self.fused)
        self.path = q4.q4mv_auto_path(self.in_dim, nb, False, self.out_dim)
        self.kernel = "mfma_kernel" if self.path == q4.PATH_MFMA else "valu_kernel"
        del c
        torch.cuda.synchronize()

    @staticmethod
    def algorithmic_bytes(name, nb, fused=False):
        """Weights + activations read (f32 x for the fused launch, else the prepared f16
        streams and chunk sums) + outputs written by one GEMV launch."""
        import workloads
        w = workloads.WORKLOADS[name]
        n_mat, out_dim, in_dim = w["n_mat"], w["out_dim"], w["in_dim"]
        rows = n_mat * nb
        xbytes = in_dim * 4 if fused else in_dim * 2 + in_dim // 32 * 4
        return workloads.weight_bytes(n_mat, out_dim, in_dim) + rows * xbytes + rows * out_dim * 4

    def prep(self):
        if not self.fused:  # the fused launch does the prep itself
            self.q4.q4mv_prepare_x(self.x, self.xe, self.xo, self.xsum)

    def gemv(self, i):
        k = i % self.R
        if self.fused:
            self.q4.q4mv_fused(self.w[k], self.s[k], self.b[k], self.x, self.nb, y=self.y)
        elif self.bits != 4:
            self.q4.q4mv_lowbit(self.bits, self.w[k], self.s[k], self.b[k], self.xe, self.xo,
                                self.xsum, self.nb, y=self.y)
        elif self.silu_div is not None:
            self.q4.q4mv_silu(self.w[k], self.s[k], self.b[k], self.xe, self.xo, self.xsum,
                              self.nb, self.silu_div, y=self.y)
        else:
            self.q4.q4mv(self.w[k], self.s[k], self.b[k], self.xe, self.xo, self.xsum, self.nb,
                         y=self.y)

    def _graph(self, body, n):
        """Capture n iterations of body(i) in a HIP graph (after two eager warm-ups)."""
        return _capture(self.torch, body, n)

    def time_path(self, path, launches=200):
        """Average ms of a fused launch (prep inside) on a forced kernel path."""
        q4 = self.q4

        def body(i):
            k = i % self.R
            q4.q4mv_fused(self.w[k], self.s[k], self.b[k], self.x, self.nb, path=path, y=self.y)
        return self._time_graph(self._graph(body, launches), launches, reps=5)

    def _time_graph(self, g, n, warmup_replays=1, reps=3, warm=None):
        """Median ms per iteration over reps timed replays of g (n iterations each); the
        per-replay figures are kept in self.trials. Each timed replay follows an untimed
        replay of `warm` (default g) with nothing in between, so the GPU is busy when the
        first timed launch starts; the events bracket exactly the n timed iterations."""
        return time_graph(self.torch, g, n, warmup_replays, reps, warm, self)

    def check_graph_output(self):
        """The graph's result equals an eager call bit for bit (weights copies are equal);
        a fused step's also equals q4mv_prepare_x + q4mv."""
        torch = self.torch
        got = self.y.clone()
        self.prep()
        self.gemv(0)
        torch.cuda.synchronize()
        if not torch.equal(got, self.y):
            raise RuntimeError("graph replay output differs from the eager call")
        if self.fused:
            xe, xo, xsum = self.q4.q4mv_prepare_x(self.x)
            two = self.q4.q4mv(self.w[0], self.s[0], self.b[0], xe, xo, xsum, self.nb)
            torch.cuda.synchronize()
            if not torch.equal(got, two):
                raise RuntimeError("fused step differs from q4mv_prepare_x + q4mv")

    def time_steps(self, steps, warmup, reps=3):
        """ms per full step (prep + GEMV), graph-captured."""
        def step(i):
            self.prep()
            self.gemv(i)
        g = self._graph(step, steps)
        ms = self._time_graph(g, steps, warmup_replays=max(1, math.ceil(warmup / steps)),
                              reps=reps)
        self.check_graph_output()
        return ms

    def time_prep(self, launches=200):
        """Average q4mv_prepare_x ms over a graph of back-to-back launches."""
        q4 = self.q4
        g = self._graph(lambda i: q4.q4mv_prepare_x(self.x, self.xe, self.xo, self.xsum),
                        launches)
        return self._time_graph(g, launches)

    def time_kernel(self, launches=200):
        """Average GEMV kernel ms over a graph of back-to-back launches."""
        g = self._graph(self.gemv, launches)
        ms = self._time_graph(g, launches)
        self.check_graph_output()
        return ms

    def time_eager(self, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            self.prep()
            self.gemv(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(steps):
            self.prep()
            self.gemv(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps


class MoeChain(Problem):
    """The expert MLP of the MoE workload: 8 experts, hidden 2560, intermediate 640, NB=4.
    One step = stacked gate|up GEMV + fused SwiGLU prep + down GEMV (three launches)."""

    def __init__(self, n_mat=8, hidden=2560, inter=640, nb=4):
        import numpy as np
        import torch

        import affine_q4_gemv_amd as q4
        import workloads
        self.q4, self.torch = q4, torch
        self.silu_div = None
        dev = torch.device("cuda:0")
        up = workloads.make_shape(n_mat, 2 * inter, hidden, nb, seed=21)
        dn = workloads.make_shape(n_mat, hidden, inter, nb, seed=22, x_scale=0.5)

        def put(c):
            w = q4.q4mv_pack_codes(torch.from_numpy(c["codes"]).to(dev))
            s = torch.from_numpy(c["scales"].view(np.int16)).to(dev).view(torch.bfloat16)
            b = torch.from_numpy(c["biases"].view(np.int16)).to(dev).view(torch.bfloat16)
            return w, s, b
        self.weight_bytes = (workloads.weight_bytes(n_mat, 2 * inter, hidden)
                             + workloads.weight_bytes(n_mat, hidden, inter))
        self.R = max(1, math.ceil(ROTATE_BYTES / self.weight_bytes))
        w1, s1, b1 = put(up)
        w2, s2, b2 = put(dn)
        self.sets = [(w1, s1, b1, w2, s2, b2)] + [
            tuple(t.clone() for t in (w1, s1, b1, w2, s2, b2)) for _ in range(self.R - 1)]
        x = torch.from_numpy(up["x"].reshape(n_mat * nb, hidden)).to(dev)
        self.x = x
        self.fused = False
        self.ids = torch.arange(n_mat, dtype=torch.int32, device=dev)
        self.xe, self.xo, self.xsum = q4.q4mv_prepare_x(x)
        self.gu = torch.empty((n_mat, nb, 2 * inter), dtype=torch.float32, device=dev)
        self.xe2 = torch.empty((n_mat * nb, inter // 2), dtype=torch.float16, device=dev)
        self.xo2 = torch.empty_like(self.xe2)
        self.xsum2 = torch.empty((n_mat * nb, inter // 32), dtype=torch.float32, device=dev)
        self.y = torch.empty((n_mat, nb, hidden), dtype=torch.float32, device=dev)
        self.nb, self.n_mat, self.inter = nb, n_mat, inter
        torch.cuda.synchronize()

    def prep(self):
        pass

    def gemv(self, i):
        w1, s1, b1, w2, s2, b2 = self.sets[i % self.R]
        q4 = self.q4
        if self.fused:
            # gate|up with the prep inside, down with the SwiGLU inside (two launches)
            q4.q4mv_fused(w1, s1, b1, self.x, self.nb, y=self.gu)
            q4.q4mv_experts_fused(w2, s2, b2, self.ids, self.gu.view(-1, 2 * self.inter),
                                  self.nb, False, swiglu=True, y=self.y)
            return
        q4.q4mv(w1, s1, b1, self.xe, self.xo, self.xsum, self.nb, y=self.gu)
        q4.q4mv_swiglu_prep(self.gu.view(self.n_mat * self.nb, 2 * self.inter), self.xe2,
                            self.xo2, self.xsum2)
        q4.q4mv(w2, s2, b2, self.xe2, self.xo2, self.xsum2, self.nb, y=self.y)

    def check_graph_output(self):
        torch = self.torch
        got = self.y.clone()
        self.gemv(0)
        torch.cuda.synchronize()
        if not torch.equal(got, self.y):
            raise RuntimeError("graph replay output differs from the eager call")


class MoeLayer(MoeChain):
    """A decode MoE layer over routed experts: a bank of 32 experts (hidden 2560, intermediate
    640), 4 tokens with synthetic top-8 routing. One step = activation prep + gate|up over the
    routed experts (shared token rows) + SwiGLU prep + down per expert + combine (five
    launches); the weights read are those of the routed experts only."""

    def __init__(self, n_exp=32, hidden=2560, inter=640, nb=4, top_k=8):
        import numpy as np
        import torch

        import affine_q4_gemv_amd as q4
        import workloads
        self.q4, self.torch = q4, torch
        self.silu_div = None
        dev = torch.device("cuda:0")
        sel, wmap = workloads.make_routing(nb, n_exp, top_k, seed=71)
        self.n_u = n_u = sel.size
        gu = workloads.make_shape(n_exp, 2 * inter, hidden, nb, seed=72)
        dn = workloads.make_weights(n_exp, hidden, inter, seed=73)

        def put(codes, scales, biases):
            w = q4.q4mv_pack_codes(torch.from_numpy(codes).to(dev))
            s = torch.from_numpy(scales.view(np.int16)).to(dev).view(torch.bfloat16)
            b = torch.from_numpy(biases.view(np.int16)).to(dev).view(torch.bfloat16)
            return w, s, b
        bank_bytes = (workloads.weight_bytes(n_exp, 2 * inter, hidden)
                      + workloads.weight_bytes(n_exp, hidden, inter))
        self.weight_bytes = (workloads.weight_bytes(n_u, 2 * inter, hidden)
                             + workloads.weight_bytes(n_u, hidden, inter))
        self.R = max(1, math.ceil(ROTATE_BYTES / bank_bytes))
        w1, s1, b1 = put(gu["codes"], gu["scales"], gu["biases"])
        w2, s2, b2 = put(*dn)
        self.sets = [(w1, s1, b1, w2, s2, b2)] + [
            tuple(t.clone() for t in (w1, s1, b1, w2, s2, b2)) for _ in range(self.R - 1)]
        self.sel = torch.from_numpy(sel).to(dev)
        self.wmap = torch.from_numpy(wmap).to(dev)
        self.fused = False
        self.x = torch.from_numpy(np.ascontiguousarray(gu["x"][0])).to(dev)
        self.xe = torch.empty((nb, hidden // 2), dtype=torch.float16, device=dev)
        self.xo = torch.empty_like(self.xe)
        self.xsum = torch.empty((nb, hidden // 32), dtype=torch.float32, device=dev)
        self.gu = torch.empty((n_u, nb, 2 * inter), dtype=torch.float32, device=dev)
        self.xe2 = torch.empty((n_u * nb, inter // 2), dtype=torch.float16, device=dev)
        self.xo2 = torch.empty_like(self.xe2)
        self.xsum2 = torch.empty((n_u * nb, inter // 32), dtype=torch.float32, device=dev)
        self.yd = torch.empty((n_u, nb, hidden), dtype=torch.float32, device=dev)
        self.y = torch.empty((nb, hidden), dtype=torch.float32, device=dev)
        self.nb, self.inter = nb, inter
        torch.cuda.synchronize()

    def gemv(self, i):
        w1, s1, b1, w2, s2, b2 = self.sets[i % self.R]
        q4, nb = self.q4, self.nb
        if self.fused:
            # three launches: gate|up from the f32 token rows, down with the SwiGLU inside,
            # combine
            q4.q4mv_experts_fused(w1, s1, b1, self.sel, self.x, nb, True, y=self.gu)
            q4.q4mv_experts_fused(w2, s2, b2, self.sel, self.gu.view(self.n_u * nb, 2 * self.inter),
                                  nb, False, swiglu=True, y=self.yd)
            q4.q4mv_combine(self.yd, self.wmap, out=self.y)
            return
        q4.q4mv_prepare_x(self.x, self.xe, self.xo, self.xsum)
        q4.q4mv_experts(w1, s1, b1, self.sel, self.xe, self.xo, self.xsum, nb, True, y=self.gu)
        q4.q4mv_swiglu_prep(self.gu.view(self.n_u * nb, 2 * self.inter), self.xe2, self.xo2,
                            self.xsum2)
        q4.q4mv_experts(w2, s2, b2, self.sel, self.xe2, self.xo2, self.xsum2, nb, False,
                        y=self.yd)
        q4.q4mv_combine(self.yd, self.wmap, out=self.y)


WARM_S = 0.3  # untimed warm-up before the first timed trial, seconds of GPU work


def time_graph(torch, g, n, warmup_replays=1, reps=3, warm=None, keep=None):
    """Median ms per iteration over reps timed replays of the graph g (n iterations each),
    each right after an untimed replay of `warm` (default g); synchronised before and after
    every trial. Before the first trial, warm is replayed at least warmup_replays times and
    for at least WARM_S seconds: from idle the GPU needs a few hundred ms of work to reach
    its steady clocks (measured: LM head NB=1 trials of 20 steps at 36.8-40.5 us after one
    warm-up replay, 35.8-36.4 us after 0.3 s). The per-replay figures go to keep.trials when
    keep is given."""
    warm = warm or g
    t0 = time.perf_counter()
    done = 0
    while done < warmup_replays or time.perf_counter() - t0 < WARM_S:
        warm.replay()
        done += 1
        if done % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        warm.replay()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / n)
    if keep is not None:
        keep.trials = ts
    return statistics.median(ts)


def probe_lib():
    """libq4mv_probe.so (reference kernels for measurement), with argument types set."""
    import ctypes
    path = os.path.join(ROOT, "affine_q4_gemv_amd", "libq4mv_probe.so")
    L = ctypes.CDLL(path)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.q4mv_probe_read.argtypes = [p, i64, p, i32, p]
    L.q4mv_probe_read.restype = i32
    L.q4mv_probe_sink_words.argtypes = [i32]
    L.q4mv_probe_sink_words.restype = i64
    L.q4mv_probe_empty.argtypes = [i32, p]
    L.q4mv_probe_empty.restype = i32
    return L


def _capture(torch, body, n):
    """A HIP graph of n calls body(i) on a side stream (after two eager warm-up calls)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(2):
            body(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            body(i)
    return g


def reference_legs(launches=200):
    """The ceilings the GEMV figures are read against, timed like the GEMV (graphs of
    back-to-back launches): a streaming read of each workload's weight bytes over rotated
    copies at 1, 2, 4 and 8 blocks per CU, and the empty-kernel launch floor."""
    import torch
    L = probe_lib()
    import workloads
    out = []

    def stream():
        return torch.cuda.current_stream().cuda_stream

    for name in ("lm_head", "up", "moe_down", "dense", "tiny"):
        w = workloads.WORKLOADS[name]
        nbytes = workloads.weight_bytes(w["n_mat"], w["out_dim"], w["in_dim"])
        nbytes = (nbytes + 15) // 16 * 16
        # (a graph of `launches` launches reads at most that many copies)
        R = min(launches, max(1, math.ceil(ROTATE_BYTES / nbytes)))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(i % 251)
                for i in range(R)]
        res = {}
        for bpc in (1, 2, 4, 8):
            sink = torch.empty(L.q4mv_probe_sink_words(bpc), dtype=torch.int32, device="cuda")

            def body(i, bpc=bpc, sink=sink):
                st = L.q4mv_probe_read(bufs[i % R].data_ptr(), nbytes, sink.data_ptr(), bpc,
                                       stream())
                if st != 0:
                    raise RuntimeError(f"q4mv_probe_read: status {st}")
            g = _capture(torch, body, launches)
            res[bpc] = time_graph(torch, g, launches, reps=5) * 1e3
            del g, sink
        best = min(res, key=res.get)
        out.append({"leg": "streaming read (q4mv_probe_read)", "workload": name,
                    "bytes": nbytes, "rotation_copies": R,
                    "us_by_blocks_per_cu": {str(k): round(v, 3) for k, v in res.items()},
                    "best_us": round(res[best], 3), "best_blocks_per_cu": best,
                    "GBps": round(nbytes / (res[best] * 1e-6) / 1e9, 1),
                    "pct_hbm_peak": round(100 * nbytes / (res[best] * 1e-6) / 1e9
                                          / HBM_PEAK_GBPS, 1)})
        del bufs
        torch.cuda.empty_cache()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for blocks in (1, 2 * cus):
        def body(i, blocks=blocks):
            st = L.q4mv_probe_empty(blocks, stream())
            if st != 0:
                raise RuntimeError(f"q4mv_probe_empty: status {st}")
        g = _capture(torch, body, launches)
        us = time_graph(torch, g, launches, reps=5) * 1e3
        out.append({"leg": "empty kernel (q4mv_probe_empty)", "blocks": blocks,
                    "us_per_launch": round(us, 3)})
    return out


def cpu_baseline(name, nb, budget_s=10.0):
    """The CPU oracle on the full workload, repeated for about budget_s seconds (at least
    three passes); the median pass time gives the rate."""
    import oracle
    import workloads
    c = workloads.make_case(name, nb=nb)
    wbytes = workloads.weight_bytes(c["n_mat"], c["out_dim"], c["in_dim"])
    threads = oracle.default_threads()
    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_start < budget_s and len(times) < 1000):
        t = time.perf_counter()
        oracle.gemv(c["codes"], c["scales"], c["biases"], c["x"], nthreads=threads)
        times.append(time.perf_counter() - t)
    t = statistics.median(times)
    return {"value": round(wbytes / t / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"full workload ({c['n_mat']}x{c['out_dim']}x{c['in_dim']}, NB={nb}), "
                      f"double-precision C oracle with {threads} threads, median of "
                      f"{len(times)} passes over {sum(times):.1f} s ({t:.4f} s per pass)"}


# --------------------------------------------------------------------------------------
# profile summaries

def _read_csv_rows(run_dir, suffix):
    rows = []
    for f in glob.glob(os.path.join(run_dir, "**", f"*{suffix}"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def summarize_trace(run_dir, out, cmd, bench_log=None):
    """Kernel statistics of a rocprofv3 --kernel-trace --stats run, the GEMV kernel's
    per-dispatch durations from the same trace (all dispatches, and the last 1000: steady-state
    graph replays at the end of a bench.py run), and the GEMV kernel time bench.py measured
    with HIP events in the same run (from its JSON line)."""
    rows = _read_csv_rows(run_dir, "kernel_stats.csv")
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {run_dir}")
    lines = [f"# rocprofv3 kernel statistics", f"# command: {cmd}",
             "# columns: calls, total_ns, average_ns, min_ns, max_ns, percent, kernel"]
    for r in sorted(rows, key=lambda r: -float(r.get("TotalDurationNs", 0))):
        name = r.get("Name", "")
        name = name[:name.index("(")] if "(" in name and not name.startswith("_Z") else name
        lines.append(f"{r.get('Calls')}, {r.get('TotalDurationNs')}, {r.get('AverageNs')}, "
                     f"{r.get('MinNs')}, {r.get('MaxNs')}, {r.get('Percentage')}, {name}")
    res = None
    if bench_log:
        for line in open(bench_log):
            if line.startswith("{"):
                res = json.loads(line)
    if res:
        kern = res["roofline"]["kernel"]
        disp = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                      for r in _read_csv_rows(run_dir, "kernel_trace.csv")
                      if kern in r.get("Kernel_Name", ""))
        durs = [d for _, d in disp]
        tail = durs[-1000:]
        if durs:
            lines.append(f"# {kern} dispatches in the trace: {len(durs)}, average "
                         f"{statistics.mean(durs) / 1e3:.3f} us, median "
                         f"{statistics.median(durs) / 1e3:.3f} us; last {len(tail)} (steady-state "
                         f"replays): average {statistics.mean(tail) / 1e3:.3f} us, median "
                         f"{statistics.median(tail) / 1e3:.3f} us")
        lines.append(f"# bench.py in the same run: {kern} {res['roofline']['kernel_us']} us per "
                     f"launch (HIP events around back-to-back launches, so launch gaps included), "
                     f"{res['roofline']['achieved']} GB/s algorithmic, frac "
                     f"{res['roofline']['frac']}, weight GB/s {res['value']}")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _pmc_by_kernel(run_dir, counter):
    rows = _read_csv_rows(run_dir, "counter_collection.csv")
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def summarize_pmc(fetch_dir, write_dir, workload, nb, cmd, out_txt):
    """FETCH_SIZE / WRITE_SIZE are in KiB per dispatch. Each is scaled by the factor that
    makes it read exactly the known bytes of the plain streaming kernel in the same
    process (256 MiB read and 256 MiB written)."""
    fetch = _pmc_by_kernel(fetch_dir, "FETCH_SIZE")
    write = _pmc_by_kernel(write_dir, "WRITE_SIZE")

    def pick(d, key):
        ks = [k for k in d if key in k]
        return (ks[0], statistics.median(d[ks[0]]) * 1024.0) if ks else (None, None)
    _, cf = pick(fetch, "neg_kernel")
    _, cw = pick(write, "neg_kernel")
    kernel = "valu_kernel" if any("valu_kernel" in k for k in fetch) else "mfma_kernel"
    kname, kf = pick(fetch, kernel)
    _, kw = pick(write, kernel)
    if None in (cf, cw, kf, kw):
        raise SystemExit(f"missing counters: copy {cf} {cw} kernel {kf} {kw}")
    sf, sw = CALIB_BYTES / cf, CALIB_BYTES / cw
    entry = {"kernel": kernel, "source_hash": kernel_source_hash(kernel),
             "fetch_bytes_counter": kf, "write_bytes_counter": kw, "fetch_scale": sf,
             "write_scale": sw, "hbm_bytes_per_launch": round(kf * sf + kw * sw),
             "command": cmd}
    d = {}
    if os.path.exists(TRAFFIC_FILE):
        try:
            d = json.load(open(TRAFFIC_FILE))
        except ValueError:
            d = {}
    d[f"{workload}_nb{nb}"] = entry
    json.dump(d, open(TRAFFIC_FILE, "w"), indent=1, sort_keys=True)
    p = Problem.algorithmic_bytes(workload, nb, fused=True)  # pmc_probe runs q4mv_fused
    lines = [f"# HBM traffic of {kname.split('(')[0]} on {workload} NB={nb}",
             f"# command (twice, COUNTER = FETCH_SIZE, then WRITE_SIZE): {cmd}",
             f"calibration kernel (torch neg, {CALIB_BYTES} B read + {CALIB_BYTES} B written): "
             f"FETCH_SIZE {cf / 1024:.1f} KiB -> scale {sf:.4f}; "
             f"WRITE_SIZE {cw / 1024:.1f} KiB -> scale {sw:.4f}",
             f"GEMV kernel, median over {len(fetch[kname])} launches: "
             f"FETCH_SIZE {kf / 1024:.1f} KiB, WRITE_SIZE {kw / 1024:.1f} KiB",
             f"scaled HBM bytes per launch: read {kf * sf:.0f}, written {kw * sw:.0f}, "
             f"total {kf * sf + kw * sw:.0f}",
             f"algorithmic bytes per launch: {p} (ratio {(kf * sf + kw * sw) / p:.4f})"]
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_counters(dirs, workload, nb, cmd, out_txt):
    """SQ counters of the GEMV kernel from rocprofv3 --pmc runs of `bench.py --pmc-probe`
    (one directory per pass; each counter's median over the kernel's dispatches), with the
    per-wave and per-cycle ratios they give."""
    vals, kname, launches = {}, None, 0
    for d in dirs:
        for r in _read_csv_rows(d, "counter_collection.csv"):
            k = r["Kernel_Name"]
            if "valu_kernel" not in k and "mfma_kernel" not in k:
                continue
            kname = k
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no GEMV kernel counters under {dirs}")
    med = {c: statistics.median(v) for c, v in vals.items()}
    launches = max(len(v) for v in vals.values())
    lines = [f"# SQ counters of {kname.split('(')[0]} on {workload} NB={nb}",
             f"# command (one run per pass, COUNTERS = the pass's list): {cmd}",
             f"# median over {launches} launches per counter (summed over the device)"]
    lines += [f"{c} {med[c]:.0f}" for c in sorted(med)]
    w = med.get("SQ_WAVES")
    if w:
        lines.append("# per wave:")
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD",
                  "SQ_INSTS_SALU", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_ANY"):
            if c in med:
                lines.append(f"{c} / SQ_WAVES = {med[c] / w:.1f}")
    wc = med.get("SQ_WAVE_CYCLES")
    if wc:
        lines.append("# share of the waves' lifetime:")
        for c in ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM"):
            if c in med:
                lines.append(f"{c} / SQ_WAVE_CYCLES = {med[c] / wc:.3f}")
    bc = med.get("SQ_BUSY_CYCLES")
    if bc and "SQ_VALU_MFMA_BUSY_CYCLES" in med:
        lines.append(f"SQ_VALU_MFMA_BUSY_CYCLES / SQ_BUSY_CYCLES = "
                     f"{med['SQ_VALU_MFMA_BUSY_CYCLES'] / bc:.3f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def pmc_probe(workload, nb):
    import torch
    src = torch.full((CALIB_BYTES // 4,), 1.0, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)  # one kernel that reads and writes exactly CALIB_BYTES
    torch.cuda.synchronize()
    del src, dst
    p = Problem(workload, nb, fused=True)
    for i in range(10):
        p.gemv(i)
    torch.cuda.synchronize()
    print("pmc probe done", flush=True)


# --------------------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="lm_head")
    ap.add_argument("--nb", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-sweep", action="store_true", help="skip the NB / shape sweep")
    ap.add_argument("--eager", action="store_true", help="time plain launches (profiling)")
    ap.add_argument("--pmc-probe", action="store_true")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR")
    ap.add_argument("--out")
    ap.add_argument("--cmd", default="")
    ap.add_argument("--bench-log", help="bench.py output of the profiled run")
    args = ap.parse_args()
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace, args.out, args.cmd, args.bench_log)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, args.workload, args.nb, args.cmd, args.out)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters, args.workload, args.nb, args.cmd,
                                  args.out)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (the GEMV shards by output rows "
              "with no cross-GPU step in the kernel); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.pmc_probe:
        return pmc_probe(args.workload, args.nb)

    prob = Problem(args.workload, args.nb, fused=True)
    if args.eager:
        step_ms = prob.time_eager(args.steps, args.warmup)
        kern_ms = step_ms
    else:
        step_ms = prob.time_steps(args.steps, args.warmup, reps=5)
        trials = sorted(prob.trials)
        # a fused step is exactly one launch of the GEMV kernel: its timed region is the
        # kernel's (HIP events around the graph of back-to-back launches on the launch stream)
        kern_ms = step_ms if prob.fused else prob.time_kernel(args.steps)
    value = prob.weight_bytes / (step_ms * 1e-3) / 1e9
    achieved = prob.algo_bytes / (kern_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "step_us_min_median_max": None if args.eager else
        [round(trials[0] * 1e3, 3), round(step_ms * 1e3, 3), round(trials[-1] * 1e3, 3)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload} {prob.n_mat}x{prob.out_dim}x{prob.in_dim} "
                               f"affine-Q4 group 64, NB={prob.nb}",
                   "n_mat": prob.n_mat, "out_dim": prob.out_dim, "in_dim": prob.in_dim,
                   "nb": prob.nb, "group": 64, "weight_bytes": prob.weight_bytes,
                   "rotation_copies": prob.R, "seed": 0, "graph_captured": not args.eager,
                   "warmup_note": f"at least {args.warmup} steps and {WARM_S} s of untimed "
                                  "replays before the first timed trial",
                   "operands": "u4 codes times f16 activations (f16 dot products and "
                               "matrix-core products), f32 accumulation, bf16 scale+bias per 64",
                   "step": "q4mv_fused (activation prep inside the GEMV launch)"},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "rows_per_s": round(prob.n_mat * prob.out_dim / (step_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic(args.workload, args.nb, prob.kernel),
                     "kernel": prob.kernel,
                     "kernel_us": round(kern_ms * 1e3, 3),
                     "algorithmic_bytes_per_launch": prob.algo_bytes},
    }
    del prob
    torch.cuda.empty_cache()

    if not args.no_sweep and not args.eager:
        sweep = []
        runs = [("lm_head", nb) for nb in (1, 4, 8, 16)] + [("up", nb) for nb in (1, 4, 8)] + \
               [("moe_down", nb) for nb in (4, 1, 8)] + [("dense", nb) for nb in (1, 4, 8)] + \
               [("tiny", 1)]  # tiny: launch-bound, its time only (no roofline claim)
        for name, nb in runs:
            # kernel_us: q4mv on prepared activations; fused_step_us: q4mv_fused (prep
            # inside, one launch); two_launch_step_us: q4mv_prepare_x + q4mv
            p = Problem(name, nb)
            ms = p.time_kernel(200)
            two = p.time_steps(200, 20)
            p.fused = True
            fused = p.time_steps(200, 20)
            gbps = p.weight_bytes / (fused * 1e-3) / 1e9
            sweep.append({"workload": name, "nb": nb, "fused_step_us": round(fused * 1e3, 3),
                          "weight_GBps": round(gbps, 1),
                          "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
                          "rows_per_s": round(p.n_mat * p.out_dim / (fused * 1e-3), 1),
                          "kernel_us": round(ms * 1e3, 3),
                          "two_launch_step_us": round(two * 1e3, 3), "path": p.path})
            del p
            torch.cuda.empty_cache()
        # single weight buffer (no rotation: the 219 MB of weights fit in the 256 MB
        # Infinity Cache, so this is a cache-resident figure, not an HBM one), and the prep
        # launch alone
        p = Problem("lm_head", 1, rotate=False, fused=True)
        ms = p.time_steps(200, 20)
        prep_ms = p.time_prep(200)
        gbps = p.weight_bytes / (ms * 1e-3) / 1e9
        sweep.append({"workload": "lm_head", "nb": 1, "hot": "single weight buffer, "
                      "cache-resident", "fused_step_us": round(ms * 1e3, 3),
                      "weight_GBps": round(gbps, 1)})
        sweep.append({"workload": "lm_head", "nb": 1, "launch": "q4mv_prepare_x alone",
                      "prep_us": round(prep_ms * 1e3, 3)})
        del p
        torch.cuda.empty_cache()
        # fused epilogues: the silu(y / div) store, and the expert MLP chain
        p = Problem("lm_head", 1, silu_div=2.0)
        ms = p.time_kernel(200)
        gbps = p.weight_bytes / (ms * 1e-3) / 1e9
        sweep.append({"workload": "lm_head", "nb": 1, "epilogue": "silu(y/2)",
                      "kernel_us": round(ms * 1e3, 3), "weight_GBps": round(gbps, 1),
                      "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1), "path": p.path})
        del p
        # the Q2 / Q3 variants (VALU kernels), next to Q4 at the same shape and batch
        for name, nb in (("lm_head", 1), ("lm_head", 4), ("moe_down", 2), ("up", 1)):
            for bits in (2, 3):
                p = Problem(name, nb, bits=bits)
                ms = p.time_kernel(200)
                gbps = p.weight_bytes / (ms * 1e-3) / 1e9
                sweep.append({"workload": name, "nb": nb, "codes": f"Q{bits}",
                              "kernel_us": round(ms * 1e3, 3), "weight_GBps": round(gbps, 1),
                              "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
                              "rows_per_s": round(p.n_mat * p.out_dim / (ms * 1e-3), 1)})
                del p
                torch.cuda.empty_cache()
        # the page's two-row claim at its shape: the 640-wide expert down projection (8
        # experts x 2560 x 640) on the one-row, two-row and MFMA kernels, fused launches
        for nb in (1, 2, 4):
            p = Problem("moe_down", nb)
            t = {path: p.time_path(path) * 1e3 for path in (1, 2, 3)}
            sweep.append({"workload": "moe_down", "nb": nb, "compare": "kernel paths",
                          "one_row_us": round(t[1], 3), "two_row_us": round(t[2], 3),
                          "mfma_us": round(t[3], 3),
                          "two_row_vs_one_row": round(t[1] / t[2] - 1.0, 3),
                          "auto_path": p.path})
            del p
            torch.cuda.empty_cache()
        # the quantiser (off the GEMV path): dense f32 LM-head weights -> packed affine-Q4
        wf = torch.randn(151936, 2560, device="cuda") * 0.02
        q4 = __import__("affine_q4_gemv_amd")
        q4.q4mv_quantize(wf)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(10):
            q4.q4mv_quantize(wf)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / 10
        moved = wf.numel() * 4 + wf.numel() // 2 + wf.numel() // 64 * 4
        sweep.append({"workload": "quantize lm_head f32 151936x2560 -> affine-Q4",
                      "kernel_us": round(ms * 1e3, 1),
                      "GBps_read_plus_written": round(moved / (ms * 1e-3) / 1e9, 1),
                      "pct_hbm_peak": round(100 * moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1)})
        del wf
        torch.cuda.empty_cache()
        for fused in (False, True):
            p = MoeChain()
            p.fused = fused
            ms = p.time_kernel(200)
            gbps = p.weight_bytes / (ms * 1e-3) / 1e9
            sweep.append({"workload": "moe_mlp 8x(2560->2x640->2560)", "nb": 4,
                          "launches": "q4mv_fused gate|up + down experts with the SwiGLU "
                                      "inside" if fused else
                                      "gate|up GEMV + SwiGLU prep + down GEMV",
                          "step_us": round(ms * 1e3, 3), "weight_GBps": round(gbps, 1),
                          "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1)})
            del p
            torch.cuda.empty_cache()
        for fused in (False, True):
            p = MoeLayer()
            p.fused = fused
            ms = p.time_kernel(200)
            gbps = p.weight_bytes / (ms * 1e-3) / 1e9
            sweep.append({"workload": f"moe_layer top-8 of 32 experts (2560->2x640->2560), "
                                      f"{p.n_u} routed", "nb": 4,
                          "launches": "gate|up experts from f32 rows + down experts with the "
                                      "SwiGLU inside + combine" if fused else
                                      "prep + gate|up experts + SwiGLU prep + down experts + "
                                      "combine",
                          "step_us": round(ms * 1e3, 3), "weight_GBps": round(gbps, 1),
                          "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1)})
            del p
            torch.cuda.empty_cache()
        sweep += reference_legs()
        result["sweep"] = sweep

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args.workload, args.nb)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
