"""Benchmark of the weight-quantized matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-grid] [--no-cpu]

Workload (one "step" = one qgemm_run): W4A16 decode GEMV, M = 1, N = K = 16384,
signed int4 weights with fp16 scales per group of 128 along K, fp16 out, fp32
accumulation, k_parts = 1 — the M = 1 point of the pages' N = K = 16384 grid
(BitBLAS issue #252 benchmark shapes).  Inputs are seeded synthetic data with
the stated distributions, resident in HBM before timing starts.  A ring of
packed-weight copies larger than twice the 256 MB Infinity Cache is cycled so
that no call reads its weights from cache.

Prints ONE JSON line: value = achieved algorithmic HBM bandwidth of the
workload (GB/s); `roofline` for its kernel; `grid` with the µs, TFLOP/s or
TOP/s, GB/s and roofline fraction of every other configuration of the grid
(M = 1..16384 at N = K = 16384, and the LLaMA-7B projection shapes of hidet
issue #364), each with the CPU oracle's single-thread time for the same call
(`cpu_us`, extrapolated from a 64-column sample); `cpu_baseline` = the CPU
oracle on the headline workload; `targets` (last) = the rows with stated targets.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12                 # B/s
PEAK = {"f16": 2.5e15, "i8": 5.0e15}   # dense MFMA FLOP/s (OP/s for int8)
BITS = {"i4": 4, "u4": 4, "i2": 2, "i8": 8, "f16": 16}
MALL_BYTES = 256 << 20
METRIC = "qgemm µs + TFLOPS/TOPS + HBM GB/s vs roofline, M=1..16384, N=K=16384"


def alg_bytes(M, N, K, w_dtype, g, zeros, bias=False, dq=False):
    """Bytes the computation must move at least once: packed W, scales, zeros, A, C
    (+ bias; + per-row and per-column scales of a dequantised int8 output)."""
    G = 0 if g == 0 else (1 if g < 0 else K // g)
    a_sz = 2 if w_dtype in ("i4", "u4", "f16") else 1
    c_sz = 2 if (a_sz == 2 or dq) else 4
    extra = (N * c_sz if bias else 0) + ((M + N) * 4 if dq else 0)
    return (N * K * BITS[w_dtype]) // 8 + N * G * 2 * (2 if zeros else 1) + M * K * a_sz + M * N * c_sz + extra


def label(c):
    if c["w"] == "quant":
        return f"quantize_rows M={c['M']} K={c['K']}"
    s = f"{c['w']} M={c['M']} N={c['N']} K={c['K']}"
    if c["w"] in ("i4", "u4"):
        s += f" g={c.get('g', 0)}"
    if c.get("zeros"):
        s += " zeros"
    if c.get("kp", 1) > 1:
        s += f" kp={c['kp']}"
        # split-K reduction: atomics unless the entry names another
        s += {"atomic": "", "det": " two-pass", "auto": " auto"}[c.get("split", "atomic")]
    if c.get("dq"):
        s += " dequant-fp16"
    if c.get("bias"):
        s += " bias"
    return s


def make_qgemm(c):
    """The plan a grid entry times (shared with the parity test of the grid)."""
    from weight_quantized_mixed_amd.device import QGemm
    g = c.get("g", 0) if c["w"] in ("i4", "u4") else 0
    split = c.get("split", "atomic")
    return QGemm(c["M"], c["N"], c["K"], c["w"], g, c.get("zeros", False), c.get("kp", 1),
                 deterministic=split == "det", split_auto=split == "auto",
                 dequant_output=bool(c.get("dq")))


def run_entry(q, c, A, W, C, ws, bias=None, rs=None, cs=None):
    """One call of a grid entry's plan, through the entry point the bench times."""
    if c.get("dq"):
        q.run_scaled(A, W, rs, cs, bias, C, ws)
    elif bias is not None:
        q.run(A, W, C, ws, bias=bias)
    else:
        q.run(A, W, C, ws)


_WEIGHTS = {}


def _weights(c, q, seed):
    """Packed weight ring for (format, N, K, g, zeros), shared by every M of the grid."""
    import numpy as np
    import synth
    from weight_quantized_mixed_amd.device import host_to_device
    key = (c["w"], c["N"], c["K"], c.get("g", 0), c.get("zeros", False))
    if key not in _WEIGHTS:
        p = synth.make_problem(1, c["N"], c["K"], c["w"], group_size=c.get("g", 0),
                               has_zeros=c.get("zeros", False), seed=seed,
                               A=np.zeros((1, c["K"]), dtype=np.float16 if c["w"] in ("i4", "u4", "f16") else np.int8))
        packed = q.pack(host_to_device(p.w), host_to_device(p.s), host_to_device(p.z))
        n_ring = 1 if q.packed_bytes >= 2 * MALL_BYTES else -(-(4 * MALL_BYTES) // q.packed_bytes)
        _WEIGHTS[key] = [packed] + [packed.clone() for _ in range(min(n_ring, 64) - 1)]
    return _WEIGHTS[key]


class Bench:
    """A configuration resident on the device with a ring of weight copies."""

    def __init__(self, c, seed):
        import torch
        import synth
        from weight_quantized_mixed_amd.device import host_to_device
        self.c = c
        M, N, K, wd = c["M"], c["N"], c["K"], c["w"]
        g, z = c.get("g", 0), c.get("zeros", False)
        if wd not in ("i4", "u4"):
            g = 0
        self.dq, bias = bool(c.get("dq")), bool(c.get("bias"))
        self.q = make_qgemm(c)
        self.packed = _weights(c, self.q, seed)
        A = host_to_device(synth.draw_activations(M, K, self.q.a_dtype, seed + M))
        n_a = 1 if A.numel() * A.element_size() >= 2 * MALL_BYTES else len(self.packed)
        self.As = [A] + [A.clone() for _ in range(n_a - 1)]
        self.C = self.q.new_output()
        self.ws = self.q.workspace()
        self.bias = host_to_device(synth.draw_bias(N, self.q.out_dtype, seed + 5)) if bias else None
        if self.dq:
            self.rs = host_to_device(synth.draw_col_scales(M, seed + 6))
            self.cs = host_to_device(synth.draw_col_scales(N, seed + 7))
        self.i = 0
        self.bytes = alg_bytes(M, N, K, wd, g, z, bias, self.dq)
        self.flops = 2.0 * M * N * K
        self.a_kind = "f16" if wd in ("i4", "u4", "f16") else "i8"
        self.path_name = "gemv" if self.q.path == 1 else "mfma"
        torch.cuda.synchronize()

    def call(self):
        j = self.i
        self.i += 1
        A, W = self.As[j % len(self.As)], self.packed[j % len(self.packed)]
        run_entry(self.q, self.c, A, W, self.C, self.ws, self.bias,
                  self.rs if self.dq else None, self.cs if self.dq else None)

    def timed(self, n):
        """Seconds per call over n back-to-back calls (HIP events on the launch stream)."""
        import torch
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(n):
            self.call()
        e1.record(st)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n

    def timed_bound(self, n):
        """As timed(), with the C ABI arguments of every ring entry resolved beforehand, so
        that each call costs the host one ctypes call: the plain path launches a kernel in
        about as long as the weights take to stream, and a host-bound loop would time the
        host instead."""
        import torch
        from weight_quantized_mixed_amd import qgemm as qmod
        assert not self.dq and self.bias is None
        fn = qmod.load().qgemm_run
        st = torch.cuda.current_stream()
        sh = st.cuda_stream
        a_ptrs = [A.data_ptr() for A in self.As]
        w_ptrs = [W.data_ptr() for W in self.packed]
        c_ptr = self.C.data_ptr()
        ws_ptr = self.ws.data_ptr() if self.ws is not None else None
        wsb = 0 if self.ws is None else self.ws.numel()
        plan, na, nw = self.q.plan, len(a_ptrs), len(w_ptrs)
        j0 = self.i
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for j in range(j0, j0 + n):
            if fn(plan, a_ptrs[j % na], w_ptrs[j % nw], c_ptr, ws_ptr, wsb, sh):
                raise RuntimeError("qgemm_run failed")
        e1.record(st)
        e1.synchronize()
        self.i = j0 + n
        return e0.elapsed_time(e1) * 1e-3 / n

    def graph(self, per):
        """A HIP graph of `per` back-to-back calls cycling through the ring (captured on
        a side stream; the library allocates nothing and launches only kernels)."""
        import torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for _ in range(per):
                    self.call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        return g

    def timed_graph(self, g, per):
        """Seconds per call of one replay of a graph of `per` calls."""
        import torch
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        g.replay()
        e1.record(st)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / per

    def roof(self, t):
        t_hbm = self.bytes / HBM_PEAK
        t_mfma = self.flops / PEAK[self.a_kind]
        bound = "hbm" if t_hbm >= t_mfma else "mfma"
        return bound, max(t_hbm, t_mfma) / t

    def close(self):
        self.q.close()


class QuantBench(Bench):
    """qgemm_quantize_rows on fp16 [M, K] activations: reads 2 bytes and writes 1 byte
    per element plus one fp32 scale per row (HBM-bound)."""

    def __init__(self, c, seed):
        import torch
        import synth
        from weight_quantized_mixed_amd.device import host_to_device
        self.c = c
        M, K = c["M"], c["K"]
        A = host_to_device(synth.draw_fp16_activations(M, K, seed))
        n = 1 if A.numel() * 2 >= 2 * MALL_BYTES else min(64, -(-(4 * MALL_BYTES) // (A.numel() * 2)))
        self.packed = [A] + [A.clone() for _ in range(n - 1)]   # the input ring
        self.Q = torch.empty((M, K), dtype=torch.int8, device=A.device)
        self.S = torch.empty(M, dtype=torch.float32, device=A.device)
        self.i = 0
        self.bytes = M * K * 3 + M * 4
        self.flops = 0.0
        self.a_kind = "f16"
        self.path_name = "quant"
        torch.cuda.synchronize()

    def call(self):
        from weight_quantized_mixed_amd.device import quantize_rows
        j = self.i
        self.i += 1
        quantize_rows(self.packed[j % len(self.packed)], self.Q, self.S)

    def close(self):
        pass


def measure_grid_entry(b, bursts=50):
    """Median (p10, p90) over bursts of back-to-back calls replayed from one HIP graph,
    so that small calls are timed on the GPU rather than at the host's launch rate."""
    import statistics
    b.timed(5)
    # at least 64 calls per replay (whole turns of the ring), so that the replay's own
    # start-up is spread over enough calls not to show in the per-call time
    ring = max(len(b.packed), 1)
    per = ring * max(1, -(-64 // ring))
    if b.flops > 1e12:
        per, bursts = 2, 5
    g = b.graph(per)
    b.timed_graph(g, per)
    samples = sorted(b.timed_graph(g, per) for _ in range(bursts))
    del g
    t = statistics.median(samples)
    bound, frac = b.roof(t)
    # compact keys: the JSON line carries every entry of the grid
    return {"c": label(b.c), "us": round(t * 1e6, 2),
            "p10": round(samples[max(0, len(samples) // 10)] * 1e6, 2),
            "p90": round(samples[min(len(samples) - 1, (9 * len(samples)) // 10)] * 1e6, 2),
            ("tflops" if b.a_kind == "f16" else "tops"): round(b.flops / t / 1e12, 2),
            "gbs": round(b.bytes / t / 1e9), "bound": bound, "frac": round(frac, 3),
            "path": b.path_name}


GRID = ([{"w": "i4", "M": M, "N": 16384, "K": 16384, "g": 128} for M in (32, 128, 512)]
        + [{"w": "i4", "M": 1, "N": 16384, "K": 16384, "g": 128, "kp": 4, "split": sp}
           for sp in ("atomic", "det")]
        + [{"w": w, "M": M, "N": 16384, "K": 16384, "kp": kp} for w in ("i8", "i2")
           for M in (1, 32, 128, 512) for kp in (1, 4)]
        + [{"w": w, "M": M, "N": 16384, "K": 16384, "kp": 4, "split": "auto"} for w in ("i8", "i2")
           for M in (128, 512)]
        + [{"w": "f16", "M": M, "N": 16384, "K": 16384} for M in (1, 32, 128, 512)]
        # the LLaMA-7B projection shapes with k-parts 1 and 4: atomic fp32 reduction (the
        # pages' parallel-k) and the ordered two-pass one
        + [{"w": "i4", "M": M, "N": N, "K": K, "g": 128, "kp": kp, "split": sp} for M in (1, 128)
           for (K, N) in ((4096, 11008), (11008, 4096), (4096, 4096), (4096, 32000))
           for (kp, sp) in ((1, "atomic"), (4, "atomic"), (4, "det"))]
        + [{"w": "i4", "M": M, "N": 16384, "K": 16384, "g": g} for g in (0, -1) for M in (1, 32, 128, 512)]
        # bias epilogue; int8 products with the dequantised fp16 output; the per-row
        # int8 quantiser of fp16 activations
        + [{"w": "i4", "M": M, "N": 16384, "K": 16384, "g": 128, "bias": True} for M in (1, 512)]
        + [{"w": w, "M": M, "N": 16384, "K": 16384, "dq": True, "bias": True} for w in ("i8", "i2")
           for M in (1, 512)]
        + [{"w": "quant", "M": M, "K": 16384} for M in (512, 16384)]
        # the per-call floor: the smallest product (one 16 x 128 weight block), one kernel
        + [{"w": "i4", "M": 1, "N": 16, "K": 128, "g": 128}]
        # M = N = K = 16384: the pages' five large-M products (fp16, int4 unscaled and with
        # one group over K, W8A8, W2A8) and uint4 with g = 128 zero points
        + [{"w": "f16", "M": 16384, "N": 16384, "K": 16384},
           {"w": "u4", "M": 16384, "N": 16384, "K": 16384, "g": 128, "zeros": True}]
        + [{"w": "i4", "M": 16384, "N": 16384, "K": 16384, "g": g} for g in (0, -1)]
        + [{"w": w, "M": 16384, "N": 16384, "K": 16384} for w in ("i8", "i2")]
        # W4A16 with g = 128 scales at M = 16384, the last M of the pages' grid
        + [{"w": "i4", "M": 16384, "N": 16384, "K": 16384, "g": 128}])


# the timed workload: W4A16 decode at M = 1, N = K = 16384, g = 128, k_parts = 1
HEADLINE = {"w": "i4", "M": 1, "N": 16384, "K": 16384, "g": 128}


def make_bench(c, seed):
    return QuantBench(c, seed) if c["w"] == "quant" else Bench(c, seed)


HEADLINE_PROFILE = os.path.join(ROOT, "profiles", "gemv_w4a16_m1_n16384_k16384.md")
HEADLINE_SOURCES = [os.path.join(ROOT, "weight_quantized_mixed_amd", "csrc", f)
                    for f in ("gemv.hip", "qgemm_internal.hpp")]


def recorded_traffic():
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE profile of the
    headline kernel, or None when the kernel source changed since it was taken."""
    import hashlib
    try:
        h = hashlib.sha256(b"".join(open(f, "rb").read() for f in HEADLINE_SOURCES)).hexdigest()[:16]
        fields = {}
        for line in open(HEADLINE_PROFILE):
            k, _, v = line.strip().partition(":")
            if k in ("traffic_bytes_per_launch", "source_hash"):
                fields[k] = v.strip()
        if fields.get("source_hash") == h:
            return int(fields["traffic_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        pass
    return None


def cpu_baseline(c, seed):
    """The CPU oracle, as it stands, on the benchmark workload (one full step)."""
    import numpy as np
    import oracle
    import synth
    from threadpoolctl import threadpool_limits
    p = synth.make_problem(c["M"], c["N"], c["K"], c["w"], group_size=c.get("g", 0), seed=seed)
    # one thread throughout (the unpack and dequantisation are single-threaded numpy
    # passes; BLAS is held to one thread for the final float64 product), full steps
    # of the workload repeated until at least 10 s of CPU work
    steps, dt = 0, 0.0
    with threadpool_limits(limits=1):
        while dt < 10.0 and steps < 8:
            t0 = time.perf_counter()
            oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=p.N, K=p.K, w_dtype=p.w_dtype, group_size=p.group_size)
            dt += time.perf_counter() - t0
            steps += 1
    nbytes = alg_bytes(c["M"], c["N"], c["K"], c["w"], c.get("g", 0), False)
    return {"value": round(steps * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "sample": f"{steps} full steps ({label(c)}), {dt:.2f} s, float64 numpy, 1 thread",
            "seconds": round(dt, 3), "host_cpus": os.cpu_count()}


# the rows that carry a stated target: >= 70 % of the HBM roofline for W4A16 and W2A8
# at M = 1, >= 60 % of the dense fp16 MFMA peak at M = N = K = 16384
TARGET_ROWS = {"w2a8_m1": ("i2 M=1 N=16384 K=16384", 0.70),
               "f16_16384": ("f16 M=16384 N=16384 K=16384", 0.60),
               "u4z_16384": ("u4 M=16384 N=16384 K=16384 g=128 zeros", 0.60)}


def targets(out):
    """µs and roofline fraction of each targeted row (last on the line, so that a
    reader of the line's tail sees them)."""
    t = {"w4a16_m1": {"us": out["config"]["us_per_call"], "frac": out["roofline"]["frac"], "goal": 0.70}}
    rows = {r["c"]: r for r in out.get("grid", [])}
    for key, (lab, goal) in TARGET_ROWS.items():
        if lab in rows:
            t[key] = {"us": rows[lab]["us"], "frac": rows[lab]["frac"], "goal": goal}
    return t


def oracle_us(c):
    """Single-thread time of the CPU oracle for one call of a grid entry, extrapolated from
    a sample (the best of three runs): all K, 64 output columns, and all rows up to 64
    (else 64): the oracle's cost grows with the columns it unpacks and with rows x
    columns of its product."""
    import numpy as np
    import oracle
    import synth
    from threadpoolctl import threadpool_limits
    M, K = c["M"], c["K"]
    Ms = min(M, 64)

    def best_of_3(f):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            f()
            ts.append(time.perf_counter() - t0)
        return min(ts)

    with threadpool_limits(limits=1):
        if c["w"] == "quant":
            A = synth.draw_fp16_activations(Ms, K, seed=1)
            return round(best_of_3(lambda: oracle.quantize_rows(A)) * 1e6 * M / Ms, 1)
        N = c["N"]
        Ns = min(N, 64)
        g = c.get("g", 0) if c["w"] in ("i4", "u4") else 0
        p = synth.make_problem(Ms, Ns, K, c["w"], group_size=g, has_zeros=c.get("zeros", False), seed=1)
        if c.get("dq"):
            run = lambda: oracle.qgemm_ref_scaled(p.A, p.w, N=Ns, K=K, w_dtype=p.w_dtype,
                                                  row_scales=np.ones(Ms, np.float32),
                                                  col_scales=np.ones(Ns, np.float32))
        else:
            run = lambda: oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=Ns, K=K, w_dtype=p.w_dtype,
                                           group_size=p.group_size)
        return round(best_of_3(run) * 1e6 * (N / Ns) * (M / Ms), 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    # about 20 ms of untimed calls: the engine clock takes several milliseconds to
    # settle after the set-up (the first 400 calls measured 23.7 against 22.1 us)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--no-grid", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="", help="substring filter on grid entries")
    ap.add_argument("--exact", action="store_true", help="--only names one grid entry exactly")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (scales HBM counters)")
    ap.add_argument("--torch-matmul", type=int, default=0, metavar="S",
                    help="only time torch.matmul (the vendor BLAS) on fp16 S x S x S, the weight stored "
                         "[N, K] as here, as a comparison for the dense fp16 rows")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path does not "
              "shard across GPUs here)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    import synth
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy << 18   # float32 elements
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4}))
        return

    if args.torch_matmul:
        S = args.torch_matmul
        g = torch.Generator(device="cuda").manual_seed(1)
        A = torch.randn((S, S), dtype=torch.float16, device="cuda", generator=g)
        W = torch.randn((S, S), dtype=torch.float16, device="cuda", generator=g)   # [N, K]
        Wt = W.t()   # a K-major view of the [N, K] weight, as qgemm stores it
        for _ in range(3):
            torch.matmul(A, Wt)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(5):
            e0.record()
            torch.matmul(A, Wt)
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        t = sorted(ts)[len(ts) // 2]
        print(json.dumps({"torch_matmul_fp16": S, "us": round(t * 1e6, 1),
                          "tflops": round(2.0 * S ** 3 / t / 1e12, 1),
                          "frac_of_2.5PF": round(2.0 * S ** 3 / t / PEAK["f16"], 4)}))
        return

    head = HEADLINE
    print(f"[bench] workload {label(head)}", file=sys.stderr, flush=True)
    hb = Bench(head, synth.seed_for(5))
    hb.timed_bound(args.warmup)
    torch.cuda.synchronize()
    t_call = hb.timed_bound(args.steps)    # barrier + synchronize on both sides (one rank)
    torch.cuda.synchronize()
    bound, frac = hb.roof(t_call)
    achieved = hb.bytes / t_call
    out = {
        "metric": METRIC, "value": round(achieved / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_call * 1e3, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded; A~N(0,1) fp16, q~U[-8,7], s~U[0.005,0.02] fp16)",
        "config": {"workload": "W4A16 GEMV M=1 N=16384 K=16384 g=128 k_parts=1", "M": 1, "N": 16384,
                   "K": 16384, "group_size": 128, "k_parts": 1, "ring_copies": len(hb.packed),
                   "us_per_call": round(t_call * 1e6, 3)},
        "roofline": {"bound": bound, "achieved": round(achieved / 1e9, 2), "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": round(frac, 4), "traffic": recorded_traffic(),
                     "alg_bytes_per_launch": hb.bytes, "kernel": "gemv_kernel<FMT_I4, 1>"},
    }
    hb.close()
    del hb
    _WEIGHTS.clear()
    torch.cuda.empty_cache()
    print(f"[bench] headline {out['config']['us_per_call']} us, {out['value']} GB/s", file=sys.stderr, flush=True)

    if not args.no_grid:
        grid = []
        for i, c in enumerate(GRID):
            if args.only and (label(c) != args.only if args.exact else args.only not in label(c)):
                continue
            b = make_bench(c, synth.seed_for(6, i))
            grid.append(measure_grid_entry(b))
            r = grid[-1]
            if not args.no_cpu:
                r["cpu_us"] = oracle_us(c)
            print(f"[bench] {r['c']}: {r['us']} us, {r['frac']}", file=sys.stderr, flush=True)
            b.close()
            del b
            time.sleep(0.05)   # gap between configurations
        out["grid"] = grid
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(head, synth.seed_for(5))
    out["targets"] = targets(out)
    print(json.dumps(out, separators=(",", ":")), flush=True)


if __name__ == "__main__":
    main()
