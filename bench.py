"""Benchmark: exact attention forward + backward through the HIP library (libfa.so).

One step = one pass of the whole path on one batch of synthetic input:
fa_fwd, then the backward's three stages (fa_bwd_preprocess, fa_bwd_dkdv,
fa_bwd_dq, which together are fa_bwd). Inputs, outputs and workspace are
resident in device memory before the timed region starts.

    python bench.py [--steps K] [--warmup W] [--workload causal8k] [--cpu-seconds 10]

Prints ONE JSON line. `value` is fwd+bwd throughput in TFLOP/s over the wall
clock of the K timed steps, counting matmul FLOPs only: forward
4*B*H*N^2*d*rho (two N x N x d products), backward 2.5x that (five products,
the recompute of S included), rho = fraction of (query, key) pairs attended.
`roofline` is the kernel with the largest share of the step, timed with HIP
events recorded on the stream the kernels run on, against the dense bf16 MFMA
peak of MI355X. `cpu_baseline` is the fp64 CPU oracle timed on a bounded sample
(whole heads, forward + backward) on this host's cores, with the same FLOP
numerator per head.

--kernel softmax times the standalone row softmax (fa_softmax_rows) on a
float32 matrix (--softmax-shape ROWSxCOLS) instead, in GB/s against HBM.

--kernel decode times decoding against a KV cache (fa_decode) on
--decode-shape BxHxNqxNkxd, in GB/s of the K/V stream against HBM.

--kernel naive times standard attention on --workload, the comparator of the
IO argument: S = Q K^T and P = softmax(S) materialised in device memory in
bf16 by torch's GEMM and softmax (a measurement tool only, not part of the
library), beside fa_fwd on the same inputs.

--probe copy runs an elementwise kernel that reads and writes a buffer of known
size, used to calibrate rocprofv3's FETCH_SIZE / WRITE_SIZE counters.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd & fwd+bwd TFLOP/s and % of bf16 MFMA peak, N=2k–32k"
# MI355X dense bf16 MFMA peak: 256 CU x 4096 FLOP/clk/CU x 2.4 GHz.
PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ("fa_api.hip", "fa_fwd.hip", "fa_bwd.hip", "fa_bwd_dq.hip", "fa_softmax.hip",
                  "fa_decode.hip", "fa_fwd_kv_outer.hip", "fa_common.hpp", "fa_kernels.hpp")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="causal8k",
                    help="tiny | dense2k | causal8k | causal32k | sparse16k")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the CPU oracle runs whole heads until this much time has passed "
                         "(at least one head; 0 = skip cpu_baseline)")
    ap.add_argument("--block-keep", type=float, default=None,
                    help="run the workload with a 128x128 block mask of this keep probability "
                         "(off-diagonal blocks; the diagonal is always kept)")
    ap.add_argument("--causal", action="store_true", help="add the causal mask to the workload")
    ap.add_argument("--kernel", choices=["attention", "softmax", "decode", "fwd-kv-outer",
                                         "naive"],
                    default="attention",
                    help="attention: the fwd+bwd step (default); softmax: the standalone row "
                         "softmax (fa_softmax_rows) on --softmax-shape; decode: the newest "
                         "queries against a KV cache (fa_decode) on --decode-shape; "
                         "fwd-kv-outer: the forward in the K/V-outer loop order "
                         "(fa_fwd_kv_outer) beside fa_fwd on --workload; naive: standard "
                         "attention with S and P materialised (torch GEMM + softmax) beside "
                         "fa_fwd on --workload")
    ap.add_argument("--decode-shape", default="4x32x16x32768x128",
                    help="BxHxNqxNkxd for --kernel decode (causal unless --decode-full)")
    ap.add_argument("--decode-full", action="store_true",
                    help="--kernel decode without the causal mask")
    ap.add_argument("--softmax-shape", default="65536x4096",
                    help="ROWSxCOLS of the float32 matrix for --kernel softmax")
    ap.add_argument("--probe", choices=["copy"], default=None)
    ap.add_argument("--probe-mib", type=int, default=1024)
    return ap.parse_args()


# The sources each measured kernel is built from (its own file, the shared
# device header, the launch interface and the C ABI): a traffic record is valid
# only while these are unchanged.
COMMON_SOURCES = ("fa_api.hip", "fa_common.hpp", "fa_kernels.hpp")
KERNEL_FILE = {"fa_fwd_kernel": "fa_fwd.hip", "fa_bwd_pre_kernel": "fa_bwd.hip",
               "fa_bwd_dkdv_kernel": "fa_bwd.hip", "fa_bwd_dq_kernel": "fa_bwd_dq.hip",
               "softmax_rows_reg": "fa_softmax.hip", "softmax_rows_stream": "fa_softmax.hip",
               "fa_decode_split_kernel": "fa_decode.hip"}


def source_digest(files=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(ROOT, "exact_io_aware_61_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_digest(kernel: str) -> str:
    """Digest of the sources one kernel is built from."""
    return source_digest((KERNEL_FILE[kernel],) + COMMON_SOURCES)


def traffic_record(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from a committed counter summary, if it was taken on this source.

    profiles/traffic_<kernel>_<workload>.md holds a line
    `traffic-record: {"src": "<digest>", "bytes_per_launch": X, ...}`, where the digest
    is kernel_digest(kernel) of the sources the counters were taken on.
    """
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic-record:"):
                rec = json.loads(line.split(":", 1)[1])
                if rec.get("src") == digest:
                    return rec
    return None


def device_info(lib, device: int = 0):
    """CU count and peak shader clock as the HIP runtime reports them, and the peak they give.

    hipDeviceGetAttribute is looked up through libfa.so, so it is the runtime the
    kernels run on. Attribute codes from ROCm 7's hip_runtime_api.h:
    hipDeviceAttributeClockRate = 5 (kHz), hipDeviceAttributeMultiprocessorCount = 63.
    """
    try:
        get = lib.hipDeviceGetAttribute
    except AttributeError:
        return None
    get.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    khz, cus = ctypes.c_int(0), ctypes.c_int(0)
    if get(ctypes.byref(khz), 5, device) != 0 or get(ctypes.byref(cus), 63, device) != 0:
        return None
    return {"cus": cus.value, "peak_clock_mhz": khz.value / 1000.0,
            "bf16_peak_tflops": round(cus.value * 4096 * khz.value * 1e3 / 1e12, 1),
            "formula": "CUs x 4096 dense bf16 FLOP/clk per CU x peak clock"}


def probe_copy(mib: int, steps: int):
    import torch
    n = mib * (1 << 20) // 4
    x = torch.randn(n, device="cuda:0", dtype=torch.float32)
    y = torch.empty_like(x)
    for _ in range(steps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "copy", "bytes_read": 4 * n, "bytes_written": 4 * n,
                      "launches": steps}), flush=True)


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (the architecture if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, q, k, v, do, bm, seconds: float):
    """Time the oracle on whole heads on the host cores: forward + backward, then forward alone.

    Heads run one after another until `seconds` have passed (at least one head,
    at most all of them); the rate is the heads done over the time they took.
    The forward alone then runs on the same heads, for at most `seconds / 2`.
    """
    import numpy as np
    import threadpoolctl
    from oracle import attention_head
    from exact_io_aware_61_amd.workloads import kept_fraction

    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()
                   if p.get("user_api") == "blas"] or [1])

    def run(with_grad: bool, budget: float, limit: int):
        done, dt = 0, 0.0
        while done < limit and (done == 0 or dt < budget):
            b, h = divmod(done, w.H)
            qa, ka, va, da = (t[b, h].double().numpy() for t in (q, k, v, do))
            t0 = time.perf_counter()
            attention_head(qa, ka, va, da if with_grad else None, scale=w.scale,
                           causal=w.causal, block_mask=bm)
            dt += time.perf_counter() - t0
            done += 1
        return done, dt

    done, dt = run(True, seconds, w.B * w.H)
    fdone, fdt = run(False, seconds / 2, done)
    rho = kept_fraction(w.N, w.causal, bm)
    fwd_head = 4.0 * w.N * w.N * w.d * rho
    # what the oracle executes: dense products over every (query, key) pair, masked
    # ones included: S and P V (4 N^2 d), then dV, dP, dQ, dK (8 N^2 d)
    exe_fwd, exe_all = 4.0 * w.N * w.N * w.d, 12.0 * w.N * w.N * w.d
    return {"value": 3.5 * fwd_head * done / dt / 1e12, "unit": "TFLOP/s",
            "executed_tflops": exe_all * done / dt / 1e12,
            "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {w.B * w.H} heads of {w.name}, forward+backward, fp64 "
                      f"NumPy with S and P materialised, {dt:.2f} s",
            "seconds": dt,
            "fwd": {"value": fwd_head * fdone / fdt / 1e12, "unit": "TFLOP/s",
                    "executed_tflops": exe_fwd * fdone / fdt / 1e12,
                    "sample": f"{fdone} heads, forward only, {fdt:.2f} s", "seconds": fdt},
            "cpu": cpu_model(), "host_cpus": os.cpu_count()}


def bench_softmax(args):
    """Row softmax: one step = one fa_softmax_rows over a [rows, cols] float32 matrix.

    Algorithmic traffic is one read and one write of the matrix (8 bytes per
    element); `value` is that over the measured time, against the HBM peak.
    """
    import numpy as np
    import torch

    import exact_io_aware_61_amd as fa
    rows, cols = (int(v) for v in args.softmax_shape.lower().split("x"))
    print(f"[bench] softmax rows={rows} cols={cols}", file=sys.stderr, flush=True)
    g = torch.Generator(device="cpu").manual_seed(4242)
    x_cpu = torch.randn((rows, cols), generator=g, dtype=torch.float32) * 4.0
    x = x_cpu.cuda()
    y = torch.empty_like(x)
    lib = fa.load()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step():
        rc = lib.fa_softmax_rows(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                 rows, cols, sp)
        if rc != 0:
            raise fa.FaError(rc, fa.strerror(rc))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(K):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_ms = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(K)]))
    nbytes = 8.0 * rows * cols
    achieved = nbytes / (per_ms * 1e-3) / 1e9
    value = nbytes / (wall / K) / 1e9
    kname = "softmax_rows_reg" if (cols % 4 == 0 and cols <= 4096) else "softmax_rows_stream"
    digest = source_digest()
    rec = traffic_record(kname, f"{rows}x{cols}", kernel_digest(kname))
    result = {
        "metric": "row softmax GB/s (one read + one write per element)", "value": round(value, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"softmax_rows {rows}x{cols}", "rows": rows, "cols": cols},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if rec is None else rec["bytes_per_launch"],
                     "avg_launch_ms": round(per_ms, 4), "bytes_per_launch": nbytes},
        "src": digest,
    }
    if args.cpu_seconds > 0:
        # the oracle on whole rows until the time is spent (same 8-byte numerator)
        import threadpoolctl
        from oracle.softmax_forms import row_softmax
        threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
        xs = x_cpu.double().numpy()
        done, dt, chunk = 0, 0.0, max(1, min(rows, (1 << 22) // max(cols, 1)))
        while done < rows and (done == 0 or dt < args.cpu_seconds):
            t1 = time.perf_counter()
            row_softmax(xs[done:done + chunk])
            dt += time.perf_counter() - t1
            done += min(chunk, rows - done)
        result["cpu_baseline"] = {"value": 8.0 * done * cols / dt / 1e9, "unit": "GB/s",
                                  "cores": int(threads), "kind": "oracle",
                                  "sample": f"{done} of {rows} rows, fp64 NumPy, {dt:.2f} s",
                                  "seconds": dt, "cpu": cpu_model(), "host_cpus": os.cpu_count()}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def bench_decode(args):
    """Decoding: one step = one fa_decode of Nq new queries against an Nk-key cache.

    Algorithmic traffic: K and V read once, Q read and O, LSE written once; the
    kernels' per-chunk partial results in the workspace are not counted.
    """
    import numpy as np
    import torch

    import exact_io_aware_61_amd as fa
    from exact_io_aware_61_amd.workloads import make_qkv
    B, H, Nq, Nk, d = (int(v) for v in args.decode_shape.lower().split("x"))
    causal = not args.decode_full
    print(f"[bench] decode B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal}", file=sys.stderr,
          flush=True)
    q, _, _, _ = make_qkv(B, H, Nq, d, 4321, with_do=False)
    _, k, v, _ = make_qkv(B, H, Nk, d, 4322, with_do=False)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    scale = float(np.float32(1 / np.sqrt(d)))
    o = torch.empty_like(qg)
    lse = torch.empty((B, H, Nq), device=qg.device, dtype=torch.float32)
    lib = fa.load()
    n = ctypes.c_size_t()
    lib.fa_decode_workspace_size(B, H, Nq, Nk, d, ctypes.byref(n))
    ws = torch.empty(max(n.value, 16), device=qg.device, dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def step():
        rc = lib.fa_decode(P(qg), P(kg), P(vg), P(o), P(lse), B, H, Nq, Nk, d, scale,
                           1 if causal else 0, P(ws), ws.numel(), sp)
        if rc != 0:
            raise fa.FaError(rc, fa.strerror(rc))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(K):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_ms = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(K)]))
    nbytes = float(B * H * (4 * Nk * d + 4 * Nq * d + 4 * Nq))
    achieved = nbytes / (per_ms * 1e-3) / 1e9
    digest = source_digest()
    shape = f"{B}x{H}x{Nq}x{Nk}x{d}"
    rec = traffic_record("fa_decode_split_kernel", shape, kernel_digest("fa_decode_split_kernel"))
    result = {
        "metric": "decode GB/s (K, V, Q read and O, LSE written once)",
        "value": round(nbytes / (wall / K) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(wall / K * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decode {shape}{' causal' if causal else ''}", "B": B, "H": H,
                   "Nq": Nq, "Nk": Nk, "d": d, "causal": causal},
        "roofline": {"bound": "hbm", "kernel": "fa_decode_split_kernel + fa_decode_combine_kernel",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if rec is None else rec["bytes_per_launch"],
                     "avg_launch_ms": round(per_ms, 4), "bytes_per_launch": nbytes},
        "src": digest,
    }
    if args.cpu_seconds > 0:
        import threadpoolctl
        from oracle.decode import decode_head
        threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
        done, dt = 0, 0.0
        while done < B * H and (done == 0 or dt < args.cpu_seconds):
            b, h = divmod(done, H)
            qa, ka, va = (t[b, h].double().numpy() for t in (q, k, v))
            t1 = time.perf_counter()
            decode_head(qa, ka, va, scale=scale, causal=causal)
            dt += time.perf_counter() - t1
            done += 1
        per_head = 4 * Nk * d + 4 * Nq * d + 4 * Nq
        result["cpu_baseline"] = {"value": per_head * done / dt / 1e9, "unit": "GB/s",
                                  "cores": int(threads), "kind": "oracle",
                                  "sample": f"{done} of {B * H} heads, fp64 NumPy, {dt:.2f} s",
                                  "seconds": dt, "cpu": cpu_model(), "host_cpus": os.cpu_count()}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def fwd_rows_per_workgroup(d: int, masked: bool) -> int:
    """Query rows per fa_fwd workgroup: 256 at d=128 without a block mask, else 128."""
    return 128 if (masked or d == 64) else 256


def pass_io_models(N: int, d: int, causal: bool, block_mask, heads: int) -> dict:
    """Device bytes of each pass of the step per launch: compulsory (every tensor read or
    written once) and the tile model (the Theta(N^2 d^2 / M) term: the streamed operand
    re-read once for every workgroup that visits it), counted from the kernels' loops.

    Forward and dQ: a workgroup per block of BM query rows streams the K/V tiles of 64
    keys (32 for the unmasked d=64 dQ) it sees. dK/dV: a workgroup per block of 128 keys
    streams the Q/dO tiles of 64 rows (plus their D and L2 rows, 8 bytes per row) it
    sees. Preprocess: O and dO read, LSE read, D and L2 written. A tile is visited if
    one of its (query, key) pairs is attended (causal: key <= query; block mask: its
    128 x 128 block kept). block_mask: [ceil(N/128)]^2 array or None.
    """
    import numpy as np
    nb = -(-N // 128)
    keep = np.ones((nb, nb), bool) if block_mask is None else np.asarray(block_mask).astype(bool)
    masked = block_mask is not None

    def visits(rows, keys):
        """(row block, key block) pairs with an attended pair; rows, keys: block sizes,
        keys <= 128 and dividing 128, so a key block lies inside one mask column."""
        nk = -(-N // keys)
        col = (np.arange(nk) * keys) // 128          # mask column of each key block
        total = 0
        for r0 in range(0, N, rows):
            r1 = min(N, r0 + rows) - 1
            seen = keep[r0 // 128:r1 // 128 + 1].any(axis=0)[col]   # kept in any of its mask rows
            upto = r1 // keys + 1 if causal else nk                 # causal: keys <= last row
            total += int(seen[:upto].sum())
        return total

    nd = N * d
    bm_fwd = fwd_rows_per_workgroup(d, masked)
    bm_dq = 128 if (masked or d == 64) else 256
    bn_dq = 32 if (d == 64 and not masked) else 64
    v_fwd, v_dq, v_kv = visits(bm_fwd, 64), visits(bm_dq, bn_dq), visits(64, 128)
    per_head = {
        "compulsory_fwd": 8 * nd + 4 * N,
        "tile_model_fwd": 4 * nd + v_fwd * 64 * d * 4 + 4 * N,
        "compulsory_pre": 4 * nd + 12 * N,
        "compulsory_dkdv": 12 * nd + 8 * N,
        "tile_model_dkdv": 8 * nd + v_kv * (64 * d * 4 + 64 * 8),
        "compulsory_dq": 10 * nd + 8 * N,
        "tile_model_dq": 6 * nd + 8 * N + v_dq * bn_dq * d * 4,
    }
    out = {k: heads * v for k, v in per_head.items()}
    out["rows_per_workgroup_fwd"] = bm_fwd
    return out


def kv_outer_io_model(N: int, d: int, causal: bool, heads: int) -> float:
    """Device bytes of the K/V-outer forward per launch, counted from its loops.

    Per head: K, V read once; for every visited (K/V block, Q block) pair the Q
    block is read and O (float32), m, l are read (except at the first K/V block)
    and written; a last sweep reads O, m, l and writes O (bf16) and LSE.
    Blocks: 128 query rows, 64 keys.
    """
    BM, BN = 128, 64
    Tr, Tc = -(-N // BM), -(-N // BN)
    visits = sum(Tr - (j * BN // BM if causal else 0) for j in range(Tc))
    per_visit_write = 4 * BM * d + 8 * BM
    per_visit = 2 * BM * d + per_visit_write
    per_head = (4 * N * d + visits * per_visit + (visits - Tr) * per_visit_write
                + 4 * N * d + 8 * N + 2 * N * d + 4 * N)
    return float(heads * per_head)


def bench_kv_outer(args):
    """The K/V-outer forward and fa_fwd on the same workload: time and device bytes."""
    import numpy as np
    import torch

    import exact_io_aware_61_amd as fa
    from exact_io_aware_61_amd.workloads import WORKLOADS, kept_fraction, make_inputs
    w = WORKLOADS[args.workload]
    if w.block_keep is not None:
        print("fwd-kv-outer has no block mask", file=sys.stderr)
        sys.exit(2)
    print(f"[bench] fwd-kv-outer on {w.name}", file=sys.stderr, flush=True)
    q, k, v, _, _ = make_inputs(w, with_do=False)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(qg)
    lse = torch.empty((w.B, w.H, w.N), device=qg.device, dtype=torch.float32)
    lib = fa.load()
    n = ctypes.c_size_t()
    lib.fa_fwd_kv_outer_workspace_size(w.B, w.H, w.N, w.d, ctypes.byref(n))
    ws = torch.empty(max(n.value, 16), device=qg.device, dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    mask = None
    if w.causal:
        mask_s = fa._binding.FaMask(fa.FA_MASK_CAUSAL, fa.MASK_BLOCK_SIZE, None, 0)
        mask = ctypes.byref(mask_s)

    def kvo():
        rc = lib.fa_fwd_kv_outer(P(qg), P(kg), P(vg), P(o), P(lse), w.B, w.H, w.N, w.d, w.scale,
                                 1 if w.causal else 0, P(ws), ws.numel(), sp)
        if rc != 0:
            raise fa.FaError(rc, fa.strerror(rc))

    def fwd():
        rc = lib.fa_fwd(P(qg), P(kg), P(vg), P(o), P(lse), w.B, w.H, w.N, w.d, w.scale, mask, sp)
        if rc != 0:
            raise fa.FaError(rc, fa.strerror(rc))

    def timed(f):
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record(stream)
        for i in range(args.steps):
            f()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]))

    t_kvo = timed(kvo)
    t_fwd = timed(fwd)
    rho = kept_fraction(w.N, w.causal, None)
    flop = 4.0 * w.B * w.H * w.N * w.N * w.d * rho
    heads = w.B * w.H
    model_kvo = kv_outer_io_model(w.N, w.d, w.causal, heads)
    br = fwd_rows_per_workgroup(w.d, False)
    model_fwd = heads * (4 * w.N * w.d + 4 * w.N * w.d * (-(-w.N // br)) * rho + 4 * w.N)
    result = {
        "metric": "forward TFLOP/s, K/V-outer loop order", "value": round(flop / t_kvo / 1e9, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_kvo, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal},
        "kv_outer_ms": round(t_kvo, 4), "fa_fwd_ms": round(t_fwd, 4),
        "io_model_bytes": {"kv_outer": model_kvo, "fa_fwd_tile_model": model_fwd},
        "roofline": None, "cpu_baseline": None, "src": source_digest(),
    }
    print(json.dumps(result), flush=True)


def naive_io_model(N: int, d: int, masked: bool, heads: int) -> dict:
    """Device bytes of the materialised standard attention, counted from its passes.

    Per head (bf16): K^T made contiguous (read and write K), Q scaled (read and
    write Q), S = Q K^T (read Q, K^T; write S), the mask applied in place (read
    and write S), P = softmax(S) (read S, write P), O = P V (read P, V; write O).
    The S and P terms are the Theta(N^2) of standard attention; the mask pass
    reads a [N, N] bool shared by all heads, not counted here.
    """
    nd, nn = 2 * N * d, 2 * N * N
    per_head = (2 * nd) + (2 * nd) + (2 * nd + nn) + (2 * nn if masked else 0) + 2 * nn \
        + (nn + 2 * nd)
    return {"naive_model": float(heads * per_head),
            "naive_s_p_bytes": float(heads * (nn * (5 if masked else 3)))}


def bench_naive(args):
    """Standard attention with S and P in device memory, and fa_fwd, on one workload.

    One naive step: K^T made contiguous, Q scaled, S = Q K^T (bf16 out), the
    causal or block mask written into S as -inf, P = softmax(S) (bf16), O = P V.
    Both paths are timed with HIP events on the stream they run on. The naive
    O is compared with fa_fwd's O (max abs difference, reported).
    """
    import numpy as np
    import torch

    import exact_io_aware_61_amd as fa
    from exact_io_aware_61_amd.workloads import WORKLOADS, kept_fraction, make_inputs, variant
    w = WORKLOADS[args.workload]
    if args.block_keep is not None or args.causal:
        w = variant(w, block_keep=args.block_keep, causal=True if args.causal else None)
    print(f"[bench] naive vs fa_fwd on {w.name}", file=sys.stderr, flush=True)
    q, k, v, _, bm = make_inputs(w, with_do=False)
    dev = torch.device("cuda:0")
    qg, kg, vg = (t.to(dev) for t in (q, k, v))
    # The mask as a dense [N, N] bool (True = dropped), built on the CPU and
    # copied once: an input of the naive path, like the block grid of fa_fwd.
    drop = None
    if w.causal or bm is not None:
        dm = torch.zeros((w.N, w.N), dtype=torch.bool)
        if w.causal:
            dm |= torch.ones((w.N, w.N), dtype=torch.bool).triu(1)
        if bm is not None:
            full = torch.from_numpy(bm).bool().repeat_interleave(128, 0).repeat_interleave(128, 1)
            dm |= ~full[:w.N, :w.N]
        drop = dm.to(dev)
    stream = torch.cuda.current_stream(dev)

    def naive():
        kt = kg.transpose(-1, -2).contiguous()
        s = torch.matmul(qg * w.scale, kt)
        if drop is not None:
            s.masked_fill_(drop, float("-inf"))
        pm = torch.softmax(s, dim=-1)
        del s
        return torch.matmul(pm, vg)

    o = torch.empty_like(qg)
    lse = torch.empty((w.B, w.H, w.N), device=dev, dtype=torch.float32)
    grid = None if bm is None else torch.from_numpy(bm).to(dev)

    def flash():
        fa.forward(qg, kg, vg, causal=w.causal, block_mask=grid, scale=w.scale, out=o, lse=lse)

    def timed(f, steps, warmup):
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            f()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]))

    t_naive = timed(naive, args.steps, args.warmup)
    print(f"[bench] naive {t_naive:.4f} ms", file=sys.stderr, flush=True)
    t_fa = timed(flash, args.steps, args.warmup)
    print(f"[bench] fa_fwd {t_fa:.4f} ms", file=sys.stderr, flush=True)
    o_naive = naive()
    torch.cuda.synchronize()
    diff = float((o_naive.float().cpu() - o.float().cpu()).abs().max())
    rho = kept_fraction(w.N, w.causal, bm)
    flop = 4.0 * w.B * w.H * w.N * w.N * w.d * rho
    heads = w.B * w.H
    br = fwd_rows_per_workgroup(w.d, bm is not None)
    io = naive_io_model(w.N, w.d, drop is not None, heads)
    io["fa_fwd_compulsory"] = float(heads * (8 * w.N * w.d + 4 * w.N))
    io["fa_fwd_tile_model"] = float(heads * (4 * w.N * w.d + 4 * w.N * w.d * (-(-w.N // br)) * rho
                                             + 4 * w.N))
    result = {
        "metric": "attention forward TFLOP/s, standard attention with S and P in HBM",
        "value": round(flop / (t_naive * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_naive, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "mask": "causal" if w.causal else ("block" if bm is not None else "none"),
                   "rho": round(rho, 6)},
        "naive_ms": round(t_naive, 4), "fa_fwd_ms": round(t_fa, 4),
        "fa_fwd_tflops": round(flop / (t_fa * 1e-3) / 1e12, 2),
        "speedup_fa_fwd": round(t_naive / t_fa, 2), "max_abs_diff_o": diff,
        "io_model_bytes": io, "roofline": None, "cpu_baseline": None, "src": source_digest(),
    }
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): attention heads are independent, so a multi-GPU run would be one "
              f"single-GPU run per head shard with no exchange between them.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_io_aware_61_amd as fa
    from exact_io_aware_61_amd.workloads import WORKLOADS, kept_fraction, make_inputs, variant

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (none visible)", file=sys.stderr)
        sys.exit(1)
    if args.probe == "copy":
        probe_copy(args.probe_mib, args.steps)
        return
    if args.kernel == "softmax":
        bench_softmax(args)
        return
    if args.kernel == "decode":
        bench_decode(args)
        return
    if args.kernel == "fwd-kv-outer":
        bench_kv_outer(args)
        return
    if args.kernel == "naive":
        bench_naive(args)
        return

    lib = fa.load()
    w = WORKLOADS[args.workload]
    if args.block_keep is not None or args.causal:
        w = variant(w, block_keep=args.block_keep, causal=True if args.causal else None)
    dev = torch.device("cuda:0")
    print(f"[bench] workload {w.name} B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} "
          f"block_keep={w.block_keep}", file=sys.stderr, flush=True)
    q, k, v, do, bm = make_inputs(w)
    qg, kg, vg, dog = (t.to(dev) for t in (q, k, v, do))
    o = torch.empty_like(qg)
    lse = torch.empty((w.B, w.H, w.N), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    ws = fa.workspace(qg)
    kind = fa.FA_MASK_CAUSAL if w.causal else 0
    grid = None
    if bm is not None:
        grid = torch.from_numpy(bm).to(dev)
        kind |= fa.FA_MASK_BLOCK
    mask = None
    if kind:
        mask_s = fa._binding.FaMask(kind, fa.MASK_BLOCK_SIZE,
                                    None if grid is None else grid.data_ptr(), 0)
        mask = ctypes.byref(mask_s)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    B, H, N, d, sc = w.B, w.H, w.N, w.d, ctypes.c_float(w.scale)
    wsn = ctypes.c_size_t(ws.numel())

    def check(rc):
        if rc != 0:
            raise fa.FaError(rc, fa.strerror(rc))

    def fwd():
        check(lib.fa_fwd(P(qg), P(kg), P(vg), P(o), P(lse), B, H, N, d, sc, mask, sp))

    def pre():
        check(lib.fa_bwd_preprocess(P(o), P(dog), P(lse), B, H, N, d, P(ws), wsn, sp))

    def dkdv():
        check(lib.fa_bwd_dkdv(P(qg), P(kg), P(vg), P(dog), P(dk), P(dv), B, H, N, d, sc,
                              mask, P(ws), wsn, sp))

    def dqk():
        check(lib.fa_bwd_dq(P(qg), P(kg), P(vg), P(dog), P(dq), B, H, N, d, sc, mask,
                            P(ws), wsn, sp))

    stages = [("fa_fwd_kernel", fwd), ("fa_bwd_pre_kernel", pre),
              ("fa_bwd_dkdv_kernel", dkdv), ("fa_bwd_dq_kernel", dqk)]

    for i in range(args.warmup):
        for _, f in stages:
            f()
        print(f"[bench] warmup step {i + 1}/{args.warmup}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        ev[s][0].record(stream)
        for j, (_, f) in enumerate(stages):
            f()
            ev[s][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] timed {K} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    times = {name: np.array([ev[s][j].elapsed_time(ev[s][j + 1]) for s in range(K)])
             for j, (name, _) in enumerate(stages)}
    per = {name: float(t.mean()) for name, t in times.items()}
    spread = {name: {"mean": round(float(t.mean()), 4), "median": round(float(np.median(t)), 4),
                     "p10": round(float(np.percentile(t, 10)), 4),
                     "p90": round(float(np.percentile(t, 90)), 4)}
              for name, t in times.items()}
    fwd_ms = per["fa_fwd_kernel"]
    bwd_ms = sum(per[n] for n, _ in stages[1:])
    rho = kept_fraction(w.N, w.causal, bm)
    fwd_flop = 4.0 * w.B * w.H * w.N * w.N * w.d * rho
    step_flop = 3.5 * fwd_flop
    ms_per_step = wall / K * 1e3
    value = step_flop / (ms_per_step * 1e-3) / 1e12

    # Algorithmic FLOPs per kernel: the dK/dV kernel's four products (S, dP, dV,
    # dK) and the dQ kernel's dQ product count; the dQ kernel's recompute of S
    # and dP is not counted, so the two sum to the backward's five products.
    kernel_flop = {"fa_fwd_kernel": fwd_flop, "fa_bwd_dkdv_kernel": 2.0 * fwd_flop,
                   "fa_bwd_dq_kernel": 0.5 * fwd_flop}
    dom = max(kernel_flop, key=lambda n: per[n])
    achieved = kernel_flop[dom] / (per[dom] * 1e-3) / 1e12
    digest = source_digest()
    rec = traffic_record(dom, w.name, kernel_digest(dom))
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": None if rec is None else rec["bytes_per_launch"],
                "avg_launch_ms": round(per[dom], 4), "flop_per_launch": kernel_flop[dom]}

    # IO accounting in bytes per launch of each pass: the compulsory traffic (every
    # tensor read or written once) and the tile model (the streamed operand re-read
    # by every workgroup that visits it: the Theta(N^2 d^2 / M) term).
    heads = w.B * w.H
    io = pass_io_models(w.N, w.d, w.causal, bm, heads)

    fwd_tf = fwd_flop / (fwd_ms * 1e-3) / 1e12
    fb_ms = fwd_ms + bwd_ms
    fb_tf = step_flop / (fb_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "mask": "causal" if w.causal else ("block" if bm is not None else "none"),
                   "block_keep": w.block_keep, "rho": round(rho, 6), "scale": w.scale},
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(fwd_tf, 2),
                "frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4)},
        "fwd_bwd": {"ms": round(fb_ms, 4), "tflops": round(fb_tf, 2),
                    "frac_of_peak": round(fb_tf / PEAK_BF16_TFLOPS, 4)},
        "kernel_ms": {n: round(t, 4) for n, t in per.items()},
        "kernel_ms_spread": spread,
        "roofline": roofline,
        "io_bytes": {k: (int(v) if k != "rows_per_workgroup_fwd" else v) for k, v in io.items()},
        "device": device_info(lib, dev.index or 0),
        "src": digest,
    }
    if args.cpu_seconds > 0:
        print(f"[bench] cpu baseline: oracle on whole heads for ~{args.cpu_seconds} s",
              file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, do, bm, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
