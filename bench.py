#!/usr/bin/env python3
"""Monarch forward+backward throughput on one MI355X.

One step = monarch_fwd + monarch_bwd (the whole hot path) over one batch of
synthetic inputs already resident in HBM. Prints one JSON line with the
throughput (Monarch algorithmic TFLOP/s = 6*batch*params per step, timed
over eager steps with no events between kernels), the roofline of the
dominant kernel (timed with HIP events recorded between the library's
kernels on the launch stream, over a second run of the same steps), the step
replayed from a HIP graph (checked bit for bit against the eager step), the
dense bf16 GEMM of the same shape and the fp64 CPU oracle timed on a bounded
sample.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA, published
# fp32 on the vector ALU without packed instructions: 256 CUs x 4 SIMDs x 16
# lanes x 2 flops (FMA) x 2.4 GHz
FP32_VALU_PEAK_TFLOPS = 78.6

DEFAULT_WORKLOAD = "square_n16384_b128"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def csrc_digest() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "monarch_block_diagonal_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_bytes(name: str, pr: dict) -> float:
    """Algorithmic HBM bytes of one launch: each tensor the kernel's role needs
    read once and each result written once (weights and weight gradients at
    the I/O width; partial sums are not counted)."""
    e, B = pr["e"], pr["batch"]
    inp, mid, out = pr["in"], pr["mid"], pr["out"]
    p1, p2 = pr["params1"], pr["params2"]
    relu = pr["act"] == 1
    table = {
        "stage1_fwd": e * B * (inp + mid) + e * p1,
        "stage2_fwd": e * B * (mid + out) + e * p2,
        "stage2_bwd_data": e * B * (out * (2 if relu else 1) + mid) + e * p2,
        "stage2_bwd_weight": e * B * (out * (2 if relu else 1) + mid) + e * p2,
        "stage2_bwd": e * B * (out * (2 if relu else 1) + 2 * mid) + 2 * e * p2,
        "stage1_bwd_data": e * B * (mid + inp) + e * p1,
        "stage1_bwd_weight": e * B * (mid + inp) + e * p1,
        "stage1_bwd": e * B * (mid + 2 * inp) + 2 * e * p1,
        # square fast path: the dV pass (dY, and Y for the ReLU mask, ->
        # block-major dV) is a layout pass with no algorithmic bytes of its
        # own (its traffic is overhead against the two-pass count); both
        # stage-2 backward kernels then read dV in place of dY
        "sq128_dv_panels": 0.0,
        "sq128_stage2_bwd_data": e * B * (out + mid) + e * p2,
        "sq128_stage2_bwd_weight": e * B * (out + mid) + e * p2,
        # fused 32x32-block path: x -> z, y; dY (and Y for the ReLU mask) ->
        # dX, plus dV and dZ for the weight-gradient GEMMs
        "sm32_fwd": e * B * (inp + mid + out) + e * (p1 + p2),
        "sm32_bwd_data": e * B * (out * (2 if relu else 1) + out + mid + inp) + e * (p1 + p2),
        "sm32_bwd_weight": e * B * (out + 2 * mid + inp),
        "reduce_dw": e * (p1 + p2),
    }
    for key in sorted(table, key=len, reverse=True):
        if name.endswith(key):
            return float(table[key])
    return 0.0


def kernel_flops(name: str, pr: dict) -> float:
    """Algorithmic flops of one launch (2 per multiply-add of the Monarch
    products the kernel's role computes)."""
    B, p1, p2 = pr["batch"], pr["params1"], pr["params2"]
    table = {
        "stage1_fwd": 2 * B * p1, "stage2_fwd": 2 * B * p2,
        "stage2_bwd_data": 2 * B * p2, "stage2_bwd_weight": 2 * B * p2, "stage2_bwd": 4 * B * p2,
        "stage1_bwd_data": 2 * B * p1, "stage1_bwd_weight": 2 * B * p1, "stage1_bwd": 4 * B * p1,
        "sm32_fwd": 2 * B * (p1 + p2), "sm32_bwd_data": 2 * B * (p1 + p2),
        "sm32_bwd_weight": 2 * B * (p1 + p2),
    }
    for key in sorted(table, key=len, reverse=True):
        if name.endswith(key):
            return float(table[key])
    return 0.0


def measure_stream_copy(torch, dev, reps: int = 10, nbytes: int = 1 << 30) -> float:
    """GB/s of the library's stream copy (2 * nbytes moved per call), timed
    with HIP events on the launch stream."""
    import monarch_block_diagonal_amd as M
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        M.monarch_stream_copy(src, dst, nbytes, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        M.monarch_stream_copy(src, dst, nbytes, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def measure_gemm_peak(torch, dev, dtype: str, reps: int = 10, n: int = 8192) -> float:
    """TFLOP/s of a large square GEMM (n x n x n) through torch's library GEMM
    (hipBLASLt) in the workload's dtype, timed with HIP events: the measured
    matrix-core reference beside the spec peak."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    a = torch.randn((n, n), device=dev, dtype=torch.float32).to(tdt)
    b = torch.randn((n, n), device=dev, dtype=torch.float32).to(tdt)
    c = torch.empty((n, n), device=dev, dtype=tdt)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        torch.matmul(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def load_traffic(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, or None
    when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("csrc_sha256") != digest:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, rows: int):
    """The fp64 oracle as it stands, on `rows` rows of the same workload."""
    import numpy as np
    import oracle as O
    from monarch_block_diagonal_amd import synthetic as S
    ins = [S.make_layer_inputs(w, li, batch=rows) for li in range(len(w.layers))]
    chain = [(d["w1"], d["w2"], l.in_features, l.out_features, l.relu)
             for d, l in zip(ins, w.layers)]
    x, dy = ins[0]["x"], ins[0]["dy"]
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    general = [l for l in w.layers if l.mid != l.out_features or l.bias
               or l.in_features % l.nblocks1 or l.out_features % l.nblocks2]
    t0 = time.perf_counter()
    if general:
        # one general layer (explicit mid, padding, bias): the MonarchLinear-variant oracle
        from oracle import monarch_linear as ML
        l, d = w.layers[0], ins[0]
        bias = d.get("bias")
        y = ML.forward_ex(x, d["w1"], d["w2"], l.in_features, l.out_features, l.mid, bias)
        dx = ML.backward_ex(dy, x, d["w1"], d["w2"], l.in_features, l.out_features, l.mid, bias)[0]
    else:
        y, _ = O.mlp_forward(x, chain)
        dx, _ = O.mlp_backward(dy, x, chain)
    dt = time.perf_counter() - t0
    flops = 6.0 * rows * w.params
    assert np.isfinite(y).all() and np.isfinite(dx).all()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} of {w.batch} rows of {w.name}: fp64 forward+backward through "
                      f"dense factor matrices (built in the timed call), {dt:.2f} s",
            "seconds": dt}


def bench_project(args) -> int:
    """Dense -> Monarch projection of an n x n bf16 matrix (n = 16384, 128
    blocks of 128 x 128 per factor: 16384 slices of 128 x 128), inputs
    resident in HBM; one JSON line."""
    import numpy as np
    import torch
    import monarch_block_diagonal_amd as M
    from monarch_block_diagonal_amd import synthetic as S
    n, b = 16384, 128
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q = n // b
    log(f"projection: {n} x {n} bf16, {b} x {b} slices of {q} x {q}, "
        f"at most {args.max_steps} products per slice")
    g = torch.Generator(device=dev)
    g.manual_seed(S.seed_for(4, S.TID_X) + 99)
    m = torch.randn((n, n), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    w1 = torch.empty((b, b, q), dtype=torch.bfloat16, device=dev)
    w2 = torch.empty((b, q, b), dtype=torch.bfloat16, device=dev)
    status = torch.empty((b * b,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def run():
        M.monarch_project(m, w1, w2, n, n, b, b, M.BF16, args.max_steps, status, stream)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(K):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / K
    ms = e0.elapsed_time(e1) / K
    # work per slice: each product with AᵀA is u = A v, w = Aᵀ u on the vector
    # ALU, 4 q² flops (2 per multiply-add); the status array holds the products
    # each slice used. The reorthogonalisation (8 (j+1) q flops at step j) and
    # the small tridiagonal solves are not counted.
    st = status.cpu().numpy()
    converged = int((st > 0).sum())
    products = float(st[st > 0].sum())
    flops = 4.0 * q * q * products
    hbm = 2.0 * n * n + 2 * 2.0 * b * b * q
    tflops = flops / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import monarch_projection as PJ
        ns = 2048
        mh = m[:, : (ns // b) * q].float().cpu().numpy().astype(np.float64)   # slices r < ns/b
        log(f"cpu baseline: oracle fit of {ns} of {b * b} slices")
        t1 = time.perf_counter()
        sl = PJ.slices(np.ascontiguousarray(mh), (ns // b) * q, n, ns // b, b)
        for gg in range(b):
            for rr in range(ns // b):
                PJ.fit_slice(sl[gg, rr])
        dt = time.perf_counter() - t1
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            threads = len(os.sched_getaffinity(0))
        cpu = {"value": round(ns / dt, 1), "unit": "slices/s", "cores": int(threads),
               "kind": "oracle",
               "sample": f"{ns} of {b * b} slices ({q} x {q}, fp64 SVD each), {dt:.2f} s",
               "seconds": dt}
    result = {
        "metric": "Monarch projection slices/s", "value": round(b * b / (ms * 1e-3), 1),
        "unit": "slices/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "wall_ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) matrix drawn on the device, stored bf16)",
        "config": {"workload": f"project_n{n}_b{b}", "n": n, "nblocks": b,
                   "max_steps": args.max_steps, "input": "bf16", "compute": "fp32"},
        "converged_slices": converged, "products_per_slice": round(products / max(converged, 1), 2),
        "roofline": {"bound": "alu", "achieved": round(tflops, 2), "peak": FP32_VALU_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / FP32_VALU_PEAK_TFLOPS, 4),
                     "traffic": None, "hbm_bytes": hbm,
                     "hbm_frac": round(hbm / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_hyper(args) -> int:
    """k-factor (hypercube) layer: forward + backward over a lattice (default
    the page's 16 x 24 x 32 = 12288 units) at `--rows` tokens, inputs resident
    in HBM; one JSON line."""
    import numpy as np
    import torch
    import monarch_block_diagonal_amd as M
    from monarch_block_diagonal_amd import synthetic as S
    dims = tuple(int(v) for v in args.dims.split("x"))
    N = int(np.prod(dims))
    B = args.rows
    bf16 = args.dtype == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32
    code = M.BF16 if bf16 else M.F32
    e = 2 if bf16 else 4
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    params = N * sum(dims)
    log(f"hypercube {dims} (N={N}, {params} params), {B} rows, {args.dtype}")
    g = torch.Generator(device=dev)
    g.manual_seed(S.seed_for(5, S.TID_X))
    x = torch.randn((B, N), generator=g, device=dev).to(tdt)
    dy = torch.randn((B, N), generator=g, device=dev).to(tdt)
    ws = [torch.randn((N // d, d, d), generator=g, device=dev).mul_(d ** -0.5).to(tdt) for d in dims]
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    dws = [torch.empty_like(w) for w in ws]
    saved = torch.empty((max(M.monarch_hyper_saved_elems(dims, B), 1),), dtype=tdt, device=dev)
    need = M.monarch_hyper_bwd_workspace_bytes(dims, B, code)
    wsb = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    fn = M.monarch_hyper_describe(0, dims, B, code)
    bn = M.monarch_hyper_describe(1, dims, B, code)
    stream = torch.cuda.current_stream()

    def step(evf=None, evb=None):
        M.monarch_hyper_fwd(x, ws, y, saved, dims, B, code, stream, events=evf)
        M.monarch_hyper_bwd(dy, x, ws, saved, dx, dws, wsb, need, dims, B, code, stream, events=evb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fn) + 1)] for _ in range(K)]
    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(len(bn) + 1)] for _ in range(K)]
    t0 = time.perf_counter()
    for k in range(K):
        step(evf[k], evb[k])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    step_ms = sorted(evf[k][0].elapsed_time(evb[k][-1]) for k in range(K))
    kern = {}
    for names, evs, pre in ((fn, evf, "fwd"), (bn, evb, "bwd")):
        for i, nm in enumerate(names):
            key = f"{pre}{i}:{nm}"
            kern[key] = sum(ev[i].elapsed_time(ev[i + 1]) for ev in evs) / K
    flops = 6.0 * B * params
    value = flops / (ms * 1e-3) / 1e12
    # every round reads its input and writes its output once (fwd), the
    # backward reads two tensors per weight product and one + writes one per
    # data product; weights and gradients once
    act = e * B * N
    bytes_step = len(dims) * 2 * act + len(dims) * (2 * act + 2 * act) + 3 * e * params
    dom = max(kern, key=kern.get)
    dom_bytes = 2.0 * act + e * params / len(dims)
    achieved = dom_bytes / (kern[dom] * 1e-3) / 1e9
    dense = None
    if not args.no_dense:
        Wd = torch.randn((N, N), device=dev).mul_(N ** -0.5).to(tdt)

        def dense_step():
            yd = x @ Wd.t()
            return yd, dy @ Wd, dy.t() @ x
        for _ in range(2):
            dense_step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(3):
            dense_step()
        torch.cuda.synchronize()
        dms = (time.perf_counter() - t1) * 1e3 / 3
        dense = {"dtype": args.dtype, "ms_per_step": round(dms, 4),
                 "tflops": round(6.0 * B * N * N / (dms * 1e-3) / 1e12, 1),
                 "speedup_monarch_vs_dense": round(dms / ms, 3)}
        del Wd
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import monarch_hypercube as H
        rows = args.cpu_rows or 256
        xs, dys = x[:rows].float().cpu().numpy(), dy[:rows].float().cpu().numpy()
        wn = [w.float().cpu().numpy() for w in ws]
        t1 = time.perf_counter()
        H.forward_fibers(xs, wn, dims)
        H.backward_fibers(dys, xs, wn, dims)
        dt = time.perf_counter() - t1
        cpu = {"value": round(6.0 * rows * params / dt / 1e12, 5), "unit": "TFLOP/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{rows} of {B} rows, fp64 fiber-by-fiber rounds, {dt:.2f} s",
               "seconds": dt}
    result = {
        "metric": "hypercube Monarch fwd+bwd TFLOP/s", "value": round(value, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": args.dtype, "data": "synthetic (seeded, drawn on the device)",
        "config": {"workload": f"hypercube_{args.dims}_rows{B}", "dims": list(dims), "N": N,
                   "rows": B, "params": params},
        "step_ms_p10_p50_p90": [round(step_ms[int(q * (K - 1))], 4) for q in (0.1, 0.5, 0.9)],
        "step_hbm_frac": round(bytes_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernels_ms": {k: round(v, 4) for k, v in kern.items()},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes": dom_bytes, "avg_ms": round(kern[dom], 4)},
        "dense_baseline": dense, "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_dyad(args) -> int:
    """DYAD-style layer (two block-sparse terms) forward + backward at
    `--n` x `--n`, `--nb` blocks, `--rows` tokens; one JSON line."""
    import torch
    import monarch_block_diagonal_amd as M
    n, nb, B = args.n, args.nb, args.rows
    bf16 = args.dtype == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32
    code = M.BF16 if bf16 else M.F32
    e = 2 if bf16 else 4
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q = n // nb
    log(f"dyad n={n} nb={nb} rows={B} {args.dtype}")
    g = torch.Generator(device=dev)
    g.manual_seed(20220401 + 600)
    x = torch.randn((B, n), generator=g, device=dev).to(tdt)
    dy = torch.randn((B, n), generator=g, device=dev).to(tdt)
    wa = torch.randn((nb, q, q), generator=g, device=dev).mul_((2 * q) ** -0.5).to(tdt)
    wb = torch.randn((nb, q, q), generator=g, device=dev).mul_((2 * q) ** -0.5).to(tdt)
    y, dx, dwa, dwb = torch.empty_like(x), torch.empty_like(x), torch.empty_like(wa), torch.empty_like(wb)
    need = M.monarch_dyad_bwd_workspace_bytes(n, n, nb, B, code)
    need_f = M.monarch_dyad_fwd_workspace_bytes(n, n, nb, B, code)
    ws = torch.empty((max(need, need_f, 1),), dtype=torch.uint8, device=dev)
    fn = M.monarch_dyad_describe(0, n, n, nb, B, code)
    bn = M.monarch_dyad_describe(1, n, n, nb, B, code)
    stream = torch.cuda.current_stream()

    def step(evf=None, evb=None):
        M.monarch_dyad_fwd(x, wa, wb, y, ws, need_f, n, n, nb, B, code, stream, events=evf)
        M.monarch_dyad_bwd(dy, x, wa, wb, dx, dwa, dwb, ws, need, n, n, nb, B, code, stream,
                           events=evb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fn) + 1)] for _ in range(K)]
    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(len(bn) + 1)] for _ in range(K)]
    t0 = time.perf_counter()
    for k in range(K):
        step(evf[k], evb[k])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    kern = {}
    for names, evs in ((fn, evf), (bn, evb)):
        for i, nm in enumerate(names):
            kern[nm] = sum(ev[i].elapsed_time(ev[i + 1]) for ev in evs) / K
    params = 2 * nb * q * q
    flops = 6.0 * B * params
    act = e * B * n
    # fwd: x read twice, y written and read back once; bwd: dy and x read
    # twice each (two weight products), dy twice and dx twice (data products)
    bytes_step = 4 * act + 8 * act + 3 * e * params
    dense = None
    if not args.no_dense:
        Wd = torch.randn((n, n), device=dev).mul_(n ** -0.5).to(tdt)

        def dense_step():
            return x @ Wd.t(), dy @ Wd, dy.t() @ x
        for _ in range(2):
            dense_step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(3):
            dense_step()
        torch.cuda.synchronize()
        dms = (time.perf_counter() - t1) * 1e3 / 3
        dense = {"dtype": args.dtype, "ms_per_step": round(dms, 4),
                 "speedup_dyad_vs_dense": round(dms / ms, 3)}
    result = {
        "metric": "DYAD fwd+bwd TFLOP/s", "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": args.dtype, "data": "synthetic (seeded, drawn on the device)",
        "config": {"workload": f"dyad_n{n}_nb{nb}_rows{B}", "n": n, "nblocks": nb, "rows": B,
                   "params": params},
        "step_hbm_frac": round(bytes_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernels_ms": {k: round(v, 4) for k, v in kern.items()},
        "dense_baseline": dense,
    }
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time the stream copy with 3 calls only (counter runs: the copy's "
                         "FETCH_SIZE / WRITE_SIZE per call calibrate the HBM counters)")
    ap.add_argument("--op", choices=("step", "project", "hyper", "dyad"), default="step",
                    help="step: forward + backward (default); project: dense -> Monarch "
                         "projection of an n x n matrix; hyper: k-factor lattice layer; "
                         "dyad: DYAD-style two-term layer")
    ap.add_argument("--n", type=int, default=4096, help="features of --op dyad")
    ap.add_argument("--nb", type=int, default=16, help="blocks of --op dyad")
    ap.add_argument("--dims", default="16x24x32", help="lattice of --op hyper")
    ap.add_argument("--rows", type=int, default=16384, help="tokens of --op hyper / dyad")
    ap.add_argument("--dtype", choices=("bf16", "f32"), default="bf16",
                    help="dtype of --op hyper / dyad")
    ap.add_argument("--max-steps", type=int, default=256,
                    help="products with AᵀA each slice may use (--op project)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the Monarch path here has no multi-GPU "
              "(sharded) implementation, so --gpus must be 1.", file=sys.stderr)
        return 2
    if args.op == "project":
        return bench_project(args)
    if args.op == "hyper":
        return bench_hyper(args)
    if args.op == "dyad":
        return bench_dyad(args)

    import numpy as np
    import torch
    import monarch_block_diagonal_amd as M
    from monarch_block_diagonal_amd import synthetic as S

    w = S.WORKLOADS[args.workload]
    dt_code = M.BF16 if w.dtype == "bf16" else M.F32
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    e = 2 if w.dtype == "bf16" else 4
    B = w.batch
    layers = w.layers
    multi = len(layers) > 1

    log(f"workload {w.name}: " + ", ".join(
        f"in={l.in_features} out={l.out_features} b1={l.nblocks1} b2={l.nblocks2}"
        f"{' +relu' if l.relu else ''}" for l in layers) + f"; batch={B} {w.dtype}")

    # seeded synthetic inputs drawn on the device (same distributions as the
    # parity tests' host draws)
    def draw(seed, shape, dist, var):
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        if dist == "normal":
            t = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
            if var != 1.0:
                t.mul_(var ** 0.5)
        else:
            t = torch.rand(shape, generator=g, device=dev, dtype=torch.float32)
        return t.to(tdt)

    x = draw(S.seed_for(w.cfg, S.TID_X), (B, layers[0].in_features), w.x_dist, w.x_var)
    dy = draw(S.seed_for(w.cfg, S.TID_DY), (B, layers[-1].out_features), "normal", w.dy_var)
    L = []
    wsb = 0
    for li, l in enumerate(layers):
        t1, t2 = (S.TID_W1, S.TID_W2) if li == 0 else (S.TID_W1_L2, S.TID_W2_L2)
        vr, vl = w.w_var[li]
        fi, fo, mid = l.in_features, l.out_features, l.mid
        d = {"l": l, "fi": fi, "fo": fo, "mid": mid,
             "w1": draw(S.seed_for(w.cfg, t1), l.w1_shape, "normal", vr),
             "w2": draw(S.seed_for(w.cfg, t2), l.w2_shape, "normal", vl),
             "y": torch.empty((B, fo), dtype=tdt, device=dev),
             "z": torch.empty((B, mid), dtype=tdt, device=dev),
             "bias": (draw(S.seed_for(w.cfg, S.TID_BIAS + 10 * li), (fo,), "normal", 0.25)
                      if l.bias else None),
             "dx": torch.empty((B, fi), dtype=tdt, device=dev),
             "act": M.ACT_RELU if l.relu else M.ACT_NONE,
             "fn": M.monarch_describe_ex(0, fi, fo, mid, l.nblocks1, l.nblocks2, B, dt_code,
                                         M.ACT_RELU if l.relu else M.ACT_NONE, l.bias),
             "bn": M.monarch_describe_ex(1, fi, fo, mid, l.nblocks1, l.nblocks2, B, dt_code,
                                         M.ACT_RELU if l.relu else M.ACT_NONE, l.bias)}
        d["dw1"] = torch.empty_like(d["w1"])
        d["dw2"] = torch.empty_like(d["w2"])
        d["db"] = torch.empty_like(d["bias"]) if l.bias else None
        d["x"] = x if li == 0 else L[li - 1]["y"]
        wsb = max(wsb, M.monarch_bwd_ex_workspace_bytes(fi, fo, mid, l.nblocks1, l.nblocks2, B,
                                                        dt_code, l.bias))
        L.append(d)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

    def strm():
        # looked up per call, so that a graph capture sees its capture stream
        return torch.cuda.current_stream()

    def fwd(evs=None):
        for li, d in enumerate(L):
            l = d["l"]
            M.monarch_fwd_ex(d["x"], d["w1"], d["w2"], d["bias"], d["y"], d["z"], d["fi"],
                             d["fo"], d["mid"], l.nblocks1, l.nblocks2, B, dt_code, d["act"],
                             strm(), events=None if evs is None else evs[li])

    def bwd(evs=None):
        g = dy
        for li in range(len(L) - 1, -1, -1):
            d, l = L[li], L[li]["l"]
            M.monarch_bwd_ex(g, d["x"], d["w1"], d["w2"], d["z"],
                             d["y"] if d["act"] == M.ACT_RELU else None, d["dx"], d["dw1"],
                             d["dw2"], d["db"], ws, wsb, d["fi"], d["fo"], d["mid"], l.nblocks1,
                             l.nblocks2, B, dt_code, d["act"], strm(),
                             events=None if evs is None else evs[li])
            g = d["dx"]

    def step(evf=None, evb=None):
        fwd(evf)
        bwd(evb)

    log(f"warmup {args.warmup} steps; kernels " + " | ".join(
        f"fwd={d['fn']} bwd={d['bn']}" for d in L))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def new_events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    K = args.steps
    stream = strm()
    # timed steps: no events between kernels, one pair around each step
    log(f"timing {K} fwd+bwd steps")
    evs_s = new_events(K + 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        evs_s[k].record(stream)
        step()
    evs_s[K].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K
    step_ms = sorted(evs_s[k].elapsed_time(evs_s[k + 1]) for k in range(K))

    # per-kernel times: the same steps again with an event between kernels
    log(f"timing {K} fwd+bwd steps kernel by kernel")
    evf = [[new_events(len(d["fn"]) + 1) for d in L] for _ in range(K)]
    evb = [[new_events(len(d["bn"]) + 1) for d in L] for _ in range(K)]
    for k in range(K):
        step(evf[k], evb[k])
    torch.cuda.synchronize()

    # the whole step captured once as a HIP graph and replayed: the same
    # kernels with the host launch path taken out; the replay's results must
    # equal the eager step's bit for bit
    graph = None
    if not args.no_graph:
        log(f"timing {K} fwd+bwd steps replayed from a HIP graph")
        outs = [d["dx"] for d in L] + [d["dw1"] for d in L] + [d["dw2"] for d in L] + [L[-1]["y"]]
        step()
        torch.cuda.synchronize()
        ref = [t.clone() for t in outs]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip(outs, ref))
        evs_g = new_events(K + 1)
        t0 = time.perf_counter()
        for k in range(K):
            evs_g[k].record(stream)
            g.replay()
        evs_g[K].record(stream)
        torch.cuda.synchronize()
        g_wall = (time.perf_counter() - t0) * 1e3 / K
        g_ms = sorted(evs_g[k].elapsed_time(evs_g[k + 1]) for k in range(K))
        graph = {"ms_per_step": round(g_wall, 4),
                 "step_ms_p50": round(g_ms[len(g_ms) // 2], 4),
                 "value": round(6.0 * B * w.params / (g_wall * 1e-3) / 1e12, 2),
                 "replay_equals_eager": same}
        del g, ref

    def pct(v, q):
        return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]

    log(f"timing {K} forward-only steps")
    evs_f = new_events(K + 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        evs_f[k].record(stream)
        fwd()
    evs_f[K].record(stream)
    torch.cuda.synchronize()
    fwd_wall_ms = (time.perf_counter() - t0) * 1e3 / K
    fwd_ms = sorted(evs_f[k].elapsed_time(evs_f[k + 1]) for k in range(K))

    per_kernel = {}
    prs = {}
    for li, d in enumerate(L):
        l = d["l"]
        pre = f"L{li + 1}:" if multi else ""
        pr = {"e": e, "batch": B, "in": d["fi"], "mid": d["mid"], "out": d["fo"],
              "act": 1 if l.relu else 0,
              "params1": int(np.prod(l.w1_shape)), "params2": int(np.prod(l.w2_shape))}
        for names, evs in ((d["fn"], [ev[li] for ev in evf]), (d["bn"], [ev[li] for ev in evb])):
            for i, nm in enumerate(names):
                ts = [ev[i].elapsed_time(ev[i + 1]) for ev in evs]
                per_kernel[pre + nm] = sum(ts) / len(ts)
                prs[pre + nm] = (nm, pr)
    dom = max(per_kernel, key=per_kernel.get)
    dom_ms = per_kernel[dom]
    dom_name, dom_pr = prs[dom]
    dom_bytes = kernel_bytes(dom_name, dom_pr)
    dom_flops = kernel_flops(dom_name, dom_pr)
    digest = csrc_digest()
    mfma_peak = MFMA_PEAK_TFLOPS[w.dtype]
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if dom_bytes > 0 and dom_flops / dom_bytes > ridge:
        achieved = dom_flops / (dom_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                    "peak": mfma_peak, "unit": "TFLOP/s", "frac": round(achieved / mfma_peak, 4)}
    else:
        achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roofline.update({"traffic": None if multi else load_traffic(dom, w.name, digest),
                     "algorithmic_bytes": dom_bytes, "algorithmic_flops": dom_flops,
                     "avg_ms": round(dom_ms, 4)})

    flops = 6.0 * B * w.params
    value = flops / (ms_per_step * 1e-3) / 1e12
    # whole step against the two-pass algorithmic bytes (each stage reads its
    # input and writes its output once, z saved; weights and gradients once)
    b2p = sum(e * B * (d["fi"] + 2 * d["mid"] + d["fo"]) + e * B * (d["fo"] + 3 * d["mid"] + 2 * d["fi"])
              + 3 * e * d["l"].params for d in L)
    t_roof = max(flops / (mfma_peak * 1e12), b2p / (HBM_PEAK_GBS * 1e9)) * 1e3
    step_roofline = {"binds": "mfma" if flops / (mfma_peak * 1e12) > b2p / (HBM_PEAK_GBS * 1e9)
                     else "hbm", "t_roof_ms": round(t_roof, 4), "bytes_2pass": b2p,
                     "flops": flops, "frac": round(t_roof / ms_per_step, 4)}

    # measured HBM reference: the library's stream copy (read + write of
    # 1 GiB, 3 untimed and 10 timed calls), beside the 8 TB/s spec peak
    copy_gbs = measure_stream_copy(torch, dev, reps=3 if args.copy_probe else 10)
    if args.copy_probe:
        # a second calibration pattern for the counters: the runtime's own
        # device copy of 1 GiB (3 calls)
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # measured matrix-core reference: an 8192^3 GEMM in the workload's dtype
    gemm_tflops = measure_gemm_peak(torch, dev, w.dtype)
    step_roofline["measured_peak_gbs"] = round(copy_gbs, 1)
    step_roofline["measured_mfma_peak_tflops"] = round(gemm_tflops, 1)
    step_roofline["frac_measured"] = round(
        max(flops / (gemm_tflops * 1e12), b2p / (copy_gbs * 1e9)) * 1e3 / ms_per_step, 4)
    if roofline.get("bound") == "hbm":
        roofline["measured_peak"] = round(copy_gbs, 1)
        roofline["frac_measured"] = round(roofline["achieved"] / copy_gbs, 4)
    else:
        roofline["measured_peak"] = round(gemm_tflops, 1)
        roofline["frac_measured"] = round(roofline["achieved"] / gemm_tflops, 4)

    dense = None
    if not args.no_dense:
        log(f"dense {w.dtype} GEMM baseline of the same shapes")
        Wd = [torch.randn((d["fo"], d["fi"]), device=dev, dtype=torch.float32)
              .mul_(d["fi"] ** -0.5).to(tdt) for d in L]

        def dense_step():
            hs = [x]
            for i, Wl in enumerate(Wd):
                h = torch.nn.functional.linear(hs[-1], Wl)
                if L[i]["l"].relu:
                    h = torch.relu(h)
                hs.append(h)
            g = dy
            for i in range(len(Wd) - 1, -1, -1):
                if L[i]["l"].relu:
                    g = g * (hs[i + 1] > 0)
                dw = g.t() @ hs[i]
                g = g @ Wd[i]
            return g, dw
        for _ in range(2):
            dense_step()
        torch.cuda.synchronize()
        reps = 5
        t0 = time.perf_counter()
        for _ in range(reps):
            dense_step()
        torch.cuda.synchronize()
        dense_ms = (time.perf_counter() - t0) * 1e3 / reps
        dflops = sum(6.0 * B * d["fi"] * d["fo"] for d in L)
        dense = {"dtype": w.dtype, "ms_per_step": round(dense_ms, 4),
                 "tflops": round(dflops / (dense_ms * 1e-3) / 1e12, 1),
                 "speedup_monarch_vs_dense": round(dense_ms / ms_per_step, 3)}
        if graph is not None:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                dense_step()
            torch.cuda.current_stream().wait_stream(side)
            gd = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gd):
                dense_step()
            gd.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                gd.replay()
            torch.cuda.synchronize()
            dg_ms = (time.perf_counter() - t0) * 1e3 / reps
            dense["graph_ms_per_step"] = round(dg_ms, 4)
            graph["speedup_monarch_vs_dense"] = round(dg_ms / graph["ms_per_step"], 3)
            del gd
        del Wd

    cpu = None
    if not args.no_cpu_baseline:
        # about 2e13 fp64 flops of dense-factor products (~10-30 s on 16 host cores)
        per_row = sum(20.0 * l.out_features * max(l.in_features, l.out_features) for l in layers)
        rows = args.cpu_rows or min(B, max(8, int(2e13 / per_row)))
        log(f"cpu baseline: oracle on {rows} rows")
        cpu = cpu_baseline(w, rows)

    result = {
        "metric": "Monarch fwd+bwd TFLOP/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded, drawn on the device)",
        "config": {"workload": w.name, "layers": [
            {"in_features": d["fi"], "out_features": d["fo"], "mid_features": d["mid"],
             "nblocks1": d["l"].nblocks1, "nblocks2": d["l"].nblocks2, "relu_after": d["l"].relu,
             "bias": d["l"].bias} for d in L],
            "batch": B, "params": w.params, "passes": "fwd+bwd"},
        "tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "step_ms_p10_p50_p90": [round(pct(step_ms, q), 4) for q in (0.1, 0.5, 0.9)],
        "fwd_ms_per_step": round(fwd_wall_ms, 4),
        "fwd_ms_p10_p50_p90": [round(pct(fwd_ms, q), 4) for q in (0.1, 0.5, 0.9)],
        "fwd_tflops": round(2.0 * B * w.params / (pct(fwd_ms, 0.5) * 1e-3) / 1e12, 2),
        "step_roofline": step_roofline,
        "graph": graph,
        "kernels_ms": {k: round(v, 4) for k, v in per_kernel.items()},
        "roofline": roofline,
        "dense_baseline": dense,
        "cpu_baseline": cpu,
        "csrc_sha256": digest,
    }
    print(json.dumps(result), flush=True)
    return 0

if __name__ == "__main__":
    sys.exit(main())
