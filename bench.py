#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X; prints ONE JSON line on stdout.

A step is one pass over both kernel families on their benchmark inputs:
  * batched fp32: 65536 matrices of 32 x 32, A_b = B_b B_b^T / 32 + I, factor
    (chol_potrf_batched) then adjoint with accumulate (chol_potrf_adjoint_batched);
  * blocked fp64: one 16384 x 16384 matrix A = G G^T / 16384 + 0.1 I, factor
    (chol_potrf, nb = 128) then adjoint with accumulate (chol_potrf_adjoint).
All inputs are built from seeds and resident in HBM before timing starts.

value  = fp64 N=16384 factor+adjoint rate, counting N^3/3 + 2N^3/3 flops, GFLOP/s.
batched.value = fp32 N=32 factor+adjoint rate, matrices/s.
roofline = the blocked kernel family carrying the most algorithmic work (found in
  one untimed step with every family timed; it is the adjoint's symmetric
  product): algorithmic work per launch / average launch time, from HIP events
  that the library records around each launch of that family, on the stream it
  runs on, over the timed steps (chol_profile_start/stop).  kernels = per-family
  times of the untimed step.
roofline.traffic = HBM bytes per launch of that kernel from the committed
  rocprofv3 FETCH_SIZE and WRITE_SIZE runs (profiles/roofline_traffic.md, scaled
  by a plain copy of known size, `--calibrate-copy`); null when no record
  matches the current kernel sources.
cpu_baseline = the plain CPU oracle on a bounded sample of the same inputs.
parity = the GPU outputs against that leg's oracle results: the factor's leading
  block, the adjoint for adj_L supported on that block, all batched factors and
  adjoints (max allclose and relative errors); plus the residual of the full
  factor on sampled rows (torch products on the device).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "potrf fwd+adjoint GFLOP/s (fp64 N=16384) and batched matrices/s (fp32 N=32)"
PEAK_FP64_TFLOPS = 78.6
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
FAMILIES = ["small_factor", "small_adjoint", "diag_factor", "diag_inverse", "panel_solve",
            "trailing_update", "adj_trailing", "adj_panel", "adj_diag_update", "adj_diag", "elementwise",
            "reduce"]
BYTE_FAMILIES = {"small_factor", "small_adjoint", "elementwise", "reduce"}
# the kernel each matrix-core family launches (names as rocprofv3 lists them)
FAMILY_KERNEL = {"trailing_update": "k_gemm<double, 0, 0, 1, 1, 128, 128>", "adj_trailing": "k_gemm<double, 4, 1, 3, 0, 128, 128>",
                 "panel_solve": "k_gemm<double, 0, 0, 2, 0, 32, 128>", "adj_panel": "k_gemm<double, 0, 1, 2, 0, 32, 128>",
                 "adj_diag_update": "k_gemm<double, 1, 1, 3, 0, 128, 128>", "adj_diag": "k_tile_adjoint_stage<double, 0..3>"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def profile_stop(lib):
    k = len(FAMILIES)
    cnt = (ctypes.c_int64 * k)()
    ms = (ctypes.c_double * k)()
    work = (ctypes.c_double * k)()
    lib.chol_profile_stop.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    st = lib.chol_profile_stop(k, ctypes.byref(cnt), ctypes.byref(ms), ctypes.byref(work))
    if st != 0:
        raise RuntimeError("chol_profile_stop failed")
    return {FAMILIES[i]: {"launches": int(cnt[i]), "ms": float(ms[i]), "work": float(work[i])}
            for i in range(k) if cnt[i] > 0}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "roofline_traffic.md")
KERNEL_SOURCES = ["differentiable_cholesky_amd/csrc/gemm.hpp", "differentiable_cholesky_amd/csrc/blocked.hip",
                  "differentiable_cholesky_amd/csrc/common.hpp", "differentiable_cholesky_amd/csrc/small.hip"]


def sources_digest() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(fam: str):
    """HBM bytes per launch of the family's kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (scaled by the copy-kernel calibration), or
    None if there is no record for it or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            text = fh.read()
    except OSError:
        return None
    digest = sources_digest()
    for line in text.splitlines():
        if line.startswith("record:"):
            f = dict(kv.split("=", 1) for kv in line[len("record:"):].split())
            if f.get("family") == fam and f.get("sources") == digest:
                return int(f["bytes_per_launch"])
    return None


def roofline_of(fam: str, rec: dict, dtype_peak_tflops: float):
    avg_s = rec["ms"] / rec["launches"] / 1e3
    per_launch = rec["work"] / rec["launches"]
    if fam in BYTE_FAMILIES:
        achieved = per_launch / avg_s / 1e9
        return {"kernel": fam, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": recorded_traffic(fam),
                "launches": rec["launches"], "avg_launch_us": round(avg_s * 1e6, 2)}
    achieved = per_launch / avg_s / 1e12
    return {"kernel": fam, "kernel_symbol": FAMILY_KERNEL.get(fam), "bound": "mfma", "achieved": round(achieved, 2),
            "peak": dtype_peak_tflops, "unit": "TFLOP/s", "frac": round(achieved / dtype_peak_tflops, 4),
            "traffic": recorded_traffic(fam), "launches": rec["launches"],
            "avg_launch_us": round(avg_s * 1e6, 2), "work_per_launch": round(per_launch)}


def _close_stats(got, ref, rel_frac):
    """max |got - ref| / (|ref| + max|ref|) (per matrix of a stack) and the max
    relative error over entries with |ref| >= rel_frac * max|ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.ndim == 2:
        got, ref = got[None], ref[None]
    scale = np.max(np.abs(ref), axis=(-2, -1), keepdims=True)
    err = np.abs(got - ref)
    ac = float(np.max(err / np.maximum(np.abs(ref) + scale, 1e-300)))
    big = (np.abs(ref) >= rel_frac * scale) & (scale > 0)
    rel = float(np.max(np.where(big, err / np.maximum(np.abs(ref), 1e-300), 0.0)))
    return {"max_allclose_err": ac, "max_rel_err": rel, "rel_over_entries_above": rel_frac}


def cpu_baseline(dc, A_gpu, L_gpu, adjL_host, Ab_host, adjLb_host, Lb_gpu, ns: int):
    """The oracle, timed on the host cores on a bounded sample of the benchmark's
    inputs; its results are also the parity reference for the GPU outputs
    (computed again outside the timed region where the benchmark's own outputs
    are not comparable)."""
    import oracle
    import torch
    threads = oracle.max_threads()
    A = A_gpu[:ns, :ns].cpu().numpy()
    Lg = L_gpu[:ns, :ns].cpu().numpy()
    adj_s = np.ascontiguousarray(adjL_host[:ns, :ns])
    t = time.perf_counter()
    Lo, info = oracle.potrf(A)
    Go = oracle.potrf_adjoint(Lg, adj_s, accumulate=False)
    tb = time.perf_counter() - t
    gflops = (ns ** 3 / 3 + 2 * ns ** 3 / 3) / tb / 1e9
    Lbg = Lb_gpu.cpu().numpy()
    t = time.perf_counter()
    Lbo, _ = oracle.potrf(Ab_host)
    Gbo = oracle.potrf_adjoint(Lbg, adjLb_host, accumulate=False)
    tm = time.perf_counter() - t
    # GPU adjoints comparable with the oracle's: adj_L supported on the
    # leading block (G is then that block's own adjoint), and the batched
    # adjoint without accumulation
    pad = torch.zeros_like(L_gpu)
    pad[:ns, :ns] = torch.from_numpy(adj_s).to(L_gpu.device)
    G = dc.chol_potrf_adjoint(L_gpu, pad, accumulate=False)
    Gb = dc.chol_potrf_adjoint_batched(Lb_gpu, torch.from_numpy(adjLb_host).to(L_gpu.device), accumulate=False)
    torch.cuda.synchronize()
    outside = float(torch.tril(G)[ns:, :].abs().max().item()) if ns < L_gpu.shape[0] else 0.0
    parity = {
        "reference": "the oracle's results from this leg",
        "factor_leading_block": dict(n=ns, **_close_stats(Lg, Lo, 1e-3)),
        "adjoint_leading_block": dict(n=ns, max_abs_outside_block=outside,
                                      **_close_stats(np.tril(G[:ns, :ns].cpu().numpy()), Go, 1e-3)),
        "batched_factor": dict(batch=int(Ab_host.shape[0]), **_close_stats(Lbg, Lbo, 1e-1)),
        "batched_adjoint": dict(batch=int(Ab_host.shape[0]), **_close_stats(Gb.cpu().numpy(), Gbo, 1e-1)),
    }
    del pad, G
    base = {"value": round(gflops, 3), "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"leading {ns}x{ns} block of the same fp64 A (factor + adjoint, rate with "
                      f"{ns}^3/3 + 2*{ns}^3/3 flops) and all {Ab_host.shape[0]} batched 32x32 matrices",
            "seconds": round(tb + tm, 2),
            "batched": {"value": round(Ab_host.shape[0] / tm, 1), "unit": "matrices/s"}}
    return base, parity


def sampled_residual(L, A, rows):
    """||L[i, :] L^T - A[i, :]|| / (||A||_F / sqrt(n)) over sampled rows i
    (plain torch products on the device)."""
    import torch
    anorm = A.norm().item() / np.sqrt(A.shape[0])
    worst = 0.0
    for i in rows:
        r = (L[i:i + 1, :] @ L.T - A[i:i + 1, :]).norm().item() / anorm
        worst = max(worst, r)
    return worst


def _timed(torch, fn, reps: int, warm: int = 1) -> float:
    """Average ms of fn() over reps calls on the current stream (events
    recorded around the whole batch of calls, after warm untimed calls)."""
    for _ in range(warm):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        fn()
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


def extra_rows(dc, workloads, torch, args):
    """The entry points beyond the headline path, timed at benchmark sizes
    (inputs resident in device memory), each with a sampled check of its
    result; one JSON line per entry point."""
    dev = "cuda"
    n, nb = args.n, args.nb
    reps = max(1, args.steps)
    HBM = 8000.0
    log(f"rows: building inputs (n={n})")
    A = workloads.gram_spd(n, seed=workloads.SEED_MATRIX, shift=0.1, device=dev)
    L, info = dc.chol_potrf(A, nb=nb)
    torch.cuda.synchronize()
    rows = [int(r) for r in np.linspace(0, n - 1, 6)]

    def emit(d):
        print(json.dumps(d), flush=True)

    # solve with the factor, fp64, 16 right-hand sides: bound by reading the
    # lower triangle of L once per sweep
    nrhs = 16
    B = torch.from_numpy(workloads.normal_rhs(n, nrhs, seed=3)).to(dev)
    X = torch.empty_like(B)
    ws = torch.empty(dc.chol_potrs_workspace_size(dc.CHOL_F64, n, nrhs, nb), dtype=torch.uint8, device=dev)
    ms = _timed(torch, lambda: dc.chol_potrs(L, B, X=X, nb=nb, workspace=ws), reps)
    res = float(torch.linalg.norm(A[rows] @ X - B[rows]) / torch.linalg.norm(B[rows]))
    byts = 2 * (n * (n + 1) / 2) * 8 + 4 * n * nrhs * 8
    emit({"row": "potrs", "dtype": "f64", "n": n, "nrhs": nrhs, "ms": round(ms, 3),
          "bound": "hbm", "algorithmic_bytes": byts, "achieved_GBs": round(byts / (ms * 1e-3) / 1e9, 1),
          "frac": round(byts / (ms * 1e-3) / 1e9 / HBM, 4), "sampled_residual": res})
    # its adjoint: the same solve, then [Q; P] = [S|X]^T tril(L) and the
    # lower-only product into adj_L (read + write of its lower triangle)
    gX = torch.from_numpy(workloads.normal_rhs(n, nrhs, seed=4)).to(dev)
    gB = torch.empty_like(gX)
    gL = torch.zeros_like(A)
    wsa = torch.empty(dc.chol_potrs_adjoint_workspace_size(dc.CHOL_F64, n, nrhs, nb), dtype=torch.uint8,
                      device=dev)
    ms = _timed(torch, lambda: dc.chol_potrs_adjoint(L, X, gX, adjB=gB, adjL=gL, accumulate=False, nb=nb,
                                                      workspace=wsa), reps)
    byts = 5 * (n * (n + 1) / 2) * 8 + 8 * n * nrhs * 8
    emit({"row": "potrs_adjoint", "dtype": "f64", "n": n, "nrhs": nrhs, "ms": round(ms, 3),
          "bound": "hbm", "algorithmic_bytes": byts, "achieved_GBs": round(byts / (ms * 1e-3) / 1e9, 1),
          "frac": round(byts / (ms * 1e-3) / 1e9 / HBM, 4)})
    del gL, wsa, gX, gB, ws, X, B

    # batched solve, fp32, 65536 systems of 32 with one right-hand side
    bt, bn = args.batch, args.batch_n
    Ab = torch.from_numpy(workloads.batched_spd(bt, bn, dtype=np.float32)).to(dev)
    Lb, _ = dc.chol_potrf_batched(Ab)
    bb = torch.from_numpy(workloads.normal_rhs(bn, 1, seed=5, batch=bt, dtype=np.float32)).to(dev)
    xb = torch.empty_like(bb)
    ms = _timed(torch, lambda: dc.chol_potrs_batched(Lb, bb, X=xb), reps * 4)
    res = float((torch.linalg.norm(Ab[:64] @ xb[:64] - bb[:64]) / torch.linalg.norm(bb[:64])))
    byts = bt * ((bn * (bn + 1) / 2) + 2 * bn) * 4
    emit({"row": "potrs_batched", "dtype": "f32", "batch": bt, "n": bn, "nrhs": 1, "ms": round(ms, 4),
          "matrices_per_s": round(bt / (ms * 1e-3), 1), "bound": "hbm", "algorithmic_bytes": byts,
          "achieved_GBs": round(byts / (ms * 1e-3) / 1e9, 1), "frac": round(byts / (ms * 1e-3) / 1e9 / HBM, 4),
          "sampled_residual": res})
    del Ab, Lb, bb, xb

    # upper form, fp64: the lower factor on transposed triangles (two extra
    # triangle transpositions); U must be exactly the lower factor transposed
    U = torch.empty_like(A)
    ms = _timed(torch, lambda: dc.chol_potrf_upper(A, U=U, nb=nb), reps)
    same = bool(torch.equal(U[rows], L.t()[rows]))
    emit({"row": "potrf_upper", "dtype": "f64", "n": n, "ms": round(ms, 3), "bound": "mfma",
          "flops": n ** 3 / 3, "achieved_TFs": round(n ** 3 / 3 / (ms * 1e-3) / 1e12, 2),
          "frac": round(n ** 3 / 3 / (ms * 1e-3) / 1e12 / 78.6, 4), "equals_lower_transposed": same})
    gU = torch.triu(torch.from_numpy(workloads.lower_normal(n, seed=6).T.copy()).to(dev))
    gA = torch.zeros_like(A)
    wsu = torch.empty(dc.chol_potrf_adjoint_upper_workspace_size(dc.CHOL_F64, n, 1, nb), dtype=torch.uint8,
                      device=dev)
    ms = _timed(torch, lambda: dc.chol_potrf_adjoint_upper(U, gU, adjA=gA, accumulate=False, nb=nb,
                                                            workspace=wsu), reps)
    emit({"row": "potrf_adjoint_upper", "dtype": "f64", "n": n, "ms": round(ms, 3), "bound": "mfma",
          "flops": 2 * n ** 3 / 3, "achieved_TFs": round(2 * n ** 3 / 3 / (ms * 1e-3) / 1e12, 2),
          "frac": round(2 * n ** 3 / 3 / (ms * 1e-3) / 1e12 / 78.6, 4)})
    del U, gU, gA, wsu, L, A
    torch.cuda.empty_cache()

    # Hermitian complex128 at n/2 (the real embedding is n x n): complex flops
    # 4 (n/2)^3 / 3 for the factor, twice that for the adjoint
    m = n // 2
    rng = np.random.default_rng(7)
    G = torch.complex(torch.from_numpy(rng.standard_normal((m, m))), torch.from_numpy(rng.standard_normal((m, m))))
    G = G.to(dev)
    Ac = G @ G.conj().t() / m
    Ac = (Ac + Ac.conj().t()) / 2 + torch.eye(m, dtype=Ac.dtype, device=dev)
    del G
    Lc = torch.empty_like(Ac)
    wsh = torch.empty(dc.chol_potrf_hermitian_workspace_size(dc.CHOL_C128, m, 1, nb), dtype=torch.uint8,
                      device=dev)
    ms = _timed(torch, lambda: dc.chol_potrf_hermitian(Ac, L=Lc, nb=nb, workspace=wsh), reps)
    rr = [int(r) for r in np.linspace(0, m - 1, 6)]
    res = float(torch.linalg.norm(Lc[rr] @ Lc.conj().t() - Ac[rr]) / torch.linalg.norm(Ac[rr]))
    cfl = 4 * m ** 3 / 3
    emit({"row": "potrf_hermitian", "dtype": "c128", "n": m, "ms": round(ms, 3), "bound": "mfma",
          "complex_flops": cfl, "achieved_TFs": round(cfl / (ms * 1e-3) / 1e12, 2),
          "real_embedding_flops": (2 * m) ** 3 / 3,
          "frac": round(cfl / (ms * 1e-3) / 1e12 / 78.6, 4), "sampled_residual": res})
    del wsh
    gLc = torch.tril(torch.complex(torch.randn(m, m, dtype=torch.float64, device=dev),
                                   torch.randn(m, m, dtype=torch.float64, device=dev)))
    gAc = torch.zeros_like(Ac)
    wsh = torch.empty(dc.chol_potrf_hermitian_workspace_size(dc.CHOL_C128, m, 1, nb, True), dtype=torch.uint8,
                      device=dev)
    ms = _timed(torch, lambda: dc.chol_potrf_adjoint_hermitian(Lc, gLc, adjA=gAc, accumulate=False, nb=nb,
                                                                workspace=wsh), reps)
    emit({"row": "potrf_adjoint_hermitian", "dtype": "c128", "n": m, "ms": round(ms, 3), "bound": "mfma",
          "complex_flops": 2 * cfl, "achieved_TFs": round(2 * cfl / (ms * 1e-3) / 1e12, 2),
          "frac": round(2 * cfl / (ms * 1e-3) / 1e12 / 78.6, 4)})


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--n", type=int, default=16384)
    ap.add_argument("--nb", type=int, default=128)
    ap.add_argument("--batch", type=int, default=65536)
    ap.add_argument("--batch-n", type=int, default=32)
    ap.add_argument("--cpu-sample-n", type=int, default=5632)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rows", action="store_true",
                    help="only time the entry points beyond the headline path (solve and its adjoint, upper "
                         "form, Hermitian complex form) at benchmark sizes, one JSON line each, and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the library's streaming kernels on 1 GiB (read, write, copy: the HBM "
                         "ceiling, and the reference for the HBM byte counters) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        # the library's own streaming kernels on 1 GiB buffers: the device-
        # memory ceiling (read-only, write-only, copy), and a copy of known size
        # whose rocprofv3 FETCH_SIZE / WRITE_SIZE give the scale factor from
        # counter KiB to bytes
        import differentiable_cholesky_amd as dc
        nbytes = 1 << 30
        src = torch.ones(nbytes // 8, dtype=torch.float64, device="cuda")
        dst = torch.empty_like(src)
        sink = torch.empty(dc._lib.HBM_READ_SINK_FLOATS, dtype=torch.float32, device="cuda")
        out = {"calibrate_copy_bytes": nbytes}
        for name, mode, a, b, moved in (("read", 0, src, sink, nbytes), ("write", 1, None, dst, nbytes),
                                        ("copy", 2, src, dst, 2 * nbytes)):
            reps = 10
            dc.chol_hbm_stream(mode, a, b, nbytes)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            for _ in range(reps):
                dc.chol_hbm_stream(mode, a, b, nbytes)
            ev[1].record()
            torch.cuda.synchronize()
            ms = ev[0].elapsed_time(ev[1]) / reps
            out[f"{name}_GBs"] = round(moved / (ms * 1e-3) / 1e9, 1)
            out[f"{name}_us"] = round(ms * 1e3, 1)
        out["launches_per_mode"] = 11
        print(json.dumps(out), flush=True)
        return

    import differentiable_cholesky_amd as dc
    import workloads

    if args.rows:
        extra_rows(dc, workloads, torch, args)
        return

    torch.cuda.set_device(0)
    dev = "cuda"
    n, nb, batch, bn = args.n, args.nb, args.batch, args.batch_n

    log(f"bench: building inputs (n={n}, batch={batch}x{bn})")
    A = workloads.gram_spd(n, seed=workloads.SEED_MATRIX, shift=0.1, device=dev)
    adjL_h = workloads.lower_normal(n, seed=workloads.SEED_ADJ)
    adjL = torch.from_numpy(adjL_h).to(dev)
    L = torch.empty_like(A)
    adjA = torch.zeros_like(A)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    ws_bytes = dc.chol_potrf_adjoint_workspace_size(dc.CHOL_F64, n, nb, True, False)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    Ab_h = workloads.batched_spd(batch, bn, seed=workloads.SEED_MATRIX, dtype=np.float32)
    adjLb_h = workloads.lower_normal(bn, seed=workloads.SEED_ADJ, batch=batch, dtype=np.float32)
    Ab = torch.from_numpy(Ab_h).to(dev)
    adjLb = torch.from_numpy(adjLb_h).to(dev)
    Lb = torch.empty_like(Ab)
    adjAb = torch.zeros_like(Ab)
    infob = torch.zeros(batch, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        # ev: four events bracketing the batched pair, the factor and the
        # adjoint; they are read after all timed steps, so the host enqueues
        # ahead of the GPU and no host time falls inside a bracket
        if ev is not None:
            ev[0].record()
        dc.chol_potrf_batched(Ab, Lb, infob)
        dc.chol_potrf_adjoint_batched(Lb, adjLb, adjAb, accumulate=True)
        if ev is not None:
            ev[1].record()
        dc.chol_potrf(A, L, info, nb=nb)
        if ev is not None:
            ev[2].record()
        dc.chol_potrf_adjoint(L, adjL, adjA, accumulate=True, nb=nb, workspace=ws)
        if ev is not None:
            ev[3].record()

    log(f"bench: {args.warmup} warmup steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(info.item()) == 0 and int(infob.abs().sum().item()) == 0

    # one untimed step with every kernel family timed, to find the dominant
    # blocked family; the timed steps then bracket only that family and the
    # two batched kernels with events, so that event records stay out of the
    # path of the many short launches
    dc.lib.chol_profile_start(0xFFFFFFFF)
    step()
    torch.cuda.synchronize()
    kern_all = profile_stop(dc.lib)
    # the dominant kernel is the one that carries the most algorithmic work (the
    # adjoint's symmetric product: 2N^3/3 of the N^3 flops); by summed time a
    # one-block kernel that runs beside it on the other stream can rank first,
    # but its elapsed time is mostly waiting for a share of a CU
    blocked_all = {k: v for k, v in kern_all.items() if k in FAMILY_KERNEL}
    dom = max(blocked_all, key=lambda k: blocked_all[k]["work"])
    mask = (1 << FAMILIES.index(dom)) | (1 << FAMILIES.index("small_factor")) | \
        (1 << FAMILIES.index("small_adjoint"))

    log(f"bench: {args.steps} timed steps (events on {dom})")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    dc.lib.chol_profile_start(mask)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # one untimed batched factor ahead of the first bracket keeps the GPU busy
    # while the host enqueues the first timed step
    dc.chol_potrf_batched(Ab, Lb, infob)
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = profile_stop(dc.lib)
    times = [(ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[3]), ev[1].elapsed_time(ev[2]),
              ev[2].elapsed_time(ev[3])) for ev in evs]

    t_small = sum(t[0] for t in times) / 1e3
    t_block = sum(t[1] for t in times) / 1e3
    t_fwd = sum(t[2] for t in times) / 1e3
    t_adj = sum(t[3] for t in times) / 1e3
    flops = n ** 3 / 3 + 2 * n ** 3 / 3
    gflops = flops * args.steps / t_block / 1e9
    mats = batch * args.steps / t_small

    roof = roofline_of(dom, kern[dom], PEAK_FP64_TFLOPS)
    small_dom = max(("small_factor", "small_adjoint"), key=lambda k: kern[k]["ms"])
    roof_b = {k: roofline_of(k, kern[k], PEAK_FP32_TFLOPS) for k in ("small_factor", "small_adjoint")}
    algo_bytes = batch * (2 + 4) * (bn * (bn + 1) // 2) * 4
    roof_b["combined"] = {"bound": "hbm", "achieved": round(algo_bytes * args.steps / t_small / 1e9, 1),
                          "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": round(algo_bytes * args.steps / t_small / 1e9 / PEAK_HBM_GBS, 4)}

    out = {
        "metric": METRIC,
        "value": round(gflops, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": f"fp64 N={n} blocked potrf+adjoint (A=GG^T/N+0.1I, nb={nb}) plus "
                               f"fp32 {batch}x{bn}x{bn} batched potrf+adjoint (A=BB^T/{bn}+I)",
                   "n": n, "nb": nb, "batch": batch, "batch_n": bn, "accumulate": True},
        "fraction_of_fp64_peak": round(gflops / 1e3 / PEAK_FP64_TFLOPS, 4),
        "blocked_ms": {"total": round(t_block * 1e3 / args.steps, 3),
                       "factor": round(t_fwd * 1e3 / args.steps, 3),
                       "adjoint": round(t_adj * 1e3 / args.steps, 3),
                       "factor_tflops": round(n ** 3 / 3 * args.steps / t_fwd / 1e12, 2),
                       "adjoint_tflops": round(2 * n ** 3 / 3 * args.steps / t_adj / 1e12, 2)},
        "batched": {"value": round(mats, 1), "unit": "matrices/s", "dtype": "f32",
                    "ms": round(t_small * 1e3 / args.steps, 4),
                    "fraction_of_hbm_roofline": roof_b["combined"]["frac"],
                    "algorithmic_bytes_per_matrix": (2 + 4) * (bn * (bn + 1) // 2) * 4},
        "roofline": roof,
        "roofline_batched": roof_b,
        "kernels": {k: {"launches": v["launches"], "ms_per_step": round(v["ms"], 4)}
                    for k, v in kern_all.items()},
    }
    rows = sorted({0, n // 3, n // 2, n - 1} | set(np.random.default_rng(5).integers(0, n, 4).tolist()))
    out["parity"] = {"residual_sampled_rows": {"rows": rows, "max": sampled_residual(L, A, rows)}}
    if not args.no_cpu_baseline:
        log(f"bench: CPU oracle baseline (sample n={args.cpu_sample_n})")
        base, par = cpu_baseline(dc, A, L, adjL_h, Ab_h, adjLb_h, Lb, min(args.cpu_sample_n, n))
        out["cpu_baseline"] = base
        out["parity"].update(par)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
