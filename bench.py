#!/usr/bin/env python3
"""Benchmark of the norm-fused GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]

A step is one call of the fused kernel over one batch of the workload's
synthetic bf16 inputs (seeded, see workloads/).  The default workload is the
largest one, GEMM + LayerNorm(gamma, beta) epilogue over full rows of 16384
columns (A 8192x8192 @ B 8192x16384: the cross-workgroup row reduction,
MFMA-bound).  Inputs sit in HBM before the timed region;
several input/output copies are rotated so that the 256 MB Infinity Cache
cannot serve a step from the previous step's data.  The fused call and the
unfused baseline (ng_gemm, ng_norm, and the pair) are timed round-robin over
five rounds of W warm-up + K timed launches each, and each reports its
median round, so that the cold start of a process is not charged to whichever
callable happens to be timed first.

Printed: one JSON line with the fused kernel's throughput (TFLOP/s of the GEMM,
2*M*N*K per step), its share of the bf16 MFMA peak, the share of standalone
norm latency it hides against the unfused ng_gemm + ng_norm pair, its roofline
position (HBM- or MFMA-bound), and the CPU oracle's throughput on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
ROUNDS = 5  # round-robin timing rounds per callable (median reported)
RIDGE_FLOP_PER_BYTE = MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
DEFAULT_WORKLOAD = workloads.WORKLOADS[4].name
ROTATE_BYTES = 768 << 20     # input+output copies rotated per step exceed this
METRIC = ("fused norm-GEMM bf16 TFLOP/s (% MFMA peak) + % norm latency hidden vs unfused")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="workload name, or 'all' for one line per workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-load-readings", action="store_true",
                    help="skip the clock/power readings under load (about a second of extra "
                         "fused calls; for profiler runs)")
    ap.add_argument("--no-library-gemm", action="store_true",
                    help="skip timing torch.matmul (hipBLASLt) on the same operands as a "
                         "reference point for the plain product")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run 3 plain device copies of this many MiB (a known-size "
                         "kernel for scaling profiler byte counters)")
    ap.add_argument("--k-walk", choices=("auto", "upward", "alternate"), default="auto",
                    help="direction of the k-loops from round to round in the library's "
                         "persistent grids (diagnostic; default: the library's own choice)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --calibrate-copy-mib 512` into profiles/traffic_<workload>.json")
    return ap.parse_args()


def _pmc_rows(d, counter):
    """(kernel name, value in KiB) per dispatch from a rocprofv3 --pmc csv."""
    import csv
    import glob
    rows = []
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % d)
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return [(k, v) for _, k, v in rows]


EPI_NUMBER = {"EPI_NONE": 0, "EPI_LAZY": 1, "EPI_ROW_RMS": 2, "EPI_ROW_LN": 3,
              "EPI_LAZY_BIAS": 4, "EPI_ROW_RMS_RES": 5, "EPI_ROW_LN_RES": 6, "EPI_PRE_LN": 7,
              "EPI_LAZY_BWD": 8}


def is_fused_dispatch(kernel_name: str, w) -> bool:
    """Whether a traced kernel symbol is the workload's fused kernel (not the
    ng_gemm of the unfused pair, whose symbol has the same base name)."""
    import re
    label = kernel_label(w)
    base = label.split("<")[0]
    if base not in kernel_name:
        return False
    if base == "gemm_xwg_kernel":
        return True
    epi = label.rstrip(">").rsplit("<", 1)[-1].rsplit(", ", 1)[-1]
    # (the plain product's grid may carry a trailing k-walk flag)
    m = re.search(r",\s*(\d+)(?:,\s*(?:true|false))?>\s*(\(|$)", kernel_name.strip())
    return m is not None and int(m.group(1)) == EPI_NUMBER[epi]


def summarize_pmc(fetch_dir, write_dir, w, copy_mib):
    """HBM bytes per launch of the fused kernel, each counter scaled by what
    it reads for a plain copy of known size (copy_mib read + written)."""
    import statistics
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(d, counter)
        # the calibration copies are the first three runtime copy kernels
        copies = [v for k, v in rows if "copybuffer" in k.lower()][:3]
        fused = [v for k, v in rows if is_fused_dispatch(k, w)]
        if not copies or not fused:
            raise SystemExit("missing copy or fused kernel rows for %s" % counter)
        copy_kib = statistics.median(copies)
        factor = (copy_mib * 1024.0) / copy_kib
        out[counter] = {"copy_kib": copy_kib, "factor": factor,
                        "fused_kib_median": statistics.median(fused),
                        "fused_bytes": statistics.median(fused) * 1024.0 * factor}
    rec = {"workload": w.name, "kernel_source_hash": kernel_source_hash(),
           "copy_mib": copy_mib, "counters": out,
           "bytes_per_launch": int(out["FETCH_SIZE"]["fused_bytes"] + out["WRITE_SIZE"]["fused_bytes"]),
           "algorithmic_bytes": algorithmic_bytes(w)}
    # the vendor library's product on the same operands, when the run timed it
    # (hipBLASLt kernels are named Cijk_...): the same counters, same scaling
    lib = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [(k, v) for k, v in _pmc_rows(d, counter) if k.startswith("Cijk_")]
        if rows:
            lib[counter] = statistics.median(v for _, v in rows) * 1024.0 * out[counter]["factor"]
            lib["kernel"] = rows[0][0].split("(")[0][:80]
    if "FETCH_SIZE" in lib and "WRITE_SIZE" in lib:
        lib["bytes_per_launch"] = int(lib["FETCH_SIZE"] + lib["WRITE_SIZE"])
        rec["library_gemm"] = lib
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % w.name)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def copy_calibration(mib: int):
    import torch
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def algorithmic_bytes(w: workloads.Workload) -> int:
    """Compulsory HBM bytes of one fused call: A, B and C once, plus gamma/beta
    (the Lazy affine form reads the folded B and an fp32 bias instead) and
    the residual R of the residual forms."""
    b = 2 * (w.M * w.K + w.K * w.N + w.M * w.N)
    if w.op == workloads.OP_LAZY_AFFINE:
        return b + 4 * w.N
    if w.op == workloads.OP_PRENORM_LN:
        return b + 8 * w.N  # fp32 colsum and bias
    if w.op == workloads.OP_LAZY_BWD_W:
        # A [M, K], dC [M, N], dB [K, N], fp32 rstd [M]
        return 2 * (w.M * w.K + w.M * w.N + w.K * w.N) + 4 * w.M
    if w.op == workloads.OP_LAZY_BWD:
        # dC [M, N], B, A [M, K] and dA [M, K], fp32 rstd [M]
        return 2 * (w.M * w.N + w.K * w.N + 2 * w.M * w.K) + 4 * w.M
    if w.op == workloads.OP_LAZY_BWD_RG:
        # as the input gradient, plus dB [K, N] written and the intermediate
        # rstd * dC [M, N] written once and read once
        return (2 * (w.M * w.N + w.K * w.N + 2 * w.M * w.K) + 4 * w.M + 2 * w.K * w.N
                + 4 * w.M * w.N)
    b += 2 * w.N * (int(w.gamma) + int(w.beta))
    if w.residual:
        b += 2 * w.M * w.N
    return b


def norm_bytes(w: workloads.Workload) -> int:
    """Standalone norm of the unfused pair: read + write the normalized matrix
    (and read R for the residual forms)."""
    rows, cols = (w.M, w.K) if prenorm(w) or w.op in (workloads.OP_LAZY_BWD,
                                                       workloads.OP_LAZY_BWD_RG) else (w.M, w.N)
    if w.op == workloads.OP_LAZY_BWD_RG:
        # the norm's backward (dA_hat, A -> dA) and the stored A_hat (A -> A_hat)
        return 10 * rows * cols
    return (6 if w.residual or w.op == workloads.OP_LAZY_BWD else 4) * rows * cols


def prenorm(w: workloads.Workload) -> bool:
    """The norm acts on A before the product (the unfused pair runs it first)."""
    return w.op in (workloads.OP_LAZY, workloads.OP_LAZY_AFFINE, workloads.OP_PRENORM_LN,
                    workloads.OP_LAZY_BWD_W)


def kernel_label(w: workloads.Workload) -> str:
    """Name of the fused kernel the workload launches (the symbol's base name)
    and its epilogue."""
    epi = {workloads.OP_LAZY: "EPI_LAZY", workloads.OP_LAZY_AFFINE: "EPI_LAZY_BIAS",
           workloads.OP_GEMM_RMSNORM: "EPI_ROW_RMS", workloads.OP_GEMM_LAYERNORM: "EPI_ROW_LN",
           workloads.OP_GEMM_ADD_RMSNORM: "EPI_ROW_RMS_RES",
           workloads.OP_GEMM_ADD_LAYERNORM: "EPI_ROW_LN_RES",
           workloads.OP_PRENORM_LN: "EPI_PRE_LN", workloads.OP_LAZY_BWD: "EPI_LAZY_BWD",
           workloads.OP_LAZY_BWD_W: "EPI_NONE", workloads.OP_LAZY_BWD_RG: "EPI_LAZY_BWD"}[w.op]
    if w.op == workloads.OP_LAZY_BWD_W:
        return "gemm_persistent_kernel<Tile<..., A stored [K,M], RS 1>, EPI_NONE>"
    if w.op == workloads.OP_LAZY_BWD_RG:
        return ("%s<EPI_LAZY_BWD> writing rstd*dC, then gemm_persistent_kernel<Tile<..., "
                "A stored [K,M]>, EPI_NONE>" % ("gemm_kernel" if w.K <= 256 else "gemm_xwg_kernel"))
    if w.op == workloads.OP_LAZY_BWD:
        return "%s<%s>" % ("gemm_kernel" if w.K <= 256 else "gemm_xwg_kernel", epi)
    if prenorm(w):
        base = "gemm_kernel" if w.N <= 128 else "gemm_persistent_kernel"
    else:
        base = "gemm_kernel" if w.N <= 256 else "gemm_xwg_kernel"
    return "%s<%s>" % (base, epi)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "normalization_gemm_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(w: workloads.Workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % w.name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


class Bench:
    def __init__(self, w: workloads.Workload, seed: int = 0):
        import numpy as np
        import torch

        import normalization_gemm_amd as ng
        self.torch, self.ng, self.np = torch, ng, np
        self.w = w
        x = workloads.workload_inputs(w, seed)
        dev = torch.device("cuda:0")

        def up(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
                torch.bfloat16)

        lazy = prenorm(w)
        per_copy = 2 * (w.M * w.K + w.M * w.N) + (2 * w.M * w.K if lazy else 0)
        per_copy += 2 * w.M * w.N if w.residual else 0
        if w.op == workloads.OP_LAZY_BWD:
            per_copy = 2 * (w.M * w.N + 3 * w.M * w.K)  # dC, A, dA, dA_hat
        if w.op == workloads.OP_LAZY_BWD_RG:
            # dC, A, dA, dA_hat, A_hat, rstd * dC, dB
            per_copy = 2 * (2 * w.M * w.N + 4 * w.M * w.K + w.K * w.N)
        self.R = max(1, min(8, math.ceil(ROTATE_BYTES / per_copy)))
        A0 = up(x.A)
        self.A = [A0] + [A0.clone() for _ in range(self.R - 1)]
        self.B = up(x.B)
        self.gamma = up(x.gamma) if x.gamma is not None else None
        self.beta = up(x.beta) if x.beta is not None else None
        self.C = [torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev) for _ in range(self.R)]
        if w.residual:
            R0 = up(x.R)
            self.res = [R0] + [R0.clone() for _ in range(self.R - 1)]
        if w.op == workloads.OP_LAZY_BWD_W:
            # the forward pass's saved rstd (untimed); the output dB is [K, N]
            self.rstd = torch.empty(w.M, dtype=torch.float32, device=dev)
            ng.rmsnorm_gemm_lazy(A0, self.B, eps=w.eps, rstd_out=self.rstd)
            G0 = up(x.dC)
            self.dC = [G0] + [G0.clone() for _ in range(self.R - 1)]
            self.C = [torch.empty((w.K, w.N), dtype=torch.bfloat16, device=dev)
                      for _ in range(self.R)]
        if w.op == workloads.OP_LAZY_BWD_RG:
            # the forward pass's saved rstd (untimed); outputs dA [M, K] and
            # dB [K, N], the scratch rstd * dC [M, N]; the unfused pair's
            # dA_hat and A_hat
            self.rstd = torch.empty(w.M, dtype=torch.float32, device=dev)
            ng.rmsnorm_gemm_lazy(A0, self.B, eps=w.eps, rstd_out=self.rstd)
            G0 = up(x.dC)
            self.dC = [G0] + [G0.clone() for _ in range(self.R - 1)]
            self.C = [torch.empty((w.M, w.K), dtype=torch.bfloat16, device=dev)
                      for _ in range(self.R)]
            self.dAh = [torch.empty((w.M, w.K), dtype=torch.bfloat16, device=dev)
                        for _ in range(self.R)]
            self.dB = [torch.empty((w.K, w.N), dtype=torch.bfloat16, device=dev)
                       for _ in range(self.R)]
            self.scratch = [torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
                            for _ in range(self.R)]
            An0 = ng.norm(A0, "rms", eps=w.eps)
            self.An = [An0] + [An0.clone() for _ in range(self.R - 1)]
        if w.op == workloads.OP_LAZY_BWD:
            # the forward pass's saved rstd (untimed); outputs are [M, K]
            self.rstd = torch.empty(w.M, dtype=torch.float32, device=dev)
            ng.rmsnorm_gemm_lazy(A0, self.B, eps=w.eps, rstd_out=self.rstd)
            G0 = up(x.dC)
            self.dC = [G0] + [G0.clone() for _ in range(self.R - 1)]
            self.C = [torch.empty((w.M, w.K), dtype=torch.bfloat16, device=dev)
                      for _ in range(self.R)]
            self.dAh = [torch.empty((w.M, w.K), dtype=torch.bfloat16, device=dev)
                        for _ in range(self.R)]
        # the library reference's transposed operands (B^T for dC @ B^T, the
        # normalized A transposed for A_hat^T @ dC), outside the timed calls
        if w.op in (workloads.OP_LAZY_BWD, workloads.OP_LAZY_BWD_RG):
            self.Bt = self.B.t().contiguous()
        if w.op in (workloads.OP_LAZY_BWD_W, workloads.OP_LAZY_BWD_RG):
            self.At = ng.norm(A0, "rms", eps=w.eps).t().contiguous()
        # unfused pair intermediates: the normalized A of the lazy form's
        # pair holds real values (the GEMM's speed depends on its data)
        if lazy:
            kind = "layer" if w.op == workloads.OP_PRENORM_LN else "rms"
            An0 = ng.norm(A0, kind, self.gamma, self.beta, eps=w.eps)
            self.An = [An0] + [An0.clone() for _ in range(self.R - 1)]
        if w.op == workloads.OP_LAZY_AFFINE:
            # the weight fold is a one-off transform, outside the timed calls
            self.Bf, self.bias = ng.lazy_fold_affine(self.B, self.gamma, self.beta)
        if w.op == workloads.OP_PRENORM_LN:
            self.Bf, self.colsum, self.bias = ng.layernorm_gemm_fold(self.B, self.gamma, self.beta)
            self.mean = torch.empty(w.M, dtype=torch.float32, device=dev)
            self.rstd = torch.empty(w.M, dtype=torch.float32, device=dev)
        self.ws = None
        op = {workloads.OP_LAZY: ng.NG_OP_RMSNORM_GEMM_LAZY,
              workloads.OP_LAZY_AFFINE: ng.NG_OP_RMSNORM_GEMM_LAZY,
              workloads.OP_PRENORM_LN: ng.NG_OP_RMSNORM_GEMM_LAZY,
              workloads.OP_LAZY_BWD: ng.NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT,
              workloads.OP_LAZY_BWD_RG: ng.NG_OP_RMSNORM_GEMM_LAZY_BWD_INPUT,
              workloads.OP_LAZY_BWD_W: ng.NG_OP_RMSNORM_GEMM_LAZY,
              workloads.OP_GEMM_RMSNORM: ng.NG_OP_GEMM_RMSNORM,
              workloads.OP_GEMM_LAYERNORM: ng.NG_OP_GEMM_LAYERNORM,
              workloads.OP_GEMM_ADD_RMSNORM: ng.NG_OP_GEMM_ADD_RMSNORM,
              workloads.OP_GEMM_ADD_LAYERNORM: ng.NG_OP_GEMM_ADD_LAYERNORM}[w.op]
        nb = ng.ng_workspace_bytes(op, w.M, w.N, w.K)
        if nb:
            self.ws = ng.Workspace(nb, dev)
        del x
        torch.cuda.synchronize()
        self._bind()

    # The timed calls go straight to the C entry points with arguments
    # marshalled once (the tensor helpers' checks cost more host time per call
    # than the small kernels take on the GPU).
    def _bind(self):
        from normalization_gemm_amd import _lib
        lib = _lib.load()  # the ctypes functions themselves
        w, ng = self.w, self.ng
        st = self.torch.cuda.current_stream().cuda_stream
        ptr = lambda t: None if t is None else t.data_ptr()
        ws, wsb = (self.ws.ptr(), self.ws.nbytes) if self.ws is not None else (None, 0)
        M, N, K, eps = w.M, w.N, w.K, float(w.eps)
        self._fused, self._gemm, self._norm = [], [], []
        for r in range(self.R):
            A, C = self.A[r].data_ptr(), self.C[r].data_ptr()
            B, g, b = self.B.data_ptr(), ptr(self.gamma), ptr(self.beta)
            if w.op == workloads.OP_LAZY_AFFINE:
                An = self.An[r].data_ptr()
                self._fused.append((lib.ng_rmsnorm_gemm_lazy_affine,
                                    (A, self.Bf.data_ptr(), self.bias.data_ptr(), C, M, N, K, 0,
                                     eps, None, st)))
                self._gemm.append((lib.ng_gemm, (An, B, C, M, N, K, 0, st)))
                self._norm.append((lib.ng_norm, (A, g, b, An, M, K, 0, eps, None, None, st)))
            elif w.op == workloads.OP_LAZY_BWD_W:
                G, An, rs = self.dC[r].data_ptr(), self.An[r].data_ptr(), self.rstd.data_ptr()
                self._fused.append((lib.ng_rmsnorm_gemm_lazy_backward_weight,
                                    (A, G, rs, C, M, N, K, 0, st)))
                # unfused: A_hat stored by ng_norm, then dB = A_hat^T @ dC
                self._gemm.append((lib.ng_gemm_at, (An, G, C, K, N, M, st)))
                self._norm.append((lib.ng_norm, (A, None, None, An, M, K, 0, eps, None, None, st)))
            elif w.op == workloads.OP_LAZY_BWD_RG:
                G, dAh, rs = self.dC[r].data_ptr(), self.dAh[r].data_ptr(), self.rstd.data_ptr()
                dB, sc, An = (self.dB[r].data_ptr(), self.scratch[r].data_ptr(),
                              self.An[r].data_ptr())
                self._fused.append((lib.ng_rmsnorm_gemm_lazy_backward,
                                    (G, B, A, rs, C, dB, sc, M, N, K, 0, ws, wsb, st)))
                # unfused: dA_hat = dC @ B^T and dB = A_hat^T @ dC (A_hat stored
                # by ng_norm); the norm's backward and the norm itself
                self._gemm.append([(lib.ng_gemm, (G, B, dAh, M, K, N, 1, st)),
                                   (lib.ng_gemm_at, (An, G, dB, K, N, M, st))])
                self._norm.append([(lib.ng_rmsnorm_backward, (dAh, A, rs, C, M, K, st)),
                                   (lib.ng_norm, (A, None, None, An, M, K, 0, eps, None, None,
                                                  st))])
            elif w.op == workloads.OP_LAZY_BWD:
                G, dAh, rs = self.dC[r].data_ptr(), self.dAh[r].data_ptr(), self.rstd.data_ptr()
                self._fused.append((lib.ng_rmsnorm_gemm_lazy_backward_input,
                                    (G, B, A, rs, C, M, N, K, 0, ws, wsb, st)))
                # dA_hat = dC @ B^T: B [K, N] read in the [N', K'] layout
                self._gemm.append((lib.ng_gemm, (G, B, dAh, M, K, N, 1, st)))
                self._norm.append((lib.ng_rmsnorm_backward, (dAh, A, rs, C, M, K, st)))
            elif w.op == workloads.OP_PRENORM_LN:
                An = self.An[r].data_ptr()
                self._fused.append((lib.ng_layernorm_gemm_prenorm,
                                    (A, self.Bf.data_ptr(), self.colsum.data_ptr(),
                                     self.bias.data_ptr(), C, M, N, K, 0, eps,
                                     self.mean.data_ptr(), self.rstd.data_ptr(), st)))
                self._gemm.append((lib.ng_gemm, (An, B, C, M, N, K, 0, st)))
                self._norm.append((lib.ng_norm, (A, g, b, An, M, K, 1, eps, None, None, st)))
            elif w.op == workloads.OP_LAZY:
                An = self.An[r].data_ptr()
                self._fused.append((lib.ng_rmsnorm_gemm_lazy,
                                    (A, B, C, M, N, K, 0, eps, None, st)))
                self._gemm.append((lib.ng_gemm, (An, B, C, M, N, K, 0, st)))
                self._norm.append((lib.ng_norm, (A, None, None, An, M, K, 0, eps, None, None, st)))
            elif w.residual:
                # post-norm with residual: the unfused pair is the GEMM, then
                # one residual-add + norm kernel (no sum output in either)
                Rr = self.res[r].data_ptr()
                ln = w.op == workloads.OP_GEMM_ADD_LAYERNORM
                if ln:
                    self._fused.append((lib.ng_gemm_add_layernorm,
                                        (A, B, Rr, g, b, C, None, M, N, K, 0, eps, None, None, ws,
                                         wsb, st)))
                else:
                    self._fused.append((lib.ng_gemm_add_rmsnorm,
                                        (A, B, Rr, g, C, None, M, N, K, 0, eps, None, ws, wsb,
                                         st)))
                self._gemm.append((lib.ng_gemm, (A, B, C, M, N, K, 0, st)))
                self._norm.append((lib.ng_add_norm, (C, Rr, g, b, C, None, M, N, int(ln), eps,
                                                     None, None, st)))
            elif w.op == workloads.OP_GEMM_RMSNORM:
                self._fused.append((lib.ng_gemm_rmsnorm,
                                    (A, B, g, C, M, N, K, 0, eps, None, ws, wsb, st)))
                self._gemm.append((lib.ng_gemm, (A, B, C, M, N, K, 0, st)))
                self._norm.append((lib.ng_norm, (C, g, None, C, M, N, 0, eps, None, None, st)))
            else:
                self._fused.append((lib.ng_gemm_layernorm,
                                    (A, B, g, b, C, M, N, K, 0, eps, None, None, ws, wsb, st)))
                self._gemm.append((lib.ng_gemm, (A, B, C, M, N, K, 0, st)))
                self._norm.append((lib.ng_norm, (C, g, b, C, M, N, 1, eps, None, None, st)))

    def _call(self, table, i):
        entry = table[i % self.R]
        for fn, args in (entry if isinstance(entry, list) else [entry]):
            status = fn(*args)
            if status != 0:
                raise self.ng.NormGemmError(status, fn.__name__)

    def fused(self, i):
        self._call(self._fused, i)

    def gemm_only(self, i):
        self._call(self._gemm, i)

    def norm_only(self, i):
        self._call(self._norm, i)

    # The vendor library's GEMM on the same operands (torch.matmul, which
    # ROCm serves from hipBLASLt): a reference point for the plain product(s)
    # on the same board at the same clock and power cap, not part of any
    # measured path.  Forward: C = A @ B.  Backward: dA_hat = dC @ B^T and/or
    # dB = A_hat^T @ dC, the transposed operands materialized once outside
    # the timed calls (the library then multiplies contiguous matrices).
    def has_library_gemm(self):
        return True

    def library_gemm(self, i):
        r = i % self.R
        op = self.w.op
        if op in (workloads.OP_LAZY_BWD, workloads.OP_LAZY_BWD_RG):
            self.torch.matmul(self.dC[r], self.Bt, out=self.dAh[r])
        if op == workloads.OP_LAZY_BWD_W:
            self.torch.matmul(self.At, self.dC[r], out=self.C[r])
        if op == workloads.OP_LAZY_BWD_RG:
            self.torch.matmul(self.At, self.dC[r], out=self.dB[r])
        if op in (workloads.OP_LAZY_BWD, workloads.OP_LAZY_BWD_W, workloads.OP_LAZY_BWD_RG):
            return
        A = self.An[r] if prenorm(self.w) else self.A[r]
        self.torch.matmul(A, self.B, out=self.C[r])

    def pair(self, i):
        if prenorm(self.w):
            self.norm_only(i)
            self.gemm_only(i)
        else:
            self.gemm_only(i)
            self.norm_only(i)

    def time_launches(self, fn, steps, warmup):
        """Returns (per-launch durations in ms from events between launches,
        wall time of the timed loop in ms, mean launch duration in ms from one
        event pair around the loop).  The loop with only the outer event pair
        is the one the wall time covers: events between launches add queue
        packets of their own."""
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3
        mean = e0.elapsed_time(e1) / steps
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            fn(i)
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        return per, wall, mean


def _read(path):
    try:
        with open(path) as f:
            return f.read().strip()
    except OSError:
        return None


def _sysfs_card():
    """sysfs device directory of the GPU torch sees as cuda:0 (matched by PCI
    address), or None."""
    import glob
    torch = __import__("torch")
    prop = torch.cuda.get_device_properties(0)
    bus = getattr(prop, "pci_bus_id", None)
    dev = getattr(prop, "pci_device_id", None)
    dom = getattr(prop, "pci_domain_id", 0) or 0
    if bus is None or dev is None:
        return None
    slot = "%04x:%02x:%02x." % (dom, bus, dev)
    for d in sorted(glob.glob("/sys/class/drm/card*/device")):
        ue = _read(os.path.join(d, "uevent")) or ""
        for line in ue.splitlines():
            if line.startswith("PCI_SLOT_NAME=") and line.split("=", 1)[1].lower().startswith(slot):
                return d
    return None


def power_and_clocks():
    """Shader clock and power readings of cuda:0 from sysfs (hwmon: sclk in
    MHz, socket power and its cap in W; the current DPM level of pp_dpm_sclk),
    falling back to rocm-smi's JSON.  Best effort: missing readings are None."""
    import glob
    out = {}
    d = _sysfs_card()
    if d:
        for hw in glob.glob(os.path.join(d, "hwmon", "hwmon*")):
            f = _read(os.path.join(hw, "freq1_input"))
            if f and f.isdigit():
                out["sclk_mhz"] = round(int(f) / 1e6)
            for name, key in (("power1_average", "power_w"), ("power1_input", "power_w"),
                              ("power1_cap", "power_cap_w")):
                v = _read(os.path.join(hw, name))
                if v and v.isdigit() and key not in out:
                    out[key] = round(int(v) / 1e6, 1)
        lv = _read(os.path.join(d, "pp_dpm_sclk"))
        if lv:
            cur = [ln for ln in lv.splitlines() if ln.rstrip().endswith("*")]
            if cur:
                out["sclk_dpm_level"] = cur[0].rstrip(" *")
    if "sclk_mhz" not in out or "power_cap_w" not in out:
        import subprocess
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--showmaxpower",
                                "--json"], capture_output=True, text=True, timeout=20)
            rec = json.loads(r.stdout)
            card = next(iter(rec.values())) if len(rec) == 1 else None
            if isinstance(card, dict):
                out["rocm_smi"] = {k: v for k, v in card.items()
                                   if "sclk" in k.lower() or "power" in k.lower()}
        except Exception:  # pragma: no cover - best effort
            pass
    return out


def readings_under_load(fn, n_launches):
    """Enqueue n_launches calls of fn (about a second of GPU work) and take
    power_and_clocks() from a thread while they run."""
    import threading
    torch = __import__("torch")
    res = {}

    def sample():
        time.sleep(0.25)
        res.update(power_and_clocks())

    th = threading.Thread(target=sample)
    th.start()
    for i in range(n_launches):
        fn(i)
    th.join()
    torch.cuda.synchronize()
    return res


def source_hash() -> str:
    """Hash of the sources a result depends on (kernels, header, bench), for
    runs made where git is not available."""
    h = hashlib.sha256()
    for rel in ("include/normgemm.h", "bench.py"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    h.update(kernel_source_hash().encode())
    return h.hexdigest()[:16]


def git_sha():
    import subprocess
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                           text=True, timeout=10)
        return r.stdout.strip() or None
    except Exception:  # pragma: no cover - best effort
        return None


def device_info():
    """Name, CU count and maximum shader clock of the device, the HIP runtime
    the process loaded (PyTorch's) and the ROCm install the library was built
    with (for the record; not used in any figure)."""
    torch = __import__("torch")
    prop = torch.cuda.get_device_properties(0)
    info = {"name": prop.name, "arch": getattr(prop, "gcnArchName", ""),
            "cus": prop.multi_processor_count,
            "hip_runtime": getattr(torch.version, "hip", None),
            "rocm_install": _read("/opt/rocm/.info/version")}
    clk = getattr(prop, "clock_rate", None)
    if clk:
        info["max_sclk_mhz"] = round(clk / 1000.0)
    return info


def blas_info():
    """BLAS library NumPy runs the oracle's products on (threadpoolctl)."""
    try:
        from threadpoolctl import threadpool_info
        for d in threadpool_info():
            if d.get("user_api") == "blas":
                return "%s %s" % (d.get("internal_api"), d.get("version"))
    except Exception:  # pragma: no cover
        pass
    return None


def cpu_baseline(w: workloads.Workload, target_s: float):
    """The CPU oracle (untuned) on a row sample of the same workload: passes
    over a growing number of output rows (capped at M) until about target_s
    seconds of CPU time are spent; throughput = GEMM flops of the rows done."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    def sample(rows):
        return workloads.make_inputs(rows, w.N, w.K, seed=1, row_scale=w.row_scale,
                                     gamma=w.gamma, beta=w.beta,
                                     gamma_len=w.K if w.op in (workloads.OP_LAZY_AFFINE,
                                                               workloads.OP_PRENORM_LN) else None,
                                     residual=w.residual, row_shift=w.row_shift,
                                     upstream=w.upstream)

    rows = min(w.M, 64)
    x = sample(rows)
    done_rows, t_total = 0, 0.0
    while t_total < target_s:
        t0 = time.perf_counter()
        if w.op == workloads.OP_LAZY:
            oracle.rmsnorm_gemm_lazy(x.A, x.B, w.eps)
        elif w.op == workloads.OP_LAZY_AFFINE:
            oracle.rmsnorm_gemm_lazy_affine(x.A, x.B, w.eps, x.gamma, x.beta)
        elif w.op == workloads.OP_PRENORM_LN:
            oracle.layernorm_gemm_prenorm(x.A, x.B, w.eps, x.gamma, x.beta)
        elif w.op in (workloads.OP_LAZY_BWD, workloads.OP_LAZY_BWD_RG):
            oracle.rmsnorm_gemm_lazy_backward(x.A, x.B, x.dC, w.eps)
        elif w.op == workloads.OP_LAZY_BWD_W:
            oracle.lazy_backward_weight(x.A, x.dC, w.eps)
        elif w.op == workloads.OP_GEMM_RMSNORM:
            oracle.gemm_rmsnorm(x.A, x.B, w.eps, x.gamma)
        elif w.op == workloads.OP_GEMM_ADD_RMSNORM:
            oracle.gemm_add_rmsnorm(x.A, x.B, x.R, w.eps, x.gamma)
        elif w.op == workloads.OP_GEMM_ADD_LAYERNORM:
            oracle.gemm_add_layernorm(x.A, x.B, x.R, w.eps, x.gamma, x.beta)
        else:
            oracle.gemm_layernorm(x.A, x.B, w.eps, x.gamma, x.beta)
        dt = time.perf_counter() - t0
        t_total += dt
        done_rows += rows
        # grow the sample while one pass is short, up to the whole workload
        if dt < target_s / 8 and rows < w.M:
            rows = min(w.M, rows * 4)
            x = sample(rows)
    # the backward oracle also forms the weight gradient: two products per row
    products = 2 if w.op in (workloads.OP_LAZY_BWD, workloads.OP_LAZY_BWD_RG) else 1
    flops = 2.0 * products * done_rows * w.N * w.K
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "blas": blas_info(),
            "sample": "%d output rows of %s in passes of up to %d rows (fp64 NumPy GEMM%s + "
                      "explicit norm, %.1f s)" % (done_rows, w.name, rows,
                                                  "s" if products == 2 else "", t_total)}


def run(w: workloads.Workload, steps: int, warmup: int, with_cpu: bool, cpu_s: float,
        load_readings: bool = True, library_reference: bool = True):
    import numpy as np
    torch_mod = __import__("torch")
    b = Bench(w)
    # The fused kernel and the unfused baseline are timed round-robin over
    # ROUNDS rounds (each: `warmup` untimed launches, then `steps` timed ones
    # with a sync on both sides); each callable reports its median round.  The
    # first round of a process runs on a cold GPU (clocks, TLBs) and would
    # otherwise penalize whichever callable is timed first.
    rounds = {"fused": [], "gemm": [], "norm": [], "pair": []}
    fns = {"fused": b.fused, "gemm": b.gemm_only, "norm": b.norm_only, "pair": b.pair}
    with_lib = library_reference and b.has_library_gemm() and w.flops >= 1e11
    if with_lib:
        rounds["library"] = []
        fns["library"] = b.library_gemm
    for _ in range(ROUNDS):
        for k, fn in fns.items():
            rounds[k].append(b.time_launches(fn, steps, warmup))

    # a cross-workgroup exchange that gave up would have left NaN in the
    # output and raised the workspace's error word: a timing of such calls
    # is not reported
    if b.ws is not None:
        st = b.ws.status()
        if st != 0:
            raise b.ng.NormGemmError(st, "cross-workgroup exchange during the timed calls")

    def median_round(k):
        rs = sorted(rounds[k], key=lambda r: r[2])
        return rs[len(rs) // 2]

    per, wall_ms, t_fused = median_round("fused")
    t_gemm = median_round("gemm")[2]
    t_norm = median_round("norm")[2]
    t_pair = median_round("pair")[2]
    flops = float(w.flops)
    tflops = flops * steps / (wall_ms * 1e-3) / 1e12
    kern_tflops = flops / (t_fused * 1e-3) / 1e12
    ai = flops / algorithmic_bytes(w)
    hbm_bound = ai < RIDGE_FLOP_PER_BYTE
    if hbm_bound:
        achieved = algorithmic_bytes(w) / (t_fused * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(kern_tflops, 1), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(kern_tflops / MFMA_PEAK_TFLOPS, 4)}
    roof["traffic"] = measured_traffic(w)
    roof["kernel"] = kernel_label(w)
    roof["avg_launch_us"] = round(t_fused * 1e3, 2)
    roof["algorithmic_bytes"] = algorithmic_bytes(w)
    hidden = (t_gemm + t_norm - t_fused) / t_norm * 100.0
    # clock and power while the fused kernel runs (about a second of calls)
    load = (readings_under_load(b.fused, max(50, int(1.0 / max(t_fused * 1e-3, 1e-6))))
            if load_readings else None)
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall_ms / steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16, shapes and distributions of the named workload)",
        "config": {"workload": w.name, "op": w.op, "M": w.M, "N": w.N, "K": w.K, "eps": w.eps,
                   "gamma": w.gamma, "beta": w.beta, "residual": w.residual, "b_layout": "kn",
                   "rotated_copies": b.R},
        "mfma_peak_pct": round(kern_tflops / MFMA_PEAK_TFLOPS * 100.0, 2),
        "norm_hidden_pct": round(hidden, 1),
        "unfused": {"gemm_us": round(t_gemm * 1e3, 2), "norm_us": round(t_norm * 1e3, 2),
                    "pair_us": round(t_pair * 1e3, 2), "fused_us": round(t_fused * 1e3, 2),
                    "norm_gbs": round(norm_bytes(w) / (t_norm * 1e-3) / 1e9, 1),
                    "fused_median_us": round(float(np.median(per)) * 1e3, 2),
                    "fused_p10_us": round(float(np.percentile(per, 10)) * 1e3, 2),
                    "fused_p90_us": round(float(np.percentile(per, 90)) * 1e3, 2)},
        "roofline": roof,
        "library_gemm": ({"callable": "torch.matmul (hipBLASLt)",
                          "us": round(median_round("library")[2] * 1e3, 2),
                          "tflops": round(flops / (median_round("library")[2] * 1e-3) / 1e12, 1)}
                         if with_lib else None),
        "device": device_info(),
        "under_load": load,
        "git_sha": git_sha(),
        "source_hash": source_hash(),
    }
    del b
    torch_mod.cuda.empty_cache()
    if with_cpu:
        line["cpu_baseline"] = cpu_baseline(w, cpu_s)
    return line


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1],
                      workloads.WORKLOAD_BY_NAME[args.workload], args.calibrate_copy_mib or 512)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested); run with --gpus 1" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy_mib:
        copy_calibration(args.calibrate_copy_mib)
    if args.k_walk != "auto":
        import normalization_gemm_amd as ng
        mode = {"upward": ng.NG_K_WALK_UPWARD, "alternate": ng.NG_K_WALK_ALTERNATE}[args.k_walk]
        if ng.ng_set_debug_option(ng.NG_DEBUG_K_WALK, mode) != 0:
            raise SystemExit("ng_set_debug_option failed")
    if args.workload == "all":
        names = [w.name for w in workloads.WORKLOADS + workloads.NEXT_WORKLOADS]
    else:
        names = [args.workload]
    for name in names:
        w = workloads.WORKLOAD_BY_NAME[name]
        small = w.flops < 1e11
        steps = args.steps if args.steps is not None else (200 if small else 30)
        warmup = args.warmup if args.warmup is not None else 20
        line = run(w, steps, warmup, not args.no_cpu_baseline, args.cpu_seconds,
                   not args.no_load_readings, not args.no_library_gemm)
        if args.k_walk != "auto":
            line["k_walk"] = args.k_walk
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
