#!/usr/bin/env python3
"""Benchmark of the MX hot path on one MI355X.

One step = the whole path on one batch of synthetic input, for one
Llama-3-8B-shaped MLP layer's training GEMMs (tokens 8192, hidden 4096, ffn
14336; the largest workload):
  1. mx_quantize_dual_layout of the six operand tensors -- activations X
     [8192][4096] and X' [8192][14336], weights W_gu [4096][28672] and W_d
     [14336][4096] in E4M3, gradients dY_gu [8192][28672] and dY_d
     [8192][4096] in E5M2 -- each read once and written as row and column
     copies with E8M0 1x32 / 32x1 block scales, round to nearest even;
  2. the six GEMMs on those copies: fprop X.W_gu, X'.W_d; dgrad dY_gu.W_gu^T,
     dY_d.W_d^T; wgrad X^T.dY_gu, X'^T.dY_d (fp32 accumulation, bf16 out).
Inputs are resident in HBM before timing starts; a 512 MiB read evicts
L2/MALL before every step (outside the timed kernels) so no step reads its
inputs from cache.  Kernel times come from HIP events recorded on the stream
the kernels run on.

Prints one JSON line (rank 0).  `--workload` selects another workload (the
MOSS two-level 4096^3 step, the FP4 wgrad step, the dual-layout quantizer
alone, ...); the default is the one above.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from fp4_quantization_block_amd import inputs as I  # noqa: E402
from fp4_quantization_block_amd import mx  # noqa: E402

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "fp4": 10100.0,   # dense scaled MFMA
                    "f16": 2500.0}                    # dense f16 MFMA (the nvfp GEMM)

# HBM-side bytes per launch of the roofline kernel, from rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE passes (KiB per dispatch) scaled by what the same
# counters read for a 512 MiB device copy (x2.0 and x1.0); the summary and
# commands are in profiles/.  Keyed by the SHA-256 of the kernel's source
# file at measurement time: a changed kernel reports null until re-measured.
MEASURED_TRAFFIC = {
    "moss": {"source": "gemm.hip", "sha256": "67670a25d4abdb9c",
             "fetch_kib": 50812.5, "write_kib": 32794.6},
    # the GEMM launches of one step together (six GEMMs, the last one's final
    # partial round of tiles as a second launch; the roofline's unit here)
    "llama": {"source": "gemm.hip", "sha256": "67670a25d4abdb9c",
              "fetch_kib": 3202689.4, "write_kib": 1164633.2},
    # the GEMM call's two launches (a full round of 256x256 tiles, then the
    # last tile rows as 256x128 half tiles)
    "fp4": {"source": "gemm.hip", "sha256": "67670a25d4abdb9c",
            "fetch_kib": 174302.8, "write_kib": 49157.1},
    "mxout": {"source": "gemm.hip", "sha256": "67670a25d4abdb9c",
              "fetch_kib": 50868.4, "write_kib": 20211.6},
    "c1": {"source": "gemm.hip", "sha256": "67670a25d4abdb9c",
           "fetch_kib": 81.7, "write_kib": 128.0},
    # the prediction call (k_amax_partial2 + k_predict_scale)
    "autoscale": {"source": "quant.hip", "sha256": "64f4e1144aaa3582",
                  "fetch_kib": 32815.3, "write_kib": 32.0},
    # the dual-layout quantizer (k_quant_tile_dma)
    "dual": {"source": "quant.hip", "sha256": "64f4e1144aaa3582",
             "fetch_kib": 229533.1, "write_kib": 496635.9},
    # k_nv_gemm
    "nvfp_global": {"source": "nvfp.hip", "sha256": "db29b3bad8a50855",
                    "fetch_kib": 193854.3, "write_kib": 232288.5},
    "nvfp_local": {"source": "nvfp.hip", "sha256": "db29b3bad8a50855",
                   "fetch_kib": 193857.4, "write_kib": 232298.3},
    # k_optstate_quant (the slower of the step's two kernels)
    "coat": {"source": "optstate.hip", "sha256": "48a84d40d196f9f8",
             "fetch_kib": 229452.1, "write_kib": 122898.1},
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


class Timer:
    """HIP events around launches on the current stream."""

    def __init__(self):
        self.samples = {}

    def run(self, name, fn):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        out = fn()
        e.record()
        self.samples.setdefault(name, []).append((s, e))
        return out

    def mean_ms(self, name):
        return float(np.mean([s.elapsed_time(e) for s, e in self.samples[name]]))

    def spread_ms(self, name):
        """(median, min) of the calls' durations."""
        v = [s.elapsed_time(e) for s, e in self.samples[name]]
        return float(np.median(v)), float(np.min(v))


# ------------------------------------------------------------------ workloads
def setup_moss(args):
    w = I.make("moss_two_level_4096")
    A = to_dev(w.tensors["A"])            # [M][K]
    B = to_dev(w.tensors["B"])            # [K][N]
    M, K = A.shape
    N = B.shape[1]
    cfg = mx.qconfig("e4m3", two_level=True)
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((N, K // 32), dtype=torch.uint8, device="cuda")
    ta = torch.empty(1, dtype=torch.float32, device="cuda")
    tb = torch.empty(1, dtype=torch.float32, device="cuda")
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step(t):
        t.run("quant_A", lambda: mx.mx_quantize(A, mx.MX_AXIS_ROW, cfg, qa, sa, ta))
        t.run("quant_B", lambda: mx.mx_quantize(B, mx.MX_AXIS_COL, cfg, qb, sb, tb))
        t.run("gemm", lambda: mx.mx_gemm(qa, sa, ta, "e4m3", qb, sb, tb, "e4m3", M, N, K,
                                         out_dtype=mx.MX_OUT_BF16, c=C))

    flops = 2.0 * M * N * K
    # algorithmic bytes of one two-level quantize of an R x C bf16 tensor:
    # amax pass (2 B/elem) + quantize pass (2 B read + 1 B code + 1/32 B scale)
    qbytes = lambda R, Cc: 2 * R * Cc + 2 * R * Cc + R * Cc + R * Cc // 32
    info = dict(flops=flops, qbytes={"quant_A": qbytes(M, K), "quant_B": qbytes(K, N)},
                gemm_kernel="gemm", mfma="fp8",
                config={"workload": "moss_two_level_e4m3_gemm_4096", "M": M, "N": N, "K": K,
                        "a": "bf16 student-t(3), 4 K-channels x100", "b": "bf16 N(0,0.02)",
                        "elem": "e4m3", "scales": "fp32 tensor + e8m0 1x32", "out": "bf16"},
                host=w.tensors)
    return step, info


def setup_c1(args):
    """MXFP8 GEMM 256^3 (fp32 A, B ~ N(0, 1); E4M3 row copy of A, column copy
    of B, round to nearest; bf16 out): the smallest configuration, dominated
    by launch and single-tile latency."""
    w = I.make("mxfp8_gemm_256")
    A, B = to_dev(w.tensors["A"]), to_dev(w.tensors["B"])
    M, K = A.shape
    N = B.shape[1]
    cfg = mx.qconfig("e4m3")
    qa, sa, _ = mx.mx_quantize(A, mx.MX_AXIS_ROW, cfg)
    qb, sb, _ = mx.mx_quantize(B, mx.MX_AXIS_COL, cfg)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step(t):
        t.run("quant_A", lambda: mx.mx_quantize(A, mx.MX_AXIS_ROW, cfg, qa, sa))
        t.run("quant_B", lambda: mx.mx_quantize(B, mx.MX_AXIS_COL, cfg, qb, sb))
        t.run("gemm", lambda: mx.mx_gemm(qa, sa, None, "e4m3", qb, sb, None, "e4m3", M, N, K,
                                         out_dtype=mx.MX_OUT_BF16, c=C))

    qbytes = lambda R, Cc: 4 * R * Cc + R * Cc + R * Cc // 32      # fp32 in, E4M3 codes + scales out
    info = dict(flops=2.0 * M * N * K, qbytes={"quant_A": qbytes(M, K), "quant_B": qbytes(K, N)},
                gemm_kernel="gemm", mfma="fp8",
                config={"workload": "mxfp8_gemm_256", "M": M, "N": N, "K": K, "elem": "e4m3",
                        "scales": "e8m0 1x32", "out": "bf16"}, host=w.tensors)
    return step, info


def setup_dual(args):
    w = I.make("dual_layout_16384x14336")
    X = to_dev(w.tensors["X"])
    R, Cc = X.shape
    cfg = mx.qconfig("e4m3")
    outs = [torch.empty((R, Cc), dtype=torch.uint8, device="cuda"),
            torch.empty((R, Cc // 32), dtype=torch.uint8, device="cuda"),
            torch.empty((Cc, R), dtype=torch.uint8, device="cuda"),
            torch.empty((Cc, R // 32), dtype=torch.uint8, device="cuda")]

    def step(t):
        t.run("dual", lambda: mx.mx_quantize_dual_layout(X, cfg, *outs))

    info = dict(flops=0.0, qbytes={"dual": 2 * R * Cc + 2 * R * Cc + 2 * R * Cc // 32},
                gemm_kernel=None, mfma=None,
                config={"workload": "dual_layout_e4m3_16384x14336", "R": R, "C": Cc},
                host=w.tensors)
    return step, info


def setup_mxout(args):
    """The MOSS two-level step with the GEMM writing its output already
    MX-quantized (E4M3 codes [M][N] + E8M0 scales [M][N/32]) for the next
    layer instead of bf16."""
    step0, info = setup_moss(args)
    w = info["host"]
    A, B = to_dev(w["A"]), to_dev(w["B"])
    M, K = A.shape
    N = B.shape[1]
    cfg = mx.qconfig("e4m3", two_level=True)
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((N, K // 32), dtype=torch.uint8, device="cuda")
    ta = torch.empty(1, dtype=torch.float32, device="cuda")
    tb = torch.empty(1, dtype=torch.float32, device="cuda")
    qc = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    sc = torch.empty((M, N // 32), dtype=torch.uint8, device="cuda")

    def step(t):
        t.run("quant_A", lambda: mx.mx_quantize(A, mx.MX_AXIS_ROW, cfg, qa, sa, ta))
        t.run("quant_B", lambda: mx.mx_quantize(B, mx.MX_AXIS_COL, cfg, qb, sb, tb))
        t.run("gemm", lambda: mx.mx_gemm_quantized(qa, sa, ta, "e4m3", qb, sb, tb, "e4m3", M, N, K,
                                                   out_fmt="e4m3", qc=qc, sc=sc))

    info = dict(info)
    info["config"] = dict(info["config"], workload="moss_two_level_e4m3_gemm_4096_mx_output",
                          out="e4m3 codes + e8m0 1x32 scales")
    return step, info


def setup_autoscale(args):
    """MOSS weight auto-scaling: the next step's per-tensor scale predicted
    from this step's weight W and gradient G (one read of each), then the
    updated weight W - lr*G quantized to its column copy with that scale
    provided -- no amax pass over the new weight."""
    w = I.make("moss_weight_autoscale_4096")
    W, G = to_dev(w.tensors["W"]), to_dev(w.tensors["G"])
    lr = w.meta["lr"]
    K, N = W.shape
    W2 = (W.float() - lr * G.float()).to(torch.bfloat16)       # the update (not timed)
    work = torch.empty(int(mx.load().mx_predict_workspace_bytes()), dtype=torch.uint8, device="cuda")
    s = torch.empty(1, dtype=torch.float32, device="cuda")
    cfg = mx.qconfig("e4m3", two_level=True, tscale_provided=True)
    q = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sc = torch.empty((N, K // 32), dtype=torch.uint8, device="cuda")

    def step(t):
        t.run("predict", lambda: mx.mx_predict_tensor_scale(W, G, lr, "e4m3", work=work, scale_out=s))
        t.run("quant_W", lambda: mx.mx_quantize(W2, mx.MX_AXIS_COL, cfg, q, sc, tensor_scale=s))

    info = dict(flops=0.0, qbytes={"predict": 2 * 2 * K * N, "quant_W": 2 * K * N + K * N + K * N // 32},
                gemm_kernel=None, mfma=None,
                config={"workload": "moss_weight_autoscale_e4m3_4096", "K": K, "N": N, "lr": lr},
                host=w.tensors)
    return step, info


def setup_coat(args):
    """COAT FP8 optimizer states: Adam's first and second moments of the
    Llama-3-8B gate-up weight (4096 x 28672 fp32 each) held as E4M3 codes
    with per-group (128) dynamic range expansion.  One step reads both
    states back (dequantize) and stores them again (quantize) -- the
    optimizer's read-modify-write of its states without the update
    arithmetic."""
    w = I.make("coat_optstate_llama_wgu")
    G = 128
    st = {}
    for name in ("m", "v"):
        x = torch.from_numpy(w.tensors[name].ravel()).cuda()
        q, amax, k = mx.mx_quantize_optstate(x, "e4m3", G)
        st[name] = (x, q, amax, k, torch.empty_like(x))

    def step(t):
        for name, (x, q, amax, k, out) in st.items():
            t.run("dequant_" + name, lambda q=q, amax=amax, k=k, out=out: mx.mx_dequantize_optstate(
                q, amax, k, "e4m3", G, out=out))
            t.run("quant_" + name, lambda x=x, q=q, amax=amax, k=k: mx.mx_quantize_optstate(
                x, "e4m3", G, q=q, amax=amax, kexp=k))

    n = w.tensors["m"].size
    # per element 4 bytes of fp32 and 1 code byte; 8 bytes of parameters per group
    b = 4 * n + n + 8 * (n // G)
    # the roofline line is the quantizer's, the slower of the two kernels
    info = dict(flops=0.0, qbytes={f"{op}_{s_}": b for op in ("dequant", "quant") for s_ in ("m", "v")},
                gemm_kernel=None, mfma=None, roofline_call="quant_m",
                config={"workload": "coat_fp8_optimizer_states_llama3_8b_wgu", "elements_per_state": n,
                        "group": G, "elem": "e4m3 + e4m3", "states": "adam m, v (fp32)"},
                host=w.tensors)
    return step, info


def setup_fp4(args):
    w = I.make("mxfp4_wgrad_qkv")
    dY = to_dev(w.tensors["dY"])          # [T][Q]
    X = to_dev(w.tensors["X"])            # [T][H]
    T, Q = dY.shape
    H = X.shape[1]
    cfg = mx.qconfig("e2m1", sr=True, hadamard=True, seed=I.SR_SEED)
    qa = torch.empty((Q, T // 2), dtype=torch.uint8, device="cuda")
    sa = torch.empty((Q, T // 32), dtype=torch.uint8, device="cuda")
    qb = torch.empty((H, T // 2), dtype=torch.uint8, device="cuda")
    sb = torch.empty((H, T // 32), dtype=torch.uint8, device="cuda")
    C = torch.empty((Q, H), dtype=torch.bfloat16, device="cuda")

    def step(t):
        t.run("quant_dY", lambda: mx.mx_quantize(dY, mx.MX_AXIS_COL, cfg, qa, sa))
        t.run("quant_X", lambda: mx.mx_quantize(X, mx.MX_AXIS_COL, cfg, qb, sb))
        t.run("gemm", lambda: mx.mx_gemm(qa, sa, None, "e2m1", qb, sb, None, "e2m1", Q, H, T,
                                         hadamard_k=True, out_dtype=mx.MX_OUT_BF16, c=C))

    qb_ = lambda R, Cc: 2 * R * Cc + R * Cc // 2 + R * Cc // 32
    info = dict(flops=2.0 * Q * H * T, qbytes={"quant_dY": qb_(T, Q), "quant_X": qb_(T, H)},
                gemm_kernel="gemm", mfma="fp4",
                config={"workload": "mxfp4_wgrad_qkv", "M": Q, "N": H, "K": T}, host=w.tensors)
    return step, info


# the six training GEMMs of one Llama-3-8B MLP layer: (name, A tensor, A copy,
# A format, B tensor, B copy, B format); C[M][N] = A[M][K] . B[N][K]^T with
# both operands K-contiguous, as the dual-layout quantizer writes them
LLAMA_GEMMS = [
    ("fprop_gate_up", "X", "row", "e4m3", "W_gu", "col", "e4m3"),
    ("fprop_down", "Xp", "row", "e4m3", "W_d", "col", "e4m3"),
    ("dgrad_gate_up", "dY_gu", "row", "e5m2", "W_gu", "row", "e4m3"),
    ("dgrad_down", "dY_d", "row", "e5m2", "W_d", "row", "e4m3"),
    ("wgrad_gate_up", "X", "col", "e4m3", "dY_gu", "col", "e5m2"),
    ("wgrad_down", "Xp", "col", "e4m3", "dY_d", "col", "e5m2"),
]


def setup_llama(args):
    """Llama-3-8B-shaped MLP training step (tokens 8192, hidden 4096, ffn
    14336): dual-layout quantization of the six operand tensors (E4M3 for
    activations and weights, E5M2 for gradients), then the six GEMMs."""
    w = I.make("llama3_8b_mlp")
    fmts = {"X": "e4m3", "Xp": "e4m3", "W_gu": "e4m3", "W_d": "e4m3", "dY_gu": "e5m2", "dY_d": "e5m2"}
    src, outs = {}, {}
    for name, fmt in fmts.items():
        x = to_dev(w.tensors[name])
        R, Cc = x.shape
        src[name] = x
        outs[name] = (torch.empty((R, Cc), dtype=torch.uint8, device="cuda"),
                      torch.empty((R, Cc // 32), dtype=torch.uint8, device="cuda"),
                      torch.empty((Cc, R), dtype=torch.uint8, device="cuda"),
                      torch.empty((Cc, R // 32), dtype=torch.uint8, device="cuda"))
    gemms, flops = [], 0.0
    for gname, an, aax, fa, bn, bax, fb in LLAMA_GEMMS:
        A, B = src[an], src[bn]
        M = A.shape[0] if aax == "row" else A.shape[1]
        K = A.shape[1] if aax == "row" else A.shape[0]
        N = B.shape[1] if bax == "col" else B.shape[0]
        qa, sa = outs[an][:2] if aax == "row" else outs[an][2:]
        qb, sb = outs[bn][:2] if bax == "row" else outs[bn][2:]
        C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        gemms.append((gname, qa, sa, fa, qb, sb, fb, M, N, K, C))
        flops += 2.0 * M * N * K

    def step(t):
        for name, fmt in fmts.items():
            t.run("quant_" + name, lambda name=name, fmt=fmt: mx.mx_quantize_dual_layout(
                src[name], mx.qconfig(fmt), *outs[name]))
        for gname, qa, sa, fa, qb, sb, fb, M, N, K, C in gemms:
            t.run(gname, lambda qa=qa, sa=sa, fa=fa, qb=qb, sb=sb, fb=fb, M=M, N=N, K=K, C=C: mx.mx_gemm(
                qa, sa, None, fa, qb, sb, None, fb, M, N, K, out_dtype=mx.MX_OUT_BF16, c=C))

    # per element: 2 bytes read, a code byte in each copy, two scale bytes per 32
    qbytes = {"quant_" + n: 4 * int(src[n].numel()) + 2 * (int(src[n].numel()) // 32) for n in fmts}
    info = dict(flops=flops, qbytes=qbytes, gemm_kernel=[g[0] for g in gemms], mfma="fp8",
                config={"workload": "llama3_8b_mlp_train", "tokens": 8192, "hidden": 4096, "ffn": 14336,
                        "gemms": [g[0] for g in gemms], "elem": "e4m3 (x, w) / e5m2 (dy)",
                        "quantizer": "dual layout, 1x32 + 32x1 e8m0", "out": "bf16"},
                host=w.tensors, gemms=gemms, fmts=fmts, outs=outs)
    return step, info


def _setup_nvfp(local):
    """nvfp route on the Llama-3-8B gate projection (Y = X W, X [8192][4096]
    activations with outlier channels, W [4096][14336]): NVFP4 row copy of
    X, column copy of W (global or CTA-local second-level scales), then the
    GEMM that consumes them (bf16 out)."""
    w = I.make("nvfp_llama3_8b_gate")
    X, W = to_dev(w.tensors["X"]), to_dev(w.tensors["W"])
    T, H = X.shape
    F = W.shape[1]
    qa, sa, ta = mx.mx_quantize_nvfp(X, mx.MX_AXIS_ROW, local)
    qb, sb, tb = mx.mx_quantize_nvfp(W, mx.MX_AXIS_COL, local)
    C = torch.empty((T, F), dtype=torch.bfloat16, device="cuda")

    def step(t):
        t.run("quant_X", lambda: mx.mx_quantize_nvfp(X, mx.MX_AXIS_ROW, local, qa, sa, ta))
        t.run("quant_W", lambda: mx.mx_quantize_nvfp(W, mx.MX_AXIS_COL, local, qb, sb, tb))
        t.run("gemm", lambda: mx.mx_gemm_nvfp(qa, sa, ta, local, qb, sb, tb, local, T, F, H,
                                              out_dtype=mx.MX_OUT_BF16, c=C))

    # per element 0.5 code byte and 1/16 scale byte written; the source read
    # once per pass: two passes for the global scale (the tensor's amax must
    # be known first), one for panel-local scales
    passes = 1 if local else 2
    qb_ = lambda n: passes * 2 * n + n // 2 + n // 16
    info = dict(flops=2.0 * T * F * H, qbytes={"quant_X": qb_(T * H), "quant_W": qb_(H * F)},
                gemm_kernel="gemm", mfma="f16", kernel_name="k_nv_gemm (f16 MFMA, exact in-loop dequantization)",
                config={"workload": f"nvfp_{'local' if local else 'global'}_llama3_8b_gate", "M": T, "N": F,
                        "K": H, "elem": "e2m1, e4m3 scale per 16, fp32 second-level scale "
                        + ("per 32-row panel" if local else "per tensor"), "out": "bf16"},
                host=w.tensors)
    return step, info


def setup_nvfp_global(args):
    return _setup_nvfp(False)


def setup_nvfp_local(args):
    return _setup_nvfp(True)


def setup_copy(args):
    """A plain 512 MiB device copy: the reference that scales the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) of a profiling run."""
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)

    def step(t):
        t.run("copy", lambda: dst.copy_(src))

    info = dict(flops=0.0, qbytes={"copy": 2 * n}, gemm_kernel=None, mfma=None,
                config={"workload": "device_copy_512MiB", "bytes_read": n, "bytes_written": n},
                host={})
    return step, info


WORKLOADS = {"c1": setup_c1, "moss": setup_moss, "dual": setup_dual, "fp4": setup_fp4, "llama": setup_llama,
             "copy": setup_copy, "autoscale": setup_autoscale, "mxout": setup_mxout, "coat": setup_coat,
             "nvfp_global": setup_nvfp_global, "nvfp_local": setup_nvfp_local}


# ------------------------------------------------------------------ CPU baseline
def cpu_baseline_moss(host, chunk=256, budget_s=20.0):
    """The oracle (plain C, all host cores) on the step: two-level
    quantization of the full A and B, then the GEMM in chunks of `chunk`
    rows of C until all M rows are done or `budget_s` seconds have passed
    (the GEMM time is then scaled to all M rows, and the sample says so)."""
    import oracle as O
    n = os.cpu_count() or 1
    A, B = host["A"], host["B"]
    M, K = A.shape
    N = B.shape[1]
    t0 = time.perf_counter()
    qa, sa, ta = O.quantize(A, O.AXIS_ROW, "e4m3", two_level=1, nthreads=n)
    qb, sb, tb = O.quantize(B, O.AXIS_COL, "e4m3", two_level=1, nthreads=n)
    t1 = time.perf_counter()
    done = 0
    while done < M:
        rows = min(chunk, M - done)
        O.gemm(qa[done:done + rows], sa[done:done + rows], ta, "e4m3", qb, sb, tb, "e4m3", rows, N, K,
               nthreads=n)
        done += rows
        if time.perf_counter() - t1 > budget_s:
            break
    t2 = time.perf_counter()
    step_s = (t1 - t0) + (t2 - t1) * (M / done)
    gemm_part = (f"GEMM, all {M} rows ({t2 - t1:.2f} s)" if done == M else
                 f"GEMM rows 0..{done - 1} of {M} ({t2 - t1:.2f} s, scaled to all rows)")
    return {"value": round(2.0 * M * N * K / step_s / 1e12, 6), "unit": "TFLOP/s", "cores": n,
            "kind": "oracle",
            "sample": f"two-level quantize of full A and B ({t1 - t0:.2f} s) + {gemm_part}"}


def cpu_baseline_llama(info, rows_per_gemm=256, per_tile=16):
    """The oracle (plain C, all host cores) on the step: dual-layout
    quantization of all six tensors in full, then the first
    `rows_per_gemm` rows of C of each GEMM (the oracle's whole-matrix
    routine on that row block), the GEMM time scaled to all rows.

    Separately (not timed), 16 entries of every 128x128 output tile of each
    GEMM, corners included, from the oracle and from the GPU's fp32-output
    GEMM (run once) give each GEMM's largest error relative to the stated
    bound |C - C_ref| <= 1e-5 (|A|.|B|) + 1e-6 and the fraction of entries
    inside it."""
    import oracle as O
    n = os.cpu_count() or 1
    host = info["host"]
    t0 = time.perf_counter()
    ora = {}
    for name, fmt in info["fmts"].items():
        qr, sr_, _ = O.quantize(host[name], O.AXIS_ROW, fmt, nthreads=n)
        qc, sc, _ = O.quantize(host[name], O.AXIS_COL, fmt, nthreads=n)
        ora[name] = {"row": (qr, sr_), "col": (qc, sc)}
    tq = time.perf_counter() - t0
    tg_sample, tg_full, macs = 0.0, 0.0, 0
    for (gname, an, aax, fa, bn, bax, fb), g in zip(LLAMA_GEMMS, info["gemms"]):
        M, N, K = g[7], g[8], g[9]
        qao, sao = ora[an][aax]
        qbo, sbo = ora[bn][bax]
        r = min(rows_per_gemm, M)
        t1 = time.perf_counter()
        O.gemm(qao[:r], sao[:r], None, fa, qbo, sbo, None, fb, r, N, K, nthreads=n)
        dt = time.perf_counter() - t1
        tg_sample += dt
        tg_full += dt * M / r
        macs += r * N * K
    step_s = tq + tg_full
    base = {"value": round(info["flops"] / step_s / 1e12, 6), "unit": "TFLOP/s", "cores": n, "kind": "oracle",
            "sample": (f"dual-layout quantization of all six tensors in full ({tq:.2f} s) + the first "
                       f"{rows_per_gemm} rows of C of each GEMM ({macs:.3g} MACs, {tg_sample:.2f} s), GEMM "
                       f"time scaled to all rows ({tg_full:.1f} s)")}
    rng = np.random.default_rng(7)
    parity = {}
    for (gname, an, aax, fa, bn, bax, fb), g in zip(LLAMA_GEMMS, info["gemms"]):
        _, qa, sa, _, qb, sb, _, M, N, K, _ = g
        qao, sao = ora[an][aax]
        qbo, sbo = ora[bn][bax]
        ii, jj = I.sample_tile_entries(rng, M, N, per_tile)
        Cref, bound = O.gemm_entries(qao, sao, None, fa, qbo, sbo, None, fb, M, N, K, ii, jj, nthreads=n)
        c = mx.mx_gemm(qa, sa, None, fa, qb, sb, None, fb, M, N, K, out_dtype=mx.MX_OUT_F32)
        got = c[torch.from_numpy(ii).cuda(), torch.from_numpy(jj).cuda()].double().cpu().numpy()
        del c
        err = np.abs(got - Cref)
        stated = 1e-5 * bound + 1e-6
        parity[gname] = {"max_err_over_stated_bound": round(float((err / stated).max()), 4),
                         "frac_within_stated_bound": round(float(np.mean(err <= stated)), 6),
                         "entries": int(ii.size)}
    return base, parity


def measured_traffic(workload):
    """Bytes per launch of the roofline kernel if the counters match the
    current kernel source, else None."""
    import hashlib
    m = MEASURED_TRAFFIC.get(workload)
    if m is None:
        return None
    src = os.path.join(ROOT, "fp4_quantization_block_amd", "csrc", m["source"])
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if digest != m["sha256"]:
        return None
    return int(round(m["fetch_kib"] * 1024 * 2.0 + m["write_kib"] * 1024 * 1.0))


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="llama", choices=sorted(WORKLOADS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--flush", default="read", choices=["write", "read", "none"],
                   help="how L2/MALL are evicted before each step (outside the timed kernels); a "
                        "512 MiB write leaves the caches full of dirty lines whose write-back then "
                        "lands in the first timed kernel, so the default evicts by reading")
    args = p.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2
    assert torch.cuda.is_available(), "needs a GPU"
    mx.load()
    log(f"workload {args.workload}: generating inputs")
    step, info = WORKLOADS[args.workload](args)
    flush = None if args.flush == "none" else torch.ones(512 << 20, dtype=torch.uint8, device="cuda")

    def one(t):
        if args.flush == "write":
            flush.zero_()
        elif args.flush == "read":
            flush.max()
        step(t)

    warm = Timer()
    for _ in range(args.warmup):
        one(warm)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    t = Timer()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        one(t)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    names = list(t.samples)
    kernel_ms = {n: t.mean_ms(n) for n in names}
    step_ms = sum(kernel_ms.values())
    log("per-call ms:", {k: round(v, 4) for k, v in kernel_ms.items()})

    quant = {}
    for n, b in info["qbytes"].items():
        gbs = b / (kernel_ms[n] * 1e-3) / 1e9
        med, mn = t.spread_ms(n)
        quant[n] = {"ms": round(kernel_ms[n], 4), "ms_median": round(med, 4), "ms_min": round(mn, 4),
                    "GB/s": round(gbs, 1),
                    "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bytes": int(b)}
    if info["gemm_kernel"]:
        gk = info["gemm_kernel"]
        g_ms = sum(kernel_ms[n] for n in gk) if isinstance(gk, list) else kernel_ms[gk]
        g_tf = info["flops"] / (g_ms * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS[info["mfma"]]
        roofline = {"bound": "mfma", "achieved": round(g_tf, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(g_tf / peak, 4), "traffic": measured_traffic(args.workload),
                    "kernel": info.get("kernel_name", f"k_gemm_w4 ({info['mfma']} scaled MFMA)"),
                    "algorithmic": f"{info['flops']:.4g} FLOP per launch"}
        value = info["flops"] / (step_ms * 1e-3) / 1e12
        metric = ("MX GEMM TFLOP/s (% scaled-MFMA peak); mx_quantize GB/s (% HBM peak)" if info["mfma"] != "f16"
                  else "nvfp GEMM TFLOP/s (% f16 MFMA peak); nvfp quantize GB/s (% HBM peak)")
        unit = "TFLOP/s"
    else:
        n = info.get("roofline_call", names[0])
        gbs = info["qbytes"][n] / (kernel_ms[n] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(args.workload),
                    "kernel": {"dual": "k_quant_tile_dma (dual layout)",
                               "autoscale": "k_amax_partial x2 + k_predict_scale",
                               "coat": "k_optstate_quant (first moment)"}.get(args.workload, n)}
        value = gbs
        metric = "mx_quantize GB/s (% HBM peak)"
        unit = "GB/s"
    out = {"metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": {"fp4": "e2m1", "llama": "e4m3/e5m2", "nvfp_global": "e2m1 (f16 MFMA)",
                     "nvfp_local": "e2m1 (f16 MFMA)"}.get(args.workload, "e4m3"),
           "data": "synthetic (seeded; no weights or datasets)",
           "config": info["config"], "roofline": roofline,
           "kernels": quant, "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
           "timing": "HIP events on the launch stream; L2/MALL evicted before each step by a 512 MiB "
                     f"{args.flush} (not timed)" if flush is not None else
                     "HIP events on the launch stream; no cache eviction between steps"}
    if info["gemm_kernel"]:
        out["kernels"]["gemm"] = {"ms": round(g_ms, 4), "TFLOP/s": roofline["achieved"],
                                  "frac_mfma": roofline["frac"]}
        if not isinstance(info["gemm_kernel"], list):
            med, mn = t.spread_ms(info["gemm_kernel"])
            out["kernels"]["gemm"].update({"ms_median": round(med, 4), "ms_min": round(mn, 4)})
        if isinstance(info["gemm_kernel"], list):
            for g in info["gemms"]:
                n, M, N, K = g[0], g[7], g[8], g[9]
                tf = 2.0 * M * N * K / (kernel_ms[n] * 1e-3) / 1e12
                med, mn = t.spread_ms(n)
                out["kernels"][n] = {"ms": round(kernel_ms[n], 4), "ms_median": round(med, 4), "ms_min": round(mn, 4),
                                     "MNK": [M, N, K], "TFLOP/s": round(tf, 1),
                                     "frac_mfma": round(tf / MFMA_PEAK_TFLOPS[info["mfma"]], 4)}
            out["roofline"]["algorithmic"] = (f"{info['flops']:.4g} FLOP over the six launches of one step "
                                              "(achieved = that / the sum of their mean durations)")
    if args.workload == "llama":
        # the six dual quantizations against the HBM roofline; dY_gu has the
        # element count of the standalone 16384x14336 dual-layout workload
        out["kernels"]["dual_layout_bar"] = {"tensor": "dY_gu [8192][28672]",
                                             "frac_hbm": quant["quant_dY_gu"]["frac_hbm"], "target": 0.70}
    if args.workload == "moss" and not args.no_cpu_baseline:
        log("timing the oracle on the host (bounded sample)")
        out["cpu_baseline"] = cpu_baseline_moss(info["host"])
    if args.workload == "llama" and not args.no_cpu_baseline:
        log("timing the oracle on the host (bounded sample)")
        out["cpu_baseline"], out["gemm_parity_sampled"] = cpu_baseline_llama(info)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
