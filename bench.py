"""Benchmark of the NVFP4 hot path on one MI355X.

One step is one pass of the whole path over resident synthetic inputs:
  1. activation fake-quant, bf16 8192x4096, max scaling (quantise -> pack -> dequantise,
     codes and block bytes written too), with the calibrated tensor scale held fixed, on
     four activation batches back to back (per-launch time = stage time / 4);
  2. MSE scale search on a bf16 12288x4096 MLP weight (tensor scale, 3.1M blocks x 126
     candidates) and its final quantisation;
  3. block Hessian of 131072 calibration tokens x 4096 (bf16) and the Local-Hessian search
     on a bf16 4096x4096 projection weight, then its final quantisation;
  4. MoE: routing of 65536 tokens (top-8, Zipf 1.1) into per-expert token lists, per-expert
     block Hessians, tensor scales and Local-Hessian search for 128 experts of 512x2048,
     then their final quantisation;
  5. the tiny configuration (W 64x256 fp32, X 512x256): scale, fake-quant, MSE, block
     Hessian, Local-Hessian (launch-latency bound; reported, not graded).
Headline value: fake-quant GB/s of stage 1 (algorithmic bytes / kernel time). The JSON
line also carries Local-Hessian blocks/s, every stage's time (median over the timed steps)
and roofline, and the CPU oracle timed on a bounded sample of the same workloads.

Rooflines count the work each kernel executes. The searches skip candidates that provably
cannot win, so their executed work comes from the library's search counters, read in a
separate counting pass after the timed steps (the counting kernels are not timed); the
figure for the exhaustive 126-candidate search is kept beside it.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_MFMA_TFLOPS = 157.3       # dense fp32 matrix
FP64_VECTOR_TFLOPS = 78.6      # fp64 vector (FMA = 2 flops)
VALU_LANE_TOPS = 256 * 64 * 2.4e9 / 1e12   # non-packed lane-ops/s: 256 CU x 64 lanes x 2.4 GHz = 39.3
MSE_OPS_PER_EVAL = 5           # compare/select x3, subtract, fma per element x candidate
FQ_BYTES_PER_ELEM = 2 + 2 + 0.5 + 1 / 16   # read bf16, write bf16 + packed code + 1/16 byte
FQ_SETS = 4                    # activation batches fake-quantised per step
CALIB_FRACTION = 0.9999        # activation clip value: this fraction of calibration values
GPTQ_DAMP = 0.01               # GPTQ damping: 1% of the mean diagonal of H
BF16_MFMA_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
FP64_TFLOPS = 78.6             # MI355X fp64 (vector and matrix) peak
STE_CLIP = 8.0               # gradient clamp of the straight-through backward


def _sha_of(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str, source_file: str):
    """HBM traffic per launch from committed rocprofv3 PMC runs, if the kernel source is
    unchanged since they were taken; None otherwise."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            tab = json.load(f)
        ent = tab[kernel_key]
        if ent.get("source_sha") != _sha_of([os.path.join(ROOT, source_file)]):
            return None
        return ent["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


COUNTER_SOURCES = {
    "fakequant_act": "scale_search_weights_amd/csrc/nvfp4_quant.hip",
    "scale_mlp": "scale_search_weights_amd/csrc/nvfp4_quant.hip",
    "scale_proj": "scale_search_weights_amd/csrc/nvfp4_quant.hip",
    "scale_moe": "scale_search_weights_amd/csrc/nvfp4_quant.hip",
    "quantize_mlp": "scale_search_weights_amd/csrc/nvfp4_quant.hip",
    "quantize_proj": "scale_search_weights_amd/csrc/nvfp4_quant.hip",
    "quantize_moe": "scale_search_weights_amd/csrc/nvfp4_quant.hip",
    "mse_mlp": "scale_search_weights_amd/csrc/nvfp4_search.hip",
    "four_over_six_mlp": "scale_search_weights_amd/csrc/nvfp4_search.hip",
    "lh_proj": "scale_search_weights_amd/csrc/nvfp4_search.hip",
    "lh_moe": "scale_search_weights_amd/csrc/nvfp4_search.hip",
    "hessian_proj": "scale_search_weights_amd/csrc/nvfp4_hessian.hip",
    "hessian_moe": "scale_search_weights_amd/csrc/nvfp4_hessian.hip",
    "full_hessian_proj": "scale_search_weights_amd/csrc/nvfp4_gram.hip",
}


def load_counters():
    """Per-stage counter figures (VALU issue, MFMA busy, HBM bytes per launch) from the
    committed rocprofv3 runs in profiles/counters.json, for the stages whose kernel source
    is unchanged since they were taken."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return {}
    out = {}
    for key, ent in tab.get("stages", {}).items():
        src = COUNTER_SOURCES.get(key)
        if src and ent.get("source_sha") == _sha_of([os.path.join(ROOT, src)]):
            out[key] = {k: v for k, v in ent.items() if k != "source_sha"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="(default) run a plain 1 GiB device copy: the measured HBM ceiling, "
                         "and the reference for PMC byte-counter scaling")
    ap.add_argument("--no-copy", action="store_true", help="skip the 1 GiB device copy")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from scale_search_weights_amd import nvfp4, synth

    L = nvfp4.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    st = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(st.cuda_stream)

    def P(t):
        return ctypes.c_void_p(t.data_ptr()) if t is not None else None

    def ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {nvfp4.status_string(rc)}")

    BF16 = nvfp4.DTYPE_BF16
    t_setup = time.time()
    # ---------------------------------------------------------------- inputs (resident)
    a2 = synth.activation(0).to(dev)                       # [8192, 4096]
    r2, c2 = a2.shape
    S2 = nvfp4.global_scale(a2)                            # calibrated, held fixed
    # FQ_SETS activation batches per step, each with its own buffers (584 MB in all, more
    # than the 256 MB Infinity Cache), quantised back to back so the per-launch time is
    # the kernel's own and no input is served from cache
    a2s = [a2] + [synth.activation(k).to(dev) for k in range(1, FQ_SETS)]
    y2s = [torch.empty_like(a2) for _ in range(FQ_SETS)]
    codes2s = [torch.empty(r2, c2 // 2, dtype=torch.uint8, device=dev) for _ in range(FQ_SETS)]
    sc2s = [torch.empty(r2, c2 // 16, dtype=torch.uint8, device=dev) for _ in range(FQ_SETS)]

    # static calibration: every step adds one activation batch to a running histogram
    hist2 = torch.zeros(nvfp4.CALIB_BINS, dtype=torch.int64, device=dev)
    S2c = torch.empty(1, dtype=torch.float32, device=dev)

    # training support: the straight-through backward of the activation's fake-quant
    # (gradient clamped to +-CLIP) and the moving-average update of its tensor scale
    g2 = a2s[1]                                            # stands in for dL/dy
    gx2 = torch.empty_like(g2)
    S2run = S2.clone()

    w3 = synth.mlp_weight(0).to(dev)                       # [12288, 4096]
    r3, c3 = w3.shape
    S3 = torch.empty(1, dtype=torch.float32, device=dev)
    sc3 = torch.empty(r3, c3 // 16, dtype=torch.uint8, device=dev)
    sc3b = torch.empty(r3, c3 // 16, dtype=torch.uint8, device=dev)   # Four Over Six bytes
    codes3 = torch.empty(r3, c3 // 2, dtype=torch.uint8, device=dev)

    w4c, x4c = synth.projection(0)
    w4, x4 = w4c.to(dev), x4c.to(dev)                      # [4096, 4096], [131072, 4096]
    del w4c, x4c
    r4, c4 = w4.shape
    t4 = x4.shape[0]
    H4 = torch.empty(c4 // 16, 16, 16, dtype=torch.float32, device=dev)
    ws4_n = L.nvfp4_block_hessian_workspace_size(t4, c4, 1, 0)
    ws4 = torch.empty(ws4_n, dtype=torch.uint8, device=dev)
    S4 = torch.empty(1, dtype=torch.float32, device=dev)
    sc4 = torch.empty(r4, c4 // 16, dtype=torch.uint8, device=dev)
    codes4 = torch.empty(r4, c4 // 2, dtype=torch.uint8, device=dev)

    # LH + GPTQ on the projection: full Gram matrix, GPTQ factor, GPTQ rounding at the LH bytes
    Hf4 = torch.empty(c4, c4, dtype=torch.float32, device=dev)
    wsf_n = L.nvfp4_full_hessian_workspace_size(t4, c4)
    wsf = torch.empty(wsf_n, dtype=torch.uint8, device=dev)
    U4 = torch.empty(c4, c4, dtype=torch.float64, device=dev)
    st4 = torch.zeros(1, dtype=torch.int32, device=dev)
    wsu_n = L.nvfp4_gptq_factor_workspace_size(c4)
    wsu = torch.empty(wsu_n, dtype=torch.uint8, device=dev)
    wsg_n = L.nvfp4_gptq_workspace_size(r4, c4)
    wsg = torch.empty(wsg_n, dtype=torch.uint8, device=dev)
    codes4g = torch.empty(r4, c4 // 2, dtype=torch.uint8, device=dev)

    w5c, x5c, ids5c = synth.moe(0)
    w5, x5, ids5 = w5c.to(dev), x5c.to(dev), ids5c.to(dev)
    del w5c, x5c
    E, r5, c5 = w5.shape
    t5, topk = ids5.shape
    off5 = torch.empty(E + 1, dtype=torch.int32, device=dev)
    tok5 = torch.empty(t5 * topk, dtype=torch.int32, device=dev)
    wsr_n = L.nvfp4_route_groups_workspace_size(t5, topk, E)
    wsr = torch.empty(max(wsr_n, 4), dtype=torch.uint8, device=dev)
    H5 = torch.empty(E, c5 // 16, 16, 16, dtype=torch.float32, device=dev)
    ws5_n = L.nvfp4_block_hessian_workspace_size(t5, c5, E, t5 * topk)
    ws5 = torch.empty(ws5_n, dtype=torch.uint8, device=dev)
    S5 = torch.empty(E, dtype=torch.float32, device=dev)
    sc5 = torch.empty(E, r5, c5 // 16, dtype=torch.uint8, device=dev)
    codes5 = torch.empty(E, r5, c5 // 2, dtype=torch.uint8, device=dev)
    w1c, x1c = synth.tiny(0)
    w1, x1 = w1c.to(dev), x1c.to(dev)
    r1, c1 = w1.shape
    # workspace of the two-launch tensor scale (per-workgroup partial maxima)
    wsS_n = max(L.nvfp4_global_scale_workspace_size(b_, n_)
                for b_, n_ in ((1, r3 * c3), (1, r4 * c4), (E, r5 * c5), (1, r1 * c1)))
    wsS = torch.empty(wsS_n, dtype=torch.uint8, device=dev)
    t1 = x1.shape[0]
    S1 = torch.empty(1, dtype=torch.float32, device=dev)
    y1 = torch.empty_like(w1)
    codes1 = torch.empty(r1, c1 // 2, dtype=torch.uint8, device=dev)
    sc1 = torch.empty(r1, c1 // 16, dtype=torch.uint8, device=dev)
    sc1m = torch.empty(r1, c1 // 16, dtype=torch.uint8, device=dev)
    sc1l = torch.empty(r1, c1 // 16, dtype=torch.uint8, device=dev)
    H1 = torch.empty(c1 // 16, 16, 16, dtype=torch.float32, device=dev)
    ws1_n = L.nvfp4_block_hessian_workspace_size(t1, c1, 1, 0)
    ws1 = torch.empty(max(ws1_n, 1), dtype=torch.uint8, device=dev)
    F32 = nvfp4.DTYPE_F32
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    # ---------------------------------------------------------------- one step
    stages = {}

    def stage(name, fn):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        fn()
        e1.record(st)
        stages.setdefault(name, []).append((e0, e1))

    def step():
        def fq():
            for k in range(FQ_SETS):
                ok(L.nvfp4_fakequant(P(a2s[k]), BF16, 1, r2, c2, P(S2), None, P(y2s[k]),
                                     P(codes2s[k]), P(sc2s[k]), sptr), "fakequant")
        stage("fakequant_act", fq)
        stage("calib_act", lambda: (ok(L.nvfp4_calib_histogram(P(a2), BF16, r2 * c2, P(hist2), sptr),
                                       "calibration histogram"),
                                    ok(L.nvfp4_calib_scale(P(hist2), ctypes.c_double(CALIB_FRACTION),
                                                           P(S2c), sptr), "calibration scale")))
        stage("ste_act", lambda: (ok(L.nvfp4_ste_backward(P(g2), BF16, r2 * c2, ctypes.c_float(STE_CLIP),
                                                          P(gx2), sptr), "ste backward"),
                                  ok(L.nvfp4_scale_ema(P(S2run), P(S2), 1, ctypes.c_float(0.9), sptr),
                                     "scale ema")))
        stage("scale_mlp", lambda: ok(L.nvfp4_global_scale_ws(P(w3), BF16, 1, r3 * c3, P(S3), P(wsS), wsS_n, sptr), "scale"))
        stage("mse_mlp", lambda: ok(L.nvfp4_scale_search_mse(
            P(w3), BF16, 1, r3, c3, P(S3), P(sc3), None, sptr), "mse"))
        stage("four_over_six_mlp", lambda: ok(L.nvfp4_scale_search_four_over_six(
            P(w3), BF16, 1, r3, c3, P(S3), P(sc3b), None, sptr), "four over six"))
        stage("quantize_mlp", lambda: ok(L.nvfp4_quantize(
            P(w3), BF16, 1, r3, c3, P(S3), P(sc3), P(codes3), None, sptr), "quantize"))
        stage("hessian_proj", lambda: ok(L.nvfp4_block_hessian(
            P(x4), BF16, t4, c4, 1, None, None, 0, P(H4), 0, P(ws4), ws4_n, sptr), "hessian"))
        stage("scale_proj", lambda: ok(L.nvfp4_global_scale_ws(P(w4), BF16, 1, r4 * c4, P(S4), P(wsS), wsS_n, sptr), "scale"))
        stage("lh_proj", lambda: ok(L.nvfp4_scale_search_local_hessian(
            P(w4), BF16, 1, r4, c4, P(S4), P(H4), P(sc4), None, sptr), "lh"))
        stage("quantize_proj", lambda: ok(L.nvfp4_quantize(
            P(w4), BF16, 1, r4, c4, P(S4), P(sc4), P(codes4), None, sptr), "quantize"))
        stage("full_hessian_proj", lambda: ok(L.nvfp4_full_hessian(
            P(x4), BF16, t4, c4, P(Hf4), 0, P(wsf), wsf_n, sptr), "full hessian"))
        stage("gptq_factor_proj", lambda: ok(L.nvfp4_gptq_factor(
            P(Hf4), c4, ctypes.c_double(GPTQ_DAMP), P(U4), P(st4), P(wsu), wsu_n, sptr), "gptq factor"))
        stage("gptq_proj", lambda: ok(L.nvfp4_gptq(
            P(w4), BF16, r4, c4, P(S4), P(sc4), P(U4), P(codes4g), P(wsg), wsg_n, sptr), "gptq"))
        stage("route_moe", lambda: ok(L.nvfp4_route_groups(
            P(ids5), t5, topk, E, P(off5), P(tok5), P(wsr), wsr_n, sptr), "route"))
        stage("hessian_moe", lambda: ok(L.nvfp4_block_hessian(
            P(x5), BF16, t5, c5, E, P(off5), P(tok5), t5 * topk, P(H5), 0, P(ws5), ws5_n, sptr),
            "hessian"))
        stage("scale_moe", lambda: ok(L.nvfp4_global_scale_ws(P(w5), BF16, E, r5 * c5, P(S5), P(wsS), wsS_n, sptr), "scale"))
        stage("lh_moe", lambda: ok(L.nvfp4_scale_search_local_hessian(
            P(w5), BF16, E, r5, c5, P(S5), P(H5), P(sc5), None, sptr), "lh"))
        stage("quantize_moe", lambda: ok(L.nvfp4_quantize(
            P(w5), BF16, E, r5, c5, P(S5), P(sc5), P(codes5), None, sptr), "quantize"))

        def tiny_all():
            ok(L.nvfp4_global_scale_ws(P(w1), F32, 1, r1 * c1, P(S1), P(wsS), wsS_n, sptr), "scale")
            ok(L.nvfp4_fakequant(P(w1), F32, 1, r1, c1, P(S1), None, P(y1), P(codes1), P(sc1), sptr),
               "fakequant")
            ok(L.nvfp4_scale_search_mse(P(w1), F32, 1, r1, c1, P(S1), P(sc1m), None, sptr), "mse")
            ok(L.nvfp4_block_hessian(P(x1), F32, t1, c1, 1, None, None, 0, P(H1), 0, P(ws1), ws1_n,
                                     sptr), "hessian")
            ok(L.nvfp4_scale_search_local_hessian(P(w1), F32, 1, r1, c1, P(S1), P(H1), P(sc1l), None,
                                                  sptr), "lh")
        stage("tiny_all", tiny_all)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stages.clear()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / max(args.steps, 1)

    ms = {k: float(np.median([a.elapsed_time(b) for a, b in v])) for k, v in stages.items()}
    ms["fakequant_act"] /= FQ_SETS  # per launch

    # counting pass (not timed): the work the searches execute on these inputs
    L.nvfp4_search_stats_enable(1)
    counts = {}
    for name, fn in (("mse_mlp", lambda: L.nvfp4_scale_search_mse(P(w3), BF16, 1, r3, c3, P(S3), P(sc3),
                                                                   None, sptr)),
                     ("lh_proj", lambda: L.nvfp4_scale_search_local_hessian(
                         P(w4), BF16, 1, r4, c4, P(S4), P(H4), P(sc4), None, sptr)),
                     ("lh_moe", lambda: L.nvfp4_scale_search_local_hessian(
                         P(w5), BF16, E, r5, c5, P(S5), P(H5), P(sc5), None, sptr))):
        ok(fn(), name)
        counts[name] = nvfp4.search_stats_read()
    L.nvfp4_search_stats_enable(0)

    copy_gbs = None
    if not args.no_copy:
        # a plain device copy of known size: its byte counters scale FETCH/WRITE_SIZE, and
        # its rate is the practical HBM ceiling on this machine
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        ce = []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            dst.copy_(src)
            e1.record(st)
            ce.append((e0, e1))
        torch.cuda.synchronize()
        copy_gbs = 2 * (1 << 30) / (min(a.elapsed_time(b) for a, b in ce) * 1e-3) / 1e9

    # peak rates this device sustains: loops of independent MFMA / VALU instructions (a
    # separate probe library), two workgroups of four waves per CU
    probe_rates = {}
    if not args.no_copy:
        pl = ctypes.CDLL(os.path.join(os.path.dirname(nvfp4.__file__), "libnvfp4_probe.so"))
        pl.nvfp4_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        blocks = 2 * cus
        pbuf = torch.empty(blocks * 256, dtype=torch.float64, device=dev)
        # kind: (name, work per wave instruction, iterations); 8 instructions per iteration
        for kind, (name, per_inst, iters) in enumerate((("mfma_f64_tflops", 2048, 2000),
                                                         ("mfma_bf16_tflops", 32768, 4000),
                                                         ("mfma_f32_tflops", 2048, 4000),
                                                         ("valu_lane_tops", 64, 40000))):
            ok(pl.nvfp4_probe_run(kind, blocks, iters, P(pbuf), sptr), "probe")
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            ok(pl.nvfp4_probe_run(kind, blocks, iters, P(pbuf), sptr), "probe")
            e1.record(st)
            torch.cuda.synchronize()
            work = per_inst * 8.0 * iters * blocks * 4
            probe_rates[name] = round(work / (e0.elapsed_time(e1) * 1e-3) / 1e12, 2)

    # ---------------------------------------------------------------- figures
    fq_bytes = r2 * c2 * FQ_BYTES_PER_ELEM
    fq_gbs = fq_bytes / (ms["fakequant_act"] * 1e-3) / 1e9
    n_lh4 = r4 * (c4 // 16)
    n_lh5 = E * r5 * (c5 // 16)
    lh4_time = ms["hessian_proj"] + ms["lh_proj"]
    lh4_blocks_s = n_lh4 / (lh4_time * 1e-3)
    lh5_time = ms["route_moe"] + ms["hessian_moe"] + ms["lh_moe"]
    lh5_blocks_s = n_lh5 / (lh5_time * 1e-3)
    gram_flops = t4 * c4 * (c4 + 1)                 # 2 T flops per unique entry of X^T X
    factor_flops = 4 * c4 ** 3 / 3                  # Cholesky + triangular inverse
    gptq_flops = r4 * c4 * c4                       # rows x n^2 / 2 multiply-adds

    def roof(bound, achieved, peak, unit, traffic=None, **extra):
        r = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
             "frac": round(achieved / peak, 4), "traffic": traffic}
        r.update(extra)
        return r

    def hbm(name, nbytes, **extra):
        return roof("hbm", nbytes / (ms[name] * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", **extra)

    def search_roof(name, w_bytes, exhaustive_evals, evals, mfma_flops_per_eval):
        """A search priced by the work it executes: per evaluated candidate, 16 elements x
        MSE_OPS_PER_EVAL non-packed VALU lane-ops (the evaluation cost model) and, for the
        Local-Hessian quadratic form, mfma_flops_per_eval fp32 MFMA flops; plus its HBM bytes.
        The binding unit is the one whose time at peak is largest."""
        t = ms[name] * 1e-3
        t_valu = evals * 16 * MSE_OPS_PER_EVAL / (VALU_LANE_TOPS * 1e12)
        t_mfma = evals * mfma_flops_per_eval / (FP32_MFMA_TFLOPS * 1e12)
        t_hbm = w_bytes / (HBM_PEAK_GBS * 1e9)
        extra = {"evaluations": int(evals), "exhaustive_evaluations": int(exhaustive_evals),
                 "hbm_frac": round(t_hbm / t, 4),
                 "exhaustive_equivalent_frac": round(t_valu * exhaustive_evals / max(evals, 1) / t
                                                     if mfma_flops_per_eval == 0 else
                                                     t_mfma * exhaustive_evals / max(evals, 1) / t, 4)}
        if t_mfma >= max(t_valu, t_hbm):
            return roof("mfma", evals * mfma_flops_per_eval / t / 1e12, FP32_MFMA_TFLOPS, "TFLOP/s", **extra)
        if t_valu >= t_hbm:
            return roof("alu", evals * 16 * MSE_OPS_PER_EVAL / t / 1e12, round(VALU_LANE_TOPS, 2), "TOP/s",
                        **extra)
        return roof("hbm", w_bytes / t / 1e9, HBM_PEAK_GBS, "GB/s", **extra)

    quant = "scale_search_weights_amd/csrc/nvfp4_quant.hip"
    fq_traffic = load_traffic("fakequant_act", quant)
    n_blk3 = r3 * (c3 // 16)
    rooflines = {
        "fakequant_act": hbm("fakequant_act", fq_bytes, traffic=fq_traffic),
        "calib_act": hbm("calib_act", r2 * c2 * 2),
        "ste_act": hbm("ste_act", r2 * c2 * 2 * 2),
        "scale_mlp": hbm("scale_mlp", r3 * c3 * 2),
        "mse_mlp": search_roof("mse_mlp", r3 * c3 * 2 + n_blk3, n_blk3 * 126,
                               counts["mse_mlp"]["mse_evals"], 0),
        "four_over_six_mlp": hbm("four_over_six_mlp", r3 * c3 * 2 + n_blk3),
        "quantize_mlp": hbm("quantize_mlp", r3 * c3 * (2 + 0.5 + 1 / 16)),
        "hessian_proj": hbm("hessian_proj", t4 * c4 * 2),
        "scale_proj": hbm("scale_proj", r4 * c4 * 2),
        "lh_proj": search_roof("lh_proj", r4 * c4 * 2 + (c4 // 16) * 1024 + n_lh4, n_lh4 * 126,
                               counts["lh_proj"]["lh_screened"], 512),
        "quantize_proj": hbm("quantize_proj", r4 * c4 * (2 + 0.5 + 1 / 16)),
        "full_hessian_proj": roof("mfma", gram_flops / (ms["full_hessian_proj"] * 1e-3) / 1e12,
                                  BF16_MFMA_TFLOPS, "TFLOP/s"),
        "gptq_factor_proj": roof("mfma", factor_flops / (ms["gptq_factor_proj"] * 1e-3) / 1e12,
                                 FP64_TFLOPS, "TFLOP/s"),
        "gptq_proj": roof("mfma", gptq_flops / (ms["gptq_proj"] * 1e-3) / 1e12, FP64_TFLOPS,
                          "TFLOP/s"),
        # the grouped Hessian needs every routed row, but each token row is one read of X
        # when its eight experts' work shares it: X read once is the algorithmic traffic
        "hessian_moe": hbm("hessian_moe", t5 * c5 * 2),
        "scale_moe": hbm("scale_moe", E * r5 * c5 * 2),
        "lh_moe": search_roof("lh_moe", E * r5 * c5 * 2 + E * (c5 // 16) * 1024 + n_lh5, n_lh5 * 126,
                              counts["lh_moe"]["lh_screened"], 512),
        "quantize_moe": hbm("quantize_moe", E * r5 * c5 * (2 + 0.5 + 1 / 16)),
    }

    def measured_peak(r):
        if r["bound"] == "hbm":
            return copy_gbs
        if r["bound"] == "alu":
            return probe_rates.get("valu_lane_tops")
        return {BF16_MFMA_TFLOPS: probe_rates.get("mfma_bf16_tflops"),
                FP32_MFMA_TFLOPS: probe_rates.get("mfma_f32_tflops"),
                FP64_TFLOPS: probe_rates.get("mfma_f64_tflops")}.get(r["peak"])

    for r in rooflines.values():
        mp = measured_peak(r)
        r["frac_of_measured"] = None if not mp else round(r["achieved"] / mp, 4)
    # issue rates of the binding units from the committed counter runs (dropped when the
    # kernel's source changed since)
    for key, ent in load_counters().items():
        if key in rooflines:
            rooflines[key]["counters"] = ent
            evals = rooflines[key].get("evaluations")
            if evals and ent.get("valu_instructions"):
                # lane-ops per (element, candidate) actually issued, against the evaluation
                # cost model's MSE_OPS_PER_EVAL (wave instructions x 64 lanes / 16 elements)
                rooflines[key]["valu_lane_ops_per_element_candidate"] = round(
                    ent["valu_instructions"] * 64 / (evals * 16), 2)

    out = {
        "metric": "NVFP4 fake-quant GB/s + Local-Hessian blocks/s, % of MI355X roofline",
        "value": round(fq_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded generators; no datasets or checkpoints)",
        "config": {
            "workload": "activation fake-quant bf16 8192x4096, max scaling (headline); per step "
                        "also the activation's calibration histogram and clip scale, its "
                        "straight-through backward and moving-average scale, MSE and "
                        "Four Over Six on bf16 12288x4096, block Hessian of "
                        "131072x4096 + Local-Hessian on 4096x4096, full Gram matrix + GPTQ "
                        "(fp64) at the Local-Hessian bytes on 4096x4096, MoE 128 experts 512x2048 with "
                        "65536 tokens top-8, and the tiny 64x256 configuration",
            "fakequant_bytes_per_launch": int(fq_bytes),
            "fakequant_launches_per_step": FQ_SETS,
        },
        "local_hessian_blocks_per_s": {
            "proj_4096x4096_incl_hessian": round(lh4_blocks_s, 1),
            "moe_128x512x2048_incl_routing_hessian": round(lh5_blocks_s, 1),
        },
        "roofline": rooflines["fakequant_act"],
        "rooflines": rooflines,
        "search_counts": counts,
        "stage_ms": {k: round(v, 4) for k, v in ms.items()},
        "stage_ms_note": "median over the timed steps (fake-quant: per launch)",
        "copy_1GiB_gbs": None if copy_gbs is None else round(copy_gbs, 1),
        "measured_peaks": None if copy_gbs is None else {
            "hbm_copy_gbs": round(copy_gbs, 1),
            **probe_rates,
            "note": "measured after the step in the same process: a plain 1 GiB device copy, "
                    "and loops of independent MFMA / non-packed VALU instructions (two "
                    "4-wave workgroups per CU); rooflines[*].frac_of_measured divides by these"},
        "setup_s": round(t_setup, 1),
    }

    # ---------------------------------------------------------------- CPU oracle baseline
    if not args.no_cpu_baseline:
        from oracle import oracle
        nthr = oracle.num_threads()
        # inputs made by the oracle itself (untimed): scales, and Hessians from a subset of
        # the tokens (search times depend on H's structure, not on how many tokens built it)
        xa = a2.float().cpu().numpy()
        s2 = oracle.tensor_scale(xa)
        rows_lh = 4096
        wl = w4[:rows_lh].float().cpu().numpy()
        s4 = oracle.tensor_scale(w4.float().cpu().numpy())
        tok_h = 8192
        x4s = x4[:tok_h].float().cpu().numpy()
        rows_mse = 8192
        w3n = w3.float().cpu().numpy()
        s3 = oracle.tensor_scale(w3n)
        wm = w3n[:rows_mse]
        n_exp = 16
        We = w5[:n_exp].float().cpu().numpy()
        Se = [oracle.tensor_scale(We[e]) for e in range(n_exp)]
        off_r, tok_r = oracle.route_groups(ids5.cpu().numpy(), E)
        x5n = x5.float().cpu().numpy()
        He = [oracle.block_hessian(x5n, tok_r[off_r[e]:min(off_r[e + 1], off_r[e] + 512)]).astype(np.float32)
              for e in range(n_exp)]
        n_g, rows_g = 1024, 64
        Hg = oracle.full_hessian_blas(x4s[:, :n_g])
        wg = w4[:rows_g, :n_g].float().cpu().numpy()
        sg = oracle.tensor_scale(wg)
        scg = oracle.scales_max(wg, sg)
        w1n, x1n = w1c.numpy(), x1c.numpy()

        def timed(fn):
            t = time.perf_counter()
            r = fn()
            return time.perf_counter() - t, r

        def tiny_stages():
            s1 = oracle.tensor_scale(w1n)
            oracle.fakequant(w1n, s1)
            oracle.scales_mse(w1n, s1)
            h1 = oracle.block_hessian(x1n).astype(np.float32)
            oracle.scales_local_hessian(w1n, s1, h1)

        # timed, on every host thread
        dt_s, _ = timed(lambda: oracle.tensor_scale(xa))
        dt_max, _ = timed(lambda: oracle.scales_max(xa, s2))
        dt_fq, _ = timed(lambda: oracle.fakequant(xa, s2))
        dt_h, Hn = timed(lambda: oracle.block_hessian(x4s))
        Hn = Hn.astype(np.float32)
        dt_lh, _ = timed(lambda: oracle.scales_local_hessian(wl, s4, Hn))
        dt_mse, _ = timed(lambda: oracle.scales_mse(wm, s3))
        dt_fos, _ = timed(lambda: oracle.scales_four_over_six(wm, s3))
        dt_cal, _ = timed(lambda: oracle.calib_scale(oracle.calib_histogram(xa.ravel()), CALIB_FRACTION))
        dt_lh5, _ = timed(lambda: [oracle.scales_local_hessian(We[e], Se[e], He[e]) for e in range(n_exp)])
        dt_gf, Ug = timed(lambda: oracle.gptq_factor(Hg, GPTQ_DAMP))
        dt_gr, _ = timed(lambda: oracle.gptq(wg, sg, scg, U=Ug))
        dt_c1, _ = timed(tiny_stages)
        # one thread: the tiny configuration, and samples of the activation and MLP weight
        rows_fq1, rows_mse1 = 512, 256
        oracle.set_num_threads(1)
        try:
            dt1_c1, _ = timed(tiny_stages)
            dt1_fq, _ = timed(lambda: oracle.fakequant(xa[:rows_fq1], s2))
            dt1_mse, _ = timed(lambda: oracle.scales_mse(w3n[:rows_mse1], s3))
        finally:
            oracle.set_num_threads(nthr)
        total = (dt_s + dt_max + dt_fq + dt_h + dt_lh + dt_mse + dt_fos + dt_cal + dt_lh5 + dt_gf
                 + dt_gr + dt_c1 + dt1_c1 + dt1_fq + dt1_mse)
        out["cpu_baseline"] = {
            "value": round(xa.size * FQ_BYTES_PER_ELEM / dt_fq / 1e9, 4),
            "unit": "GB/s",
            "cores": nthr,
            "kind": "oracle",
            "sample": f"fake-quant, tensor scale, max bytes and calibration histogram of the whole "
                      f"8192x4096 activation; block Hessian of {tok_h} of the 131072 tokens x 4096; "
                      f"Local-Hessian on {rows_lh} rows ({rows_lh * (c4 // 16)} blocks) of the "
                      f"4096x4096 weight; MSE and Four Over Six on {rows_mse} rows "
                      f"({rows_mse * (c3 // 16)} blocks) of the 12288x4096 weight; Local-Hessian on "
                      f"{n_exp} of the 128 experts; GPTQ factor at n = {n_g} and GPTQ rounding of "
                      f"{rows_g} rows x {n_g}; the whole tiny configuration; on one thread: the tiny "
                      f"configuration, fake-quant of {rows_fq1} activation rows, MSE on {rows_mse1} "
                      f"weight rows",
            "stages": {
                "tensor_scale_gbs": round(xa.size * 2 / dt_s / 1e9, 3),
                "max_bytes_blocks_per_s": round(xa.size / 16 / dt_max, 1),
                "fakequant_gbs": round(xa.size * FQ_BYTES_PER_ELEM / dt_fq / 1e9, 4),
                "mse_blocks_per_s": round(rows_mse * (c3 // 16) / dt_mse, 1),
                "block_hessian_gbs": round(x4s.size * 2 / dt_h / 1e9, 3),
                "local_hessian_blocks_per_s": round(rows_lh * (c4 // 16) / dt_lh, 1),
                "four_over_six_blocks_per_s": round(rows_mse * (c3 // 16) / dt_fos, 1),
                "calibration_gbs": round(xa.size * 2 / dt_cal / 1e9, 3),
                "local_hessian_moe_blocks_per_s": round(n_exp * r5 * (c5 // 16) / dt_lh5, 1),
                "gptq_factor_n1024_s": round(dt_gf, 3),
                "gptq_factor_tflops": round((4 * n_g ** 3 / 3) / dt_gf / 1e12, 5),
                "gptq_rows_tflops": round(rows_g * n_g * n_g / dt_gr / 1e12, 5),
                "tiny_all_ms": round(dt_c1 * 1e3, 2),
            },
            "one_thread": {
                "cores": 1,
                "tiny_all_ms": round(dt1_c1 * 1e3, 2),
                "fakequant_gbs": round(rows_fq1 * c2 * FQ_BYTES_PER_ELEM / dt1_fq / 1e9, 4),
                "mse_blocks_per_s": round(rows_mse1 * (c3 // 16) / dt1_mse, 1),
            },
            "seconds": round(total, 2),
        }
        out["gpu_over_cpu"] = {
            "fakequant": round(out["value"] / out["cpu_baseline"]["value"], 1),
            "local_hessian_proj": round((n_lh4 / (ms["lh_proj"] * 1e-3)) /
                                        out["cpu_baseline"]["stages"]["local_hessian_blocks_per_s"], 1),
            "tiny_all": round(dt_c1 * 1e3 / ms["tiny_all"], 1),
        }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
