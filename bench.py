#!/usr/bin/env python3
"""Benchmark of the NVFP4 fake-quant attention hot path on one MI355X.

One step runs every stage of the hot path once, on synthetic inputs already
resident in HBM (Wan2.1-T2V-1.3B attention shape at 448x896, 61 frames:
B=1, H=12, L=16*28*56=25088, D=128):
  1. fq_nvfp4, unit global scale, on a bf16 [301056, 128] tensor (25088 tokens x
     12 heads x D=128; 4 rotating input/output pairs, 616 MB, so the 256 MB
     Infinity Cache cannot serve it);
  2. attn_qat_fwd in training mode (Q, K, V and P fake-quantized; lse, chunk
     maxima and the high-precision auxiliary output written);
  3. attn_qat_bwd, the straight-through backward;
  4. vsa_qat_fwd in training mode, the cube-sparse forward (196 cubes of 4x4x8,
     top-20; its fine stage's lse, chunk maxima and auxiliary output written);
  5. vsa_qat_bwd, the straight-through backward of the cube-sparse fine stage.

value = the metric's own quantity: dense fake-quant attention forward + backward
TFLOP/s at H=12, L=25088, D=128, i.e. (4 + 10)*B*H*L^2*D FLOP over the time of
stages 2 and 3 inside the step (HIP events on the launch stream).  ms_per_step
is the wall time of the whole step; the "step" object reports the step's
composite rate, where the cube-sparse forward counts 4*B*H*n*k*128^2*D for its
fine stage plus 4*B*H*n^2*D for its coarse stage, its backward 2.5x the fine
stage, and fq contributes time but no FLOP.  After the step loop, the dense and cube-sparse inference forwards and
fq on its own (back-to-back launches) are timed for the "attention" and "fq"
objects, the attention variants (final-max statistics, static scales,
smooth-K, two-level P, smooth-Q) for the "variants" object, and the NVFP4 QAD linear on the model's
feed-forward projections (25088 tokens, 1536 -> 8960 -> 1536) for the "linear"
object.  Per-kernel durations come
from HIP events the library records around each of its launches on the launch
stream while kernel timing is on (aq_kernel_timing).

Prints one JSON line.  Only one GPU is supported: --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn_qat fwd+bwd TFLOP/s @H=12,L=25088,D=128 (%BF16 MFMA peak); fq GB/s"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

B, H, D = 1, 12, 128
GRID = (16, 28, 56)
L = GRID[0] * GRID[1] * GRID[2]
CUBE = (4, 4, 8)
SPARSITY = 0.9


def flops():
    fwd = 4.0 * B * H * L * L * D
    n = L // (CUBE[0] * CUBE[1] * CUBE[2])
    k = max(1, min(math.ceil((1 - SPARSITY) * n), n))
    fine = 4.0 * B * H * n * k * 128 * 128 * D
    return {"fwd": fwd, "bwd": 2.5 * fwd, "vsa_fine": fine, "vsa": fine + 4.0 * B * H * n * n * D,
            "vsa_bwd": 2.5 * fine, "topk": k, "cubes": n}


def cpu_baseline(q, k, v, do, seconds: float):
    """The oracle, as it stands, on a bounded sample of the same workload: forward and dQ rows of
    head 0, in the metric's unit."""
    import numpy as np

    import oracle
    cores = len(os.sched_getaffinity(0))
    oracle.set_threads(cores)
    oracle.build()
    from synth import to_bhld_bits
    qb, kb, vb, db = (to_bhld_bits(t[:, :, :1]) for t in (q, k, v, do))
    scale = 1.0 / math.sqrt(D)

    def run(rows):
        t0 = time.perf_counter()
        oracle.attn_fwd(qb, kb, vb, scale, rows=rows)
        oracle.attn_bwd(qb, kb, vb, db, scale, qrows=rows, krows=np.zeros(0, np.int64))
        return time.perf_counter() - t0

    # Each call has a fixed part (quantizing the head's K and V) and a per-row part; size the
    # sample from both so the timed call takes about `seconds`.
    run(np.arange(0, L, L // 16)[:16])  # first call: library load and thread start-up
    t16 = run(np.linspace(0, L - 1, 16).astype(np.int64))
    t256 = run(np.linspace(0, L - 1, 256).astype(np.int64))  # enough rows to keep every core busy
    per_row = max((t256 - t16) / 240, 1e-5)
    fixed = max(t16 - 16 * per_row, 0.0)
    R = int(min(L, max(16, (seconds - fixed) / per_row)))
    rows = np.linspace(0, L - 1, R).astype(np.int64)
    t = run(rows)
    # per query row: forward 4*L*D (logits, P@V); dQ row 6*L*D (logits, dP, dQ)
    fl = R * (4.0 + 6.0) * L * D
    return {"value": fl / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"oracle forward + dQ backward for {R} query rows of head 0 at L={L}, D={D} "
                      f"(fp64 C, OpenMP), {t:.1f} s; per row 4*L*D + 6*L*D FLOP"}


# Sources each timed kernel is built from: the HBM traffic recorded under profiles/ for a kernel is
# reported only while the sha256 of these files matches the one recorded with the counters.
KERNEL_SOURCES = {
    "bwd_dkdv": ("attn_bwd.hip", "attn_common.hpp", "aq_device.hpp"),
    "bwd_dq": ("attn_bwd.hip", "attn_common.hpp", "aq_device.hpp"),
    "attn_fwd_train": ("attn_fwd.hip", "attn_common.hpp", "aq_device.hpp"),
    "attn_fwd": ("attn_fwd.hip", "attn_common.hpp", "aq_device.hpp"),
    "fq_contig_unit": ("fq.hip", "aq_device.hpp"),
    "vsa_fwd_train": ("attn_fwd.hip", "attn_common.hpp", "aq_device.hpp"),
    "vsa_fwd": ("attn_fwd.hip", "attn_common.hpp", "aq_device.hpp"),
    "vsa_bwd_dkdv": ("attn_bwd.hip", "attn_common.hpp", "aq_device.hpp"),
    "vsa_bwd_dq": ("attn_bwd.hip", "attn_common.hpp", "aq_device.hpp"),
    "dkdv_reduce": ("attn_bwd.hip", "attn_common.hpp", "aq_device.hpp"),
    "dq_reduce": ("attn_bwd.hip", "attn_common.hpp", "aq_device.hpp"),
    # the QAD linear's three GEMMs of the 1536 -> 8960 projection, in launch order
    "gemm_tn_y": ("linear.hip", "attn_common.hpp", "aq_device.hpp"),
    "gemm_tn_grad_x": ("linear.hip", "attn_common.hpp", "aq_device.hpp"),
    "gemm_tn_grad_w": ("linear.hip", "attn_common.hpp", "aq_device.hpp"),
    "transpose_colsum": ("linear.hip", "aq_device.hpp"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_qat_step_wan448x896x61_hbm_traffic.md")


def kernel_source_hash(name):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, "quantization_aware_attention_nvfp4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(name):
    """HBM bytes per launch of kernel `name` from the counter summary (rows
    `| name | sha | fetch KiB | write KiB | bytes |`), or None when absent or when the kernel's
    sources changed since the counters were taken."""
    if name not in KERNEL_SOURCES or not os.path.exists(TRAFFIC_FILE):
        return None
    want = kernel_source_hash(name)
    for line in open(TRAFFIC_FILE):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 5 and cells[0] == name and cells[1] == want:
            try:
                return float(cells[4])
            except ValueError:
                return None
    return None


def pmc_probe():
    """One pass of every stage (no timing), the QAD linear's forward and backward on the
    1536 -> 8960 feed-forward projection, and a plain 1 GiB device copy, for counter runs: the
    copy's FETCH_SIZE / WRITE_SIZE readings calibrate the counters' unit."""
    import torch

    import quantization_aware_attention_nvfp4_amd as m
    import synth
    dev = torch.device("cuda", 0)
    x = synth.fq_tensor().to(dev)
    y = torch.empty_like(x)
    q, k, v = (t.to(dev) for t in synth.wan_448x896x61())
    do = synth.normal_bf16((B, L, H, D), 2003).to(dev)
    qv, kv, vv = (t.to(dev) for t in synth.vsa_inputs())
    dov = synth.normal_bf16((B, L, H, D), 2005).to(dev)
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)  # 1 GiB
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    m.fq_nvfp4(x, out=y)
    m.attn_qat_fwd(q, k, v)
    o, aux = m.attn_qat_fwd(q, k, v, training=True)
    m.attn_qat_bwd(q, k, v, aux, do)
    ov, auxv = m.vsa_qat_fwd(qv, kv, vv, grid=GRID, cube=CUBE, sparsity=SPARSITY, training=True)
    m.vsa_qat_bwd(qv, kv, vv, auxv, dov, grid=GRID, cube=CUBE, sparsity=SPARSITY)
    xl, wl, bl, gl = (t.to(dev) for t in synth.wan_ffn(1536, 8960))
    m.qad_linear_fwd(xl, wl, bl)
    m.qad_linear_bwd(gl, xl, wl)
    torch.cuda.synchronize()
    print("pmc probe done: copy bytes", 2 * src.numel(), flush=True)


def profile_step(steps: int):
    """The benchmark step's launches only (448x896x61: fq, training forward, backward, cube-sparse
    training forward and backward), `steps` times after one warm-up, then the dense and the
    cube-sparse inference forward three times each and one QAD linear forward + backward (1536 -> 8960, 25088 tokens),
    preceded by a plain 1 GiB device copy whose FETCH_SIZE / WRITE_SIZE readings calibrate the
    traffic counters.  For rocprofv3 kernel-trace and counter runs: every
    attention launch it makes is one of the timed workload's."""
    import torch

    import quantization_aware_attention_nvfp4_amd as m
    import synth
    dev = torch.device("cuda", 0)
    x = synth.fq_tensor().to(dev)
    y = torch.empty_like(x)
    q, k, v = (t.to(dev) for t in synth.wan_448x896x61())
    do = synth.normal_bf16((B, L, H, D), 2003).to(dev)
    qv, kv, vv = (t.to(dev) for t in synth.vsa_inputs())
    dov = synth.normal_bf16((B, L, H, D), 2005).to(dev)
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)  # 1 GiB
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    vsa_args = dict(grid=GRID, cube=CUBE, sparsity=SPARSITY)
    for i in range(steps + 1):
        m.fq_nvfp4(x, out=y)
        o, aux = m.attn_qat_fwd(q, k, v, training=True)
        m.attn_qat_bwd(q, k, v, aux, do)
        ov, auxv = m.vsa_qat_fwd(qv, kv, vv, training=True, **vsa_args)
        m.vsa_qat_bwd(qv, kv, vv, auxv, dov, **vsa_args)
        torch.cuda.synchronize()
        print(f"profile step {i} done", flush=True)
    for _ in range(3):
        m.attn_qat_fwd(q, k, v)
        m.vsa_qat_fwd(qv, kv, vv, **vsa_args)
    torch.cuda.synchronize()
    print("profile step: inference forward done", flush=True)
    # one QAD linear forward + backward on the 1536 -> 8960 feed-forward projection (25088 tokens)
    xl, wl, bl, gl = (t.to(dev) for t in synth.wan_ffn(1536, 8960))
    m.qad_linear_fwd(xl, wl, bl)
    m.qad_linear_bwd(gl, xl, wl)
    torch.cuda.synchronize()
    print("profile step: done", flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-probe", action="store_true", help="one untimed pass of each stage plus a 1 GiB copy")
    ap.add_argument("--profile-step", action="store_true",
                    help="only the step's launches (--steps of them after one warm-up) and the inference forward, "
                         "for rocprofv3")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library and this benchmark run on one GPU only (asked for --gpus {args.gpus}); sharding the "
              "heads of a call over several GPUs is not built.", file=sys.stderr)
        sys.exit(2)

    if args.pmc_probe:
        pmc_probe()
        return
    if args.profile_step:
        profile_step(args.steps)
        return

    import torch

    import quantization_aware_attention_nvfp4_amd as m
    import synth
    from quantization_aware_attention_nvfp4_amd import _lib

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    fl = flops()

    x = synth.fq_tensor()
    xs = [x.to(dev) for _ in range(4)]
    ys = [torch.empty_like(xs[0]) for _ in range(4)]
    q, k, v = synth.wan_448x896x61()
    do = synth.normal_bf16((B, L, H, D), 2003)
    qv, kv, vv = synth.vsa_inputs()
    dov = synth.normal_bf16((B, L, H, D), 2005)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    qvd, kvd, vvd, dovd = (t.to(dev) for t in (qv, kv, vv, dov))

    phases = ("fq", "fwd", "bwd", "vsa_fwd", "vsa_bwd")
    vsa_args = dict(grid=GRID, cube=CUBE, sparsity=SPARSITY)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record()
        m.fq_nvfp4(xs[i % 4], out=ys[i % 4])
        if ev is not None:
            ev[1].record()
        o, aux = m.attn_qat_fwd(qd, kd, vd, training=True)
        if ev is not None:
            ev[2].record()
        m.attn_qat_bwd(qd, kd, vd, aux, dod)
        if ev is not None:
            ev[3].record()
        ov, auxv = m.vsa_qat_fwd(qvd, kvd, vvd, training=True, **vsa_args)
        if ev is not None:
            ev[4].record()
        m.vsa_qat_bwd(qvd, kvd, vvd, auxv, dovd, **vsa_args)
        if ev is not None:
            ev[5].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(args.steps)]
    _lib.kernel_times(reset=True)
    _lib.kernel_timing(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    _lib.kernel_timing(False)
    kt = _lib.kernel_times(reset=True)

    # The cube-sparse inference forward (no training outputs), outside the step.
    vev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for i in range(5):
        vev[i].record()
        m.vsa_qat_fwd(qvd, kvd, vvd, **vsa_args)
    vev[5].record()
    torch.cuda.synchronize()
    vsa_inf_ms = sum(vev[i].elapsed_time(vev[i + 1]) for i in range(1, 5)) / 4

    # The dense inference forward (the forward-only workload's kernel), outside the step.
    iev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    m.attn_qat_fwd(qd, kd, vd)
    iev[0].record()
    for _ in range(5):
        m.attn_qat_fwd(qd, kd, vd)
    iev[1].record()
    torch.cuda.synchronize()
    fwd_inf_ms = iev[0].elapsed_time(iev[1]) / 5

    # The attention variants (include/attnqat.h flag bits) on the same workload: the inference
    # forward under each, and the training forward + backward under all of them together.
    def timed(fn, reps=3):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    fl_fwd = fl["fwd"]  # conventional 4*B*H*L^2*D (the final-max row-maximum pass is not counted)
    variants = {}
    for name, flg in (("final_max", 15 | 16), ("gsf_qkv", 15 | 32), ("gsf_p", 15 | 64), ("smooth_k", 15 | 128),
                      ("two_level_p", 15 | 256), ("smooth_q", 15 | 512), ("all", 255)):
        ms = timed(lambda: m.attn_qat_fwd(qd, kd, vd, quant_flags=flg))
        variants[name] = {"flags": flg, "inference_fwd_ms": round(ms, 4),
                          "inference_fwd_TFLOP/s": round(fl_fwd / (ms * 1e-3) / 1e12, 1)}

    def train_all():
        o, aux = m.attn_qat_fwd(qd, kd, vd, training=True, quant_flags=255)
        m.attn_qat_bwd(qd, kd, vd, aux, dod, quant_flags=255)

    ms = timed(train_all, 2)
    variants["all"]["fwd_bwd_ms"] = round(ms, 4)
    variants["all"]["fwd_bwd_TFLOP/s"] = round((fl["fwd"] + fl["bwd"]) / (ms * 1e-3) / 1e12, 1)

    # The Wan2.1 480x832, 81-frame workload (L = 21*30*52 = 32760, a ragged multiple of the 128-key
    # chunk): the training forward (with the auxiliary high-precision output) alone and followed by
    # the backward, over back-to-back calls.  TFLOP/s on the conventional 4*B*H*L^2*D forward and
    # 2.5x that backward; the auxiliary P.V adds half a forward of executed MFMA work.
    q4, k4, v4, do4 = (t.to(dev) for t in synth.wan_480x832x81())
    L4 = q4.shape[1]
    fl4 = 4.0 * B * H * L4 * L4 * D

    def train4():
        o, aux = m.attn_qat_fwd(q4, k4, v4, training=True)
        m.attn_qat_bwd(q4, k4, v4, aux, do4)

    fwd4_ms = timed(lambda: m.attn_qat_fwd(q4, k4, v4, training=True), 3)
    fb4_ms = timed(train4, 3)
    wan480 = {"L": L4, "fwd_flop": fl4, "bwd_flop": 2.5 * fl4, "aux_pv_flop": 0.5 * fl4,
              "train_fwd_ms": round(fwd4_ms, 4), "train_fwd_TFLOP/s": round(fl4 / (fwd4_ms * 1e-3) / 1e12, 1),
              "train_fwd_executed_TFLOP/s": round(1.5 * fl4 / (fwd4_ms * 1e-3) / 1e12, 1),
              "fwd_bwd_ms": round(fb4_ms, 4), "fwd_bwd_TFLOP/s": round(3.5 * fl4 / (fb4_ms * 1e-3) / 1e12, 1),
              "frac_bf16_peak": round(3.5 * fl4 / (fb4_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del q4, k4, v4, do4

    # The NVFP4 QAD linear on the Wan2.1 1.3B feed-forward projections at this token count (25088
    # tokens, 1536 -> 8960 and 8960 -> 1536): the forward (activation and weight fake-quant, BF16
    # MFMA GEMM, bias) and the straight-through backward, each timed over back-to-back calls; the
    # kernels' own per-launch times from the library's events over three forward + backward pairs;
    # torch's bf16 linear (a library GEMM) on the same operands for context.
    linear = {}
    for lname, (kin, kout) in (("ffn_up", (1536, 8960)), ("ffn_down", (8960, 1536))):
        xl, wl, bl, gl = (t.to(dev) for t in synth.wan_ffn(kin, kout))
        fl_lin = 2.0 * xl.shape[0] * kin * kout
        f_ms = timed(lambda: m.qad_linear_fwd(xl, wl, bl), 5)
        b_ms = timed(lambda: m.qad_linear_bwd(gl, xl, wl), 3)
        t_ms = timed(lambda: torch.nn.functional.linear(xl, wl, bl), 5)
        _lib.kernel_times(reset=True)
        _lib.kernel_timing(True)
        for _ in range(3):
            m.qad_linear_fwd(xl, wl, bl)
            m.qad_linear_bwd(gl, xl, wl)
        torch.cuda.synchronize()
        _lib.kernel_timing(False)
        kl = _lib.kernel_times(reset=True)
        g_cnt, g_ms = kl["gemm_tn"]
        g_avg = g_ms / g_cnt  # the three GEMMs (y, grad_x, grad_w) have the same FLOP count
        linear[lname] = {
            "M": xl.shape[0], "K": kin, "N": kout, "fwd_ms": round(f_ms, 4),
            "fwd_TFLOP/s": round(fl_lin / (f_ms * 1e-3) / 1e12, 1), "bwd_ms": round(b_ms, 4),
            "bwd_TFLOP/s": round(2 * fl_lin / (b_ms * 1e-3) / 1e12, 1), "gemm_tn_avg_ms": round(g_avg, 4),
            "gemm_tn_TFLOP/s": round(fl_lin / (g_avg * 1e-3) / 1e12, 1),
            "gemm_tn_frac_bf16_peak": round(fl_lin / (g_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "torch_bf16_linear_ms": round(t_ms, 4),
            "gemm_tn_traffic": ({g: recorded_traffic("gemm_tn_" + g) for g in ("y", "grad_x", "grad_w")}
                                if lname == "ffn_up" else None),
            "kernels_avg_ms": {kn: round(v[1] / v[0], 4) for kn, v in sorted(kl.items())}}
        del xl, wl, bl, gl

    # fq on its own: 40 back-to-back launches over the 4 rotating pairs between one pair of events
    # (a per-launch event pair adds about a microsecond to a 26 us kernel).
    fev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for i in range(4):
        m.fq_nvfp4(xs[i], out=ys[i])
    fev[0].record()
    for i in range(40):
        m.fq_nvfp4(xs[i % 4], out=ys[i % 4])
    fev[1].record()
    torch.cuda.synchronize()
    fq_alone_ms = fev[0].elapsed_time(fev[1]) / 40

    ms_step = wall * 1e3 / args.steps
    phase_ms = {p: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j, p in enumerate(phases)}
    total_flop = fl["fwd"] + fl["bwd"] + fl["vsa"] + fl["vsa_bwd"]
    value_ms = phase_ms["fwd"] + phase_ms["bwd"]
    value = (fl["fwd"] + fl["bwd"]) / (value_ms * 1e-3) / 1e12

    # Per-kernel averages and their algorithmic work per launch.
    fq_bytes = 2.0 * 2 * xs[0].numel()
    alg = {  # kernel name -> (work per launch, unit)
        "attn_fwd_train": (fl["fwd"], "flop"),
        "bwd_dkdv": (0.8 * fl["bwd"], "flop"),  # S, dP, dV, dK: 4 of the 5 backward products
        "bwd_dq": (0.2 * fl["bwd"], "flop"),    # dQ (its S and dP recomputation counts as overhead)
        "fq_contig_unit": (fq_bytes, "byte"),
        "vsa_fwd_train": (fl["vsa_fine"], "flop"),
        "vsa_bwd_dkdv": (0.8 * fl["vsa_bwd"], "flop"),
        "vsa_bwd_dq": (0.2 * fl["vsa_bwd"], "flop"),
    }
    # The dense backward kernels split the units of a partly filled last round into pieces whose
    # sums a reduction kernel adds: their work per launch is timed with that reduction.
    reduction = {"bwd_dkdv": "dkdv_reduce", "bwd_dq": "dq_reduce"}

    def with_reduction(name):
        avg = kt[name][1] / kt[name][0]
        r = reduction.get(name)
        if r in kt:
            avg += kt[r][1] / kt[name][0]
        return avg

    kernels = {}
    for name, (cnt, ms) in kt.items():
        avg = ms / max(cnt, 1)
        entry = {"launches_per_step": cnt / args.steps, "avg_ms": round(avg, 5)}
        if name in reduction and reduction[name] in kt:
            avg = with_reduction(name)
            entry["with_reduction_avg_ms"] = round(avg, 5)
        if name in alg:
            w, unit = alg[name]
            if unit == "flop":
                entry["TFLOP/s"] = round(w / (avg * 1e-3) / 1e12, 1)
                entry["frac_bf16_peak"] = round(w / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
            else:
                entry["GB/s"] = round(w / (avg * 1e-3) / 1e9, 1)
                entry["frac_hbm_peak"] = round(w / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        kernels[name] = entry
    dominant = max((n for n in kt if n in alg and alg[n][1] == "flop"), key=lambda n: kt[n][1])
    dom_avg = with_reduction(dominant)
    achieved = alg[dominant][0] / (dom_avg * 1e-3) / 1e12
    traffic = recorded_traffic(dominant)
    red = reduction.get(dominant)
    if red in kt and traffic is not None:
        red_traffic = recorded_traffic(red)
        traffic = None if red_traffic is None else traffic + red_traffic * kt[red][0] / kt[dominant][0]
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": None if traffic is None else int(traffic),
                "traffic_unit": "HBM bytes per launch (TCC FETCH_SIZE + WRITE_SIZE, copy-calibrated)"}
    if red in kt:
        roofline["includes"] = red
    fq_step_ms = kt["fq_contig_unit"][1] / kt["fq_contig_unit"][0]
    fq_gbs = fq_bytes / (fq_alone_ms * 1e-3) / 1e9
    fq_traffic = recorded_traffic("fq_contig_unit")
    fq = {"kernel": "fq_contig_unit", "bytes_per_launch": fq_bytes, "avg_us": round(fq_alone_ms * 1e3, 2),
          "GB/s": round(fq_gbs, 1), "peak": PEAK_HBM_GBS, "frac": round(fq_gbs / PEAK_HBM_GBS, 4),
          "timing": "40 back-to-back launches over 4 rotating 154 MB pairs, one event pair",
          "in_step_avg_us": round(fq_step_ms * 1e3, 2),
          "traffic": None if fq_traffic is None else int(fq_traffic)}
    attn_ms = phase_ms["fwd"] + phase_ms["bwd"]
    attn = {"fwd_bwd_ms": round(attn_ms, 4),
            "fwd_bwd_TFLOP/s": round((fl["fwd"] + fl["bwd"]) / (attn_ms * 1e-3) / 1e12, 1),
            "frac_bf16_peak": round((fl["fwd"] + fl["bwd"]) / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "fwd_TFLOP/s": round(fl["fwd"] / (phase_ms["fwd"] * 1e-3) / 1e12, 1),
            "bwd_TFLOP/s": round(fl["bwd"] / (phase_ms["bwd"] * 1e-3) / 1e12, 1),
            "vsa_fwd_train_TFLOP/s": round(fl["vsa"] / (phase_ms["vsa_fwd"] * 1e-3) / 1e12, 1),
            "vsa_bwd_TFLOP/s": round(fl["vsa_bwd"] / (phase_ms["vsa_bwd"] * 1e-3) / 1e12, 1),
            "inference_fwd_ms": round(fwd_inf_ms, 4),
            "inference_fwd_TFLOP/s": round(fl["fwd"] / (fwd_inf_ms * 1e-3) / 1e12, 1),
            "inference_fwd_frac_bf16_peak": round(fl["fwd"] / (fwd_inf_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "vsa_inference_fwd_ms": round(vsa_inf_ms, 4),
            "vsa_inference_fwd_TFLOP/s": round(fl["vsa"] / (vsa_inf_ms * 1e-3) / 1e12, 1)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(q, k, v, do, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Wan2.1-T2V-1.3B attention at 448x896, 61 frames: NVFP4 fake-quant training forward "
                               "+ straight-through backward (value); the step also runs fq, the cube-sparse "
                               "forward and its backward",
                   "B": B, "H": H, "L": L, "D": D, "causal": False, "quant": "Q,K,V,P NVFP4 unit scale",
                   "vsa_cubes": fl["cubes"], "vsa_topk": fl["topk"], "fq_shape": list(xs[0].shape)},
        "value_basis": {"flop": fl["fwd"] + fl["bwd"], "ms": round(value_ms, 4),
                        "timing": "HIP events around the training forward and the backward inside each timed step"},
        "step": {"stages": list(phases), "ms": round(ms_step, 4), "flop": total_flop,
                 "TFLOP/s": round(total_flop / (ms_step * 1e-3) / 1e12, 2)},
        "roofline": roofline, "cpu_baseline": cpu, "attention": attn, "fq": fq,
        "phases_ms": {p: round(t, 4) for p, t in phase_ms.items()}, "kernels": kernels, "variants": variants,
        "linear": linear, "wan_480x832x81": wan480,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
