"""Benchmark of the fine-grained FP8 linear-layer hot path on one MI355X.

One step = the forward pass of the fine-grained FP8 linear layer at the
4096 x 7168 x 7168 workload: quantize the activations per 1x128 tile,
quantize the weights per 128x128 block, and run the block-scaled GEMM with
bf16 output.  Inputs (bf16, seeded, synthetic: X ~ Student-t(3) with 7 outlier
columns x100, W ~ N(0, 0.02)) are resident in HBM before timing and rotate
over enough copies to defeat the 256 MB last-level cache.

Printed: one JSON line.  `value` is the GEMM's 2*M*N*K flops per step divided
by the whole step time (the quantizers count as overhead).  `roofline` is the
GEMM kernel's achieved TFLOP/s (per-launch HIP-event time) against the peak of
the matrix-core datapath it uses.  `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.  `rows` holds per-kernel measurements of
the other steps of the path (Wgrad requantization, 128x1 gradient
quantization, Wgrad GEMM, grouped GEMM) on their own workloads.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

M, N, K = 4096, 7168, 7168
PEAK_F16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 matrix peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
MALL_BYTES = 256 << 20

# HBM-side bytes per launch of the fprop GEMM, from two rocprofv3 PMC passes
# (FETCH_SIZE, WRITE_SIZE) over this bench, each scaled by what the same counter
# reads for a plain 1 GiB device copy (FETCH x2.0, WRITE x1.0).  The figure is
# tied to the GEMM source it was taken on: once gemm.hip changes it is reported
# as null until the counters are taken again (the digest covers the source and
# its extra compiler flags).
GEMM_PMC = {"src_sha256_16": "62f4ae2859854f45", "read_bytes": 346_217_728, "write_bytes": 58_721_376}


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clocks ramp up over the first ~100-200 ms of sustained matrix
    # work (the same kernel runs ~12 % slower before that), so the default
    # warm-up is ~200 ms of steps.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--no-rows", action="store_true", help="skip the per-kernel rows of the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for PMC byte-counter scaling)")
    return ap.parse_args()


def _gemm_traffic():
    import hashlib
    src = os.path.join(ROOT, "fp8_fine_grained_x128_amd", "csrc", "gemm.hip")
    from fp8_fine_grained_x128_amd._build import SOURCE_FLAGS
    with open(src, "rb") as f:
        text = f.read() + " ".join(SOURCE_FLAGS.get("gemm.hip", [])).encode()
    digest = hashlib.sha256(text).hexdigest()[:16]
    if digest != GEMM_PMC["src_sha256_16"]:
        return None
    return GEMM_PMC["read_bytes"] + GEMM_PMC["write_bytes"]


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


_BACKLOG = []


def _backlog(torch):
    """Enqueue a few ms of device copies so that the host runs ahead of the
    GPU: the per-launch events around a short kernel then time the kernel, not
    the host's launch overhead."""
    if not _BACKLOG:
        _BACKLOG.append(torch.empty(1 << 26, dtype=torch.float32, device="cuda"))
        _BACKLOG.append(torch.empty_like(_BACKLOG[0]))
    for _ in range(24):
        _BACKLOG[1].copy_(_BACKLOG[0])


def _time_ring(torch, fns, iters):
    """Mean per-call time (ms) of `iters` calls that cycle through `fns`, timed
    as one back-to-back run between a single event pair on the current stream.
    Each fn reads its own copy of the inputs; for HBM-bound kernels the copies
    together exceed twice the 256 MB last-level cache, so every call streams
    its input from HBM (one event pair per call would add ~3 us of device time
    to each call, and one reused input stays cache-resident)."""
    for f in fns:
        f()
    _backlog(torch)
    e0, e1 = _events(torch, 2)
    e0.record()
    for i in range(iters):
        fns[i % len(fns)]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def _ring_copies(nbytes):
    """Input copies whose total exceeds twice the last-level cache."""
    return max(1, min(16, -(-2 * MALL_BYTES // max(nbytes, 1)) + 1))


def main():
    args = _parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_fine_grained_x128_amd as fp8q
    from fp8_fine_grained_x128_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------------------------------------------------------- inputs
    wl = W.fprop(seed=0)
    per_copy = wl.x.numel() * 2 + wl.w.numel() * 2
    copies = max(1, -(-2 * MALL_BYTES // per_copy) + 1)
    xs = [wl.x.to(dev)]
    ws = [wl.w.to(dev)]
    for r in range(1, copies):  # rotated copies: same values, distinct buffers
        xs.append(xs[0].clone())
        ws.append(ws[0].clone())
    torch.cuda.synchronize()

    def step(r):
        qx, sx = fp8q.quantize_act(xs[r])
        qw, sw = fp8q.quantize_weight(ws[r])
        return fp8q.gemm(qx, sx, qw, sw, out_dtype=torch.bfloat16)

    for i in range(args.warmup):
        step(i % copies)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed steps
    # The K steps behind `value` are bracketed by one event pair only: an event
    # recorded between two kernels costs ~3 us of device time per record on
    # this GPU (measured: four per step added 12 us to a 405 us step).  The
    # GEMM's duration (the roofline's `achieved`) comes from an identical pass
    # of K steps right after, with an event pair around every GEMM on the
    # launch stream; the quantizers' rows time back-to-back runs over the same
    # rotated inputs.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(i % copies)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps

    ev = _events(torch, 2 * args.steps)
    for i in range(args.steps):
        r = i % copies
        qx, sx = fp8q.quantize_act(xs[r])
        qw, sw = fp8q.quantize_weight(ws[r])
        ev[2 * i].record()
        fp8q.gemm(qx, sx, qw, sw, out_dtype=torch.bfloat16)
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    t_gm = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)]
    mean = lambda a: sum(a) / len(a)  # noqa: E731
    qa_ms = _time_ring(torch, [lambda t=t: fp8q.quantize_act(t) for t in xs], 8 * copies)
    qw_ms = _time_ring(torch, [lambda t=t: fp8q.quantize_weight(t) for t in ws], 8 * copies)

    flops = W.gemm_flops(M, N, K)
    gemm_ms = mean(t_gm)
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    qa_bytes = W.quant_bytes(M * K, 2, M * (K // 128))
    qw_bytes = W.quant_bytes(N * K, 2, (N // 128) * (K // 128))
    kernels = {
        "quantize_act_1x128": {"us": qa_ms * 1e3, "GB/s": qa_bytes / (qa_ms * 1e-3) / 1e9,
                               "bytes": qa_bytes},
        "quantize_weight_128x128": {"us": qw_ms * 1e3, "GB/s": qw_bytes / (qw_ms * 1e-3) / 1e9,
                                    "bytes": qw_bytes},
        "gemm_bf16": {"us": gemm_ms * 1e3, "TFLOP/s": gemm_tflops,
                      "frac_fp8_peak": gemm_tflops / PEAK_FP8_TFLOPS,
                      "frac_f16_peak": gemm_tflops / PEAK_F16_TFLOPS, "flops": flops},
    }

    out = {
        "metric": "FP8 block-scaled GEMM TFLOP/s @4096x7168x7168 + % FP8 MFMA peak; quantize GB/s",
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "mma_dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "fprop 4096x7168x7168: X bf16 Student-t(3) + 7 outlier columns x100, "
                        "W bf16 N(0,0.02); step = quantize_act 1x128 + quantize_weight 128x128 + "
                        "block-scaled GEMM -> bf16",
            "M": M, "N": N, "K": K, "input_copies": copies,
        },
        "kernels": kernels,
        "frac_fp8_peak_step": flops / (ms_step * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
        "roofline": {
            "kernel": "gemm_strip_kernel (block-scaled, f16 MFMA on exact E4M3 operands, bf16 out, 256x448 strips)",
            "bound": "mfma",
            "achieved": gemm_tflops,
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": gemm_tflops / PEAK_F16_TFLOPS,
            "traffic": _gemm_traffic(),
        },
        "wall_s": wall,
    }

    # ---------------------------------------------------------------- other rows
    if not args.no_rows:
        out["rows"] = _rows(torch, fp8q, W, dev)

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel() * 4

    # ---------------------------------------------------------------- CPU baseline
    if not args.no_cpu:
        out["cpu_baseline"] = _cpu_baseline(np, wl)

    print(json.dumps(out), flush=True)


def _rows(torch, fp8q, W, dev):
    """Per-kernel timings of the Wgrad side, the opt-in datapaths, Dgrad, the
    FP8 dispatch and the grouped GEMM (device-side seeded inputs of the same
    shapes and distributions as the parity tests).  HBM-bound kernels cycle
    through input copies larger than twice the last-level cache; every row is
    a back-to-back run between one event pair (`_time_ring`)."""
    import numpy as np

    def ring(t):
        return [t] + [t.clone() for _ in range(_ring_copies(t.numel() * t.element_size()) - 1)]

    rows = {}
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    # Wgrad: dY [8192 x 4096] ~ N(0, 1e-3), X [8192 x 7168] ~ N(0, 1)
    T, Cout, Cin = 8192, 4096, 7168
    dy = (torch.randn((T, Cout), generator=g, device=dev) * 1e-3).to(torch.bfloat16)
    x = torch.randn((T, Cin), generator=g, device=dev).to(torch.bfloat16)
    qx, sx = fp8q.quantize_act(x)
    qxs = ring(qx)
    ms = _time_ring(torch, [lambda q=q: fp8q.requant_transpose(q, sx) for q in qxs], 40)
    b = W.requant_bytes(T * Cin, T * (Cin // 128), (T // 128) * Cin)
    rows["requant_transpose_8192x7168"] = {"us": ms * 1e3, "GB/s": b / (ms * 1e-3) / 1e9, "bytes": b}
    del qxs
    dys = ring(dy)
    ms = _time_ring(torch, [lambda d=d: fp8q.quantize_act(d, fp8q.FP8Q_TILE_128x1) for d in dys], 40)
    b = W.quant_bytes(T * Cout, 2, (T // 128) * Cout)
    rows["quantize_act_128x1_8192x4096"] = {"us": ms * 1e3, "GB/s": b / (ms * 1e-3) / 1e9, "bytes": b}
    del dys
    qxt, sxt = fp8q.requant_transpose(qx, sx)
    qdy, sdy = fp8q.quantize_act(dy, fp8q.FP8Q_TILE_128x1)
    dw = torch.empty((Cout, Cin), dtype=torch.float32, device=dev)
    ms = _time_ring(torch, [lambda: fp8q.gemm(qdy, sdy, qxt, sxt, bscale=fp8q.FP8Q_BSCALE_ROW,
                                              out_dtype=torch.float32, c=dw)], 20)
    fl = W.gemm_flops(Cout, Cin, T)
    rows["gemm_wgrad_4096x7168x8192_f32"] = {"us": ms * 1e3, "TFLOP/s": fl / (ms * 1e-3) / 1e12,
                                             "frac_f16_peak": fl / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS}
    del dy, x, qx, sx, qxt, sxt, qdy, sdy, dw
    # The fprop GEMM on the opt-in datapaths (same 4096x7168x7168 shape):
    # native FP8 MFMA with promotion, and the two power-of-two-scale paths.
    wl = W.fprop(seed=0)
    x2, w2 = wl.x.to(dev), wl.w.to(dev)
    fl = W.gemm_flops(M, N, K)
    y2 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    for name, mode, flags in (("fp8_mfma", fp8q.FP8Q_SCALE_FP32, fp8q.FP8Q_GEMM_MMA_FP8),
                              ("pow2_bf16_fold", fp8q.FP8Q_SCALE_POW2, fp8q.FP8Q_GEMM_POW2_SCALES),
                              ("pow2_fp8_scaled", fp8q.FP8Q_SCALE_POW2,
                               fp8q.FP8Q_GEMM_POW2_SCALES | fp8q.FP8Q_GEMM_MMA_FP8)):
        qx2, sx2 = fp8q.quantize_act(x2, scale_mode=mode)
        qw2, sw2 = fp8q.quantize_weight(w2, scale_mode=mode)
        ms = _time_ring(torch, [lambda: fp8q.gemm(qx2, sx2, qw2, sw2, c=y2, flags=flags)], 20)
        tf = fl / (ms * 1e-3) / 1e12
        rows[f"gemm_{name}_4096x7168x7168_bf16"] = {
            "us": ms * 1e3, "TFLOP/s": tf, "frac_f16_peak": tf / PEAK_F16_TFLOPS,
            "frac_fp8_peak": tf / PEAK_FP8_TFLOPS}
        if name == "pow2_bf16_fold":
            xs2 = ring(x2)
            ms = _time_ring(torch, [lambda t=t: fp8q.quantize_act(t, scale_mode=mode) for t in xs2], 40)
            b = W.quant_bytes(M * K, 2, M * (K // 128))
            rows["quantize_act_1x128_pow2_4096x7168"] = {"us": ms * 1e3, "GB/s": b / (ms * 1e-3) / 1e9}
            del xs2
            ws2 = ring(w2)
            ms = _time_ring(torch, [lambda t=t: fp8q.quantize_weight(t, scale_mode=mode) for t in ws2], 40)
            b = W.quant_bytes(N * K, 2, (N // 128) * (K // 128))
            rows["quantize_weight_128x128_pow2_7168x7168"] = {"us": ms * 1e3, "GB/s": b / (ms * 1e-3) / 1e9}
            del ws2
        del qx2, sx2, qw2, sw2
    del x2, w2, y2
    # Dgrad at the same layer: dX[4096][7168] = dY[4096][7168] W[7168][7168]
    g2 = torch.Generator(device=dev)
    g2.manual_seed(1)
    dy = (torch.randn((M, N), generator=g2, device=dev) * 1e-3).to(torch.bfloat16)
    w3 = (torch.randn((N, K), generator=g2, device=dev) * 0.02).to(torch.bfloat16)
    qdy, sdy = fp8q.quantize_act(dy)
    qw3, sw3 = fp8q.quantize_weight(w3)
    qw3s = ring(qw3)
    ms = _time_ring(torch, [lambda q=q: fp8q.transpose_weight(q, sw3) for q in qw3s], 40)
    b = 2 * N * K + 8 * (N // 128) * (K // 128)
    rows["transpose_weight_7168x7168"] = {"us": ms * 1e3, "GB/s": b / (ms * 1e-3) / 1e9, "bytes": b}
    del qw3s
    qt3, st3 = fp8q.transpose_weight(qw3, sw3)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    ms = _time_ring(torch, [lambda: fp8q.gemm(qdy, sdy, qt3, st3, c=dx)], 20)
    tf = fl / (ms * 1e-3) / 1e12
    rows["gemm_dgrad_4096x7168x7168_bf16"] = {"us": ms * 1e3, "TFLOP/s": tf, "frac_f16_peak": tf / PEAK_F16_TFLOPS}
    del dy, w3, qdy, sdy, qw3, sw3, qt3, st3, dx
    # FP8 MoE dispatch: gather 32768 expert slots from 16384 tokens and
    # quantize them 1x128 in one pass (each slot reads its source row once)
    d = W.dispatch()
    xds = ring(d.x.to(dev))
    idx = torch.from_numpy(d.row_index).to(dev)
    ms = _time_ring(torch, [lambda t=t: fp8q.gather_quantize_act(t, idx) for t in xds], 20)
    b = W.quant_bytes(32768 * 7168, 2, 32768 * 56) + 4 * 32768
    rows["gather_quantize_act_16384to32768x7168"] = {"us": ms * 1e3, "GB/s": b / (ms * 1e-3) / 1e9, "bytes": b}
    del d, xds, idx
    # Grouped: 64 experts, 32768 rows (Zipf 1.1 counts), N 2048, K 7168
    G, Mt, Ng, Kg = 64, 32768, 2048, 7168
    counts = W.zipf_counts(Mt, G, 1.1, np.random.default_rng(0))
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(counts)
    xg = torch.randn((Mt, Kg), generator=g, device=dev).to(torch.bfloat16)
    wg = (torch.randn((G, Ng, Kg), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    xgs = ring(xg)
    ms = _time_ring(torch, [lambda t=t: fp8q.quantize_act(t) for t in xgs], 10)
    b = W.quant_bytes(Mt * Kg, 2, Mt * (Kg // 128))
    rows["quantize_act_1x128_32768x7168"] = {"us": ms * 1e3, "GB/s": b / (ms * 1e-3) / 1e9, "bytes": b}
    del xgs
    wflat = wg.view(G * Ng, Kg)
    ms = _time_ring(torch, [lambda: fp8q.quantize_weight(wflat)], 5)
    b = W.quant_bytes(G * Ng * Kg, 2, G * (Ng // 128) * (Kg // 128))
    rows["quantize_weight_128x128_64x2048x7168"] = {"us": ms * 1e3, "GB/s": b / (ms * 1e-3) / 1e9,
                                                    "bytes": b}
    qxg, sxg = fp8q.quantize_act(xg)
    qwg, swg = fp8q.quantize_weight(wflat)
    qwg = qwg.reshape(G, Ng, Kg)
    swg = swg.reshape(G, Ng // 128, Kg // 128)
    offd = torch.from_numpy(off).to(dev)
    yg = torch.empty((Mt, Ng), dtype=torch.bfloat16, device=dev)
    ms = _time_ring(torch, [lambda: fp8q.grouped_gemm(qxg, sxg, qwg, swg, offd, c=yg)], 10)
    fl = W.gemm_flops(Mt, Ng, Kg)
    rows["grouped_gemm_64x(2048x7168)_32768rows_bf16"] = {
        "us": ms * 1e3, "TFLOP/s": fl / (ms * 1e-3) / 1e12,
        "frac_f16_peak": fl / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS}
    return rows


def W_quant_bytes_fprop_act():
    return M * K * (2 + 1) + 4 * M * (K // 128)


def _cpu_baseline(np, wl):
    """The CPU oracle on the host cores: full quantizers, GEMM on 256 output
    rows (scaled to the whole step)."""
    import oracle

    oracle.lib()
    x = wl.x.float().numpy()
    w = wl.w.float().numpy()
    t0 = time.perf_counter()
    qx, sx = oracle.quantize_act_1x128(x)
    t1 = time.perf_counter()
    qw, sw = oracle.quantize_weight_128x128(w)
    t2 = time.perf_counter()
    rows = 256
    mm, nn = np.meshgrid(np.arange(rows), np.arange(N), indexing="ij")
    oracle.gemm_entries(qx, sx, qw, sw, mm.ravel(), nn.ravel(), 0)
    t3 = time.perf_counter()
    gemm_full_s = (t3 - t2) * (M / rows)
    step_s = (t1 - t0) + (t2 - t1) + gemm_full_s
    cores = oracle.threads()
    # single-thread quantizer figure on 512 of the 4096 activation rows
    oracle.set_threads(1)
    t4 = time.perf_counter()
    oracle.quantize_act_1x128(x[:512])
    t5 = time.perf_counter()
    oracle.set_threads(cores)
    qa_bytes_1t = 512 * K * (2 + 1) + 4 * 512 * (K // 128)
    return {
        "value": 2.0 * M * N * K / step_s / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"quantize_act 4096x7168 and quantize_weight 7168x7168 in full "
                  f"({t1 - t0:.2f} s, {t2 - t1:.2f} s); FP64 GEMM on {rows} of 4096 output rows "
                  f"({t3 - t2:.2f} s), scaled x{M // rows} to the full step",
        "quantize_act_GBps": W_quant_bytes_fprop_act() / (t1 - t0) / 1e9,
        "quantize_act_1thread_GBps": qa_bytes_1t / (t5 - t4) / 1e9,
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
