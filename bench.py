"""Benchmark of the KDA hot path on one MI355X.

One step = one pass of the whole hot path over one synthetic batch:
  * kda_chunk_fwd on the prefill workload B=4, H=32, T=32768, dk=dv=128 (bf16 q/k/v/beta,
    float32 g and state, bf16 output, final state returned), and
  * kda_recurrent_step on the decode workload 1024 sequences x 32 heads (float32 128x128 states
    updated in place, one token each).
Inputs are generated on the GPU before the timed region (seeded; see inputs.py for the recipe).

Prints one JSON line.  ``value`` is prefill tokens per second: B*T tokens over the prefill
launch's own time (HIP events on its stream, averaged over the timed steps); ``ms_per_step`` is
the whole step, decode included, and ``decode`` reports the decode launch separately.
``roofline`` is for the prefill kernel (the dominant one): algorithmic HBM bytes per launch / its
average launch time.  ``mfma_busy`` is the prefill kernel's MFMA-busy fraction from the
committed counter summary (profiles/kernel_counters.json), when it was taken on the current
kernel source.  The variants after the steps cover the other workloads: the decay map in the
kernel, multi-token and fused decode (with and without the short convolution), the packed
64-sequence prefill, and the one-million-token prefill, plain and split in time.
``cpu_baseline`` times the C float64 reference token loop on a bounded sample of the prefill
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def prefill_alg_bytes(B, T, H, dk, dv, N, in_bytes=2, out_bytes=2):
    """Algorithmic HBM bytes of one prefill launch: every input read once, the output and the
    final state written once (q, k, v, beta in the input dtype; g float32; S0, S_T float32)."""
    th = B * T * H
    per_th = (2 * dk + dv) * in_bytes + dk * 4 + in_bytes + dv * out_bytes
    return th * per_th + 2 * N * H * dk * dv * 4


def prefill_alg_flops(B, T, H, dk, dv, C=32):
    """Algorithmic MFMA flops of the chunkwise form per launch, counting causal 16x16 tiles only
    (intra: A_kk, A_qk, T K~, T V; inter: W S, Q~ S, K_end^T V~, A_qk V~)."""
    th = B * T * H
    tiles = C // 16
    causal = tiles * (tiles + 1) // 2 / (tiles * tiles)       # fraction of causal tiles
    intra = 2 * (2 * C * dk * causal) + 2 * C * dk * causal + 2 * C * dv * causal
    inter = 2 * dk * dv * 3 + 2 * C * dv * causal
    return th * (intra + inter)


def prefill_gate_alg_bytes(B, T, H, dk, dv, N, in_bytes=2, out_bytes=2):
    """As prefill_alg_bytes with the decay map in the kernel: the logits z (input dtype) are read
    instead of float32 g, plus H float32 log-scales."""
    th = B * T * H
    per_th = (3 * dk + dv) * in_bytes + in_bytes + dv * out_bytes
    return th * per_th + 2 * N * H * dk * dv * 4 + H * 4


def decode_alg_bytes(N, H, dk, dv, in_bytes=2, out_bytes=2, K=1):
    """State read and written once per launch; K tokens of q, k, v, g, beta in, o out."""
    return N * H * (2 * dk * dv * 4 + K * ((2 * dk + dv) * in_bytes + dk * 4 + in_bytes +
                                           dv * out_bytes))


def plan_summary(ws, N):
    """What the automatic split planned, read from the head of its workspace: the segment length
    (0: no split), the layout (eager: every segment in the first pass) and the segment count of
    the longest sequence."""
    if ws is None:
        return {"segment_len": 0}
    p = ws[: (4 + N) * 4].cpu().view(torch.int32).tolist()
    return {"segment_len": p[0], "layout": "eager" if p[3] else "deferred", "segments_of_longest": max(p[4:4 + N])}


def time_launches(fn, reps=10, groups=3, warmup=5):
    """Duration of one of fn's launches in ms (HIP events on the current stream): the median over
    `groups` groups of `reps` back-to-back launches, after `warmup` launches."""
    import statistics
    for _ in range(warmup):
        fn()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    out = []
    for _ in range(groups):
        e[0].record()
        for _ in range(reps):
            fn()
        e[1].record()
        torch.cuda.synchronize()
        out.append(e[0].elapsed_time(e[1]) / reps)
    return statistics.median(out)


def kernel_source_hash(name):
    path = os.path.join(ROOT, "linear_attention_chunkwise_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _counters(kernel_key, source_name):
    """The kernel's record in the committed rocprofv3 counter summary, or None when it is missing
    or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "kernel_counters.json")
    try:
        rec = json.load(open(path))[kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256_16") != kernel_source_hash(source_name):
        return None
    return rec


def measured_traffic(kernel_key, source_name):
    """HBM bytes per launch (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the
    counter reads for a plain device copy of known size), or None."""
    rec = _counters(kernel_key, source_name)
    if rec is None or "fetch_kib" not in rec:
        return None
    return (rec["fetch_kib"] * rec["fetch_scale"] + rec["write_kib"] * rec["write_scale"]) * 1024


def measured_mfma_busy(kernel_key, source_name):
    """Fraction of SIMD cycles with the MFMA unit busy during the kernel, or None:
    SQ_VALU_MFMA_BUSY_CYCLES / (SQ_BUSY_CYCLES / 32 shader engines x 1024 SIMDs) per dispatch
    (SQ_BUSY_CYCLES sums the shader engines, SQ_VALU_MFMA_BUSY_CYCLES every SIMD; the same
    expression reads 0.985 for a loop of independent MFMAs)."""
    rec = _counters(kernel_key, source_name)
    return None if rec is None else rec.get("mfma_busy_frac")


def calibrate_copy():
    """A plain 1 GiB device-to-device copy (1 GiB read + 1 GiB written per launch), run under
    rocprofv3 to find the scale of the FETCH_SIZE / WRITE_SIZE counters."""
    x = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    x.fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(2):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": x.numel() * 4,
                      "bytes_written": x.numel() * 4, "launches": 2}), flush=True)


def calibrate_peaks(dev):
    """Measured ceilings on this machine (bench_calib.so, built beside this file): the issue rate
    of v_mfma_f32_16x16x32_bf16 with independent accumulators on every SIMD, and a grid-stride
    device copy of 1 GiB (1 GiB read + 1 GiB written).  None if the library was not built."""
    import ctypes
    path = os.path.join(ROOT, "bench_calib.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.calib_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.calib_mfma_flops.restype = ctypes.c_double
    lib.calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                               ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    blocks, iters = 2048, 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)

    def mfma():
        assert lib.calib_mfma(ctypes.c_void_p(out.data_ptr()), blocks, iters, stream) == 0

    m_ms = time_launches(mfma, reps=5)
    x = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)

    def copy():
        assert lib.calib_copy(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                              x.numel() // 4, 1024, stream) == 0

    c_ms = time_launches(copy)
    mfma = lib.calib_mfma_flops(blocks, iters) / (m_ms * 1e-3) / 1e12
    return {"mfma_bf16_TFLOPs": mfma,
            "copy_GBps": 2 * x.numel() * 4 / (c_ms * 1e-3) / 1e9,
            "what": "bench_calib.hip: 8 independent v_mfma_f32_16x16x32_bf16 chains per wave, "
                    "2048 x 256 threads; grid-stride float4 copy, 1024 x 256 threads"}


def cpu_baseline(x, units_wanted=None):
    """The C float64 reference token loop on the first `units_wanted` (sequence, head) units (all
    of them by default: the whole prefill workload is a few seconds of host work)."""
    from oracle import c_oracle
    B, T, H, dk = x["q"].shape
    units = [(n, h) for n in range(B) for h in range(H)]
    if units_wanted is not None:
        units = units[:units_wanted]
    seqs = sorted({n for n, _ in units})
    sub = {k: x[k][seqs].cpu() for k in ("q", "k", "v", "g", "beta")}
    S0 = x["S0"][seqs].cpu()
    remap = {n: i for i, n in enumerate(seqs)}
    u2 = [(remap[n], h) for n, h in units]
    threads = c_oracle.threads()
    t0 = time.perf_counter()
    c_oracle.kda_units(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], S0, None, u2)
    dt = time.perf_counter() - t0
    token_heads = len(units) * T
    return {"value": token_heads / H / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(units)} of {B * H} (sequence, head) units x {T} tokens of the prefill "
                      f"workload ({token_heads} token-heads, float64 C token loop, OpenMP over units, "
                      f"{dt:.1f} s wall, {cpu_model()}); tokens/s = token-heads/s / H"}


def props_cu(dev):
    return torch.cuda.get_device_properties(dev).multi_processor_count


def cpu_model():
    """The host CPU's model name as the kernel reports it (unknown if it does not)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "CPU model unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the variants timed after the steps (decay map in the kernel, "
                         "multi-token and fused decode, packed and long prefill)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="profile helper: run only the prefill launch per step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: every workload here fits "
                                   "one MI355X; --gpus must be 1"}))
        sys.exit(2)

    from linear_attention_chunkwise_amd import binding, inputs
    binding.load()
    dev = torch.device("cuda:0")
    cfg = inputs.CONFIGS["prefill_b4_h32_t32k_d128"]
    dcfg = inputs.DECODE_CONFIG
    x = inputs.make_prefill_inputs(cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv, dtype=cfg.dtype, seed=0,
                                   device=dev, A_std=cfg.A_std, S0_std=cfg.S0_std,
                                   near_gmin_frac=cfg.near_gmin_frac,
                                   with_logits=not args.no_extras)
    d = inputs.make_decode_inputs(dcfg.N, dcfg.H, dcfg.dk, dcfg.dv, seed=0, device=dev)
    B, T, H, dk, dv = cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    ST = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    od = torch.empty((dcfg.N, dcfg.H, dcfg.dv), dtype=torch.bfloat16, device=dev)
    S = d["S"]
    torch.cuda.synchronize()

    def step(evs=None):
        if evs: evs[0].record()
        binding.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], o=o, S_T=ST)
        if evs: evs[1].record()
        if not args.prefill_only:
            binding.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], S, o=od)
        if evs: evs[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    pbytes = prefill_alg_bytes(B, T, H, dk, dv, B)
    pflops = prefill_alg_flops(B, T, H, dk, dv)
    dbytes = decode_alg_bytes(dcfg.N, dcfg.H, dcfg.dk, dcfg.dv)
    achieved = pbytes / (pre_ms * 1e-3) / 1e9
    res = {
        "metric": "KDA prefill tokens/s (H=32,d=128,T=32K) + %MFMA peak; decode GB/s vs HBM",
        "value": B * T / (pre_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, generated on the GPU: q,k L2-normalised N(0,1), v N(0,1), "
                "g=-5*sigmoid(exp(A)z), beta=sigmoid(N(0,1)), S0 N(0,0.1))",
        "config": {"workload": "prefill B=4 H=32 T=32768 dk=dv=128 bf16 + decode 1024 seq x 32 "
                               "heads fp32 128x128 state", "global_batch": B, "seq_len": T,
                   "heads": H, "dk": dk, "dv": dv, "decode_sequences": dcfg.N,
                   "parallelism": "single GPU"},
        "prefill": {"ms": pre_ms, "tokens_per_s": B * T / (pre_ms * 1e-3),
                    "alg_bytes": pbytes, "alg_GBps": achieved,
                    "alg_mfma_tflops": pflops / (pre_ms * 1e-3) / 1e12,
                    "mfma_frac": pflops / (pre_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                    "mfma_busy": measured_mfma_busy("prefill_kernel<128,bf16,bf16>",
                                                    "kda_prefill.hip"),
                    "what": "mfma_frac: the chunkwise form's algorithmic MFMA flops (causal tiles "
                            "only) per second over the dense bf16 peak; mfma_busy: the kernel's "
                            "measured MFMA-busy fraction of SIMD cycles (rocprofv3 counters)"},
        "decode": None if args.prefill_only else {
            "us": dec_ms * 1e3, "alg_bytes": dbytes, "GBps": dbytes / (dec_ms * 1e-3) / 1e9,
            "frac_hbm": dbytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": measured_traffic("decode_kernel<128,128,bf16,bf16>", "kda_decode.hip"),
            "what": "kda_recurrent_step: one token per (sequence, head), 1024 sequences x 32 heads, "
                    "float32 128x128 states updated in place"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic("prefill_kernel<128,bf16,bf16>", "kda_prefill.hip"),
                     "kernel": "prefill_kernel<128,bf16,bf16 out>",
                     "limiter": "instruction issue and dependent-chain latency inside a workgroup "
                                "(about 905 VALU and 90 MFMA instructions per SIMD per 32-token "
                                "chunk); neither HBM (frac above) nor the MFMA pipes (prefill."
                                "mfma_busy) is saturated"},
    }
    if not args.no_extras and not args.prefill_only:
        # variants, timed after the steps (not part of ms_per_step)
        g_ms = time_launches(lambda: binding.chunk_fwd_gate(
            x["q"], x["k"], x["v"], x["z"], x["A_log"], x["beta"], x["S0"], o=o, S_T=ST))
        gbytes = prefill_gate_alg_bytes(B, T, H, dk, dv, B)
        res["prefill_gate"] = {"ms": g_ms, "tokens_per_s": B * T / (g_ms * 1e-3),
                               "alg_bytes": gbytes, "alg_GBps": gbytes / (g_ms * 1e-3) / 1e9,
                               "what": "kda_chunk_fwd_gate: g = -5 Sigmoid(exp(A_h) z) formed "
                                       "in the kernel from bf16 z"}
        K = 4
        m = inputs.make_prefill_inputs(dcfg.N, K, dcfg.H, dcfg.dk, dcfg.dv, seed=1, device=dev)
        om = torch.empty((dcfg.N, K, dcfg.H, dcfg.dv), dtype=torch.bfloat16, device=dev)
        Sm = m["S0"]
        m_ms = time_launches(lambda: binding.recurrent_multi(m["q"], m["k"], m["v"], m["g"],
                                                             m["beta"], Sm, o=om))
        mbytes = decode_alg_bytes(dcfg.N, dcfg.H, dcfg.dk, dcfg.dv, K=K)
        res["decode_multi"] = {"K": K, "us": m_ms * 1e3, "us_per_token": m_ms * 1e3 / K,
                               "alg_bytes": mbytes, "GBps": mbytes / (m_ms * 1e-3) / 1e9,
                               "what": "kda_recurrent_multi: 4 tokens per (sequence, head) per "
                                       "state pass, 1024 sequences x 32 heads"}
        del m, om, Sm
        f = inputs.make_fused_decode_inputs(dcfg.N, K, dcfg.H, dcfg.dk, dcfg.dv, seed=2, device=dev)
        yf = torch.empty((dcfg.N, K, dcfg.H, dcfg.dv), dtype=torch.bfloat16, device=dev)
        f_ms = time_launches(lambda: binding.recurrent_multi_fused(
            f["q"], f["k"], f["v"], f["z"], f["A_log"], f["beta_logit"], f["G"], f["S"],
            norm_weight=f["norm_weight"], y=yf))
        # per token-head: q, k, z, v, G, beta logit in, y out (bf16); state read + written once
        fbytes = dcfg.N * dcfg.H * (2 * dcfg.dk * dcfg.dv * 4 +
                                    K * ((3 * dcfg.dk + 2 * dcfg.dv) * 2 + 2 + dcfg.dv * 2))
        res["decode_multi_fused"] = {"K": K, "us": f_ms * 1e3, "us_per_token": f_ms * 1e3 / K,
                                     "alg_bytes": fbytes, "GBps": fbytes / (f_ms * 1e-3) / 1e9,
                                     "frac_hbm": fbytes / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                     "what": "kda_recurrent_multi_fused: the 4-token pass with q/k "
                                             "L2Norm, beta = Sigmoid(logit), decay map, "
                                             "Sigmoid(G) * RMSNorm(o~) fused in"}
        W = 4
        cv = inputs.make_conv_inputs(dcfg.N, dcfg.H, dcfg.dk, dcfg.dv, W, seed=3, device=dev)
        fc_ms = time_launches(lambda: binding.recurrent_multi_fused(
            f["q"], f["k"], f["v"], f["z"], f["A_log"], f["beta_logit"], f["G"], f["S"],
            norm_weight=f["norm_weight"], y=yf, conv_weight=cv["conv_weight"],
            conv_state=cv["conv_state"]))
        # plus the window read and written once (bf16) and the taps (float32, per head)
        nch = 2 * dcfg.dk + dcfg.dv
        fcbytes = fbytes + dcfg.N * dcfg.H * nch * (W - 1) * 2 * 2 + dcfg.H * nch * W * 4
        res["decode_multi_fused_conv"] = {
            "K": K, "W": W, "us": fc_ms * 1e3, "us_per_token": fc_ms * 1e3 / K,
            "alg_bytes": fcbytes, "GBps": fcbytes / (fc_ms * 1e-3) / 1e9,
            "frac_hbm": fcbytes / (fc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "what": "the fused 4-token pass with the 4-tap short convolution and Swish on q, k, v "
                    "in front, its window committed with the state"}
        del f, yf, cv
        # packed prefill: 64 sequences, lognormal lengths (median 1024, longest 65536)
        vcfg = inputs.CONFIGS["varlen64_h32_d128"]
        xv = inputs.make_config_inputs(vcfg, seed=0, device=dev)
        Tv = xv["q"].shape[1]
        ov = torch.empty((1, Tv, vcfg.H, vcfg.dv), dtype=torch.bfloat16, device=dev)
        STv = torch.empty((xv["N"], vcfg.H, vcfg.dk, vcfg.dv), dtype=torch.float32, device=dev)
        vneed = binding.chunk_fwd_workspace_size(xv["N"], Tv, vcfg.H, vcfg.dk, vcfg.dv, True)
        wsv = torch.empty(vneed, dtype=torch.uint8, device=dev) if vneed else None
        v_ms = time_launches(lambda: binding.chunk_fwd(xv["q"], xv["k"], xv["v"], xv["g"], xv["beta"],
                                                       xv["S0"], xv["cu_seqlens"], o=ov, S_T=STv,
                                                       workspace=wsv))
        plan = plan_summary(wsv, xv["N"])
        vw_ms = time_launches(lambda: binding.chunk_fwd(xv["q"], xv["k"], xv["v"], xv["g"], xv["beta"],
                                                        xv["S0"], xv["cu_seqlens"], o=ov, S_T=STv,
                                                        workspace=None))
        lens = xv["cu_seqlens"][1:] - xv["cu_seqlens"][:-1]
        vbytes = prefill_alg_bytes(1, Tv, vcfg.H, vcfg.dk, vcfg.dv, xv["N"])
        res["prefill_varlen64"] = {"ms": v_ms, "whole_ms": vw_ms, "plan": plan,
                                   "tokens": Tv, "tokens_per_s": Tv / (v_ms * 1e-3),
                                   "longest": int(lens.max()), "alg_GBps": vbytes / (v_ms * 1e-3) / 1e9,
                                   "what": "kda_chunk_fwd on 64 packed sequences (cu_seqlens), "
                                           "H=32, d=128, with the workspace of its automatic plan "
                                           "(ms; plan: its segment length, 0 for no split, its "
                                           "layout and the longest sequence's segments) and with "
                                           "no workspace (whole_ms: every sequence whole, the "
                                           "longest first)"}
        del xv, ov, STv, wsv
        # long prefill: one sequence of 2^20 tokens, 32 heads: plain (64 workgroups) and split in
        # time with the library's segment count for this GPU (kda_chunk_fwd_cp_segments)
        lcfg = inputs.CONFIGS["long_b1_h32_t1m_d128"]
        xl = inputs.make_config_inputs(lcfg, seed=0, device=dev)
        ol = torch.empty((1, lcfg.T, lcfg.H, lcfg.dv), dtype=torch.bfloat16, device=dev)
        STl = torch.empty((1, lcfg.H, lcfg.dk, lcfg.dv), dtype=torch.float32, device=dev)
        lbytes = prefill_alg_bytes(1, lcfg.T, lcfg.H, lcfg.dk, lcfg.dv, 1)
        l_ms = time_launches(lambda: binding.chunk_fwd(xl["q"], xl["k"], xl["v"], xl["g"], xl["beta"],
                                                       xl["S0"], o=ol, S_T=STl, workspace=None),
                             reps=2, groups=1, warmup=1)
        need = binding.chunk_fwd_workspace_size(1, lcfg.T, lcfg.H, lcfg.dk, lcfg.dv, False)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        la_ms = time_launches(lambda: binding.chunk_fwd(xl["q"], xl["k"], xl["v"], xl["g"], xl["beta"],
                                                        xl["S0"], o=ol, S_T=STl, workspace=ws),
                              reps=2, groups=1, warmup=1)
        res["prefill_long_t1m"] = {
            "tokens": lcfg.T, "ms": la_ms, "whole_ms": l_ms, "plan": plan_summary(ws if need else None, 1),
            "tokens_per_s": lcfg.T / (la_ms * 1e-3), "alg_GBps": lbytes / (la_ms * 1e-3) / 1e9,
            "what": "B=1, H=32, T=1048576, d=128 (13 of 128 key channels per head near g_min): "
                    "kda_chunk_fwd with the workspace of its automatic split (ms; plan as for "
                    "varlen64) and without (whole_ms, 64 workgroups)"}
        # the same sequence from logits: g formed in the kernel, whole and split in time
        del xl
        xz = inputs.make_prefill_inputs(lcfg.B, lcfg.T, lcfg.H, lcfg.dk, lcfg.dv, seed=0, device=dev,
                                        A_std=lcfg.A_std, near_gmin_frac=lcfg.near_gmin_frac,
                                        with_logits=True)
        del xz["g"]
        lz_ms = time_launches(lambda: binding.chunk_fwd_gate(xz["q"], xz["k"], xz["v"], xz["z"], xz["A_log"],
                                                             xz["beta"], xz["S0"], o=ol, S_T=STl, workspace=None),
                              reps=2, groups=1, warmup=1)
        lza_ms = time_launches(lambda: binding.chunk_fwd_gate(xz["q"], xz["k"], xz["v"], xz["z"], xz["A_log"],
                                                              xz["beta"], xz["S0"], o=ol, S_T=STl, workspace=ws),
                               reps=2, groups=1, warmup=1)
        res["prefill_long_t1m_gate"] = {
            "tokens": lcfg.T, "ms": lza_ms, "whole_ms": lz_ms, "plan": plan_summary(ws if need else None, 1),
            "tokens_per_s": lcfg.T / (lza_ms * 1e-3),
            "what": "the same sequence from bf16 logits z and A_h: kda_chunk_fwd_gate with the "
                    "workspace (ms) and without (whole_ms)"}
        del xz, ol, STl, ws
        # context for the HBM fractions: what the vendor's own read+write kernels reach here
        xb = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        yb = torch.empty_like(xb)
        nb = 2 * xb.numel() * 4
        c_ms = time_launches(lambda: yb.copy_(xb))
        r_ms = time_launches(lambda: xb.mul_(1.0))
        res["hbm_reference"] = {
            "device_copy_GBps": nb / (c_ms * 1e-3) / 1e9,
            "inplace_scale_GBps": nb / (r_ms * 1e-3) / 1e9,
            "decode_vs_best": dbytes / (dec_ms * 1e-3) / 1e9 / (nb / (min(c_ms, r_ms) * 1e-3) / 1e9),
            "what": "torch device copy and in-place multiply of a 1 GiB float32 buffer (1 GiB read "
                    "+ 1 GiB written per launch), timed like the variants; decode_vs_best = decode "
                    "GB/s over the faster of the two"}
        del xb, yb
        cal = calibrate_peaks(dev)
        if cal is not None:
            cal["prefill_alg_mfma_frac_of_measured"] = pflops / (pre_ms * 1e-3) / 1e12 / cal["mfma_bf16_TFLOPs"]
            cal["decode_frac_of_measured_copy"] = dbytes / (dec_ms * 1e-3) / 1e9 / cal["copy_GBps"]
        res["calibration"] = cal
    if not args.no_cpu_baseline:
        del o, od
        res["cpu_baseline"] = cpu_baseline(x)
    props = torch.cuda.get_device_properties(dev)
    res["env"] = {"device": props.name, "arch": getattr(props, "gcnArchName", None),
                  "compute_units": props.multi_processor_count, "hip": torch.version.hip,
                  "torch": torch.__version__}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
