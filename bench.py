"""Benchmark of the SpinQuant online hot path on one MI355X.

One step = the R4 / down_proj path on a Qwen3-8B-shaped batch:
    spin_fwht_quant  X [4096][12288] fp16 -> Hadamard 12288 (H_12 (x) H_1024)
                     / sqrt(12288) -> per-token INT4 codes + scales
    spin_w4a4_gemm   codes x INT4 weights [4096][12288] (Hadamard folded
                     offline, untimed) -> Y [4096][4096] fp32
Inputs are synthetic (seeded, 0.1% outlier channels x100) and resident in HBM
before timing starts.  Several input / output buffer sets rotate so that each
step reads activations that the 256 MB Infinity Cache no longer holds.

Prints ONE JSON line.  `value` is fwht_quant's achieved GB/s (algorithmic
bytes per launch / mean launch time, from HIP events on the launch stream);
the GEMM's TOPS follow in `gemm_tops`; `roofline` describes the kernel that
dominates the step (the GEMM, against the dense INT8 peak the metric names and,
in `issued`, against the dense FP6 peak of the instruction it issues) and
`roofline_fwht_quant` the other one.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--gpus 1]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0       # MI355X dense INT8 MFMA
FP6_PEAK_TOPS = 10100.0       # MI355X dense FP6 / FP4 MFMA (the instruction the down_proj GEMM issues)
M, K, N, HAD_N = 4096, 12288, 4096, 12288
FWHT_BYTES_PER_TOKEN = 2 * K + K // 2 + 4          # fp16 in + packed codes + fp32 scale
# The VALU view of fwht_quant_k12288_mfma: one wave per row issues 2181.2
# VALU instructions, 72 of them MFMA (rocprofv3 SQ_INSTS_VALU and
# SQ_INSTS_MFMA over SQ_WAVES on the down_proj workload), so 2109.2 vector
# lane-operations per lane for its 192 elements (the hi/lo split, the
# 50-operation H12, absmax, quantize and pack): 10.99 per element, against
# the chip's 256 CUs x 64 lanes x 2.4 GHz = 39.3 T lane-operations per second.
FWHT_VALU_OPS_PER_ELEMENT = (8934272.0 - 294912.0) / 4096.0 / 192.0
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
KV_T, KV_H, KV_D = 4096, 32, 128
KV_BYTES_PER_GROUP = 2 * KV_D + KV_D // 2 + 2      # fp16 in + packed codes + fp16 scale

# Measured HBM traffic per launch (bytes read, bytes written) from two
# rocprofv3 passes (--pmc FETCH_SIZE, then --pmc WRITE_SIZE) over
# `bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-extra --no-fused
# --copy-calibration`.
# Each counter is scaled by what it reads for a 1 GiB device-to-device copy in
# the same run: FETCH_SIZE reported 524326.5 KiB (factor 2.0), WRITE_SIZE
# 1048576 KiB (factor 1.0).  A figure holds only for the kernel code it was
# taken on (SHA-256 prefixes of the sources without comments, below); after
# any change to that code it reports null.
CSRC = os.path.join(ROOT, "rotation_bit_quantization_amd", "csrc")
TRAFFIC = {
    "fwht_quant": {"sources": {"fwht_quant.hip": "534a39ba359043de", "fwht12288.h": "aeebefa0ba05bd5b",
                              "spin_device.h": "cf499208765bf25d"},
                  "read": 101783406, "write": 25296984},
    "w4a4_gemm": {"sources": {"w4a4_gemm.hip": "3844c69f6b0ec334", "w4a4_gemm_fp6.hip": "135e165e956c950d",
                              "gemm_fp6_tile.h": "935c1f9d3fce0dba", "gemm_common.h": "0d5f030ce5ed28cd",
                              "spin_device.h": "cf499208765bf25d"},
                 "read": 151337580, "write": 67108864},
    "w4a4_gemm_f6f6": {"sources": {"w4a4_gemm_fp6.hip": "135e165e956c950d", "gemm_fp6_tile.h": "935c1f9d3fce0dba",
                                   "gemm_common.h": "0d5f030ce5ed28cd", "spin_device.h": "cf499208765bf25d"},
                      "read": 227252450, "write": 67108864},
    "kv_quant": {"sources": {"kv_quant.hip": "72f25f38e706d384", "spin_device.h": "cf499208765bf25d"},
                "read": 33640465, "write": 8650752},
}


def source_digest(path):
    """SHA-256 prefix of a C++/HIP source with its comments and blank lines
    removed, so that only a change to the code itself invalidates a figure."""
    import hashlib
    import re
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic(kernel):
    """Measured bytes per launch, or None if the kernel's code has changed."""
    entry = TRAFFIC[kernel]
    for name, digest in entry["sources"].items():
        try:
            if source_digest(os.path.join(CSRC, name)) != digest:
                return None
        except OSError:
            return None
    return entry["read"] + entry["write"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=4, help="rotating buffer sets (cold HBM)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kv", action="store_true")
    ap.add_argument("--no-fused", action="store_true", help="skip the one-launch down_proj A/B")
    ap.add_argument("--no-f6", action="store_true", help="skip the FP6-operand-layout step")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the qkv_proj GEMM and the decoder-layer chain measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    return ap.parse_args()


def cpu_baseline(x_host):
    """Time the oracle (untuned) on a bounded sample of the same workload."""
    import oracle
    from oracle import gemm as ogemm
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - informational only
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    rows_f = M                                     # the whole activation batch
    oracle.hadamard(HAD_N)                         # build H once, outside the timed region
    t0 = time.perf_counter()
    pk, s, _ = oracle.fwht_quant(x_host[:rows_f], HAD_N)
    t_f = time.perf_counter() - t0
    rows_g = M
    qx = oracle.unpack_int4(pk[:rows_g])
    # weight codes for the timing sample: seeded uniform codes of the workload's shape
    wq_codes = np.random.default_rng(7).integers(-7, 8, size=(N, K)).astype(np.int8)
    t0 = time.perf_counter()
    ogemm.gemm_int_codes(qx, wq_codes)
    t_g = time.perf_counter() - t0
    # the qkv_proj shape, 4096 tokens x 6144 x 4096, on seeded uniform codes
    rng4 = np.random.default_rng(8)
    qx4 = rng4.integers(-7, 8, size=(M, 4096)).astype(np.int8)
    qw4 = rng4.integers(-7, 8, size=(6144, 4096)).astype(np.int8)
    t0 = time.perf_counter()
    ogemm.gemm_int_codes(qx4, qw4)
    t_g4 = time.perf_counter() - t0
    omp = ogemm.num_threads()
    return {
        "value": rows_f * FWHT_BYTES_PER_TOKEN / t_f / 1e9,
        "unit": "GB/s",
        "cores": max(omp, blas_threads or 1),
        "kind": "oracle",
        "sample": (f"the whole down_proj workload: fwht_quant on all {rows_f} tokens (dense float64 "
                   f"X.H_12288 + float32 quantizer) in {t_f:.2f} s; int64 C GEMM on {rows_g} tokens x "
                   f"{N} x {K} in {t_g:.2f} s (seeded uniform weight codes); int64 C GEMM at the qkv_proj "
                   f"shape {M} x 6144 x 4096 in {t_g4:.2f} s"),
        "gemm_tops": 2.0 * rows_g * N * K / t_g / 1e12,
        "gemm_qkv_tops": 2.0 * M * 6144 * 4096 / t_g4 / 1e12,
        "host_cpus": cores,
        "blas_threads": blas_threads,
        "omp_threads": omp,
    }


def _time(fn, reps, stream):
    """Mean milliseconds of fn() over `reps` launches, HIP events (without the
    system-scope fence) on `stream`."""
    import torch
    from rotation_bit_quantization_amd.timing import hip_events
    he = hip_events()
    ev = [[he.new() for _ in range(2)] for _ in range(reps)]
    for i in range(reps):
        he.record(ev[i][0], stream)
        fn(i)
        he.record(ev[i][1], stream)
    torch.cuda.synchronize()
    t = float(np.mean([he.ms(a, b) for a, b in ev]))
    he.release()
    return t


def kv_qkv_workload(args, dev, stream, kv, sets):
    """The KV step of one attention layer in one launch (spin_kv_qkv): K rotated +
    INT4, V INT4, then the same with Q rotated (fp32 out); against K and V as two
    spin_kv_quant launches.  Buffer sets rotate as in the timed step."""
    import torch
    from rotation_bit_quantization_amd import spin
    src = {n: torch.from_numpy(kv[n]).to(dev) for n in ("q", "k", "v")}
    ins = [src] + [{n: t.clone() for n, t in src.items()} for _ in range(sets - 1)]
    outs = []
    for _ in range(sets):
        outs.append({
            "K_codes": torch.empty((KV_T, KV_H, KV_D // 2), dtype=torch.uint8, device=dev),
            "K_scale": torch.empty((KV_T, KV_H), dtype=torch.float16, device=dev),
            "V_codes": torch.empty((KV_T, KV_H, KV_D // 2), dtype=torch.uint8, device=dev),
            "V_scale": torch.empty((KV_T, KV_H), dtype=torch.float16, device=dev),
            "Q_rot": torch.empty((KV_T, KV_H, KV_D), dtype=torch.float32, device=dev)})

    def kv_one(i):
        j = i % sets
        spin.spin_kv_qkv(ins[j]["k"], ins[j]["v"], out=outs[j])

    def qkv_one(i):
        j = i % sets
        spin.spin_kv_qkv(ins[j]["k"], ins[j]["v"], ins[j]["q"], out=outs[j])

    def kv_two(i):
        j = i % sets
        o = outs[j]
        spin.spin_kv_quant(ins[j]["k"], 1, codes=o["K_codes"], scale=o["K_scale"])
        spin.spin_kv_quant(ins[j]["v"], 0, codes=o["V_codes"], scale=o["V_scale"])

    res = {"workload": "K, V [4096][32][128] fp16 (R3 H_128 on K, INT4 + fp16 scale both); Q [4096][32][128] "
                       "rotated to fp32"}
    kv_bytes = 2 * KV_T * KV_H * KV_BYTES_PER_GROUP
    q_bytes = KV_T * KV_H * (2 * KV_D + 4 * KV_D)
    for name, fn, nbytes in (("kv_one_launch", kv_one, kv_bytes), ("kv_two_launches", kv_two, kv_bytes),
                             ("qkv_one_launch", qkv_one, kv_bytes + q_bytes)):
        for i in range(args.warmup):
            fn(i)
        s = _time(fn, args.steps, stream) / 1e3
        res[name] = {"us": s * 1e6, "GBps": nbytes / s / 1e9, "frac_of_hbm": nbytes / s / 1e9 / HBM_PEAK_GBPS}
    return res


def machine_ceilings(fwht_tbps, gemm_tops):
    """Measured ceilings of this GPU (libspin_probe), reported beside the
    published peaks that the roofline fractions use: the INT8 and FP16 MFMA
    instructions the hot path issues, run back to back on the hot path's kind of
    data by eight waves per CU, with the shader clock meanwhile, a streaming
    read of 2 GiB, one CU's LDS bytes per cycle in the FP6 GEMM's access
    patterns (operand reads, field writes) and for contiguous 16-byte reads,
    a 1 GiB device copy, and the event-timed duration of a streaming read of
    as many bytes as kv_quant and fwht_quant move, from buffers that rotate
    out of the caches (the floor those kernels are timed against)."""
    from rotation_bit_quantization_amd import machine
    i8 = machine.mfma_rate(0)
    f16 = machine.mfma_rate(1)
    f6 = machine.mfma_rate(2)
    rd = machine.read_bandwidth()
    lds = [machine.lds_rate(m) for m in (0, 1, 2)]
    cp = machine.copy_rate()
    floors = {f"{nb / 1e6:.1f} MB ({name})": round(machine.read_floor_us(nb), 2)
              for name, nb in (("kv_quant's bytes", KV_T * KV_H * KV_BYTES_PER_GROUP),
                               ("fwht_quant's bytes", M * FWHT_BYTES_PER_TOKEN))}
    return {
        "mfma_i32_32x32x32_i8": {"tops": round(i8["tops"], 1), "clock_ghz": round(i8["clock_ghz"], 3)},
        "mfma_f32_32x32x16_f16": {"tflops": round(f16["tops"], 1), "clock_ghz": round(f16["clock_ghz"], 3)},
        "mfma_scale_f32_32x32x64_fp6": {"tops": round(f6["tops"], 1), "clock_ghz": round(f6["clock_ghz"], 3)},
        "hbm_read_tbps": round(rd["tbps"], 3),
        "copy_tbps": round(cp["tbps"], 3),
        "read_floor_us": floors,
        "lds_bytes_per_clk_per_cu": {"fp6_operand_reads_b64": round(lds[0]["bytes_per_clk_per_cu"], 1),
                                     "fp6_field_writes_b64": round(lds[1]["bytes_per_clk_per_cu"], 1),
                                     "contiguous_reads_b128": round(lds[2]["bytes_per_clk_per_cu"], 1)},
        "w4a4_gemm_frac_of_measured_int8": round(gemm_tops / i8["tops"], 4),
        "w4a4_gemm_frac_of_measured_fp6": round(gemm_tops / f6["tops"], 4),
        "fwht_quant_frac_of_measured_read": round(fwht_tbps / rd["tbps"], 4),
        "note": "measured on this GPU; the roofline objects keep the published peaks",
    }


def tiny_workload(args, dev, stream):
    """The tiny configuration, X 64 x 256 fp32 (4 outlier channels x50), W
    256 x 256: latency of its two chains, (i) fwht_quant with H_256 + the GEMM on
    W folded with H_256, (ii) quant-only activations X.R (R a Haar rotation
    of order 256, applied on the host) + the GEMM on W folded with R.  74 KB of
    data: launch-bound, reported as microseconds per call."""
    import torch
    from rotation_bit_quantization_amd import spin, synth
    cfg = synth.tiny_config()
    X = torch.from_numpy(cfg["x"]).to(dev)
    XR = torch.from_numpy((cfg["x"].astype(np.float64) @ cfg["r"].astype(np.float64)).astype(np.float32)).to(dev)
    W = torch.from_numpy(cfg["w"]).to(dev)
    R = torch.from_numpy(cfg["r"].astype(np.float32)).to(dev)
    _, Wh, wsh = spin.spin_fold_rotation(W, None, 256)
    _, Wr, wsr = spin.spin_fold_rotation(W, R, 256)
    Xq, xs, _ = spin.spin_fwht_quant(X, 256)
    Xq2, xs2, _ = spin.spin_fwht_quant(XR, 1)
    Y = torch.empty((64, 256), dtype=torch.float32, device=dev)
    reps = max(20, args.steps)
    for _ in range(args.warmup):
        spin.spin_fwht_quant(X, 256, Xq=Xq, x_scale=xs)
        spin.spin_w4a4_gemm(Xq, xs, Wh, wsh, Y=Y)
    torch.cuda.synchronize()
    return {"workload": "X 64x256 fp32, W 256x256: (i) H_256 fwht_quant + GEMM on the H_256 fold, "
                        "(ii) quant-only X.R + GEMM on the Haar-R fold",
            "fwht_quant_h256_us": _time(lambda i: spin.spin_fwht_quant(X, 256, Xq=Xq, x_scale=xs), reps, stream) * 1e3,
            "gemm_h256_us": _time(lambda i: spin.spin_w4a4_gemm(Xq, xs, Wh, wsh, Y=Y), reps, stream) * 1e3,
            "quant_only_us": _time(lambda i: spin.spin_fwht_quant(XR, 1, Xq=Xq2, x_scale=xs2), reps, stream) * 1e3,
            "gemm_haar_us": _time(lambda i: spin.spin_w4a4_gemm(Xq2, xs2, Wr, wsr, Y=Y), reps, stream) * 1e3}


def vendor_int8_workload(args, dev, stream):
    """The vendor int8 GEMM (torch._int_mm; hipBLASLt on ROCm) on the down_proj
    shape, M = N = 4096, K = 12288, with the same INT4 values held one per byte
    and activations rotating over the buffer sets as in the timed step: a
    reference for the W4A4 kernel, which reads half the operand bytes but has to
    widen or convert them.  Three outputs are checked against numpy on the host."""
    import torch
    rng = np.random.default_rng(7)
    sets = max(1, args.sets)
    a0 = rng.integers(-7, 8, size=(M, K), dtype=np.int8)
    w = rng.integers(-7, 8, size=(N, K), dtype=np.int8)
    A = [torch.from_numpy(a0).to(dev)]
    A += [A[0].clone() for _ in range(1, sets)]
    B = torch.from_numpy(w).to(dev).t()            # [K, N], column-major
    reps = max(10, args.steps)
    for i in range(args.warmup):
        c = torch._int_mm(A[i % sets], B)
    torch.cuda.synchronize()
    got = c[0, :3].cpu().numpy().astype(np.int64)
    ref = a0[0].astype(np.int64) @ w[:3].astype(np.int64).T
    t = _time(lambda i: torch._int_mm(A[i % sets], B), reps, stream)
    tops = 2.0 * M * N * K / (t * 1e-3) / 1e12
    return {"workload": "torch._int_mm (hipBLASLt) int8 x int8 -> int32, 4096 x 4096 x 12288, codes in [-7, 7]",
            "us": t * 1e3, "tops": tops, "frac_of_int8_peak": tops / INT8_PEAK_TOPS,
            "checked": bool(np.array_equal(got, ref))}


def extra_workloads(args, dev, stream):
    """qkv_proj (R1 folded, quant-only activations) and the decoder-layer linear
    chain at M = 8192 and M = 16 (decode).  Folds run once, untimed."""
    import torch
    from rotation_bit_quantization_amd import spin, synth
    out = {}
    reps = max(5, args.steps // 2)

    # qkv_proj: X 4096 x 4096 fp16 (residual in the R1 basis), W 4096 x 6144 folded with R1
    q = synth.qkv_config()
    from rotation_bit_quantization_amd import checks
    r1 = torch.from_numpy(q["r"]).to(dev)
    out["rotation_inputs_orthogonality"] = {"R1 Haar 4096 (qkv_proj)": checks.orthogonality_error(r1)}
    _, Wq0, ws = spin.spin_fold_rotation(torch.from_numpy(q["w"]).to(dev), r1, 4096)
    # buffer sets rotate as for the headline step, so that operands come from HBM
    sets = max(1, args.sets)
    X = [torch.from_numpy(q["x"]).to(dev)] + [None] * (sets - 1)
    for i in range(1, sets):
        X[i] = X[0].clone()
    Wq = [Wq0] + [Wq0.clone() for _ in range(1, sets)]
    qs = [spin.spin_fwht_quant(x, 1) for x in X]
    Xq, xs = [t[0] for t in qs], [t[1] for t in qs]
    Y = [torch.empty((4096, 6144), dtype=torch.float32, device=dev) for _ in range(sets)]
    for i in range(args.warmup):
        spin.spin_w4a4_gemm(Xq[i % sets], xs[i % sets], Wq[i % sets], ws, Y=Y[i % sets])
    t_q = _time(lambda i: spin.spin_fwht_quant(X[i % sets], 1, Xq=Xq[i % sets], x_scale=xs[i % sets]), reps, stream)
    t_g = _time(lambda i: spin.spin_w4a4_gemm(Xq[i % sets], xs[i % sets], Wq[i % sets], ws, Y=Y[i % sets]), reps,
                stream)
    # the same GEMM with both operands in the FP6 operand layout: the weights
    # packed once (offline, untimed), the activation codes rewritten by
    # spin_codes_f6 after the quantizer (timed)
    f6w = [spin.spin_codes_f6(w) for w in Wq]
    f6x = [spin.spin_codes_f6(x) for x in Xq]
    for i in range(args.warmup):
        j = i % sets
        spin.spin_fwht_quant_f6(X[j], Xf6=f6x[j][0], x_sum=f6x[j][1], x_scale=xs[j], had_n=1)
        spin.spin_w4a4_gemm_f6f6(f6x[j][0], f6x[j][1], xs[j], f6w[j][0], f6w[j][1], ws, 4096, Y=Y[j])
    t_c = _time(lambda i: spin.spin_codes_f6(Xq[i % sets], f6x[i % sets][0], f6x[i % sets][1]), reps, stream)
    t_q6 = _time(lambda i: spin.spin_fwht_quant_f6(X[i % sets], Xf6=f6x[i % sets][0], x_sum=f6x[i % sets][1],
                                                   x_scale=xs[i % sets], had_n=1), reps, stream)
    t_g6 = _time(lambda i: spin.spin_w4a4_gemm_f6f6(f6x[i % sets][0], f6x[i % sets][1], xs[i % sets],
                                                    f6w[i % sets][0], f6w[i % sets][1], ws, 4096, Y=Y[i % sets]),
                 reps, stream)
    ops = 2.0 * 4096 * 6144 * 4096
    out["qkv_proj"] = {"workload": "X 4096x4096 fp16 quant-only, W 4096x6144 (R1 4096 folded), M=4096",
                       "quant_us": t_q * 1e3, "gemm_us": t_g * 1e3,
                       "gemm_tops": ops / (t_g * 1e-3) / 1e12,
                       "gemm_frac_of_int8_peak": ops / (t_g * 1e-3) / 1e12 / INT8_PEAK_TOPS,
                       "codes_f6_us": t_c * 1e3, "quant_f6_us": t_q6 * 1e3, "gemm_f6f6_us": t_g6 * 1e3,
                       "step_f6f6_us": (t_q6 + t_g6) * 1e3,
                       "gemm_f6f6_tops": ops / (t_g6 * 1e-3) / 1e12,
                       "gemm_f6f6_frac_of_int8_peak": ops / (t_g6 * 1e-3) / 1e12 / INT8_PEAK_TOPS}
    del X, Xq, xs, Y, Wq, ws, f6w, f6x

    # decoder-layer chain: qkv, o_proj (R2 128), gate/up (2 x 12288), down (H_12288)
    c = synth.chain_config(M=8192)
    layers = []
    for name in ("qkv", "o", "gate_up", "down"):
        L = c[name]
        K, N = L["w"].shape
        R = None if L["r"] is None else torch.from_numpy(L["r"]).to(dev)
        if name == "o":
            out["rotation_inputs_orthogonality"]["R2 Haar 128 (o_proj)"] = checks.orthogonality_error(R)
        _, Wq, ws = spin.spin_fold_rotation(torch.from_numpy(L["w"]).to(dev), R, L["r_block"])
        layers.append({"name": name, "x": torch.from_numpy(L["x"]).to(dev), "K": K, "N": N,
                       "had_n": L["had_n"], "wq": [Wq], "ws": [ws]})
    torch.cuda.synchronize()

    def chain(M, copy):
        for L in layers:
            xq, sc, _ = spin.spin_fwht_quant(L["x"][:M], L["had_n"], Xq=L["xq"][:M], x_scale=L["sc"][:M])
            spin.spin_w4a4_gemm(xq, sc, L["wq"][copy], L["ws"][copy], Y=L["y"][:M])

    for L in layers:
        L["xq"] = torch.empty((8192, L["K"] // 2), dtype=torch.uint8, device=dev)
        L["sc"] = torch.empty((8192,), dtype=torch.float32, device=dev)
        L["y"] = torch.empty((8192, L["N"]), dtype=torch.float32, device=dev)
    ops = 2.0 * 8192 * sum(L["K"] * L["N"] for L in layers)
    for _ in range(2):
        chain(8192, 0)
    t8 = _time(lambda i: chain(8192, 0), max(3, reps // 3), stream)
    out["chain_m8192"] = {"workload": "qkv + o_proj + gate/up + down (activation quant incl. R4 FWHT), M=8192",
                          "us": t8 * 1e3, "tops": ops / (t8 * 1e-3) / 1e12,
                          "frac_of_int8_peak": ops / (t8 * 1e-3) / 1e12 / INT8_PEAK_TOPS}

    # the same chain with both GEMM operands in the FP6 operand layout: the
    # weights packed once by spin_codes_f6 (offline, untimed); every input
    # quantized by spin_fwht_quant_f6 straight into the layout (had_n 12288
    # for down_proj, 1 for the others), timed
    for L in layers:
        L["wf6"] = spin.spin_codes_f6(L["wq"][0])
        L["xf6"] = torch.empty((spin.f6_bytes(8192, L["K"]),), dtype=torch.uint8, device=dev)
        L["xsum"] = torch.empty((8192,), dtype=torch.int32, device=dev)

    def chain6():
        for L in layers:
            spin.spin_fwht_quant_f6(L["x"], Xf6=L["xf6"], x_sum=L["xsum"], x_scale=L["sc"], had_n=L["had_n"])
            spin.spin_w4a4_gemm_f6f6(L["xf6"], L["xsum"], L["sc"], L["wf6"][0], L["wf6"][1], L["ws"][0], L["K"],
                                     Y=L["y"])

    for _ in range(2):
        chain6()
    t86 = _time(lambda i: chain6(), max(3, reps // 3), stream)
    out["chain_m8192_f6f6"] = {"workload": "the same chain at M=8192 with both GEMM operands in the FP6 operand "
                                           "layout (weights packed offline; activation codes written by "
                                           "spin_fwht_quant_f6, timed)",
                               "us": t86 * 1e3, "tops": ops / (t86 * 1e-3) / 1e12,
                               "frac_of_int8_peak": ops / (t86 * 1e-3) / 1e12 / INT8_PEAK_TOPS}
    for L in layers:
        del L["wf6"], L["xf6"], L["xsum"]

    # decode, M = 16: weight bytes dominate; four weight copies rotate so they come from HBM
    for L in layers:
        for _ in range(3):
            L["wq"].append(L["wq"][0].clone())
            L["ws"].append(L["ws"][0].clone())
    wbytes = sum(L["N"] * (L["K"] // 2 + 4) for L in layers)
    for i in range(4):
        chain(16, i)
    t16 = _time(lambda i: chain(16, i % 4), 4 * max(3, reps // 3), stream)
    out["chain_m16"] = {"workload": "same chain at M=16 (first 16 tokens), weights cold in HBM",
                        "us": t16 * 1e3, "weight_GBps": wbytes / (t16 * 1e-3) / 1e9,
                        "frac_of_hbm": wbytes / (t16 * 1e-3) / 1e9 / HBM_PEAK_GBPS}

    # the same decode chain captured once per weight copy in a HIP graph and
    # replayed: the eight launches no longer wait on the host
    graphs = []
    cap = torch.cuda.Stream()
    for i in range(4):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            chain(16, i)
        graphs.append(g)
    for i in range(4):
        graphs[i].replay()
    t16g = _time(lambda i: graphs[i % 4].replay(), 4 * max(3, reps // 3), stream)
    out["chain_m16_graph"] = {"workload": "chain at M=16 as one HIP graph replay per token batch, weights cold",
                              "us": t16g * 1e3, "weight_GBps": wbytes / (t16g * 1e-3) / 1e9,
                              "frac_of_hbm": wbytes / (t16g * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    return out


def w4a8_workloads(args, dev, stream):
    """The W4A8KV8 variant on the same shapes: fwht_quant8 + w4a8_gemm on the
    down_proj workload (INT8 codes, 1 byte per element out) and kv_quant8 on K."""
    import torch
    from rotation_bit_quantization_amd import spin, synth
    cfg = synth.down_config()
    sets = max(1, args.sets)
    X = [torch.from_numpy(cfg["x"]).to(dev)]
    X += [X[0].clone() for _ in range(1, sets)]
    _, Wq, ws = spin.spin_fold_rotation(torch.from_numpy(cfg["w"]).to(dev), None, HAD_N)
    q = [spin.spin_fwht_quant8(x, HAD_N) for x in X]
    Y = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(sets)]
    reps = max(10, args.steps)
    for i in range(args.warmup):
        spin.spin_w4a8_gemm(q[i % sets][0], q[i % sets][1], Wq, ws, Y=Y[i % sets])
    t_f = _time(lambda i: spin.spin_fwht_quant8(X[i % sets], HAD_N, Xq8=q[i % sets][0], x_scale=q[i % sets][1]),
                reps, stream)
    t_g = _time(lambda i: spin.spin_w4a8_gemm(q[i % sets][0], q[i % sets][1], Wq, ws, Y=Y[i % sets]), reps, stream)
    fbytes = M * (2 * K + K + 4)
    out = {"workload": "fwht_quant8 X 4096x12288 fp16 (H12 x H1024, INT8 codes) + w4a8_gemm M=N=4096 K=12288",
           "fwht_quant8_us": t_f * 1e3, "fwht_quant8_GBps": fbytes / (t_f * 1e-3) / 1e9,
           "fwht_quant8_frac_of_hbm": fbytes / (t_f * 1e-3) / 1e9 / HBM_PEAK_GBPS,
           "gemm_us": t_g * 1e3, "gemm_tops": 2.0 * M * N * K / (t_g * 1e-3) / 1e12,
           "gemm_frac_of_int8_peak": 2.0 * M * N * K / (t_g * 1e-3) / 1e12 / INT8_PEAK_TOPS}
    del X, q, Y
    kv = synth.kv_config()
    Kd = [torch.from_numpy(kv["k"]).to(dev)] + [None] * (sets - 1)
    for i in range(1, sets):
        Kd[i] = Kd[0].clone()
    codes = [torch.empty((KV_T, KV_H, KV_D), dtype=torch.int8, device=dev) for _ in range(sets)]
    sc = [torch.empty((KV_T, KV_H), dtype=torch.float16, device=dev) for _ in range(sets)]
    for i in range(args.warmup):
        spin.spin_kv_quant8(Kd[i % sets], 1, codes=codes[i % sets], scale=sc[i % sets])
    t_k = _time(lambda i: spin.spin_kv_quant8(Kd[i % sets], 1, codes=codes[i % sets], scale=sc[i % sets]), reps,
                stream)
    kbytes = KV_T * KV_H * (2 * KV_D + KV_D + 2)
    out["kv_quant8_us"] = t_k * 1e3
    out["kv_quant8_GBps"] = kbytes / (t_k * 1e-3) / 1e9
    return out


def probe_workload(args):
    """Rotation-choice probe on one synthetic layer (2048 tokens, 1024 -> 1024,
    8 outlier channels x100): W4A4 error under 32 randomised Hadamards and 32
    Haar rotations, each a fold of the activations and of the weights plus one
    GEMM on the device; with the CPU leg, one rotation through the oracle."""
    import oracle
    from rotation_bit_quantization_amd import probe, synth
    cfg = synth.probe_config()
    res = probe.rotation_probe(cfg)
    res.pop("errors")
    res["workload"] = "one layer, 2048 tokens x 1024 -> 1024, 32 randomised Hadamards vs 32 Haar"
    if not args.no_cpu_baseline:
        x, w, r = cfg["x"], cfg["w"], cfg["haar"][0]
        t0 = time.perf_counter()
        _, xq, xs = oracle.fold_rotation(np.ascontiguousarray(x.T), r, x.shape[1])
        _, wq, ws = oracle.fold_rotation(w, r, x.shape[1])
        oracle.w4a4_gemm(xq, xs, wq, ws)
        res["oracle_seconds_per_rotation"] = time.perf_counter() - t0
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(fwht_quant and kv_quant shard by tokens with no communication; the GEMM shards by output "
              f"columns, or by K with an exact int32 all-reduce before the epilogue)", file=sys.stderr)
        sys.exit(2)

    import torch
    import oracle
    from rotation_bit_quantization_amd import spin, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    spin.load()

    cfg = synth.down_config()
    x_host, w_host = cfg["x"], cfg["w"]

    # Offline fold (untimed): W' = (H_12288 / sqrt(12288))^T W, per-channel INT4.
    _, Wq, ws = spin.spin_fold_rotation(torch.from_numpy(w_host).to(dev), None, HAD_N)

    sets = max(1, args.sets)
    X = [torch.from_numpy(x_host).to(dev)]
    for i in range(1, sets):                 # same values, distinct HBM buffers
        X.append(X[0].clone())
    Xq = [torch.empty((M, K // 2), dtype=torch.uint8, device=dev) for _ in range(sets)]
    xs = [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(sets)]
    Y = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(sets)]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    from rotation_bit_quantization_amd.timing import hip_events
    he = hip_events()

    def step(i, ev=None):
        j = i % sets
        if ev is not None:
            he.record(ev[0], stream)
        spin.spin_fwht_quant(X[j], HAD_N, Xq=Xq[j], x_scale=xs[j])
        if ev is not None:
            he.record(ev[1], stream)
        spin.spin_w4a4_gemm(Xq[j], xs[j], Wq, ws, Y=Y[j])
        if ev is not None:
            he.record(ev[2], stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    events = [[he.new() for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    f_ms = np.array([he.ms(e[0], e[1]) for e in events])
    g_ms = np.array([he.ms(e[1], e[2]) for e in events])
    he.release()

    # Warm figures, after and outside the timed region: every step reuses buffer
    # set 0, so its activations (100 MB) come back from the Infinity Cache.
    warm_ev = [[he.new() for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(0, warm_ev[i])
    torch.cuda.synchronize()
    warm = {"fwht_quant_us": float(np.median([he.ms(e[0], e[1]) for e in warm_ev])) * 1e3,
            "gemm_us": float(np.median([he.ms(e[1], e[2]) for e in warm_ev])) * 1e3,
            "note": "medians over the same number of steps with one buffer set (activations warm in the "
                    "Infinity Cache); not the metric"}
    he.release()
    f_s, g_s = f_ms.mean() / 1e3, g_ms.mean() / 1e3
    fwht_bytes = M * FWHT_BYTES_PER_TOKEN
    fwht_gbps = fwht_bytes / f_s / 1e9
    gemm_ops = 2.0 * M * N * K
    gemm_tops = gemm_ops / g_s / 1e12

    # Parity spot check of this run's output (first row of the last set) against the oracle.
    j = (args.steps - 1) % sets
    xq_row = Xq[j][:2].cpu().numpy()
    pk, _, _ = oracle.fwht_quant(x_host[:2], HAD_N)
    mism = float(np.mean(oracle.unpack_int4(xq_row) != oracle.unpack_int4(pk)))

    extra = {}
    if not args.no_f6:
        # The same step with the activation codes in the FP6 operand layout
        # (spin_fwht_quant_f6 + spin_w4a4_gemm_f6), same buffers rotating.
        Xf6 = [torch.empty((spin.f6_bytes(M, K),), dtype=torch.uint8, device=dev) for _ in range(sets)]
        xsum = [torch.empty((M,), dtype=torch.int32, device=dev) for _ in range(sets)]

        def step6(i, ev=None):
            j = i % sets
            if ev is not None:
                he.record(ev[0], stream)
            spin.spin_fwht_quant_f6(X[j], Xf6=Xf6[j], x_sum=xsum[j], x_scale=xs[j])
            if ev is not None:
                he.record(ev[1], stream)
            spin.spin_w4a4_gemm_f6(Xf6[j], xsum[j], xs[j], Wq, ws, Y=Y[j])
            if ev is not None:
                he.record(ev[2], stream)

        for i in range(args.warmup):
            step6(i)
        torch.cuda.synchronize()
        ev6 = [[he.new() for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            step6(i, ev6[i])
        torch.cuda.synchronize()
        f6_us = float(np.mean([he.ms(e[0], e[1]) for e in ev6])) * 1e3
        g6_us = float(np.mean([he.ms(e[1], e[2]) for e in ev6])) * 1e3
        he.release()
        extra["down_proj_f6"] = {
            "workload": "the down_proj step with the activation codes in the FP6 operand layout: "
                        "spin_fwht_quant_f6 (4096 x 12288 fp16, H_12288) + spin_w4a4_gemm_f6 (4096 x 4096 x 12288)",
            "fwht_quant_f6_us": f6_us, "gemm_f6_us": g6_us, "gemm_f6_tops": gemm_ops / g6_us / 1e6,
            "step_us": f6_us + g6_us}

        # ... and with the weights too in the FP6 operand layout, packed once
        # (spin_codes_f6, offline, untimed): spin_w4a4_gemm_f6f6
        Wf6, wsum = spin.spin_codes_f6(Wq)

        def step66(i, ev=None):
            j = i % sets
            if ev is not None:
                he.record(ev[0], stream)
            spin.spin_fwht_quant_f6(X[j], Xf6=Xf6[j], x_sum=xsum[j], x_scale=xs[j])
            if ev is not None:
                he.record(ev[1], stream)
            spin.spin_w4a4_gemm_f6f6(Xf6[j], xsum[j], xs[j], Wf6, wsum, ws, K, Y=Y[j])
            if ev is not None:
                he.record(ev[2], stream)

        for i in range(args.warmup):
            step66(i)
        torch.cuda.synchronize()
        ev66 = [[he.new() for _ in range(3)] for _ in range(args.steps)]
        for i in range(args.steps):
            step66(i, ev66[i])
        torch.cuda.synchronize()
        f66_us = float(np.mean([he.ms(e[0], e[1]) for e in ev66])) * 1e3
        g66 = [he.ms(e[1], e[2]) * 1e3 for e in ev66]
        g66_us = float(np.mean(g66))
        he.release()
        g66_tops = gemm_ops / g66_us / 1e6
        extra["down_proj_f6f6"] = {
            "workload": "the down_proj step with both operands in the FP6 operand layout: spin_fwht_quant_f6 "
                        "(4096 x 12288 fp16, H_12288) + spin_w4a4_gemm_f6f6 (4096 x 4096 x 12288), the weights "
                        "packed once by spin_codes_f6 (offline, untimed)",
            "fwht_quant_f6_us": f66_us, "gemm_f6f6_us": g66_us, "gemm_f6f6_median_us": float(np.median(g66)),
            "step_us": f66_us + g66_us,
            "roofline_gemm_f6f6": {"kernel": "w4a4_gemm_fp6_f6ab", "bound": "mfma", "achieved": g66_tops,
                                   "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": g66_tops / INT8_PEAK_TOPS,
                                   "traffic": traffic("w4a4_gemm_f6f6")}}
        del Xf6, xsum, Wf6, wsum

    if not args.no_fused:
        # The same step as one launch (spin_fwht_quant_gemm) against the two calls,
        # both timed as whole steps on the rotating buffer sets.
        def two(i):
            j = i % sets
            spin.spin_fwht_quant(X[j], HAD_N, Xq=Xq[j], x_scale=xs[j])
            spin.spin_w4a4_gemm(Xq[j], xs[j], Wq, ws, Y=Y[j])

        def one(i):
            j = i % sets
            spin.spin_fwht_quant_gemm(X[j], Wq, ws, Xq=Xq[j], x_scale=xs[j], Y=Y[j])

        res = {"workload": "the down_proj step (fwht_quant 4096 x 12288 fp16, H_12288, INT4 + w4a4_gemm "
                           "4096 x 4096 x 12288) as one cooperative launch against the two calls"}
        for name, fn in (("two_calls_us", two), ("one_launch_us", one), ("two_calls_again_us", two)):
            for i in range(args.warmup):
                fn(i)
            res[name] = _time(fn, args.steps, stream) * 1e3
        res["saved_us"] = 0.5 * (res["two_calls_us"] + res["two_calls_again_us"]) - res["one_launch_us"]
        extra["down_proj_fused"] = res

    if not args.no_kv:
        kv = synth.kv_config()
        Kd = [torch.from_numpy(kv["k"]).to(dev)] + [None] * (sets - 1)
        for i in range(1, sets):
            Kd[i] = Kd[0].clone()
        kc = [torch.empty((KV_T, KV_H, KV_D // 2), dtype=torch.uint8, device=dev) for _ in range(sets)]
        ksc = [torch.empty((KV_T, KV_H), dtype=torch.float16, device=dev) for _ in range(sets)]
        for i in range(args.warmup):
            spin.spin_kv_quant(Kd[i % sets], 1, codes=kc[i % sets], scale=ksc[i % sets])
        k_s = _time(lambda i: spin.spin_kv_quant(Kd[i % sets], 1, codes=kc[i % sets], scale=ksc[i % sets]),
                    args.steps, stream) / 1e3
        kv_bytes = KV_T * KV_H * KV_BYTES_PER_GROUP
        extra["kv_quant"] = {"workload": "K [4096][32][128] fp16, H_128 + INT4, fp16 scale",
                             "us": k_s * 1e6, "GBps": kv_bytes / k_s / 1e9,
                             "frac_of_hbm": kv_bytes / k_s / 1e9 / HBM_PEAK_GBPS,
                             "traffic": traffic("kv_quant")}
        extra["kv_qkv"] = kv_qkv_workload(args, dev, stream, kv, sets)
        del Kd, kc, ksc

    machine = None
    if not args.no_extra:
        extra.update(extra_workloads(args, dev, stream))
        extra["vendor_int8_gemm"] = vendor_int8_workload(args, dev, stream)
        extra["tiny"] = tiny_workload(args, dev, stream)
        machine = machine_ceilings(M * FWHT_BYTES_PER_TOKEN / f_s / 1e12, gemm_tops)

    if not args.no_extra:
        extra["w4a8kv8"] = w4a8_workloads(args, dev, stream)
        extra["rotation_probe"] = probe_workload(args)
        from rotation_bit_quantization_amd import cayley
        r2 = cayley.r2_experiment()
        r2.pop("R2")
        r2["workload"] = "R2 (128 x 128, 32 heads) learned by Cayley SGD on a 512-token o_proj slice, 120 iterations"
        extra["r2_cayley"] = r2

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = 1 << 30

    line = {
        "metric": "fwht_quant GB/s (% of 8 TB/s) + W4A4 GEMM TOPS (% INT8 MFMA peak), M=4096",
        "value": round(fwht_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # what the path computes in: the Hadamard's 32-point stages on fp16
        # matrix cores (fp16 row, fp32 intermediate as an fp16 hi + lo pair,
        # fp32 accumulation), the rest of the transform and the quantizer in
        # fp32; the GEMM on INT4 codes carried exactly as FP6 E2M3 operands
        # (fp32 accumulation of integer products), epilogue in fp32
        "dtype": "fwht: f16 MFMA (hi+lo) + f32; gemm: int4 codes as FP6-E2M3 MFMA, exact f32 acc",
        "data": "synthetic (seeded N(0,1) activations, 0.1% channels x100; N(0,0.02) weights)",
        "config": {"workload": "R4 down_proj path: fwht_quant X 4096x12288 fp16, had_n 12288 "
                               "(H12 x H1024), per-token INT4; w4a4_gemm M=4096 N=4096 K=12288",
                   "M": M, "K": K, "N": N, "had_n": HAD_N, "buffer_sets": sets},
        "fwht_quant_us": round(f_s * 1e6, 3),
        "fwht_quant_frac_of_hbm": round(fwht_gbps / HBM_PEAK_GBPS, 4),
        "gemm_us": round(g_s * 1e6, 3),
        "gemm_tops": round(gemm_tops, 2),
        "gemm_frac_of_int8_peak": round(gemm_tops / INT8_PEAK_TOPS, 4),
        "roofline": {"kernel": "w4a4_gemm", "bound": "mfma", "achieved": round(gemm_tops, 2),
                     "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "traffic": traffic("w4a4_gemm"),
                     "issued": {"instruction": "v_mfma_scale_f32_32x32x64_f8f6f4 (FP6 E2M3)",
                                "peak": FP6_PEAK_TOPS, "frac": round(gemm_tops / FP6_PEAK_TOPS, 4)}},
        "roofline_fwht_quant": {"kernel": "fwht_quant", "bound": "hbm", "achieved": round(fwht_gbps, 2),
                                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                "frac": round(fwht_gbps / HBM_PEAK_GBPS, 4),
                                "traffic": traffic("fwht_quant")},
        "roofline_fwht_quant_alu": {"kernel": "fwht_quant", "bound": "alu",
                                    "achieved": round(M * K * FWHT_VALU_OPS_PER_ELEMENT / f_s / 1e12, 2),
                                    "peak": round(VALU_PEAK_TOPS, 2), "unit": "T lane-op/s",
                                    "frac": round(M * K * FWHT_VALU_OPS_PER_ELEMENT / f_s / 1e12 / VALU_PEAK_TOPS, 4)},
        # the same product with both operands in the FP6 operand layout (weights
        # packed offline): extra.down_proj_f6f6, repeated here for visibility
        "roofline_w4a4_gemm_f6f6": (extra.get("down_proj_f6f6") or {}).get("roofline_gemm_f6f6"),
        "launch_us": {name: {"mean": round(float(v.mean()) * 1e3, 3), "median": round(float(np.median(v)) * 1e3, 3),
                             "p10": round(float(np.percentile(v, 10)) * 1e3, 3),
                             "p90": round(float(np.percentile(v, 90)) * 1e3, 3)}
                      for name, v in (("fwht_quant", f_ms), ("w4a4_gemm", g_ms))},
        "warm": {k: (round(v, 3) if isinstance(v, float) else v) for k, v in warm.items()},
        "parity_spot_code_mismatch": mism,
        "machine": machine,
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x_host)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
