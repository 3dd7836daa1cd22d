"""Throughput of the KDA forward hot path on one MI355X.

One step = one kda_fwd_chunked call over the B=4, H=16, T=16384, d=128,
C=64 bf16 prefill workload (inputs resident in HBM).  The same run also
times the batched T=1 decode (B=256, H=16, d=128, 1000 consecutive steps)
and the long-context prefill (B=1, H=16, T=131072), and times the fp64 CPU
oracle on a bounded sample of the prefill workload on the host cores.

Prints one JSON line.  `value` is prefill tokens/s (tokens = batch x
sequence positions, all 16 heads each); the decode state-update HBM GB/s is
in `decode`.  A dense bf16 MFMA loop (libkda_calibrate.so) measures the
attainable matrix-core rate next to the nominal peak.

    python bench.py [--steps K] [--warmup W] [--decode-steps N] [--no-cpu] [--no-long]
    python bench.py --profile-pass     # short fixed run for rocprofv3 counters
    python bench.py --summarize DIR... # rocprofv3 counter CSVs -> profile summary text
    python bench.py --summarize-trace CSV  # kernel trace of a default run -> per-kernel table
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (H=16,d=128) + decode state-update HBM GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
PREFILL = "prefill_b4_h16_t16k"
SMALL = "prefill_h8_t4k"
LONG = "prefill_h16_t128k"
DECODE = "decode_b256_h16"


def prefill_alg_bytes(B, T, H, dk, dv, elem=2, gate_per_channel=True) -> int:
    """Algorithmic HBM bytes of one prefill call: read q, k, alpha, v, beta,
    write o (elem bytes each), read S0 and write S_T (fp32).  A per-head gate
    is one element per token-head instead of d_k."""
    ga = dk if gate_per_channel else 1
    per_tok_head = (2 * dk + ga + dv) * elem + elem + dv * elem
    return B * T * H * per_tok_head + 2 * B * H * dk * dv * 4


def prefill_alg_flops(B, T, H, dk, dv, C) -> int:
    """Algorithmic flops of the chunked method per call (2 per MAC).  Per
    chunk: the strictly lower key-key Gram C(C-1)/2*dk, the lower query-key
    Gram C(C+1)/2*dk, the triangular solve C(C-1)/2*(dk+dv), the two state
    products 2*C*dk*dv and the output C*dk*dv + C(C+1)/2*dv.  Per token-head
    that is 3*dk*dv + dk*(C + (C-1)/2) + dv*C MACs (69 568 at d=128, C=64)."""
    macs_per_tok_head = 3 * dk * dv + dk * C + (dk * (C - 1)) // 2 + dv * C
    return 2 * macs_per_tok_head * B * T * H


def decode_alg_bytes(B, H, dk, dv, elem=2) -> int:
    """One decode step: read and write the fp32 state, read q, k, alpha, v,
    beta, write o."""
    return 2 * B * H * dk * dv * 4 + B * H * ((3 * dk + dv) * elem + elem + dv * elem)


def _src_hash(name: str) -> str:
    p = os.path.join(ROOT, "gated_delta_rule_76_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def _recorded(kernel_file: str, summary: str, key: str = "hbm_bytes_per_launch"):
    """A figure from a committed rocprofv3 counter summary (HBM bytes per
    launch by default), or None when the summary is absent or the kernel
    source changed since it was taken."""
    p = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(p):
        return None
    vals = {}
    for line in open(p):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != _src_hash(kernel_file):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def _recorded_traffic(kernel_file: str, summary: str):
    return _recorded(kernel_file, summary, "hbm_bytes_per_launch")


def _upload(x, names, dtype):
    import torch
    out = {}
    for n in names:
        t = torch.from_numpy(x[n])
        out[n] = (t.to(torch.bfloat16) if dtype == "bf16" else t).cuda()
    return out


def _time_launches(fn, steps: int, warmup: int):
    """Warm up, then time `steps` back-to-back launches on torch's current
    stream (the stream the library launches on) with HIP events at the two
    ends of the timed region, bracketed by device synchronisation.  Returns
    (total seconds, average launch duration in ms = total / steps).  No events
    sit between the launches: on an 80 us decode step they would add several
    percent of measurement to the work."""
    import torch
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(steps):
        fn()
    t_end.record(stream)
    torch.cuda.synchronize()
    total = t_start.elapsed_time(t_end) / 1e3
    return total, total * 1e3 / steps


def bench_prefill(name: str, steps: int, warmup: int, gate: str = "channel", x=None):
    """Time kda_fwd_chunked on a workload; `x` are its host inputs when
    already drawn (they are left untouched)."""
    import torch
    import gated_delta_rule_76_amd as kda
    from synth import WORKLOADS, workload_inputs

    w = WORKLOADS[name]
    if x is None:
        x = workload_inputs(w)
    if gate == "head":  # one decay per (token, head): the first channel of the drawn gate
        x = dict(x, alpha=np.ascontiguousarray(x["alpha"][..., 0]))
    d = _upload(x, ("q", "k", "v", "alpha", "beta"), w.dtype)
    s0 = torch.from_numpy(x["S0"]).cuda()
    x = None
    o = torch.empty((w.B, w.T, w.H, w.d_v), dtype=d["q"].dtype, device="cuda")
    st = torch.empty((w.B, w.H, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    code = kda.KDA_BF16 if w.dtype == "bf16" else kda.KDA_F32
    ws = torch.empty(kda.workspace_bytes(w.B, w.T, w.H, w.d_k, w.d_v, w.chunk, code),
                     dtype=torch.uint8, device="cuda")

    def fn():
        kda.kda_fwd_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], s0, chunk=w.chunk,
                            o=o, S_T=st, workspace=ws, gate=gate)

    total, per = _time_launches(fn, steps, warmup)
    ok = bool(torch.isfinite(o.float()).all().item() and torch.isfinite(st).all().item())
    del d, o, st, s0, ws
    torch.cuda.empty_cache()
    return w, total, per, ok


def bench_decode(steps: int, warmup: int):
    """warmup + steps consecutive decode steps, each with its own inputs (drawn
    on the host in blocks and uploaded once before timing), on the carried
    fp32 state."""
    import torch
    import gated_delta_rule_76_amd as kda
    from synth import WORKLOADS, decode_state, decode_steps

    w = WORKLOADS[DECODE]
    n = warmup + steps
    S = torch.from_numpy(decode_state(w.B, w.H, w.d_k, w.d_v, s0_std=w.s0_std, seed=w.seed)).cuda()
    names = ("q", "k", "v", "alpha", "beta")
    dims = {"q": (w.d_k,), "k": (w.d_k,), "v": (w.d_v,), "alpha": (w.d_k,), "beta": ()}
    d = {nm: torch.empty((n, w.B, w.H) + dims[nm], dtype=torch.bfloat16, device="cuda")
         for nm in names}
    blk = 100
    first_block = None
    for first in range(0, n, blk):
        cnt = min(blk, n - first)
        p = decode_steps(w.B, w.H, w.d_k, w.d_v, first, cnt, dtype=w.dtype, gate_c=w.gate_c,
                         seed=w.seed)
        for nm in names:
            d[nm][first:first + cnt].copy_(torch.from_numpy(p[nm]).to(torch.bfloat16))
        if first_block is None:
            first_block = p
        del p
    o = torch.empty((w.B, w.H, w.d_v), dtype=torch.bfloat16, device="cuda")
    # Pointers are resolved once so the timed loop is the C entry point alone.
    ptrs = [tuple(d[nm][i].data_ptr() for nm in names) for i in range(n)]
    sp, op = S.data_ptr(), o.data_ptr()
    stream = torch.cuda.current_stream().cuda_stream
    call = kda.lib().kda_decode_step
    step = [0]

    def fn():
        i = step[0]
        step[0] += 1
        st = call(*ptrs[i], sp, op, w.B, w.H, w.d_k, w.d_v, kda.KDA_BF16, stream)
        if st != 0:
            raise kda.KdaError(st, "kda_decode_step")

    total, per = _time_launches(fn, steps, warmup)
    ok = bool(torch.isfinite(S).all().item())
    del d, S, o
    torch.cuda.empty_cache()
    return w, total, per, ok, first_block


ATTNRES = dict(L=64, N=4096, d_k=128, d=4096)  # earlier layers, tokens, key and model width


def attnres_alg_bytes(L, N, dk, d, elem=2) -> int:
    """Read h (L*N*d), k (L*N*d_k), q (N*d_k); write out (N*d)."""
    return (L * N * d + L * N * dk + N * dk + N * d) * elem


def bench_attnres(steps: int, warmup: int):
    """AttnRes depth aggregation on seeded synthetic bf16 tensors generated on
    the GPU (torch's generator, seed 0): q, k scaled so q.k has unit variance."""
    import torch
    import gated_delta_rule_76_amd as kda
    c = ATTNRES
    g = torch.Generator(device="cuda").manual_seed(0)
    s = c["d_k"] ** -0.25
    q = (s * torch.randn(c["N"], c["d_k"], generator=g, device="cuda")).to(torch.bfloat16)
    k = (s * torch.randn(c["L"], c["N"], c["d_k"], generator=g, device="cuda")).to(torch.bfloat16)
    h = torch.randn(c["L"], c["N"], c["d"], generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty(c["N"], c["d"], dtype=torch.bfloat16, device="cuda")
    total, per = _time_launches(lambda: kda.attnres_forward(q, k, h, out=out), steps, warmup)
    ok = bool(torch.isfinite(out.float()).all().item())
    del q, k, h, out
    torch.cuda.empty_cache()
    return total, per, ok


def _calibration_lib():
    path = os.path.join(ROOT, "gated_delta_rule_76_amd", "libkda_calibrate.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m gated_delta_rule_76_amd.build`")
    L = ctypes.CDLL(path)
    L.kda_calibrate_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p]
    L.kda_calibrate_mfma.restype = ctypes.c_int
    L.kda_calibrate_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.kda_calibrate_flops.restype = ctypes.c_double
    L.kda_calibrate_threads_per_block.restype = ctypes.c_int
    L.kda_calibrate_lds.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
    L.kda_calibrate_lds.restype = ctypes.c_int
    return L


# LDS bank probe (kda_calibrate_lds): access forms, in the library's order.
_LDS_FORMS = ["ds_read_b32", "ds_read_b64", "ds_read_b128", "ds_read2_b64", "ds_read2_b32",
              "ds_write_b32", "ds_write_b64", "ds_write_b128", "ds_write2_b32"]
_LDS_BASES = {2: (0, 4, 32, 36)}  # base lanes probed for each form (default: lane 0)
_LDS_BLOCKS, _LDS_ITERS = 16, 256


def _prep_store_offset(l: int, upper_first: bool) -> int:
    """Byte offset of the first 8-byte tile store of lane l in the prep's
    operand-order tile (d_k = 128: 288-byte rows, lane groups of 16 one row
    each, row groups 4 rows apart): chunk 4s + (j & 3) of the row, half j >> 2,
    for the thread's 4-channel unit u = 8s + j."""
    r, cg = 4 * (l >> 4), l & 15
    u = 2 * cg + (1 if upper_first and cg >= 8 else 0)
    s, j = u >> 3, u & 7
    return r * 288 + 2 * (8 * (4 * s + (j & 3)) + 4 * (j >> 2))


def _lds_cases():
    """The LDS probe list: (key, form, 64 byte offsets, -1 = inactive lane).
    For each access form: a base lane j0 at byte 0 against every other lane k
    at byte 256 (the same banks at 32 or 64 banks; a conflict means the LDS
    serves the two lanes together), then lanes 0 and 1 at 128 bytes apart (a
    conflict means the form spreads over 32 banks, none 64).  Then whole-wave
    patterns of the prep's operand tiles."""
    cases = []
    for f in range(len(_LDS_FORMS)):
        for j0 in _LDS_BASES.get(f, (0,)):
            for k in range(64):
                if k != j0:
                    off = [-1] * 64
                    off[j0], off[k] = 0, 256
                    cases.append((("pair", f, j0, k), f, off))
        off = [-1] * 64
        off[0], off[1] = 0, 128
        cases.append((("span", f), f, off))
    pats = [
        ("prep pair read, row-major tile, 272-byte rows (former layout)", 3,
         [(l & 15) * 272 + 8 * (l >> 4) for l in range(64)]),
        ("prep operand read, operand-order tile, 288-byte rows", 2,
         [(l & 15) * 288 + 16 * (l >> 4) for l in range(64)]),
        ("prep first tile store, both halves in channel order", 6,
         [_prep_store_offset(l, False) for l in range(64)]),
        ("prep first tile store, upper half first for channels 64-127", 6,
         [_prep_store_offset(l, True) for l in range(64)]),
    ]
    for name, f, off in pats:
        cases.append((("pattern", name), f, off))
    return cases


def run_lds_probes():
    """Launch every LDS probe case once, in the order of _lds_cases()."""
    import torch
    L = _calibration_lib()
    sink = torch.empty(_LDS_BLOCKS * 64, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    cases = _lds_cases()
    for _, f, off in cases:
        arr = (ctypes.c_int * 64)(*off)
        rc = L.kda_calibrate_lds(f, arr, _LDS_BLOCKS, _LDS_ITERS, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"kda_calibrate_lds failed ({rc})")
    torch.cuda.synchronize()
    del sink
    return len(cases)


def bench_mfma_calibration(launches: int = 5, iters: int = 4000):
    """Attainable dense bf16 MFMA rate: the calibration loop (eight
    workgroups of four waves per CU, independent accumulators) for 16x16x32
    and 32x32x16 instructions; the best of `launches` timed launches each."""
    import torch
    L = _calibration_lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 8 * cus
    sink = torch.empty(blocks * L.kda_calibrate_threads_per_block(), dtype=torch.float32,
                       device="cuda")
    stream = torch.cuda.current_stream()
    out = {}
    for kind, name in ((0, "16x16x32"), (1, "32x32x16")):
        def fn():
            rc = L.kda_calibrate_mfma(kind, blocks, iters, sink.data_ptr(), stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"kda_calibrate_mfma failed ({rc})")
        best = float("inf")
        for _ in range(2):
            fn()
        for _ in range(launches):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / 1e3)
        out[name] = L.kda_calibrate_flops(kind, blocks, iters) / best / 1e12
    del sink
    return {"measured_peak_tflops": round(max(out.values()), 1),
            "by_instruction_tflops": {k: round(v, 1) for k, v in out.items()},
            "kernel": "dense bf16 MFMA loop, 8 independent accumulators per wave, 8 waves per SIMD"}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _host_threads() -> int:
    """Host threads the oracle may use: the OpenMP setting of the environment
    (the share of the host that goes with one GPU) when there is one, else
    all cores."""
    n = os.cpu_count() or 1
    try:
        return max(1, min(n, int(os.environ.get("OMP_NUM_THREADS", n))))
    except ValueError:
        return n


def cpu_baseline(x2, x3, decode_block, decode_sample_steps: int = 32):
    """Time the fp64 oracle (the reported CPU baseline, not a target) on the
    host: the headline prefill's inputs on all its (batch, head) chains with
    N threads and on one chain with one thread; the long-context prefill's
    first tokens on all its chains; the first decode steps on all heads."""
    import oracle
    from synth import WORKLOADS

    N = _host_threads()
    w = WORKLOADS[PREFILL]
    arr = lambda x, sl: {n: x[n][sl] for n in ("q", "k", "v", "alpha", "beta")}
    nt = min(N, w.B * w.H)
    t0 = time.perf_counter()
    oracle.kda_forward(x2["q"], x2["k"], x2["v"], x2["alpha"], x2["beta"], x2["S0"], threads=nt)
    dt = time.perf_counter() - t0
    one = arr(x2, (slice(0, 1), slice(None), slice(0, 1)))
    t1 = time.perf_counter()
    oracle.kda_forward(one["q"], one["k"], one["v"], one["alpha"], one["beta"], x2["S0"][:1, :1],
                       threads=1)
    dt1 = time.perf_counter() - t1
    out = {"value": round(w.B * w.T / dt, 1), "unit": "tokens/s", "cores": nt, "kind": "oracle",
           "sample": f"{PREFILL}: the whole workload (all {w.B * w.H} (batch, head) chains, "
                     f"{w.T} tokens), fp64 token recurrence, {dt:.2f} s wall on {nt} threads",
           "cpu_model": _cpu_model(), "host_threads_available": N,
           "single_thread": {"value": round(w.T / dt1, 1), "unit": "tokens/s per (batch, head) chain",
                             "token_heads_per_s": round(w.T / dt1, 1),
                             "sample": f"{PREFILL}: one chain, all {w.T} tokens, 1 thread, "
                                       f"{dt1:.2f} s"}}
    if x3 is not None:
        wl = WORKLOADS[LONG]
        T3 = x3["q"].shape[1]
        n3 = min(N, wl.B * wl.H)
        t2 = time.perf_counter()
        oracle.kda_forward(x3["q"], x3["k"], x3["v"], x3["alpha"], x3["beta"], x3["S0"], threads=n3)
        dt2 = time.perf_counter() - t2
        out["long_context"] = {"value": round(wl.B * T3 / dt2, 1), "unit": "tokens/s",
                               "cores": n3,
                               "sample": f"{LONG}: all {wl.B * wl.H} chains, first {T3} of {wl.T} "
                                         f"tokens, {dt2:.2f} s on {n3} threads"}
    if decode_block is not None:
        wd = WORKLOADS[DECODE]
        k = decode_sample_steps
        tr = lambda a: np.ascontiguousarray(np.moveaxis(a[:k], 0, 1))  # [steps,B,H,..] -> [B,steps,H,..]
        nd = min(N, wd.B * wd.H)
        from synth import decode_state
        S = decode_state(wd.B, wd.H, wd.d_k, wd.d_v, s0_std=wd.s0_std, seed=wd.seed)
        t3 = time.perf_counter()
        oracle.kda_forward(tr(decode_block["q"]), tr(decode_block["k"]), tr(decode_block["v"]),
                           tr(decode_block["alpha"]), tr(decode_block["beta"]), S, threads=nd)
        dt3 = time.perf_counter() - t3
        out["decode"] = {"value": round(k / dt3, 2), "unit": "steps/s",
                         "token_heads_per_s": round(k * wd.B * wd.H / dt3, 1), "cores": nd,
                         "sample": f"{DECODE}: all {wd.B * wd.H} heads, the first {k} of "
                                   f"{wd.decode_steps} steps, {dt3:.2f} s on {nd} threads"}
    return out


def profile_pass():
    """Fixed short run for rocprofv3 counter passes: a plain 1 GiB copy (the
    traffic calibration), the dense MFMA loops (the MFMA-busy calibration),
    the LDS bank probes, 3 prefill launches, 3 decode launches, 3 AttnRes
    launches."""
    import torch
    n = 1 << 28  # 2^28 fp32 = 1 GiB read + 1 GiB written
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy: {n * 4} bytes read and written per launch", flush=True)
    del src, dst
    torch.cuda.empty_cache()
    cal = bench_mfma_calibration(launches=1, iters=2000)
    print(f"mfma loops: {cal['by_instruction_tflops']}", flush=True)
    print(f"lds probes: {run_lds_probes()} launches", flush=True)
    bench_prefill(PREFILL, 3, 0)
    print("prefill: 3 launches", flush=True)
    bench_decode(3, 0)
    print("decode: 3 launches", flush=True)
    bench_attnres(3, 0)
    print("attnres: 3 launches", flush=True)


# Kernels of a profile pass: (name substring, label).  The pass launches each
# KDA entry point 3 times and each calibration kernel 3 times; one prefill
# call runs several segments, each a prep and a state-pass dispatch.
_PROFILED = [("chunk_prep_kernel", "chunk_prep_kernel"), ("state_pass_kernel", "state_pass_kernel"),
             ("decode_kernel", "decode_kernel"), ("attnres_kernel", "attnres_kernel"),
             ("mfma16_loop", "mfma16_loop"), ("mfma32_loop", "mfma32_loop")]
_CALLS = 3


def summarize(dirs):
    """Read rocprofv3 counter CSVs (*_counter_collection.csv under `dirs`) of
    `bench.py --profile-pass` runs and print, per kernel, counter means per
    dispatch and per call; HBM bytes scaled by what FETCH_SIZE / WRITE_SIZE
    read for the 1 GiB copy; and the MFMA busy rate (SQ_VALU_MFMA_BUSY_CYCLES
    per GRBM_GUI_ACTIVE cycle) relative to the saturated calibration loop."""
    import glob
    tot, n = {}, {}
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            rows = list(csv.DictReader(open(f)))
            # the 1 GiB device-to-device copy runs as the runtime's copy
            # kernel, its largest launch in the pass
            blit = [int(r["Grid_Size"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
            big = max(blit) if blit else -1
            per = {}
            for r in rows:
                name, cnt, v = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
                if "copyBuffer" in name and int(r["Grid_Size"]) == big:
                    label = "copy"
                else:
                    label = next((lb for pat, lb in _PROFILED if pat in name), None)
                    if label is None:
                        continue
                k = (label, cnt, r["Dispatch_Id"])
                per[k] = per.get(k, 0.0) + v
            for (label, cnt, _), v in per.items():
                tot[(label, cnt)] = tot.get((label, cnt), 0.0) + v
                n[(label, cnt)] = n.get((label, cnt), 0) + 1
    mean = {k: tot[k] / n[k] for k in tot}
    fcal = mean.get(("copy", "FETCH_SIZE"), 0) * 1024 / float(1 << 30)
    wcal = mean.get(("copy", "WRITE_SIZE"), 0) * 1024 / float(1 << 30)
    print("# counter means per dispatch (FETCH_SIZE / WRITE_SIZE in KiB as rocprofv3 reports)")
    if fcal and wcal:
        print(f"# calibration on the 1 GiB copy: FETCH_SIZE reads {fcal:.3f} x the bytes read, "
              f"WRITE_SIZE {wcal:.3f} x the bytes written; HBM bytes below are divided by these")
    labels = [lb for _, lb in _PROFILED if any(k[0] == lb for k in mean)]
    for lb in labels:
        cs = sorted(c for (l, c) in mean if l == lb)
        nd = max(n[(lb, c)] for c in cs)
        print(f"# {lb} ({nd} dispatches, {nd / _CALLS:g} per call):")
        for c in cs:
            print(f"#   {c:26s} {mean[(lb, c)]:.6g}")
        if fcal and (lb, "FETCH_SIZE") in mean and (lb, "WRITE_SIZE") in mean:
            rd = tot[(lb, "FETCH_SIZE")] / _CALLS * 1024 / fcal
            wr = tot[(lb, "WRITE_SIZE")] / _CALLS * 1024 / wcal
            print(f"#   -> HBM read {rd / 1e6:.1f} MB, write {wr / 1e6:.1f} MB per call")
        if mean.get((lb, "SQ_ACTIVE_INST_LDS"), 0) > 0 and (lb, "SQ_LDS_BANK_CONFLICT") in mean:
            print(f"#   -> LDS bank-conflict cycles / active LDS instruction cycles "
                  f"{mean[(lb, 'SQ_LDS_BANK_CONFLICT')] / mean[(lb, 'SQ_ACTIVE_INST_LDS')]:.3f}")
    rate = {lb: tot[(lb, "SQ_VALU_MFMA_BUSY_CYCLES")] / tot[(lb, "GRBM_GUI_ACTIVE")]
            for lb in labels if tot.get((lb, "GRBM_GUI_ACTIVE"), 0) > 0
            and (lb, "SQ_VALU_MFMA_BUSY_CYCLES") in tot}
    ref = max((rate[lb] for lb in ("mfma16_loop", "mfma32_loop") if lb in rate), default=0)
    if ref:
        print("# MFMA busy rate relative to the saturated calibration loop (issued work):")
        for lb, v in rate.items():
            print(f"#   {lb}: {v / ref:.3f}")
    print()
    out = {}
    pre = [lb for lb in ("chunk_prep_kernel", "state_pass_kernel") if lb in labels]
    if pre and fcal and all((lb, c) in tot for lb in pre for c in ("FETCH_SIZE", "WRITE_SIZE")):
        rd = sum(tot[(lb, "FETCH_SIZE")] for lb in pre) / _CALLS * 1024 / fcal
        wr = sum(tot[(lb, "WRITE_SIZE")] for lb in pre) / _CALLS * 1024 / wcal
        out["prefill"] = {"hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
                          "hbm_bytes_per_launch": rd + wr}
    if ref and pre and all((lb, "GRBM_GUI_ACTIVE") in tot for lb in pre):
        busy = sum(tot[(lb, "SQ_VALU_MFMA_BUSY_CYCLES")] for lb in pre)
        gui = sum(tot[(lb, "GRBM_GUI_ACTIVE")] for lb in pre)
        out.setdefault("prefill", {}).update(
            {f"mfma_busy_rel_{lb}": rate[lb] / ref for lb in pre})
        out["prefill"]["mfma_busy_rel_call"] = busy / gui / ref
    for lb in ("decode_kernel", "attnres_kernel"):
        if fcal and (lb, "FETCH_SIZE") in tot and (lb, "WRITE_SIZE") in tot:
            rd = tot[(lb, "FETCH_SIZE")] / _CALLS * 1024 / fcal
            wr = tot[(lb, "WRITE_SIZE")] / _CALLS * 1024 / wcal
            out[lb] = {"hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
                       "hbm_bytes_per_launch": rd + wr}
    _summarize_lds(dirs)
    for group, kv in out.items():
        print(f"[{group}]")
        for k, v in kv.items():
            print(f"{k}: {v:.6g}" if isinstance(v, float) and abs(v) < 100 else f"{k}: {v:.0f}")
    return out


def _ranges(xs):
    """[0, 1, 2, 5, 6] -> '0-2,5-6'"""
    out, i = [], 0
    while i < len(xs):
        j = i
        while j + 1 < len(xs) and xs[j + 1] == xs[j] + 1:
            j += 1
        out.append(f"{xs[i]}-{xs[j]}" if j > i else f"{xs[i]}")
        i = j + 1
    return ",".join(out)


def _summarize_lds(dirs):
    """The LDS bank model from the lds_probe dispatches of a profile pass
    with SQ_LDS_BANK_CONFLICT: dispatches in launch order are the cases of
    _lds_cases(); conflict cycles are per wave access."""
    import glob
    per = {}
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            for r in csv.DictReader(open(f)):
                if "lds_probe" in r["Kernel_Name"] and r["Counter_Name"] == "SQ_LDS_BANK_CONFLICT":
                    k = int(r["Dispatch_Id"])
                    per[k] = per.get(k, 0.0) + float(r["Counter_Value"])
    if not per:
        return
    cases = _lds_cases()
    vals = [per[k] / (_LDS_BLOCKS * _LDS_ITERS) for k in sorted(per)]
    if len(vals) != len(cases):
        print(f"# lds_probe: {len(vals)} dispatches, expected {len(cases)}; not summarised")
        return
    res = {key: v for (key, _, _), v in zip(cases, vals)}
    print(f"# LDS bank model (lds_probe, {len(vals)} dispatches of {_LDS_BLOCKS} one-wave workgroups x "
          f"{_LDS_ITERS} accesses; two active lanes, the base lane j0 at byte 0 and lane k at byte 256):")
    print("#   access form     | lanes served together with the base lane          | banks (4 bytes)")
    for f, name in enumerate(_LDS_FORMS):
        groups = []
        for j0 in _LDS_BASES.get(f, (0,)):
            same = sorted([j0] + [k for k in range(64) if k != j0 and res[("pair", f, j0, k)] > 0.5])
            groups.append(f"j0={j0}: {_ranges(same)}")
        banks = 32 if res[("span", f)] > 0.5 else 64
        print(f"#   {name:15s} | {'; '.join(groups):49s} | {banks}")
    print("# whole-wave patterns, conflict cycles per access:")
    for (key, _, _), v in zip(cases, vals):
        if key[0] == "pattern":
            print(f"#   {key[1]}: {v:.2f}")


# Phases of a default run, in order: (label, kernels of one call).  A prefill
# call is its segments' prep and pass kernels; the segment counts follow the
# library's 512 MiB ring (4 at B4 H16 T16K, 8 at H16 T128K).
_TRACE_PHASES = [("prefill_b4_h16_t16k", ("chunk_prep_kernel", "state_pass_kernel"), 4),
                 ("mfma calibration", ("mfma16_loop", "mfma32_loop"), 1),
                 ("decode_b256_h16", ("decode_kernel",), 1),
                 ("prefill_h16_t128k", ("chunk_prep_kernel", "state_pass_kernel"), 8),
                 ("prefill_h8_t4k", ("chunk_prep_kernel", "state_pass_kernel"), 1),
                 ("prefill_b4_h16_t16k (per-head gate)", ("chunk_prep_kernel", "state_pass_kernel"), 4),
                 ("attnres_l64_n4096_d4096", ("attnres_kernel",), 1)]


def summarize_trace(path):
    """Per-kernel durations of a rocprofv3 kernel trace of a default bench
    run (warm-up launches included), split into the run's phases, plus the
    whole prefill call (first prep start to last pass end)."""
    import statistics as st
    rows = [r for r in csv.DictReader(open(path))]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    names = [k for _, ks, _ in _TRACE_PHASES for k in ks]
    seq = []
    for r in rows:
        k = next((k for k in names if k in r["Kernel_Name"]), None)
        if k is not None:
            seq.append((k, r))
    # split into phases at the host-side pauses between them (input drawing
    # takes seconds; launches inside a phase follow each other within
    # milliseconds)
    groups, cur, last = [], [], None
    for k, r in seq:
        t = int(r["Start_Timestamp"])
        if last is not None and t - last > 50_000_000:  # 50 ms
            groups.append(cur)
            cur = []
        cur.append((k, r))
        last = int(r["End_Timestamp"])
    if cur:
        groups.append(cur)
    # a phase that follows without a pause (no host-side input drawing) is
    # split off at its first kernel of another kind
    split = []
    for g in groups:
        while g:
            ph = next(ks for _, ks, _ in _TRACE_PHASES if g[0][0] in ks)
            j = next((j for j, (k, _) in enumerate(g) if k not in ph), len(g))
            split.append(g[:j])
            g = g[j:]
    groups = split
    print("| workload | kernel | grid (threads) | block | LDS B | VGPR/AGPR | scratch | dispatches "
          "| avg us | median us | min us | max us |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    calls_out = []
    for (label, ks, nseg), run in zip(_TRACE_PHASES, groups):
        for k in ks:
            rs = [r for kk, r in run if kk == k]
            if not rs:
                continue
            d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]
            r0 = rs[0]
            grid = r0["Grid_Size_X"] + ("x" + r0["Grid_Size_Y"] if r0["Grid_Size_Y"] != "1" else "")
            print(f"| {label} | `{k}` | {grid} | {r0['Workgroup_Size_X']} | {r0['LDS_Block_Size']} "
                  f"| {r0['VGPR_Count']}/{r0['Accum_VGPR_Count']} | {r0['Scratch_Size']} | {len(d)} "
                  f"| {sum(d) / len(d):.2f} | {st.median(d):.2f} | {min(d):.2f} | {max(d):.2f} |")
        if "chunk_prep_kernel" in ks and run:
            per = 2 * nseg
            calls = [run[j:j + per] for j in range(0, len(run) - per + 1, per)]
            span = [(int(c[-1][1]["End_Timestamp"]) - int(c[0][1]["Start_Timestamp"])) / 1e3
                    for c in calls]
            calls_out.append((label, len(span), sum(span) / len(span), st.median(span), min(span)))
    print()
    print("| workload | calls | avg us | median us | min us |")
    print("|---|---|---|---|---|")
    for label, n, a, m, lo in calls_out:
        print(f"| {label} | {n} | {a:.1f} | {m:.1f} | {lo:.1f} |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--long-steps", type=int, default=5)
    ap.add_argument("--cpu-long-tokens", type=int, default=16384,
                    help="tokens of each long-context chain the CPU baseline runs")
    ap.add_argument("--cpu-decode-steps", type=int, default=32,
                    help="decode steps (all heads) the CPU baseline runs")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-small", action="store_true")
    ap.add_argument("--no-gdn", action="store_true")
    ap.add_argument("--no-attnres", action="store_true")
    ap.add_argument("--no-calibration", action="store_true")
    ap.add_argument("--profile-pass", action="store_true")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 counter CSVs under DIR(s) and exit (no GPU)")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="summarise a rocprofv3 kernel trace of a default run and exit (no GPU)")
    args = ap.parse_args()

    if args.summarize:
        summarize(args.summarize)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the KDA hot path here runs on a single "
              "MI355X and has no multi-GPU mode (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import gated_delta_rule_76_amd  # noqa: F401  (fails loudly if libkda.so is missing)

    if args.profile_pass:
        profile_pass()
        return

    from synth import WORKLOADS, workload_inputs

    # ---- headline: prefill B4 H16 T16K (host inputs kept for the CPU baseline)
    x2 = workload_inputs(WORKLOADS[PREFILL])
    w, total, per, ok_p = bench_prefill(PREFILL, args.steps, args.warmup, x=x2)
    tokens = w.B * w.T
    value = tokens * args.steps / total
    launch_ms = per
    by = prefill_alg_bytes(w.B, w.T, w.H, w.d_k, w.d_v)
    fl = prefill_alg_flops(w.B, w.T, w.H, w.d_k, w.d_v, w.chunk)
    gbs = by / (launch_ms / 1e3) / 1e9
    tfl = fl / (launch_ms / 1e3) / 1e12
    roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4),
                "traffic": _recorded_traffic("kda_prefill.hip", "prefill_b4_h16_t16k_counters.txt"),
                "alg_bytes_per_launch": by, "launch_ms": round(launch_ms, 4),
                "launch": "one kda_fwd_chunked call: chunk_prep_kernel + state_pass_kernel",
                "mfma": {"achieved_tflops": round(tfl, 2), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                         "frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4), "alg_flops_per_launch": fl,
                         "counter_busy_rel": _recorded("kda_prefill.hip",
                                                       "prefill_b4_h16_t16k_counters.txt",
                                                       "mfma_busy_rel_call"),
                         "counter_busy_note": "SQ_VALU_MFMA_BUSY_CYCLES per GRBM_GUI_ACTIVE cycle "
                                              "over one call, relative to the saturated MFMA "
                                              "loop (issued work; from the committed profile "
                                              "summary, null once the kernel source changed)"}}
    if not args.no_calibration:
        cal = bench_mfma_calibration()
        roofline["mfma"]["measured_peak_tflops"] = cal["measured_peak_tflops"]
        roofline["mfma"]["frac_of_measured_peak"] = round(tfl / cal["measured_peak_tflops"], 4)
        roofline["mfma"]["calibration"] = cal
    # Attainable roofline min(MFMA, AI * BW) for the algorithmic work: HBM here.
    attain = min(MFMA_BF16_PEAK_TFLOPS * 1e12, fl / by * HBM_PEAK_GBS * 1e9)
    roofline["attainable_frac"] = round((fl / (launch_ms / 1e3)) / attain, 4)

    # ---- decode B256 H16, 1000 consecutive steps
    wd, dtot, dper, ok_d, dec_block = bench_decode(args.decode_steps, 10)
    dby = decode_alg_bytes(wd.B, wd.H, wd.d_k, wd.d_v)
    d_launch = dper
    d_gbs = dby / (d_launch / 1e3) / 1e9
    decode = {"value": round(dby * args.decode_steps / dtot / 1e9, 1), "unit": "GB/s",
              "steps": args.decode_steps, "ms_per_step": round(dtot * 1e3 / args.decode_steps, 4),
              "tokens_per_s": round(wd.B * args.decode_steps / dtot, 1),
              "config": {"workload": DECODE, "batch": wd.B, "heads": wd.H, "d_k": wd.d_k,
                         "d_v": wd.d_v, "state": "fp32", "io": "bf16"},
              "roofline": {"bound": "hbm", "achieved": round(d_gbs, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(d_gbs / HBM_PEAK_GBS, 4),
                           "traffic": _recorded_traffic("kda_decode.hip",
                                                        "decode_b256_h16_counters.txt"),
                           "alg_bytes_per_launch": dby, "launch_ms": round(d_launch, 4),
                           "launch": "one kda_decode_step call: decode_kernel"}}

    long_ctx = None
    x3 = None
    if not args.no_long:
        x3full = workload_inputs(WORKLOADS[LONG])
        if not args.no_cpu:  # the CPU baseline's share: the first tokens of every chain
            t3 = min(args.cpu_long_tokens, x3full["q"].shape[1])
            x3 = {n: np.ascontiguousarray(x3full[n][:, :t3]) for n in ("q", "k", "v", "alpha", "beta")}
            x3["S0"] = x3full["S0"]
        wl, ltot, lper, ok_l = bench_prefill(LONG, args.long_steps, 1, x=x3full)
        del x3full
        l_ms = lper
        lby = prefill_alg_bytes(wl.B, wl.T, wl.H, wl.d_k, wl.d_v)
        long_ctx = {"value": round(wl.B * wl.T * args.long_steps / ltot, 1), "unit": "tokens/s",
                    "ms_per_call": round(l_ms, 3), "finite": ok_l,
                    "config": {"workload": LONG, "batch": wl.B, "seq_len": wl.T, "heads": wl.H,
                               "chunk": wl.chunk},
                    "hbm_frac": round(lby / (l_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}

    # B1 H8 T4K: 8 chains of 64 chunks, a launch-latency-sized call
    small = None
    if not args.no_small:
        ws_, stot, sper, ok_s = bench_prefill(SMALL, 4 * args.steps, args.warmup)
        sby = prefill_alg_bytes(ws_.B, ws_.T, ws_.H, ws_.d_k, ws_.d_v)
        small = {"value": round(ws_.B * ws_.T * 4 * args.steps / stot, 1), "unit": "tokens/s",
                 "ms_per_call": round(sper, 4), "finite": ok_s,
                 "config": {"workload": SMALL, "batch": ws_.B, "seq_len": ws_.T, "heads": ws_.H,
                            "chunk": ws_.chunk},
                 "hbm_frac": round(sby / (sper / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}

    # Gated DeltaNet variant (one decay per token and head) on the headline shape
    gdn = None
    if not args.no_gdn:
        wg, gtot, gper, ok_g = bench_prefill(PREFILL, args.steps, args.warmup, gate="head", x=x2)
        g_ms = gper
        gby = prefill_alg_bytes(wg.B, wg.T, wg.H, wg.d_k, wg.d_v, gate_per_channel=False)
        gdn = {"value": round(wg.B * wg.T * args.steps / gtot, 1), "unit": "tokens/s",
               "ms_per_call": round(g_ms, 4), "finite": ok_g, "gate": "head",
               "config": {"workload": PREFILL, "batch": wg.B, "seq_len": wg.T, "heads": wg.H,
                          "chunk": wg.chunk},
               "roofline": {"bound": "hbm", "achieved": round(gby / (g_ms / 1e3) / 1e9, 1),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(gby / (g_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                            "alg_bytes_per_launch": gby}}

    attnres = None
    if not args.no_attnres:
        atot, aper, ok_a = bench_attnres(args.steps, args.warmup)
        a_ms = aper
        c = ATTNRES
        aby = attnres_alg_bytes(c["L"], c["N"], c["d_k"], c["d"])
        attnres = {"value": round(c["N"] * args.steps / atot, 1), "unit": "tokens/s",
                   "ms_per_call": round(a_ms, 4), "finite": ok_a,
                   "config": {"workload": "attnres_l64_n4096_d4096", "layers": c["L"],
                              "tokens": c["N"], "d_k": c["d_k"], "d": c["d"], "dtype": "bf16"},
                   "roofline": {"bound": "hbm", "achieved": round(aby / (a_ms / 1e3) / 1e9, 1),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(aby / (a_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                "alg_bytes_per_launch": aby,
                                "traffic": _recorded_traffic("attnres.hip",
                                                             "attnres_l64_n4096_d4096_counters.txt"),
                                "launch": "one attnres_forward call: attnres_kernel"}}

    cpu = None if args.no_cpu else cpu_baseline(x2, x3, dec_block, args.cpu_decode_steps)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(total * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PREFILL, "global_batch": w.B, "seq_len": w.T, "heads": w.H,
                   "d_k": w.d_k, "d_v": w.d_v, "chunk": w.chunk, "state": "fp32",
                   "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "decode": decode, "long_context": long_ctx,
        "small_prefill": small,
        "gated_deltanet": gdn, "attnres": attnres,
        "finite": bool(ok_p and ok_d),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
