"""Throughput of the KDA forward hot path on one MI355X.

One step = one kda_fwd_chunked call over the B=4, H=16, T=16384, d=128,
C=64 bf16 prefill workload (inputs resident in HBM).  The same run also
times the batched T=1 decode (B=256, H=16, d=128, 1000 consecutive steps)
and the long-context prefill (B=1, H=16, T=131072), and times the fp64 CPU
oracle on a bounded sample of the prefill workload on the host cores.

Prints one JSON line.  `value` is prefill tokens/s (tokens = batch x
sequence positions, all 16 heads each); the decode state-update HBM GB/s is
in `decode`.

    python bench.py [--steps K] [--warmup W] [--decode-steps N] [--no-cpu] [--no-long]
    python bench.py --profile-pass     # short fixed run for rocprofv3 counters
"""
from __future__ import annotations

import argparse
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


def _recorded_traffic(kernel_file: str, summary: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when the summary is absent or the kernel source changed since."""
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
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


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


def bench_prefill(name: str, steps: int, warmup: int, gate: str = "channel"):
    import torch
    import gated_delta_rule_76_amd as kda
    from synth import WORKLOADS, workload_inputs

    w = WORKLOADS[name]
    x = workload_inputs(w)
    if gate == "head":  # one decay per (token, head): the first channel of the drawn gate
        x["alpha"] = np.ascontiguousarray(x["alpha"][..., 0])
    d = _upload(x, ("q", "k", "v", "alpha", "beta"), w.dtype)
    s0 = torch.from_numpy(x["S0"]).cuda()
    del x
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
    for first in range(0, n, blk):
        cnt = min(blk, n - first)
        p = decode_steps(w.B, w.H, w.d_k, w.d_v, first, cnt, dtype=w.dtype, gate_c=w.gate_c,
                         seed=w.seed)
        for nm in names:
            d[nm][first:first + cnt].copy_(torch.from_numpy(p[nm]).to(torch.bfloat16))
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
    return w, total, per, ok


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


def cpu_baseline(sample_tokens: int):
    """Time the fp64 oracle on the first `sample_tokens` positions of every
    (batch, head) chain of the prefill workload on all host cores, and on one
    chain with a single thread."""
    import oracle
    from synth import WORKLOADS, workload_inputs

    w = WORKLOADS[PREFILL]
    x = workload_inputs(w, T=sample_tokens)
    threads = min(os.cpu_count() or 1, w.B * w.H)
    t0 = time.perf_counter()
    oracle.kda_forward(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], threads=threads)
    dt = time.perf_counter() - t0
    # one (batch, head) chain, one thread: per token-head rate
    one = {n: x[n][:1, :, :1] for n in ("q", "k", "v", "alpha", "beta")}
    t1 = time.perf_counter()
    oracle.kda_forward(one["q"], one["k"], one["v"], one["alpha"], one["beta"], x["S0"][:1, :1],
                       threads=1)
    dt1 = time.perf_counter() - t1
    return {"value": w.B * sample_tokens / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{PREFILL}: all {w.B * w.H} (batch, head) chains, first {sample_tokens} "
                      f"of {w.T} tokens, fp64 token recurrence, {dt:.2f} s wall on {threads} "
                      f"threads",
            "single_thread_token_heads_per_s": round(sample_tokens / dt1, 1)}


def profile_pass():
    """Fixed short run for rocprofv3 counter passes: a plain 1 GiB copy (the
    calibration kernel), 3 prefill launches, 3 decode launches, 3 AttnRes
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
    bench_prefill(PREFILL, 3, 0)
    print("prefill: 3 launches", flush=True)
    bench_decode(3, 0)
    print("decode: 3 launches", flush=True)
    bench_attnres(3, 0)
    print("attnres: 3 launches", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--long-steps", type=int, default=5)
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-gdn", action="store_true")
    ap.add_argument("--no-attnres", action="store_true")
    ap.add_argument("--profile-pass", action="store_true")
    args = ap.parse_args()

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

    # ---- headline: prefill B4 H16 T16K
    w, total, per, ok_p = bench_prefill(PREFILL, args.steps, args.warmup)
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
                         "frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4), "alg_flops_per_launch": fl}}

    # ---- decode B256 H16, 1000 consecutive steps
    wd, dtot, dper, ok_d = bench_decode(args.decode_steps, 10)
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
    if not args.no_long:
        wl, ltot, lper, ok_l = bench_prefill(LONG, args.long_steps, 1)
        l_ms = lper
        lby = prefill_alg_bytes(wl.B, wl.T, wl.H, wl.d_k, wl.d_v)
        long_ctx = {"value": round(wl.B * wl.T * args.long_steps / ltot, 1), "unit": "tokens/s",
                    "ms_per_call": round(l_ms, 3), "finite": ok_l,
                    "config": {"workload": LONG, "batch": wl.B, "seq_len": wl.T, "heads": wl.H,
                               "chunk": wl.chunk},
                    "hbm_frac": round(lby / (l_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}

    # Gated DeltaNet variant (one decay per token and head) on the headline shape
    gdn = None
    if not args.no_gdn:
        wg, gtot, gper, ok_g = bench_prefill(PREFILL, args.steps, args.warmup, gate="head")
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

    cpu = None if args.no_cpu else cpu_baseline(args.cpu_sample_tokens)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(total * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PREFILL, "global_batch": w.B, "seq_len": w.T, "heads": w.H,
                   "d_k": w.d_k, "d_v": w.d_v, "chunk": w.chunk, "state": "fp32",
                   "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "decode": decode, "long_context": long_ctx,
        "gated_deltanet": gdn, "attnres": attnres,
        "finite": bool(ok_p and ok_d),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
