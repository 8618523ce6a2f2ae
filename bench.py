"""Benchmark of the exact attention forward on one MI355X.

One step = one pass of the whole hot path over one batch of seeded synthetic
input: the causal bf16 prefill (B=1, H=32, L=8192, D=128, x8 queries on
heads 0-3) followed by the split-KV bf16 decode (B=16, H=32, Lk=32768,
D=128).  Inputs are resident in device memory before timing starts.  W
untimed warm-up steps, then exactly K timed steps bracketed by device
synchronisation; each kernel call is also bracketed by HIP events on the
stream it runs on, which gives the per-launch durations behind the roofline
figures.

Prints ONE JSON line.  ``value`` is the prefill throughput in TFLOP/s
(4 B H Lq Lk D flops, halved for causal, over the prefill's own average
duration); the decode throughput (K+V bytes over the decode call's average
duration) is reported under ``decode``; the backward of the prefill
workload (dQ, dK, dV through ``attn_bwd``, timed on its own) under
``backward``.  ``cpu_baseline`` times the float64
CPU oracle on a bounded sample of the prefill workload (test infrastructure,
never part of the timed path), and the oracle's time per row on the
long-context workload's sampled rows with a labelled extrapolation;
``parity`` compares the timed prefill's output on those heads with the
oracle's.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

PREFILL = "causal_bf16_8k"
DECODE = "decode_bf16_32k"


def _parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # The GPU's clocks take a few tens of milliseconds of sustained load to
    # settle; the default warm-up (about 100 ms) reaches that state first.
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--splits", type=int, default=0, help="decode split count (0 = library choice)")
    p.add_argument("--parts", default="prefill,decode,backward",
                   help="comma-separated parts to run: prefill and decode (the step), backward "
                        "(timed on its own, reported under 'backward')")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-heads", type=int, default=24, help="heads of the prefill workload the oracle times")
    return p.parse_args()


def _traffic(kernel_file: str, summary: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None if there is none or the kernel source changed since it was taken."""
    path = ROOT / "profiles" / summary
    src = ROOT / "io_aware_softmax_amd" / "csrc" / kernel_file
    if not path.exists():
        return None
    fields = {}
    for line in path.read_text().splitlines():
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != hashlib.sha256(src.read_bytes()).hexdigest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _to_device(bits, dtype):
    import numpy as np
    import torch
    if dtype == "f32":
        return torch.from_numpy(bits).cuda()
    t = torch.from_numpy(bits.view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def _cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _round_to(x, dtype):
    """float64 values rounded once, to nearest-even, to the output's storage
    type (bf16 keeps 8 significant bits)."""
    import numpy as np
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def _cpu_baseline(wl, heads: int, out=None, lse=None):
    """Time the float64 oracle on the first ``heads`` heads (all rows).

    With the device's output ``out`` [B, H, Lq, D] and ``lse`` [B, H, Lq]
    also returns the parity of those heads against the oracle's result:
    max|O - O_ref|, max|O - round(O_ref)| (the distance to the reference
    rounded to the output type) and the largest relative LSE error."""
    import numpy as np
    import oracle
    from io_aware_softmax_amd import inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    slabs = [{t: inputs.slab_values(wl, t, 0, h)[None, None] for t in "qkv"} for h in range(heads)]
    refs = []
    t0 = time.perf_counter()
    for s in slabs:
        refs.append(oracle.attention(s["q"], s["k"], s["v"], wl.scale, wl.causal))
    dt = time.perf_counter() - t0
    flops = wl.flops() * heads / (wl.B * wl.H)
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu": _cpu_model(),
            "sample": f"heads 0-{heads - 1} of {wl.H} (all {wl.Lq} rows) of the causal bf16 prefill, "
                      f"float64 NumPy, {dt:.1f} s for {flops:.3e} algorithmic flops"}
    # The long-context workload (B1 H8 L65536 causal) on its 256 sampled rows
    # per head: the oracle's time per row and a labelled extrapolation to
    # every row (the sampled rows are uniform over the sequence, so their
    # mean cost stands for the mean row).
    wl5 = inputs.WORKLOADS["long_causal_bf16_64k"]
    t5 = 0.0
    n5 = 0
    for h in range(wl5.H):
        rows = inputs.sample_rows(wl5, h, 256)
        qkv = {t: inputs.slab_values(wl5, t, 0, h)[None, None] for t in "qkv"}
        t1 = time.perf_counter()
        oracle.attention(qkv["q"], qkv["k"], qkv["v"], wl5.scale, wl5.causal, rows=rows)
        t5 += time.perf_counter() - t1
        n5 += len(rows)
    base["long_context_sampled_rows"] = {
        "workload": "causal bf16 B1 H8 L65536 D128", "rows": n5, "s": t5, "ms_per_row": 1e3 * t5 / n5,
        "extrapolated_full_s": t5 / n5 * wl5.B * wl5.H * wl5.Lq,
        "note": "oracle time on the 256 sampled rows per head; full-workload time extrapolated, not measured"}
    parity = None
    if out is not None:
        eo = er = el = 0.0
        for h, (O_ref, L_ref) in enumerate(refs):
            O = out[0, h].float().cpu().numpy().astype(np.float64)
            L = lse[0, h].cpu().numpy().astype(np.float64)
            O_ref, L_ref = O_ref[0, 0], L_ref[0, 0]
            eo = max(eo, float(np.max(np.abs(O - O_ref))))
            er = max(er, float(np.max(np.abs(O - _round_to(O_ref, wl.dtype)))))
            el = max(el, float(np.max(np.abs(L - L_ref) / np.maximum(1.0, np.abs(L_ref)))))
        parity = {"heads": f"0-{heads - 1} of {wl.H}, every row", "max_abs_O": eo,
                  "max_abs_O_vs_rounded_ref": er, "max_rel_lse": el, "o_tol": 2e-2}
    return base, parity


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from io_aware_softmax_amd import binding, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load()
    dev = torch.cuda.current_device()
    props = torch.cuda.get_device_properties(dev)

    wp = inputs.WORKLOADS[PREFILL]
    wd = inputs.WORKLOADS[DECODE]
    parts = {x.strip() for x in args.parts.split(",") if x.strip()}
    if not parts or parts - {"prefill", "decode", "backward"}:
        print("--parts takes prefill, decode and/or backward", file=sys.stderr)
        sys.exit(2)
    run_p, run_d, run_b = "prefill" in parts, "decode" in parts, "backward" in parts

    t_gen = time.perf_counter()
    if run_p or run_b:
        bp = inputs.generate(wp, ("q", "k", "v", "do") if run_b else ("q", "k", "v"))
        qp, kp, vp = (_to_device(bp[t], wp.dtype) for t in "qkv")
        gp = _to_device(bp["do"], wp.dtype) if run_b else None
        del bp
        op = torch.empty_like(qp)
        lp = torch.empty(wp.B, wp.H, wp.Lq, dtype=torch.float32, device="cuda")
    if run_d:
        bd = inputs.generate(wd)
        qd, kd, vd = (_to_device(bd[t], wd.dtype) for t in "qkv")
        del bd
        od = torch.empty_like(qd)
        ld = torch.empty(wd.B, wd.H, 1, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen
    splits = args.splits or binding.attn_decode_auto_splits(wd.B, wd.H, wd.Lk, wd.D)

    stream = torch.cuda.current_stream()

    def step(evs=None):
        if run_p:
            if evs is not None:
                evs[0].record(stream)
            binding.attn_fwd(qp, kp, vp, causal=wp.causal, scale=wp.scale, out=op, lse=lp)
            if evs is not None:
                evs[1].record(stream)
        if run_d:
            if evs is not None:
                evs[2].record(stream)
            binding.attn_decode_fwd(qd, kd, vd, scale=wd.scale, num_splits=splits, out=od, lse=ld)
            if evs is not None:
                evs[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    p_ms = [e[0].elapsed_time(e[1]) for e in evs] if run_p else [0.0]
    d_ms = [e[2].elapsed_time(e[3]) for e in evs] if run_d else [0.0]
    p_avg = float(np.mean(p_ms))
    d_avg = float(np.mean(d_ms))
    ms_per_step = wall * 1e3 / args.steps

    rec = {
        "metric": "attention fwd TFLOP/s (causal bf16 prefill B1 H32 L8192 D128)",
        "value": None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal bf16 prefill B1 H32 Lq=Lk=8192 D128 (q x8 on heads 0-3) "
                        "+ split-KV bf16 decode B16 H32 Lk32768 D128",
            "prefill": {"B": wp.B, "H": wp.H, "Lq": wp.Lq, "Lk": wp.Lk, "D": wp.D, "causal": True,
                        "scale": wp.scale, "flops": wp.flops()},
            "decode": {"B": wd.B, "H": wd.H, "Lq": 1, "Lk": wd.Lk, "D": wd.D, "splits": splits,
                       "kv_bytes": wd.kv_bytes()},
            "parallelism": "single GPU",
        },
    }
    if run_p:
        tflops = wp.flops() / (p_avg * 1e-3) / 1e12
        rec["value"] = tflops
        rec["ms_prefill"] = p_avg
        rec["ms_prefill_min"] = float(np.min(p_ms))
        rec["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                           "traffic": _traffic("prefill_pp.hip", "prefill_causal_bf16_8k_traffic.txt"),
                           "kernel": "prefill_pp_kernel<bf16, D=128, causal>"}
    if run_d:
        gbs = wd.kv_bytes() / (d_avg * 1e-3) / 1e9
        rec["decode"] = {"metric": "decode HBM GB/s (K+V bytes / decode call time)", "value": gbs,
                         "unit": "GB/s", "ms": d_avg, "ms_min": float(np.min(d_ms)),
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": gbs / PEAK_HBM_GBS,
                                      "traffic": _traffic("decode.hip", "decode_bf16_32k_traffic.txt"),
                                      "kernel": "decode_split_kernel<bf16, D=128> + decode_combine_kernel"}}
    if run_d:
        # Not part of the step: the ragged-length KV-cache decode on the same
        # cache, with seeded per-sequence lengths in [1, Lk]; bytes are the
        # K+V rows actually attended.
        lens = inputs.ragged_lengths(4, wd.B, wd.Lk)
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        for _ in range(10):
            binding.attn_decode_varlen_fwd(qd, kd, vd, sl, scale=wd.scale, out=od, lse=ld)
        torch.cuda.synchronize()
        vev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for a, b in vev:
            a.record(stream)
            binding.attn_decode_varlen_fwd(qd, kd, vd, sl, scale=wd.scale, out=od, lse=ld)
            b.record(stream)
        torch.cuda.synchronize()
        v_ms = float(np.mean([a.elapsed_time(b) for a, b in vev]))
        v_bytes = int(lens.astype(np.int64).sum()) * wd.H * 2 * wd.D * 2
        rec["decode_varlen"] = {"metric": "ragged KV-cache decode HBM GB/s (attended K+V bytes / call time)",
                                "value": v_bytes / (v_ms * 1e-3) / 1e9, "unit": "GB/s", "ms": v_ms,
                                "bytes": v_bytes, "lengths": "seeded uniform in [1, 32768] per sequence",
                                "frac_of_hbm_peak": v_bytes / (v_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    if run_b:
        # Not part of the step: the backward (dQ, dK, dV) of the prefill
        # workload from the forward's O and LSE and a seeded upstream
        # gradient.  Flops: the five L x L x D products of the chain rule
        # (recomputed scores, dP, dV, dK, dQ), 2 flops per multiply-add,
        # halved for causal.
        binding.attn_fwd(qp, kp, vp, causal=wp.causal, scale=wp.scale, out=op, lse=lp)
        dq, dk, dv = torch.empty_like(qp), torch.empty_like(kp), torch.empty_like(vp)

        def bwd():
            binding.attn_bwd(qp, kp, vp, op, lp, gp, causal=wp.causal, scale=wp.scale, dq=dq, dk=dk, dv=dv)

        for _ in range(10):
            bwd()
        torch.cuda.synchronize()
        bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for a, b in bev:
            a.record(stream)
            bwd()
            b.record(stream)
        torch.cuda.synchronize()
        b_ms = float(np.mean([a.elapsed_time(b) for a, b in bev]))
        b_flops = 2.5 * wp.flops()
        rec["backward"] = {"metric": "attention bwd TFLOP/s (causal bf16 B1 H32 L8192 D128, whole attn_bwd call)",
                           "value": b_flops / (b_ms * 1e-3) / 1e12, "unit": "TFLOP/s", "ms": b_ms,
                           "ms_min": float(np.min([a.elapsed_time(b) for a, b in bev])), "flops": b_flops,
                           "frac_of_mfma_peak": b_flops / (b_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                           "kernels": "bwd_stats_kernel + bwd_dkdv_kernel + bwd_dq_kernel"}
    rec["device"] = {"name": props.name, "cus": props.multi_processor_count,
                     "arch": getattr(props, "gcnArchName", "")}
    rec["input_gen_s"] = gen_s
    if run_p and not args.no_cpu_baseline:
        # The timed loop's last prefill output is still in ``op``/``lp``
        # (the backward leg rewrites them with the same values).
        rec["cpu_baseline"], rec["parity"] = _cpu_baseline(wp, args.cpu_heads, op, lp)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
