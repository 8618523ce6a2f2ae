"""Measurement driver: kernels for profilers, copy calibration, length sweep.

Subcommands (run as ``python -m io_aware_softmax_amd.measure <cmd>``):

* ``kernels`` - uploads the causal bf16 prefill (B1 H32 L8192 D128) and the
  bf16 decode (B16 H32 Lk32768 D128) inputs and runs each kernel call
  (prefill forward, its backward with a seeded upstream gradient, decode)
  ``--reps`` times, for rocprofv3 kernel traces and counter passes; with
  ``--workload NAME`` only that workload's forward.
* ``copy`` - copies a 1 GiB device buffer ``--reps`` times (torch's copy
  kernel): reads and writes exactly 2^30 bytes per launch, the reference
  that scales the FETCH_SIZE / WRITE_SIZE counters to bytes.
* ``sweep_ext`` - shapes past the five workloads: the fp16 sweep at
  L = 8192, bf16 D128 lengths causal and not, one sequence with one or a few
  heads (few workgroups), the long-context workload's shape (B1 H8 L65536
  causal), and chunked prefill (Lq new queries against Lk cached keys).  One
  JSON line per case.
* ``ex`` - forward and backward of the causal bf16 8k prefill through the
  plain entry points and through attn_fwd_ex / attn_bwd_ex with boolean and
  additive masks and dropout.  One JSON line per case.
* ``sweep`` - the fp16 length sweep (B4 H8 D64, L = 64 ... 4096,
  non-causal): TFLOP/s of ``attn_fwd`` next to a materialised-softmax GPU
  baseline that writes the scores and weights to device memory (the naive
  multi-pass algorithm: QK^T, softmax, PV as three torch kernels in fp16,
  with the transposed operand made contiguous).  Prints one JSON line per L.

Every step of the attention itself runs in libattn.so; torch only provides
memory, streams, timing events and the comparison baseline.
"""

from __future__ import annotations

import argparse
import json
import math
import sys
import time

import numpy as np
import torch

from . import binding, inputs


def _dev(bits, dtype):
    if dtype == "f32":
        return torch.from_numpy(bits).cuda()
    t = torch.from_numpy(bits.view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def _upload(wl):
    bits = inputs.generate(wl)
    return [_dev(bits[t], wl.dtype) for t in "qkv"]


def cmd_kernels(args):
    if args.workload:
        # One forward workload on its own (e.g. the fp16 sweep's L = 4096
        # point), for counter passes on the kernel that serves it.
        wl = inputs.WORKLOADS[args.workload]
        q, k, v = _upload(wl)
        o = torch.empty_like(q)
        lse = torch.empty(wl.B, wl.H, wl.Lq, dtype=torch.float32, device="cuda")
        print(f"forward {wl.name}: {args.reps} launches", flush=True)
        for _ in range(args.reps):
            binding.attn_fwd(q, k, v, causal=wl.causal, scale=wl.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        print("done", flush=True)
        return
    wp = inputs.WORKLOADS["causal_bf16_8k"]
    wd = inputs.WORKLOADS["decode_bf16_32k"]
    q, k, v = _upload(wp)
    print(f"prefill {wp.name}: {args.reps} launches", flush=True)
    for _ in range(args.reps):
        O, L = binding.attn_fwd(q, k, v, causal=True, scale=wp.scale)
    torch.cuda.synchronize()
    g = _dev(inputs.generate(wp, ("do",))["do"], wp.dtype)
    print(f"backward {wp.name}: {args.reps} launches", flush=True)
    for _ in range(args.reps):
        binding.attn_bwd(q, k, v, O, L, g, causal=True, scale=wp.scale)
    torch.cuda.synchronize()
    del q, k, v, O, L, g
    torch.cuda.empty_cache()
    q, k, v = _upload(wd)
    splits = binding.attn_decode_auto_splits(wd.B, wd.H, wd.Lk, wd.D)
    print(f"decode {wd.name}: {args.reps} launches, {splits} splits", flush=True)
    for _ in range(args.reps):
        binding.attn_decode_fwd(q, k, v, scale=wd.scale, num_splits=splits)
    torch.cuda.synchronize()
    print("done", flush=True)


def cmd_copy(args):
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    print(f"copy: {args.reps} launches of {n} bytes", flush=True)
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("done", flush=True)


def _time(fn, reps, warm_s=0.2):
    """Median and minimum event time of ``reps`` calls, after at least
    ``warm_s`` seconds of back-to-back calls: the shader clock needs tens of
    milliseconds of load to settle, and a few warm-up calls would time the
    ramp instead of the steady state."""
    t0 = time.perf_counter()
    n = 0
    while n < 3 or time.perf_counter() - t0 < warm_s:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    return float(np.median(ms)), float(ms[0])


def _materialised(q, k, v, scale):
    # Scores and weights are written to device memory between the kernels.
    s = torch.matmul(q, k.transpose(-2, -1).contiguous()) * scale
    p = torch.softmax(s, dim=-1)
    return torch.matmul(p, v)


def cmd_sweep(args):
    for L in inputs.SWEEP_LENGTHS:
        wl = inputs.WORKLOADS[f"sweep_f16_L{L}"]
        q, k, v = _upload(wl)
        o = torch.empty_like(q)
        lse = torch.empty(wl.B, wl.H, L, dtype=torch.float32, device="cuda")
        ours = _time(lambda: binding.attn_fwd(q, k, v, causal=False, scale=wl.scale, out=o, lse=lse), args.reps)
        base = _time(lambda: _materialised(q, k, v, wl.scale), args.reps)
        ref = _materialised(q, k, v, wl.scale)
        torch.cuda.synchronize()
        diff = float((o.float() - ref.float()).abs().max())
        rec = {"workload": wl.name, "L": L, "flops": wl.flops(),
               "attn_fwd_ms": ours[0], "attn_fwd_tflops": wl.flops() / ours[0] / 1e9,
               "materialised_ms": base[0], "materialised_tflops": wl.flops() / base[0] / 1e9,
               "speedup": base[0] / ours[0], "max_abs_diff_vs_materialised": diff}
        print(json.dumps(rec), flush=True)
        del q, k, v, o, lse, ref
        torch.cuda.empty_cache()


def cmd_sweep_ext(args):
    """Shapes beyond the five workloads: the fp16 sweep at L = 8192, bf16 D = 128
    lengths, a single sequence and head (few workgroups), the long-context
    workload's shape (B1 H8 L65536 causal), and chunked prefill (Lq new
    queries against Lk cached keys, bottom-right causal)."""
    cases = [
        # (label, B, H, Lq, Lk, D, dtype, causal, materialised baseline)
        ("fp16 sweep extension", 4, 8, 8192, 8192, 64, "f16", False, True),
        ("bf16 D128 non-causal", 1, 32, 2048, 2048, 128, "bf16", False, False),
        ("bf16 D128 non-causal", 1, 32, 16384, 16384, 128, "bf16", False, False),
        ("bf16 D128 causal", 1, 32, 2048, 2048, 128, "bf16", True, False),
        ("bf16 D128 causal", 1, 32, 16384, 16384, 128, "bf16", True, False),
        ("single sequence, one head", 1, 1, 16384, 16384, 128, "bf16", True, False),
        ("single sequence, one head", 1, 1, 65536, 65536, 128, "bf16", True, False),
        ("single sequence, 8 heads", 1, 8, 16384, 16384, 128, "bf16", True, False),
        ("long-context causal prefill", 1, 8, 65536, 65536, 128, "bf16", True, False),
        ("chunked prefill", 1, 32, 512, 8192, 128, "bf16", True, False),
        ("chunked prefill", 1, 32, 2048, 8192, 128, "bf16", True, False),
    ]
    for i, (label, B, H, Lq, Lk, D, dt, causal, mat) in enumerate(cases):
        wl = inputs.custom(f"ext_{i}", B, H, Lq, Lk, D, dt, causal, seed=900 + i)
        q, k, v = _upload(wl)
        o = torch.empty_like(q)
        lse = torch.empty(B, H, Lq, dtype=torch.float32, device="cuda")
        scale = 1.0 / math.sqrt(D)
        # Algorithmic flops: 4 D per allowed (query, key) pair.
        if causal:
            off = Lk - Lq
            pairs = sum(min(Lk, i + off + 1) for i in range(Lq))
        else:
            pairs = Lq * Lk
        flops = 4.0 * B * H * D * pairs
        ours = _time(lambda: binding.attn_fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse), args.reps)
        rec = {"case": label, "B": B, "H": H, "Lq": Lq, "Lk": Lk, "D": D, "dtype": dt, "causal": causal,
               "flops": flops, "attn_fwd_ms": ours[0], "attn_fwd_tflops": flops / ours[0] / 1e9}
        if mat:
            base = _time(lambda: _materialised(q, k, v, scale), max(3, args.reps // 4))
            rec["materialised_ms"] = base[0]
            rec["speedup"] = base[0] / ours[0]
        print(json.dumps(rec), flush=True)
        del q, k, v, o, lse
        torch.cuda.empty_cache()


def cmd_ex(args):
    """Forward and backward of the causal bf16 prefill shape (B1 H32 L8192
    D128) through the plain entry points and through the general ones with a
    boolean mask (broadcast over heads, half the keys of every row kept),
    an additive mask, dropout 0.1, and mask plus dropout.  Flops are the
    algorithmic ones of the causal problem (forward 4 D per allowed pair,
    backward 2.5 times that) whatever the mask removes."""
    wl = inputs.WORKLOADS["causal_bf16_8k"]
    q, k, v = _upload(wl)
    g = _dev(inputs.generate(wl, ("do",))["do"], wl.dtype)
    L = wl.Lq
    bmask = torch.from_numpy(inputs.bool_mask(5, (1, 1, L, L), keep=0.5)).cuda()
    amask = torch.from_numpy(inputs.additive_mask(6, (1, 1, L, L), neg_inf=0.0)).cuda()
    cases = [("plain", None, 0.0), ("bool mask", bmask, 0.0), ("additive mask", amask, 0.0),
             ("dropout 0.1", None, 0.1), ("bool mask + dropout 0.1", bmask, 0.1)]
    for label, mask, p in cases:
        if args.case and label != args.case:
            continue
        if label == "plain":
            fwd = lambda: binding.attn_fwd(q, k, v, causal=True, scale=wl.scale)
        else:
            fwd = lambda: binding.attn_fwd_ex(q, k, v, causal=True, scale=wl.scale, mask=mask, dropout_p=p, seed=3)
        O, Lse = fwd()
        if label == "plain":
            bwd = lambda: binding.attn_bwd(q, k, v, O, Lse, g, causal=True, scale=wl.scale)
        else:
            bwd = lambda: binding.attn_bwd_ex(q, k, v, O, Lse, g, causal=True, scale=wl.scale, mask=mask,
                                              dropout_p=p, seed=3)
        tf = _time(fwd, args.reps)
        tb = _time(bwd, args.reps)
        rec = {"case": label, "workload": wl.name, "fwd_ms": tf[0], "fwd_tflops": wl.flops() / tf[0] / 1e9,
               "bwd_ms": tb[0], "bwd_tflops": 2.5 * wl.flops() / tb[0] / 1e9,
               "mask_bytes": 0 if mask is None else mask.numel() * mask.element_size()}
        print(json.dumps(rec), flush=True)


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("cmd", choices=["kernels", "copy", "sweep", "sweep_ext", "ex"])
    p.add_argument("--reps", type=int, default=5)
    p.add_argument("--case", default="", help="ex: run only the case with this label")
    p.add_argument("--workload", default="", help="kernels: run only this workload's forward")
    args = p.parse_args(argv)
    if not torch.cuda.is_available():
        print("needs a GPU", file=sys.stderr)
        return 1
    binding.load()
    {"kernels": cmd_kernels, "copy": cmd_copy, "sweep": cmd_sweep, "sweep_ext": cmd_sweep_ext,
     "ex": cmd_ex}[args.cmd](args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
