"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--settle S]

A step is one ``fa_fwd`` call over the whole workload with inputs resident
in HBM.  Untimed steps for ``--settle`` seconds (0.25 by default: the GPU
clock of a fresh process settles after about 80 ms of load) and W untimed
steps, then exactly K timed steps bracketed by device synchronisation; a pair of HIP events on the stream the kernels run on
brackets the K steps too, which gives the average device time of a step
used for the roofline.  Prints ONE JSON line.

Default workload: causal GQA prefill shaped like Qwen3-4B attention
(B=1, Hq=32, Hkv=8, N=8192, d=128), the configuration the headline metric
is quoted on.  ``--workload decode`` runs the single-query KV-split decode
(B=16, Hq=32, Hkv=8, Nk=32768, d=128) and reports HBM GB/s instead; its
timed step is the KV-split call with a workspace allocated once (partial
kernel + merge kernel).  ``--workload gqa_prefill_bwd`` times the backward
pass of the GQA prefill: one ``fa_bwd`` call (row preprocessing, dK/dV
kernel, dQ kernel) per step, from the O and lse of one untimed forward,
priced at 2.5 times the forward FLOPs; its roofline covers the whole call.
``--workload gqa_prefill_window`` runs ``fa_fwd_window`` on the GQA prefill
with a 4096-key sliding window (causal), priced at 4 d FLOPs per visible
pair, counted exactly.  ``--workload decode_window`` runs the decode workload through
``fa_fwd_window`` with a 4096-key window (KV split over the window's keys),
priced at the bytes of the keys it must read.  ``--workload decode_paged`` runs ``fa_fwd_paged`` on the decode workload's
shape stored in 256-key pages scattered over the pool, priced like the
decode.  ``--workload gqa_prefill_paged`` runs ``fa_fwd_paged`` on the GQA
prefill's shape stored in 256-key pages scattered over the pool (the tiled
prefill kernel reading each block from its page), priced like the GQA
prefill.  ``--workload gqa_prefill_fp8`` runs ``fa_fwd_fp8`` on the GQA prefill's shape
with E4M3 inputs and reports TFLOP/s against the FP8 matrix-core peak.
``--workload gqa_prefill_sparse`` runs ``fa_fwd_block_sparse`` on the GQA
prefill with a seeded block mask (a quarter of the 128 x 64 blocks plus the
diagonal), priced at the visible pairs of the kept blocks.
``--workload decode_d256`` runs the decode with head dimension 256 over
16384 keys (the same K/V bytes as the decode workload), and
``--workload gqa_prefill_d256`` the GQA prefill with head dimension 256 over
16 query heads and 8 KV heads (the same FLOPs).
``--workload gqa_prefill_docmask`` runs ``fa_fwd_colmask`` on the GQA
prefill's shape with the 8192 tokens split into causal documents of seeded
lengths in [300, 2500] (a column-interval mask), priced at the exact visible
pairs.
``--workload varlen_prefill`` runs ``fa_fwd_varlen`` over a packed batch of
causal prompts (seeded log-uniform lengths in [256, 8192], 32768 tokens,
the GQA heads above), priced at the causal FLOPs of each sequence.

The CPU baseline is the float64 oracle (test infrastructure) timed on the
host on a bounded sample of the same workload: whole heads of the prefill,
added one at a time until about 10 s of CPU work has been done.
"""
from __future__ import annotations

import dataclasses
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from fa_inputs import (VARLEN_PREFILL, document_column_bounds,  # noqa: E402
                       make_dout, make_fp8, make_inputs, make_paged,
                       make_varlen, random_doc_lens, sparse_block_mask,
                       varlen_lengths, workload)
from exact_io_aware_05_amd.metrics import (  # noqa: E402
    PEAK_BF16_MFMA_TFLOPS, PEAK_FP8_MFMA_TFLOPS, PEAK_HBM_GBS,
    attention_bwd_flops,
    attention_fwd_bytes, attention_fwd_flops, attention_window_flops,
    block_pair_counts, column_mask_pairs, visible_keys)

METRIC = "attn fwd TFLOP/s & % bf16 MFMA peak (causal GQA d=128 N=8192)"
WORKLOADS = {"gqa_prefill": 3, "decode": 4, "mha_d64": 1, "causal_outlier": 2,
             "tiny": 0, "gqa_prefill_bwd": 3, "varlen_prefill": None,
             "gqa_prefill_window": 3, "decode_window": 4,
             "gqa_prefill_window_bwd": 3, "decode_paged": None,
             "gqa_prefill_fp8": None, "gqa_prefill_sparse": None,
             "gqa_prefill_docmask": None, "decode_d256": 4,
             "gqa_prefill_paged": None, "gqa_prefill_d256": 3}
# workloads that change one configuration's shape: head dimension 256 on
# the decode (half the keys, so the same K/V bytes)
VARIANTS = {"decode_d256": dict(name="decode_b16_hq32_hkv8_nq1_nk16384_d256",
                                Nk=16384, d=256, scale=0.0625),
            # head dimension 256 on the GQA prefill: the same total head
            # width (16 query heads over 8 KV heads), the same FLOPs
            "gqa_prefill_d256": dict(
                name="gqa_prefill_b1_hq16_hkv8_n8192_d256_causal", Hq=16,
                Hkv=8, d=256, scale=0.0625)}
# sliding-window workloads: (left, right) bounds, run through fa_fwd_window
# (and fa_bwd_window)
WINDOWS = {"gqa_prefill_window": (4096, -1), "decode_window": (4096, -1),
           "gqa_prefill_window_bwd": (4096, -1)}
# HBM bytes per launch of each workload's dominant kernel, from two
# rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch; summaries under profiles/).  Each counter is scaled by what it
# reads for a plain device copy of known size (``--calibrate-copy``): a
# 1 GiB copy reads FETCH_SIZE = 524301 KiB and WRITE_SIZE = 1048576 KiB.
# A figure is reported only while the kernel source and the headers it
# includes still hash to the value it was taken on; otherwise traffic is
# null.
FETCH_SCALE = 1048576.0 / 524301.0
WRITE_SCALE = 1048576.0 / 1048576.0
MEASURED_TRAFFIC = {
    "gqa_prefill_b1_hq16_hkv8_n8192_d256_causal": {
        "source": "fa_prefill.hip",
        "sha256": "9b9b9698dd11d0c43cf794d84c00fd747c7571b8763e1a12d6ef6bd0fe536f5c",
        "fetch_kib": 113879.5, "write_kib": 66076.8},
    "gqa_prefill_paged_b1_hq32_hkv8_n8192_d128_causal_p256": {
        "source": "fa_prefill.hip",
        "sha256": "9b9b9698dd11d0c43cf794d84c00fd747c7571b8763e1a12d6ef6bd0fe536f5c",
        "fetch_kib": 71241.3, "write_kib": 66616.3},
    "gqa_prefill_b1_hq32_hkv8_n8192_d128_causal": {
        "source": "fa_prefill.hip",
        "sha256": "9b9b9698dd11d0c43cf794d84c00fd747c7571b8763e1a12d6ef6bd0fe536f5c",
        "fetch_kib": 71198.9, "write_kib": 66560.5},
    "mha_b4_h16_n2048_d64": {
        "source": "fa_prefill.hip",
        "sha256": "9b9b9698dd11d0c43cf794d84c00fd747c7571b8763e1a12d6ef6bd0fe536f5c",
        "fetch_kib": 41049.5, "write_kib": 16896.0},
    "causal_outlier_b2_h16_n4096_d128": {
        "source": "fa_prefill.hip",
        "sha256": "9b9b9698dd11d0c43cf794d84c00fd747c7571b8763e1a12d6ef6bd0fe536f5c",
        "fetch_kib": 76681.5, "write_kib": 33418.3},
    "varlen_prefill_t32768_hq32_hkv8_d128_causal": {
        "source": "fa_prefill.hip",
        "sha256": "9b9b9698dd11d0c43cf794d84c00fd747c7571b8763e1a12d6ef6bd0fe536f5c",
        "fetch_kib": 250547.0, "write_kib": 266269.5},
    "gqa_prefill_window": {
        "source": "fa_prefill.hip",
        "sha256": "9b9b9698dd11d0c43cf794d84c00fd747c7571b8763e1a12d6ef6bd0fe536f5c",
        "fetch_kib": 67555.6, "write_kib": 66560.4},
    "gqa_prefill_b1_hq32_hkv8_n8192_d128_causal_sparse25": {
        "source": "fa_prefill.hip",
        "sha256": "9b9b9698dd11d0c43cf794d84c00fd747c7571b8763e1a12d6ef6bd0fe536f5c",
        "fetch_kib": 74004.6, "write_kib": 70656.1},
    "gqa_prefill_b1_hq32_hkv8_n8192_d128_causal_docmask": {
        "source": "fa_prefill.hip",
        "sha256": "9b9b9698dd11d0c43cf794d84c00fd747c7571b8763e1a12d6ef6bd0fe536f5c",
        "fetch_kib": 54351.9, "write_kib": 74180.9},
    "gqa_prefill_b1_hq32_hkv8_n8192_d128_causal_fp8": {
        "source": "fa_prefill_fp8.hip",
        "sha256": "dab1cbc0965c5dcf285d570693bab4a13bd9ac0427ae06ed6a211b042298aa0c",
        "fetch_kib": 33978.0, "write_kib": 66560.6},
    # the partial kernel (the merge kernel reads the 2 MB of partials)
    "decode_b16_hq32_hkv8_nq1_nk32768_d128": {
        "source": "fa_splitkv.hip",
        "sha256": "cbae59c9b79c3f43b4c024ebe9392a2b2bad2f84acbb2fc164c2e4da4d61511c",
        "fetch_kib": 1048840.5, "write_kib": 2112.0},
    "decode_b16_hq32_hkv8_nq1_nk16384_d256": {
        "source": "fa_splitkv.hip",
        "sha256": "cbae59c9b79c3f43b4c024ebe9392a2b2bad2f84acbb2fc164c2e4da4d61511c",
        "fetch_kib": 1048963.0, "write_kib": 4160.3},
    "decode_window": {
        "source": "fa_splitkv.hip",
        "sha256": "cbae59c9b79c3f43b4c024ebe9392a2b2bad2f84acbb2fc164c2e4da4d61511c",
        "fetch_kib": 132366.0, "write_kib": 2112.0},
    "decode_paged_b16_hq32_hkv8_nq1_nk32768_d128_p256": {
        "source": "fa_splitkv.hip",
        "sha256": "cbae59c9b79c3f43b4c024ebe9392a2b2bad2f84acbb2fc164c2e4da4d61511c",
        "fetch_kib": 1048863.5, "write_kib": 2112.0},
    # the whole fa_bwd call: row preprocessing + dK/dV + dQ kernels
    "gqa_prefill_bwd": {
        "source": "fa_backward.hip",
        "sha256": "ea262dd0d9899bfa6c10edee3451a0dcd920fd2beaa6170ef3d0561d1a661e4d",
        "fetch_kib": 406973.1, "write_kib": 100352.0},
    "gqa_prefill_window_bwd": {
        "source": "fa_backward.hip",
        "sha256": "ea262dd0d9899bfa6c10edee3451a0dcd920fd2beaa6170ef3d0561d1a661e4d",
        "fetch_kib": 298627.6, "write_kib": 100352.5},
}


def kernel_source_hash(source):
    """SHA-256 over a kernel source, the headers every kernel source
    includes (names, lengths and contents) and the compiler flags the
    library build gives that source."""
    import hashlib
    from exact_io_aware_05_amd import build
    h = hashlib.sha256()
    for name in (source, "fa_device.h", "fa_internal.h"):
        path = os.path.join(ROOT, "exact_io_aware_05_amd", "csrc", name)
        with open(path, "rb") as f:
            data = f.read()
        h.update(name.encode() + b"\0" + len(data).to_bytes(8, "little") + data)
    flags = build.hash_flags(build._flags()) + list(build.EXTRA.get(source, []))
    h.update("\0".join(flags).encode())
    return h.hexdigest()


def measured_traffic(name):
    """HBM bytes per launch (counter-based) or None if not measured for the
    current kernel source."""
    rec = MEASURED_TRAFFIC.get(name)
    if rec is None:
        return None
    if kernel_source_hash(rec["source"]) != rec["sha256"]:
        return None
    return int(round((rec["fetch_kib"] * FETCH_SCALE +
                      rec["write_kib"] * WRITE_SCALE) * 1024))


def _dev_tensor(bits):
    import torch
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def _cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _blas_threads():
    """Threads of the BLAS behind numpy (the oracle's matmuls)."""
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("internal_api") in ("openblas", "mkl", "blis")),
                   default=os.cpu_count())
    except Exception:
        return os.cpu_count()


def cpu_baseline(w, q, k, v, budget_s=10.0, do=None, window=None):
    """Oracle TFLOP/s on whole heads of batch 0, one head at a time (the
    gradient oracle when ``do`` is given)."""
    from fa_inputs import bf16_bits_to_f64
    from oracle import reference_attention, reference_attention_backward
    threads = _blas_threads()
    G = w.Hq // w.Hkv
    scale = float(np.float32(w.scale))
    done, t_total = 0, 0.0
    while done < w.Hq and t_total < budget_s:
        h = done
        qh = bf16_bits_to_f64(q[:1, h:h + 1])
        kh = bf16_bits_to_f64(k[:1, h // G:h // G + 1])
        vh = bf16_bits_to_f64(v[:1, h // G:h // G + 1])
        t0 = time.perf_counter()
        if do is None:
            reference_attention(qh, kh, vh, causal=w.causal, scale=scale,
                                window=window)
        else:
            reference_attention_backward(
                qh, kh, vh, bf16_bits_to_f64(do[:1, h:h + 1]),
                causal=w.causal, scale=scale, window=window)
        t_total += time.perf_counter() - t0
        done += 1
    count = attention_fwd_flops if do is None else attention_bwd_flops
    flops = count(1, done, w.Nq, w.Nk, w.d, w.causal)
    if window is not None:
        flops = attention_window_flops(1, done, w.Nq, w.Nk, w.d, w.causal,
                                       window) * (1.0 if do is None else 2.5)
    return {
        "value": round(flops / t_total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "cpu": _cpu_model(),
        "sample": f"{'gradients of ' if do is not None else ''}"
                  f"{done} of {w.B * w.Hq} heads (batch 0, heads 0..{done - 1}), "
                  f"all {w.Nq} query rows each, float64 numpy; {t_total:.1f} s",
    }


def calibrate_copy(mib, steps, warmup):
    """Plain device-to-device copy of a known size: each launch reads and
    writes exactly mib MiB, which calibrates the HBM byte counters."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    print(json.dumps({"calibration": "device copy", "bytes_read": n,
                      "bytes_written": n, "steps": steps,
                      "ms_per_copy": round(ms, 4),
                      "GB/s_read+write": round(2 * n / ms / 1e6, 1)}),
          flush=True)
    return 0


# Untimed load before the warm-up steps, in seconds of wall time.  On a
# fresh process the GPU's clock is not settled: the causal GQA prefill takes
# 544-573 us for its first calls, 596-669 us for calls 4-20 while the power
# manager pulls the clock down, and settles at 503-508 us after about 80 ms
# of load (per-call HIP event times, MI355X).  A few warm-up steps alone would
# time that transient instead of the sustained rate.
SETTLE_S = 0.25
_settle = {"s": SETTLE_S, "steps": 0}


def _emit(out):
    """Print one bench line, with the untimed settle load beside W."""
    line = {}
    for key, val in out.items():
        line[key] = val
        if key == "warmup":
            line["settle"] = {"seconds": _settle["s"], "steps": _settle["steps"]}
    print(json.dumps(line), flush=True)


def _time_steps(step, steps, warmup, stream):
    """Untimed steps for SETTLE_S seconds, W untimed steps, then K steps
    between device synchronisations with one HIP event pair on the launch
    stream: (wall ms, device ms) per step."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < _settle["s"]:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
    _settle["steps"] = n
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, start.elapsed_time(end) / steps


def cpu_baseline_varlen(spec, lens, q, k, v, cu, budget_s=10.0):
    """Oracle TFLOP/s on whole (sequence, head) pairs of the packed batch,
    in order (sequence 0 head 0, head 1, ...), until about 10 s of work."""
    from fa_inputs import bf16_bits_to_f64
    from oracle import reference_attention
    G = spec["Hq"] // spec["Hkv"]
    scale = float(np.float32(spec["scale"]))
    flops, t_total, done = 0.0, 0.0, 0
    pairs = [(b, h) for b in range(len(lens)) for h in range(spec["Hq"])]
    for b, h in pairs:
        if t_total >= budget_s:
            break
        r = slice(int(cu[b]), int(cu[b + 1]))
        qh = bf16_bits_to_f64(q[r, h])[None, None]
        kh = bf16_bits_to_f64(k[r, h // G])[None, None]
        vh = bf16_bits_to_f64(v[r, h // G])[None, None]
        t0 = time.perf_counter()
        reference_attention(qh, kh, vh, causal=spec["causal"], scale=scale)
        t_total += time.perf_counter() - t0
        flops += attention_fwd_flops(1, 1, lens[b], lens[b], spec["d"],
                                     spec["causal"])
        done += 1
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(_blas_threads()), "kind": "oracle",
            "cpu": _cpu_model(),
            "sample": f"{done} of {len(pairs)} (sequence, head) pairs, in "
                      f"order from sequence 0 head 0, float64 numpy; "
                      f"{t_total:.1f} s"}


def bench_varlen(args):
    """One fa_fwd_varlen call over a packed batch of causal prompts."""
    import torch
    from exact_io_aware_05_amd import ops
    spec = VARLEN_PREFILL
    lens = varlen_lengths(spec["total"], spec["lo"], spec["hi"], seed=0)
    q, k, v, cu_q, cu_k = make_varlen(lens, lens, spec["Hq"], spec["Hkv"],
                                      spec["d"], seed=0)
    Q, K, V = _dev_tensor(q), _dev_tensor(k), _dev_tensor(v)
    CQ = torch.from_numpy(cu_q).cuda()
    CK = torch.from_numpy(cu_k).cuda()
    total, Hq, d = Q.shape
    o = torch.empty((total, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Hq, total), dtype=torch.float32, device="cuda")
    mx = max(lens)

    def step():
        ops.fa_fwd_varlen(Q, K, V, CQ, CK, mx, mx, causal=spec["causal"],
                          scale=spec["scale"], o=o, lse=lse)

    ms, kern_ms = _time_steps(step, args.steps, args.warmup,
                              torch.cuda.current_stream())
    flops = sum(attention_fwd_flops(1, Hq, n, n, d, spec["causal"])
                for n in lens)
    achieved = flops / (kern_ms * 1e-3) / 1e12
    out = {
        "metric": f"attn fwd TFLOP/s ({spec['name']})",
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) fp32 rounded to bf16; seeded "
                "log-uniform lengths)",
        "config": {"workload": spec["name"], "B": len(lens), "Hq": Hq,
                   "Hkv": spec["Hkv"], "d": d, "causal": spec["causal"],
                   "scale": spec["scale"], "total_tokens": total,
                   "seqlens": lens, "out_dtype": "bf16",
                   "kernel_ms": round(kern_ms, 4),
                   "pct_bf16_mfma_peak": round(
                       100 * achieved / PEAK_BF16_MFMA_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_MFMA_TFLOPS, 4),
                     "traffic": measured_traffic(spec["name"])},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_varlen(spec, lens, q, k, v, cu_q)
    _emit(out)
    return 0


# the decode workload's shape over a paged cache: 256-key pages, 128 per
# sequence, scattered over the pool (KV-split form)
PAGED_DECODE = dict(name="decode_paged_b16_hq32_hkv8_nq1_nk32768_d128_p256",
                    B=16, Hq=32, Hkv=8, Nq=1, d=128, page_size=256,
                    max_pages=128, causal=False, scale=1.0 / math.sqrt(128))
# the GQA prefill's shape over a paged cache: 8192 queries over their own
# 8192 keys in 32 scattered 256-key pages (prefill form)
PAGED_PREFILL = dict(
    name="gqa_prefill_paged_b1_hq32_hkv8_n8192_d128_causal_p256",
    B=1, Hq=32, Hkv=8, Nq=8192, d=128, page_size=256, max_pages=32,
    causal=True, scale=1.0 / math.sqrt(128))


def bench_paged(args, sp):
    """One fa_fwd_paged call over a shape stored in scattered pages: the
    decode (partial + merge kernels, workspace allocated once), priced at
    its K/V bytes, or the prefill (the tiled kernel reading each block from
    its page), priced at the forward FLOPs."""
    import torch
    from exact_io_aware_05_amd import ops
    B, Hq, Hkv, Nq, d = sp["B"], sp["Hq"], sp["Hkv"], sp["Nq"], sp["d"]
    P, maxp = sp["page_size"], sp["max_pages"]
    Nk = P * maxp
    lens = [Nk] * B
    q, kc, vc, table, sl = make_paged(B, Hq, Hkv, Nq, d, P, maxp, lens, seed=0)
    Q, KC, VC = _dev_tensor(q), _dev_tensor(kc), _dev_tensor(vc)
    del kc, vc
    T = torch.from_numpy(table).cuda()
    SL = torch.from_numpy(sl).cuda()
    splits = ops.paged_num_splits(B, Hq, Hkv, Nq, d, P, maxp)
    ws = torch.empty(max(ops.splitkv_workspace_bytes(B, Hq, Nq, d, splits)
                         if splits else 0, 16),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")

    def step():
        ops.fa_fwd_paged(Q, KC, VC, T, SL, causal=sp["causal"],
                         scale=sp["scale"], o=o, lse=lse, num_splits=splits,
                         workspace=ws)

    ms, kern_ms = _time_steps(step, args.steps, args.warmup,
                              torch.cuda.current_stream())
    data = ("synthetic (seeded N(0,1) fp32 rounded to bf16; seeded page "
            "permutation)")
    config = {"workload": sp["name"], "B": B, "Hq": Hq, "Hkv": Hkv, "Nq": Nq,
              "Nk": Nk, "d": d, "page_size": P, "pages_per_seq": maxp,
              "causal": sp["causal"], "scale": sp["scale"],
              "out_dtype": "bf16", "kv_splits": splits,
              "kernel_ms": round(kern_ms, 4)}
    if splits:
        nbytes = attention_fwd_bytes(B, Hq, Hkv, Nq, Nk, d)
        achieved = nbytes / (kern_ms * 1e-3) / 1e9
        out = {"metric": f"attn decode HBM GB/s ({sp['name']})",
               "value": round(nbytes / (ms * 1e-3) / 1e9, 3), "unit": "GB/s"}
        roof = {"bound": "hbm", "achieved": round(achieved, 2),
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        flops = attention_fwd_flops(B, Hq, Nq, Nk, d, sp["causal"])
        achieved = flops / (kern_ms * 1e-3) / 1e12
        out = {"metric": f"attn fwd TFLOP/s ({sp['name']})",
               "value": round(flops / (ms * 1e-3) / 1e12, 3),
               "unit": "TFLOP/s"}
        roof = {"bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_MFMA_TFLOPS, 4)}
    roof["traffic"] = measured_traffic(sp["name"])
    out.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": round(ms, 4), "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                "data": data, "config": config, "roofline": roof,
                "cpu_baseline": None})
    _emit(out)
    return 0


def bench_fp8(args):
    """One fa_fwd_fp8 call on the GQA prefill's shape with E4M3 inputs
    (per-head descales, V transposed), priced like the bf16 forward and
    held against the FP8 matrix-core peak."""
    import torch
    from exact_io_aware_05_amd import ops
    w = workload(3)
    q8, k8, vt8, qd, kd, vd = make_fp8(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d,
                                       seed=0)
    ldv = (w.Nk + 63) // 64 * 64
    if ldv != w.Nk:
        pad = np.zeros(vt8.shape[:3] + (ldv,), np.uint8)
        pad[..., :w.Nk] = vt8
        vt8 = pad
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    Q, K, VT, QD, KD, VD = t(q8), t(k8), t(vt8), t(qd), t(kd), t(vd)
    o = torch.empty((w.B, w.Hq, w.Nq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")

    def step():
        ops.fa_fwd_fp8(Q, K, VT, QD, KD, VD, causal=w.causal, scale=w.scale,
                       o=o, lse=lse)

    ms, kern_ms = _time_steps(step, args.steps, args.warmup,
                              torch.cuda.current_stream())
    flops = attention_fwd_flops(w.B, w.Hq, w.Nq, w.Nk, w.d, w.causal)
    achieved = flops / (kern_ms * 1e-3) / 1e12
    name = w.name + "_fp8"
    out = {
        "metric": f"attn fwd TFLOP/s ({name})",
        "value": round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
        "data": "synthetic (seeded N(0,1) fp32, per-head amax/448 descale, "
                "rounded to E4M3)",
        "config": {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "causal": w.causal,
                   "scale": w.scale, "out_dtype": "bf16", "v_layout":
                   "transposed [B, Hkv, d, Nk]",
                   "kernel_ms": round(kern_ms, 4),
                   "pct_fp8_mfma_peak": round(100 * achieved /
                                              PEAK_FP8_MFMA_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_FP8_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP8_MFMA_TFLOPS, 4),
                     "traffic": measured_traffic(name)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import reference_attention_fp8
        G = w.Hq // w.Hkv
        t_total, done = 0.0, 0
        while done < w.Hq and t_total < 10.0:
            h = done
            t0 = time.perf_counter()
            reference_attention_fp8(q8[:, h:h + 1], k8[:, h // G:h // G + 1],
                                    vt8[:, h // G:h // G + 1, :, :w.Nk],
                                    qd[:, h:h + 1], kd[:, h // G:h // G + 1],
                                    vd[:, h // G:h // G + 1], causal=w.causal,
                                    scale=float(np.float32(w.scale)))
            t_total += time.perf_counter() - t0
            done += 1
        out["cpu_baseline"] = {
            "value": round(attention_fwd_flops(1, done, w.Nq, w.Nk, w.d,
                                               w.causal) / t_total / 1e12, 6),
            "unit": "TFLOP/s", "cores": int(_blas_threads()), "kind": "oracle",
            "cpu": _cpu_model(),
            "sample": f"{done} of {w.Hq} heads, all {w.Nq} query rows each, "
                      f"float64 numpy on the decoded inputs; {t_total:.1f} s"}
    _emit(out)
    return 0


def bench_sparse(args):
    """One fa_fwd_block_sparse call on the GQA prefill (causal) with a
    block mask keeping a quarter of the 128 x 64 blocks at random plus every
    query block's diagonal blocks, priced at 4 d FLOPs per visible pair of
    the kept blocks."""
    import torch
    from exact_io_aware_05_amd import ops
    w = workload(3)
    q, k, v = make_inputs(w, seed=0)
    bm = sparse_block_mask(w.Hq, w.Nq, w.Nk, 0.25, seed=0)
    Q, K, V = _dev_tensor(q), _dev_tensor(k), _dev_tensor(v)
    M = torch.from_numpy(bm).cuda()
    o = torch.empty((w.B, w.Hq, w.Nq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")

    def step():
        ops.fa_fwd_block_sparse(Q, K, V, M, causal=w.causal, scale=w.scale,
                                o=o, lse=lse)

    ms, kern_ms = _time_steps(step, args.steps, args.warmup,
                              torch.cuda.current_stream())
    counts = block_pair_counts(w.Nq, w.Nk, w.causal, (128, 64))
    pairs = int((bm[0].astype(np.int64) * counts[None]).sum())
    flops = 4.0 * w.d * w.B * pairs
    achieved = flops / (kern_ms * 1e-3) / 1e12
    name = w.name + "_sparse25"
    out = {
        "metric": f"attn fwd TFLOP/s ({name})",
        "value": round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) fp32 rounded to bf16; seeded "
                "block mask)",
        "config": {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "causal": w.causal,
                   "scale": w.scale, "block": [128, 64],
                   "kept_block_fraction": round(float(bm.mean()), 4),
                   "visible_pair_fraction": round(
                       pairs / (w.Hq * float(counts.sum())), 4),
                   "out_dtype": "bf16", "kernel_ms": round(kern_ms, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_MFMA_TFLOPS, 4),
                     "traffic": measured_traffic(name)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from fa_inputs import bf16_bits_to_f64
        from oracle import reference_attention
        G = w.Hq // w.Hkv
        t_total, done, fl = 0.0, 0, 0.0
        while done < w.Hq and t_total < 10.0:
            h = done
            t0 = time.perf_counter()
            reference_attention(bf16_bits_to_f64(q[:1, h:h + 1]),
                                bf16_bits_to_f64(k[:1, h // G:h // G + 1]),
                                bf16_bits_to_f64(v[:1, h // G:h // G + 1]),
                                causal=w.causal,
                                scale=float(np.float32(w.scale)),
                                block_mask=bm[:, h:h + 1],
                                block_size=(128, 64))
            t_total += time.perf_counter() - t0
            fl += 4.0 * w.d * float((bm[0, h].astype(np.int64) * counts).sum())
            done += 1
        out["cpu_baseline"] = {
            "value": round(fl / t_total / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(_blas_threads()), "kind": "oracle",
            "cpu": _cpu_model(),
            "sample": f"{done} of {w.Hq} heads, all {w.Nq} query rows each, "
                      f"float64 numpy; {t_total:.1f} s"}
    _emit(out)
    return 0


DOCMASK_LENS = (300, 2500)


def bench_docmask(args):
    """One fa_fwd_colmask call on the GQA prefill's shape, the tokens split
    into causal documents (a column-interval mask), priced at 4 d FLOPs per
    visible pair."""
    import torch
    from exact_io_aware_05_amd import ops
    w = workload(3)
    q, k, v = make_inputs(w, seed=0)
    lens = random_doc_lens(w.Nk, *DOCMASK_LENS, seed=0)
    cb = np.ascontiguousarray(document_column_bounds(lens)[None])
    Q, K, V = _dev_tensor(q), _dev_tensor(k), _dev_tensor(v)
    CB = torch.from_numpy(cb).cuda()
    o = torch.empty((w.B, w.Hq, w.Nq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")

    def step():
        ops.fa_fwd_colmask(Q, K, V, CB, causal=w.causal, scale=w.scale, o=o,
                           lse=lse)

    ms, kern_ms = _time_steps(step, args.steps, args.warmup,
                              torch.cuda.current_stream())
    pairs = column_mask_pairs(cb[0], w.Nq, w.Nk, w.causal)
    flops = 4.0 * w.d * w.B * w.Hq * pairs
    achieved = flops / (kern_ms * 1e-3) / 1e12
    name = w.name + "_docmask"
    out = {
        "metric": f"attn fwd TFLOP/s ({name})",
        "value": round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) fp32 rounded to bf16; seeded "
                "document lengths)",
        "config": {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "causal": w.causal,
                   "scale": w.scale, "documents": len(lens),
                   "doc_len_range": list(DOCMASK_LENS),
                   "visible_pair_fraction": round(
                       pairs / float(w.Nq * (w.Nq + 1) // 2), 4),
                   "out_dtype": "bf16", "kernel_ms": round(kern_ms, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_MFMA_TFLOPS, 4),
                     "traffic": measured_traffic(name)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from fa_inputs import bf16_bits_to_f64
        from oracle import reference_attention
        G = w.Hq // w.Hkv
        t_total, done = 0.0, 0
        while done < w.Hq and t_total < 10.0:
            h = done
            t0 = time.perf_counter()
            reference_attention(bf16_bits_to_f64(q[:1, h:h + 1]),
                                bf16_bits_to_f64(k[:1, h // G:h // G + 1]),
                                bf16_bits_to_f64(v[:1, h // G:h // G + 1]),
                                causal=w.causal,
                                scale=float(np.float32(w.scale)),
                                col_bounds=cb)
            t_total += time.perf_counter() - t0
            done += 1
        out["cpu_baseline"] = {
            "value": round(4.0 * w.d * pairs * done / t_total / 1e12, 6),
            "unit": "TFLOP/s", "cores": int(_blas_threads()), "kind": "oracle",
            "cpu": _cpu_model(),
            "sample": f"{done} of {w.Hq} heads, all {w.Nq} query rows each, "
                      f"float64 numpy; {t_total:.1f} s"}
    _emit(out)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="gqa_prefill", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle", type=float, default=SETTLE_S, metavar="S",
                    help="seconds of untimed steps before the warm-up steps "
                         "(the GPU clock settles after about 80 ms of load)")
    ap.add_argument("--splits", type=int, default=0,
                    help="decode: KV splits (0: the library's default)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="time a plain device-to-device copy of MIB MiB "
                         "instead (the reference kernel for scaling HBM "
                         "byte counters)")
    args = ap.parse_args(argv)
    _settle["s"] = max(0.0, args.settle)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention forward runs on "
              "one MI355X and no multi-GPU path is built (see DESIGN.md for "
              "how it would shard). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    from exact_io_aware_05_amd import ops

    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy, args.steps, args.warmup)

    if args.workload == "varlen_prefill":
        return bench_varlen(args)
    if args.workload == "decode_paged":
        return bench_paged(args, PAGED_DECODE)
    if args.workload == "gqa_prefill_paged":
        return bench_paged(args, PAGED_PREFILL)
    if args.workload == "gqa_prefill_fp8":
        return bench_fp8(args)
    if args.workload == "gqa_prefill_sparse":
        return bench_sparse(args)
    if args.workload == "gqa_prefill_docmask":
        return bench_docmask(args)
    w = workload(WORKLOADS[args.workload])
    if args.workload in VARIANTS:
        w = dataclasses.replace(w, **VARIANTS[args.workload])
    backward = args.workload.endswith("_bwd")
    window = WINDOWS.get(args.workload)
    q, k, v = make_inputs(w, seed=0)
    Q, K, V = _dev_tensor(q), _dev_tensor(k), _dev_tensor(v)
    o = torch.empty((w.B, w.Hq, w.Nq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    if window is not None and not backward:
        # fa_fwd_window picks the form itself (KV split for a single query,
        # its workspace from the stream-ordered pool)
        splits = 0

        def step():
            ops.fa_fwd_window(Q, K, V, window, causal=w.causal, scale=w.scale,
                              o=o, lse=lse)
    elif w.Nq == 1:
        # single-query decode: the KV-split path with a workspace allocated
        # once, as a serving loop would hold it
        splits = args.splits or ops.default_num_splits(w.B, w.Hq, w.Hkv, w.Nq,
                                                       w.Nk, w.d)
        ws = torch.empty(ops.splitkv_workspace_bytes(w.B, w.Hq, w.Nq, w.d,
                                                     splits),
                         dtype=torch.uint8, device="cuda")

        def step():
            ops.fa_fwd_splitkv(Q, K, V, splits, causal=w.causal, scale=w.scale,
                               o=o, lse=lse, workspace=ws)
    elif backward:
        splits = 0
        do = make_dout(w.B, w.Hq, w.Nq, w.d, seed=0)
        DO = _dev_tensor(do)
        if window is None:
            ops.fa_fwd(Q, K, V, causal=w.causal, scale=w.scale, o=o, lse=lse)
        else:
            ops.fa_fwd_window(Q, K, V, window, causal=w.causal, scale=w.scale,
                              o=o, lse=lse)
        dq = torch.empty_like(Q)
        dk = torch.empty_like(K)
        dv = torch.empty_like(V)
        ws = torch.empty(ops.bwd_workspace_bytes(w.B, w.Hq, w.Nq),
                         dtype=torch.uint8, device="cuda")

        def step():
            ops.fa_bwd(Q, K, V, o, lse, DO, causal=w.causal, scale=w.scale,
                       dq=dq, dk=dk, dv=dv, workspace=ws, window=window)
    else:
        splits = 0

        def step():
            ops.fa_fwd(Q, K, V, causal=w.causal, scale=w.scale, o=o, lse=lse)

    # one HIP event pair on the launch stream around the K timed steps: the
    # average device time of a step, back to back as a real loop runs them
    ms_per_step, kern_ms = _time_steps(step, args.steps, args.warmup, stream)

    count = attention_bwd_flops if backward else attention_fwd_flops
    flops = count(w.B, w.Hq, w.Nq, w.Nk, w.d, w.causal)
    if window is not None:
        flops = attention_window_flops(w.B, w.Hq, w.Nq, w.Nk, w.d, w.causal,
                                       window) * (2.5 if backward else 1.0)
    nbytes = attention_fwd_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)
    if window is not None:   # only the keys some row sees must be read
        nbytes = attention_fwd_bytes(
            w.B, w.Hq, w.Hkv, w.Nq,
            visible_keys(w.Nq, w.Nk, w.causal, window), w.d)
    traffic = measured_traffic(args.workload if (backward or window)
                               else w.name)
    if w.Nq == 1:
        value = nbytes / (ms_per_step * 1e-3) / 1e9
        unit, metric = "GB/s", f"attn decode HBM GB/s ({w.name})"
        if window is not None:
            metric = (f"attn decode HBM GB/s ({w.name}, window {window[0]},"
                      f"{window[1]})")
        achieved = nbytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2),
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        value = flops / (ms_per_step * 1e-3) / 1e12
        if backward:
            metric = f"attn bwd TFLOP/s ({w.name})"
            if window is not None:
                metric = (f"attn bwd TFLOP/s ({w.name}, window {window[0]},"
                          f"{window[1]})")
        elif window is not None:
            metric = (f"attn fwd TFLOP/s ({w.name}, window {window[0]},"
                      f"{window[1]})")
        elif w.name == workload(3).name:
            metric = METRIC
        else:
            metric = f"attn fwd TFLOP/s ({w.name})"
        unit = "TFLOP/s"
        achieved = flops / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_MFMA_TFLOPS, 4),
                "traffic": traffic}

    out = {
        "metric": metric,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) fp32 rounded to bf16)",
        "config": {"workload": w.name + ("_backward" if backward else "") +
                   (f"_window{window[0]}" if window is not None else ""),
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "causal": w.causal,
                   "scale": w.scale,
                   ("grad_dtype" if backward else "out_dtype"): "bf16",
                   "kv_splits": splits if window is None else None,
                   "window": list(window) if window is not None else None,
                   "kernel_ms": round(kern_ms, 4),
                   "pct_bf16_mfma_peak": round(100 * flops / (kern_ms * 1e-3)
                                               / 1e12 / PEAK_BF16_MFMA_TFLOPS, 2)},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v,
                                           do=do if backward else None,
                                           window=window)
        if w.Nq == 1:
            cb = out["cpu_baseline"]
            cb["note"] = "oracle TFLOP/s (decode bytes are not a CPU metric)"
    _emit(out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
