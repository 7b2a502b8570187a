#!/usr/bin/env python3
"""Benchmark: causal attention forward + backward of one context-parallel
rank on one MI355X.

Workload (the metric's configuration, workloads.CONFIGS["cp4_rank"]): rank 0
of a 32768-token causal sequence under CP4 with the dual-chunk balance, so
the rank holds query chunks 0 and 7 (4096 rows each, global positions kept)
and all 32768 keys; 32 heads, QK/V head dims 192/128, bf16 inputs drawn from
N(0, 1).  One step = the whole path on one batch:
  * 9 forward partials (query chunk x visible 4096-key block); each one
    after a chunk's first block is merged by LSE into the chunk's fp32
    accumulator in the forward kernel's epilogue (7 merges; the last
    writes the bf16 O),
  * pack + unpack of O and the fp32 LSE into 4 head-group segments,
  * the backward (D, main kernel, dQ cast) over both chunks and all keys.
Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line.  value = algorithmic TFLOP/s of the whole step:
fwd 2*N_vis*(D_qk+D_v)*H + bwd 2*N_vis*(3*D_qk+2*D_v)*H, N_vis = visible
(query, key) pairs per head (masked work and skipped tiles not counted).
roofline = the dominant kernel (the backward's key-outer kernel, which forms
S, dP, dS and accumulates dK, dV: 2*N_vis*(2*D_qk + 2*D_v)*H algorithmic
FLOPs), those FLOPs per launch over its average launch time from HIP events
on its own stream.  (dQ = dS K runs in a separate query-outer kernel.)
cpu_baseline = the fp64 oracle on one head of the same workload.
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

METRIC = "causal attn fwd+bwd ms & TFLOP/s (BF16, % MFMA peak), 32K-seq CP4 rank shape"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_kv_kernel_cp4_rank_traffic.md")
KERNEL_SOURCES = ("bwd_causal_flash_amd/csrc/bwd.hip", "bwd_causal_flash_amd/csrc/device_common.h",
                  "bwd_causal_flash_amd/csrc/internal.h")
COPY_BYTES = 512 << 20        # calibration copy: reads and writes this many bytes


def visible_pairs(q_positions, n_keys):
    """Visible (query, key) pairs per head when key j has position j."""
    import numpy as np
    p = np.asarray(q_positions, dtype=np.int64)
    return int(np.minimum(np.maximum(p + 1, 0), n_keys).sum())


def flops(nvis, heads, dqk, dv):
    return 2.0 * nvis * (dqk + dv) * heads, 2.0 * nvis * (3 * dqk + 2 * dv) * heads


def kv_kernel_flops(nvis, heads, dqk, dv):
    """S = Q K^T, dP = dO V^T, dV += P^T dO, dK += dS^T Q."""
    return 2.0 * nvis * (2 * dqk + 2 * dv) * heads


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the key-outer backward kernel, from the
    committed rocprofv3 counter summary, or None when that summary is
    missing or was taken on different kernel sources."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if ":" in line and line.strip().startswith(("source_sha256", "traffic_bytes_per_launch")):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip().strip("`")
        if fields.get("source_sha256") != kernel_source_hash():
            return None
        return int(float(fields["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(w, x, qpos):
    """Time the oracle (fp64 numpy, as it stands) on one head, fwd + bwd."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    h = 0
    a = [x[n][0, :, h:h + 1].double().numpy() for n in ("q", "k", "v", "do")]
    t0 = time.perf_counter()
    oracle.forward(a[0], a[1], a[2], w.scale, qpos)
    oracle.backward(*a, w.scale, qpos)
    dt = time.perf_counter() - t0
    nvis = visible_pairs(qpos, w.seqlen_k)
    f, b = flops(nvis, 1, w.d_qk, w.d_v)
    return {"value": round((f + b) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"1 of {w.heads_q} heads of cp4_rank (8192 query rows x 32768 keys, "
                      f"D 192/128), fwd+bwd in fp64 numpy: {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true",
                    help="also print per-phase times (stderr)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a plain elementwise copy of a known size "
                         "(for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: this library "
              "has no collectives and multi-GPU runs are out of scope", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads
    from bwd_causal_flash_amd.pipeline import RankStep, cp_chunks
    import oracle  # noqa: F401  (cpu baseline only)

    w = workloads.CONFIGS["cp4_rank"]
    x = workloads.draw_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(torch.bfloat16).to(dev) for n in ("q", "k", "v", "do"))
    chunks = cp_chunks(w.seqlen_k, w.cp, w.cp_rank)
    rs = RankStep(q, k, v, do, chunks, w.kv_blocks, scale=w.scale, pack_groups=w.cp)
    qpos = np.concatenate([np.arange(c[2], c[2] + c[1]) for c in chunks])
    nvis = visible_pairs(qpos, w.seqlen_k)
    f_fwd, f_bwd = flops(nvis, w.heads_q, w.d_qk, w.d_v)
    f_kv = kv_kernel_flops(nvis, w.heads_q, w.d_qk, w.d_v)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        rs.step(stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        rs.step(stream, main_events=ev[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    main_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    achieved = f_kv / (main_ms * 1e-3) / 1e12

    if args.breakdown:
        phases = {}
        for name, fn in (("forward(9 partials, 7 merged in the epilogue)", lambda: rs.forward(stream)),
                         ("pack+unpack", lambda: rs.pack_roundtrip(stream)),
                         ("backward(pre+main+dq+post)", lambda: rs.backward(stream))):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(5):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            phases[name] = round(a.elapsed_time(b) / 5, 4)
        # head-parallel exchange buffer: this rank's Q, K, V, O, dO rows and LSE
        # packed seq -> heads into 4 head-group segments (and unpacked back)
        import bwd_causal_flash_amd as cpa
        rows = torch.cat([torch.arange(c[0], c[0] + c[1]) for c in chunks]).to(dev)
        kpos = torch.cat([torch.arange(c[2], c[2] + c[1]) for c in chunks]).to(dev)
        fields = [rs.q, k[:, kpos].contiguous(), v[:, kpos].contiguous(), rs.o, rs.dout,
                  rs.lse]
        every = [[(0, int(rows.numel()))]] * w.cp
        xbuf = cpa.xchg_pack(fields, groups=w.cp, ranges=every, split=True, stream=stream)
        outs = [torch.empty_like(f) for f in fields]
        for name, fn in (("xchg_pack", lambda: cpa.xchg_pack(fields, groups=w.cp, ranges=every,
                                                             split=True, buf=xbuf, stream=stream)),
                         ("xchg_unpack", lambda: cpa.xchg_unpack(xbuf, outs, groups=w.cp,
                                                                 ranges=every, split=True,
                                                                 stream=stream))):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(10):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / 10
            phases[name] = round(ms, 4)
            phases[name + "_GBps(read+write)"] = round(2 * xbuf.numel() / (ms * 1e-3) / 1e9, 1)
        print(json.dumps({"phase_ms": phases, "main_ms": round(main_ms, 4),
                          "fwd_tflops": round(f_fwd / 1e12, 4),
                          "bwd_tflops": round(f_bwd / 1e12, 4)}), file=sys.stderr)

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)    # one elementwise kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()

    cpu = None if args.no_cpu_baseline else cpu_baseline(w, x, qpos)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "cp4_rank", "seq_len": w.seqlen_k, "cp": w.cp,
                   "rank": w.cp_rank, "q_rows": w.seqlen_q, "kv_blocks": w.kv_blocks,
                   "heads": w.heads_q, "d_qk": w.d_qk, "d_v": w.d_v, "batch": w.batch,
                   "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
                   "wall_s_timed": round(wall, 3)},
        "roofline": {"bound": "mfma", "kernel": "bwd_kv_kernel<192,128>",
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "avg_launch_ms": round(main_ms, 4), "traffic": measured_traffic()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
