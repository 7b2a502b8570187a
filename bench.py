#!/usr/bin/env python3
"""Benchmark: causal attention forward + backward of one context-parallel
rank on one MI355X.

Default workload (the metric's configuration, workloads.CONFIGS["cp4_rank"]):
rank 0 of a 32768-token causal sequence under CP4 with the dual-chunk
balance, so the rank holds query chunks 0 and 7 (4096 rows each, global
positions kept) and all 32768 keys; 32 heads, QK/V head dims 192/128, bf16
inputs drawn from N(0, 1).  One step = the whole path on one batch:
  * 9 forward partials (query chunk x visible 4096-key block); each one
    after a chunk's first block is merged by LSE into the chunk's fp32
    accumulator in the forward kernel's epilogue (7 merges; the last
    writes the bf16 O),
  * pack + unpack of O and the fp32 LSE into 4 head-group segments,
  * the backward (D, main kernel, dQ written by the dq kernel in one pass)
    over both chunks and all keys.
Inputs are resident in HBM before the timed region starts.

--workload dense8k | thd_gqa | d512 times the other full-size configurations
(B1 H32 S8192 D128; packed THD 32768 tokens Hq32/Hkv8 D128; B1 S16384
Hq16/Hkv4 D512): one step = attn_fwd + attn_bwd on the whole problem.

Prints ONE JSON line.  value = algorithmic TFLOP/s of the whole step:
fwd 2*N_vis*(D_qk+D_v)*H + bwd 2*N_vis*(3*D_qk+2*D_v)*H, N_vis = visible
(query, key) pairs per head (masked work and skipped tiles not counted).
ms_per_step is the timed region over the step count; the per-step times
(HIP events between consecutive steps) give median, p10 and p90.
roofline = the dominant kernel, the backward's key-outer main step (S, dP,
dS, dK, dV: 2*N_vis*(2*D_qk + 2*D_v)*H algorithmic FLOPs), those FLOPs per
launch over its average launch time from HIP events on its own stream.
cpu_baseline = the fp64 oracle on a bounded sample of the same workload.
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
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_kv_kernel_cp4_rank_traffic.md")
KERNEL_SOURCES = ("bwd_causal_flash_amd/csrc/bwd.hip", "bwd_causal_flash_amd/csrc/device_common.h",
                  "bwd_causal_flash_amd/csrc/internal.h")
COPY_BYTES = 512 << 20        # calibration copy: reads and writes this many bytes
WORKLOADS = ("cp4_rank", "dense8k", "thd_gqa", "d512")
MAIN_KERNEL = {"cp4_rank": "bwd_kv_kernel<192,128>", "dense8k": "bwd_kv_kernel<128,128>",
               "thd_gqa": "bwd_kv_kernel<128,128>",
               "d512": "bwd_sdp_kernel<512> + bwd_dkv_kernel<512>"}


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


def cpu_info():
    """CPU model (from /proc/cpuinfo) and the cores this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_baseline(w, x):
    """Time the oracle (fp64 numpy, as it stands) on one head of the
    workload, forward + backward; d512 on the last 2048 query rows of one
    head (they see the most keys).  Returns the contract's object."""
    import numpy as np
    import oracle
    h = 0
    t0 = time.perf_counter()
    if w.layout == "thd":
        used, cu = x["seqused"], x["cu_seqlens"]
        kvh = h // (w.heads_q // w.heads_kv)
        a = [x[n][:, sl].double().numpy() for n, sl in
             (("q", slice(h, h + 1)), ("k", slice(kvh, kvh + 1)), ("v", slice(kvh, kvh + 1)),
              ("do", slice(h, h + 1)))]
        oracle.thd_forward(a[0], a[1], a[2], w.scale, cu, cu, used, used)
        oracle.thd_backward(*a, w.scale, cu, cu, used, used)
        nvis = int(sum(int(n) * (int(n) + 1) // 2 for n in used))
        sample = f"q-head 0 of thd_gqa over all {len(used)} documents"
    else:
        kvh = h // (w.heads_q // w.heads_kv)
        a = [x[n][0, :, sl].double().numpy() for n, sl in
             (("q", slice(h, h + 1)), ("k", slice(kvh, kvh + 1)), ("v", slice(kvh, kvh + 1)),
              ("do", slice(h, h + 1)))]
        if w.name == "cp4_rank":
            from bwd_causal_flash_amd.pipeline import cp_chunks
            qpos = np.concatenate([np.arange(c[2], c[2] + c[1])
                                   for c in cp_chunks(w.seqlen_k, w.cp, w.cp_rank)])
            sample = (f"1 of {w.heads_q} heads of cp4_rank (8192 query rows x 32768 keys, "
                      f"D 192/128)")
        elif w.name == "d512":
            rows = np.arange(w.seqlen_q - 2048, w.seqlen_q)
            a[0], a[3] = a[0][rows], a[3][rows]
            qpos = rows
            sample = f"1 of {w.heads_q} heads of d512, last 2048 query rows x {w.seqlen_k} keys"
        else:
            qpos = np.arange(w.seqlen_q)
            sample = f"1 of {w.heads_q} heads of {w.name} ({w.seqlen_q} rows, D {w.d_qk})"
        oracle.forward(a[0], a[1], a[2], w.scale, qpos)
        oracle.backward(*a, w.scale, qpos)
        nvis = visible_pairs(qpos, w.seqlen_k)
    dt = time.perf_counter() - t0
    f, b = flops(nvis, 1, w.d_qk, w.d_v)
    model, aff = cpu_info()
    return {"value": round((f + b) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads()),
            "kind": "oracle", "sample": f"{sample}, fwd+bwd in fp64 numpy: {dt:.2f} s",
            "cpu_model": model, "affinity_cores": aff}


class SimpleStep:
    """attn_fwd + attn_bwd over a whole problem (dense BSHD or packed THD),
    every buffer and workspace allocated once."""

    def __init__(self, w, x, dev):
        import torch
        import bwd_causal_flash_amd as cpa
        self.cpa = cpa
        bf = torch.bfloat16
        self.q, self.k, self.v, self.dout = (x[n].to(bf).to(dev) for n in ("q", "k", "v", "do"))
        self.scale = w.scale
        self.varlen = None
        if w.layout == "thd":
            used, cu = x["seqused"], x["cu_seqlens"]
            tcu, tused = torch.tensor(cu, device=dev), torch.tensor(used, device=dev)
            self.varlen = cpa.Varlen(tcu, tcu, tused, tused, int(used.max()), int(used.max()))
            self.lse = torch.empty(w.heads_q, w.seqlen_q, dtype=torch.float32, device=dev)
        else:
            self.lse = torch.empty(w.batch, w.heads_q, w.seqlen_q, dtype=torch.float32, device=dev)
        self.o = torch.empty(*self.q.shape[:-1], w.d_v, dtype=bf, device=dev)
        self.dq, self.dk, self.dv = (torch.empty_like(t) for t in (self.q, self.k, self.v))
        self.fwd_ws = torch.empty(256, dtype=torch.uint8, device=dev)
        n = cpa.bwd_workspace_bytes(self.q, self.k, self.v, varlen=self.varlen)
        self.bwd_ws = torch.empty(n, dtype=torch.uint8, device=dev)

    def step(self, stream, main_events=None):
        cpa = self.cpa
        cpa.attn_fwd(self.q, self.k, self.v, self.o, self.lse, scale=self.scale, varlen=self.varlen,
                     workspace=self.fwd_ws, stream=stream)
        # full workspace, one main and one dq: the dq step writes dq itself
        kw = dict(scale=self.scale, varlen=self.varlen, workspace=self.bwd_ws, stream=stream,
                  flags=cpa.CPA_FLAG_DQ_DIRECT)
        args = (self.q, self.k, self.v, self.o, self.dout, self.lse, self.dq, self.dk, self.dv)
        cpa.attn_bwd(*args, step="attn_bwd_pre", **kw)
        if main_events:
            main_events[0].record(stream)
        cpa.attn_bwd(*args, step="attn_bwd_main", **kw)
        if main_events:
            main_events[1].record(stream)
        cpa.attn_bwd(*args, step="attn_bwd_dq", **kw)
        cpa.attn_bwd(*args, step="attn_bwd_post", **kw)


def time_fn(fn, stream, reps):
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def breakdown_cp4(rs, w, x, chunks, stream, dev):
    """Per-phase times of the cp4_rank step and the memory-bound kernels
    alone, with algorithmic GB/s against the HBM peak."""
    import torch
    import bwd_causal_flash_amd as cpa
    out = {}
    out["forward_ms"] = time_fn(lambda: rs.forward(stream), stream, 5)
    out["pack_unpack_ms"] = time_fn(lambda: rs.pack_roundtrip(stream), stream, 10)
    out["backward_ms"] = time_fn(lambda: rs.backward(stream), stream, 5)
    kw = dict(causal=True, scale=rs.scale, q_segments=rs.segments, k_pos_begin=0,
              workspace=rs.bwd_ws, stream=stream)
    args = (rs.q, rs.k, rs.v, rs.o, rs.dout, rs.lse, rs.dq, rs.dk, rs.dv)
    rows_heads = w.seqlen_q * w.heads_q

    def hbm(name, ms, nbytes):
        out[name] = {"ms": round(ms, 4), "bytes": int(nbytes),
                     "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}

    # D = rowsum(dO*O) + zeroed dQ accumulator (+ the tiny tile table): per
    # (row, head) reads 2*D_v*2 B, writes 4 B + D_qk*4 B
    hbm("bwd_pre", time_fn(lambda: cpa.attn_bwd(*args, step="attn_bwd_pre", **kw), stream, 20),
        rows_heads * (2 * w.d_v * 2 + 4 + w.d_qk * 4))
    # dQ = s*acc: reads D_qk*4 B, writes D_qk*2 B per (row, head)
    hbm("bwd_post", time_fn(lambda: cpa.attn_bwd(*args, step="attn_bwd_post", **kw), stream, 20),
        rows_heads * (w.d_qk * 4 + w.d_qk * 2))
    # pack and unpack: O (bf16) + LSE, read and written once each way
    nb = rows_heads * (w.d_v * 2 + 4)
    hbm("pack_saved", time_fn(lambda: cpa.pack_saved(rs.o, rs.lse, rs.pack_groups, rs.pack_buf,
                                                     stream=stream), stream, 20), 2 * nb)
    hbm("unpack_saved", time_fn(lambda: cpa.unpack_saved(rs.pack_buf, rs.o_recv, rs.lse_recv,
                                                         rs.pack_groups, stream=stream),
                                stream, 20), 2 * nb)
    # a ring step's LSE merge alone at this shape: one 4096-row chunk, fp32
    # accumulator and fp32 partial, in place (reads 2 x (D_v*4 + 4) B, writes
    # D_v*4 + 4 B per (row, head))
    c = chunks[1]
    n = c[1]
    g = torch.Generator(device=dev).manual_seed(5)
    o_acc = torch.randn(1, n, w.heads_q, w.d_v, device=dev, generator=g)
    o_part = torch.randn(1, n, w.heads_q, w.d_v, device=dev, generator=g)
    l_acc = torch.randn(1, w.heads_q, n, device=dev, generator=g)
    l_part = torch.randn(1, w.heads_q, n, device=dev, generator=g)
    hbm("attn_merge_lse", time_fn(lambda: cpa.attn_merge_lse(o_acc, l_acc, o_part, l_part,
                                                             stream=stream), stream, 20),
        n * w.heads_q * 3 * (w.d_v * 4 + 4))
    # the backward with smaller workspaces: the keys in bands of 128-key
    # blocks (attn_bwd_workspace_min = one block per band, and a ~2 GiB band)
    full = rs.bwd_ws.numel()
    least = cpa.bwd_workspace_bytes(rs.q, rs.k, rs.v, minimum=True)
    for name, nbytes in (("backward_ws_min", least), ("backward_ws_2GiB", min(full, 2 << 30))):
        ws = rs.bwd_ws[:nbytes]
        kwb = dict(kw, workspace=ws)
        out[name] = {"workspace_bytes": int(nbytes),
                     "ms": round(time_fn(lambda: cpa.attn_bwd(*args, **kwb), stream, 3), 4)}
    out["backward_ws_full"] = {"workspace_bytes": int(full), "ms": round(out["backward_ms"], 4)}
    for k_ in ("forward_ms", "pack_unpack_ms", "backward_ms"):
        out[k_] = round(out[k_], 4)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=WORKLOADS, default="cp4_rank")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true",
                    help="cp4_rank: also time each phase and the memory-bound kernels alone "
                         "(added to the JSON line as 'breakdown')")
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

    w = workloads.CONFIGS[args.workload]
    x = workloads.draw_inputs(w)
    dev = torch.device("cuda:0")
    chunks = None
    if w.name == "cp4_rank":
        from bwd_causal_flash_amd.pipeline import RankStep, cp_chunks
        q, k, v, do = (x[n].to(torch.bfloat16).to(dev) for n in ("q", "k", "v", "do"))
        chunks = cp_chunks(w.seqlen_k, w.cp, w.cp_rank)
        runner = RankStep(q, k, v, do, chunks, w.kv_blocks, scale=w.scale, pack_groups=w.cp)
        qpos = np.concatenate([np.arange(c[2], c[2] + c[1]) for c in chunks])
        nvis = visible_pairs(qpos, w.seqlen_k)
        config = {"workload": "cp4_rank", "seq_len": w.seqlen_k, "cp": w.cp, "rank": w.cp_rank,
                  "q_rows": w.seqlen_q, "kv_blocks": w.kv_blocks, "heads": w.heads_q,
                  "d_qk": w.d_qk, "d_v": w.d_v, "batch": w.batch}
    else:
        runner = SimpleStep(w, x, dev)
        if w.layout == "thd":
            nvis = int(sum(int(n) * (int(n) + 1) // 2 for n in x["seqused"]))
        else:
            nvis = w.batch * w.seqlen_q * (w.seqlen_q + 1) // 2
        config = {"workload": w.name, "layout": w.layout, "batch": w.batch,
                  "seq_len": w.seqlen_q, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                  "d_qk": w.d_qk, "d_v": w.d_v}
        if w.layout == "thd":
            config["documents"] = int(len(x["seqused"]))
    f_fwd, f_bwd = flops(nvis, w.heads_q, w.d_qk, w.d_v)
    f_kv = kv_kernel_flops(nvis, w.heads_q, w.d_qk, w.d_v)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        runner.step(stream)
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
    ev = [(E(), E()) for _ in range(args.steps)]
    marks = [E() for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        marks[i].record(stream)
        runner.step(stream, main_events=ev[i])
    marks[-1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])
    ms_step = marks[0].elapsed_time(marks[-1]) / args.steps
    main_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    achieved = f_kv / (main_ms * 1e-3) / 1e12

    # device memory the step holds: inputs, outputs, partial/accumulator
    # buffers, pack buffers and the backward workspace (the library itself
    # allocates nothing)
    extra = {"peak_device_bytes": int(torch.cuda.max_memory_allocated(dev))}
    if args.breakdown and w.name == "cp4_rank":
        extra["breakdown"] = breakdown_cp4(runner, w, x, chunks, stream, dev)

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)    # one elementwise kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()

    cpu = None if args.no_cpu_baseline else cpu_baseline(w, x)
    config.update({"frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
                   "ms_median": round(float(np.median(step_ms)), 4),
                   "ms_p10": round(float(np.percentile(step_ms, 10)), 4),
                   "ms_p90": round(float(np.percentile(step_ms, 90)), 4),
                   "fwd_tflop": round(f_fwd / 1e12, 4), "bwd_tflop": round(f_bwd / 1e12, 4),
                   "wall_s_timed": round(wall, 3)})
    out = {
        "metric": METRIC if w.name == "cp4_rank" else
        f"causal attn fwd+bwd ms & TFLOP/s (BF16, % MFMA peak), {w.description}",
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
        "config": config,
        "roofline": {"bound": "mfma", "kernel": MAIN_KERNEL[w.name],
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "avg_launch_ms": round(main_ms, 4),
                     "traffic": measured_traffic() if w.name == "cp4_rank" else None},
        "cpu_baseline": cpu,
        **extra,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
