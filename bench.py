#!/usr/bin/env python3
"""Throughput of the block-sparse prefill path on one MI355X.

A step is one pass of the whole sparse path over one batch of synthetic input:
seer_build_mask (TopK on the fp32 block scores) followed by seer_sparse_prefill
(schedule + block-sparse flash attention), on the 32k-token Llama-3.1-8B
attention shape at density 0.1 with inputs already resident in HBM.

The headline value is computed-block TFLOP/s: every listed 64x64 tile counts
4*64*64*D FLOP (a diagonal tile counts whole, since it is computed).  The JSON
line also carries the roofline of the dominant call, the CPU oracle timed on a
bounded sample of the same workload, the speedup over the same kernel at
density 1.0, and the pooled-map pass on the Qwen2.5-32B shape.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PMC_FILE = os.path.join(ROOT, "profiles", "sparse_prefill_kernel_llama8b_t32768_d0.1_pmc.txt")
KERNEL_SOURCE = os.path.join(ROOT, "block_sparse_attention_prefill_amd", "csrc", "attention.hip")


def log(msg: str) -> None:
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def tile_flops(d: int) -> int:
    return 4 * 64 * 64 * d


def source_digest() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(launch_s: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    if absent or taken on a different kernel source."""
    if not os.path.exists(PMC_FILE):
        return None
    vals = {}
    with open(PMC_FILE) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                key, _, val = line.partition(":")
                vals[key.strip()] = val.strip()
    if vals.get("kernel_source_sha256_16") != source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_calls(fn, n: int, torch, flush=None):
    """Mean duration (ms) of fn() over n calls, bracketed by events on torch's
    current stream -- the stream the library launches on.  With `flush` (a 1 GiB
    fp32 device buffer) it is read before each call, outside the events, so that
    the call starts with L2 and MALL holding other, clean data (a write would
    leave dirty lines whose write-back the call would pay for)."""
    evs = []
    for _ in range(n):
        if flush is not None:
            flush.sum()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    return statistics.mean(a.elapsed_time(b) for a, b in evs)


def settle(fn, torch, seconds: float = 0.1, max_calls: int = 400) -> None:
    """Untimed calls of fn for about `seconds` of GPU time, so that the calls timed
    next run at the clock the socket power controller holds under this load (it
    moves the clock for a few tens of ms after the load changes)."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    one = max(a.elapsed_time(b) * 1e-3, 1e-6)
    for _ in range(min(max_calls, int(seconds / one))):
        fn()
    torch.cuda.synchronize()


def call_stats(fn, n: int, torch, flush=None) -> dict:
    """Median, min and max duration (ms) of fn() over n calls, timed as in
    time_calls."""
    evs = []
    for _ in range(n):
        if flush is not None:
            flush.sum()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in evs]
    return {"median": round(statistics.median(ts), 4), "min": round(min(ts), 4),
            "max": round(max(ts), 4), "calls": n}


def device_info(torch) -> dict:
    """Compute units and the clock the runtime reports for device 0."""
    import ctypes
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        # hipDeviceAttributeClockRate: peak shader clock in kHz
        attr = 5
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, 0) == 0 and v.value > 0:
            info["peak_clock_mhz"] = round(v.value / 1000)
    except OSError:
        pass
    return info


def cpu_baseline(w, q, k, v, scores, max_k, blocks_per_head: int):
    import numpy as np

    import oracle
    from block_sparse_attention_prefill_amd import workloads as wl

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    rows = wl.sample_qblocks(w, blocks_per_head)
    t0 = time.perf_counter()
    lists = oracle.mask_rows_ref(scores.numpy(), rows, w.mode, w.threshold, w.density,
                                 w.keep_sink, max_k)
    idx = np.full((w.batch, w.hq, w.nqb, max_k), -1, np.int32)
    cnt = np.zeros((w.batch, w.hq, w.nqb), np.int32)
    for (b, h, i), sel in lists.items():
        idx[b, h, i, : len(sel)] = sel
        cnt[b, h, i] = len(sel)
    oracle.sparse_attention_blocks_ref(q, k, v, idx, cnt, None, rows)
    dt = time.perf_counter() - t0
    flops = int(cnt.sum()) * tile_flops(w.head_dim)
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{len(rows)} seeded query blocks ({blocks_per_head} per head incl. first and "
                   f"last) of {w.name}: mask rows + fp64 attention, {dt:.1f} s"),
    }


def clock_during(fn, torch, seconds: float = 2.5, settle: float = 1.5) -> dict:
    """Shader clock and socket power while fn() runs back to back on the GPU: the
    calling thread keeps launching fn() for `seconds` while a second thread reads
    the AMD SMI GPU metrics (current gfx clock of each XCD, socket power) every
    5 ms; readings from the first `settle` seconds are dropped (the metrics lag
    the load by up to about a second).  The 2516.6
    TFLOP/s peak assumes the 2400 MHz peak clock; under a sustained MFMA load the
    clock settles lower, at the power cap."""
    import threading
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as e:  # pragma: no cover - telemetry is optional
        return {"error": f"amdsmi unavailable: {e}"}
    fn()
    torch.cuda.synchronize()
    stop = threading.Event()
    samples = []

    def sample():
        t0 = time.perf_counter()
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            except Exception:  # pragma: no cover
                break
            xs = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int) and c < 65535]
            p = m.get("current_socket_power")
            samples.append((time.perf_counter() - t0, statistics.mean(xs) if xs else None,
                            float(p) if isinstance(p, (int, float)) else None))
            time.sleep(0.005)

    th = threading.Thread(target=sample, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        fn()
    launched = time.perf_counter() - t0
    torch.cuda.synchronize()
    stop.set()
    th.join()
    busy = [x for x in samples if settle <= x[0] <= launched]
    clocks = [c for _, c, _ in busy if c is not None]
    powers = [p for _, _, p in busy if p is not None]
    out = {"samples": len(busy)}
    if clocks:
        out["gfx_clock_mhz"] = round(statistics.median(clocks), 1)
    if powers:
        out["socket_power_w"] = round(statistics.median(powers), 1)
    try:
        out["power_cap_w"] = round(amdsmi.amdsmi_get_power_cap_info(h)["power_cap"] / 1e6, 1)
    except Exception:  # pragma: no cover
        pass
    return out


def sparse_config_line(seer, wl, torch, dev, w, args) -> dict:
    """One workload through seer_build_mask + seer_sparse_prefill: mask and prefill
    time (mean of per-call events), computed-tile TFLOP/s and fraction of the bf16
    peak, and the same kernel with every causal block listed (density 1.0)."""
    log(f"[bench] {w.name}")
    q, k, v = (t.to(dev) for t in wl.make_qkv(w))
    sd = wl.make_scores(w).to(dev)
    max_k = seer.topk_budget(w.nqb, w.density, w.keep_sink) if w.mode == wl.MODE_TOPK else w.nqb
    idx = torch.empty((w.batch, w.hq, w.nqb, max_k), dtype=torch.int32, device=dev)
    cnt = torch.empty((w.batch, w.hq, w.nqb), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    ws = torch.empty((seer.sparse_prefill_workspace_size(w.batch, w.hq, w.hkv, w.seq),),
                     dtype=torch.uint8, device=dev)
    mask = lambda: seer.seer_build_mask(sd, w.mode, w.threshold, w.density, w.keep_sink, max_k,
                                        kv_idx=idx, kv_cnt=cnt)
    pre = lambda: seer.seer_sparse_prefill(q, k, v, idx, cnt, out=out, workspace=ws)
    mask()
    settle(pre, torch)
    n = max(3, args.steps // 2)
    settle(mask, torch)
    m_ms = time_calls(mask, n, torch)
    settle(pre, torch)
    p_ms = time_calls(pre, n, torch)
    blocks = int(cnt.sum().item())
    tf = blocks * tile_flops(w.head_dim) / (p_ms * 1e-3) / 1e12
    res = {
        "mask": "topk" if w.mode == wl.MODE_TOPK else "threshold",
        "density": w.density if w.mode == wl.MODE_TOPK else None,
        "threshold": w.threshold if w.mode == wl.MODE_THRESHOLD else None,
        "keep_sink": w.keep_sink, "seq_len": w.seq, "q_heads": w.hq, "kv_heads": w.hkv,
        "head_dim": w.head_dim, "computed_blocks": blocks,
        "density_eff": round(blocks / (w.batch * w.hq * w.nqb * (w.nqb + 1) / 2), 5),
        "mask_build_ms": round(m_ms, 4), "sparse_prefill_ms": round(p_ms, 4),
        "tflops": round(tf, 3), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
    }
    del idx
    idx1 = torch.empty((w.batch, w.hq, w.nqb, w.nqb), dtype=torch.int32, device=dev)
    seer.seer_build_mask(sd, wl.MODE_TOPK, 0.0, 1.0, w.keep_sink, w.nqb, kv_idx=idx1, kv_cnt=cnt)
    call1 = lambda: seer.seer_sparse_prefill(q, k, v, idx1, cnt, out=out, workspace=ws)
    settle(call1, torch)
    d_ms = time_calls(call1, max(2, args.steps // 5), torch)
    blocks1 = int(cnt.sum().item())
    res["density1"] = {
        "prefill_ms": round(d_ms, 4),
        "tflops": round(blocks1 * tile_flops(w.head_dim) / (d_ms * 1e-3) / 1e12, 3),
        "speedup": round(d_ms / p_ms, 3), "ideal_speedup": round(blocks1 / blocks, 3)}
    del q, k, v, sd, idx1, cnt, out, ws
    torch.cuda.empty_cache()
    return res


def cpu_oracle_extrapolated(w, blocks_per_head: int) -> dict:
    """The oracle (as is) on `blocks_per_head` seeded sampled query blocks per head
    of w, and that time scaled by the ratio of computed blocks of the whole
    workload to those of the sample (an extrapolation, labelled as such)."""
    import numpy as np

    import oracle
    from block_sparse_attention_prefill_amd import workloads as wl

    q, k, v = wl.make_qkv(w)
    scores = wl.make_scores(w).numpy()
    max_k = oracle.topk_count(w.nqb - 1, w.density, w.keep_sink)
    rows = wl.sample_qblocks(w, blocks_per_head)
    t0 = time.perf_counter()
    lists = oracle.mask_rows_ref(scores, rows, w.mode, w.threshold, w.density, w.keep_sink,
                                 max_k)
    idx = np.full((w.batch, w.hq, w.nqb, max_k), -1, np.int32)
    cnt = np.zeros((w.batch, w.hq, w.nqb), np.int32)
    for (b, h, i), sel in lists.items():
        idx[b, h, i, : len(sel)] = sel
        cnt[b, h, i] = len(sel)
    oracle.sparse_attention_blocks_ref(q, k, v, idx, cnt, None, rows)
    dt = time.perf_counter() - t0
    sample_blocks = int(cnt.sum())
    total_blocks = sum(oracle.topk_count(i, w.density, w.keep_sink) for i in range(w.nqb)) \
        * w.batch * w.hq
    return {"sample": f"{len(rows)} seeded query blocks ({blocks_per_head} per head)",
            "sample_s": round(dt, 2), "sample_blocks": sample_blocks,
            "tflops": round(sample_blocks * tile_flops(w.head_dim) / dt / 1e12, 6),
            "extrapolated_full_s": round(dt * total_blocks / sample_blocks, 1),
            "extrapolation": "sample time x (computed blocks of the workload / of the sample)"}


def decode_bench(seer, wl, torch, dev, args):
    import dataclasses
    import numpy as np
    dw = wl.DEC1
    log(f"[bench] decode {dw.name}")
    q, k, v, kv_len = wl.make_decode_inputs(dw)
    qd, kd, vd, ld = (t.to(dev) for t in (q, k, v, kv_len))
    del q, k, v
    od = torch.empty_like(qd)
    out = {"workload": dw.name, "batch": dw.batch, "kv_len": dw.kv_lens[0], "block": dw.block,
           "budget_tokens": dw.budget_tokens, "hbm_peak_gbps": 8000.0}
    d, g = dw.head_dim, dw.hq // dw.hkv
    flush = torch.ones((1 << 28,), dtype=torch.float32, device=dev)  # 1 GiB > L2 + 256 MB MALL
    # The per-token gate over the same cache (Dg 128, seeded weights): gate keys of every
    # block once, then per step the keys of each sequence's last block and the new
    # tokens' block scores (the input of the decode mask build).
    wq, wk = (t.to(dev) for t in wl.make_gate_weights(wl.WORKLOADS[3], 128))  # 32/8/128 weights
    gsc = torch.empty((dw.batch, dw.hq, dw.nkb), dtype=torch.float32, device=dev)
    gws = torch.empty((seer.attn_gate_decode_keys_workspace_size(dw.batch, dw.hkv, dw.tmax, d,
                                                                 dw.block),),
                      dtype=torch.uint8, device=dev)
    kg = seer.seer_attn_gate_decode_keys(kd, ld, wk, dw.block, workspace=gws)
    kall = lambda: seer.seer_attn_gate_decode_keys(kd, ld, wk, dw.block, k_gate=kg, workspace=gws)
    kstep = lambda: (seer.seer_attn_gate_decode_keys(kd, ld, wk, dw.block, last_block_only=True,
                                                     k_gate=kg),
                     seer.seer_attn_gate_decode_scores(qd, kg, ld, wq, dw.tmax, dw.block,
                                                       scores=gsc))
    kstep()
    out["gate_keys_all_blocks_ms"] = round(time_calls(kall, max(3, args.steps // 2), torch,
                                                      flush), 4)
    out["gate_step_ms"] = round(time_calls(kstep, max(5, args.steps), torch, flush), 4)
    # Gate step through to per-query-head lists: keys of the last blocks, then scores
    # and the mask build as two calls, or the one-pass scores-to-lists call.
    dv = wl.DEC2
    gmax_k = min(dv.nkb, max(dv.k_blocks, 2))
    gidx, gcnt = seer.seer_build_mask_decode(gsc, ld, dv.block, wl.MODE_TOPK, 0.0, dv.k_blocks,
                                             dv.keep_sink, gmax_k)
    two = lambda: (kstep(), seer.seer_build_mask_decode(
        gsc, ld, dv.block, wl.MODE_TOPK, 0.0, dv.k_blocks, dv.keep_sink, gmax_k, kv_idx=gidx,
        kv_cnt=gcnt))
    one = lambda: (seer.seer_attn_gate_decode_keys(kd, ld, wk, dw.block, last_block_only=True,
                                                   k_gate=kg),
                   seer.seer_attn_gate_decode_mask(qd, kg, ld, wq, dw.tmax, wl.MODE_TOPK, 0.0,
                                                   dv.k_blocks, dv.keep_sink, gmax_k, dw.block,
                                                   kv_idx=gidx, kv_cnt=gcnt))
    one()
    out["gate_to_lists_two_call_ms"] = round(time_calls(two, max(5, args.steps), torch, flush),
                                             4)
    out["gate_to_lists_fused_ms"] = round(time_calls(one, max(5, args.steps), torch, flush), 4)
    del wq, wk, gsc, gws, kg, gidx, gcnt
    for var in (dw, wl.DEC2):
        sc = wl.make_decode_scores(var).to(dev)
        max_k = min(var.nkb, max(var.k_blocks, 2))
        idx, cnt = seer.seer_build_mask_decode(sc, ld, var.block, wl.MODE_TOPK, 0.0, var.k_blocks,
                                               var.keep_sink, max_k)
        mcall = lambda: seer.seer_build_mask_decode(sc, ld, var.block, wl.MODE_TOPK, 0.0,
                                                    var.k_blocks, var.keep_sink, max_k,
                                                    kv_idx=idx, kv_cnt=cnt)
        wsd = torch.empty((seer.sparse_decode_workspace_size(
            dw.batch, dw.hq, dw.hkv, dw.tmax, d, var.lh, max_k, var.block),),
            dtype=torch.uint8, device=dev)
        call = lambda: seer.seer_sparse_decode(qd, kd, vd, ld, idx, cnt, var.block, out=od,
                                               workspace=wsd)
        call()
        m_ms = time_calls(mcall, max(5, args.steps), torch, flush)
        d_ms = time_calls(call, max(5, args.steps), torch, flush)
        # Blocks each KV group reads: the union of its heads' lists.
        ii, cc = idx.cpu().numpy(), cnt.cpu().numpy()
        tokens = 0
        for b in range(dw.batch):
            for grp in range(dw.hkv):
                heads = range(grp * g, grp * g + g) if var.lh == dw.hq else [grp]
                blocks = {int(j) for h in heads for j in ii[b, h, : cc[b, h]]}
                tokens += sum(min(var.block, dw.kv_lens[b] - j * var.block) for j in blocks)
        nbytes = tokens * d * 2 * 2 + 2 * 2 * qd.numel() + 4 * (idx.numel() + cnt.numel())
        key = "lists_per_kv_head" if var.lh == dw.hkv else "lists_per_q_head"
        out[key] = {"mask_ms": round(m_ms, 4), "decode_ms": round(d_ms, 4),
                    "algorithmic_bytes": nbytes,
                    "gbps": round(nbytes / (d_ms * 1e-3) / 1e9, 1)}
        del sc, idx, cnt, wsd
    # The same kernel with every block listed (dense decode) for the speedup.
    dense = dataclasses.replace(dw, wid=13)
    nkb = dense.nkb
    idx = torch.arange(nkb, dtype=torch.int32, device=dev).repeat(dw.batch, dw.hkv, 1).contiguous()
    cnt = torch.full((dw.batch, dw.hkv), nkb, dtype=torch.int32, device=dev)
    wsd = torch.empty((seer.sparse_decode_workspace_size(dw.batch, dw.hq, dw.hkv, dw.tmax, d,
                                                         dw.hkv, nkb, dw.block),),
                      dtype=torch.uint8, device=dev)
    call = lambda: seer.seer_sparse_decode(qd, kd, vd, ld, idx, cnt, dw.block, out=od,
                                           workspace=wsd)
    call()
    dn_ms = time_calls(call, max(3, args.steps // 2), torch, flush)
    dn_bytes = sum(dw.kv_lens) * dw.hkv * d * 2 * 2 + 2 * 2 * qd.numel()
    out["dense"] = {"decode_ms": round(dn_ms, 4),
                    "gbps": round(dn_bytes / (dn_ms * 1e-3) / 1e9, 1)}
    out["speedup_vs_dense"] = round(dn_ms / out["lists_per_kv_head"]["decode_ms"], 3)
    del qd, kd, vd, ld, od, idx, cnt, wsd, flush
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first: the power controller settles within about 0.1 s")
    ap.add_argument("--workload", type=int, default=3, help="workload id (default 3: 32k, density 0.1)")
    ap.add_argument("--cpu-blocks-per-head", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the density-1.0 and pooled-map measurements")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run one plain device copy of this many MiB (to scale HBM "
                         "byte counters) and exit")
    ap.add_argument("--decode-only", action="store_true",
                    help="only run the sparse decode measurement and print it as JSON")
    args = ap.parse_args(argv)

    if args.copy_calibration_mib:
        import torch
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}), flush=True)
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by KV head with no exchange; see the design notes)",
              file=sys.stderr)
        return 2

    import torch

    import block_sparse_attention_prefill_amd as seer
    from block_sparse_attention_prefill_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    seer.load()
    dev = torch.device("cuda:0")
    if args.decode_only:
        print(json.dumps({"decode": decode_bench(seer, wl, torch, dev, args)}), flush=True)
        return 0
    w = wl.WORKLOADS[args.workload]
    assert w.kind == "sparse"
    log(f"[bench] generating {w.name}")
    q, k, v = wl.make_qkv(w)
    scores = wl.make_scores(w)
    qd, kd, vd, sd = (t.to(dev) for t in (q, k, v, scores))
    max_k = seer.topk_budget(w.nqb, w.density, w.keep_sink) if w.mode == wl.MODE_TOPK else w.nqb
    idx = torch.empty((w.batch, w.hq, w.nqb, max_k), dtype=torch.int32, device=dev)
    cnt = torch.empty((w.batch, w.hq, w.nqb), dtype=torch.int32, device=dev)
    out = torch.empty_like(qd)
    ws = torch.empty((seer.sparse_prefill_workspace_size(w.batch, w.hq, w.hkv, w.seq),),
                     dtype=torch.uint8, device=dev)

    def build_mask():
        seer.seer_build_mask(sd, w.mode, w.threshold, w.density, w.keep_sink, max_k,
                             kv_idx=idx, kv_cnt=cnt)

    def prefill():
        seer.seer_sparse_prefill(qd, kd, vd, idx, cnt, out=out, workspace=ws)

    for _ in range(args.warmup):
        build_mask()
        prefill()
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    # The steps of `value`: nothing but the calls between the two synchronisations.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        build_mask()
        prefill()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # The same steps again with HIP events around each call (the per-call times and
    # the roofline); the event records themselves take a little GPU time.
    ev_mask, ev_pre = [], []
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        build_mask()
        e[1].record()
        prefill()
        e[2].record()
        ev_mask.append((e[0], e[1]))
        ev_pre.append((e[1], e[2]))
    torch.cuda.synchronize()
    mask_ms = statistics.mean(a.elapsed_time(b) for a, b in ev_mask)
    pre_ms = statistics.mean(a.elapsed_time(b) for a, b in ev_pre)

    blocks = int(cnt.sum().item())
    flops = blocks * tile_flops(w.head_dim)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (pre_ms * 1e-3) / 1e12
    causal_exact = (blocks - w.batch * w.hq * w.nqb * 0.5) * tile_flops(w.head_dim)
    traffic = read_traffic(pre_ms * 1e-3)
    algo_bytes = (qd.numel() * 2 * 2 + kd.numel() * 2 * 2 + idx.numel() * 4 + cnt.numel() * 4)

    result = {
        "metric": "sparse-prefill attention TFLOP/s (computed blocks) & % bf16 MFMA peak, 32k",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, local+stripe block scores)",
        "config": {
            "workload": w.name, "batch": w.batch, "q_heads": w.hq, "kv_heads": w.hkv,
            "head_dim": w.head_dim, "seq_len": w.seq, "block": 64, "mask": "topk",
            "density": w.density, "keep_sink": w.keep_sink, "computed_blocks": blocks,
            "density_eff": round(blocks / (w.batch * w.hq * w.nqb * (w.nqb + 1) / 2), 5),
        },
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "mask_build_ms": round(mask_ms, 4),
        "sparse_prefill_ms": round(pre_ms, 4),
        "sparse_prefill_call_ms": {
            "median": round(statistics.median(a.elapsed_time(b) for a, b in ev_pre), 4),
            "min": round(min(a.elapsed_time(b) for a, b in ev_pre), 4),
            "max": round(max(a.elapsed_time(b) for a, b in ev_pre), 4)},
        "device": device_info(torch),
        "causal_exact_tflops": round(causal_exact / (ms_per_step * 1e-3) / 1e12, 3),
        "roofline": {
            "kernel": "seer_sparse_prefill (schedule + sparse_prefill_kernel)",
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_hbm_bytes": algo_bytes,
        },
    }

    # Shader clock and socket power during sustained prefill calls (not timed).
    log("[bench] clock during sustained prefill")
    clk = clock_during(prefill, torch)
    result["clock_during_prefill"] = clk
    if "gfx_clock_mhz" in clk:
        peak_at = PEAK_BF16_TFLOPS * clk["gfx_clock_mhz"] / 2400.0
        result["roofline"]["frac_at_measured_clock"] = round(achieved / peak_at, 4)

    if not args.no_extras:
        # The prefill call with L2 and the 256 MB MALL flushed before each call (a
        # 1 GiB read), so that K/V start in HBM: median, min and max.
        log("[bench] flushed prefill calls")
        flush = torch.ones((1 << 28,), dtype=torch.float32, device=dev)
        result["sparse_prefill_flushed_ms"] = call_stats(prefill, max(20, args.steps), torch,
                                                         flush)
        del flush

        # Same kernel at density 1.0 (every causal block listed).
        log("[bench] density 1.0 reference")
        idx1 = torch.empty((w.batch, w.hq, w.nqb, w.nqb), dtype=torch.int32, device=dev)
        cnt1 = torch.empty((w.batch, w.hq, w.nqb), dtype=torch.int32, device=dev)
        seer.seer_build_mask(sd, wl.MODE_TOPK, 0.0, 1.0, w.keep_sink, w.nqb, kv_idx=idx1,
                             kv_cnt=cnt1)
        dense = lambda: seer.seer_sparse_prefill(qd, kd, vd, idx1, cnt1, out=out, workspace=ws)
        settle(dense, torch)
        dense_ms = time_calls(dense, max(2, args.steps // 5), torch)
        blocks1 = int(cnt1.sum().item())
        result["density1"] = {
            "prefill_ms": round(dense_ms, 4),
            "tflops": round(blocks1 * tile_flops(w.head_dim) / (dense_ms * 1e-3) / 1e12, 3),
            "speedup": round(dense_ms / pre_ms, 3),
            "ideal_speedup": round(blocks1 / blocks, 3),
        }
        del idx1, cnt1

        # Pooled-map pass on the Qwen2.5-32B shape.
        w5 = wl.C5
        log(f"[bench] pooled map {w5.name}")
        q5, k5, v5 = (t.to(dev) for t in wl.make_qkv(w5))
        o5 = torch.empty_like(q5)
        a5 = torch.empty((w5.batch, w5.hq, w5.nqb, w5.nqb), dtype=torch.float32, device=dev)
        ws5 = torch.empty((seer.pooled_attn_map_workspace_size(w5.batch, w5.hq, w5.seq),),
                          dtype=torch.uint8, device=dev)
        call = lambda: seer.seer_pooled_attn_map(q5, k5, v5, out=o5, amap=a5, workspace=ws5)
        settle(call, torch)
        pm_ms = time_calls(call, max(2, args.steps // 5), torch)
        tiles = w5.batch * w5.hq * w5.nqb * (w5.nqb + 1) // 2
        result["pooled_map"] = {
            "workload": w5.name,
            "ms": round(pm_ms, 4),
            "tflops": round(tiles * tile_flops(w5.head_dim) / (pm_ms * 1e-3) / 1e12, 3),
            "pct_of_bf16_peak": round(100 * tiles * tile_flops(w5.head_dim) / (pm_ms * 1e-3)
                                      / 1e12 / PEAK_BF16_TFLOPS, 2),
        }

        # Row-normalised target + MSE on that map against gate-like scores
        # (HBM-bound: causal halves of map and gate read, full target written).
        log("[bench] distillation target + MSE on the pooled map")
        gate = wl.make_scores(wl.custom(105, w5.batch, w5.hq, 1, 64, w5.seq,
                                        scores="softmax_normal")).to(dev)
        tgt = torch.empty_like(a5)
        rsse = torch.empty((w5.batch, w5.hq, w5.nqb), dtype=torch.float32, device=dev)
        lossd = torch.empty((1,), dtype=torch.float32, device=dev)
        tcall = lambda: seer.seer_pooled_target_mse(a5, gate, target=tgt, row_sse=rsse,
                                                    loss=lossd)
        settle(tcall, torch)
        tg_ms = time_calls(tcall, max(3, args.steps // 2), torch)
        rows = w5.batch * w5.hq * w5.nqb
        tg_bytes = 4 * (2 * tiles + rows * w5.nqb + rows + 1)
        result["pooled_target_mse"] = {
            "ms": round(tg_ms, 4),
            "gbps": round(tg_bytes / (tg_ms * 1e-3) / 1e9, 1),
            "hbm_peak_gbps": 8000.0,
            "algorithmic_bytes": tg_bytes,
        }
        del q5, k5, v5, o5, a5, ws5, gate, tgt, rsse, lossd

        # AttnGate soft scores on the bench shape (Dg 128, random-init weights): pool +
        # project + RoPE, then the causal Q~K~^T softmax (read Q and K once: HBM-bound).
        log(f"[bench] AttnGate scores on {w.name}")
        dg = 128
        wq, wk = (t.to(dev) for t in wl.make_gate_weights(w, dg))
        gs = torch.empty((w.batch, w.hq, w.nqb, w.nqb), dtype=torch.float32, device=dev)
        gws = torch.empty((seer.load().seer_attn_gate_workspace_size(
            w.batch, w.hq, w.hkv, w.seq, dg),), dtype=torch.uint8, device=dev)
        gcall = lambda: seer.seer_attn_gate_scores(qd, kd, wq, wk, scores=gs, workspace=gws)
        settle(gcall, torch)
        g_ms = time_calls(gcall, max(3, args.steps // 2), torch)
        g_bytes = 2 * (qd.numel() + kd.numel()) + 4 * gs.numel()
        # The same gate straight into the bench's TopK lists in one call (no score
        # map written), against scores + seer_build_mask.
        gmk = seer.topk_budget(w.nqb, w.density, w.keep_sink)
        gidx = torch.empty((w.batch, w.hq, w.nqb, gmk), dtype=torch.int32, device=dev)
        gcnt = torch.empty((w.batch, w.hq, w.nqb), dtype=torch.int32, device=dev)
        gws2 = torch.empty((seer.attn_gate_mask_workspace_size(
            w.batch, w.hq, w.hkv, w.seq, dg, False),), dtype=torch.uint8, device=dev)
        fcall = lambda: seer.seer_attn_gate_mask(qd, kd, wq, wk, w.mode, w.threshold, w.density,
                                                 w.keep_sink, gmk, kv_idx=gidx, kv_cnt=gcnt,
                                                 workspace=gws2)
        tcall2 = lambda: (gcall(), seer.seer_build_mask(gs, w.mode, w.threshold, w.density,
                                                        w.keep_sink, gmk, kv_idx=gidx,
                                                        kv_cnt=gcnt))
        # The one-call path in passes of two tile rows (128 query blocks) of logits.
        gws3 = torch.empty((seer.attn_gate_mask_pass_workspace_size(
            w.batch, w.hq, w.hkv, w.seq, dg, 2),), dtype=torch.uint8, device=dev)
        pcall = lambda: seer.seer_attn_gate_mask(qd, kd, wq, wk, w.mode, w.threshold, w.density,
                                                 w.keep_sink, gmk, kv_idx=gidx, kv_cnt=gcnt,
                                                 workspace=gws3)
        settle(fcall, torch)
        f_ms = time_calls(fcall, max(3, args.steps // 2), torch)
        settle(tcall2, torch)
        t2_ms = time_calls(tcall2, max(3, args.steps // 2), torch)
        settle(pcall, torch)
        p_ms = time_calls(pcall, max(3, args.steps // 2), torch)
        result["attn_gate"] = {
            "ms": round(g_ms, 4),
            "gate_dim": dg,
            "gbps": round(g_bytes / (g_ms * 1e-3) / 1e9, 1),
            "algorithmic_bytes": g_bytes,
            "gate_to_lists_fused_ms": round(f_ms, 4),
            "gate_then_build_mask_ms": round(t2_ms, 4),
            "gate_to_lists_passes_of_128_rows_ms": round(p_ms, 4),
            "logits_workspace_bytes_one_pass_vs_passes": [
                gws2.numel() - gws.numel(), gws3.numel() - gws.numel()],
        }
        del wq, wk, gs, gws, gws2, gws3, gidx, gcnt

        # The bench workload's shape with 128-token blocks (TopK at the same density).
        w128 = wl.custom(103, w.batch, w.hq, w.hkv, w.head_dim, w.seq, mode=w.mode,
                         name=w.name + "_block128",
                         density=w.density, keep_sink=w.keep_sink, scores=w.scores, block=128)
        log(f"[bench] 128-token blocks on {w.name}")
        s128 = wl.make_scores(w128).to(dev)
        mk128 = seer.topk_budget(w128.nqb, w128.density, w128.keep_sink)
        idx128, cnt128 = seer.seer_build_mask(s128, w128.mode, w128.threshold, w128.density,
                                              w128.keep_sink, mk128)
        call128 = lambda: seer.seer_sparse_prefill_block(qd, kd, vd, idx128, cnt128, 128, out=out,
                                                         workspace=ws)
        settle(call128, torch)
        b128_ms = time_calls(call128, max(3, args.steps // 2), torch)
        # 64-token tiles computed: a listed 128-block gives both of its tiles to each
        # 64-row half, except the diagonal block, whose upper tile the first half skips.
        c = cnt128.to(torch.int64)
        tiles128 = int((4 * c - 1).clamp(min=0).sum().item())
        result["block128"] = {
            "workload": w128.name,
            "prefill_ms": round(b128_ms, 4),
            "computed_tiles64": tiles128,
            "tflops": round(tiles128 * tile_flops(w.head_dim) / (b128_ms * 1e-3) / 1e12, 3),
        }
        del s128, idx128, cnt128

        # The other sparse workloads at their stated shapes: 8k with threshold 2e-3
        # lists, and 128k with TopK 0.17 lists.
        result["c2_t8192_threshold"] = sparse_config_line(seer, wl, torch, dev, wl.C2, args)
        result["c4_t131072_topk0.17"] = sparse_config_line(seer, wl, torch, dev, wl.C4, args)

        # Decode: one new token per sequence over a 40k-token cache, 4K-token budget
        # (90 % sparsity), lists per KV group and per query head.  HBM-bound: the
        # algorithmic bytes are the K and V rows of each KV group's selected blocks
        # (read once per group), plus q, o and the lists.
        result["decode"] = decode_bench(seer, wl, torch, dev, args)

    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, scores, max_k, args.cpu_blocks_per_head)
        if not args.no_extras and "c4_t131072_topk0.17" in result:
            log("[bench] CPU oracle on the 128k workload's sampled blocks")
            del q, k, v, scores
            result["c4_t131072_topk0.17"]["cpu_oracle"] = cpu_oracle_extrapolated(
                wl.C4, wl.C4.sample_qblocks)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
