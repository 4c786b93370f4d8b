#!/usr/bin/env python3
"""Benchmark of the compressed-KV hot path on one MI355X.

One step of the headline workload is the decode attention of a whole serving
batch: 32 layers (4 protected bf16 layers, 28 compressed with seeded per-layer
key/value bit widths from {(4,4), (4,3), (3,3), (3,2)}), batch 64 with context
lengths drawn uniformly from 512..32768, 32 query / 8 KV heads, head_dim 128,
16-token pages and random block tables, bf16 N(0,1) K/V with 4 outlier channels
per head scaled x10 (keys: k_bits codebook + 1-bit QJL; values: v_bits groups of
32).  It is the largest of the five workloads that fit one GPU.  The other four
are measured in the same run and reported under "configs", each with its own
roofline fraction: the tiny fp32 parity case (1 head, 1024 tokens), the
Llama-3-8B-shaped decode layer (batch 16, context 4096, K4/V4), the fused
compress of 1,048,576 tokens x 8 heads (K2 + QJL / V3) and the long-context
decode (batch 1, context 131072, K3/V2).  Decode stores that fit the 256 MB
last-level cache are rotated over several copies so that reads come from HBM.

The float64 CPU oracle is timed on bounded samples of the same workloads on this
host (cpu_baseline and configs.*.cpu_baseline).

Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps of the headline (32-layer) workload")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--pools", type=int, default=6, help="store copies rotated to defeat the cache")
    ap.add_argument("--compress-iters", type=int, default=5)
    ap.add_argument("--no-compress", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=256,
                    help="size of one plain device copy run before the workloads (counter calibration)")
    ap.add_argument("--all-configs", action="store_true",
                    help="also time the compress variants (key modes, Hadamard rotation), decompress and MSE values")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc counter files (FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="summarise a rocprofv3 --kernel-trace file per kernel and grid and exit")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "hbm_traffic_by_workload.txt")
# kernels whose HBM traffic is taken from counters: (kernel, workload tag) -> (grid in
# workgroups x*y*z, or None for any grid; the sources that define the kernel; which
# half of the matching dispatches in launch order: None all, 0 the first, 1 the second
# -- the compress workload launches the contiguous store, then the prefill batch)
TRAFFIC_KERNELS = {
    ("splitk_mfma_kernel<4,4,4,false,true>", "serving"): (8 * 8 * 64, ["decode_mainloop.hip", "split_items.hpp"], None),
    ("splitk_mfma_kernel<4,4,4,false,true>", "layer"): (4 * 8 * 16, ["decode_mainloop.hip", "split_items.hpp"], None),
    ("splitk_mfma_kernel<4,3,2,false,true>", "long"): (64 * 8 * 1, ["decode_mainloop.hip", "split_items.hpp"], None),
    ("compress_mfma_kernel<2,3,3,false,true,false>", "compress"): (None, ["compress_mfma.hip"], 0),
    ("compress_mfma_kernel<2,3,3,false,true,false>", "compress-prefill"): (None, ["compress_mfma.hip"], 1),
    ("decompress_ring_kernel<4,4,true,true,false>", "decompress"): (None, ["decompress.hip"], None),
}


def sources_sha(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, "compressed_decode_attention_tq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def copy_probe(torch, mib):
    """One plain device copy (elementwise negate) of a known size: reads and writes
    mib MiB.  Its FETCH_SIZE / WRITE_SIZE calibrate the counters of a run."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def copy_bandwidth(torch, mib=1024, reps=10):
    """Achievable HBM bandwidth on this device: a plain device-to-device copy of
    mib MiB (read + write), timed over reps copies with events."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2.0 * mib * (1 << 20) / (ms / 1e3) / 1e9


def _norm(name):
    """Kernel name without spaces, namespaces, argument list or return type."""
    n = name.replace(" ", "")
    if n.startswith("void"):
        n = n[4:]
    n = n.replace("tq::(anonymousnamespace)::", "").replace("tq::", "")
    if "(" in n:
        n = n[:n.index("(")]
    return n


def traffic_summary(fetch_csv, write_csv, mib):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the traffic kernels, grouped by
    kernel and grid, scaled by what the same counters read for the copy probe."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals, grid = {}, {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
            grid[key] = int(r.get("Grid_Size", 0) or 0) // max(int(r.get("Workgroup_Size", 1) or 1), 1)
        out = {}
        for (name, d), v in sorted(vals.items(), key=lambda kv: int(kv[0][1])):
            out.setdefault((_norm(name), grid[(name, d)]), []).append(v * 1024.0)
        return out

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    probe = [k for k in fetch if "neg" in k[0] and "elementwise" in k[0]]
    if not probe:
        raise SystemExit("copy probe kernel not found in " + fetch_csv)
    nbytes = mib * (1 << 20)
    f_scale = nbytes / statistics.median(fetch[probe[0]])
    w_scale = nbytes / statistics.median(write[probe[0]])
    lines = ["copy_probe bytes=%d fetch_factor=%.4f write_factor=%.4f" % (nbytes, f_scale, w_scale)]
    def part(vals, half):
        if half is None:
            return vals
        m = len(vals) // 2
        return vals[:m] if half == 0 else vals[m:]

    for (kern, tag), (wgs, files, half) in TRAFFIC_KERNELS.items():
        keys = [k for k in fetch if k[0] == kern and (wgs is None or k[1] == wgs)]
        if not keys or (half is not None and len(fetch[keys[0]]) < 2):
            continue
        k = keys[0]
        fb = statistics.median(part(fetch[k], half)) * f_scale
        wb = statistics.median(part(write[k], half)) * w_scale
        lines.append("kernel=%s workload=%s grid_wgs=%d sources_sha=%s fetch_bytes=%d write_bytes=%d "
                     "traffic_bytes=%d dispatches=%d" % (kern, tag, k[1], sources_sha(files), fb, wb, fb + wb,
                                                          len(part(fetch[k], half))))
    return lines


def trace_summary(trace_csv):
    """Per kernel and grid: dispatches, mean, median and minimum duration (us) from a
    rocprofv3 --kernel-trace CSV."""
    import csv
    import statistics
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        name = _norm(r["Kernel_Name"])
        if not any(x in name for x in ("splitk", "prologue", "combine", "compress", "decompress", "store_bypass")):
            continue
        grid = tuple(int(r["Grid_Size_" + a]) // max(int(r["Workgroup_Size_" + a]), 1) for a in "XYZ")
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault((name, grid, int(r["Workgroup_Size_X"])), []).append(dur)
    lines = ["| kernel | grid (WGs) | WG size | dispatches | mean (us) | median (us) | min (us) |",
             "|---|---|---|---|---|---|---|"]
    for (name, grid, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append("| `%s` | %dx%dx%d | %d | %d | %.2f | %.2f | %.2f |" % (
            name, grid[0], grid[1], grid[2], wg, len(d), statistics.mean(d), statistics.median(d), min(d)))
    return lines


def traffic_for(kernel, tag):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernel's sources changed since the counters were taken."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        f = dict(x.split("=", 1) for x in ln.split() if "=" in x)
        if f.get("kernel") == kernel and f.get("workload") == tag:
            if f.get("sources_sha") != sources_sha(TRAFFIC_KERNELS[(kernel, tag)][1]):
                return None
            return int(f["traffic_bytes"])
    return None


def _events_avg_us(torch, tq, kernel_id, fn, n):
    """Average duration (us) of the library's `kernel_id` launches over n calls of fn,
    from HIP events the library records around each launch on its own stream."""
    tq.profile_reset()
    tq.profile_enable(1 << kernel_id)
    _time_steps(torch, fn, n)
    ms, launches = tq.profile_read(kernel_id)
    tq.profile_enable(0)
    return ms / max(launches, 1) * 1e3, launches


def _splitk_bytes(lens, Hkv, Hq, rec):
    """Algorithmic bytes of one split-K launch: the KV records of every live token,
    the used block-table entries, the lengths and the rotated query / projection (f32)."""
    import numpy as np
    lens = np.asarray(lens, dtype=np.int64)
    return int(lens.sum()) * Hkv * rec + int(((lens + 15) // 16).sum()) * 4 + len(lens) * 4 + \
        len(lens) * Hq * 2 * 128 * 4


def _roofline(nbytes, avg_us, kernel, launches, traffic=None):
    gbs = nbytes / (avg_us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
            "avg_us": round(avg_us, 3), "launches": launches, "bytes_per_launch": int(nbytes)}


def serving_workload(torch, tq, synth, args):
    """Ragged mixed-bit serving batch: 32 layers, B = 64, lengths U{512..32768}.  One
    step = decode attention of all 64 sequences through all 32 layers."""
    import numpy as np
    W, sd = synth.WORKLOADS[5], synth.seeds(5)
    B, Hq, Hkv = W["B"], W["Hq"], W["Hkv"]
    lens = synth.ragged_lengths(sd["lens"], B, W["min_len"], W["max_len"])
    alloc = synth.mixed_bit_allocation(sd["alloc"], W["layers"])
    table, _ = _compact_table(sd["table"], lens)
    bt = torch.from_numpy(table).cuda()
    sl = torch.from_numpy(lens).cuda()
    maxlen = int(lens.max())
    q = torch.from_numpy(synth.queries_host(sd["data"], B, Hq)).to("cuda", torch.bfloat16)
    layers, pools, outs, wss = [], [], [], []
    for li, kv in enumerate(alloc):
        kb, vb = kv if kv else (4, 4)
        lay = tq.Layer(tq.config(Hkv, kb, vb, seed=sd["state"], layer=li, bypass=kv is None))
        layers.append(lay)
        pools.append(_fill(torch, tq, synth, lay, table, lens, Hkv, sd["data"] * 100 + li, W["outliers"]))
        outs.append(torch.empty((B, Hq, 128), dtype=torch.bfloat16, device="cuda"))
        wss.append(tq.new_workspace(lay, B, Hq, maxlen))

    def run_layer(li):
        tq.decode_attn(layers[li], q, pools[li], bt, sl, maxlen, out=outs[li], workspace=wss[li])

    def step(i):
        for li in range(len(layers)):
            run_layer(li)

    for i in range(args.warmup):
        step(i)
    ms = _time_steps(torch, step, args.steps)
    # split-K launches of each layer kind, timed with events in a second pass
    kinds = {}
    for li, kv in enumerate(alloc):
        kinds.setdefault(kv, []).append(li)
    n_ev = max(2, min(args.steps, 10))
    per_kind = {}
    for kv, lis in kinds.items():
        tot, cnt = 0.0, 0
        for li in lis:
            us, n = _events_avg_us(torch, tq, tq.K_SPLITK, lambda i, li=li: run_layer(li), n_ev)
            tot += us * n
            cnt += n
        rec = _record_bytes(*(kv if kv else (4, 4)), bypass=kv is None)
        nbytes = _splitk_bytes(lens, Hkv, Hq, rec) if kv else int(lens.sum()) * Hkv * rec + \
            int(((lens + 15) // 16).sum()) * 4 + B * 4 + B * Hq * 128 * 2
        name = "bypass" if kv is None else "K%d/V%d" % kv
        kern = "splitk_bypass_kernel<4,true>" if kv is None else "splitk_mfma_kernel<4,%d,%d,false,true>" % kv
        per_kind[name] = dict(_roofline(nbytes, tot / cnt, kern, cnt), layers=len(lis))
    total_bytes = sum(int(lens.sum()) * Hkv * _record_bytes(*(kv if kv else (4, 4)), bypass=kv is None)
                      for kv in alloc)
    dominant = max(per_kind, key=lambda k: per_kind[k]["avg_us"] * per_kind[k]["layers"])
    roof = dict(per_kind[dominant])
    roof["traffic"] = traffic_for(roof["kernel"], "serving")
    res = {
        "ms_per_step": ms, "value": B / (ms / 1e3),
        "kv_tok_s": float(lens.sum()) * len(layers) / (ms / 1e3),
        "step_hbm_gbs": total_bytes / (ms / 1e3) / 1e9,
        "record_bytes_per_step": total_bytes,
        "roofline": roof, "splitk_by_layer_kind": per_kind,
        "config": {"workload": W["name"], "layers": W["layers"], "bypass_layers": [i for i, kv in enumerate(alloc)
                                                                                    if kv is None],
                   "layer_bits": [list(kv) if kv else None for kv in alloc], "batch": B, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": 128, "seq_len_min": int(lens.min()), "seq_len_max": maxlen,
                   "tokens": int(lens.sum()), "qjl_bits": 1, "v_group": 32, "page": 16,
                   "outlier_channels": W["outliers"], "table": "random"},
    }
    ctx = {"lens": lens, "table": table, "alloc": alloc, "q": q, "W": W, "sd": sd}
    for lay in layers:
        lay.close()
    del pools, outs, wss
    torch.cuda.empty_cache()
    return res, ctx


def layer_workload(torch, tq, synth, args):
    """Llama-3-8B-shaped decode layer: B = 16, 32/8 heads, ctx 4096, K4/V4."""
    W = synth.WORKLOADS[2]
    sd = synth.seeds(2)
    B, Hq, Hkv, T = W["B"], W["Hq"], W["Hkv"], W["ctx"]
    kb, vb = W["k_bits"], W["v_bits"]
    layer = tq.Layer(tq.config(Hkv, kb, vb, seed=sd["state"]))
    maxb = T // 16
    table = synth.block_table(sd["table"], B, maxb, W["table"])
    k, v = synth.kv_device(sd["data"], B * T, Hkv, outliers=W["outliers"])
    pos = torch.arange(T, device="cuda").repeat(B)
    seq = torch.arange(B, device="cuda").repeat_interleave(T)
    bt = torch.from_numpy(table).cuda()
    slots = bt[seq, pos // 16].long() * 16 + pos % 16
    pool0 = layer.new_pool(B * maxb)
    tq.compress_kv(layer, k, v, slots, pool0)
    pools = [pool0] + [pool0.clone() for _ in range(args.pools - 1)]
    last = torch.arange(B, device="cuda") * T + (T - 1)
    k_new, v_new, slot_new = k[last].contiguous(), v[last].contiguous(), slots[last].contiguous()
    q = torch.from_numpy(synth.queries_host(sd["data"], B, Hq)).to("cuda", torch.bfloat16)
    sl = torch.full((B,), T, dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = tq.new_workspace(layer, B, Hq, T)
    torch.cuda.synchronize()

    def step(i):
        tq.decode_attn(layer, q, pools[i % len(pools)], bt, sl, T, out=out, workspace=ws)

    _time_steps(torch, step, 50)
    ms = _time_steps(torch, step, 200)
    sk_us, sk_n = _events_avg_us(torch, tq, tq.K_SPLITK, step, 200)
    append_ms = _time_steps(torch, lambda i: tq.compress_kv(layer, k_new, v_new, slot_new, pools[i % len(pools)]),
                            200)
    rec = _record_bytes(kb, vb)
    splitk_bytes = _splitk_bytes([T] * B, Hkv, Hq, rec)
    step_bytes = splitk_bytes + B * Hq * 128 * 2 * 2  # + q in, out (bf16)
    roof = _roofline(splitk_bytes, sk_us, "splitk_mfma_kernel<4,4,4,false,true>", sk_n, traffic_for("splitk_mfma_kernel<4,4,4,false,true>",
                                                                                           "layer"))
    res = {"workload": W["name"], "decode_us": round(ms * 1e3, 3), "decode_tok_s": round(B / (ms / 1e3), 1),
           "kv_tok_s": round(B * T / (ms / 1e3), 1), "step_hbm_gbs": round(step_bytes / (ms / 1e3) / 1e9, 1),
           "step_frac": round(step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "roofline": roof,
           "append_us": round(append_ms * 1e3, 2), "steps": 200, "warmup": 50,
           "config": {"batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": 128, "context": T, "k_bits": kb,
                      "qjl_bits": 1, "v_bits": vb, "v_group": 32, "page": 16, "outlier_channels": W["outliers"],
                      "store_copies_rotated": len(pools)}}
    ctx = {"k": k, "v": v, "q": q, "table": table, "W": W, "sd": sd}
    layer.close()
    del pools, pool0
    return res, ctx


def long_context_workload(torch, tq, synth, args):
    """B = 1, ctx 131072, K3/V2, seeded random block table; three store copies rotated."""
    W, sd = synth.WORKLOADS[4], synth.seeds(4)
    T, Hkv, Hq = W["ctx"], W["Hkv"], W["Hq"]
    layer = tq.Layer(tq.config(Hkv, W["k_bits"], W["v_bits"], seed=sd["state"]))
    table = synth.block_table(sd["table"], 1, T // 16, "random")
    pool0 = _fill(torch, tq, synth, layer, table, [T], Hkv, sd["data"], W["outliers"])
    pools = [pool0] + [pool0.clone() for _ in range(2)]
    q = torch.from_numpy(synth.queries_host(sd["data"], 1, Hq)).to("cuda", torch.bfloat16)
    bt = torch.from_numpy(table).cuda()
    sl = torch.full((1,), T, dtype=torch.int32, device="cuda")
    ws = tq.new_workspace(layer, 1, Hq, T)
    out = torch.empty((1, Hq, 128), dtype=torch.bfloat16, device="cuda")
    step = lambda i: tq.decode_attn(layer, q, pools[i % 3], bt, sl, T, out=out, workspace=ws)
    _time_steps(torch, step, 10)
    ms = _time_steps(torch, step, 60)
    sk_us, sk_n = _events_avg_us(torch, tq, tq.K_SPLITK, step, 60)
    nbytes = _splitk_bytes([T], Hkv, Hq, _record_bytes(W["k_bits"], W["v_bits"]))
    layer.close()
    del pools, pool0
    return {"workload": W["name"], "decode_us": round(ms * 1e3, 2), "decode_tok_s": round(1 / (ms / 1e3), 1),
            "kv_tok_s": round(T / (ms / 1e3), 1), "step_frac": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "roofline": _roofline(nbytes, sk_us, "splitk_mfma_kernel<4,3,2,false,true>", sk_n,
                                  traffic_for("splitk_mfma_kernel<4,3,2,false,true>", "long")),
            "steps": 60, "warmup": 10,
            "config": {"batch": 1, "q_heads": Hq, "kv_heads": Hkv, "head_dim": 128, "context": T,
                       "k_bits": W["k_bits"], "qjl_bits": 1, "v_bits": W["v_bits"], "v_group": 32, "page": 16,
                       "outlier_channels": W["outliers"], "table": "random", "store_copies_rotated": 3}}


def tiny_workload(torch, tq, synth, args):
    """1 KV head, 1024 fp32 tokens, K2 + QJL / V3: launch-latency bound (latency reported)."""
    W, sd = synth.WORKLOADS[1], synth.seeds(1)
    layer = tq.Layer(tq.config(W["Hkv"], W["k_bits"], W["v_bits"], seed=sd["state"]))
    table = synth.block_table(sd["table"], 1, W["ctx"] // 16, "identity")
    pool = _fill(torch, tq, synth, layer, table, [W["ctx"]], W["Hkv"], sd["data"], 0, dtype="f32")
    q = torch.from_numpy(synth.queries_host(sd["data"], 1, W["Hq"], dtype="f32")).cuda()
    bt = torch.from_numpy(table).cuda()
    sl = torch.full((1,), W["ctx"], dtype=torch.int32, device="cuda")
    ws = tq.new_workspace(layer, 1, W["Hq"], W["ctx"])
    out = torch.empty((1, W["Hq"], 128), dtype=torch.float32, device="cuda")
    step = lambda i: tq.decode_attn(layer, q, pool, bt, sl, W["ctx"], out=out, workspace=ws)
    _time_steps(torch, step, 20)
    ms = _time_steps(torch, step, 200)
    sk_us, sk_n = _events_avg_us(torch, tq, tq.K_SPLITK, step, 200)
    nbytes = _splitk_bytes([W["ctx"]], W["Hkv"], W["Hq"], _record_bytes(W["k_bits"], W["v_bits"]))
    layer.close()
    return {"workload": W["name"], "decode_us": round(ms * 1e3, 2), "decode_tok_s": round(1 / (ms / 1e3), 1),
            "roofline": _roofline(nbytes, sk_us, "splitk_mfma_kernel<1,2,3,false,true>", sk_n),
            "note": "0.12 MB per launch: launch-latency bound, the HBM fraction is not meaningful",
            "steps": 200, "warmup": 20,
            "config": {"batch": 1, "q_heads": W["Hq"], "kv_heads": W["Hkv"], "head_dim": 128, "context": W["ctx"],
                       "dtype": "f32", "k_bits": W["k_bits"], "qjl_bits": 1, "v_bits": W["v_bits"], "v_group": 32}}


def compress_workload(torch, tq, synth, args, key_mode=0, rotation=0):
    W = synth.WORKLOADS[3]
    sd = synth.seeds(3)
    N, H = W["N"], W["Hkv"]
    layer = tq.Layer(tq.config(H, W["k_bits"], W["v_bits"], seed=sd["state"], key_mode=key_mode,
                               rotation=rotation))
    k, v = synth.kv_device(sd["data"], N, H)
    pool = layer.new_pool(N // 16)
    slots = torch.arange(N, dtype=torch.int64, device="cuda")
    tq.compress_kv(layer, k, v, slots, pool)
    torch.cuda.synchronize()
    tq.profile_reset()
    tq.profile_enable(1 << tq.K_COMPRESS)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.compress_iters):
        tq.compress_kv(layer, k, v, slots, pool)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.compress_iters
    c_ms, c_n = tq.profile_read(tq.K_COMPRESS)
    tq.profile_enable(0)
    rec = layer.block_bytes // 16  # per token-head; the key modes without QJL store no sign field
    nbytes = N * H * (512 + rec) + N * 8
    avg_s = c_ms / max(c_n, 1) / 1e3
    prefill = None
    if not (key_mode or rotation):
        prefill = _prefill_batch_leg(torch, tq, synth, args, layer, k, v, N, H, rec)
    layer.close()
    del k, v, pool
    if key_mode or rotation:
        return {"workload": W["name"], "key_mode": ["qjl", "mse", "mse_nc"][key_mode],
                "rotation": ["haar", "hadamard"][rotation], "record_bytes": rec, "ms": round(ms, 4),
                "mtok_s": round(N / (ms / 1e3) / 1e6, 2), "gbs": round(nbytes / avg_s / 1e9, 1),
                "frac": round(nbytes / avg_s / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes}
    return {"workload": W["name"], "tokens": N, "kv_heads": H, "k_bits": W["k_bits"], "v_bits": W["v_bits"],
            "ms": round(ms, 4), "mtok_s": round(N / (ms / 1e3) / 1e6, 2), "prefill_batch": prefill,
            "roofline": {"bound": "hbm", "achieved": round(nbytes / avg_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(nbytes / avg_s / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": traffic_for("compress_mfma_kernel<2,3,3,false,true,false>", "compress"),
                         "kernel": "compress_mfma_kernel<2,3,3,false,true,false>",
                         "avg_us": round(avg_s * 1e6, 2), "bytes_per_launch": nbytes}}


def _prefill_batch_leg(torch, tq, synth, args, layer, k, v, N, H, rec):
    """The same tokens as a prefill batch: 64 sequences of seeded lengths U{512..32768},
    scaled to N tokens in all, laid end to end in the input, each written from offset
    0 of its own shuffled pages (so the compressor's 16-token tiles straddle pages)."""
    import numpy as np
    lens = synth.ragged_lengths(606, 64, 512, 32768).astype(np.int64)
    lens = np.maximum(lens * N // int(lens.sum()), 1)
    lens[-1] += N - int(lens.sum())
    table, _ = _compact_table(607, lens)
    b_of = np.repeat(np.arange(len(lens)), lens)
    pos = np.concatenate([np.arange(x) for x in lens])
    slots = torch.from_numpy(table[b_of, pos // 16].astype(np.int64) * 16 + pos % 16).cuda()
    pool = layer.new_pool(int(table.max()) + 1)
    tq.compress_kv(layer, k, v, slots, pool)
    torch.cuda.synchronize()
    tq.profile_reset()
    tq.profile_enable(1 << tq.K_COMPRESS)
    for _ in range(args.compress_iters):
        tq.compress_kv(layer, k, v, slots, pool)
    torch.cuda.synchronize()
    c_ms, c_n = tq.profile_read(tq.K_COMPRESS)
    tq.profile_enable(0)
    avg_s = c_ms / max(c_n, 1) / 1e3
    nbytes = N * H * (512 + rec) + N * 8
    del pool
    return {"sequences": len(lens), "tokens": N, "avg_us": round(avg_s * 1e6, 1),
            "mtok_s": round(N / avg_s / 1e6, 2), "frac": round(nbytes / avg_s / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_launch": nbytes,
            "traffic": traffic_for("compress_mfma_kernel<2,3,3,false,true,false>", "compress-prefill")}


def _time_steps(torch, fn, n):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _record_bytes(kb, vb, bypass=False):
    return 512 if bypass else kb * 16 + 20 + vb * 16 + 16


def _compact_table(seed, lens):
    """Block table [B, max_blocks] whose sequences own a seeded random permutation of
    exactly the blocks they need (unused entries 0)."""
    import numpy as np
    nb = (np.asarray(lens, dtype=np.int64) + 15) // 16
    perm = np.random.default_rng(seed).permutation(int(nb.sum()))
    table = np.zeros((len(lens), int(nb.max())), dtype=np.int32)
    o = 0
    for b, n in enumerate(nb):
        table[b, :n] = perm[o:o + n]
        o += n
    return table, int(nb.sum())


def _fill(torch, tq, synth, layer, table, lens, Hkv, seed, outliers, dtype="bf16"):
    """Compress synthetic K/V of every sequence into a new pool (token-major order)."""
    import numpy as np
    nblocks = int(table.max()) + 1
    pool = layer.new_pool(nblocks)
    N = int(np.sum(lens))
    k, v = synth.kv_device(seed, N, Hkv, outliers=outliers, dtype=dtype)
    b_of = np.repeat(np.arange(len(lens)), lens)
    pos = np.concatenate([np.arange(n) for n in lens])
    slots = table[b_of, pos // 16].astype(np.int64) * 16 + pos % 16
    tq.compress_kv(layer, k, v, torch.from_numpy(slots).cuda(), pool)
    torch.cuda.synchronize()
    del k, v
    return pool


def decompress_workload(torch, tq, synth, args):
    """The headline store (16 x 4096 tokens x 8 KV heads, K4/V4) reconstructed to bf16 K and V."""
    W, sd = synth.WORKLOADS[2], synth.seeds(2)
    B, Hkv, T = W["B"], W["Hkv"], W["ctx"]
    layer = tq.Layer(tq.config(Hkv, W["k_bits"], W["v_bits"], seed=sd["state"]))
    table = synth.block_table(sd["table"], B, T // 16, W["table"])
    pool = _fill(torch, tq, synth, layer, table, [T] * B, Hkv, sd["data"], W["outliers"])
    import numpy as np
    b_of = np.repeat(np.arange(B), T)
    pos = np.tile(np.arange(T), B)
    slots = torch.from_numpy(table[b_of, pos // 16].astype(np.int64) * 16 + pos % 16).cuda()
    N = B * T
    kd = torch.empty((N, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    vd = torch.empty_like(kd)
    step = lambda i: tq.decompress_kv(layer, pool, slots, k_out=kd, v_out=vd)
    _time_steps(torch, step, 5)
    ms = _time_steps(torch, step, 50)
    layer.close()
    rec = _record_bytes(W["k_bits"], W["v_bits"])
    nbytes = N * Hkv * (rec + 512) + N * 8
    # matrix-core floor: 6 passes x 4 K-steps x 8 column tiles per 16 token-heads,
    # 16 cycles each at 1024 SIMDs x 2.4 GHz
    mfma_us = N * Hkv / 16 * 192 * 16 / (1024 * 2.4e9) * 1e6
    kern = "decompress_ring_kernel<4,4,true,true,false>"
    return {"workload": "decompress-llama3-8b-layer-store", "token_heads": N * Hkv, "out_dtype": "bf16",
            "ms": round(ms, 4), "gbs": round(nbytes / (ms / 1e3) / 1e9, 1),
            "frac": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes,
            "mfma_floor_us": round(mfma_us, 1),
            "roofline": _roofline(nbytes, ms * 1e3, kern, 50, traffic_for(kern, "decompress"))}


def mse_values_workload(torch, tq, synth, args):
    """The Llama-3-8B layer's shape (16 x 4096 tokens x 8 KV heads, 32 query heads) with
    2-bit keys + QJL and 3-bit values coded like the keys (the 102-byte record): the
    fused compress into the store, the decode step over it (three store copies
    rotated) and the decompress to bf16 K and V."""
    B, Hkv, Hq, T = 16, 8, 32, 4096
    N = B * T
    layer = tq.Layer(tq.config(Hkv, 2, 3, seed=361, value_mode=tq.VAL_MSE))
    k, v = synth.kv_device(362, N, Hkv, outliers=4)
    pool = layer.new_pool(N // 16)
    slots = torch.arange(N, dtype=torch.int64, device="cuda")
    comp = lambda i: tq.compress_kv(layer, k, v, slots, pool)
    _time_steps(torch, comp, 2)
    ms_c = _time_steps(torch, comp, 10)
    pools = [pool] + [pool.clone() for _ in range(2)]
    table = torch.arange(N // 16, dtype=torch.int32, device="cuda").view(B, T // 16)
    sl = torch.full((B,), T, dtype=torch.int32, device="cuda")
    q = torch.from_numpy(synth.queries_host(363, B, Hq)).to("cuda", torch.bfloat16)
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = tq.new_workspace(layer, B, Hq, T)
    step = lambda i: tq.decode_attn(layer, q, pools[i % 3], table, sl, T, out=out, workspace=ws)
    _time_steps(torch, step, 20)
    ms_s = _time_steps(torch, step, 100)
    sk_us, sk_n = _events_avg_us(torch, tq, tq.K_SPLITK, step, 100)
    kd = torch.empty((N, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    vd = torch.empty_like(kd)
    dec = lambda i: tq.decompress_kv(layer, pool, slots, k_out=kd, v_out=vd)
    _time_steps(torch, dec, 5)
    ms_d = _time_steps(torch, dec, 50)
    rec = layer.block_bytes // 16
    layer.close()
    nbytes = N * Hkv * (512 + rec) + N * 8  # bf16 K+V and the record, either direction, + slots
    sk_bytes = _splitk_bytes([T] * B, Hkv, Hq, rec)
    return {"workload": "mse-values-k2qjl-v3-layer", "token_heads": N * Hkv, "record_bytes": rec,
            "compress_ms": round(ms_c, 4), "compress_gbs": round(nbytes / (ms_c / 1e3) / 1e9, 1),
            "compress_frac": round(nbytes / (ms_c / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "decode_us": round(ms_s * 1e3, 3), "decode_tok_s": round(B / (ms_s / 1e3), 1),
            "splitk": _roofline(sk_bytes, sk_us, "splitk_mfma_kernel<4,2,3,true,true>", sk_n),
            "decompress_ms": round(ms_d, 4), "decompress_gbs": round(nbytes / (ms_d / 1e3) / 1e9, 1),
            "decompress_frac": round(nbytes / (ms_d / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes}


def _oracle_job(job):
    """One oracle job in a worker process (one BLAS thread): set up untimed, wait
    for the other workers at the barrier, then run the timed part.  Returns
    (start, end) on the shared monotonic clock.
      ("decode", K, V, q, table_row, T, Hkv, kb, vb, seed, layer, bypass):
          compress the sequence's context into a store (untimed), then decode
      ("compress", K, V, Hkv, kb, vb, seed): compress the tokens into a store"""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import compress as ocomp, decode as odec, layout as olay, state as ostate

    from compressed_decode_attention_tq_amd import synth

    with threadpool_limits(1):
        if job[0] == "compress":
            _, K, V, Hkv, kb, vb, seed = job
            st = ostate.LayerState(seed, 0, Hkv, 128, kb, vb, 32)
            lay = olay.StoreLayout(128, kb, vb, 32)
            pool = olay.new_pool((len(K) + 15) // 16, Hkv, lay)
            _BARRIER.wait()
            t0 = time.perf_counter()
            ocomp.compress_into_pool(K, V, np.arange(len(K)), pool, lay, st, keep=False)
            return t0, time.perf_counter()
        _, K, V, q, table_row, T, Hkv, kb, vb, seed, layer, bypass = job
        lay = olay.StoreLayout(128, kb, vb, 32, bypass=bypass)
        nb = int(table_row.max()) + 1
        pool = olay.new_pool(nb, Hkv, lay)
        pos = np.arange(T)
        slots = table_row[pos // 16].astype(np.int64) * 16 + pos % 16
        if bypass:
            st = None
            ocomp.store_bypass(synth.bf16_bits(K), synth.bf16_bits(V), slots, pool, lay, Hkv)
        else:
            st = ostate.LayerState(seed, layer, Hkv, 128, kb, vb, 32)
            ocomp.compress_into_pool(K, V, slots, pool, lay, st, keep=False)
        _BARRIER.wait()
        t0 = time.perf_counter()
        odec.decode(q, pool, lay, Hkv, table_row[None, :], np.array([T]), st)
        return t0, time.perf_counter()


_BARRIER = None


def _worker_init(barrier):
    global _BARRIER
    _BARRIER = barrier


def _run_oracle_jobs(jobs):
    """Run jobs side by side in worker processes (at most 16 at a time: the host
    cores the run may use); per job its (start, end).  Raises if workers cannot start."""
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(cores, 16, len(jobs)))
    mctx = mp.get_context("spawn")  # fresh interpreters: nothing of this process's GPU state
    spans = []
    for r0 in range(0, len(jobs), workers):
        batch = jobs[r0:r0 + workers]
        barrier = mctx.Barrier(len(batch))
        with mctx.Pool(len(batch), initializer=_worker_init, initargs=(barrier,)) as pool:
            spans += pool.map(_oracle_job, batch)
    return spans, workers, cores


def _host_rows(t, rows):
    return t[rows].float().cpu().numpy()


def cpu_baseline_serving(torch, synth, ctx):
    """Oracle decode of a bounded sample of the serving batch: sequences 0, 31, 63
    through one layer of each kind (bf16, K4/V4, K3/V2, K4/V3, K3/V3); the cost per
    token of each layer kind is extrapolated to all 64 sequences x 32 layers run on
    the same number of worker processes."""
    import numpy as np
    lens, table, alloc, W, sd = ctx["lens"], ctx["table"], ctx["alloc"], ctx["W"], ctx["sd"]
    B, Hkv = W["B"], W["Hkv"]
    q = ctx["q"].float().cpu().numpy().astype(np.float64)
    picks, seen = [], set()
    for li, kv in enumerate(alloc):
        if kv not in seen:
            seen.add(kv)
            picks.append(li)
    sample = [0, 31, 63]
    off = np.concatenate([[0], np.cumsum(lens)])
    jobs, meta = [], []
    for li in picks:
        kv = alloc[li]
        kb, vb = kv if kv else (4, 4)
        k, v = synth.kv_device(sd["data"] * 100 + li, int(lens.sum()), Hkv, outliers=W["outliers"])
        for b in sample:
            rows = torch.arange(int(off[b]), int(off[b + 1]), device="cuda")
            jobs.append(("decode", _host_rows(k, rows), _host_rows(v, rows), q[b:b + 1], table[b], int(lens[b]), Hkv,
                         kb, vb, sd["state"], li, kv is None))
            meta.append((kv, int(lens[b])))
        del k, v
    spans, workers, cores = _run_oracle_jobs(jobs)
    per_tok = {}
    for (kv, T), (t0, t1) in zip(meta, spans):
        per_tok.setdefault(kv, []).append((t1 - t0) / T)
    cost = {kv: float(np.mean(c)) for kv, c in per_tok.items()}
    serial_s = sum(float(lens.sum()) * cost[kv] for kv in alloc)
    step_s = serial_s / workers
    return {"value": round(B / step_s, 4), "unit": "decode tok/s", "cores": workers, "kind": "oracle",
            "sample": "float64 NumPy oracle, %d worker processes of one thread: decode of sequences %s (%s tokens) "
                      "through layers %s (one of each kind: bf16, K4/V4, K3/V2, K4/V3, K3/V3), 32 query heads each; "
                      "the measured seconds per token of each layer kind extrapolated to all %d sequences x 32 "
                      "layers on the same workers (%.0f s of oracle work per step)"
                      % (workers, sample, [int(lens[b]) for b in sample], picks, B, serial_s),
            "measured_s": round(sum(t1 - t0 for t0, t1 in spans), 2), "host_cores_available": cores,
            "extrapolated": True}


def cpu_baseline_layer(torch, synth, ctx):
    """Oracle decode of all 16 sequences of the Llama-3-8B-shaped layer, side by side."""
    import numpy as np
    W, sd = ctx["W"], ctx["sd"]
    B, Hkv, T = W["B"], W["Hkv"], W["ctx"]
    q = ctx["q"].float().cpu().numpy().astype(np.float64)
    jobs = [("decode", ctx["k"][b * T:(b + 1) * T].float().cpu().numpy(),
             ctx["v"][b * T:(b + 1) * T].float().cpu().numpy(), q[b:b + 1], ctx["table"][b], T, Hkv, W["k_bits"],
             W["v_bits"], sd["state"], 0, False) for b in range(B)]
    spans, workers, cores = _run_oracle_jobs(jobs)
    wall = max(e for _, e in spans) - min(s for s, _ in spans)
    return {"value": round(B / wall, 3), "unit": "decode tok/s", "cores": workers, "kind": "oracle",
            "sample": "all %d sequences (float64 NumPy), %d worker processes of one thread; timed: wall clock of "
                      "the decode steps (32 query heads over 4096 compressed tokens each)" % (B, workers),
            "seconds": round(wall, 2), "host_cores_available": cores, "extrapolated": False}


def cpu_baseline_compress(torch, synth):
    """Oracle compress of the first 65,536 tokens of the 1,048,576-token workload,
    split over the worker processes (4,096 tokens x 8 heads each)."""
    W, sd = synth.WORKLOADS[3], synth.seeds(3)
    n_sample, H = 65536, W["Hkv"]
    k, v = synth.kv_device(sd["data"], W["N"], H)
    chunk = 4096
    jobs = [("compress", k[i:i + chunk].float().cpu().numpy(), v[i:i + chunk].float().cpu().numpy(), H,
             W["k_bits"], W["v_bits"], sd["state"]) for i in range(0, n_sample, chunk)]
    del k, v
    spans, workers, cores = _run_oracle_jobs(jobs)
    rounds = (len(jobs) + workers - 1) // workers
    wall = max(e for _, e in spans) - min(s for s, _ in spans)
    return {"value": round(n_sample / wall / 1e6, 6), "unit": "Mtok/s", "cores": workers, "kind": "oracle",
            "sample": "the first %d of %d tokens x %d heads (float64 NumPy), %d jobs of %d tokens on %d worker "
                      "processes of one thread (%d round%s); timed: wall clock of the compress calls"
                      % (n_sample, W["N"], H, len(jobs), chunk, workers, rounds, "s" if rounds > 1 else ""),
            "seconds": round(wall, 2), "host_cores_available": cores, "extrapolated": False}


def cpu_baseline_long(torch, synth):
    """Oracle decode of the first 8,192 tokens of the 131,072-token context (one
    worker), extrapolated linearly to the whole context."""
    import numpy as np
    W, sd = synth.WORKLOADS[4], synth.seeds(4)
    T, Hkv, Hq, n = W["ctx"], W["Hkv"], W["Hq"], 8192
    table = synth.block_table(sd["table"], 1, T // 16, "random")
    k, v = synth.kv_device(sd["data"], T, Hkv, outliers=W["outliers"])
    q = synth.queries_host(sd["data"], 1, Hq).astype(np.float64)
    rows = torch.arange(n, device="cuda")
    jobs = [("decode", _host_rows(k, rows), _host_rows(v, rows), q, table[0], n, Hkv, W["k_bits"], W["v_bits"],
             sd["state"], 0, False)]
    del k, v
    spans, workers, cores = _run_oracle_jobs(jobs)
    t = spans[0][1] - spans[0][0]
    step_s = t * T / n
    return {"value": round(1.0 / step_s, 5), "unit": "decode tok/s", "cores": 1, "kind": "oracle",
            "sample": "decode of the first %d of %d context tokens (float64 NumPy, one thread, 32 query heads), "
                      "extrapolated linearly in the context length" % (n, T),
            "measured_s": round(t, 2), "host_cores_available": cores, "extrapolated": True}


def cpu_baseline_tiny(torch, synth):
    """Oracle decode of the whole tiny case (1 head, 1024 fp32 tokens)."""
    W, sd = synth.WORKLOADS[1], synth.seeds(1)
    K, V = synth.kv_host(sd["data"], W["ctx"], W["Hkv"], dtype="f32")
    import numpy as np
    q = synth.queries_host(sd["data"], 1, W["Hq"], dtype="f32").astype(np.float64)
    table = synth.block_table(sd["table"], 1, W["ctx"] // 16, "identity")
    jobs = [("decode", K, V, q, table[0], W["ctx"], W["Hkv"], W["k_bits"], W["v_bits"], sd["state"], 0, False)]
    spans, workers, cores = _run_oracle_jobs(jobs)
    t = spans[0][1] - spans[0][0]
    return {"value": round(t * 1e6, 1), "unit": "decode us", "cores": 1, "kind": "oracle",
            "sample": "the whole case (float64 NumPy, one thread)", "host_cores_available": cores,
            "extrapolated": False}


def main():
    args = parse()
    if args.traffic_from:
        print("\n".join(traffic_summary(args.traffic_from[0], args.traffic_from[1], args.copy_probe_mib)))
        return
    if args.trace_summary:
        print("\n".join(trace_summary(args.trace_summary)))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the compressed-KV path runs on one device per process and "
              "the library has no multi-GPU path (--gpus %d refused)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import compressed_decode_attention_tq_amd as tq
    from compressed_decode_attention_tq_amd import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    tq.lib()
    if args.copy_probe_mib > 0:
        copy_probe(torch, args.copy_probe_mib)
    copy_gbs = copy_bandwidth(torch)
    log("serving batch (headline): 32 layers, B=64")
    head, head_ctx = serving_workload(torch, tq, synth, args)
    configs = {}
    log("tiny fp32 case")
    configs["1"] = tiny_workload(torch, tq, synth, args)
    log("llama3-8b-shaped decode layer")
    configs["2"], layer_ctx = layer_workload(torch, tq, synth, args)
    comp = None
    if not args.no_compress:
        log("fused compress, 1M tokens x 8 heads")
        comp = compress_workload(torch, tq, synth, args)
        configs["3"] = comp
    log("long-context decode")
    configs["4"] = long_context_workload(torch, tq, synth, args)
    configs["5"] = {"workload": head["config"]["workload"], "decode_ms": round(head["ms_per_step"], 4),
                    "decode_tok_s": round(head["value"], 2), "kv_tok_s": round(head["kv_tok_s"], 1),
                    "step_hbm_gbs": round(head["step_hbm_gbs"], 1),
                    "step_frac": round(head["step_hbm_gbs"] / HBM_PEAK_GBS, 4),
                    "roofline": head["roofline"], "splitk_by_layer_kind": head["splitk_by_layer_kind"],
                    "steps": args.steps, "warmup": args.warmup}
    extra = None
    if args.all_configs:
        extra = {}
        if not args.no_compress:
            log("compress workload, key modes without QJL")
            extra["fused-compress-key-mse"] = compress_workload(torch, tq, synth, args, key_mode=tq.KEY_MSE)
            extra["fused-compress-key-mse-nc"] = compress_workload(torch, tq, synth, args, key_mode=tq.KEY_MSE_NC)
            log("compress workload, randomised Hadamard rotation")
            extra["fused-compress-hadamard"] = compress_workload(torch, tq, synth, args, rotation=tq.ROT_HADAMARD)
            extra["fused-compress-hadamard-key-mse-nc"] = compress_workload(
                torch, tq, synth, args, key_mode=tq.KEY_MSE_NC, rotation=tq.ROT_HADAMARD)
        log("decompress workload")
        extra["decompress"] = decompress_workload(torch, tq, synth, args)
        log("mse values")
        extra["mse_values"] = mse_values_workload(torch, tq, synth, args)
    cpu = None
    if not args.no_cpu_baseline:
        for key, name, fn in (("5", "serving", lambda: cpu_baseline_serving(torch, synth, head_ctx)),
                              ("1", "tiny", lambda: cpu_baseline_tiny(torch, synth)),
                              ("2", "layer", lambda: cpu_baseline_layer(torch, synth, layer_ctx)),
                              ("3", "compress", lambda: cpu_baseline_compress(torch, synth)),
                              ("4", "long context", lambda: cpu_baseline_long(torch, synth))):
            if key not in configs:
                continue
            log("cpu baseline:", name)
            try:
                configs[key]["cpu_baseline"] = fn()
            except Exception as e:  # a reported baseline; the GPU figures stand without it
                log("cpu baseline %s failed: %r" % (name, e))
                configs[key]["cpu_baseline"] = None
        cpu = configs["5"].get("cpu_baseline")
    layer_roof = configs["2"]["roofline"]
    line = {
        "metric": "compressed-KV decode attn tokens/s + HBM GB/s (% of peak); compress Mtok/s",
        "value": round(head["value"], 2),
        "unit": "decode tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_note": "scores, softmax and accumulation in float32; matrix-core operands are float16 hi + lo "
                      "pieces (about 22 significant bits) of float32 values, bf16 K/V and queries in",
        "data": "synthetic (seeded N(0,1) bf16 K/V with 4 outlier channels per head x10; ragged lengths; "
                "random block tables)",
        "config": head["config"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "kv_tok_s": round(head["kv_tok_s"], 1),
        "step_hbm_gbs": round(head["step_hbm_gbs"], 1),
        "step_hbm_frac": round(head["step_hbm_gbs"] / HBM_PEAK_GBS, 4),
        "device_copy_gbs": round(copy_gbs, 1),
        "splitk_frac_of_copy": round(head["roofline"]["achieved"] / copy_gbs, 4),
        "layer_splitk_frac": layer_roof["frac"],
        "compress_mtok_s": comp["mtok_s"] if comp else None,
        "compress_frac": comp["roofline"]["frac"] if comp else None,
        "configs": configs,
    }
    if extra is not None:
        line["other_workloads"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
